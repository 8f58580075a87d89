"""GPU: the conv step's SiLU for bfloat16 outputs, bit for bit, over every input.

The kernels form bf16(silu(pre)) from a fast estimate and fall back to the exact
float path only when the estimate's error interval holds a bf16 rounding
boundary (or pre is outside the estimate's range).  With one-hot taps the
pre-activation is the input itself, so a conv step over all 65536 bfloat16 bit
patterns checks the rounding of every bf16 input against the oracle's exact
float arithmetic (NaN inputs and NaN results are compared as NaN, since the
payload of a NaN is not part of the result).  Random taps with a wide spread
cover general float pre-activations, including the range where the exact path
is taken.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from speculative_verify_gdn_amd import gdn

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load()
    yield
    torch.cuda.synchronize()


def _run(x, w, hist):
    y = torch.empty_like(x, device="cuda")
    gdn.conv_step(x.cuda(), w.cuda(), hist.cuda(), y)     # hist.cuda() is a copy: the write-back stays on it
    torch.cuda.synchronize()
    return y.cpu()


def _compare(y_gpu, x, w, hist):
    y_ref, _, _ = oracle.conv_step_f32(x.float().numpy(), w.numpy(), hist.float().numpy(), True)
    ref = torch.from_numpy(y_ref).to(torch.bfloat16)
    g, r = y_gpu.view(torch.int16).numpy(), ref.view(torch.int16).numpy()
    gn, rn = torch.isnan(y_gpu).numpy(), torch.isnan(ref).numpy()
    assert np.array_equal(gn, rn), "NaN pattern differs"
    bad = (g != r) & ~gn
    assert not bad.any(), "bits differ at %d places" % int(bad.sum())


def test_every_bf16_input_through_one_hot_taps():
    say("conv silu: all 65536 bf16 inputs")
    C, W = 65536, 4
    x = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).reshape(1, 1, C).clone()
    w = torch.zeros(C, W)
    w[:, W - 1] = 1.0                       # the newest token only: pre = x
    hist = torch.zeros(1, W - 1, C, dtype=torch.bfloat16)
    _compare(_run(x, w, hist), x, w, hist)


@pytest.mark.parametrize("scale", [0.5, 8.0, 40.0])
def test_wide_random_preactivations(scale):
    say("conv silu: random taps, scale", scale)
    g = torch.Generator().manual_seed(int(scale * 10))
    B, T, C, W = 2, 16, 8192, 4
    x = torch.randn(B, T, C, generator=g).to(torch.bfloat16)
    w = torch.randn(C, W, generator=g) * scale
    hist = torch.randn(B, W - 1, C, generator=g).to(torch.bfloat16)
    _compare(_run(x, w, hist), x, w, hist)
