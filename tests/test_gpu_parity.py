"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars:
  - conv step: bit-exact against the oracle's same-precision float conv
    (y, the written-back history and the rollback window);
  - GDN: for every sequence, head and state (S_out and every H_t)
    max |S_gpu - S_ref| <= 2e-3 * ||S_ref||_F (fp32 state, bf16 inputs);
    outputs: |o_gpu - o_ref| <= 2e-3 * ||S_t||_F (|o_t| <= ||S_t||_F when
    ||q^|| = 1), plus half a bf16 ulp of o when o is bf16;
  - rollback: bit-exact copies.
Every test prints the case it runs before touching the device.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from speculative_verify_gdn_amd import gdn, synth

pytestmark = pytest.mark.gpu

TOL = 2e-3
# regression guard, beside the bar: the observed worst state error is below 1e-6 of the state's
# Frobenius norm (fp32 arithmetic on the oracle's own bf16 inputs; largest seen 7e-7, in the
# prefill), so a 100x regression fails here long before it reaches the 2e-3 bar
GUARD = 1e-4


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


def dev(t):
    return t.contiguous().cuda()


def f64(t):
    return t.double().cpu().numpy()


# ------------------------------------------------------------------ helpers
def run_verify_gpu(wl, inp, qkv, capture=True, o_dtype=None, raw=True, S_out_inplace=False):
    B, K, Hv, dv, dk = wl.B, wl.T, wl.Hv, wl.dv, wl.dk
    io = torch.bfloat16 if wl.bf16 else torch.float32
    o_dtype = o_dtype or torch.float32
    d = {k: dev(v) for k, v in inp.items()}
    d_qkv = dev(qkv)
    S_out = d["S_in"] if S_out_inplace else torch.empty_like(d["S_in"])
    H = torch.empty(B, K - 1, Hv, dv, dk, device="cuda") if (capture and K > 1) else None
    o = torch.empty(B, K, Hv, dv, device="cuda", dtype=o_dtype)
    dt, alog = (d["dt_bias"], d["A_log"]) if raw else (None, None)
    gdn.verify(d_qkv, d["beta_raw"], d["alpha"], dt, alog, d["S_in"], S_out, H, o, wl.Hk)
    torch.cuda.synchronize()
    return S_out, H, o, d


def check_states(gpu, ref, what):
    gpu = gpu.astype(np.float64)
    err = np.abs(gpu - ref).max(axis=(-1, -2))
    fro = np.linalg.norm(ref, axis=(-1, -2))
    bad = err > TOL * fro
    worst = float(np.max(err / np.maximum(fro, 1e-30)))
    print("[parity] %s worst err/fro %.3g" % (what, worst), flush=True)
    assert not np.any(bad), "%s: worst err/fro = %.3g" % (what, worst)
    assert worst <= GUARD, "%s: worst err/fro %.3g above the regression guard" % (what, worst)
    return worst


def check_outputs(o_gpu, o_ref, states_ref, bf16_out):
    # states_ref [B][K][Hv][dv][dk]: the state after each token
    fro = np.linalg.norm(states_ref, axis=(-1, -2))  # [B][K][Hv]
    o = o_gpu.astype(np.float64)
    bound = TOL * fro[..., None] + (np.abs(o_ref) * 2.0 ** -8 if bf16_out else 0.0)
    err = np.abs(o - o_ref)
    assert np.all(err <= bound), "o: worst err = %.3g" % float(np.max(err / np.maximum(bound, 1e-30)))


def oracle_verify(wl, inp, qkv, raw=True, capture=True):
    dt, alog = (f64(inp["dt_bias"]), f64(inp["A_log"])) if raw else (None, None)
    return oracle.gdn_recurrent_f64(f64(qkv), f64(inp["beta_raw"]), f64(inp["alpha"]), dt, alog,
                                    f64(inp["S_in"]), wl.Hk, capture=capture)


def all_states(S_out, H):
    # [B][K][Hv][dv][dk]: H_0..H_{K-2}, then the final state
    if H is None or H.shape[1] == 0:
        return S_out[:, None]
    return np.concatenate([H, S_out[:, None]], axis=1)


# ------------------------------------------------------------------ conv step
CONV_CASES = [
    ("tiny", dict()),
    ("verify16", dict()),
    ("decode", dict()),
    ("batched", dict()),
    ("tiny", dict(T=13, B=3)),
    ("verify16", dict(T=5, B=2)),
    ("verify16", dict(T=1, B=2, W=2)),
    ("verify16", dict(T=2, B=2, W=8)),
    ("verify16", dict(T=9, B=1, W=3)),
    ("tiny", dict(Hk=1, Hv=3, dk=32, dv=40, T=7)),    # C = 184: not a multiple of 8 -> ragged tail
]


@pytest.mark.parametrize("name,over", CONV_CASES)
def test_conv_step_bit_exact(name, over):
    wl = synth.small(name, **over)
    say("conv", name, over, "C=%d" % wl.C)
    inp = synth.make_inputs(wl, seed=1)
    x, w, hist = dev(inp["x"]), dev(inp["w"]), dev(inp["hist"])
    y = torch.empty_like(x)
    win = torch.empty(wl.B, wl.W - 1 + wl.T, wl.C, dtype=x.dtype, device="cuda")
    gdn.conv_step(x, w, hist, y, win)
    torch.cuda.synchronize()
    y_ref, hist_ref, win_ref = oracle.conv_step_f32(inp["x"].float().numpy(), inp["w"].numpy(),
                                                    inp["hist"].float().numpy(), round_bf16=wl.bf16)
    yg = y.float().cpu().numpy()
    assert np.array_equal(yg.view(np.uint32), y_ref.view(np.uint32)), \
        "y mismatch at %d of %d" % (int(np.sum(yg.view(np.uint32) != y_ref.view(np.uint32))), y_ref.size)
    assert np.array_equal(hist.float().cpu().numpy().view(np.uint32), hist_ref.view(np.uint32))
    assert np.array_equal(win.float().cpu().numpy().view(np.uint32), win_ref.view(np.uint32))


def test_conv_step_without_window_and_empty_batch():
    wl = synth.small("verify16", B=2, T=3)
    say("conv no-window")
    inp = synth.make_inputs(wl, seed=2)
    x, w, hist = dev(inp["x"]), dev(inp["w"]), dev(inp["hist"])
    y = torch.empty_like(x)
    gdn.conv_step(x, w, hist, y, None)
    torch.cuda.synchronize()
    y_ref, hist_ref, _ = oracle.conv_step_f32(inp["x"].float().numpy(), inp["w"].numpy(),
                                              inp["hist"].float().numpy(), round_bf16=True)
    assert np.array_equal(y.float().cpu().numpy(), y_ref)
    assert np.array_equal(hist.float().cpu().numpy(), hist_ref)
    e = torch.empty(0, 3, wl.C, dtype=torch.bfloat16, device="cuda")
    gdn.conv_step(e, w, torch.empty(0, 3, wl.C, dtype=torch.bfloat16, device="cuda"), torch.empty_like(e), None)


# ------------------------------------------------------------------ verify
VERIFY_CASES = [
    ("tiny", dict(), {}),
    ("verify16", dict(), {}),
    ("decode", dict(), {}),
    ("batched", dict(), {}),
    ("verify16", dict(T=3, Hk=2, Hv=6), {}),
    ("verify16", dict(T=5, Hk=4, Hv=4, dk=64, dv=64), {}),
    ("verify16", dict(T=12, Hk=2, Hv=4, dk=32, dv=32), {}),
    ("verify16", dict(T=20, Hk=2, Hv=6), {}),
    ("verify16", dict(T=32, Hk=2, Hv=4), {}),
    ("verify16", dict(T=48, Hk=2, Hv=6), {}),                       # the longest windows (K <= 64)
    ("verify16", dict(T=64, Hk=2, Hv=4, dk=64, dv=64), {}),
    ("verify16", dict(T=64, Hk=1, Hv=2, dk=32, dv=32), dict(o_bf16=True)),
    ("verify16", dict(T=16, Hk=2, Hv=4, dk=64, dv=128), {}),
    ("verify16", dict(T=16, Hk=2, Hv=4, dk=128, dv=24), {}),
    ("verify16", dict(Hk=4, Hv=12), dict(weak=True)),
    ("verify16", dict(Hk=4, Hv=12), dict(o_bf16=True)),
    ("verify16", dict(Hk=4, Hv=12), dict(activated=True)),
    ("tiny", dict(T=16, B=3), dict(weak=True)),
]


@pytest.mark.parametrize("name,over,opt", VERIFY_CASES)
def test_verify_parity(name, over, opt):
    wl = synth.small(name, **over)
    say("verify", name, over, opt)
    inp = synth.make_inputs(wl, seed=3, weak_decay=opt.get("weak", False))
    if opt.get("activated"):
        # already-activated gates: beta in (0,1), g <= 0
        inp["beta_raw"] = torch.sigmoid(inp["beta_raw"].float()).to(inp["beta_raw"].dtype)
        inp["alpha"] = (-torch.nn.functional.softplus(inp["alpha"].float())).to(inp["alpha"].dtype)
    qkv = synth.make_qkv(wl, seed=3)
    o_dtype = torch.bfloat16 if opt.get("o_bf16") else torch.float32
    raw = not opt.get("activated")
    capture = wl.T > 1
    S_out, H, o, _ = run_verify_gpu(wl, inp, qkv, capture=capture, o_dtype=o_dtype, raw=raw)
    S_ref, H_ref, o_ref = oracle_verify(wl, inp, qkv, raw=raw, capture=capture)
    check_states(S_out.cpu().numpy(), S_ref, "S_out")
    if capture:
        check_states(H.cpu().numpy(), H_ref, "H")
    check_outputs(o.float().cpu().numpy(), o_ref, all_states(S_ref, H_ref), o_dtype == torch.bfloat16)


def test_verify_zero_gates_leave_state():
    """beta = 0, g = 0 (activated mode): every H_t and S_out equal S_in."""
    wl = synth.small("verify16", Hk=2, Hv=4)
    say("verify zero gates")
    inp = synth.make_inputs(wl, seed=4)
    inp["beta_raw"] = torch.zeros_like(inp["beta_raw"])
    inp["alpha"] = torch.zeros_like(inp["alpha"])
    qkv = synth.make_qkv(wl, seed=4)
    S_out, H, o, d = run_verify_gpu(wl, inp, qkv, raw=False)
    S_in = inp["S_in"].numpy()
    assert np.array_equal(S_out.cpu().numpy(), S_in)
    for t in range(wl.T - 1):
        assert np.array_equal(H[:, t].cpu().numpy(), S_in)


def test_verify_in_place_decode():
    wl = synth.WORKLOADS["decode"]
    say("verify decode in place")
    inp = synth.make_inputs(wl, seed=5)
    qkv = synth.make_qkv(wl, seed=5)
    S_out, _, o, d = run_verify_gpu(wl, inp, qkv, capture=False, S_out_inplace=True)
    S_ref, _, o_ref = oracle_verify(wl, inp, qkv, capture=False)
    assert S_out.data_ptr() == d["S_in"].data_ptr()
    check_states(S_out.cpu().numpy(), S_ref, "S_out in place")
    check_outputs(o.cpu().numpy(), o_ref, S_ref[:, None], False)


def test_verify_deterministic_and_k_invariant():
    """Two identical runs agree bit for bit; H_{j-1} of a K=16 window equals the final state of a j-window."""
    wl = synth.WORKLOADS["verify16"]
    say("verify determinism / K invariance")
    inp = synth.make_inputs(wl, seed=6)
    qkv = synth.make_qkv(wl, seed=6)
    S1, H1, o1, _ = run_verify_gpu(wl, inp, qkv)
    S2, H2, o2, _ = run_verify_gpu(wl, inp, qkv)
    assert torch.equal(S1, S2) and torch.equal(H1, H2) and torch.equal(o1, o2)
    for j in (1, 3, 8, 15):
        wj = synth.small("verify16", T=j)
        inj = dict(inp)
        inj["beta_raw"], inj["alpha"] = inp["beta_raw"][:, :j].contiguous(), inp["alpha"][:, :j].contiguous()
        Sj, _, oj, _ = run_verify_gpu(wj, inj, qkv[:, :j].contiguous(), capture=False)
        ref = H1[:, j - 1]
        err = (Sj - ref).abs().amax(dim=(-1, -2))
        fro = torch.linalg.norm(ref, dim=(-1, -2))
        assert torch.all(err <= 1e-5 * fro + 1e-30), j
        assert torch.allclose(oj, o1[:, :j], rtol=0, atol=1e-5)


# ------------------------------------------------------------------ rollback
@pytest.mark.parametrize("name", ["verify16", "batched", "tiny"])
def test_rollback_bit_exact(name):
    wl = synth.WORKLOADS[name]
    say("rollback", name)
    inp = synth.make_inputs(wl, seed=7)
    B, K = wl.B, wl.T
    acc = inp["accept"].clone()
    if B >= 3:
        acc[0], acc[1], acc[2] = 0, K, K - 1
    qkv_x, w, hist0 = dev(inp["x"]), dev(inp["w"]), dev(inp["hist"])
    hist = hist0.clone()
    y = torch.empty_like(qkv_x)
    win = torch.empty(B, wl.W - 1 + K, wl.C, dtype=qkv_x.dtype, device="cuda")
    gdn.conv_step(qkv_x, w, hist, y, win)
    S_out, H, o, d = run_verify_gpu(wl, inp, y.cpu(), capture=True)
    S_before = S_out.clone()
    hist_before = hist.clone()
    gdn.rollback(dev(acc), K, d["S_in"], H, S_out, hist, win)
    torch.cuda.synchronize()
    # the oracle's byte-copy rollback applied to the GPU's own buffers
    S_ref = S_before.cpu().numpy().copy()
    hist_ref = hist_before.cpu().view(torch.int16).numpy().copy() if wl.bf16 else hist_before.cpu().numpy().copy()
    win_np = win.cpu().view(torch.int16).numpy() if wl.bf16 else win.cpu().numpy()
    oracle.rollback(acc.numpy(), K, d["S_in"].cpu().numpy(), H.cpu().numpy(), S_ref, win=win_np, hist=hist_ref)
    assert np.array_equal(S_out.cpu().numpy(), S_ref)
    hg = hist.cpu().view(torch.int16).numpy() if wl.bf16 else hist.cpu().numpy()
    assert np.array_equal(hg, hist_ref)


# gdn_rollback_conv_step: the rollback of a previous window and the conv step of the
# next tokens in one launch; against the oracle's byte-copy rollback followed by its
# same-precision conv, bit for bit, and against the two separate GPU calls.
# (name, sizes, previous window K_prev, new tokens T)
ROLLCONV_CASES = [
    ("verify16", dict(Hk=2, Hv=6, B=3), 16, 16),
    ("tiny", dict(B=3), 4, 4),                                    # fp32
    ("verify16", dict(Hk=2, Hv=6, B=3, W=2), 16, 1),              # decode-size new window
    ("tiny", dict(Hk=1, Hv=3, dk=32, dv=40, B=3), 7, 2),          # C = 184 (ragged), T < W-1
    ("verify16", dict(Hk=2, Hv=6, B=3, W=8), 16, 3),              # T < W-1
]


@pytest.mark.parametrize("name,over,Kp,Tn", ROLLCONV_CASES)
def test_rollback_conv_step_bit_exact(name, over, Kp, Tn):
    wl = synth.small(name, T=Kp, **over)
    say("rollback+conv", name, over, "K_prev=%d T=%d C=%d" % (Kp, Tn, wl.C))
    io = torch.bfloat16 if wl.bf16 else torch.float32
    inp = synth.make_inputs(wl, seed=21)
    B, C, W = wl.B, wl.C, wl.W
    g = torch.Generator().manual_seed(22)
    acc = torch.tensor([0, Kp, Kp // 2][:B], dtype=torch.int32)
    win_prev = torch.randn(B, W - 1 + Kp, C, generator=g).to(io)
    H = torch.randn(B, Kp - 1, wl.Hv, wl.dv, wl.dk, generator=g) * 0.1 if Kp > 1 else None
    S_out0 = torch.randn(B, wl.Hv, wl.dv, wl.dk, generator=g)
    x = torch.randn(B, Tn, C, generator=g).to(io)
    hist0 = torch.randn(B, W - 1, C, generator=g).to(io)   # overwritten: only written by the call

    def bits(t):
        return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.numpy().view(np.int32)

    # oracle: byte-copy rollback, then the same-precision conv from the restored history
    S_ref = S_out0.numpy().copy()
    hist_r = bits(hist0.clone()).copy()
    oracle.rollback(acc.numpy(), Kp, inp["S_in"].numpy(), H.numpy() if H is not None else None, S_ref,
                    win=bits(win_prev), hist=hist_r)
    hist_restored = torch.from_numpy(hist_r).view(io) if wl.bf16 else torch.from_numpy(hist_r.view(np.float32))
    y_ref, hist_ref, win_ref = oracle.conv_step_f32(x.float().numpy(), inp["w"].numpy(),
                                                    hist_restored.float().numpy(), round_bf16=wl.bf16)

    d_S_in, d_H, d_w = dev(inp["S_in"]), dev(H) if H is not None else None, dev(inp["w"])
    S_out, hist = dev(S_out0), dev(hist0)
    y = torch.empty(B, Tn, C, dtype=io, device="cuda")
    win = torch.empty(B, W - 1 + Tn, C, dtype=io, device="cuda")
    gdn.rollback_conv_step(dev(acc), Kp, d_S_in, d_H, S_out, dev(win_prev), dev(x), d_w, hist, y, win)
    torch.cuda.synchronize()
    assert np.array_equal(S_out.cpu().numpy(), S_ref)
    for got, ref, what in ((y, y_ref, "y"), (hist, hist_ref, "hist"), (win, win_ref, "win")):
        assert np.array_equal(got.float().cpu().numpy().view(np.uint32), ref.view(np.uint32)), what

    # the two separate calls give the same bytes
    S2, hist2 = dev(S_out0), dev(hist0)
    y2, win2 = torch.empty_like(y), torch.empty_like(win)
    gdn.rollback(dev(acc), Kp, d_S_in, d_H, S2, hist2, dev(win_prev))
    gdn.conv_step(dev(x), d_w, hist2, y2, win2)
    torch.cuda.synchronize()
    assert torch.equal(S2, S_out) and torch.equal(y2, y) and torch.equal(win2, win) and torch.equal(hist2, hist)


def test_rollback_equals_rerun_of_accepted_prefix():
    """State after rollback(a) matches a fresh verify of the first a tokens (oracle and GPU)."""
    wl = synth.WORKLOADS["verify16"]
    say("rollback == rerun")
    inp = synth.make_inputs(wl, seed=8)
    qkv = synth.make_qkv(wl, seed=8)
    S_out, H, _, d = run_verify_gpu(wl, inp, qkv)
    for a in (0, 1, 7, 15, 16):
        S = S_out.clone()
        gdn.rollback(torch.tensor([a], dtype=torch.int32, device="cuda"), wl.T, d["S_in"], H, S)
        torch.cuda.synchronize()
        if a == 0:
            ref = inp["S_in"].double().numpy()
        else:
            ref, _, _ = oracle.gdn_recurrent_f64(f64(qkv[:, :a]), f64(inp["beta_raw"][:, :a]),
                                                 f64(inp["alpha"][:, :a]), f64(inp["dt_bias"]),
                                                 f64(inp["A_log"]), f64(inp["S_in"]), wl.Hk, capture=False)
        check_states(S.cpu().numpy(), ref, "rollback a=%d" % a)


# ------------------------------------------------------------------ ragged batches, stacked gates
SENT = 7.25  # sentinel for slots a ragged sequence must leave untouched


def test_verify_ragged_matches_per_sequence_oracle():
    """lens = [16, 1, 5, 11]: sequence b is a verify of lens[b] tokens on its own; its other slots stay."""
    wl = synth.small("verify16", Hk=2, Hv=6, B=4)
    lens = torch.tensor([16, 1, 5, 11], dtype=torch.int32)
    say("verify ragged", lens.tolist())
    inp = synth.make_inputs(wl, seed=31, weak_decay=True)
    qkv = synth.make_qkv(wl, seed=31)
    d = {k: dev(v) for k, v in inp.items()}
    B, K = wl.B, wl.T
    S_out = torch.full_like(d["S_in"], SENT)
    H = torch.full((B, K - 1, wl.Hv, wl.dv, wl.dk), SENT, device="cuda")
    o = torch.full((B, K, wl.Hv, wl.dv), SENT, device="cuda")
    gdn.verify(dev(qkv), d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], S_out, H, o, wl.Hk,
               lens=dev(lens))
    torch.cuda.synchronize()
    S_out, H, o = S_out.cpu().numpy(), H.cpu().numpy(), o.cpu().numpy()
    for b, L in enumerate(lens.tolist()):
        S_ref, H_ref, o_ref = oracle.gdn_recurrent_f64(f64(qkv[b:b + 1, :L]), f64(inp["beta_raw"][b:b + 1, :L]),
                                                       f64(inp["alpha"][b:b + 1, :L]), f64(inp["dt_bias"]),
                                                       f64(inp["A_log"]), f64(inp["S_in"][b:b + 1]), wl.Hk)
        check_states(S_out[b:b + 1], S_ref, "ragged S_out b=%d" % b)
        if L > 1:
            check_states(H[b:b + 1, :L - 1], H_ref, "ragged H b=%d" % b)
        assert np.all(H[b, max(L - 1, 0):] == SENT), "b=%d: H slots past the window were written" % b
        states = all_states(S_ref, H_ref)
        check_outputs(o[b:b + 1, :L], o_ref, states, False)
        assert np.all(o[b, L:] == SENT), "b=%d: o slots past the window were written" % b


def test_verify_stacked_gates_equal_separate_buffers():
    """beta|alpha read out of one [B][K][2Hv] row (gate_stride = 2 Hv): same bytes as separate buffers."""
    wl = synth.small("verify16", Hk=2, Hv=6, B=2)
    say("verify stacked gates")
    inp = synth.make_inputs(wl, seed=32)
    qkv = dev(synth.make_qkv(wl, seed=32))
    d = {k: dev(v) for k, v in inp.items()}
    stacked = torch.cat([d["beta_raw"], d["alpha"]], dim=-1).contiguous()   # [B][K][2 Hv]
    outs = []
    for gates in ((d["beta_raw"], d["alpha"], None), (stacked[..., :wl.Hv], stacked[..., wl.Hv:], 2 * wl.Hv)):
        S_out = torch.empty_like(d["S_in"])
        H = torch.empty(wl.B, wl.T - 1, wl.Hv, wl.dv, wl.dk, device="cuda")
        o = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, device="cuda")
        gdn.verify(qkv, gates[0], gates[1], d["dt_bias"], d["A_log"], d["S_in"], S_out, H, o, wl.Hk,
                   gate_stride=gates[2])
        outs.append((S_out, H, o))
    torch.cuda.synchronize()
    for a_, b_ in zip(outs[0], outs[1]):
        assert torch.equal(a_, b_)
    S_ref, H_ref, o_ref = oracle_verify(wl, inp, qkv.cpu())
    check_states(outs[1][0].cpu().numpy(), S_ref, "stacked S_out")


def test_conv_and_rollback_ragged_match_oracle():
    """Ragged conv step (history = window rows lens[b]..) and ragged rollback (a == lens[b] keeps the state)."""
    wl = synth.small("verify16", Hk=2, Hv=6, B=4)
    lens = torch.tensor([16, 1, 5, 11], dtype=torch.int32)
    acc = torch.tensor([3, 1, 0, 11], dtype=torch.int32)     # a < len, a == len, a == 0, a == len
    say("conv + rollback ragged", lens.tolist(), acc.tolist())
    inp = synth.make_inputs(wl, seed=33)
    B, K, C, W = wl.B, wl.T, wl.C, wl.W
    x, w, hist = dev(inp["x"]), dev(inp["w"]), dev(inp["hist"])
    y = torch.empty_like(x)
    win = torch.empty(B, W - 1 + K, C, dtype=x.dtype, device="cuda")
    gdn.conv_step(x, w, hist, y, win, lens=dev(lens))
    torch.cuda.synchronize()
    for b, L in enumerate(lens.tolist()):
        y_ref, hist_ref, win_ref = oracle.conv_step_f32(inp["x"][b:b + 1, :L].float().numpy(), inp["w"].numpy(),
                                                        inp["hist"][b:b + 1].float().numpy(), round_bf16=True)
        assert np.array_equal(y[b:b + 1, :L].float().cpu().numpy(), y_ref)
        assert np.array_equal(hist[b:b + 1].float().cpu().numpy(), hist_ref)
        assert np.array_equal(win[b:b + 1, :W - 1 + L].float().cpu().numpy(), win_ref)
    # verify on the conv output, then roll back
    d = {k: dev(v) for k, v in inp.items()}
    S_out = torch.empty_like(d["S_in"])
    H = torch.empty(B, K - 1, wl.Hv, wl.dv, wl.dk, device="cuda")
    o = torch.empty(B, K, wl.Hv, wl.dv, device="cuda")
    gdn.verify(y, d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], S_out, H, o, wl.Hk,
               lens=dev(lens))
    torch.cuda.synchronize()
    S_before, H_np, win_np = S_out.cpu().numpy().copy(), H.cpu().numpy(), win.cpu().view(torch.int16).numpy()
    hist_before = hist.cpu().view(torch.int16).numpy().copy()
    gdn.rollback(dev(acc), K, d["S_in"], H, S_out, hist, win, lens=dev(lens))
    torch.cuda.synchronize()
    S_in_np = inp["S_in"].numpy()
    for b, L in enumerate(lens.tolist()):
        S_ref = S_before[b:b + 1].copy()
        hist_ref = hist_before[b:b + 1].copy()
        oracle.rollback(acc[b:b + 1].numpy(), L, S_in_np[b:b + 1], np.ascontiguousarray(H_np[b:b + 1, :max(L - 1, 0)]),
                        S_ref, win=np.ascontiguousarray(win_np[b:b + 1, :W - 1 + L]), hist=hist_ref)
        assert np.array_equal(S_out[b:b + 1].cpu().numpy(), S_ref), "rollback b=%d" % b
        assert np.array_equal(hist[b:b + 1].cpu().view(torch.int16).numpy(), hist_ref), "hist b=%d" % b


def test_replay_matches_oracle_and_capture_rollback():
    """Checkpoint + replay: verify without capture, then rebuild the accepted prefix from the checkpoint."""
    wl = synth.small("verify16", Hk=2, Hv=6, B=4)
    acc = torch.tensor([0, 16, 5, 11], dtype=torch.int32)
    say("replay", acc.tolist())
    inp = synth.make_inputs(wl, seed=34, weak_decay=True)
    B, K, C, W = wl.B, wl.T, wl.C, wl.W
    d = {k: dev(v) for k, v in inp.items()}
    x, w = d["x"], d["w"]
    y = torch.empty_like(x)
    win = torch.empty(B, W - 1 + K, C, dtype=x.dtype, device="cuda")
    hist_c = d["hist"].clone()
    gdn.conv_step(x, w, hist_c, y, win)
    # capture path
    S_cap = torch.empty_like(d["S_in"])
    H = torch.empty(B, K - 1, wl.Hv, wl.dv, wl.dk, device="cuda")
    o = torch.empty(B, K, wl.Hv, wl.dv, device="cuda")
    gdn.verify(y, d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], S_cap, H, o, wl.Hk)
    hist_cap = hist_c.clone()
    gdn.rollback(dev(acc), K, d["S_in"], H, S_cap, hist_cap, win)
    # checkpoint + replay path
    S_rep = torch.empty_like(d["S_in"])
    gdn.verify(y, d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], S_rep, None, o, wl.Hk)
    torch.cuda.synchronize()
    S_final = S_rep.clone()
    hist_rep = hist_c.clone()
    gdn.replay(dev(acc), y, d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], S_rep, wl.Hk,
               hist=hist_rep, win=win)
    torch.cuda.synchronize()
    assert torch.equal(hist_rep, hist_cap)
    assert torch.equal(S_rep[0], d["S_in"][0])          # a = 0: the checkpoint
    assert torch.equal(S_rep[1], S_final[1])            # a = K: untouched
    yc = y.cpu()
    for b, a in enumerate(acc.tolist()):
        if 0 < a < K:
            S_ref, _, _ = oracle.gdn_recurrent_f64(f64(yc[b:b + 1, :a]), f64(inp["beta_raw"][b:b + 1, :a]),
                                                   f64(inp["alpha"][b:b + 1, :a]), f64(inp["dt_bias"]),
                                                   f64(inp["A_log"]), f64(inp["S_in"][b:b + 1]), wl.Hk, capture=False)
            check_states(S_rep[b:b + 1].cpu().numpy(), S_ref, "replay b=%d" % b)
            check_states(S_cap[b:b + 1].cpu().numpy(), S_ref, "capture b=%d" % b)


# ------------------------------------------------------------------ prefill
PREFILL_CASES = [
    ("tiny", dict(T=100), 64),
    ("tiny", dict(T=37, B=2), 16),
    ("tiny", dict(T=70, B=2, dk=64, dv=64), 32),
    ("prefill", dict(B=1, T=130, Hk=2, Hv=6), 64),
    ("prefill", dict(B=2, T=200, Hk=1, Hv=3, dk=64, dv=64), 64),
]


def oracle_segments(qkv, br, al, dt, alog, S_in, Hk, seg=64):
    """The oracle over a long window in segments of `seg` tokens (state chained).

    Returns the final state, every o_t and the Frobenius norm of the state after
    every token, [B][T][Hv]."""
    T = qkv.shape[1]
    S = S_in
    os_, norms = [], []
    for t0 in range(0, T, seg):
        t1 = min(T, t0 + seg)
        S_new, H, o = oracle.gdn_recurrent_f64(qkv[:, t0:t1], br[:, t0:t1], al[:, t0:t1], dt, alog, S, Hk)
        norms.append(np.linalg.norm(all_states(S_new, H), axis=(-1, -2)))
        os_.append(o)
        S = S_new
    return S, np.concatenate(os_, axis=1), np.concatenate(norms, axis=1)


@pytest.mark.parametrize("name,over,chunk", PREFILL_CASES)
def test_prefill_parity(name, over, chunk):
    wl = synth.small(name, **over)
    say("prefill", name, over, chunk)
    inp = synth.make_inputs(wl, seed=9)
    qkv = synth.make_qkv(wl, seed=9)
    d = {k: dev(v) for k, v in inp.items()}
    S_out = torch.empty_like(d["S_in"])
    o = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, device="cuda")
    gdn.prefill_chunked(dev(qkv), d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], S_out, o,
                        wl.Hk, chunk=chunk)
    torch.cuda.synchronize()
    S_ref, o_ref, norms = oracle_segments(f64(qkv), f64(inp["beta_raw"]), f64(inp["alpha"]), f64(inp["dt_bias"]),
                                          f64(inp["A_log"]), f64(inp["S_in"]), wl.Hk)
    check_states(S_out.cpu().numpy(), S_ref, "prefill S_out")
    err = np.abs(o.cpu().numpy() - o_ref)
    assert np.all(err <= TOL * norms[..., None])


# bf16 slabs run the chunkwise WY kernel on MFMA.  These cases cover its tiling:
# every chunk length, exactly one chunk, T < chunk, ragged last chunks, dk of
# 32/64/128, dv that leaves part of the 64-row workgroup empty, the state
# updated in place, bf16 outputs, activated gates, and weak decay (the initial
# state still matters after hundreds of tokens).
WY_CASES = [
    (dict(B=1, T=64, Hk=1, Hv=2), 64, dict()),
    (dict(B=2, T=77, Hk=2, Hv=4, dk=32, dv=32), 16, dict(weak=True)),
    (dict(B=1, T=100, Hk=1, Hv=3, dk=64, dv=40), 32, dict(weak=True, inplace=True, o_bf16=True)),
    (dict(B=1, T=5, Hk=2, Hv=2), 64, dict(activated=True)),
    (dict(B=1, T=300, Hk=1, Hv=1), 64, dict(weak=True)),
    (dict(B=1, T=129, Hk=1, Hv=2), 32, dict(weak=True, o_bf16=True)),
    (dict(B=1, T=47, Hk=1, Hv=2), 16, dict()),
    (dict(B=3, T=96, Hk=2, Hv=2, dk=64, dv=64), 64, dict(activated=True, weak=True)),
    # dk = 128 with chunks of 64 (32-row state waves): rows past dv inside a wave and whole waves
    # past it, two row blocks per head, one token, a one-token last chunk
    (dict(B=1, T=200, Hk=1, Hv=2, dv=48), 64, dict(weak=True)),
    (dict(B=2, T=150, Hk=1, Hv=1, dv=160), 64, dict(o_bf16=True, inplace=True)),
    (dict(B=1, T=1, Hk=1, Hv=1), 64, dict()),
    (dict(B=1, T=65, Hk=2, Hv=4), 64, dict(activated=True)),
]


@pytest.mark.parametrize("over,chunk,opt", WY_CASES)
def test_prefill_wy_parity(over, chunk, opt):
    wl = synth.small("prefill", **over)
    say("prefill wy", over, chunk, opt)
    inp = synth.make_inputs(wl, seed=11, weak_decay=opt.get("weak", False))
    raw = not opt.get("activated")
    if not raw:
        inp["beta_raw"] = torch.sigmoid(inp["beta_raw"].float()).to(inp["beta_raw"].dtype)
        inp["alpha"] = (-torch.nn.functional.softplus(inp["alpha"].float())).to(inp["alpha"].dtype)
    qkv = synth.make_qkv(wl, seed=11)
    S_in_ref = f64(inp["S_in"])
    d = {k: dev(v) for k, v in inp.items()}
    S_out = d["S_in"] if opt.get("inplace") else torch.empty_like(d["S_in"])
    o_bf16 = opt.get("o_bf16", False)
    o = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, device="cuda", dtype=torch.bfloat16 if o_bf16 else torch.float32)
    dt, alog = (d["dt_bias"], d["A_log"]) if raw else (None, None)
    gdn.prefill_chunked(dev(qkv), d["beta_raw"], d["alpha"], dt, alog, d["S_in"], S_out, o, wl.Hk, chunk=chunk)
    torch.cuda.synchronize()
    dt_r, alog_r = (f64(inp["dt_bias"]), f64(inp["A_log"])) if raw else (None, None)
    S_ref, o_ref, norms = oracle_segments(f64(qkv), f64(inp["beta_raw"]), f64(inp["alpha"]), dt_r, alog_r,
                                          S_in_ref, wl.Hk)
    check_states(S_out.cpu().numpy(), S_ref, "prefill S_out")
    err = np.abs(o.float().cpu().numpy() - o_ref)
    bound = TOL * norms[..., None] + (np.abs(o_ref) * 2.0 ** -8 if o_bf16 else 0.0)
    assert np.all(err <= bound), "o: worst err/bound = %.3g" % float(np.max(err / np.maximum(bound, 1e-30)))


def test_prefill_full_size_sampled_heads():
    """B=4 x T=4096, 48 value heads, d=128: six (sequence, head) pairs re-run on the oracle."""
    wl = synth.WORKLOADS["prefill"]
    say("prefill full size, sampled heads")
    inp = synth.make_inputs(wl, seed=10)
    qkv = synth.make_qkv(wl, seed=10)
    d = {k: dev(v) for k, v in inp.items()}
    S_out = torch.empty_like(d["S_in"])
    o = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, device="cuda", dtype=torch.bfloat16)
    gdn.prefill_chunked(dev(qkv), d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], S_out, o,
                        wl.Hk, chunk=64)
    torch.cuda.synchronize()
    S_out = S_out.cpu().numpy()
    o = o.float().cpu().numpy()
    grp = wl.Hv // wl.Hk
    for b, h in [(0, 0), (0, 47), (1, 17), (2, 30), (3, 5), (3, 46)]:
        hk = h // grp
        q = qkv[b:b + 1, :, hk * wl.dk:(hk + 1) * wl.dk]
        k = qkv[b:b + 1, :, wl.Hk * wl.dk + hk * wl.dk: wl.Hk * wl.dk + (hk + 1) * wl.dk]
        v = qkv[b:b + 1, :, 2 * wl.Hk * wl.dk + h * wl.dv: 2 * wl.Hk * wl.dk + (h + 1) * wl.dv]
        sub = torch.cat([q, k, v], dim=-1)
        S_ref, o_ref, norms = oracle_segments(
            f64(sub), f64(inp["beta_raw"][b:b + 1, :, h:h + 1]), f64(inp["alpha"][b:b + 1, :, h:h + 1]),
            f64(inp["dt_bias"][h:h + 1]), f64(inp["A_log"][h:h + 1]), f64(inp["S_in"][b:b + 1, h:h + 1]), 1)
        check_states(S_out[b:b + 1, h:h + 1], S_ref, "prefill b=%d h=%d" % (b, h))
        err = np.abs(o[b, :, h] - o_ref[0, :, 0])
        assert np.all(err <= TOL * norms[0, :, 0][:, None] + np.abs(o_ref[0, :, 0]) * 2.0 ** -8)


# ------------------------------------------------------------------ the whole step
def test_full_step_verify16_end_to_end():
    """conv -> verify -> rollback on the K=16 workload against the oracle's chain."""
    wl = synth.WORKLOADS["verify16"]
    say("end-to-end verify16")
    inp = synth.make_inputs(wl, seed=0)
    d = {k: dev(v) for k, v in inp.items()}
    hist = d["hist"].clone()
    y = torch.empty_like(d["x"])
    win = torch.empty(wl.B, wl.W - 1 + wl.T, wl.C, dtype=torch.bfloat16, device="cuda")
    S_out = torch.empty_like(d["S_in"])
    H = torch.empty(wl.B, wl.T - 1, wl.Hv, wl.dv, wl.dk, device="cuda")
    o = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, device="cuda")
    gdn.conv_step(d["x"], d["w"], hist, y, win)
    gdn.verify(y, d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], S_out, H, o, wl.Hk)
    gdn.rollback(d["accept"], wl.T, d["S_in"], H, S_out, hist, win)
    torch.cuda.synchronize()
    a = int(inp["accept"][0])
    say("accept length", a)
    y_ref, hist_full, win_ref = oracle.conv_step_f32(inp["x"].float().numpy(), inp["w"].numpy(),
                                                     inp["hist"].float().numpy(), round_bf16=True)
    assert np.array_equal(y.float().cpu().numpy(), y_ref)
    S_ref, H_ref, o_ref = oracle.gdn_recurrent_f64(y_ref.astype(np.float64), f64(inp["beta_raw"]),
                                                   f64(inp["alpha"]), f64(inp["dt_bias"]), f64(inp["A_log"]),
                                                   f64(inp["S_in"]), wl.Hk)
    check_outputs(o.cpu().numpy(), o_ref, all_states(S_ref, H_ref), False)
    states = np.concatenate([f64(inp["S_in"])[:, None], all_states(S_ref, H_ref)], axis=1)
    check_states(S_out.cpu().numpy(), states[:, a], "state after rollback to %d" % a)
    assert np.array_equal(hist.float().cpu().numpy(), win_ref[:, a:a + wl.W - 1])
