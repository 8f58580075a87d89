"""GPU: the debug build's count of clamped accept lengths (libgdn_debug.so,
gdn_debug_clamped_accepts).

Accept lengths outside 0..K are clamped by every kernel that reads one; the
debug build counts each such sequence once per call.  The calls here run the
debug library (gdn.using), check the count after each one, and check that the
debug build's outputs are the release build's, bit for bit.  Every test prints
its case before touching the device.
"""
import pytest
import torch

from speculative_verify_gdn_amd import gdn, synth

pytestmark = pytest.mark.gpu

WILD = [-3, 99, 5, 8]          # at K = 8: the first two are out of range
TAME = [0, 8, 5, 8]            # what they clamp to


def say(*a):
    print("[gpu case]", *a, flush=True)


@pytest.fixture(scope="module")
def dbg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load()
    # built with the release library by the package build (build() of the entry module)
    return gdn.open_library(gdn.DEBUG_LIB_PATH)


def dev(t):
    return t.contiguous().cuda()


def outputs(wl):
    B, K, Hv, dv, dk, C, W = wl.B, wl.T, wl.Hv, wl.dv, wl.dk, wl.C, wl.W
    return dict(S_ckpt=torch.empty(B, Hv, dv, dk, device="cuda"), S_out=torch.empty(B, Hv, dv, dk, device="cuda"),
                H=torch.empty(B, K - 1, Hv, dv, dk, device="cuda"),
                o=torch.empty(B, K, Hv, dv, device="cuda", dtype=torch.bfloat16),
                y=torch.empty(B, K, C, device="cuda", dtype=torch.bfloat16),
                win=torch.empty(B, W - 1 + K, C, device="cuda", dtype=torch.bfloat16))


def step(wl, d, out, prev=None):
    gdn.verify_step(d["x"], d["w"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], out["S_out"], out["H"],
                    out["o"], wl.Hk, prev=prev, S_in=None if prev else d["S_in"], hist=None if prev else d["hist"],
                    S_ckpt=out["S_ckpt"], y=out["y"], win=out["win"])


def count():
    torch.cuda.synchronize()
    return gdn.debug_clamped_accepts()


@pytest.mark.parametrize("Hv", [6, 4])   # three value heads per key head (the step kernel), two (verify kernel)
def test_clamped_accepts_are_counted(dbg, Hv):
    wl = synth.small("verify16", B=4, Hk=2, Hv=Hv, T=8)
    say("clamp count", "Hv", Hv, "accept", WILD)
    d1 = {k: dev(v) for k, v in synth.make_inputs(wl, seed=91).items()}
    d2 = {k: dev(v) for k, v in synth.make_inputs(wl, seed=92).items()}
    d2["w"] = d1["w"]
    wild = torch.tensor(WILD, dtype=torch.int32, device="cuda")
    tame = torch.tensor(TAME, dtype=torch.int32, device="cuda")
    n_out = sum(1 for a in WILD if a < 0 or a > wl.T)

    # the release build's results of the same calls
    A_rel, B_rel = outputs(wl), outputs(wl)
    step(wl, d1, A_rel)
    step(wl, d2, B_rel, prev=(wild, A_rel["S_ckpt"], A_rel["H"], A_rel["S_out"], A_rel["win"]))

    with gdn.using(dbg):
        gdn.debug_clamped_accepts(reset=True)
        assert count() == 0
        A = outputs(wl)
        step(wl, d1, A)                                   # first window: no accept lengths
        assert count() == 0
        Bw, Bt = outputs(wl), outputs(wl)
        step(wl, d2, Bw, prev=(wild, A["S_ckpt"], A["H"], A["S_out"], A["win"]))
        assert count() == n_out
        step(wl, d2, Bt, prev=(tame, A["S_ckpt"], A["H"], A["S_out"], A["win"]))
        assert count() == n_out                           # in range: nothing counted
        for k in Bw:
            assert torch.equal(Bw[k], B_rel[k]), "debug build differs from the release build: %s" % k
            assert torch.equal(Bw[k], Bt[k]), "wild accept lengths differ from their clamped values: %s" % k

        # gdn_rollback
        S = A["S_out"].clone()
        hist = d1["hist"].clone()
        gdn.rollback(wild, wl.T, A["S_ckpt"], A["H"], S, hist, A["win"])
        assert count() == 2 * n_out
        # gdn_rollback_conv_step
        S = A["S_out"].clone()
        hist = torch.empty_like(d1["hist"])
        y, win = torch.empty_like(d2["x"]), torch.empty_like(A["win"])
        gdn.rollback_conv_step(wild, wl.T, A["S_ckpt"], A["H"], S, A["win"], d2["x"], d1["w"], hist, y, win)
        assert count() == 3 * n_out
        # gdn_replay (the verify kernel's replay mode counts; its conv-row launch does not count again)
        S = torch.empty_like(A["S_out"])
        hist = torch.empty_like(d1["hist"])
        gdn.replay(wild, A["y"], d1["beta_raw"], d1["alpha"], d1["dt_bias"], d1["A_log"], A["S_ckpt"], S, wl.Hk,
                   hist=hist, win=A["win"])
        assert count() == 4 * n_out
        # reset: the count is returned, then zero
        assert gdn.debug_clamped_accepts(reset=True) == 4 * n_out
        assert count() == 0
