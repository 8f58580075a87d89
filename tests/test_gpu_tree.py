"""GPU parity of the tree verify calls (gdn_conv_tree, gdn_verify_tree,
gdn_rollback_tree) against the CPU oracle.

Bars as for the chain path: the conv bit for bit against the oracle's
same-precision conv over the node's path window; every node's state within
2e-3 * ||S_ref||_F per head, o within 2e-3 * ||S_node||_F (plus half a bf16 ulp
for bf16 o); the rollback a byte copy.  Trees are seeded (synth.make_tree):
chain, star, random (parent among the 4 previous nodes), forest (roots mixed
in) and binary (breadth-first numbering, parents far back).  Every test prints its case before touching the device.
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


def bits(t):
    t = t.cpu().contiguous()
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.view(torch.int32).numpy()


def check_states(gpu, ref, what):
    err = np.abs(gpu.astype(np.float64) - ref).max(axis=(-1, -2))
    fro = np.linalg.norm(ref, axis=(-1, -2))
    worst = float(np.max(err / np.maximum(fro, 1e-30)))
    print("[parity] %s worst err/fro %.3g" % (what, worst), flush=True)
    assert np.all(err <= TOL * fro), "%s: worst err/fro = %.3g" % (what, worst)
    assert worst <= GUARD, "%s: worst err/fro %.3g above the regression guard" % (what, worst)
    return worst


def check_outputs(o_gpu, o_ref, H_ref, bf16_out):
    fro = np.linalg.norm(H_ref, axis=(-1, -2))  # [B][N][Hv]
    bound = TOL * fro[..., None] + (np.abs(o_ref) * 2.0 ** -8 if bf16_out else 0.0)
    err = np.abs(o_gpu.astype(np.float64) - o_ref)
    assert np.all(err <= bound), "o: worst err/bound = %.3g" % float(np.max(err / np.maximum(bound, 1e-30)))


# ------------------------------------------------------------------ conv
CONV_CASES = [
    ("verify16", dict(T=16, B=2), "random"),
    ("verify16", dict(T=32, B=1), "forest"),
    ("verify16", dict(T=9, B=2, W=2), "random"),
    ("verify16", dict(T=7, B=2, W=8), "forest"),
    ("verify16", dict(T=16, B=1), "chain"),
    ("verify16", dict(T=5, B=3), "star"),
    ("tiny", dict(T=12, B=2), "random"),                         # fp32
    ("tiny", dict(Hk=1, Hv=3, dk=32, dv=40, T=11), "forest"),    # C = 184: ragged channel tail
    ("verify16", dict(T=1, B=2), "random"),
]


@pytest.mark.parametrize("name,over,shape", CONV_CASES)
def test_conv_tree_bit_exact(name, over, shape):
    wl = synth.small(name, **over)
    say("conv_tree", name, over, shape, "C=%d" % wl.C)
    inp = synth.make_inputs(wl, seed=3)
    par = synth.make_tree(wl.B, wl.T, seed=4, shape=shape)
    x, w, hist = dev(inp["x"]), dev(inp["w"]), dev(inp["hist"])
    hist0 = hist.clone()
    y = torch.empty_like(x)
    gdn.conv_tree(x, w, hist, dev(par), y)
    torch.cuda.synchronize()
    y_ref = oracle.conv_tree_f32(inp["x"].float().numpy(), inp["w"].numpy(), inp["hist"].float().numpy(),
                                 par.numpy(), wl.bf16)
    y_ref_t = torch.from_numpy(y_ref).to(inp["x"].dtype)
    assert np.array_equal(bits(y), bits(y_ref_t))
    assert torch.equal(hist, hist0), "gdn_conv_tree must not write the history"


def test_conv_tree_chain_equals_conv_step():
    wl = synth.small("verify16", T=16, B=2)
    say("conv_tree chain == conv_step", "C=%d" % wl.C)
    inp = synth.make_inputs(wl, seed=5)
    x, w = dev(inp["x"]), dev(inp["w"])
    y1, y2 = torch.empty_like(x), torch.empty_like(x)
    gdn.conv_tree(x, w, dev(inp["hist"]), dev(synth.make_tree(wl.B, wl.T, shape="chain")), y1)
    gdn.conv_step(x, w, dev(inp["hist"]), y2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


# ------------------------------------------------------------------ GDN
VERIFY_CASES = [
    # (workload, overrides, tree shape, o dtype)
    ("verify16", dict(B=2, Hk=4, Hv=12), "random", torch.float32),
    ("verify16", dict(B=1, T=32, Hk=4, Hv=12), "forest", torch.float32),
    ("verify16", dict(B=2, T=16, Hk=2, Hv=6), "star", torch.bfloat16),
    ("verify16", dict(B=3, T=7, Hk=2, Hv=6, dk=64, dv=64), "forest", torch.float32),
    ("verify16", dict(B=2, T=16, Hk=2, Hv=4, dk=32, dv=32), "random", torch.float32),   # more tokens than lanes per row
    ("verify16", dict(B=1, T=24, Hk=2, Hv=4, dk=64, dv=48), "random", torch.float32),   # dv not a tile multiple
    ("verify16", dict(B=2, T=32, Hk=4, Hv=12), "binary", torch.float32),                # parents far back
    ("verify16", dict(B=1, T=15, Hk=2, Hv=4, dk=32, dv=32), "binary", torch.bfloat16),
    ("tiny", dict(T=9), "forest", torch.float32),                                       # fp32 inputs
    ("verify16", dict(B=2, T=1, Hk=2, Hv=6), "random", torch.float32),
    # the bench's shapes: the full verify16 layer (B=1, 16 key heads, 48 value heads, d=128)
    ("verify16", dict(), "random", torch.bfloat16),                                     # N=16 random
    ("verify16", dict(T=32), "binary", torch.float32),                                  # N=32 binary
]


def _tree_case(wl, shape, seed):
    inp = synth.make_inputs(wl, seed=seed)
    qkv = synth.make_qkv(wl, seed=seed)
    par = synth.make_tree(wl.B, wl.T, seed=seed, shape=shape)
    return inp, qkv, par


def _verify_tree_gpu(wl, inp, qkv, par, o_dtype=torch.float32):
    d = {k: dev(v) for k, v in inp.items()}
    H = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, wl.dk, device="cuda")
    o = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, device="cuda", dtype=o_dtype)
    gdn.verify_tree(dev(qkv), d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], dev(par), d["S_in"], H, o,
                    wl.Hk)
    torch.cuda.synchronize()
    return H, o


@pytest.mark.parametrize("name,over,shape,o_dtype", VERIFY_CASES)
def test_verify_tree_matches_oracle(name, over, shape, o_dtype):
    wl = synth.small(name, **over)
    say("verify_tree", name, over, shape, o_dtype)
    inp, qkv, par = _tree_case(wl, shape, seed=11)
    H, o = _verify_tree_gpu(wl, inp, qkv, par, o_dtype)
    H_ref, o_ref = oracle.gdn_tree_f64(f64(qkv), f64(inp["beta_raw"]), f64(inp["alpha"]), f64(inp["dt_bias"]),
                                       f64(inp["A_log"]), par.numpy(), f64(inp["S_in"]), wl.Hk)
    worst = check_states(H.cpu().numpy(), H_ref, "H")
    check_outputs(o.float().cpu().numpy(), o_ref, H_ref, o_dtype == torch.bfloat16)
    say("worst state err/fro %.3g" % worst)


def test_verify_tree_chain_outputs_match_chain_verify():
    # a chain-shaped tree and the chain verify evaluate one recurrence in two orders (the
    # tree's WY form with ancestor masks, the chain's token recurrence): every state and
    # output agree to well inside the parity bar (2e-4 of the state's Frobenius norm)
    wl = synth.small("verify16", B=2, Hk=4, Hv=12)
    say("verify_tree chain ~ verify", wl)
    inp, qkv, par = _tree_case(wl, "chain", seed=12)
    H, o = _verify_tree_gpu(wl, inp, qkv, par)
    d = {k: dev(v) for k, v in inp.items()}
    S_out = torch.empty_like(d["S_in"])
    Hc = torch.empty(wl.B, wl.T - 1, wl.Hv, wl.dv, wl.dk, device="cuda")
    oc = torch.empty_like(o)
    gdn.verify(dev(qkv), d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], S_out, Hc, oc, wl.Hk)
    torch.cuda.synchronize()
    Hch = torch.cat([Hc, S_out[:, None]], dim=1).double().cpu()
    fro = torch.linalg.norm(Hch, dim=(-1, -2))
    err = (H.double().cpu() - Hch).abs().amax(dim=(-1, -2))
    assert bool((err <= 2e-4 * fro).all()), float((err / fro).max())
    # o_t[i] is row i of H_t against a unit vector: bounded by the state's norm
    oerr = (o.double().cpu() - oc.double().cpu()).abs().amax(dim=-1)
    assert bool((oerr <= 2e-4 * fro).all()), float((oerr / fro).max())


def test_verify_tree_stacked_gates_and_bad_parents():
    # beta|alpha read from one stacked row; parent entries outside [0, i) act as roots
    wl = synth.small("verify16", B=2, T=8, Hk=2, Hv=6)
    say("verify_tree stacked gates, out-of-range parents")
    inp, qkv, _ = _tree_case(wl, "random", seed=13)
    bad = torch.tensor([[5, 0, 2, -7, 3, 100, 1, 6], [-1, 0, 0, 1, -2, 4, 9, 2]], dtype=torch.int32)
    good = torch.tensor([[-1, 0, -1, -1, 3, -1, 1, 6], [-1, 0, 0, 1, -1, 4, -1, 2]], dtype=torch.int32)
    d = {k: dev(v) for k, v in inp.items()}
    stacked = torch.cat([d["beta_raw"], d["alpha"]], dim=-1).contiguous()
    H1 = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, wl.dk, device="cuda")
    o1 = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, device="cuda")
    gdn.verify_tree(dev(qkv), stacked[..., :wl.Hv], stacked[..., wl.Hv:], d["dt_bias"], d["A_log"], dev(bad),
                    d["S_in"], H1, o1, wl.Hk, gate_stride=2 * wl.Hv)
    H2, o2 = _verify_tree_gpu(wl, inp, qkv, good)
    assert torch.equal(H1, H2) and torch.equal(o1, o2)


# ------------------------------------------------------------------ rollback
@pytest.mark.parametrize("bf16,W", [(True, 4), (False, 4), (True, 2), (True, 8)])
def test_rollback_tree_bit_exact(bf16, W):
    B, N, Hv, dv, dk, C = 4, 12, 3, 16, 32, 200
    say("rollback_tree", bf16, W)
    g = torch.Generator().manual_seed(21)
    io = torch.bfloat16 if bf16 else torch.float32
    S_in = torch.randn(B, Hv, dv, dk, generator=g)
    H = torch.randn(B, N, Hv, dv, dk, generator=g)
    x = torch.randn(B, N, C, generator=g).to(io)
    hist = torch.randn(B, W - 1, C, generator=g).to(io)
    par = synth.make_tree(B, N, seed=6, shape="forest")
    node = torch.tensor([-1, 0, 7, N - 1], dtype=torch.int32)
    S_out = torch.zeros_like(S_in)
    d_S_out, d_hist = dev(S_out), dev(hist)
    gdn.rollback_tree(dev(node), dev(par), dev(S_in), dev(H), d_S_out, dev(x), d_hist)
    torch.cuda.synchronize()
    ref_S = S_out.numpy().copy()
    ref_hist = (hist.view(torch.int16) if bf16 else hist).numpy().copy()
    xs = (x.view(torch.int16) if bf16 else x).numpy()
    oracle.tree_rollback(node.numpy(), par.numpy(), S_in.numpy(), H.numpy(), ref_S, x=xs, hist=ref_hist)
    assert np.array_equal(bits(d_S_out), ref_S.view(np.int32))
    assert np.array_equal(bits(d_hist), ref_hist.view(np.int16) if bf16 else ref_hist.view(np.int32))


# ------------------------------------------------------------------ the whole tree step
def test_tree_step_conv_verify_rollback_against_oracle():
    wl = synth.small("verify16", B=2, T=16, Hk=4, Hv=12)
    say("tree step conv -> verify -> rollback", wl)
    inp = synth.make_inputs(wl, seed=31)
    par = synth.make_tree(wl.B, wl.T, seed=31, shape="random")
    node = torch.tensor([9, -1], dtype=torch.int32)
    d = {k: dev(v) for k, v in inp.items()}
    y = torch.empty_like(d["x"])
    gdn.conv_tree(d["x"], d["w"], d["hist"], dev(par), y)
    H = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, wl.dk, device="cuda")
    o = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, device="cuda")
    gdn.verify_tree(y, d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], dev(par), d["S_in"], H, o, wl.Hk)
    S_out = torch.empty_like(d["S_in"])
    gdn.rollback_tree(dev(node), dev(par), d["S_in"], H, S_out, d["x"], d["hist"])
    torch.cuda.synchronize()

    y_ref = oracle.conv_tree_f32(inp["x"].float().numpy(), inp["w"].numpy(), inp["hist"].float().numpy(),
                                 par.numpy(), True)
    y_ref_bf = torch.from_numpy(y_ref).to(torch.bfloat16)
    assert torch.equal(y.cpu(), y_ref_bf)
    H_ref, o_ref = oracle.gdn_tree_f64(f64(y_ref_bf), f64(inp["beta_raw"]), f64(inp["alpha"]), f64(inp["dt_bias"]),
                                       f64(inp["A_log"]), par.numpy(), f64(inp["S_in"]), wl.Hk)
    check_outputs(o.cpu().numpy(), o_ref, H_ref, False)
    S_ref = np.stack([H_ref[0, 9], f64(inp["S_in"])[1]])
    check_states(S_out.cpu().numpy(), S_ref, "S_out")
    hist_ref = inp["hist"].view(torch.int16).numpy().copy()
    S_dummy = np.zeros((wl.B, 1), np.float32)
    oracle.tree_rollback(node.numpy(), par.numpy(), S_dummy, np.zeros((wl.B, wl.T, 1), np.float32), S_dummy.copy(),
                         x=inp["x"].view(torch.int16).numpy(), hist=hist_ref)
    assert np.array_equal(d["hist"].cpu().view(torch.int16).numpy(), hist_ref)


# ------------------------------------------------------------------ the fused tree step
def _tree_step_outputs(wl, o_dtype=torch.float32):
    B, N, Hv, dv, dk, C, W = wl.B, wl.T, wl.Hv, wl.dv, wl.dk, wl.C, wl.W
    io = torch.bfloat16 if wl.bf16 else torch.float32
    return dict(S_ckpt=torch.empty(B, Hv, dv, dk, device="cuda"), H=torch.empty(B, N, Hv, dv, dk, device="cuda"),
                o=torch.empty(B, N, Hv, dv, device="cuda", dtype=o_dtype),
                y=torch.empty(B, N, C, device="cuda", dtype=io),
                hist_out=torch.empty(B, W - 1, C, device="cuda", dtype=io))


def _tree_step(wl, d, par, out, S_prev_ckpt, hist_prev, prev=None):
    gdn.verify_tree_step(d["x"], d["w"], par, d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], out["H"],
                         out["o"], out["y"], wl.Hk, S_prev_ckpt, hist_prev, prev=prev, S_ckpt=out["S_ckpt"],
                         hist_out=out["hist_out"])


def _tree_separate(wl, d, par, out, S_start, hist):
    """conv_tree + verify_tree from S_start and hist: what the fused step must give."""
    gdn.conv_tree(d["x"], d["w"], hist, par, out["y"])
    gdn.verify_tree(out["y"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], par, S_start, out["H"], out["o"],
                    wl.Hk)
    out["S_ckpt"].copy_(S_start)
    out["hist_out"].copy_(hist)


TREE_STEP_CASES = [
    # (overrides, first tree's shape, second tree's shape, accepted nodes of the first tree)
    (dict(B=4, T=16, Hk=4, Hv=12), "random", "random", [9, -1, 0, 15]),
    (dict(B=3, T=12, Hk=2, Hv=6, W=2), "forest", "binary", [11, 3, 40]),
    (dict(B=2, T=7, Hk=2, Hv=4, dk=64, dv=64, W=8), "binary", "star", [6, 2]),
    (dict(B=2, T=32, Hk=2, Hv=6), "binary", "random", [31, 17]),
    (dict(B=2, T=5, Hk=2, Hv=6, dk=32, dv=32), "chain", "forest", [4, 0]),
    (dict(), "random", "random", [13]),                       # the bench's verify16 shape, N = 16
]


@pytest.mark.parametrize("over,shape1,shape2,acc", TREE_STEP_CASES + [(dict(name="tiny", B=2), "random", "forest",
                                                                          [3, 1])])   # fp32 inputs
def test_tree_step_equals_separate_calls(over, shape1, shape2, acc):
    """gdn_verify_tree_step gives the bits of gdn_rollback_tree + gdn_conv_tree + gdn_verify_tree: a first tree
    from the committed state, then a second tree from the first one's buffers and accepted nodes."""
    over = dict(over)
    wl = synth.small(over.pop("name", "verify16"), **over)
    say("verify_tree_step", over, shape1, shape2, "accept", acc)
    inp1 = synth.make_inputs(wl, seed=43)
    inp2 = synth.make_inputs(wl, seed=44)
    d1 = {k: dev(v) for k, v in inp1.items()}
    d2 = {k: dev(v) for k, v in inp2.items()}
    d2["w"] = d1["w"]
    par1 = dev(synth.make_tree(wl.B, wl.T, seed=45, shape=shape1))
    par2 = dev(synth.make_tree(wl.B, wl.T, seed=46, shape=shape2))
    node = torch.tensor(acc, dtype=torch.int32, device="cuda")

    A, A_ref = _tree_step_outputs(wl), _tree_step_outputs(wl)
    _tree_step(wl, d1, par1, A, d1["S_in"], d1["hist"])
    _tree_separate(wl, d1, par1, A_ref, d1["S_in"], d1["hist"])
    torch.cuda.synchronize()
    for k in A:
        assert torch.equal(A[k], A_ref[k]), "first tree: %s differs" % k

    Bo, B_ref = _tree_step_outputs(wl), _tree_step_outputs(wl)
    _tree_step(wl, d2, par2, Bo, A["S_ckpt"], A["hist_out"], prev=(node, par1, A["H"], d1["x"]))
    S_start = torch.empty_like(d1["S_in"])
    hist = A_ref["hist_out"].clone()
    gdn.rollback_tree(node, par1, A_ref["S_ckpt"], A_ref["H"], S_start, d1["x"], hist)
    _tree_separate(wl, d2, par2, B_ref, S_start, hist)
    torch.cuda.synchronize()
    for k in Bo:
        assert torch.equal(Bo[k], B_ref[k]), "second tree: %s differs" % k


def test_tree_step_chain_against_oracle():
    """Two fused tree steps against the oracle: conv and GDN of tree 1, the rollback to its accepted node, then
    tree 2 from there (conv bit for bit, states within the bar)."""
    wl = synth.small("verify16", B=2, T=16, Hk=4, Hv=12)
    say("verify_tree_step two trees vs oracle", wl)
    inp1 = synth.make_inputs(wl, seed=53)
    inp2 = synth.make_inputs(wl, seed=54)
    d1 = {k: dev(v) for k, v in inp1.items()}
    d2 = {k: dev(v) for k, v in inp2.items()}
    d2["w"] = d1["w"]
    par1 = synth.make_tree(wl.B, wl.T, seed=55, shape="random")
    par2 = synth.make_tree(wl.B, wl.T, seed=56, shape="forest")
    node = torch.tensor([10, -1], dtype=torch.int32)
    A, Bo = _tree_step_outputs(wl), _tree_step_outputs(wl)
    _tree_step(wl, d1, dev(par1), A, d1["S_in"], d1["hist"])
    _tree_step(wl, d2, dev(par2), Bo, A["S_ckpt"], A["hist_out"], prev=(dev(node), dev(par1), A["H"], d1["x"]))
    torch.cuda.synchronize()

    w = inp1["w"].numpy()
    gates = lambda inp: (f64(inp["beta_raw"]), f64(inp["alpha"]), f64(inp["dt_bias"]), f64(inp["A_log"]))
    y1 = oracle.conv_tree_f32(inp1["x"].float().numpy(), w, inp1["hist"].float().numpy(), par1.numpy(), True)
    y1b = torch.from_numpy(y1).to(torch.bfloat16)
    H1, _ = oracle.gdn_tree_f64(f64(y1b), *gates(inp1), par1.numpy(), f64(inp1["S_in"]), wl.Hk)
    # rollback of tree 1 to its accepted nodes: the state and the history
    S_keep = np.empty_like(f64(inp1["S_in"]))
    hist2 = inp1["hist"].view(torch.int16).numpy().copy()
    oracle.tree_rollback(node.numpy(), par1.numpy(), f64(inp1["S_in"]), H1, S_keep,
                         x=inp1["x"].view(torch.int16).numpy(), hist=hist2)
    hist2_f = torch.from_numpy(hist2).view(torch.bfloat16).float().numpy()
    assert np.array_equal(Bo["hist_out"].cpu().view(torch.int16).numpy(), hist2)
    check_states(Bo["S_ckpt"].cpu().numpy(), S_keep, "S_ckpt")
    y2 = oracle.conv_tree_f32(inp2["x"].float().numpy(), w, hist2_f, par2.numpy(), True)
    y2b = torch.from_numpy(y2).to(torch.bfloat16)
    assert torch.equal(Bo["y"].cpu(), y2b)
    H2, o2 = oracle.gdn_tree_f64(f64(y2b), *gates(inp2), par2.numpy(), S_keep, wl.Hk)
    check_states(Bo["H"].cpu().numpy(), H2, "H")
    check_outputs(Bo["o"].cpu().numpy(), o2, H2, False)


@pytest.mark.parametrize("N1,N2,acc", [(8, 16, [7, 3]), (32, 5, [31, -4]), (1, 12, [0, 1])])
def test_tree_step_previous_tree_of_another_size(N1, N2, acc):
    """A tree of N2 nodes after one of N1 != N2: the previous tree's node states (N1 planes), parents and tokens
    are read with N1, checked against gdn_rollback_tree + the separate calls."""
    wl1 = synth.small("verify16", B=2, T=N1, Hk=2, Hv=6)
    wl2 = synth.small("verify16", B=2, T=N2, Hk=2, Hv=6)
    say("verify_tree_step N_prev=%d N=%d" % (N1, N2), "accept", acc)
    inp1 = synth.make_inputs(wl1, seed=63)
    inp2 = synth.make_inputs(wl2, seed=64)
    d1 = {k: dev(v) for k, v in inp1.items()}
    d2 = {k: dev(v) for k, v in inp2.items()}
    d2["w"] = d1["w"]
    par1 = dev(synth.make_tree(wl1.B, N1, seed=65, shape="random"))
    par2 = dev(synth.make_tree(wl2.B, N2, seed=66, shape="forest"))
    node = torch.tensor(acc, dtype=torch.int32, device="cuda")
    A = _tree_step_outputs(wl1)
    _tree_step(wl1, d1, par1, A, d1["S_in"], d1["hist"])
    Bo, B_ref = _tree_step_outputs(wl2), _tree_step_outputs(wl2)
    _tree_step(wl2, d2, par2, Bo, A["S_ckpt"], A["hist_out"], prev=(node, par1, A["H"], d1["x"]))
    S_start = torch.empty_like(d1["S_in"])
    hist = A["hist_out"].clone()
    gdn.rollback_tree(node, par1, A["S_ckpt"], A["H"], S_start, d1["x"], hist)
    _tree_separate(wl2, d2, par2, B_ref, S_start, hist)
    torch.cuda.synchronize()
    for k in Bo:
        assert torch.equal(Bo[k], B_ref[k]), "second tree: %s differs" % k
