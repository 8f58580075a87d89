"""Pins of the oracle's tree verify.

The drafter proposes a tree of tokens instead of a chain (lucebox PR #637:
DDTree drafting and the tree variant of the conv, ggml_ssm_conv_tree, in the
commit messages and the review excerpt of ggml.c).  The oracle reads it as the
chain step applied along every root path: a node continues its parent's conv
window and GDN state, a root continues the committed ones.  Pinned against the
chain functions (themselves pinned in the other files), not against itself:
  - a chain-shaped tree equals the chain verify (conv bit for bit, GDN states
    and outputs), a star equals N independent one-token steps;
  - every node of a random tree equals the chain verify run over the tokens of
    its root path (brute force over all nodes, 2-head d=4 and d=32 cases);
  - the rollback to a node equals the history a conv step over the path writes
    back, and the state after the path;
  - parent entries outside [0, i) act as roots.
"""
import numpy as np
import pytest

from speculative_verify_gdn_amd import synth


def _gdn_inputs(B, N, Hk=2, Hv=2, d=4, seed=0):
    wl = synth.Workload("t", B=B, T=N, Hk=Hk, Hv=Hv, dk=d, dv=d, bf16=False)
    inp = synth.make_inputs(wl, seed=seed)
    qkv = synth.make_qkv(wl, seed=seed).double().numpy()
    f = lambda k: inp[k].double().numpy()
    return qkv, f("beta_raw"), f("alpha"), f("dt_bias"), f("A_log"), f("S_in")


def _conv_inputs(B, N, C=64, W=4, seed=0):
    wl = synth.Workload("t", B=B, T=N, Hk=1, Hv=1, dk=C // 4, dv=C // 2, W=W, bf16=True)
    inp = synth.make_inputs(wl, seed=seed)
    return inp["x"].float().numpy(), inp["w"].numpy(), inp["hist"].float().numpy()


def _path(par, b, i):
    """Root-first node list of the path ending at node i (entries outside [0, i) are roots)."""
    out = []
    while i >= 0:
        out.append(i)
        p = int(par[b, i])
        i = p if 0 <= p < i else -1
    return out[::-1]


# ------------------------------------------------------------------ GDN
@pytest.mark.parametrize("N", [1, 5, 16])
def test_chain_tree_equals_chain_verify(orc, N):
    qkv, br, al, dt, alog, S = _gdn_inputs(2, N, d=8, seed=N)
    par = synth.make_tree(2, N, shape="chain").numpy()
    H, o = orc.gdn_tree_f64(qkv, br, al, dt, alog, par, S, Hk=2)
    S_out, Hc, oc = orc.gdn_recurrent_f64(qkv, br, al, dt, alog, S, Hk=2)
    assert np.allclose(o, oc, rtol=0, atol=1e-12)
    assert np.allclose(H[:, N - 1], S_out, rtol=0, atol=1e-12)
    if N > 1:
        assert np.allclose(H[:, : N - 1], Hc, rtol=0, atol=1e-12)


def test_star_tree_is_independent_single_steps(orc):
    N = 6
    qkv, br, al, dt, alog, S = _gdn_inputs(1, N, d=8, seed=3)
    par = synth.make_tree(1, N, shape="star").numpy()
    H, o = orc.gdn_tree_f64(qkv, br, al, dt, alog, par, S, Hk=2)
    for i in range(N):
        S1, _, o1 = orc.gdn_recurrent_f64(qkv[:, i:i + 1], br[:, i:i + 1], al[:, i:i + 1], dt, alog, S, Hk=2)
        assert np.allclose(H[:, i], S1, rtol=0, atol=1e-12)
        assert np.allclose(o[:, i], o1[:, 0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape,N,d", [("random", 12, 4), ("forest", 12, 4), ("random", 20, 32)])
def test_every_node_equals_chain_over_its_root_path(orc, shape, N, d):
    B = 2
    qkv, br, al, dt, alog, S = _gdn_inputs(B, N, d=d, seed=N + d)
    par = synth.make_tree(B, N, seed=N, shape=shape).numpy()
    H, o = orc.gdn_tree_f64(qkv, br, al, dt, alog, par, S, Hk=2)
    for b in range(B):
        for i in range(N):
            p = _path(par, b, i)
            S_p, _, o_p = orc.gdn_recurrent_f64(qkv[b:b + 1, p], br[b:b + 1, p], al[b:b + 1, p], dt, alog,
                                                S[b:b + 1], Hk=2)
            assert np.allclose(H[b, i], S_p[0], rtol=0, atol=1e-12), (b, i, p)
            assert np.allclose(o[b, i], o_p[0, -1], rtol=0, atol=1e-12), (b, i, p)


def test_out_of_range_parents_are_roots(orc):
    N = 5
    qkv, br, al, dt, alog, S = _gdn_inputs(1, N, seed=9)
    bad = np.array([[7, 0, 2, -5, 3]], np.int32)     # 7 >= 0's index, 2 == own index, -5 < -1
    good = np.array([[-1, 0, -1, -1, 3]], np.int32)
    H1, o1 = orc.gdn_tree_f64(qkv, br, al, dt, alog, bad, S, Hk=2)
    H2, o2 = orc.gdn_tree_f64(qkv, br, al, dt, alog, good, S, Hk=2)
    assert np.array_equal(H1, H2) and np.array_equal(o1, o2)


def test_zero_gates_leave_every_node_state(orc):
    N = 7
    qkv, br, al, dt, alog, S = _gdn_inputs(1, N, seed=4)
    par = synth.make_tree(1, N, shape="random").numpy()
    H, o = orc.gdn_tree_f64(qkv, np.zeros_like(br), np.zeros_like(al), None, None, par, S, Hk=2)
    for i in range(N):
        assert np.array_equal(H[0, i], S[0])


# ------------------------------------------------------------------ conv
@pytest.mark.parametrize("N,W", [(1, 4), (3, 4), (16, 4), (8, 2)])
def test_chain_tree_conv_equals_conv_step_bitwise(orc, N, W):
    x, w, hist = _conv_inputs(2, N, W=W, seed=N)
    par = synth.make_tree(2, N, shape="chain").numpy()
    y = orc.conv_tree_f32(x, w, hist, par, True)
    yc, _, _ = orc.conv_step_f32(x, w, hist, True)
    assert np.array_equal(y.view(np.uint32), yc.view(np.uint32))


@pytest.mark.parametrize("shape", ["random", "forest", "star"])
def test_tree_conv_node_equals_conv_step_over_its_path(orc, shape):
    B, N = 2, 14
    x, w, hist = _conv_inputs(B, N, seed=21)
    par = synth.make_tree(B, N, seed=2, shape=shape).numpy()
    y = orc.conv_tree_f32(x, w, hist, par, True)
    for b in range(B):
        for i in range(N):
            p = _path(par, b, i)
            yc, _, _ = orc.conv_step_f32(x[b:b + 1, p], w, hist[b:b + 1], True)
            assert np.array_equal(y[b, i].view(np.uint32), yc[0, -1].view(np.uint32)), (b, i, p)


def test_tree_conv_leaves_history_untouched(orc):
    x, w, hist = _conv_inputs(1, 6, seed=5)
    h0 = hist.copy()
    orc.conv_tree_f32(x, w, hist, synth.make_tree(1, 6, shape="random").numpy(), False)
    assert np.array_equal(hist, h0)


# ------------------------------------------------------------------ rollback
@pytest.mark.parametrize("W", [2, 4])
def test_tree_rollback_equals_path_rerun(orc, W):
    B, N, d = 3, 10, 4
    qkv, br, al, dt, alog, S = _gdn_inputs(B, N, d=d, seed=11)
    x, w, hist = _conv_inputs(B, N, W=W, seed=12)
    par = synth.make_tree(B, N, seed=3, shape="forest").numpy()
    H, _ = orc.gdn_tree_f64(qkv, br, al, dt, alog, par, S, Hk=2)
    for node in (-1, 0, 4, N - 1, N + 3):
        nd = np.full(B, node, np.int32)
        S_out = np.zeros_like(S)
        hist_new = hist.copy()
        orc.tree_rollback(nd, par, S, H, S_out, x=x, hist=hist_new)
        for b in range(B):
            if node < 0 or node >= N:
                assert np.array_equal(S_out[b], S[b]) and np.array_equal(hist_new[b], hist[b])
                continue
            p = _path(par, b, node)
            S_p, _, _ = orc.gdn_recurrent_f64(qkv[b:b + 1, p], br[b:b + 1, p], al[b:b + 1, p], dt, alog,
                                              S[b:b + 1], Hk=2)
            assert np.allclose(S_out[b], S_p[0], rtol=0, atol=1e-12)
            _, hist_ref, _ = orc.conv_step_f32(x[b:b + 1, p], w, hist[b:b + 1], True)
            assert np.array_equal(hist_new[b], hist_ref[0]), (b, node, p)


def test_tree_rollback_bf16_bytes(orc):
    # the conv part is a byte copy of whatever element type the rows hold
    import torch
    B, N, C, W = 2, 6, 24, 4
    g = torch.Generator().manual_seed(0)
    x = torch.randn(B, N, C, generator=g).to(torch.bfloat16).view(torch.int16).numpy()
    hist = torch.randn(B, W - 1, C, generator=g).to(torch.bfloat16).view(torch.int16).numpy()
    par = np.array([[-1, 0, 1, 1, 3, 4], [-1, -1, 1, 0, 2, 2]], np.int32)
    S = np.zeros((B, 1), np.float32)
    H = np.zeros((B, N, 1), np.float32)
    hn = hist.copy()
    orc.tree_rollback(np.array([5, 1], np.int32), par, S, H, S.copy(), x=x, hist=hn)
    # b=0: path 0,1,3,4,5 -> last three rows x3, x4, x5; b=1: path 1 (a root) -> hist[2], x1 ... oldest first
    assert np.array_equal(hn[0], x[0, [3, 4, 5]])
    assert np.array_equal(hn[1], np.stack([hist[1, 1], hist[1, 2], x[1, 1]]))
