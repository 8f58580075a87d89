"""Pins of the oracle's gated delta rule.

The recurrence (named by the pages, written out in its plainest reading):
    S_t = e^{g_t} S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t,
with q, k L2-normalised, beta = sigmoid(raw beta),
g = -softplus(alpha + dt_bias) * e^{A_log}  (lucebox PR #637, commit message on
raw gates and the review excerpt of gated_delta_net.cu), evaluated over a
K-token verify window with every intermediate state kept (atlas PR #297,
commit message on gated_delta_rule_wy16.cu).

The oracle computes it as the delta-rule update (u = beta (v - S k)).  It is
pinned here against things that are not that update:
  - the gates against scipy's expit and numpy's logaddexp, and closed values;
  - the explicit matrix product form S_{t-1} A_t + beta v k^T and the closed
    product sum, with A_t = gamma_t (I - beta_t k k^T), on 2-head d=4 cases;
  - the delta identities S_t k_t = (1-beta) gamma S_{t-1} k_t + beta v and
    S_t x = gamma S_{t-1} x for x orthogonal to k_t;
  - beta = 0, g = 0 leaves S unchanged with o_t = S q_t (numpy matvec);
  - one token from S = 0 gives beta v k^T;
  - K=1 equals one decode step, and H_0 of a K-window equals it;
  - the chunkwise WY form (a different algorithm) equals the sequential one;
  - rollback to j tokens equals re-running j tokens;
  - the head map (value head h reads key head h // (Hv/Hk)) and the q|k|v slab
    order.
"""
import numpy as np
import pytest
import scipy.special

from speculative_verify_gdn_amd import synth


def _inputs(B=1, K=4, Hk=2, Hv=2, d=32, seed=0, weak=False):
    wl = synth.Workload("t", B=B, T=K, Hk=Hk, Hv=Hv, dk=d, dv=d, bf16=False)
    inp = synth.make_inputs(wl, seed=seed, weak_decay=weak)
    qkv = synth.make_qkv(wl, seed=seed).double().numpy()
    f = lambda k: inp[k].double().numpy()
    return wl, qkv, f("beta_raw"), f("alpha"), f("dt_bias"), f("A_log"), f("S_in")


def _norm(x):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-6)


def _split(qkv, Hk, Hv, d):
    q = qkv[..., : Hk * d].reshape(*qkv.shape[:-1], Hk, d)
    k = qkv[..., Hk * d: 2 * Hk * d].reshape(*qkv.shape[:-1], Hk, d)
    v = qkv[..., 2 * Hk * d:].reshape(*qkv.shape[:-1], Hv, d)
    return q, k, v


# ------------------------------------------------------------------ gates
def test_gates_against_library_routines(orc):
    rng = np.random.default_rng(0)
    br = rng.normal(0, 3, (64, 8))
    al = rng.normal(0, 3, (64, 8))
    dt = rng.uniform(-1, 1, 8)
    alog = rng.uniform(-2, np.log(16), 8)
    beta, g = orc.gates_f64(br, al, dt, alog)
    assert np.allclose(beta, scipy.special.expit(br), rtol=1e-15, atol=0)
    assert np.allclose(g, -np.logaddexp(0.0, al + dt) * np.exp(alog), rtol=1e-14, atol=0)
    # activated mode passes the values through
    b2, g2 = orc.gates_f64(br, al, None, None)
    assert np.array_equal(b2, br) and np.array_equal(g2, al)


def test_gate_closed_values(orc):
    br = np.array([[0.0, -np.inf, np.inf, 0.0]])
    al = np.array([[0.0, 0.0, 0.0, 1000.0]])
    dt = np.zeros(4)
    alog = np.array([0.0, 0.0, -np.inf, 0.0])
    beta, g = orc.gates_f64(br, al, dt, alog)
    assert beta[0, 0] == 0.5 and beta[0, 1] == 0.0 and beta[0, 2] == 1.0
    assert g[0, 0] == -np.log(2.0)           # softplus(0) = ln 2
    assert g[0, 2] == 0.0                    # A = -e^{-inf} = 0: no decay
    assert g[0, 3] == -1000.0                # softplus(a) = a for large a


# ------------------------------------------------------------------ brute force product form
@pytest.mark.parametrize("Hk,Hv", [(2, 2), (2, 4), (1, 3)])
@pytest.mark.parametrize("K", [1, 3, 6])
def test_brute_force_matrix_product_d4(orc, Hk, Hv, K):
    d = 4
    wl, qkv, br, al, dt, alog, S0 = _inputs(B=2, K=K, Hk=Hk, Hv=Hv, d=d, seed=K + 10 * Hv)
    S_out, H, o = orc.gdn_recurrent_f64(qkv, br, al, dt, alog, S0, Hk)
    q, k, v = _split(qkv, Hk, Hv, d)
    beta = scipy.special.expit(br)
    g = -np.logaddexp(0.0, al + dt) * np.exp(alog)
    I = np.eye(d)
    for b in range(2):
        for h in range(Hv):
            hk = h // (Hv // Hk)
            S = S0[b, h].copy()
            Amats, adds = [], []
            for t in range(K):
                kh = _norm(k[b, t, hk])
                qh = _norm(q[b, t, hk])
                At = np.exp(g[b, t, h]) * (I - beta[b, t, h] * np.outer(kh, kh))
                add = beta[b, t, h] * np.outer(v[b, t, h], kh)
                S = S @ At + add
                Amats.append(At)
                adds.append(add)
                assert np.allclose(o[b, t, h], S @ qh, rtol=0, atol=1e-13)
                if t < K - 1:
                    assert np.allclose(H[b, t, h], S, rtol=0, atol=1e-13)
            assert np.allclose(S_out[b, h], S, rtol=0, atol=1e-13)
            # closed form: S_K = S_0 prod A_t + sum_t add_t prod_{s>t} A_s
            P = np.eye(d)
            for At in Amats:
                P = P @ At
            closed = S0[b, h] @ P
            for t in range(K):
                R = np.eye(d)
                for s in range(t + 1, K):
                    R = R @ Amats[s]
                closed = closed + adds[t] @ R
            assert np.allclose(S_out[b, h], closed, rtol=0, atol=1e-13)


# ------------------------------------------------------------------ delta identities
def test_delta_identities_every_step(orc):
    d, K, Hk, Hv = 32, 8, 2, 4
    wl, qkv, br, al, dt, alog, S0 = _inputs(B=1, K=K, Hk=Hk, Hv=Hv, d=d, seed=3, weak=True)
    S_out, H, o = orc.gdn_recurrent_f64(qkv, br, al, dt, alog, S0, Hk)
    q, k, v = _split(qkv, Hk, Hv, d)
    beta = scipy.special.expit(br)
    gam = np.exp(-np.logaddexp(0.0, al + dt) * np.exp(alog))
    states = [S0[0]] + [H[0, t] for t in range(K - 1)] + [S_out[0]]
    rng = np.random.default_rng(4)
    for t in range(K):
        for h in range(Hv):
            kh = _norm(k[0, t, h // (Hv // Hk)])
            prev, cur = states[t][h], states[t + 1][h]
            lhs = cur @ kh
            # ||k_hat||^2 = |k|^2 / (|k|^2 + eps) is 1 up to eps; keep it exact
            n2 = kh @ kh
            gp = gam[0, t, h] * (prev @ kh)
            rhs = gp + beta[0, t, h] * (v[0, t, h] - gp) * n2
            assert np.allclose(lhs, rhs, rtol=0, atol=1e-12)
            assert np.allclose(lhs, (1 - beta[0, t, h]) * gp + beta[0, t, h] * v[0, t, h], rtol=0, atol=1e-6)
            x = rng.normal(size=d)
            x -= (x @ kh) / (kh @ kh) * kh
            assert np.allclose(cur @ x, gam[0, t, h] * (prev @ x), rtol=0, atol=1e-12)


# ------------------------------------------------------------------ special cases
@pytest.mark.parametrize("mode", ["activated", "raw"])
def test_zero_beta_zero_decay_leaves_state(orc, mode):
    d, K, Hk, Hv = 32, 5, 2, 2
    wl, qkv, br, al, dt, alog, S0 = _inputs(K=K, Hk=Hk, Hv=Hv, d=d, seed=5)
    if mode == "activated":
        br, al, dt, alog = np.zeros_like(br), np.zeros_like(al), None, None
    else:
        br = np.full_like(br, -np.inf)
        alog = np.full_like(alog, -np.inf)
    S_out, H, o = orc.gdn_recurrent_f64(qkv, br, al, dt, alog, S0, Hk)
    assert np.array_equal(S_out, S0)
    for t in range(K - 1):
        assert np.array_equal(H[:, t], S0)
    q, _, _ = _split(qkv, Hk, Hv, d)
    for t in range(K):
        for h in range(Hv):
            assert np.allclose(o[0, t, h], S0[0, h] @ _norm(q[0, t, h]), rtol=0, atol=1e-14)


def test_one_token_from_zero_state(orc):
    d, Hk, Hv = 16, 1, 2
    wl, qkv, br, al, dt, alog, S0 = _inputs(K=1, Hk=Hk, Hv=Hv, d=d, seed=6)
    qkv[..., :d] = qkv[..., d:2 * d]          # q = k
    S0 = np.zeros_like(S0)
    S_out, _, o = orc.gdn_recurrent_f64(qkv, br, al, dt, alog, S0, Hk)
    _, k, v = _split(qkv, Hk, Hv, d)
    beta = scipy.special.expit(br)
    kh = _norm(k[0, 0, 0])
    for h in range(Hv):
        assert np.allclose(S_out[0, h], beta[0, 0, h] * np.outer(v[0, 0, h], kh), rtol=0, atol=1e-15)
        # o = beta v (k.q) = beta v ||k_hat||^2 ~ beta v
        assert np.allclose(o[0, 0, h], beta[0, 0, h] * v[0, 0, h] * (kh @ kh), rtol=0, atol=1e-15)
        assert np.allclose(o[0, 0, h], beta[0, 0, h] * v[0, 0, h], rtol=1e-6, atol=0)


def test_k1_equals_decode_and_first_intermediate(orc):
    d, K, Hk, Hv = 32, 6, 2, 4
    wl, qkv, br, al, dt, alog, S0 = _inputs(B=2, K=K, Hk=Hk, Hv=Hv, d=d, seed=7)
    S_out, H, o = orc.gdn_recurrent_f64(qkv, br, al, dt, alog, S0, Hk)
    S1, _, o1 = orc.gdn_recurrent_f64(qkv[:, :1], br[:, :1], al[:, :1], dt, alog, S0, Hk, capture=False)
    assert np.array_equal(H[:, 0], S1)
    assert np.array_equal(o[:, 0], o1[:, 0])
    # decode one token at a time reproduces every intermediate and the final state
    S = S0
    for t in range(K):
        S, _, ot = orc.gdn_recurrent_f64(qkv[:, t:t + 1], br[:, t:t + 1], al[:, t:t + 1], dt, alog, S, Hk,
                                         capture=False)
        assert np.array_equal(ot[:, 0], o[:, t])
        ref = H[:, t] if t < K - 1 else S_out
        assert np.array_equal(S, ref)


@pytest.mark.parametrize("K", [1, 4, 9])
def test_rollback_equals_rerun(orc, K):
    d, Hk, Hv, B = 16, 2, 4, 3
    wl, qkv, br, al, dt, alog, S0 = _inputs(B=B, K=K, Hk=Hk, Hv=Hv, d=d, seed=8 + K)
    S_fin, H, _ = orc.gdn_recurrent_f64(qkv, br, al, dt, alog, S0, Hk)
    Hbuf = H if K > 1 else np.zeros((B, 1, Hv, d, d))
    for j in range(K + 1):
        S_out = S_fin.copy()
        orc.rollback(np.full(B, j, np.int32), K, S0, Hbuf, S_out)
        if j == 0:
            ref = S0
        else:
            ref, _, _ = orc.gdn_recurrent_f64(qkv[:, :j], br[:, :j], al[:, :j], dt, alog, S0, Hk, capture=False)
        assert np.array_equal(S_out, ref), j
    # per-sequence accept lengths, and clamping outside 0..K
    acc = np.array([0, K, -5][:B], np.int32)
    S_out = S_fin.copy()
    orc.rollback(acc, K, S0, Hbuf, S_out)
    assert np.array_equal(S_out[0], S0[0]) and np.array_equal(S_out[1], S_fin[1])
    assert np.array_equal(S_out[2], S0[2])


# ------------------------------------------------------------------ WY == sequential
@pytest.mark.parametrize("K,chunk,weak", [(4, 4, False), (16, 16, False), (16, 4, True), (16, 5, True),
                                          (37, 16, False), (130, 64, False), (130, 64, True), (64, 64, False)])
def test_chunked_wy_equals_sequential(orc, K, chunk, weak):
    d, Hk, Hv = 32, 2, 4
    wl, qkv, br, al, dt, alog, S0 = _inputs(B=2, K=K, Hk=Hk, Hv=Hv, d=d, seed=K + chunk, weak=weak)
    capture = K <= 40
    Sr, Hr, orr = orc.gdn_recurrent_f64(qkv, br, al, dt, alog, S0, Hk, capture=capture)
    Sc, Hc, oc = orc.gdn_chunked_f64(qkv, br, al, dt, alog, S0, Hk, chunk, capture=capture)
    scale = max(1.0, float(np.max(np.abs(Sr))))
    assert np.max(np.abs(Sr - Sc)) <= 1e-12 * scale
    assert np.max(np.abs(orr - oc)) <= 1e-12 * max(1.0, float(np.max(np.abs(orr))))
    if capture and K > 1:
        assert np.max(np.abs(Hr - Hc)) <= 1e-12 * scale


def test_chunked_wy_strong_decay_no_ratio_overflow(orc):
    """G reaches about -460 over a 64-token chunk; only e^{G_t - G_s}, s <= t, is formed."""
    d, K, Hk, Hv = 32, 64, 1, 2
    wl, qkv, br, al, dt, alog, S0 = _inputs(K=K, Hk=Hk, Hv=Hv, d=d, seed=9)
    al = np.full_like(al, 3.0)
    alog = np.full_like(alog, np.log(2.3))
    _, g = orc.gates_f64(br, al, dt, alog)
    assert np.sum(g[0, :, 0]) < -400
    Sr, _, orr = orc.gdn_recurrent_f64(qkv, br, al, dt, alog, S0, Hk, capture=False)
    Sc, _, oc = orc.gdn_chunked_f64(qkv, br, al, dt, alog, S0, Hk, 64, capture=False)
    assert np.all(np.isfinite(Sc)) and np.all(np.isfinite(oc))
    assert np.max(np.abs(Sr - Sc)) <= 1e-12 and np.max(np.abs(orr - oc)) <= 1e-12


# ------------------------------------------------------------------ layout pins
def test_head_map_value_head_reads_key_head_h_div_group(orc):
    d, Hk, Hv = 8, 2, 6
    wl, qkv, br, al, dt, alog, S0 = _inputs(K=1, Hk=Hk, Hv=Hv, d=d, seed=11)
    qkv[..., Hk * d + d: 2 * Hk * d] = 0.0      # k of key head 1 is zero -> k_hat = 0
    S_out, _, _ = orc.gdn_recurrent_f64(qkv, br, al, dt, alog, S0, Hk)
    gam = np.exp(-np.logaddexp(0.0, al + dt) * np.exp(alog))
    for h in range(Hv):
        pure_decay = np.allclose(S_out[0, h], gam[0, 0, h] * S0[0, h], rtol=0, atol=1e-15)
        assert pure_decay == (h >= 3), h


def test_slab_order_q_then_k_then_v(orc):
    d, Hk, Hv = 8, 2, 4
    wl, qkv, br, al, dt, alog, S0 = _inputs(K=1, Hk=Hk, Hv=Hv, d=d, seed=12)
    q, k, v = _split(qkv, Hk, Hv, d)
    eye = np.broadcast_to(np.eye(d), S0.shape).copy()
    # beta = 0, g = 0, S = I: o = q_hat
    _, _, o = orc.gdn_recurrent_f64(qkv, np.zeros_like(br), np.zeros_like(al), None, None, eye, Hk)
    for h in range(Hv):
        assert np.allclose(o[0, 0, h], _norm(q[0, 0, h // 2]), rtol=0, atol=1e-14)
        assert np.isclose(np.linalg.norm(o[0, 0, h]), 1.0, rtol=1e-7)
    # beta = 1, g = 0, S = 0: S_1 = v k_hat^T
    S1, _, _ = orc.gdn_recurrent_f64(qkv, np.ones_like(br), np.zeros_like(al), None, None,
                                     np.zeros_like(S0), Hk)
    for h in range(Hv):
        assert np.allclose(S1[0, h], np.outer(v[0, 0, h], _norm(k[0, 0, h // 2])), rtol=0, atol=1e-15)
