"""GPU: seeded random shapes, widening the shapes the fixed cases of the other GPU files cover.

- gdn_verify_step against gdn_rollback + gdn_conv_step + gdn_verify, and gdn_verify_tree_step against
  gdn_rollback_tree + gdn_conv_tree + gdn_verify_tree, bit for bit, over two chained windows (trees) whose
  sizes differ;
- gdn_verify and gdn_prefill_chunked against the oracle, at the stated bar (2e-3 of each state's Frobenius
  norm) and the 1e-4 regression guard beside it;
- ragged gdn_verify_ex and gdn_conv_step_ex against one call per sequence with its own length, bit for bit.
Shapes are drawn from fixed seeds: head counts and ratios, dk, dv (rows past a workgroup's block), window,
tree and prompt sizes up to the limits, chunk lengths, conv widths, bf16 and fp32 inputs and outputs, weak
decay, accept lengths and accepted nodes inside and outside their range.  Every case prints its shape
before touching the device.
"""
import random

import numpy as np
import pytest
import torch

import oracle
from speculative_verify_gdn_amd import gdn, synth

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu case]", *a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load()
    yield
    torch.cuda.synchronize()


def dev(t):
    return t.contiguous().cuda()


def draw_heads(rng):
    dk = rng.choice([32, 64, 128])
    Hk = rng.choice([1, 2, 3])
    Hv = Hk * rng.choice([1, 2, 3, 4, 6])
    dv = rng.choice([8, 16, 24, 40, 64, 128, 136])
    return dict(Hk=Hk, Hv=Hv, dk=dk, dv=dv)


def step_cases(n, seed=2024):
    rng = random.Random(seed)
    out = []
    while len(out) < n:
        h = draw_heads(rng)
        K1 = rng.choice([1, 2, 3, 5, 8, 13, 16, 17, 31, 33, 48, 64])
        K2 = rng.choice([1, 2, 4, 7, 16, 29, 64])
        B = rng.randint(1, 4)
        # keep every case small: the captured states of the longer window under 48 MB
        if B * max(K1, K2) * h["Hv"] * h["dv"] * h["dk"] * 4 > 48 << 20:
            continue
        bf16 = rng.random() < 0.75
        o_bf16 = rng.random() < 0.5
        acc = [rng.randint(-2, K1 + 2) for _ in range(B)]
        out.append((dict(B=B, bf16=bf16, **h), K1, K2, o_bf16, acc))
    return out


def tree_cases(n, seed=4049):
    rng = random.Random(seed)
    out = []
    while len(out) < n:
        h = draw_heads(rng)
        N1, N2 = rng.randint(1, 32), rng.randint(1, 32)
        B = rng.randint(1, 3)
        if B * max(N1, N2) * h["Hv"] * h["dv"] * h["dk"] * 4 > 48 << 20:
            continue
        W = rng.randint(2, 8)
        bf16 = rng.random() < 0.75
        o_bf16 = rng.random() < 0.5
        shapes = (rng.choice(["random", "forest", "binary", "star", "chain"]),
                  rng.choice(["random", "forest", "binary", "star", "chain"]))
        node = [rng.randint(-2, N1 + 1) for _ in range(B)]
        out.append((dict(B=B, W=W, bf16=bf16, **h), N1, N2, o_bf16, shapes, node))
    return out


def _step_out(wl, o_dtype):
    B, K, Hv, dv, dk, C, W = wl.B, wl.T, wl.Hv, wl.dv, wl.dk, wl.C, wl.W
    io = torch.bfloat16 if wl.bf16 else torch.float32
    return dict(S_ckpt=torch.empty(B, Hv, dv, dk, device="cuda"), S_out=torch.empty(B, Hv, dv, dk, device="cuda"),
                H=torch.empty(B, K - 1, Hv, dv, dk, device="cuda") if K > 1 else None,
                o=torch.empty(B, K, Hv, dv, device="cuda", dtype=o_dtype),
                y=torch.empty(B, K, C, device="cuda", dtype=io), win=torch.empty(B, W - 1 + K, C, device="cuda", dtype=io))


def _fused(wl, d, out, prev=None):
    gdn.verify_step(d["x"], d["w"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], out["S_out"], out["H"],
                    out["o"], wl.Hk, prev=prev, S_in=None if prev else d["S_in"], hist=None if prev else d["hist"],
                    S_ckpt=out["S_ckpt"], y=out["y"], win=out["win"])


def _separate(wl, d, out, S_start, hist):
    hist = hist.clone()
    gdn.conv_step(d["x"], d["w"], hist, out["y"], out["win"])
    gdn.verify(out["y"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], S_start, out["S_out"], out["H"],
               out["o"], wl.Hk)
    out["S_ckpt"].copy_(S_start)


def _same(a, b, what, K):
    for k in a:
        if a[k] is None:
            continue
        if K == 1 and k in ("S_out", "o"):
            # at K = 1 the separate gdn_verify takes its decode kernel (another rounding order)
            ref = b[k].double()
            assert (a[k].double() - ref).abs().max() <= 1e-5 * max(1.0, float(ref.abs().max())), \
                "%s: %s differs" % (what, k)
            continue
        assert torch.equal(a[k], b[k]), "%s: %s differs" % (what, k)


@pytest.mark.parametrize("over,K1,K2,o_bf16,acc", step_cases(36))
def test_verify_step_random_shapes(over, K1, K2, o_bf16, acc):
    wl1 = synth.small("verify16", T=K1, **over)
    wl2 = synth.small("verify16", T=K2, **over)
    o_dtype = torch.bfloat16 if o_bf16 else torch.float32
    say("verify_step sweep", over, "K", K1, "->", K2, "o bf16" if o_bf16 else "o f32", "accept", acc)
    d1 = {k: dev(v) for k, v in synth.make_inputs(wl1, seed=K1 + 7 * K2).items()}
    d2 = {k: dev(v) for k, v in synth.make_inputs(wl2, seed=K1 + 7 * K2 + 1).items()}
    d2["w"] = d1["w"]
    accept = torch.tensor(acc, dtype=torch.int32, device="cuda")
    A, A_ref = _step_out(wl1, o_dtype), _step_out(wl1, o_dtype)
    _fused(wl1, d1, A)
    _separate(wl1, d1, A_ref, d1["S_in"], d1["hist"])
    torch.cuda.synchronize()
    _same(A, A_ref, "first window", K1)
    Bo, B_ref = _step_out(wl2, o_dtype), _step_out(wl2, o_dtype)
    _fused(wl2, d2, Bo, prev=(accept, A["S_ckpt"], A["H"], A["S_out"], A["win"]))
    # the reference continues from the fused first window, so the second window is compared on its own
    S_start = A["S_out"].clone()
    hist = d1["hist"].clone()
    gdn.rollback(accept, K1, A["S_ckpt"], A["H"], S_start, hist, A["win"])
    _separate(wl2, d2, B_ref, S_start, hist)
    torch.cuda.synchronize()
    _same(Bo, B_ref, "second window", K2)


def _tree_out(wl, o_dtype):
    B, N, Hv, dv, dk, C, W = wl.B, wl.T, wl.Hv, wl.dv, wl.dk, wl.C, wl.W
    io = torch.bfloat16 if wl.bf16 else torch.float32
    return dict(S_ckpt=torch.empty(B, Hv, dv, dk, device="cuda"), H=torch.empty(B, N, Hv, dv, dk, device="cuda"),
                o=torch.empty(B, N, Hv, dv, device="cuda", dtype=o_dtype),
                y=torch.empty(B, N, C, device="cuda", dtype=io), hist_out=torch.empty(B, W - 1, C, device="cuda", dtype=io))


def _tree_fused(wl, d, par, out, S_prev_ckpt, hist_prev, prev=None):
    gdn.verify_tree_step(d["x"], d["w"], par, d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], out["H"],
                         out["o"], out["y"], wl.Hk, S_prev_ckpt, hist_prev, prev=prev, S_ckpt=out["S_ckpt"],
                         hist_out=out["hist_out"])


def _tree_separate(wl, d, par, out, S_start, hist):
    gdn.conv_tree(d["x"], d["w"], hist, par, out["y"])
    gdn.verify_tree(out["y"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], par, S_start, out["H"], out["o"],
                    wl.Hk)
    out["S_ckpt"].copy_(S_start)
    out["hist_out"].copy_(hist)


@pytest.mark.parametrize("over,N1,N2,o_bf16,shapes,node", tree_cases(30))
def test_verify_tree_step_random_shapes(over, N1, N2, o_bf16, shapes, node):
    wl1 = synth.small("verify16", T=N1, **over)
    wl2 = synth.small("verify16", T=N2, **over)
    o_dtype = torch.bfloat16 if o_bf16 else torch.float32
    say("verify_tree_step sweep", over, "N", N1, "->", N2, shapes, "o bf16" if o_bf16 else "o f32", "node", node)
    d1 = {k: dev(v) for k, v in synth.make_inputs(wl1, seed=N1 + 5 * N2).items()}
    d2 = {k: dev(v) for k, v in synth.make_inputs(wl2, seed=N1 + 5 * N2 + 1).items()}
    d2["w"] = d1["w"]
    par1 = dev(synth.make_tree(wl1.B, N1, seed=N1, shape=shapes[0]))
    par2 = dev(synth.make_tree(wl2.B, N2, seed=N2 + 1, shape=shapes[1]))
    nd = torch.tensor(node, dtype=torch.int32, device="cuda")
    A, A_ref = _tree_out(wl1, o_dtype), _tree_out(wl1, o_dtype)
    _tree_fused(wl1, d1, par1, A, d1["S_in"], d1["hist"])
    _tree_separate(wl1, d1, par1, A_ref, d1["S_in"], d1["hist"])
    torch.cuda.synchronize()
    for k in A:
        assert torch.equal(A[k], A_ref[k]), "first tree: %s differs" % k
    Bo, B_ref = _tree_out(wl2, o_dtype), _tree_out(wl2, o_dtype)
    _tree_fused(wl2, d2, par2, Bo, A["S_ckpt"], A["hist_out"], prev=(nd, par1, A["H"], d1["x"]))
    S_start = torch.empty_like(d1["S_in"])
    hist = A["hist_out"].clone()
    gdn.rollback_tree(nd, par1, A["S_ckpt"], A["H"], S_start, d1["x"], hist)
    _tree_separate(wl2, d2, par2, B_ref, S_start, hist)
    torch.cuda.synchronize()
    for k in Bo:
        assert torch.equal(Bo[k], B_ref[k]), "second tree: %s differs" % k


# ------------------------------------------------------------------ against the oracle
TOL = 2e-3
GUARD = 1e-4    # regression guard beside the bar (observed worst ~1e-6 of the state norm)


def f64(t):
    return t.double().cpu().numpy()


def check_states(gpu, ref, what):
    err = np.abs(gpu.astype(np.float64) - ref).max(axis=(-1, -2))
    fro = np.linalg.norm(ref, axis=(-1, -2))
    worst = float(np.max(err / np.maximum(fro, 1e-30)))
    print("[parity] %s worst err/fro %.3g" % (what, worst), flush=True)
    assert np.all(err <= TOL * fro), "%s: worst err/fro = %.3g" % (what, worst)
    assert worst <= GUARD, "%s: worst err/fro %.3g above the regression guard" % (what, worst)


def check_o(o_gpu, o_ref, norms, bf16_out):
    # norms [B][T][Hv]: the Frobenius norm of the state after each token (|o_t| <= it when |q^| = 1)
    bound = TOL * norms[..., None] + (np.abs(o_ref) * 2.0 ** -8 if bf16_out else 0.0)
    err = np.abs(o_gpu.astype(np.float64) - o_ref)
    assert np.all(err <= bound), "o: worst err/bound = %.3g" % float(np.max(err / np.maximum(bound, 1e-30)))


def verify_cases(n, seed=8081):
    rng = random.Random(seed)
    out = []
    while len(out) < n:
        h = draw_heads(rng)
        K = rng.randint(1, 64)
        B = rng.randint(1, 3)
        if B * K * h["Hv"] * h["dv"] * h["dk"] > 24 << 20:
            continue
        out.append((dict(B=B, T=K, bf16=rng.random() < 0.75, **h), rng.random() < 0.5, rng.random() < 0.3))
    return out


@pytest.mark.parametrize("over,o_bf16,weak", verify_cases(20))
def test_verify_random_shapes_against_oracle(over, o_bf16, weak):
    wl = synth.small("verify16", **over)
    say("verify sweep vs oracle", over, "o bf16" if o_bf16 else "o f32", "weak decay" if weak else "")
    inp = synth.make_inputs(wl, seed=wl.T + 3 * wl.Hv, weak_decay=weak)
    qkv = synth.make_qkv(wl, seed=wl.T + 3 * wl.Hv)
    d = {k: dev(v) for k, v in inp.items()}
    S_out = torch.empty_like(d["S_in"])
    H = torch.empty(wl.B, wl.T - 1, wl.Hv, wl.dv, wl.dk, device="cuda") if wl.T > 1 else None
    o = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, device="cuda", dtype=torch.bfloat16 if o_bf16 else torch.float32)
    gdn.verify(dev(qkv), d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], S_out, H, o, wl.Hk)
    torch.cuda.synchronize()
    S_ref, H_ref, o_ref = oracle.gdn_recurrent_f64(f64(qkv), f64(inp["beta_raw"]), f64(inp["alpha"]),
                                                   f64(inp["dt_bias"]), f64(inp["A_log"]), f64(inp["S_in"]), wl.Hk)
    check_states(S_out.cpu().numpy(), S_ref, "S_out")
    states = S_ref[:, None] if H is None else np.concatenate([H_ref, S_ref[:, None]], axis=1)
    if H is not None:
        check_states(H.cpu().numpy(), H_ref, "H")
    check_o(o.float().cpu().numpy(), o_ref, np.linalg.norm(states, axis=(-1, -2)), o_bf16)


def prefill_cases(n, seed=1213):
    rng = random.Random(seed)
    out = []
    while len(out) < n:
        dk = rng.choice([32, 64, 128])
        Hk = rng.choice([1, 2])
        Hv = Hk * rng.choice([1, 2, 3])
        dv = rng.choice([16, 40, 64, 128, 160])
        T = rng.choice([1, 9, 64, 65, 130, 257, 400])
        chunk = rng.choice([16, 32, 64])
        B = rng.randint(1, 2)
        bf16 = rng.random() < 0.85
        out.append((dict(B=B, T=T, Hk=Hk, Hv=Hv, dk=dk, dv=dv, bf16=bf16), chunk, rng.random() < 0.3,
                    rng.random() < 0.5))
    return out


@pytest.mark.parametrize("over,chunk,o_bf16,weak", prefill_cases(16))
def test_prefill_random_shapes_against_oracle(over, chunk, o_bf16, weak):
    wl = synth.small("prefill", **over)
    say("prefill sweep vs oracle", over, "chunk", chunk, "o bf16" if o_bf16 else "o f32",
        "weak decay" if weak else "")
    inp = synth.make_inputs(wl, seed=wl.T + wl.dv, weak_decay=weak)
    qkv = synth.make_qkv(wl, seed=wl.T + wl.dv)
    d = {k: dev(v) for k, v in inp.items()}
    S_out = torch.empty_like(d["S_in"])
    o = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, device="cuda", dtype=torch.bfloat16 if o_bf16 else torch.float32)
    gdn.prefill_chunked(dev(qkv), d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], S_out, o, wl.Hk,
                        chunk=chunk)
    torch.cuda.synchronize()
    # the oracle in segments of 64 tokens, the state chained, with the state norm after every token
    S = f64(inp["S_in"])
    q, br, al = f64(qkv), f64(inp["beta_raw"]), f64(inp["alpha"])
    os_, norms = [], []
    for t0 in range(0, wl.T, 64):
        t1 = min(wl.T, t0 + 64)
        S_new, H, o_seg = oracle.gdn_recurrent_f64(q[:, t0:t1], br[:, t0:t1], al[:, t0:t1], f64(inp["dt_bias"]),
                                                   f64(inp["A_log"]), S, wl.Hk)
        states = S_new[:, None] if H is None or H.shape[1] == 0 else np.concatenate([H, S_new[:, None]], axis=1)
        norms.append(np.linalg.norm(states, axis=(-1, -2)))
        os_.append(o_seg)
        S = S_new
    check_states(S_out.cpu().numpy(), S, "prefill S_out")
    check_o(o.float().cpu().numpy(), np.concatenate(os_, axis=1), np.concatenate(norms, axis=1), o_bf16)


# ------------------------------------------------------------------ ragged batches against one call per sequence
def ragged_cases(n, seed=5151):
    rng = random.Random(seed)
    out = []
    while len(out) < n:
        h = draw_heads(rng)
        K = rng.choice([2, 5, 8, 16, 23, 32, 64])
        B = rng.randint(2, 5)
        if B * K * h["Hv"] * h["dv"] * h["dk"] * 4 > 48 << 20:
            continue
        lens = [rng.randint(1, K) for _ in range(B)]
        out.append((dict(B=B, T=K, bf16=rng.random() < 0.75, **h), lens, rng.random() < 0.5))
    return out


@pytest.mark.parametrize("over,lens,stacked", ragged_cases(16))
def test_ragged_verify_equals_one_call_per_sequence(over, lens, stacked):
    """gdn_verify_ex with per-sequence lengths (and, half the cases, gates read out of one stacked beta|alpha row)
    against gdn_verify on each sequence alone with its own length: the same bits (a one-token sequence alone takes
    the decode kernel, another rounding order: within 1e-5); slots past a sequence's length stay untouched."""
    wl = synth.small("verify16", **over)
    say("ragged verify sweep", over, "lens", lens, "stacked gates" if stacked else "")
    inp = synth.make_inputs(wl, seed=sum(lens) + wl.Hv)
    qkv = dev(synth.make_qkv(wl, seed=sum(lens) + wl.Hv))
    d = {k: dev(v) for k, v in inp.items()}
    B, K, Hv, dv, dk = wl.B, wl.T, wl.Hv, wl.dv, wl.dk
    S_out = torch.full_like(d["S_in"], 7.0)
    H = torch.full((B, K - 1, Hv, dv, dk), 7.0, device="cuda")
    o = torch.full((B, K, Hv, dv), 7.0, device="cuda")
    if stacked:
        st = torch.cat([d["beta_raw"], d["alpha"]], dim=-1).contiguous()
        gdn.verify(qkv, st[..., :Hv], st[..., Hv:], d["dt_bias"], d["A_log"], d["S_in"], S_out, H, o, wl.Hk,
                   lens=dev(torch.tensor(lens, dtype=torch.int32)), gate_stride=2 * Hv)
    else:
        gdn.verify(qkv, d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], S_out, H, o, wl.Hk,
                   lens=dev(torch.tensor(lens, dtype=torch.int32)))
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        S1 = torch.empty_like(d["S_in"][b:b + 1])
        H1 = torch.empty(1, L - 1, Hv, dv, dk, device="cuda") if L > 1 else None
        o1 = torch.empty(1, L, Hv, dv, device="cuda")
        gdn.verify(qkv[b:b + 1, :L].contiguous(), d["beta_raw"][b:b + 1, :L].contiguous(),
                   d["alpha"][b:b + 1, :L].contiguous(), d["dt_bias"], d["A_log"], d["S_in"][b:b + 1].contiguous(),
                   S1, H1, o1, wl.Hk)
        torch.cuda.synchronize()
        if L == 1:
            ref = S1[0].double()
            assert (S_out[b].double() - ref).abs().max() <= 1e-5 * max(1.0, float(ref.abs().max()))
            ref = o1[0].double()
            assert (o[b, :1].double() - ref).abs().max() <= 1e-5 * max(1.0, float(ref.abs().max()))
        else:
            assert torch.equal(S_out[b], S1[0]), "sequence %d: S_out" % b
            assert torch.equal(H[b, :L - 1], H1[0]), "sequence %d: H" % b
            assert torch.equal(o[b, :L], o1[0]), "sequence %d: o" % b
        assert bool((H[b, L - 1:] == 7.0).all()) and bool((o[b, L:] == 7.0).all()), "sequence %d: slots past it" % b


@pytest.mark.parametrize("over,lens,stacked", ragged_cases(8, seed=6262))
def test_ragged_conv_step_equals_one_call_per_sequence(over, lens, stacked):
    """gdn_conv_step_ex with per-sequence lengths against gdn_conv_step on each sequence alone, bit for bit:
    y, the window and the written-back history (window rows lens[b] .. lens[b]+W-2)."""
    wl = synth.small("verify16", **over)
    say("ragged conv sweep", over, "lens", lens)
    inp = synth.make_inputs(wl, seed=sum(lens) + 3)
    x, w, hist0 = dev(inp["x"]), dev(inp["w"]), dev(inp["hist"])
    B, K, C, W = wl.B, wl.T, wl.C, wl.W
    hist = hist0.clone()
    y = torch.zeros_like(x)
    win = torch.zeros(B, W - 1 + K, C, device="cuda", dtype=x.dtype)
    gdn.conv_step(x, w, hist, y, win, lens=dev(torch.tensor(lens, dtype=torch.int32)))
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        h1 = hist0[b:b + 1].clone()
        y1 = torch.empty(1, L, C, device="cuda", dtype=x.dtype)
        w1 = torch.empty(1, W - 1 + L, C, device="cuda", dtype=x.dtype)
        gdn.conv_step(x[b:b + 1, :L].contiguous(), w, h1, y1, w1)
        torch.cuda.synchronize()
        assert torch.equal(y[b, :L], y1[0]), "sequence %d: y" % b
        assert torch.equal(win[b, :W - 1 + L], w1[0]), "sequence %d: window" % b
        assert torch.equal(hist[b], h1[0]), "sequence %d: history" % b
