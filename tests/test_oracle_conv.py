"""Pins of the oracle's conv step.

The conv step takes the W-1 history rows plus the new tokens, computes
silu(conv) per channel, writes the last W-1 rows back as the new history and
keeps the whole window for rollback (lucebox PR #637, commit message on
ggml_ssm_conv_step and the review note on its four sources).  Pins:
  - the double-precision pre-activation equals numpy's correlate per channel
    (a library routine), and y = pre * expit(pre) (scipy);
  - one-hot taps fix the tap order: the last tap meets the newest token, the
    first tap reaches W-1 tokens back into the history;
  - the float version stays within one bf16 ulp (bf16 mode) or a few float
    ulps (f32 mode) of the double definition;
  - history write-back and window are exact copies;
  - the conv state after a accepted tokens, taken from the window, equals the
    history a fresh conv step over only those a tokens writes back.
"""
import numpy as np
import pytest
import scipy.special

from speculative_verify_gdn_amd import synth


def _draw(B, T, C, W, seed, bf16=True):
    wl = synth.Workload("t", B=B, T=T, Hk=1, Hv=1, dk=C // 4, dv=C // 2, W=W, bf16=bf16)
    assert wl.C == C
    inp = synth.make_inputs(wl, seed=seed)
    return inp["x"].float().numpy(), inp["w"].numpy(), inp["hist"].float().numpy()


@pytest.mark.parametrize("T", [1, 2, 3, 4, 16])
@pytest.mark.parametrize("W", [2, 4])
def test_conv_f64_is_correlation_then_silu(orc, T, W):
    x, w, hist = _draw(2, T, 64, W, seed=T * 10 + W)
    y, pre, hist_out, win = orc.conv_step_f64(x, w, hist)
    for b in range(2):
        for c in range(64):
            col = np.concatenate([hist[b, :, c], x[b, :, c]]).astype(np.float64)
            ref = np.correlate(col, w[c].astype(np.float64), mode="valid")
            assert np.allclose(pre[b, :, c], ref, rtol=1e-14, atol=1e-14)
    assert np.allclose(y, pre * scipy.special.expit(pre), rtol=1e-14, atol=1e-300)


@pytest.mark.parametrize("W", [2, 3, 4])
def test_conv_one_hot_taps(orc, W):
    T, C = 5, 32
    x, _, hist = _draw(1, T, C, W, seed=W)
    col = np.concatenate([hist, x], axis=1)  # [1][W-1+T][C]
    # last tap: pre_t = x_t
    w = np.zeros((C, W), np.float32)
    w[:, W - 1] = 1.0
    y, pre, _, _ = orc.conv_step_f64(x, w, hist)
    assert np.array_equal(pre, x.astype(np.float64))
    y32, _, _ = orc.conv_step_f32(x, w, hist, round_bf16=True)
    bits = orc.bf16_rne_bits(orc.silu32(x.reshape(-1))).reshape(x.shape)
    assert np.array_equal(y32.view(np.uint32) >> 16, bits.astype(np.uint32))
    # first tap: pre_t = window row t, i.e. the history for t < W-1
    w = np.zeros((C, W), np.float32)
    w[:, 0] = 1.0
    _, pre, _, _ = orc.conv_step_f64(x, w, hist)
    assert np.array_equal(pre[0], col[0, :T].astype(np.float64))


@pytest.mark.parametrize("bf16", [True, False])
def test_conv_f32_close_to_f64(orc, bf16):
    x, w, hist = _draw(3, 16, 256, 4, seed=5, bf16=bf16)
    y64, pre64, _, _ = orc.conv_step_f64(x, w, hist)
    y32, _, _ = orc.conv_step_f32(x, w, hist, round_bf16=bf16)
    y32 = y32.astype(np.float64)
    if bf16:
        # float result within a few float ulps, then one rounding to bf16
        ulp_bf16 = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(y64), 1e-30))) - 7)
        assert np.all(np.abs(y32 - y64) <= ulp_bf16 * 0.5 + 1e-6 * np.abs(y64) + 1e-30)
        # and y32 is bf16-representable
        assert np.all((y32.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)
    else:
        xcol = np.concatenate([hist, x], axis=1).astype(np.float64)
        mag = np.zeros_like(y64)
        for t in range(16):
            mag[:, t, :] = np.sum(np.abs(w.T[None, :, :].astype(np.float64) * np.transpose(
                xcol[:, t:t + 4, :], (0, 1, 2))), axis=1)
        tol = 8 * 2.0 ** -24 * (mag + np.abs(y64)) + 1e-30
        assert np.all(np.abs(y32 - y64) <= tol)


@pytest.mark.parametrize("T", [1, 2, 3, 8])
def test_conv_history_and_window_are_copies(orc, T):
    W = 4
    x, w, hist = _draw(2, T, 64, W, seed=T)
    col = np.concatenate([hist, x], axis=1)
    for round_bf16 in (True, False):
        _, hist_out, win = orc.conv_step_f32(x, w, hist, round_bf16)
        assert np.array_equal(win, col)
        assert np.array_equal(hist_out, col[:, T:T + W - 1])
    _, _, hist_out64, win64 = orc.conv_step_f64(x, w, hist)
    assert np.array_equal(win64, col) and np.array_equal(hist_out64, col[:, T:T + W - 1])


@pytest.mark.parametrize("K", [1, 3, 8])
def test_conv_rollback_equals_rerun(orc, K):
    """History restored from the window after a accepted tokens == conv over a tokens."""
    W, B, C = 4, 3, 64
    x, w, hist = _draw(B, K, C, W, seed=K + 100)
    _, hist_final, win = orc.conv_step_f32(x, w, hist, True)
    for a in range(K + 1):
        acc = np.full(B, a, np.int32)
        h = hist_final.copy()
        S = np.zeros((B, 1), np.float32)
        orc.rollback(acc, K, S.copy(), np.zeros((B, max(K - 1, 1), 1), np.float32), S, win=win, hist=h)
        if a == 0:
            ref = hist
        else:
            _, ref, _ = orc.conv_step_f32(x[:, :a], w, hist, True)
        assert np.array_equal(h, ref), a
