"""ctypes binding of libgdn.so (include/gdn.h) for torch device tensors.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Each function takes torch tensors that already live on the GPU,
passes their device pointers, the sizes and torch's current HIP stream to the
C entry point of the same name, and raises GdnError on a non-zero status.
There is no fallback: if libgdn.so is missing or cannot be loaded, the first
call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("GDN_LIB", os.path.join(_PKG, "libgdn.so"))
# the debug build (also counts clamped accept lengths: debug_clamped_accepts)
DEBUG_LIB_PATH = os.path.join(_PKG, "libgdn_debug.so")

GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_EHIP = 0, -1, -2, -3
GDN_F32, GDN_BF16 = 0, 1
EXPORTS = ("gdn_version", "gdn_last_error", "gdn_conv_step", "gdn_verify", "gdn_rollback", "gdn_prefill_chunked",
           "gdn_rollback_conv_step", "gdn_conv_step_ex", "gdn_verify_ex", "gdn_rollback_ex", "gdn_replay",
           "gdn_conv_tree", "gdn_verify_tree", "gdn_rollback_tree", "gdn_verify_step",
           "gdn_debug_clamped_accepts", "gdn_verify_tree_step")


class GdnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("libgdn error %d: %s" % (code, msg))
        self.code = code


_lib = None
_lock = threading.Lock()
_using = threading.local()


def load(path: str = LIB_PATH):
    """Load libgdn.so (once) and declare the C signatures."""
    global _lib
    with _lock:
        if _lib is None:
            _lib = open_library(path)
        return _lib


def _L():
    """The library the calls of this thread go to: load()'s, or the one a `using` block names."""
    lib = getattr(_using, "lib", None)
    return lib if lib is not None else load()


@contextlib.contextmanager
def using(lib):
    """Route this thread's calls to another build of the library (e.g. open_library(DEBUG_LIB_PATH))."""
    prev = getattr(_using, "lib", None)
    _using.lib = lib
    try:
        yield lib
    finally:
        _using.lib = prev


def debug_clamped_accepts(reset: bool = False) -> int:
    """gdn_debug_clamped_accepts: clamped accept lengths counted by the debug build (raises GdnError
    GDN_EUNSUPPORTED on the release build)."""
    n = ctypes.c_longlong(0)
    _check(_L().gdn_debug_clamped_accepts(ctypes.byref(n), int(bool(reset))))
    return n.value


def open_library(path: str):
    """Open a build of libgdn at `path` and declare the C signatures (no caching)."""
    if not os.path.exists(path):
        raise FileNotFoundError("libgdn not built (%s); run python -m speculative_verify_gdn_amd.build" % path)
    lib = ctypes.CDLL(path)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.gdn_version.restype = I
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_conv_step.argtypes = [P, P, P, P, P, I, I, I, I, I, P]
    lib.gdn_verify.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, P]
    lib.gdn_rollback.argtypes = [P, I, P, P, P, P, P, I, I, I, I, I, I, I, P]
    lib.gdn_prefill_chunked.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, P]
    lib.gdn_rollback_conv_step.argtypes = [P, I, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, P]
    lib.gdn_conv_step_ex.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P]
    lib.gdn_verify_ex.argtypes = [P, P, P, I, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, P]
    lib.gdn_rollback_ex.argtypes = [P, P, I, P, P, P, P, P, I, I, I, I, I, I, I, P]
    lib.gdn_replay.argtypes = [P, P, P, P, I, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, P]
    lib.gdn_verify_step.argtypes = [P, I, P, P, P, P, P, P, P, P, P, P, I, P, P, P, P, P, P, P, P,
                                    I, I, I, I, I, I, I, I, I, F, P]
    lib.gdn_conv_tree.argtypes = [P, P, P, P, P, I, I, I, I, I, P]
    lib.gdn_verify_tree.argtypes = [P, P, P, I, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, P]
    lib.gdn_rollback_tree.argtypes = [P, P, I, P, P, P, P, P, I, I, I, I, I, I, I, P]
    lib.gdn_debug_clamped_accepts.argtypes = [P, I]
    lib.gdn_verify_tree_step.argtypes = [P, I, P, P, P, P, P, P, P, P, P, P, I, P, P, P, P, P, P, P,
                                         I, I, I, I, I, I, I, I, I, F, P]
    for name in EXPORTS:
        getattr(lib, name).restype = ctypes.c_char_p if name == "gdn_last_error" else I
    return lib


def _check(rc: int):
    if rc != GDN_OK:
        raise GdnError(rc, _L().gdn_last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype(t) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError("unsupported dtype %s" % t.dtype)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("libgdn takes device tensors")
            if not t.is_contiguous():
                raise ValueError("libgdn takes contiguous tensors")


def version() -> int:
    return _L().gdn_version()


def conv_step(x, w, hist, y, win=None, lens=None, stream=None):
    """gdn_conv_step(_ex): x [B][T][C], w [C][W] f32, hist [B][W-1][C] (updated), y, win [B][W-1+T][C];
    lens [B] int32 (device) for a ragged batch."""
    _dev(x, w, hist, y, win, lens)
    B, T, C = x.shape
    W = w.shape[1]
    _check(_L().gdn_conv_step_ex(_p(x), _p(w), _p(hist), _p(y), _p(win), _p(lens), B, T, C, W, _dtype(x),
                                   _stream(stream)))


def verify(qkv, beta_raw, alpha, dt_bias, A_log, S_in, S_out, H, o, Hk, eps=1e-6, lens=None, gate_stride=None,
           stream=None):
    """gdn_verify(_ex): qkv [B][K][C], gates [B][K][Hv], S [B][Hv][dv][dk] f32, H [B][K-1][Hv][dv][dk] or None,
    o [B][K][Hv][dv]; lens [B] int32 (device) for a ragged batch; gate_stride for gates read out of a
    stacked beta|alpha buffer (beta_raw and alpha are then views of it: their data pointers are used)."""
    _dev(qkv, S_in, S_out, H, o, lens, dt_bias, A_log)
    if gate_stride is None:
        _dev(beta_raw, alpha)
    elif not (beta_raw.is_cuda and alpha.is_cuda):
        raise ValueError("libgdn takes device tensors")
    B, K, _ = qkv.shape
    _, Hv, dv, dk = S_in.shape
    gs = Hv if gate_stride is None else int(gate_stride)
    _check(_L().gdn_verify_ex(_p(qkv), _p(beta_raw), _p(alpha), gs, _p(dt_bias), _p(A_log), _p(S_in),
                                _p(S_out), _p(H), _p(o), _p(lens), B, K, Hk, Hv, dk, dv, _dtype(qkv), _dtype(o),
                                float(eps), _stream(stream)))


def rollback(accept, K, S_in, H, S_out, hist=None, win=None, lens=None, stream=None):
    """gdn_rollback(_ex): accept [B] int32 (device), S_in/S_out [B][Hv][dv][dk], H [B][K-1][...] or None;
    lens [B] int32 (device) for a ragged batch."""
    _dev(accept, S_in, H, S_out, hist, win, lens)
    B, Hv, dv, dk = S_in.shape
    if hist is not None:
        W = hist.shape[1] + 1
        C = hist.shape[2]
        io = _dtype(hist)
    else:
        W, C, io = 2, 1, GDN_F32
    _check(_L().gdn_rollback_ex(_p(accept), _p(lens), int(K), _p(S_in), _p(H), _p(S_out), _p(hist), _p(win),
                                  B, Hv, dv, dk, C, W, io, _stream(stream)))


def rollback_conv_step(accept, K_prev, S_in, H, S_out, win_prev, x, w, hist, y, win, stream=None):
    """gdn_rollback_conv_step: gdn_rollback of the previous window (accept, K_prev, S_in, H, S_out, win_prev)
    then gdn_conv_step of x [B][T][C] into y and win [B][W-1+T][C], in one launch; hist is written only."""
    _dev(accept, S_in, H, S_out, win_prev, x, w, hist, y, win)
    B, Hv, dv, dk = S_in.shape
    _, T, C = x.shape
    W = w.shape[1]
    _check(_L().gdn_rollback_conv_step(_p(accept), int(K_prev), _p(S_in), _p(H), _p(S_out), _p(win_prev), _p(x),
                                         _p(w), _p(hist), _p(y), _p(win), B, Hv, dv, dk, T, C, W, _dtype(x),
                                         _stream(stream)))


def replay(accept, qkv, beta_raw, alpha, dt_bias, A_log, S_ckpt, S_out, Hk, hist=None, win=None, eps=1e-6,
           stream=None):
    """gdn_replay: S_out <- state after accept[b] tokens of the window from the checkpoint S_ckpt (untouched when
    accept[b] == K); hist <- win rows accept[b].. when given."""
    _dev(accept, qkv, beta_raw, alpha, dt_bias, A_log, S_ckpt, S_out, hist, win)
    B, K, _ = qkv.shape
    _, Hv, dv, dk = S_ckpt.shape
    W = hist.shape[1] + 1 if hist is not None else 2
    _check(_L().gdn_replay(_p(accept), _p(qkv), _p(beta_raw), _p(alpha), Hv, _p(dt_bias), _p(A_log), _p(S_ckpt),
                             _p(S_out), _p(hist), _p(win), B, K, Hk, Hv, dk, dv, W, _dtype(qkv), float(eps),
                             _stream(stream)))


def prefill_chunked(qkv, beta_raw, alpha, dt_bias, A_log, S_in, S_out, o, Hk, chunk=64, eps=1e-6, stream=None):
    """gdn_prefill_chunked: qkv [B][T][C], gates [B][T][Hv], S [B][Hv][dv][dk], o [B][T][Hv][dv]."""
    _dev(qkv, beta_raw, alpha, dt_bias, A_log, S_in, S_out, o)
    B, T, _ = qkv.shape
    _, Hv, dv, dk = S_in.shape
    _check(_L().gdn_prefill_chunked(_p(qkv), _p(beta_raw), _p(alpha), _p(dt_bias), _p(A_log), _p(S_in),
                                      _p(S_out), _p(o), B, T, int(chunk), Hk, Hv, dk, dv, _dtype(qkv), _dtype(o),
                                      float(eps), _stream(stream)))


def conv_tree(x, w, hist, parent, y, stream=None):
    """gdn_conv_tree: x [B][N][C], w [C][W], hist [B][W-1][C] (read only), parent [B][N] int32 -> y [B][N][C]."""
    _dev(x, w, hist, parent, y)
    B, N, C = x.shape
    W = w.shape[1]
    _check(_L().gdn_conv_tree(_p(x), _p(w), _p(hist), _p(parent), _p(y), B, N, C, W, _dtype(x), _stream(stream)))


def verify_tree(qkv, beta_raw, alpha, dt_bias, A_log, parent, S_in, H, o, Hk, eps=1e-6, gate_stride=None,
                stream=None):
    """gdn_verify_tree: qkv [B][N][C], gates [B][N][Hv] (or a strided view with gate_stride), parent [B][N]
    int32, S_in [B][Hv][dv][dk] -> H [B][N][Hv][dv][dk] (every node's state), o [B][N][Hv][dv]."""
    if gate_stride is None:
        _dev(beta_raw, alpha)
        gate_stride = S_in.shape[1]
    elif not (beta_raw.is_cuda and alpha.is_cuda):
        raise ValueError("libgdn takes device tensors")
    _dev(qkv, dt_bias, A_log, parent, S_in, H, o)
    B, N, _ = qkv.shape
    _, Hv, dv, dk = S_in.shape
    _check(_L().gdn_verify_tree(_p(qkv), _p(beta_raw), _p(alpha), int(gate_stride), _p(dt_bias), _p(A_log),
                                  _p(parent), _p(S_in), _p(H), _p(o), B, N, Hk, Hv, dk, dv, _dtype(qkv), _dtype(o),
                                  float(eps), _stream(stream)))


def rollback_tree(node, parent, S_in, H, S_out, x=None, hist=None, stream=None):
    """gdn_rollback_tree: node [B] int32 (outside [0, N): nothing kept), parent [B][N], H [B][N][...];
    S_out <- H[node] or S_in, hist <- the W-1 newest rows of [hist ; x along the path] when x/hist given."""
    _dev(node, parent, S_in, H, S_out, x, hist)
    B, N = parent.shape
    _, Hv, dv, dk = S_in.shape
    if hist is not None:
        W, C, io = hist.shape[1] + 1, hist.shape[2], _dtype(hist)
    else:
        W, C, io = 2, 1, GDN_F32
    _check(_L().gdn_rollback_tree(_p(node), _p(parent), N, _p(S_in), _p(H), _p(S_out), _p(x), _p(hist),
                                    B, Hv, dv, dk, C, W, io, _stream(stream)))


def verify_step(x, w, beta_raw, alpha, dt_bias, A_log, S_out, H, o, Hk, prev=None, S_in=None, hist=None,
                S_ckpt=None, y=None, win=None, eps=1e-6, gate_stride=None, stream=None):
    """gdn_verify_step: rollback of the previous window + conv step + verify in one launch.

    prev = (accept, S_ckpt, H, S_out, win) of the previous step (K_prev from its window), or None with
    S_in, hist for the first window.  x [B][K][C] raw tokens, w [C][4]; outputs S_out, H, o and the
    optional S_ckpt (this window's start state), y (conv outputs) and win (this window's conv window)."""
    if gate_stride is None:
        _dev(beta_raw, alpha)
        gate_stride = S_out.shape[1]
    elif not (beta_raw.is_cuda and alpha.is_cuda):
        raise ValueError("libgdn takes device tensors")
    _dev(x, w, dt_bias, A_log, S_out, H, o, S_in, hist, S_ckpt, y, win)
    B, K, C = x.shape
    _, Hv, dv, dk = S_out.shape
    W = w.shape[1]
    if prev is not None:
        acc, p_ckpt, p_H, p_out, p_win = prev
        _dev(acc, p_ckpt, p_H, p_out, p_win)
        K_prev = p_win.shape[1] - (W - 1)
    else:
        acc = p_ckpt = p_H = p_out = p_win = None
        K_prev = 0
    _check(_L().gdn_verify_step(_p(acc), int(K_prev), _p(p_ckpt), _p(p_H), _p(p_out), _p(p_win), _p(S_in),
                                  _p(hist), _p(x), _p(w), _p(beta_raw), _p(alpha), int(gate_stride), _p(dt_bias),
                                  _p(A_log), _p(S_ckpt), _p(S_out), _p(H), _p(o), _p(y), _p(win), B, K, Hk, Hv, dk,
                                  dv, W, _dtype(x), _dtype(o), float(eps), _stream(stream)))


def verify_tree_step(x, w, parent, beta_raw, alpha, dt_bias, A_log, H, o, y, Hk, S_prev_ckpt, hist_prev,
                     prev=None, S_ckpt=None, hist_out=None, eps=1e-6, gate_stride=None, stream=None):
    """gdn_verify_tree_step: rollback of the previous tree to its accepted node + conv_tree + verify_tree, two
    launches. x [B][N][C] raw tokens, parent [B][N] int32, H [B][N][Hv][dv][dk], o [B][N][Hv][dv], y [B][N][C];
    S_prev_ckpt [B][Hv][dv][dk] and hist_prev [B][W-1][C]: the previous tree's start state and history (for the
    first tree the committed state and history); prev = (node_prev [B] int32, parent_prev [B][N_prev],
    H_prev [B][N_prev][...], x_prev [B][N_prev][C]) or None for the first tree; S_ckpt and hist_out receive this
    tree's start state and history."""
    _dev(x, w, parent, dt_bias, A_log, H, o, y, S_prev_ckpt, hist_prev, S_ckpt, hist_out)
    if gate_stride is None:
        _dev(beta_raw, alpha)
    elif not (beta_raw.is_cuda and alpha.is_cuda):
        raise ValueError("libgdn takes device tensors")
    B, N, C = x.shape
    W = w.shape[1]
    _, Hv, dv, dk = S_prev_ckpt.shape
    node_prev = parent_prev = H_prev = x_prev = None
    N_prev = 0
    if prev is not None:
        node_prev, parent_prev, H_prev, x_prev = prev
        _dev(node_prev, parent_prev, H_prev, x_prev)
        N_prev = parent_prev.shape[1]
    gs = Hv if gate_stride is None else int(gate_stride)
    _check(_L().gdn_verify_tree_step(_p(node_prev), N_prev, _p(parent_prev), _p(S_prev_ckpt), _p(H_prev), _p(x_prev),
                                     _p(hist_prev), _p(x), _p(w), _p(parent), _p(beta_raw), _p(alpha), gs,
                                     _p(dt_bias), _p(A_log), _p(S_ckpt), _p(H), _p(o), _p(y), _p(hist_out),
                                     B, N, Hk, Hv, dk, dv, W, _dtype(x), _dtype(o), float(eps), _stream(stream)))
