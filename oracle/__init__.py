"""CPU oracle for the GDN speculative-verify step -- TEST INFRASTRUCTURE ONLY.

The plain, slow, sequential reference that the HIP path is checked against.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` import it; the library in ``speculative_verify_gdn_amd`` never
does, and the two share no code.

The arithmetic lives in ``gdn_oracle.c`` (double precision for the GDN part,
a float version of the conv step with a fixed rounding order for the
bit-exact check).  This module compiles it with gcc and wraps it for numpy
arrays; the C source cites the passage each function follows.

``Oracle(path)`` wraps any build of the C source (the tests load deliberately
broken copies to show that the pins catch them); the module-level functions
use the default build ``oracle/liboracle.so``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "gdn_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11"]


def build(force: bool = False, src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle C source with gcc (no vendor math, fp-contract off)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, src, "-lm"])
        os.replace(tmp, out)
    return out


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _f32(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.float32))


class Oracle:
    """numpy front end of one build of gdn_oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P, I, L, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_long, ctypes.c_double
        lib.oracle_exp32_constants.argtypes = [P]
        lib.oracle_exp32_array.argtypes = [P, P, L]
        lib.oracle_silu32_array.argtypes = [P, P, L]
        lib.oracle_bf16_rne_array.argtypes = [P, P, L]
        lib.oracle_conv_step_f32.argtypes = [P, P, P, P, P, P, I, I, I, I, I]
        lib.oracle_conv_step_f64.argtypes = [P, P, P, P, P, P, P, I, I, I, I]
        lib.oracle_gates_f64.argtypes = [P, P, P, P, P, P, I, I]
        lib.oracle_gdn_recurrent_f64.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, D]
        lib.oracle_gdn_chunked_f64.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, D, I]
        lib.oracle_rollback.argtypes = [P, I, I, P, P, P, L, P, P, L, I]
        lib.oracle_conv_tree_f32.argtypes = [P, P, P, P, P, I, I, I, I, I]
        lib.oracle_gdn_tree_f64.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, D]
        lib.oracle_tree_rollback.argtypes = [P, P, I, I, P, P, P, L, P, P, I, I, I]
        self.lib = lib
        self.path = path

    # ------------------------------------------------------------------
    # float primitives of the bit-exact conv step
    # ------------------------------------------------------------------
    def exp32(self, x):
        """The conv step's float exp (Cody-Waite reduction + degree-7 Taylor)."""
        x = _f32(np.atleast_1d(x))
        out = np.empty_like(x)
        self.lib.oracle_exp32_array(_ptr(x), _ptr(out), x.size)
        return out

    def silu32(self, x):
        """p / (1 + exp32(-p)) with every step rounded to float."""
        x = _f32(np.atleast_1d(x))
        out = np.empty_like(x)
        self.lib.oracle_silu32_array(_ptr(x), _ptr(out), x.size)
        return out

    def bf16_rne_bits(self, x):
        """float32 -> bfloat16 bit pattern, round to nearest even."""
        x = _f32(np.atleast_1d(x))
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.oracle_bf16_rne_array(_ptr(x), _ptr(out), x.size)
        return out

    def exp32_constants(self):
        """(LOG2E, LN2_HI, LN2_LO, C0..C7) as the oracle's exp uses them."""
        out = np.empty(11, dtype=np.float32)
        self.lib.oracle_exp32_constants(_ptr(out))
        return out

    # ------------------------------------------------------------------
    # conv step
    # ------------------------------------------------------------------
    def conv_step_f32(self, x, w, hist, round_bf16: bool):
        """Same-precision conv step (fmaf chain, exp32, float divide, bf16 RNE).

        x [B][T][C], w [C][W], hist [B][W-1][C] (float32 values; bf16 inputs
        are passed as their exact float32 values).  Returns (y, hist_out, win).
        """
        x, w, hist = _f32(x), _f32(w), _f32(hist)
        B, T, C = x.shape
        W = w.shape[1]
        y = np.empty((B, T, C), np.float32)
        hist_out = np.empty((B, W - 1, C), np.float32)
        win = np.empty((B, W - 1 + T, C), np.float32)
        self.lib.oracle_conv_step_f32(_ptr(x), _ptr(w), _ptr(hist), _ptr(y), _ptr(hist_out), _ptr(win),
                                      B, T, C, W, int(bool(round_bf16)))
        return y, hist_out, win

    def conv_step_f64(self, x, w, hist):
        """Double-precision definition.  Returns (y, pre, hist_out, win)."""
        x, w, hist = _f64(x), _f64(w), _f64(hist)
        B, T, C = x.shape
        W = w.shape[1]
        y = np.empty((B, T, C))
        pre = np.empty((B, T, C))
        hist_out = np.empty((B, W - 1, C))
        win = np.empty((B, W - 1 + T, C))
        self.lib.oracle_conv_step_f64(_ptr(x), _ptr(w), _ptr(hist), _ptr(y), _ptr(pre), _ptr(hist_out),
                                      _ptr(win), B, T, C, W)
        return y, pre, hist_out, win

    # ------------------------------------------------------------------
    # gates and GDN
    # ------------------------------------------------------------------
    def gates_f64(self, beta_raw, alpha, dt_bias=None, A_log=None):
        """(beta, g) from raw gates [..][Hv]; dt_bias = A_log = None: already activated."""
        br, al = _f64(beta_raw), _f64(alpha)
        N, Hv = br.reshape(-1, br.shape[-1]).shape
        beta = np.empty_like(br)
        g = np.empty_like(br)
        self.lib.oracle_gates_f64(_ptr(br), _ptr(al), _ptr(_f64(dt_bias)), _ptr(_f64(A_log)),
                                  _ptr(beta), _ptr(g), N, Hv)
        return beta, g

    @staticmethod
    def _gdn_args(qkv, beta_raw, alpha, dt_bias, A_log, S_in, Hk):
        qkv = _f64(qkv)
        B, K, C = qkv.shape
        S_in = _f64(S_in)
        _, Hv, dv, dk = S_in.shape
        assert C == 2 * Hk * dk + Hv * dv, "C must be 2*Hk*dk + Hv*dv"
        assert Hv % Hk == 0
        br, al = _f64(beta_raw), _f64(alpha)
        assert br.shape == (B, K, Hv) and al.shape == (B, K, Hv)
        dt, alog = _f64(dt_bias), _f64(A_log)
        assert (dt is None) == (alog is None)
        return qkv, br, al, dt, alog, S_in, B, K, Hv, dv, dk

    def gdn_recurrent_f64(self, qkv, beta_raw, alpha, dt_bias, A_log, S_in, Hk, eps=1e-6, capture=True):
        """Sequential definition.  Returns (S_out, H or None, o)."""
        qkv, br, al, dt, alog, S_in, B, K, Hv, dv, dk = self._gdn_args(qkv, beta_raw, alpha, dt_bias,
                                                                       A_log, S_in, Hk)
        S_out = np.empty_like(S_in)
        H = np.empty((B, max(K - 1, 0), Hv, dv, dk)) if capture else None
        o = np.empty((B, K, Hv, dv))
        self.lib.oracle_gdn_recurrent_f64(_ptr(qkv), _ptr(br), _ptr(al), _ptr(dt), _ptr(alog), _ptr(S_in),
                                          _ptr(S_out), _ptr(H) if (capture and K > 1) else None, _ptr(o),
                                          B, K, Hk, Hv, dk, dv, float(eps))
        return S_out, H, o

    def gdn_chunked_f64(self, qkv, beta_raw, alpha, dt_bias, A_log, S_in, Hk, chunk, eps=1e-6, capture=True):
        """Chunkwise WY form.  Returns (S_out, H or None, o)."""
        qkv, br, al, dt, alog, S_in, B, K, Hv, dv, dk = self._gdn_args(qkv, beta_raw, alpha, dt_bias,
                                                                       A_log, S_in, Hk)
        S_out = np.empty_like(S_in)
        H = np.empty((B, max(K - 1, 0), Hv, dv, dk)) if capture else None
        o = np.empty((B, K, Hv, dv))
        self.lib.oracle_gdn_chunked_f64(_ptr(qkv), _ptr(br), _ptr(al), _ptr(dt), _ptr(alog), _ptr(S_in),
                                        _ptr(S_out), _ptr(H) if (capture and K > 1) else None, _ptr(o),
                                        B, K, Hk, Hv, dk, dv, float(eps), int(chunk))
        return S_out, H, o

    def rollback(self, accept, K, S_in, H, S_out, win=None, hist=None):
        """Byte-copy rollback on numpy arrays of any element type.

        S_in, S_out [B][...state...]; H [B][K-1][...state...] (None only if
        K == 1); win [B][W-1+K][C]; hist [B][W-1][C] (both None to skip the
        conv part).  S_out and hist are modified in place.
        """
        acc = np.ascontiguousarray(np.asarray(accept, dtype=np.int32))
        B = S_out.shape[0]
        assert S_out.flags.c_contiguous and S_in.flags.c_contiguous
        state_bytes = S_out.nbytes // B
        if hist is not None:
            assert hist.flags.c_contiguous and win.flags.c_contiguous
            W = hist.shape[1] + 1
            row_bytes = hist.nbytes // (B * (W - 1)) if W > 1 else 0
        else:
            W, row_bytes = 1, 0
        self.lib.oracle_rollback(_ptr(acc), int(K), int(B), _ptr(S_in), _ptr(H) if H is not None else None,
                                 _ptr(S_out), state_bytes, _ptr(win) if win is not None else None,
                                 _ptr(hist) if hist is not None else None, row_bytes, W)

    # ------------------------------------------------------------------
    # tree verify
    # ------------------------------------------------------------------
    @staticmethod
    def _parent(parent, B, N):
        p = np.ascontiguousarray(np.asarray(parent, dtype=np.int32))
        assert p.shape == (B, N), "parent must be [B][N]"
        return p

    def conv_tree_f32(self, x, w, hist, parent, round_bf16: bool):
        """Conv of every node of a draft tree, same precision as conv_step_f32.

        x [B][N][C], w [C][W], hist [B][W-1][C] (not modified), parent [B][N]
        (an entry outside [0, i) marks a root).  Returns y [B][N][C].
        """
        x, w, hist = _f32(x), _f32(w), _f32(hist)
        B, N, C = x.shape
        W = w.shape[1]
        par = self._parent(parent, B, N)
        y = np.empty((B, N, C), np.float32)
        self.lib.oracle_conv_tree_f32(_ptr(x), _ptr(w), _ptr(hist), _ptr(par), _ptr(y), B, N, C, W,
                                      int(bool(round_bf16)))
        return y

    def gdn_tree_f64(self, qkv, beta_raw, alpha, dt_bias, A_log, parent, S_in, Hk, eps=1e-6):
        """GDN over a draft tree, one step per node from its parent's state.

        Returns (H [B][N][Hv][dv][dk], o [B][N][Hv][dv]).
        """
        qkv, br, al, dt, alog, S_in, B, N, Hv, dv, dk = self._gdn_args(qkv, beta_raw, alpha, dt_bias,
                                                                       A_log, S_in, Hk)
        par = self._parent(parent, B, N)
        H = np.empty((B, N, Hv, dv, dk))
        o = np.empty((B, N, Hv, dv))
        self.lib.oracle_gdn_tree_f64(_ptr(qkv), _ptr(br), _ptr(al), _ptr(dt), _ptr(alog), _ptr(par), _ptr(S_in),
                                     _ptr(H), _ptr(o), B, N, Hk, Hv, dk, dv, float(eps))
        return H, o

    def tree_rollback(self, node, parent, S_in, H, S_out, x=None, hist=None):
        """Byte-copy rollback to a tree node on numpy arrays of any element type.

        node [B] (outside [0, N): nothing accepted), parent [B][N],
        S_in, S_out [B][...state...], H [B][N][...state...], x [B][N][C],
        hist [B][W-1][C].  S_out and hist are modified in place.
        """
        B, N = H.shape[0], H.shape[1]
        nd = np.ascontiguousarray(np.asarray(node, dtype=np.int32))
        par = self._parent(parent, B, N)
        assert S_out.flags.c_contiguous and S_in.flags.c_contiguous and H.flags.c_contiguous
        state_bytes = S_out.nbytes // B
        if hist is not None:
            assert hist.flags.c_contiguous and x.flags.c_contiguous and hist.dtype == x.dtype
            W, C, eb = hist.shape[1] + 1, hist.shape[2], hist.itemsize
        else:
            W, C, eb = 1, 0, 1
        self.lib.oracle_tree_rollback(_ptr(nd), _ptr(par), int(N), int(B), _ptr(S_in), _ptr(H), _ptr(S_out),
                                      state_bytes, _ptr(x) if hist is not None else None,
                                      _ptr(hist) if hist is not None else None, C, W, eb)


_lock = threading.Lock()
_default = None


def default() -> Oracle:
    global _default
    with _lock:
        if _default is None:
            _default = Oracle(build())
        return _default


def __getattr__(name):
    # module-level access to the default build: oracle.gdn_recurrent_f64(...)
    if name in ("exp32", "silu32", "bf16_rne_bits", "exp32_constants", "conv_step_f32", "conv_step_f64",
                "gates_f64", "gdn_recurrent_f64", "gdn_chunked_f64", "rollback", "conv_tree_f32", "gdn_tree_f64",
                "tree_rollback"):
        return getattr(default(), name)
    raise AttributeError(name)


def split_qkv(y, Hk, Hv, dk, dv):
    """Views of the conv output slab: q [.., Hk, dk], k [.., Hk, dk], v [.., Hv, dv]."""
    q = y[..., : Hk * dk].reshape(*y.shape[:-1], Hk, dk)
    k = y[..., Hk * dk: 2 * Hk * dk].reshape(*y.shape[:-1], Hk, dk)
    v = y[..., 2 * Hk * dk:].reshape(*y.shape[:-1], Hv, dv)
    return q, k, v
