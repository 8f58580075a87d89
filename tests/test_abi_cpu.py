"""The C ABI without a GPU: the library loads, exports every entry point that
include/gdn.h declares, and rejects every invalid argument on the host with
the documented status code before anything is launched.

Fake device addresses are fine here because validation fails (or B == 0
returns) before any HIP call.
"""
import ctypes
import os
import re
import subprocess

import pytest

from speculative_verify_gdn_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

A = 0x7F0000000000  # a fake, 16-byte aligned "device" address; never dereferenced
MB = 1 << 24


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.LIB_PATH):
        pytest.skip("libgdn.so not built")
    return gdn.load()


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(gdn.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (gdn_[a-z_]+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_debug_library_exports_every_declared_symbol():
    if not os.path.exists(gdn.DEBUG_LIB_PATH):
        pytest.skip("libgdn_debug.so not built")
    dbg = gdn.open_library(gdn.DEBUG_LIB_PATH)
    for name in declared_functions():
        assert hasattr(dbg, name), name
    # a null count is rejected on the host (no device access)
    assert dbg.gdn_debug_clamped_accepts(None, 0) == gdn.GDN_EINVAL


def test_release_library_counts_no_clamped_accepts(lib):
    n = ctypes.c_longlong(-1)
    assert lib.gdn_debug_clamped_accepts(ctypes.byref(n), 0) == gdn.GDN_EUNSUPPORTED
    assert n.value == -1
    assert b"debug build" in lib.gdn_last_error()
    with pytest.raises(gdn.GdnError):
        gdn.debug_clamped_accepts()


def test_version_matches_header(lib):
    m = re.search(r"#define GDN_VERSION (\d+)", open(HEADER).read())
    assert lib.gdn_version() == int(m.group(1))


def p(off=0):
    return ctypes.c_void_p(A + off * MB)


def verify_call(lib, **kw):
    args = dict(qkv=p(0), beta=p(1), alpha=p(2), dt=p(3), alog=p(4), S_in=p(5), S_out=p(6), H=p(8), o=p(12),
                B=1, K=4, Hk=2, Hv=2, dk=32, dv=32, ind=gdn.GDN_F32, od=gdn.GDN_F32, eps=1e-6)
    args.update(kw)
    return lib.gdn_verify(args["qkv"], args["beta"], args["alpha"], args["dt"], args["alog"], args["S_in"],
                          args["S_out"], args["H"], args["o"], args["B"], args["K"], args["Hk"], args["Hv"],
                          args["dk"], args["dv"], args["ind"], args["od"], args["eps"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(qkv=None), gdn.GDN_EINVAL),
    (dict(S_in=None), gdn.GDN_EINVAL),
    (dict(o=None), gdn.GDN_EINVAL),
    (dict(qkv=ctypes.c_void_p(A + 4)), gdn.GDN_EINVAL),          # misaligned
    (dict(K=0), gdn.GDN_EINVAL),
    (dict(K=65), gdn.GDN_EUNSUPPORTED),
    (dict(dk=48, dv=48), gdn.GDN_EUNSUPPORTED),
    (dict(dv=20), gdn.GDN_EUNSUPPORTED),
    (dict(Hk=2, Hv=3), gdn.GDN_EINVAL),
    (dict(Hk=0), gdn.GDN_EINVAL),
    (dict(B=-1), gdn.GDN_EINVAL),
    (dict(dt=None), gdn.GDN_EINVAL),                              # one of the two gate params
    (dict(ind=7), gdn.GDN_EINVAL),
    (dict(eps=-1.0), gdn.GDN_EINVAL),
    (dict(S_out=ctypes.c_void_p(A + 5 * MB + 64)), gdn.GDN_EINVAL),  # partial overlap with S_in
    (dict(H=ctypes.c_void_p(A + 5 * MB)), gdn.GDN_EINVAL),        # H overlaps S_in
    (dict(o=ctypes.c_void_p(A + 0)), gdn.GDN_EINVAL),             # o overlaps qkv
])
def test_verify_rejects(lib, kw, code):
    assert verify_call(lib, **kw) == code
    assert lib.gdn_last_error().decode().startswith("gdn_verify")


def test_verify_empty_batch_is_ok(lib):
    assert verify_call(lib, B=0) == gdn.GDN_OK
    assert lib.gdn_last_error().decode() == ""


def conv_call(lib, **kw):
    a = dict(x=p(0), w=p(1), hist=p(2), y=p(3), win=p(4), B=1, T=4, C=192, W=4, io=gdn.GDN_BF16)
    a.update(kw)
    return lib.gdn_conv_step(a["x"], a["w"], a["hist"], a["y"], a["win"], a["B"], a["T"], a["C"], a["W"], a["io"],
                             None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), gdn.GDN_EINVAL),
    (dict(hist=None), gdn.GDN_EINVAL),
    (dict(T=0), gdn.GDN_EINVAL),
    (dict(C=0), gdn.GDN_EINVAL),
    (dict(W=1), gdn.GDN_EUNSUPPORTED),
    (dict(W=9), gdn.GDN_EUNSUPPORTED),
    (dict(io=5), gdn.GDN_EINVAL),
    (dict(y=p(0)), gdn.GDN_EINVAL),                                # y aliases x
    (dict(win=p(3)), gdn.GDN_EINVAL),                              # win aliases y
    (dict(hist=ctypes.c_void_p(A + 2 * MB + 2)), gdn.GDN_EINVAL),  # misaligned
])
def test_conv_rejects(lib, kw, code):
    assert conv_call(lib, **kw) == code


def test_conv_empty_batch_is_ok(lib):
    assert conv_call(lib, B=0) == gdn.GDN_OK


def rollback_call(lib, **kw):
    a = dict(acc=p(0), K=4, S_in=p(1), H=p(2), S_out=p(6), hist=p(8), win=p(9), B=1, Hv=2, dv=32, dk=32, C=192,
             W=4, io=gdn.GDN_BF16)
    a.update(kw)
    return lib.gdn_rollback(a["acc"], a["K"], a["S_in"], a["H"], a["S_out"], a["hist"], a["win"], a["B"], a["Hv"],
                            a["dv"], a["dk"], a["C"], a["W"], a["io"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(acc=None), gdn.GDN_EINVAL),
    (dict(K=0), gdn.GDN_EINVAL),
    (dict(H=None), gdn.GDN_EINVAL),             # needed for K > 1
    (dict(S_out=p(1)), gdn.GDN_EINVAL),         # in place is not recoverable
    (dict(hist=None), gdn.GDN_EINVAL),          # hist without win
    (dict(W=1), gdn.GDN_EUNSUPPORTED),
    (dict(S_out=p(2)), gdn.GDN_EINVAL),         # overlaps H
])
def test_rollback_rejects(lib, kw, code):
    assert rollback_call(lib, **kw) == code


def test_rollback_k1_without_capture_and_empty_batch(lib):
    assert rollback_call(lib, B=0) == gdn.GDN_OK


def rollconv_call(lib, **kw):
    a = dict(acc=p(0), Kp=4, S_in=p(1), H=p(2), S_out=p(6), win_prev=p(9), x=p(10), w=p(11), hist=p(12), y=p(13),
             win=p(14), B=1, Hv=2, dv=32, dk=32, T=4, C=192, W=4, io=gdn.GDN_BF16)
    a.update(kw)
    return lib.gdn_rollback_conv_step(a["acc"], a["Kp"], a["S_in"], a["H"], a["S_out"], a["win_prev"], a["x"],
                                      a["w"], a["hist"], a["y"], a["win"], a["B"], a["Hv"], a["dv"], a["dk"],
                                      a["T"], a["C"], a["W"], a["io"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(acc=None), gdn.GDN_EINVAL),
    (dict(Kp=0), gdn.GDN_EINVAL),
    (dict(T=0), gdn.GDN_EINVAL),
    (dict(H=None), gdn.GDN_EINVAL),              # needed for K_prev > 1
    (dict(win=None), gdn.GDN_EINVAL),            # the new window is required
    (dict(S_out=p(1)), gdn.GDN_EINVAL),          # the pre-window state is needed
    (dict(win=p(9)), gdn.GDN_EINVAL),            # new window on the previous one
    (dict(y=p(10)), gdn.GDN_EINVAL),             # y on x
    (dict(hist=p(13)), gdn.GDN_EINVAL),          # two outputs on each other
    (dict(W=9), gdn.GDN_EUNSUPPORTED),
    (dict(io=7), gdn.GDN_EINVAL),
    (dict(hist=ctypes.c_void_p(A + 12 * MB + 4)), gdn.GDN_EINVAL),  # misaligned
])
def test_rollback_conv_rejects(lib, kw, code):
    assert rollconv_call(lib, **kw) == code


def test_rollback_conv_empty_batch_is_ok(lib):
    assert rollconv_call(lib, B=0) == gdn.GDN_OK


def verify_ex_call(lib, **kw):
    a = dict(qkv=p(0), beta=p(1), alpha=p(2), gs=2, dt=p(3), alog=p(4), S_in=p(5), S_out=p(6), H=p(7), o=p(8),
             lens=p(9), B=1, K=4, Hk=2, Hv=2, dk=32, dv=32, ind=gdn.GDN_BF16, od=gdn.GDN_F32, eps=1e-6)
    a.update(kw)
    return lib.gdn_verify_ex(a["qkv"], a["beta"], a["alpha"], a["gs"], a["dt"], a["alog"], a["S_in"], a["S_out"],
                             a["H"], a["o"], a["lens"], a["B"], a["K"], a["Hk"], a["Hv"], a["dk"], a["dv"], a["ind"],
                             a["od"], a["eps"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(gs=1), gdn.GDN_EINVAL),                                  # gate rows narrower than Hv
    (dict(lens=ctypes.c_void_p(A + 9 * MB + 2)), gdn.GDN_EINVAL),  # lens misaligned
    (dict(beta=ctypes.c_void_p(A + MB + 1)), gdn.GDN_EINVAL),      # bf16 gate misaligned
    (dict(lens=p(6)), gdn.GDN_EINVAL),                             # S_out over lens
    (dict(o=p(1)), gdn.GDN_EINVAL),                                # o over the gates
])
def test_verify_ex_rejects(lib, kw, code):
    assert verify_ex_call(lib, **kw) == code


def test_ex_forms_empty_batch_is_ok(lib):
    assert verify_ex_call(lib, B=0) == gdn.GDN_OK
    assert lib.gdn_conv_step_ex(p(0), p(1), p(2), p(3), p(4), p(5), 0, 4, 192, 4, gdn.GDN_BF16, None) == gdn.GDN_OK
    assert lib.gdn_rollback_ex(p(0), p(1), 4, p(2), p(3), p(6), None, None, 0, 2, 32, 32, 1, 2, gdn.GDN_F32,
                               None) == gdn.GDN_OK


def test_ex_forms_reject_misaligned_lens(lib):
    bad = ctypes.c_void_p(A + 5 * MB + 2)
    assert lib.gdn_conv_step_ex(p(0), p(1), p(2), p(3), p(4), bad, 1, 4, 192, 4, gdn.GDN_BF16,
                                None) == gdn.GDN_EINVAL
    assert lib.gdn_rollback_ex(p(0), bad, 4, p(2), p(3), p(6), None, None, 1, 2, 32, 32, 1, 2, gdn.GDN_F32,
                               None) == gdn.GDN_EINVAL


def replay_call(lib, **kw):
    a = dict(acc=p(0), qkv=p(1), beta=p(2), alpha=p(3), gs=2, dt=p(4), alog=p(5), S_c=p(6), S_out=p(7), hist=p(8),
             win=p(9), B=1, K=4, Hk=2, Hv=2, dk=32, dv=32, W=4, ind=gdn.GDN_BF16, eps=1e-6)
    a.update(kw)
    return lib.gdn_replay(a["acc"], a["qkv"], a["beta"], a["alpha"], a["gs"], a["dt"], a["alog"], a["S_c"],
                          a["S_out"], a["hist"], a["win"], a["B"], a["K"], a["Hk"], a["Hv"], a["dk"], a["dv"], a["W"],
                          a["ind"], a["eps"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(acc=None), gdn.GDN_EINVAL),
    (dict(S_out=p(6)), gdn.GDN_EINVAL),        # the checkpoint must survive
    (dict(hist=None), gdn.GDN_EINVAL),         # hist without win
    (dict(gs=1), gdn.GDN_EINVAL),
    (dict(K=65), gdn.GDN_EUNSUPPORTED),
    (dict(S_out=p(1)), gdn.GDN_EINVAL),        # over qkv
    (dict(W=9), gdn.GDN_EUNSUPPORTED),
])
def test_replay_rejects(lib, kw, code):
    assert replay_call(lib, **kw) == code


def test_replay_empty_batch_is_ok(lib):
    assert replay_call(lib, B=0) == gdn.GDN_OK


def prefill_call(lib, **kw):
    a = dict(qkv=p(0), beta=p(1), alpha=p(2), dt=p(3), alog=p(4), S_in=p(5), S_out=p(6), o=p(8), B=1, T=100,
             chunk=64, Hk=2, Hv=2, dk=32, dv=32, ind=gdn.GDN_BF16, od=gdn.GDN_BF16, eps=1e-6)
    a.update(kw)
    return lib.gdn_prefill_chunked(a["qkv"], a["beta"], a["alpha"], a["dt"], a["alog"], a["S_in"], a["S_out"],
                                   a["o"], a["B"], a["T"], a["chunk"], a["Hk"], a["Hv"], a["dk"], a["dv"], a["ind"],
                                   a["od"], a["eps"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(chunk=48), gdn.GDN_EUNSUPPORTED),
    (dict(T=0), gdn.GDN_EINVAL),
    (dict(o=None), gdn.GDN_EINVAL),
    (dict(alog=None), gdn.GDN_EINVAL),
    (dict(dk=16, dv=16), gdn.GDN_EUNSUPPORTED),
])
def test_prefill_rejects(lib, kw, code):
    assert prefill_call(lib, **kw) == code


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(gdn, "_lib", None)
    with pytest.raises(FileNotFoundError):
        gdn.load(str(tmp_path / "missing.so"))


def conv_tree_call(lib, **kw):
    a = dict(x=p(0), w=p(1), hist=p(2), par=p(3), y=p(4), B=1, N=8, C=64, W=4, io=gdn.GDN_BF16)
    a.update(kw)
    return lib.gdn_conv_tree(a["x"], a["w"], a["hist"], a["par"], a["y"], a["B"], a["N"], a["C"], a["W"], a["io"],
                             None)


@pytest.mark.parametrize("kw,code", [
    (dict(par=None), gdn.GDN_EINVAL),
    (dict(par=ctypes.c_void_p(A + 3 * MB + 2)), gdn.GDN_EINVAL),   # parent not 4-byte aligned
    (dict(N=0), gdn.GDN_EINVAL),
    (dict(N=33), gdn.GDN_EUNSUPPORTED),
    (dict(W=9), gdn.GDN_EUNSUPPORTED),
    (dict(y=p(0)), gdn.GDN_EINVAL),                                 # y over x
    (dict(y=p(3)), gdn.GDN_EINVAL),                                 # y over parent
    (dict(io=5), gdn.GDN_EINVAL),
])
def test_conv_tree_rejects(lib, kw, code):
    assert conv_tree_call(lib, **kw) == code


def verify_tree_call(lib, **kw):
    a = dict(qkv=p(0), beta=p(1), alpha=p(2), gs=2, dt=p(3), alog=p(4), par=p(5), S_in=p(6), H=p(8), o=p(12),
             B=1, N=8, Hk=2, Hv=2, dk=32, dv=32, ind=gdn.GDN_BF16, od=gdn.GDN_F32, eps=1e-6)
    a.update(kw)
    return lib.gdn_verify_tree(a["qkv"], a["beta"], a["alpha"], a["gs"], a["dt"], a["alog"], a["par"], a["S_in"],
                               a["H"], a["o"], a["B"], a["N"], a["Hk"], a["Hv"], a["dk"], a["dv"], a["ind"], a["od"],
                               a["eps"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(par=None), gdn.GDN_EINVAL),
    (dict(H=None), gdn.GDN_EINVAL),                 # every node's state is the output
    (dict(N=33), gdn.GDN_EUNSUPPORTED),
    (dict(N=0), gdn.GDN_EINVAL),
    (dict(gs=1), gdn.GDN_EINVAL),
    (dict(H=p(6)), gdn.GDN_EINVAL),                 # H over S_in
    (dict(o=p(5)), gdn.GDN_EINVAL),                 # o over parent
    (dict(dk=48, dv=48), gdn.GDN_EUNSUPPORTED),
    (dict(alog=None), gdn.GDN_EINVAL),
])
def test_verify_tree_rejects(lib, kw, code):
    assert verify_tree_call(lib, **kw) == code


def rollback_tree_call(lib, **kw):
    a = dict(node=p(0), par=p(1), N=8, S_in=p(2), H=p(3), S_out=p(6), x=p(7), hist=p(8), B=1, Hv=2, dv=32, dk=32,
             C=64, W=4, io=gdn.GDN_BF16)
    a.update(kw)
    return lib.gdn_rollback_tree(a["node"], a["par"], a["N"], a["S_in"], a["H"], a["S_out"], a["x"], a["hist"],
                                 a["B"], a["Hv"], a["dv"], a["dk"], a["C"], a["W"], a["io"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(node=None), gdn.GDN_EINVAL),
    (dict(S_out=p(2)), gdn.GDN_EINVAL),             # S_out must not be S_in
    (dict(S_out=p(3)), gdn.GDN_EINVAL),             # S_out over H
    (dict(hist=None), gdn.GDN_EINVAL),              # x without hist
    (dict(N=40), gdn.GDN_EUNSUPPORTED),
    (dict(W=1), gdn.GDN_EUNSUPPORTED),
    (dict(hist=p(7)), gdn.GDN_EINVAL),              # hist over x
])
def test_rollback_tree_rejects(lib, kw, code):
    assert rollback_tree_call(lib, **kw) == code


def test_tree_calls_empty_batch_are_ok(lib):
    assert conv_tree_call(lib, B=0) == gdn.GDN_OK
    assert verify_tree_call(lib, B=0) == gdn.GDN_OK
    assert rollback_tree_call(lib, B=0) == gdn.GDN_OK
    assert rollback_tree_call(lib, x=None, hist=None, B=0) == gdn.GDN_OK


def step_call(lib, **kw):
    a = dict(acc=p(0), Kp=16, pck=p(1), pH=p(2), pout=p(3), pwin=p(4), S_in=None, hist=None, x=p(5), w=p(6),
             beta=p(7), alpha=p(8), gs=2, dt=p(9), alog=p(10), ck=p(11), S_out=p(12), H=p(13), o=p(14), y=p(15),
             win=p(16), B=1, K=16, Hk=2, Hv=2, dk=32, dv=32, W=4, ind=gdn.GDN_BF16, od=gdn.GDN_F32, eps=1e-6)
    a.update(kw)
    return lib.gdn_verify_step(a["acc"], a["Kp"], a["pck"], a["pH"], a["pout"], a["pwin"], a["S_in"], a["hist"],
                               a["x"], a["w"], a["beta"], a["alpha"], a["gs"], a["dt"], a["alog"], a["ck"],
                               a["S_out"], a["H"], a["o"], a["y"], a["win"], a["B"], a["K"], a["Hk"], a["Hv"],
                               a["dk"], a["dv"], a["W"], a["ind"], a["od"], a["eps"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(W=3), gdn.GDN_EUNSUPPORTED),                       # the fused step takes conv width 4
    (dict(K=65), gdn.GDN_EUNSUPPORTED),
    (dict(Kp=0), gdn.GDN_EINVAL),
    (dict(Kp=65), gdn.GDN_EINVAL),                           # the previous window is a verify window too
    (dict(pck=None), gdn.GDN_EINVAL),                        # the previous window needs its checkpoint
    (dict(pH=None), gdn.GDN_EINVAL),                         # ... and its capture when K_prev > 1
    (dict(acc=None), gdn.GDN_EINVAL),                        # first window without S_in / hist
    (dict(x=None), gdn.GDN_EINVAL),
    (dict(S_out=p(3)), gdn.GDN_EINVAL),                      # S_out over the previous final state
    (dict(win=p(4)), gdn.GDN_EINVAL),                        # win over win_prev
    (dict(ck=p(12)), gdn.GDN_EINVAL),                        # two outputs overlap
    (dict(acc=ctypes.c_void_p(A + 2)), gdn.GDN_EINVAL),      # accept not 4-byte aligned
    (dict(gs=1), gdn.GDN_EINVAL),
])
def test_verify_step_rejects(lib, kw, code):
    assert step_call(lib, **kw) == code


def test_verify_step_first_window_and_empty_batch(lib):
    assert step_call(lib, B=0) == gdn.GDN_OK
    assert step_call(lib, acc=None, S_in=p(20), hist=p(21), B=0) == gdn.GDN_OK
    assert step_call(lib, acc=None, S_in=p(20), hist=None) == gdn.GDN_EINVAL


def tree_step_call(lib, **kw):
    a = dict(node=p(0), Np=16, ppar=p(1), pck=p(2), pH=p(3), px=p(4), phist=p(5), x=p(6), w=p(7), par=p(8),
             beta=p(9), alpha=p(10), gs=2, dt=p(11), alog=p(12), ck=p(13), H=p(14), o=p(15), y=p(16), hout=p(17),
             B=1, N=16, Hk=2, Hv=2, dk=32, dv=32, W=4, ind=gdn.GDN_BF16, od=gdn.GDN_F32, eps=1e-6)
    a.update(kw)
    return lib.gdn_verify_tree_step(a["node"], a["Np"], a["ppar"], a["pck"], a["pH"], a["px"], a["phist"], a["x"],
                                    a["w"], a["par"], a["beta"], a["alpha"], a["gs"], a["dt"], a["alog"], a["ck"],
                                    a["H"], a["o"], a["y"], a["hout"], a["B"], a["N"], a["Hk"], a["Hv"], a["dk"],
                                    a["dv"], a["W"], a["ind"], a["od"], a["eps"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(N=33), gdn.GDN_EUNSUPPORTED),                      # ancestor masks are 32-bit words
    (dict(W=9), gdn.GDN_EUNSUPPORTED),
    (dict(Np=0), gdn.GDN_EINVAL),
    (dict(Np=33), gdn.GDN_EINVAL),
    (dict(ppar=None), gdn.GDN_EINVAL),                       # a previous tree needs its parents,
    (dict(pH=None), gdn.GDN_EINVAL),                         # its node states
    (dict(px=None), gdn.GDN_EINVAL),                         # and its tokens
    (dict(pck=None), gdn.GDN_EINVAL),
    (dict(phist=None), gdn.GDN_EINVAL),
    (dict(y=None), gdn.GDN_EINVAL),                          # the verify reads the conv outputs
    (dict(H=None), gdn.GDN_EINVAL),
    (dict(hout=p(5)), gdn.GDN_EINVAL),                       # the history out over the history in
    (dict(ck=p(3)), gdn.GDN_EINVAL),                         # the checkpoint over the previous states
    (dict(ck=p(14)), gdn.GDN_EINVAL),                        # two outputs overlap
    (dict(node=ctypes.c_void_p(A + 2)), gdn.GDN_EINVAL),     # node not 4-byte aligned
    (dict(gs=1), gdn.GDN_EINVAL),
    (dict(dk=48), gdn.GDN_EUNSUPPORTED),
])
def test_verify_tree_step_rejects(lib, kw, code):
    assert tree_step_call(lib, **kw) == code


def test_verify_tree_step_first_tree_and_empty_batch(lib):
    assert tree_step_call(lib, B=0) == gdn.GDN_OK
    # the first tree needs none of the previous tree's buffers
    assert tree_step_call(lib, node=None, Np=0, ppar=None, pH=None, px=None, B=0) == gdn.GDN_OK
    assert tree_step_call(lib, node=None, Np=0, ppar=None, pH=None, px=None, phist=None) == gdn.GDN_EINVAL


def test_binding_routes_calls_to_another_build(lib):
    """gdn.using(lib) sends this thread's calls to another build of the library (here the debug build), and
    only inside the block."""
    if not os.path.exists(gdn.DEBUG_LIB_PATH):
        pytest.skip("libgdn_debug.so not built")
    dbg = gdn.open_library(gdn.DEBUG_LIB_PATH)
    assert gdn._L() is lib
    with gdn.using(dbg):
        assert gdn._L() is dbg
        assert gdn.version() == lib.gdn_version()
        with gdn.using(lib):
            assert gdn._L() is lib
        assert gdn._L() is dbg
    assert gdn._L() is lib
