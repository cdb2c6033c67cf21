"""Host-side tests of the C ABI (no GPU needed).

The library validates every argument before its first HIP call, so each
rejected call below returns its documented status without touching a device.
Pointers passed here are never dereferenced: they are fake addresses chosen
to exercise the NULL, alignment and overlap checks.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "eqlinear.h")
LIB = os.path.join(ROOT, "group_wise_dft_amd", "libeqlinear.so")

OK, NULL, SHAPE, UNSUP, ALIGN, WS, ALIAS, HIP = range(8)
F32, F16 = 0, 1


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from group_wise_dft_amd.build import build_library
        build_library()
    L = ctypes.CDLL(LIB)
    vp, i64, i32, sz, ci = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t,
                            ctypes.c_int)
    L.eqlinear_weight_spectrum.argtypes = [vp, vp, i64, i64, i32, ci, vp]
    L.eqlinear_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, ci, vp]
    L.eqlinear_backward_input.argtypes = [vp, vp, vp, i64, i64, i64, i32, ci, vp]
    L.eqlinear_backward_weight.argtypes = [vp, vp, vp, vp, sz, i64, i64, i64, i32, ci, vp]
    L.eqlinear_backward_bias.argtypes = [vp, vp, vp, sz, i64, i64, i32, ci, vp]
    L.eqlinear_bias_workspace_size.argtypes = [i64, i64, i32, ci]
    L.eqlinear_bias_workspace_size.restype = sz
    L.eqlinear_workspace_size.argtypes = [i64, i64, i64, i32, ci]
    L.eqlinear_workspace_size.restype = sz
    L.eqlinear_spectrum_size.argtypes = [i64, i64, i32, ci]
    L.eqlinear_spectrum_size.restype = sz
    L.eqlinear_status_string.argtypes = [ci]
    L.eqlinear_status_string.restype = ctypes.c_char_p
    return L


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(eqlinear_\w+)\s*\(", src)))


def test_header_declares_the_entry_points_and_helpers():
    names = declared_functions()
    for n in ("eqlinear_weight_spectrum", "eqlinear_forward", "eqlinear_backward_input",
              "eqlinear_backward_weight", "eqlinear_backward_bias", "eqlinear_workspace_size",
              "eqlinear_bias_workspace_size", "eqlinear_spectrum_size", "eqlinear_status_string"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(8):
        s = lib.eqlinear_status_string(code)
        assert s and s != b"unknown status"
    assert lib.eqlinear_status_string(99) == b"unknown status"


A = 0x10000000   # fake, 16-byte aligned, never dereferenced
B = 0x20000000
C = 0x30000000
D = 0x40000000


def fwd(lib, x=A, w=B, bias=None, y=C, N=64, C_T=16, D_T=16, T=4, dt=F32):
    return lib.eqlinear_forward(x, w, bias, y, N, C_T, D_T, T, dt, None)


def test_forward_validation(lib):
    assert fwd(lib, x=None) == NULL
    assert fwd(lib, w=None) == NULL
    assert fwd(lib, y=None) == NULL
    assert fwd(lib, N=-1) == SHAPE
    assert fwd(lib, C_T=-8) == SHAPE
    assert fwd(lib, T=9) == UNSUP
    assert fwd(lib, T=1) == UNSUP
    assert fwd(lib, T=16) == UNSUP
    assert fwd(lib, dt=7) == UNSUP
    assert fwd(lib, C_T=0) == UNSUP           # at least one channel each way
    assert fwd(lib, D_T=0) == UNSUP
    assert fwd(lib, bias=D + 8) == ALIGN
    assert fwd(lib, bias=C) == ALIAS          # bias inside y
    assert fwd(lib, bias=C + 64 * 16 * 4 * 4 - 16) == ALIAS   # tail of y
    assert fwd(lib, x=A + 8) == ALIGN
    assert fwd(lib, y=C + 4) == ALIGN
    assert fwd(lib, y=A) == ALIAS
    assert fwd(lib, y=A + 16 * 64) == ALIAS   # overlaps the tail of x
    assert fwd(lib, y=B) == ALIAS
    # w_hat holds both orientations (2*T*D_T*C_T elements): its second half
    # is an input too
    assert fwd(lib, y=B + 4 * 16 * 16 * 4 + 16) == ALIAS
    assert fwd(lib, C_T=65544) == UNSUP       # past the channel limit
    assert fwd(lib, C_T=65536, D_T=65536) == UNSUP   # spectrum >= 2 GiB
    # N == 0 is a valid no-op that returns before any HIP call
    assert fwd(lib, N=0) == OK
    assert fwd(lib, x=None, y=None, N=0) == OK


def test_backward_input_validation(lib):
    f = lambda **k: lib.eqlinear_backward_input(k.get("dy", A), k.get("w", B), k.get("dx", C),
                                                k.get("N", 64), k.get("C_T", 16), k.get("D_T", 16),
                                                k.get("T", 4), k.get("dt", F16), None)
    assert f(dy=None) == NULL
    assert f(dx=None) == NULL
    assert f(T=9) == UNSUP
    assert f(dx=A) == ALIAS
    assert f(dx=C + 2) == ALIGN
    assert f(N=0) == OK


def test_backward_weight_validation(lib):
    N, C_T, D_T, T = 12608, 192, 768, 4
    need = lib.eqlinear_workspace_size(N, C_T, D_T, T, F16)
    assert need > 0 and need % 16 == 0
    W = 0x50000000

    def f(**k):
        return lib.eqlinear_backward_weight(k.get("x", A), k.get("dy", B), k.get("dw", C),
                                            k.get("ws", W), k.get("wsb", need), k.get("N", N),
                                            C_T, D_T, T, F16, None)
    assert f(x=None) == NULL
    assert f(ws=None) == WS
    assert f(wsb=need - 1) == WS
    assert f(ws=W + 8) == ALIGN
    assert f(dw=A) == ALIAS
    assert f(ws=A) == ALIAS
    assert f(ws=C) == ALIAS
    assert f(N=-3) == SHAPE


def test_backward_bias_validation(lib):
    N, D_T, T = 12608, 768, 4
    need = lib.eqlinear_bias_workspace_size(N, D_T, T, F16)
    assert need > 0 and need % (4 * D_T) == 0
    assert lib.eqlinear_bias_workspace_size(N, D_T, T, F16) == need
    assert lib.eqlinear_bias_workspace_size(0, D_T, T, F16) == 0
    assert lib.eqlinear_bias_workspace_size(N, D_T, 9, F16) == 0
    assert lib.eqlinear_bias_workspace_size(N, 0, T, F16) == 0
    assert lib.eqlinear_bias_workspace_size(N, 13, T, F16) > 0     # any channel count >= 1
    W = 0x50000000

    def f(**k):
        return lib.eqlinear_backward_bias(k.get("dy", A), k.get("db", C), k.get("ws", W),
                                          k.get("wsb", need), k.get("N", N), k.get("D_T", D_T),
                                          k.get("T", T), k.get("dt", F16), None)
    assert f(dy=None) == NULL
    assert f(db=None) == NULL
    assert f(ws=None) == WS
    assert f(wsb=need - 1) == WS
    assert f(ws=W + 8) == ALIGN
    assert f(db=C + 2) == ALIGN
    assert f(db=A) == ALIAS
    assert f(ws=A + 64) == ALIAS
    assert f(ws=C) == ALIAS
    assert f(N=-1) == SHAPE
    assert f(T=9) == UNSUP
    assert f(dt=5) == UNSUP
    assert f(D_T=65544) == UNSUP


def test_workspace_size_is_a_pure_function(lib):
    a = lib.eqlinear_workspace_size(12608, 192, 768, 4, F16)
    b = lib.eqlinear_workspace_size(12608, 192, 768, 4, F16)
    assert a == b
    assert lib.eqlinear_workspace_size(0, 192, 768, 4, F16) == 0
    assert lib.eqlinear_workspace_size(100, 192, 768, 9, F16) == 0
    assert lib.eqlinear_workspace_size(-1, 192, 768, 4, F16) == 0
    # the partial planes are fp32 and a whole number of [T][D_T][C_T] blocks
    for (N, C_T, D_T, T) in [(12608, 96, 288, 4), (16384, 128, 512, 8), (32768, 1024, 1024, 4),
                            (12608, 128, 384, 3), (5000, 40, 72, 5), (9000, 64, 64, 7),
                            (7000, 5, 13, 4), (9000, 100, 1, 8), (20000, 13, 100, 3)]:
        for dt in (F32, F16):
            s = lib.eqlinear_workspace_size(N, C_T, D_T, T, dt)
            assert s % (4 * T * C_T * D_T) == 0


def test_spectrum_size(lib):
    # blocked layout: [ceil(NC/32)][ceil(K/KC)][P][32][KC] for both orientations,
    # P = T planes, or for fp32 at T = 4, 6, 8 the three-multiplication planes
    # T + (T-1)/2 (12 at T = 8)
    def expect(C_T, D_T, T, dt):
        kc = 16 if dt == F16 else 8
        e = 2 if dt == F16 else 4
        P = {4: 5, 6: 8, 8: 12}.get(T, T) if dt == F32 else T
        part = lambda nc, k: -(-nc // 32) * -(-k // kc) * P * 32 * kc
        return (part(D_T, C_T) + part(C_T, D_T)) * e
    for shape in [(16, 16, 4), (192, 768, 4), (96, 288, 4), (128, 512, 8), (24, 40, 2), (8, 8, 8),
                  (16, 24, 3), (40, 8, 5), (64, 96, 6), (8, 16, 7),
                  (1, 1, 4), (5, 13, 4), (13, 100, 8), (1, 5, 3), (33, 7, 2)]:   # ragged channel counts
        for dt in (F32, F16):
            assert lib.eqlinear_spectrum_size(*shape, dt) == expect(*shape, dt)
    assert lib.eqlinear_spectrum_size(16, 16, 9, F32) == 0
    assert lib.eqlinear_spectrum_size(-8, 16, 4, F32) == 0
    assert lib.eqlinear_spectrum_size(65536, 65536, 4, F16) == 0


def test_spectrum_validation(lib):
    f = lambda **k: lib.eqlinear_weight_spectrum(k.get("w", A), k.get("wh", B), k.get("C_T", 16),
                                                 k.get("D_T", 16), k.get("T", 4), k.get("dt", F32),
                                                 None)
    assert f(w=None) == NULL
    assert f(wh=None) == NULL
    assert f(wh=A) == ALIAS
    assert f(T=1) == UNSUP
    assert f(D_T=-1) == SHAPE
    assert f(wh=B + 4) == ALIGN
    # the spectrum is 2*T*D_T*C_T elements: a buffer ending inside w_tilde aliases it
    assert f(wh=A - 4 * 16 * 16 * 4 - 16) == ALIAS


def test_python_binding_imports():
    from group_wise_dft_amd import eqlinear as E
    assert E.eqlinear_workspace_size(0, 16, 16, 4, 0) == 0
    assert E.eqlinear_status_string(6).startswith("an output")


def test_backward_weight_noalloc_validation(lib):
    """Rejections of the no-allocation weight gradient, all before any HIP call."""
    lib.eqlinear_backward_weight_noalloc.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 3 + \
        [ctypes.c_int32, ctypes.c_int, ctypes.c_void_p]
    f = lambda **k: lib.eqlinear_backward_weight_noalloc(
        k.get("x", A), k.get("dy", B), k.get("dw", C), k.get("N", 64), k.get("C_T", 16), k.get("D_T", 16),
        k.get("T", 4), k.get("dt", F16), None)
    assert f(x=None) == NULL
    assert f(dw=None) == NULL
    assert f(dw=C + 2) == ALIGN
    assert f(dw=A) == ALIAS
    assert f(T=9) == UNSUP
    assert f(N=-1) == SHAPE
    # partials beyond the 64 MiB static scratch
    N, C_T, D_T, T = 65536, 2048, 2048, 8
    assert lib.eqlinear_workspace_size(N, C_T, D_T, T, F32) > (64 << 20)
    assert f(x=0x100000000, dy=0x900000000, dw=0x1100000000, N=N, C_T=C_T, D_T=D_T, T=T, dt=F32) == WS


def test_octic_sizes_and_validation(lib):
    """The octic entry points: sizes (eight stored planes in both dtypes) and
    the same argument checks as the cyclic calls, all before any HIP call."""
    vp, i64, sz, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    lib.eqlinear_octic_spectrum_size.argtypes = [i64, i64, ci]
    lib.eqlinear_octic_spectrum_size.restype = sz
    lib.eqlinear_octic_workspace_size.argtypes = [i64, i64, i64, ci]
    lib.eqlinear_octic_workspace_size.restype = sz
    lib.eqlinear_octic_weight_spectrum.argtypes = [vp, vp, i64, i64, ci, vp]
    lib.eqlinear_octic_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, vp]
    lib.eqlinear_octic_backward_input.argtypes = [vp, vp, vp, i64, i64, i64, ci, vp]
    lib.eqlinear_octic_backward_weight.argtypes = [vp, vp, vp, vp, sz, i64, i64, i64, ci, vp]

    for (C_T, D_T) in [(16, 16), (96, 384), (5, 13), (1, 1), (128, 512)]:
        for dt in (F32, F16):
            kc, e = (16, 2) if dt == F16 else (8, 4)
            part = lambda nc, k: -(-nc // 32) * -(-k // kc) * 8 * 32 * kc
            assert lib.eqlinear_octic_spectrum_size(C_T, D_T, dt) == (part(D_T, C_T) + part(C_T, D_T)) * e
    assert lib.eqlinear_octic_spectrum_size(0, 16, F32) == 0
    assert lib.eqlinear_octic_spectrum_size(16, 16, 3) == 0
    for (N, C_T, D_T) in [(12608, 96, 384), (16384, 128, 512), (5000, 40, 72), (20000, 13, 100)]:
        for dt in (F32, F16):
            s = lib.eqlinear_octic_workspace_size(N, C_T, D_T, dt)
            assert s % (4 * 8 * C_T * D_T) == 0
    assert lib.eqlinear_octic_workspace_size(0, 96, 384, F16) == 0
    assert lib.eqlinear_octic_workspace_size(-1, 96, 384, F16) == 0

    f = lambda **k: lib.eqlinear_octic_forward(k.get("x", A), k.get("w", B), k.get("bias"), k.get("y", C),
                                               k.get("N", 64), k.get("C_T", 16), k.get("D_T", 16),
                                               k.get("dt", F32), None)
    assert f(x=None) == NULL
    assert f(w=None) == NULL
    assert f(y=A) == ALIAS
    assert f(y=C + 4) == ALIGN
    assert f(bias=D + 8) == ALIGN
    assert f(bias=C) == ALIAS
    assert f(N=-1) == SHAPE
    assert f(C_T=0) == UNSUP
    assert f(dt=4) == UNSUP
    assert f(N=0) == OK
    g = lambda **k: lib.eqlinear_octic_backward_input(k.get("dy", A), k.get("w", B), k.get("dx", C),
                                                      k.get("N", 64), 16, 16, F16, None)
    assert g(dy=None) == NULL
    assert g(dx=B) == ALIAS
    assert g(N=0) == OK
    h = lambda **k: lib.eqlinear_octic_weight_spectrum(k.get("w", A), k.get("wh", B), 16, k.get("D_T", 16),
                                                       F32, None)
    assert h(w=None) == NULL
    assert h(wh=A) == ALIAS
    assert h(D_T=-2) == SHAPE
    N, C_T, D_T = 12608, 96, 384
    need = lib.eqlinear_octic_workspace_size(N, C_T, D_T, F16)
    assert need > 0
    W = 0x50000000
    q = lambda **k: lib.eqlinear_octic_backward_weight(k.get("x", A), k.get("dy", B), k.get("dw", C),
                                                       k.get("ws", W), k.get("wsb", need), N, C_T, D_T, F16,
                                                       None)
    assert q(ws=None) == WS
    assert q(wsb=need - 1) == WS
    assert q(ws=W + 8) == ALIGN
    assert q(dw=A) == ALIAS
    assert q(ws=B) == ALIAS
