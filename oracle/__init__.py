"""float64 CPU oracle for EQ-Linear (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
this package.  The product library never imports it, and it imports nothing
from the product package.

The arithmetic lives in ``eqlinear_oracle.c`` (plain direct sums of the
definition, see that file's header for the passages it follows).  This module
only marshals numpy float64 arrays into it and builds it with gcc on first
use if ``liboracle.so`` is missing.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "eqlinear_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the C oracle with gcc (OpenMP) into a shared library."""
    if force or not os.path.exists(out) or (os.path.getmtime(out) < os.path.getmtime(src)):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-o", tmp, src, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, out)
    return out


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _sel(idx):
    if idx is None:
        return None, 0, None
    arr = np.ascontiguousarray(np.asarray(idx, dtype=np.int64).reshape(-1))
    return arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), arr.size, arr


class Oracle:
    """numpy front end over one build of eqlinear_oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        lib.oracle_forward.argtypes = [dp, dp, dp, dp, i64, i64, i64, i64, ip, i64]
        lib.oracle_backward_bias.argtypes = [dp, dp, i64, i64, i64]
        lib.oracle_backward_input.argtypes = [dp, dp, dp, i64, i64, i64, i64, ip, i64]
        lib.oracle_backward_weight.argtypes = [dp, dp, dp, i64, i64, i64, i64, ip, i64]
        lib.oracle_spectrum.argtypes = [dp, dp, i64, i64, i64]
        lib.oracle_octic_forward.argtypes = [dp, dp, dp, dp, i64, i64, i64, ip, i64]
        lib.oracle_octic_backward_input.argtypes = [dp, dp, dp, i64, i64, i64, ip, i64]
        lib.oracle_octic_backward_weight.argtypes = [dp, dp, dp, i64, i64, i64, ip, i64]
        lib.oracle_octic_spectrum.argtypes = [dp, dp, i64, i64]
        lib.oracle_num_threads.restype = ctypes.c_int
        for f in (lib.oracle_forward, lib.oracle_backward_input,
                  lib.oracle_backward_weight, lib.oracle_spectrum,
                  lib.oracle_backward_bias, lib.oracle_octic_forward,
                  lib.oracle_octic_backward_input, lib.oracle_octic_backward_weight,
                  lib.oracle_octic_spectrum):
            f.restype = None
        self.lib = lib

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def forward(self, x, w, rows=None, bias=None) -> np.ndarray:
        """Y = EQ-Linear(X; Wt) (+ bias).  x [N,C_T,T], w [D_T,C_T,T], bias [D_T]
        or None; rows selects outputs."""
        x, w = _f64(x), _f64(w)
        N, C_T, T = x.shape
        D_T = w.shape[0]
        assert w.shape == (D_T, C_T, T)
        b = None
        if bias is not None:
            b = _f64(bias)
            assert b.shape == (D_T,)
        p, cnt, keep = _sel(rows)
        if keep is not None:
            assert keep.size == 0 or (keep.min() >= 0 and keep.max() < N)
        y = np.empty((cnt if keep is not None else N, D_T, T), np.float64)
        self.lib.oracle_forward(_ptr(x), _ptr(w), _ptr(b) if b is not None else None, _ptr(y),
                                N, C_T, D_T, T, p, cnt)
        return y

    def backward_bias(self, dy) -> np.ndarray:
        """db [D_T] for upstream gradient dy [N,D_T,T]."""
        dy = _f64(dy)
        N, D_T, T = dy.shape
        db = np.empty((D_T,), np.float64)
        self.lib.oracle_backward_bias(_ptr(dy), _ptr(db), N, D_T, T)
        return db

    def backward_input(self, dy, w, rows=None) -> np.ndarray:
        """dX for upstream gradient dy [N,D_T,T] and weight w [D_T,C_T,T]."""
        dy, w = _f64(dy), _f64(w)
        N, D_T, T = dy.shape
        C_T = w.shape[1]
        assert w.shape == (D_T, C_T, T)
        p, cnt, keep = _sel(rows)
        if keep is not None:
            assert keep.size == 0 or (keep.min() >= 0 and keep.max() < N)
        dx = np.empty((cnt if keep is not None else N, C_T, T), np.float64)
        self.lib.oracle_backward_input(_ptr(dy), _ptr(w), _ptr(dx), N, C_T, D_T, T, p, cnt)
        return dx

    def backward_weight(self, x, dy, dsel=None) -> np.ndarray:
        """dWt for input x [N,C_T,T] and upstream gradient dy [N,D_T,T]."""
        x, dy = _f64(x), _f64(dy)
        N, C_T, T = x.shape
        D_T = dy.shape[1]
        assert dy.shape == (N, D_T, T)
        p, cnt, keep = _sel(dsel)
        if keep is not None:
            assert keep.size == 0 or (keep.min() >= 0 and keep.max() < D_T)
        dw = np.empty((cnt if keep is not None else D_T, C_T, T), np.float64)
        self.lib.oracle_backward_weight(_ptr(x), _ptr(dy), _ptr(dw), N, C_T, D_T, T, p, cnt)
        return dw

    def spectrum(self, w) -> np.ndarray:
        """Weight spectrum as T real planes [T, D_T, C_T] (see eqlinear_oracle.c)."""
        w = _f64(w)
        D_T, C_T, T = w.shape
        out = np.empty((T, D_T, C_T), np.float64)
        self.lib.oracle_spectrum(_ptr(w), _ptr(out), C_T, D_T, T)
        return out


    # ---- the octic group (rotations by 90 degrees and reflections) ----
    def octic_forward(self, x, w, rows=None, bias=None) -> np.ndarray:
        """Y of the octic-group layer: x [N,C_T,8], w [D_T,C_T,8], bias [D_T] or
        None (see eqlinear_oracle.c for the element order and the definition)."""
        x, w = _f64(x), _f64(w)
        N, C_T, T = x.shape
        D_T = w.shape[0]
        assert T == 8 and w.shape == (D_T, C_T, 8)
        b = None
        if bias is not None:
            b = _f64(bias)
            assert b.shape == (D_T,)
        p, cnt, keep = _sel(rows)
        if keep is not None:
            assert keep.size == 0 or (keep.min() >= 0 and keep.max() < N)
        y = np.empty((cnt if keep is not None else N, D_T, 8), np.float64)
        self.lib.oracle_octic_forward(_ptr(x), _ptr(w), _ptr(b) if b is not None else None, _ptr(y),
                                      N, C_T, D_T, p, cnt)
        return y

    def octic_backward_input(self, dy, w, rows=None) -> np.ndarray:
        dy, w = _f64(dy), _f64(w)
        N, D_T, T = dy.shape
        C_T = w.shape[1]
        assert T == 8 and w.shape == (D_T, C_T, 8)
        p, cnt, keep = _sel(rows)
        if keep is not None:
            assert keep.size == 0 or (keep.min() >= 0 and keep.max() < N)
        dx = np.empty((cnt if keep is not None else N, C_T, 8), np.float64)
        self.lib.oracle_octic_backward_input(_ptr(dy), _ptr(w), _ptr(dx), N, C_T, D_T, p, cnt)
        return dx

    def octic_backward_weight(self, x, dy, dsel=None) -> np.ndarray:
        x, dy = _f64(x), _f64(dy)
        N, C_T, T = x.shape
        D_T = dy.shape[1]
        assert T == 8 and dy.shape == (N, D_T, 8)
        p, cnt, keep = _sel(dsel)
        if keep is not None:
            assert keep.size == 0 or (keep.min() >= 0 and keep.max() < D_T)
        dw = np.empty((cnt if keep is not None else D_T, C_T, 8), np.float64)
        self.lib.oracle_octic_backward_weight(_ptr(x), _ptr(dy), _ptr(dw), N, C_T, D_T, p, cnt)
        return dw

    def octic_spectrum(self, w) -> np.ndarray:
        """Group Fourier transform of w [D_T,C_T,8] as 8 planes [8, D_T, C_T]:
        A1, A2, B1, B2, E11, E12, E21, E22."""
        w = _f64(w)
        D_T, C_T, T = w.shape
        assert T == 8
        out = np.empty((8, D_T, C_T), np.float64)
        self.lib.oracle_octic_spectrum(_ptr(w), _ptr(out), C_T, D_T)
        return out


def _default() -> Oracle:
    global _lib
    if _lib is None:
        _lib = Oracle(build())
    return _lib


def num_threads() -> int:
    return _default().num_threads()


def forward(x, w, rows=None, bias=None):
    return _default().forward(x, w, rows, bias)


def backward_bias(dy):
    return _default().backward_bias(dy)


def backward_input(dy, w, rows=None):
    return _default().backward_input(dy, w, rows)


def backward_weight(x, dy, dsel=None):
    return _default().backward_weight(x, dy, dsel)


def spectrum(w):
    return _default().spectrum(w)


def octic_forward(x, w, rows=None, bias=None):
    return _default().octic_forward(x, w, rows, bias)


def octic_backward_input(dy, w, rows=None):
    return _default().octic_backward_input(dy, w, rows)


def octic_backward_weight(x, dy, dsel=None):
    return _default().octic_backward_weight(x, dy, dsel)


def octic_spectrum(w):
    return _default().octic_spectrum(w)
