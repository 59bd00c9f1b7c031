"""Loader for the oracle's plain-C fp64 SpMM (test infrastructure only).

``build()`` compiles ``spmm_f64.c`` with gcc into ``_spmm_f64.so`` next to
it; the library is loaded on first use and compiled then if missing.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spmm_f64.c")
_LIB = os.path.join(_HERE, "_spmm_f64.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle's C code (gcc, OpenMP, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        L.orc_spmm_f64.argtypes = [i64, vp, vp, vp, vp, i64, i64, vp, i64, ctypes.c_int]
        L.orc_spmm_f64.restype = None
        L.orc_spmm_rows_f64.argtypes = [i64, vp, vp, vp, vp, vp, i64, i64, vp, i64, ctypes.c_int]
        L.orc_spmm_rows_f64.restype = None
        L.orc_spmm_f32.argtypes = [i64, vp, vp, vp, vp, i64, i64, vp, i64, ctypes.c_int]
        L.orc_spmm_f32.restype = None
        L.orc_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def spmm(indptr, indices, values, X, abs_mode=False, rows=None):
    """fp64 CSR x dense: Y = A X (or only rows ``rows`` of it).

    indptr int64[n+1], indices int32[nnz], values float32[nnz] or None (all
    ones), X float64 [n_cols, d].  Returns float64 [n or len(rows), d].
    A float32 X runs the same loops in fp32 (the timing instantiation; all
    rows only) and returns float32."""
    indptr = np.ascontiguousarray(indptr, np.int64)
    indices = np.ascontiguousarray(indices, np.int32)
    values = None if values is None else np.ascontiguousarray(values, np.float32)
    if np.asarray(X).dtype == np.float32 and rows is None:
        X = np.ascontiguousarray(X, np.float32)
        n, d = indptr.size - 1, X.shape[1]
        Y = np.empty((n, d), np.float32)
        lib().orc_spmm_f32(n, _p(indptr), _p(indices), _p(values), _p(X), d, d, _p(Y), d,
                           int(bool(abs_mode)))
        return Y
    X = np.ascontiguousarray(X, np.float64)
    n = indptr.size - 1
    d = X.shape[1]
    if indices.size and (indices.min() < 0 or indices.max() >= X.shape[0]):
        raise ValueError("column index out of range of X")
    if rows is None:
        Y = np.empty((n, d), np.float64)
        lib().orc_spmm_f64(n, _p(indptr), _p(indices), _p(values), _p(X), d, d,
                           _p(Y), d, int(bool(abs_mode)))
    else:
        rows = np.ascontiguousarray(rows, np.int64)
        Y = np.empty((rows.size, d), np.float64)
        lib().orc_spmm_rows_f64(rows.size, _p(rows), _p(indptr), _p(indices), _p(values),
                                _p(X), d, d, _p(Y), d, int(bool(abs_mode)))
    return Y


def num_threads() -> int:
    return int(lib().orc_num_threads())
