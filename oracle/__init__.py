"""fp64 CPU oracle for Kronecker-sparse (KS) matrix multiplication.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(``kronecker_sparse_structured_amd``) never imports it, and the two share no
code: this wrapper only marshals NumPy arrays into ``ks_oracle.c``.

The arithmetic lives in ``ks_oracle.c``; see its header for the definition it
follows (KS abstract page, taxoreview.com "dblp:303/4794", first paragraph:
supports are Kronecker products of identity and all-ones blocks).

Every input is widened exactly to fp64 here: fp32 by ``astype``, bf16 from its
16 stored bits (the upper half of an fp32 word).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ks_oracle.c")
_LIB = os.path.join(_HERE, "libks_oracle.so")

_lib = None


def build(force: bool = False, out: str = _LIB, extra_flags: Sequence[str] = (),
          src: str = _SRC) -> str:
    """Compile ks_oracle.c with the host C compiler (no -ffast-math)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", *extra_flags, src, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    lib.ks_oracle_matmul.argtypes = [ctypes.c_int] * 4 + [dp, dp, dp, ctypes.c_longlong]
    lib.ks_oracle_matmul.restype = ctypes.c_int
    lib.ks_oracle_chain.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                    ctypes.POINTER(dp), dp, dp, ctypes.c_longlong]
    lib.ks_oracle_chain.restype = ctypes.c_int
    lib.ks_oracle_chain_err.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                        ctypes.POINTER(dp), dp,
                                        ctypes.POINTER(ctypes.c_float), ctypes.c_longlong,
                                        dp, dp, dp]
    lib.ks_oracle_chain_err.restype = ctypes.c_int
    lib.ks_oracle_matmul_dx.argtypes = [ctypes.c_int] * 4 + [dp, dp, dp, ctypes.c_longlong]
    lib.ks_oracle_matmul_dx.restype = ctypes.c_int
    lib.ks_oracle_matmul_dw.argtypes = [ctypes.c_int] * 4 + [dp, dp, dp, ctypes.c_longlong]
    lib.ks_oracle_matmul_dw.restype = ctypes.c_int
    lib.ks_oracle_num_threads.argtypes = []
    lib.ks_oracle_num_threads.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def widen(arr: np.ndarray, dtype: str = "f32") -> np.ndarray:
    """Exact fp64 copy of stored values. ``dtype`` is "f32", "f64" or "bf16"
    (for bf16, ``arr`` holds the raw uint16 bit patterns)."""
    if dtype == "bf16":
        bits = np.ascontiguousarray(arr, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    return np.ascontiguousarray(arr).astype(np.float64)


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("%s failed with oracle status %d" % (what, rc))


def ks_matmul(pattern: Sequence[int], K: np.ndarray, X: np.ndarray, lib=None) -> np.ndarray:
    """Y = X W^T for one KS factor; K has shape (a, d, b, c); X is batch x a*c*d.
    Inputs must already be fp64 (see ``widen``)."""
    lib = lib or load()
    a, b, c, d = (int(v) for v in pattern)
    K = np.ascontiguousarray(K, dtype=np.float64).reshape(-1)
    X = np.ascontiguousarray(X, dtype=np.float64)
    if K.size != a * b * c * d:
        raise ValueError("K has %d values, pattern needs %d" % (K.size, a * b * c * d))
    batch = X.shape[0]
    if X.size != batch * a * c * d:
        raise ValueError("X width does not match a*c*d")
    Y = np.empty((batch, a * b * d), dtype=np.float64)
    _check(lib.ks_oracle_matmul(a, b, c, d, _dptr(K), _dptr(X), _dptr(Y), batch), "ks_matmul")
    return Y


def ks_matmul_dx(pattern: Sequence[int], K: np.ndarray, dY: np.ndarray, lib=None) -> np.ndarray:
    """dL/dX = dY W for one factor (see ks_oracle.c); dY is batch x a*b*d, fp64."""
    lib = lib or load()
    a, b, c, d = (int(v) for v in pattern)
    K = np.ascontiguousarray(K, dtype=np.float64).reshape(-1)
    dY = np.ascontiguousarray(dY, dtype=np.float64)
    if K.size != a * b * c * d:
        raise ValueError("K has %d values, pattern needs %d" % (K.size, a * b * c * d))
    batch = dY.shape[0]
    if dY.size != batch * a * b * d:
        raise ValueError("dY width does not match a*b*d")
    dX = np.empty((batch, a * c * d), dtype=np.float64)
    _check(lib.ks_oracle_matmul_dx(a, b, c, d, _dptr(K), _dptr(dY), _dptr(dX), batch), "ks_matmul_dx")
    return dX


def ks_matmul_dw(pattern: Sequence[int], dY: np.ndarray, X: np.ndarray, lib=None) -> np.ndarray:
    """dL/dK for one factor, shape (a, d, b, c) (see ks_oracle.c); fp64 inputs."""
    lib = lib or load()
    a, b, c, d = (int(v) for v in pattern)
    dY = np.ascontiguousarray(dY, dtype=np.float64)
    X = np.ascontiguousarray(X, dtype=np.float64)
    batch = dY.shape[0]
    if dY.size != batch * a * b * d or X.size != batch * a * c * d:
        raise ValueError("dY / X widths do not match the pattern")
    dK = np.empty((a, d, b, c), dtype=np.float64)
    _check(lib.ks_oracle_matmul_dw(a, b, c, d, _dptr(dY), _dptr(X), _dptr(dK), batch), "ks_matmul_dw")
    return dK


def _chain_args(patterns, Ks):
    pats = np.ascontiguousarray(np.asarray(patterns, dtype=np.int32).reshape(-1))
    keep = [np.ascontiguousarray(K, dtype=np.float64).reshape(-1) for K in Ks]
    arr = (ctypes.POINTER(ctypes.c_double) * len(keep))(*[_dptr(k) for k in keep])
    return pats, keep, arr


def ks_chain_matmul(patterns: Sequence[Sequence[int]], Ks: Sequence[np.ndarray],
                    X: np.ndarray, lib=None) -> np.ndarray:
    """Apply the factors in the order given (factor 0 first), in fp64."""
    lib = lib or load()
    pats, keep, arr = _chain_args(patterns, Ks)
    X = np.ascontiguousarray(X, dtype=np.float64)
    last = patterns[-1]
    n_out = int(last[0]) * int(last[1]) * int(last[3])
    Y = np.empty((X.shape[0], n_out), dtype=np.float64)
    rc = lib.ks_oracle_chain(len(keep), pats.ctypes.data_as(ctypes.POINTER(ctypes.c_int)),
                             arr, _dptr(X), _dptr(Y), X.shape[0])
    _check(rc, "ks_chain_matmul")
    return Y


def ks_chain_err(patterns, Ks, X: np.ndarray, Ycand: np.ndarray, lib=None):
    """Streaming comparison of a float32 candidate with the fp64 chain result.
    Returns (sum sq err, sum sq ref, max abs err)."""
    lib = lib or load()
    pats, keep, arr = _chain_args(patterns, Ks)
    X = np.ascontiguousarray(X, dtype=np.float64)
    Yc = np.ascontiguousarray(Ycand, dtype=np.float32)
    se, sr, ma = ctypes.c_double(0.0), ctypes.c_double(0.0), ctypes.c_double(0.0)
    rc = lib.ks_oracle_chain_err(len(keep), pats.ctypes.data_as(ctypes.POINTER(ctypes.c_int)),
                                 arr, _dptr(X), Yc.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                 X.shape[0], ctypes.byref(se), ctypes.byref(sr), ctypes.byref(ma))
    _check(rc, "ks_chain_err")
    return se.value, sr.value, ma.value


def num_threads(lib=None) -> int:
    lib = lib or load()
    return int(lib.ks_oracle_num_threads())
