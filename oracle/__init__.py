"""LAPLEX CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The GPU library never calls it and shares no
code with it.

Two parts, both float64:

* ``dense_*``: the plain definition of the operator of "LAPLEX: The FFT of
  Learnable Laplace Kernels" (technical summary, section 2.1 "The Operator"),
  ``y_i = sum_j exp(-|a_i - b_j|) [cos(phi_i - psi_j)] x_j``, written out with
  NumPy in row chunks and no sort.  O(n k m); for small sizes and spot rows.
* ``gram_dense`` / ``gram_block``: the weighted Gram matrix M = A diag(D) A^T
  of section 2.2 ("Gram operators") by its plain definition, whole or a block
  of entries.
* ``sym_apply`` / ``general_apply`` / ``phased_apply`` / ``stable_argsort``:
  the sequential scan algebra of section 2.2 ("Exact Scan Algebra") in plain C
  (``laplex_oracle.c``), O(n log n).
* ``sym_apply_par`` / ``stable_argsort_par``: the same symmetric operator on
  all host cores (``laplex_oracle_par.c``, OpenMP: a merge sort split among
  the threads and a chunked two-pass scan), the CPU baseline of the
  benchmark; checked against the one-core functions.

Pins (the test-suite checks these against facts other than the oracle
itself): the closed-form Kac-Murdock-Szego inverse for equispaced anchors, the
tridiagonal inverse of the exponential (Markov) covariance for arbitrary
distinct anchors, the Toeplitz/FFT reduction on a uniform grid, geometric-series
row sums, symmetry and adjointness, K e_j = column j, the zero-temperature
permutation limit, and brute force on tiny inputs.  No function here is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "laplex_oracle.c")
_SO = os.path.join(_HERE, "liblaplex_oracle.so")
_lock = threading.Lock()
_lib_handle = None


def build(force: bool = False, out: Optional[str] = None, src: Optional[str] = None) -> str:
    """Compile the C oracle with gcc (plain -O2, IEEE arithmetic)."""
    out = out or _SO
    src = src or _SRC
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-o", tmp, src, "-lm"], check=True)
        os.replace(tmp, out)
    return out


_SRC_PAR = os.path.join(_HERE, "laplex_oracle_par.c")
_SO_PAR = os.path.join(_HERE, "liblaplex_oracle_par.so")
_par_handle = None


def build_par(force: bool = False) -> str:
    """Compile the all-cores oracle with gcc -fopenmp."""
    if force or not os.path.exists(_SO_PAR) or os.path.getmtime(_SO_PAR) < os.path.getmtime(_SRC_PAR):
        tmp = _SO_PAR + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=gnu11", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC_PAR, "-lm"], check=True)
        os.replace(tmp, _SO_PAR)
    return _SO_PAR


def load_par():
    """Load (building if needed) the all-cores oracle."""
    global _par_handle
    with _lock:
        if _par_handle is None:
            lib = ctypes.CDLL(build_par())
            i64 = ctypes.c_int64
            lib.lop_stable_argsort.argtypes = [ctypes.POINTER(ctypes.c_float), i64, ctypes.POINTER(ctypes.c_uint32)]
            lib.lop_sym_apply.argtypes = [ctypes.POINTER(ctypes.c_float), i64, i64, ctypes.POINTER(ctypes.c_float),
                                          ctypes.POINTER(ctypes.c_double)]
            for fn in (lib.lop_stable_argsort, lib.lop_sym_apply, lib.lop_threads):
                fn.restype = ctypes.c_int
            _par_handle = lib
        return _par_handle


def par_threads() -> int:
    """OpenMP threads the all-cores oracle runs on (OMP_NUM_THREADS or the host's cores)."""
    return int(load_par().lop_threads())


def stable_argsort_par(a) -> np.ndarray:
    """stable_argsort on all host cores."""
    a = _f32(a).ravel()
    perm = np.empty(a.size, np.uint32)
    _check(load_par().lop_stable_argsort(_ptr(a, ctypes.c_float), a.size, _ptr(perm, ctypes.c_uint32)))
    return perm


def sym_apply_par(a, x) -> np.ndarray:
    """sym_apply on all host cores (float64, n x m)."""
    a = _f32(a).ravel()
    x2 = _as2d(x, a.size)
    y = np.empty(x2.shape, np.float64)
    _check(load_par().lop_sym_apply(_ptr(a, ctypes.c_float), a.size, x2.shape[1], _ptr(x2, ctypes.c_float),
                                    _ptr(y, ctypes.c_double)))
    return y


def load(path: Optional[str] = None):
    """Load (building if needed) the C oracle library and declare its signatures."""
    global _lib_handle
    with _lock:
        if path is None and _lib_handle is not None:
            return _lib_handle
        lib = ctypes.CDLL(path or build())
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        i64 = ctypes.c_int64
        lib.lo_stable_argsort.argtypes = [f32p, i64, u32p]
        lib.lo_sym_apply.argtypes = [f32p, i64, i64, f32p, f64p]
        lib.lo_general_apply.argtypes = [f32p, i64, f32p, i64, i64, f32p, f64p]
        lib.lo_phased_apply.argtypes = [f32p, f32p, i64, f32p, f32p, i64, i64, f32p, f64p]
        lib.lo_dense_rows.argtypes = [f32p, f32p, ctypes.POINTER(ctypes.c_int64), i64, f32p, f32p, i64, i64, f32p, f64p,
                                      f64p]
        lib.lo_sym_backward.argtypes = [f32p, i64, i64, f32p, f32p, f64p, f64p]
        lib.lo_general_backward.argtypes = [f32p, i64, f32p, i64, i64, f32p, f32p, f64p, f64p, f64p]
        lib.lo_backward_rows.argtypes = [f32p, i64, i64, f32p, f32p, ctypes.POINTER(ctypes.c_int64), i64, f64p, f64p]
        for fn in (lib.lo_stable_argsort, lib.lo_sym_apply, lib.lo_general_apply, lib.lo_phased_apply, lib.lo_dense_rows,
                   lib.lo_sym_backward, lib.lo_general_backward, lib.lo_backward_rows):
            fn.restype = ctypes.c_int
        if path is None:
            _lib_handle = lib
        return lib


def _f32(v):
    return np.ascontiguousarray(v, dtype=np.float32)


def _ptr(arr, ct):
    return arr.ctypes.data_as(ctypes.POINTER(ct))


def _check(rc):
    if rc == -1:
        raise ValueError("non-finite anchor")
    if rc != 0:
        raise MemoryError("oracle allocation failed (rc=%d)" % rc)


def _as2d(x, rows):
    x = _f32(x)
    if x.ndim == 1:
        x = x.reshape(rows, 1)
    return x


def stable_argsort(a, lib=None) -> np.ndarray:
    """Ascending stable argsort (ties by input index, -0.0 == +0.0), uint32."""
    lib = lib or load()
    a = _f32(a).ravel()
    perm = np.empty(a.size, np.uint32)
    _check(lib.lo_stable_argsort(_ptr(a, ctypes.c_float), a.size, _ptr(perm, ctypes.c_uint32)))
    return perm


def sym_apply(a, x, lib=None) -> np.ndarray:
    """K(a, a) x by the sorted prefix/suffix recurrences (float64, n x m)."""
    lib = lib or load()
    a = _f32(a).ravel()
    x2 = _as2d(x, a.size)
    y = np.empty(x2.shape, np.float64)
    _check(lib.lo_sym_apply(_ptr(a, ctypes.c_float), a.size, x2.shape[1], _ptr(x2, ctypes.c_float), _ptr(y, ctypes.c_double)))
    return y


def sym_backward(a, x, g, lib=None):
    """Backward of y = K(a, a) x for an upstream gradient g = dL/dy (float64):
    returns (dx = K g, n x m; da, n) with sign(0) = 0 at tied anchors."""
    lib = lib or load()
    a = _f32(a).ravel()
    x2, g2 = _as2d(x, a.size), _as2d(g, a.size)
    dx = np.empty(g2.shape, np.float64)
    da = np.empty(a.size, np.float64)
    _check(lib.lo_sym_backward(_ptr(a, ctypes.c_float), a.size, x2.shape[1], _ptr(x2, ctypes.c_float),
                               _ptr(g2, ctypes.c_float), _ptr(dx, ctypes.c_double), _ptr(da, ctypes.c_double)))
    return dx, da


def backward_rows(rows, a, x, g, lib=None):
    """Symmetric anchor gradient da and its envelope at selected rows, by the
    plain definition (O(n) per row)."""
    lib = lib or load()
    a = _f32(a).ravel()
    x2, g2 = _as2d(x, a.size), _as2d(g, a.size)
    rows = np.ascontiguousarray(rows, np.int64)
    da = np.empty(rows.size, np.float64)
    env = np.empty(rows.size, np.float64)
    rc = lib.lo_backward_rows(_ptr(a, ctypes.c_float), a.size, x2.shape[1], _ptr(x2, ctypes.c_float), _ptr(g2, ctypes.c_float),
                              rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), rows.size, _ptr(da, ctypes.c_double),
                              _ptr(env, ctypes.c_double))
    if rc == -3:
        raise IndexError("row out of range")
    _check(rc)
    return da, env


def general_backward(a, b, x, g, lib=None):
    """Backward of y = K(a, b) x (n x k operator) for g = dL/dy (float64):
    returns (dx = K^T g, k x m; da, n; db, k)."""
    lib = lib or load()
    a, b = _f32(a).ravel(), _f32(b).ravel()
    x2, g2 = _as2d(x, b.size), _as2d(g, a.size)
    m = x2.shape[1]
    dx = np.zeros((b.size, m), np.float64)
    da = np.empty(a.size, np.float64)
    db = np.empty(b.size, np.float64)
    _check(lib.lo_general_backward(_ptr(a, ctypes.c_float), a.size, _ptr(b, ctypes.c_float), b.size, m,
                                   _ptr(x2, ctypes.c_float), _ptr(g2, ctypes.c_float), _ptr(dx, ctypes.c_double),
                                   _ptr(da, ctypes.c_double), _ptr(db, ctypes.c_double)))
    return dx, da, db


def general_apply(a, b, x, lib=None) -> np.ndarray:
    """K(a, b) x by interval aggregation into u, v and two scans (float64, n x m)."""
    lib = lib or load()
    a = _f32(a).ravel()
    b = _f32(b).ravel()
    x2 = _as2d(x, b.size)
    y = np.empty((a.size, x2.shape[1]), np.float64)
    _check(lib.lo_general_apply(_ptr(a, ctypes.c_float), a.size, _ptr(b, ctypes.c_float), b.size, x2.shape[1],
                                _ptr(x2, ctypes.c_float), _ptr(y, ctypes.c_double)))
    return y


def phased_apply(a, phi, x, b=None, psi=None, lib=None) -> np.ndarray:
    """Phased operator by complex scans.  ``b is None`` selects b = a, psi = phi."""
    lib = lib or load()
    a = _f32(a).ravel()
    phi = _f32(phi).ravel()
    if b is None:
        x2 = _as2d(x, a.size)
        y = np.empty(x2.shape, np.float64)
        _check(lib.lo_phased_apply(_ptr(a, ctypes.c_float), _ptr(phi, ctypes.c_float), a.size, None, None, 0,
                                   x2.shape[1], _ptr(x2, ctypes.c_float), _ptr(y, ctypes.c_double)))
        return y
    b = _f32(b).ravel()
    psi = _f32(psi).ravel()
    x2 = _as2d(x, b.size)
    y = np.empty((a.size, x2.shape[1]), np.float64)
    _check(lib.lo_phased_apply(_ptr(a, ctypes.c_float), _ptr(phi, ctypes.c_float), a.size, _ptr(b, ctypes.c_float),
                               _ptr(psi, ctypes.c_float), b.size, x2.shape[1], _ptr(x2, ctypes.c_float),
                               _ptr(y, ctypes.c_double)))
    return y


def dense_rows_c(rows, a, x, b=None, phi=None, psi=None, lib=None):
    """Rows ``rows`` of y and of K0|x| by the plain definition, in C (one pass
    over the input anchors; for spot checks at sizes too large for NumPy
    temporaries).  Returns (y_rows, env_rows), float64, len(rows) x m."""
    lib = lib or load()
    a = _f32(a).ravel()
    bb = a if b is None else _f32(b).ravel()
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    x2 = _as2d(x, bb.size)
    m = x2.shape[1]
    y = np.empty((rows.size, m), np.float64)
    env = np.empty((rows.size, m), np.float64)
    ph = None if phi is None else _f32(phi).ravel()
    ps = None if phi is None else (ph if psi is None else _f32(psi).ravel())
    _check(lib.lo_dense_rows(_ptr(a, ctypes.c_float), None if ph is None else _ptr(ph, ctypes.c_float),
                             rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), rows.size, _ptr(bb, ctypes.c_float),
                             None if ps is None else _ptr(ps, ctypes.c_float), bb.size, m, _ptr(x2, ctypes.c_float),
                             _ptr(y, ctypes.c_double), _ptr(env, ctypes.c_double)))
    return y, env


from .dense import (dense_apply, dense_backward, dense_envelope, dense_phased_backward, gram_block,  # noqa: E402,F401
                    gram_dense, normwise_error, phased_backward_rows)
