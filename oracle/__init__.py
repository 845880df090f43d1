"""CPU oracle for the KDA recurrence (TEST INFRASTRUCTURE).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this
package. ``kda_oracle`` holds the NumPy fp64 definitions; ``c_recurrence_fwd`` calls the
plain C fp64 twin in libkda_oracle.so (built by oracle/build.py).
"""
import ctypes
import os

import numpy as np

from . import kda_oracle  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "libkda_oracle.so")
        if not os.path.exists(path):
            from .build import build
            build()
        lib = ctypes.CDLL(path)
        f = lib.kda_oracle_recurrence
        P = ctypes.c_void_p
        I = ctypes.c_int64
        D = ctypes.c_double
        f.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, D, D, I, P, P, ctypes.c_int]
        f.restype = ctypes.c_int
        lib.kda_oracle_max_threads.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def max_threads():
    return int(_lib().kda_oracle_max_threads())


def c_recurrence_fwd(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=1.0, g_min=-5.0,
                     col_block=16, n_threads=0):
    """C fp64 per-token recurrence. Inputs are taken as float32 (must be exact copies of the
    device values); returns (o [T, H, d_v], ht [N, H, d_k, d_v]) in float64."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    g = np.ascontiguousarray(g, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    T, H, dk = k.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens).reshape(-1), dtype=np.int64)
    N = cu.shape[0] - 1
    h0a = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float32)
    o = np.zeros((T, H, dv), dtype=np.float64)
    ht = np.zeros((N, H, dk, dv), dtype=np.float64)
    ptr = lambda a: None if a is None else a.ctypes.data
    rc = _lib().kda_oracle_recurrence(ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), ptr(h0a),
                                      ptr(cu), N, T, H, dk, dv, float(scale), float(g_min),
                                      int(col_block), ptr(o), ptr(ht), int(n_threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_recurrence failed with {rc}")
    return o, ht
