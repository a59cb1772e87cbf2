"""CPU oracle for OAL causal attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package. The GPU library never calls it and shares no code with it.

Wraps ``oal_oracle.c`` (fp64 loops, OpenMP over output rows) through ctypes:

* ``dense``       -- the definition: kappa-weighted causal average, O(T^2) (reproduction notes
                     of arXiv 2610.13674, section "核心公式", kernel and readout displays);
* ``dense_rows``  -- the same definition for selected rows (b, h, i);
* ``kappa``/``kappa_matrix`` -- kappa = eps + ||L^T s-bar||^2 for pairs;
* ``recurrence``  -- the H0/H1/H2 recurrence of the same section with full d x d H2;
* ``state``       -- the prefix states with H2 as an upper triangle (the library's layout);
* ``contribution`` -- the causal contribution score chi of every q/k dim per prompt and its
                     mean over prompts (same section, first display), O(T^2) over pairs;
* ``backward``    -- gradients of the dense definition (dq, dk, dv, dL, deps) for an upstream
                     gradient dy, by the chain rule through every causal pair.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oal_oracle.c")
_LIB = os.path.join(_HERE, "liboal_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, strict IEEE: no -ffast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oal_oracle_dense.argtypes = [I, I, I, I, I, I, P, P, P, P, P, I, P, P, P, P]
        lib.oal_oracle_dense_rows.argtypes = [I, I, I, I, I, I, P, P, P, P, P, I, P, P, I, P, P, P]
        lib.oal_oracle_recurrence.argtypes = [I, I, I, I, I, I, P, P, P, P, P, I, P, P, P, P]
        lib.oal_oracle_state.argtypes = [I, I, I, I, I, P, P, P]
        lib.oal_oracle_kappa.argtypes = [I, I, I, P, P, ctypes.c_double, P, P]
        lib.oal_oracle_kappa.restype = ctypes.c_double
        lib.oal_oracle_kappa_matrix.argtypes = [I, I, I, I, I, P, P, P, P, I, P, P, I, I, P]
        lib.oal_oracle_contribution.argtypes = [I, I, I, I, I, P, P, P, P]
        lib.oal_oracle_backward.argtypes = [I, I, I, I, I, I, P, P, P, P, P, I, P, P, P, P, P, P, P, P]
        lib.oal_oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _params(params):
    ng = np.ascontiguousarray(params.n_groups, dtype=np.int32)
    gam = np.ascontiguousarray(params.group_of_dim, dtype=np.uint8)
    L = _f64(params.L)
    eps = _f64(params.eps)
    return ng, gam, int(L.shape[1]) - 1, L, eps


def num_threads() -> int:
    return int(_load().oal_oracle_num_threads())


def dense(q, k, v, params, return_den: bool = False):
    """y [B,Hq,T,dv] (fp64) of the dense definition; optionally the denominators [B,Hq,T]."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, T, d = q.shape
    Hkv, dv = k.shape[1], v.shape[-1]
    ng, gam, gmax, L, eps = _params(params)
    y = np.empty((B, Hq, T, dv))
    den = np.empty((B, Hq, T))
    rc = lib.oal_oracle_dense(B, Hq, Hkv, T, d, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(ng),
                              _ptr(gam), gmax, _ptr(L), _ptr(eps), _ptr(y), _ptr(den))
    if rc:
        raise ValueError(f"oal_oracle_dense: bad arguments (code {rc})")
    return (y, den) if return_den else y


def dense_rows(q, k, v, params, rows, return_den: bool = False):
    """Dense definition for rows = [(b, h, i), ...]; returns y [n, dv] (and den [n])."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, T, d = q.shape
    Hkv, dv = k.shape[1], v.shape[-1]
    ng, gam, gmax, L, eps = _params(params)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    n = rows.shape[0]
    y = np.empty((n, dv))
    den = np.empty(n)
    rc = lib.oal_oracle_dense_rows(B, Hq, Hkv, T, d, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(ng),
                                   _ptr(gam), gmax, _ptr(L), _ptr(eps), n, _ptr(rows), _ptr(y),
                                   _ptr(den))
    if rc:
        raise ValueError(f"oal_oracle_dense_rows: bad arguments (code {rc})")
    return (y, den) if return_den else y


def recurrence(q, k, v, params, return_state: bool = False):
    """Naive H0/H1/H2 recurrence; y [B,Hq,T,dv] and optionally H [B,Hkv,1+d+d*d,dv+1]."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, T, d = q.shape
    Hkv, dv = k.shape[1], v.shape[-1]
    ng, gam, gmax, L, eps = _params(params)
    y = np.empty((B, Hq, T, dv))
    H = np.empty((B, Hkv, 1 + d + d * d, dv + 1)) if return_state else None
    rc = lib.oal_oracle_recurrence(B, Hq, Hkv, T, d, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(ng),
                                   _ptr(gam), gmax, _ptr(L), _ptr(eps), _ptr(y), _ptr(H))
    if rc:
        raise ValueError(f"oal_oracle_recurrence: bad arguments (code {rc})")
    return (y, H) if return_state else y


def state(k, v):
    """Prefix states after all tokens, H2 as upper triangle: [B,Hkv,1+d+d(d+1)/2,dv+1]."""
    lib = _load()
    k, v = _f64(k), _f64(v)
    B, Hkv, T, d = k.shape
    dv = v.shape[-1]
    H = np.empty((B, Hkv, 1 + d + d * (d + 1) // 2, dv + 1))
    rc = lib.oal_oracle_state(B, Hkv, T, d, dv, _ptr(k), _ptr(v), _ptr(H))
    if rc:
        raise ValueError(f"oal_oracle_state: bad arguments (code {rc})")
    return H


def kappa(q_vec, k_vec, params, h: int) -> float:
    """kappa for one pair under head h's parameters."""
    lib = _load()
    ng, gam, gmax, L, eps = _params(params)
    qv, kv = _f64(q_vec), _f64(k_vec)
    d = qv.shape[0]
    return float(lib.oal_oracle_kappa(d, int(ng[h]), gmax, _ptr(np.ascontiguousarray(gam[h])),
                                      _ptr(np.ascontiguousarray(L[h])), float(eps[h]),
                                      _ptr(qv), _ptr(kv)))


def kappa_matrix(q, k, params, b: int, h: int):
    """Causal kappa matrix [T, T] (zero above the diagonal) of row block (b, h)."""
    lib = _load()
    q, k = _f64(q), _f64(k)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    ng, gam, gmax, L, eps = _params(params)
    kap = np.empty((T, T))
    rc = lib.oal_oracle_kappa_matrix(B, Hq, Hkv, T, d, _ptr(q), _ptr(k), _ptr(ng), _ptr(gam),
                                     gmax, _ptr(L), _ptr(eps), b, h, _ptr(kap))
    if rc:
        raise ValueError(f"oal_oracle_kappa_matrix: bad arguments (code {rc})")
    return kap


def contribution(q, k):
    """chi [B,Hq,d] and chi_mean [Hq,d] (fp64): mean over the T(T+1)/2 causal pairs of
    |q_ir k_jr| / sqrt(d) per prompt, query head and dim; chi_mean averages over prompts."""
    lib = _load()
    q, k = _f64(q), _f64(k)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, T, d):
        raise ValueError("contribution: k must be [B, Hkv, T, d] with q's B, T, d")
    chi = np.empty((B, Hq, d))
    chi_mean = np.empty((Hq, d))
    rc = lib.oal_oracle_contribution(B, Hq, Hkv, T, d, _ptr(q), _ptr(k), _ptr(chi),
                                     _ptr(chi_mean))
    if rc:
        raise ValueError(f"oal_oracle_contribution: bad arguments (code {rc})")
    return chi, chi_mean


def backward(q, k, v, params, dy):
    """Gradients (dq, dk, dv, dL, deps) of sum(dy * y) for y = dense(q, k, v, params), fp64.
    dL has the shape of params.L (lower triangle of rows/cols 0..G_h, the rest zero)."""
    lib = _load()
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    B, Hq, T, d = q.shape
    Hkv, dv = k.shape[1], v.shape[-1]
    ng, gam, gmax, L, eps = _params(params)
    dq, dk, dvo = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    dL = np.empty_like(L)
    deps = np.empty(Hq)
    rc = lib.oal_oracle_backward(B, Hq, Hkv, T, d, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(ng),
                                 _ptr(gam), gmax, _ptr(L), _ptr(eps), _ptr(dy), _ptr(dq),
                                 _ptr(dk), _ptr(dvo), _ptr(dL), _ptr(deps))
    if rc:
        raise ValueError(f"oal_oracle_backward: bad arguments (code {rc})")
    return dq, dk, dvo, dL, deps


def row_error(y, y_ref):
    """max over rows of ||y_i - y*_i||_inf / ||y*_i||_inf (row-normwise relative error)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    num = np.abs(y - y_ref).max(axis=-1)
    den = np.abs(y_ref).max(axis=-1)
    return float((num / np.maximum(den, 1e-300)).max()) if num.size else 0.0
