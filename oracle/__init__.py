"""fp64 CPU oracle of the KDA gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library in
``kda_gated_delta_amd``) never imports it, and this package imports nothing
from there.

The recurrence's arithmetic lives in ``kda_oracle.c`` (plain C, double
precision, token by token); this module marshals numpy arrays into it, and
holds two row-wise helpers of the layer around the recurrence (``l2norm``,
``gated_rmsnorm``) as plain float64 numpy.  Every array handed
in is converted to float64, which is exact for the fp32 and bf16 values the
GPU consumes.  See ``kda_oracle.c`` for the passages each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE double, no fast-math, no FMA)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
            "-ffp-contract=off", "-Wall", "-Wextra", "-Wno-unused-parameter",
            _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.kda_ref_gate.argtypes = [_D, _D, _D, _D, ctypes.c_int64, ctypes.c_int32,
                                 ctypes.c_int32, ctypes.c_double, _D, _D]
    lib.kda_ref_gate.restype = None
    lib.kda_ref_step.argtypes = [_D, _D, _D, _D, _D, ctypes.c_double,
                                 ctypes.c_double, ctypes.c_int32, ctypes.c_int32, _D]
    lib.kda_ref_step.restype = None
    lib.kda_ref_prefill.argtypes = [_I64, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, _D, _D, _D,
                                    _D, _D, ctypes.c_double, _D, _D, _D, ctypes.c_int]
    lib.kda_ref_prefill.restype = ctypes.c_int
    lib.kda_ref_decode.argtypes = [_D, _D, _D, _D, _D, ctypes.c_double, _D,
                                   ctypes.c_int64, _I64, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   _D, ctypes.c_int]
    lib.kda_ref_decode.restype = ctypes.c_int
    lib.kda_ref_verify.argtypes = [_D, _D, _D, _D, _D, ctypes.c_double, _D,
                                   ctypes.c_int64, _I64, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, _D, _D, ctypes.c_int]
    lib.kda_ref_verify.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(x: np.ndarray | None):
    if x is None:
        return None
    return x.ctypes.data_as(_D)


def _threads(nthreads: int | None) -> int:
    return int(nthreads) if nthreads else (os.cpu_count() or 1)


def gate(a, b, A_log, dt_bias=None, lower_bound: float = 0.0):
    """g [T,H,K] and beta [T,H] in float64 from raw a [T,H,K], b [T,H]."""
    a = _f64(a)
    b = _f64(b)
    A_log = _f64(A_log)
    T, H, K = a.shape
    assert b.shape == (T, H) and A_log.shape == (H,)
    dtb = None if dt_bias is None else _f64(dt_bias).reshape(H, K)
    g = np.empty_like(a)
    beta = np.empty_like(b)
    _load().kda_ref_gate(_p(a), _p(b), _p(A_log), _p(dtb), T, H, K,
                         float(lower_bound), _p(g), _p(beta))
    return g, beta


def step(S, q, k, v, g, beta: float, scale: float = 1.0):
    """One token on a single head.  Returns (S_new [K,V], o [V])."""
    S = _f64(S).copy()
    K, V = S.shape
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    assert q.shape == (K,) and k.shape == (K,) and v.shape == (V,) and g.shape == (K,)
    o = np.empty(V, dtype=np.float64)
    _load().kda_ref_step(_p(S), _p(q), _p(k), _p(v), _p(g), float(beta),
                         float(scale), K, V, _p(o))
    return S, o


def prefill(q, k, v, g, beta, cu_seqlens, scale: float, h0=None,
            nthreads: int | None = None):
    """Varlen prefill.  q,k,g [T,H,K]; v [T,H,V]; beta [T,H]; h0 [N,H,K,V].

    Returns (o [T,H,V], ht [N,H,K,V]) in float64.
    """
    q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    T, H, K = q.shape
    V = v.shape[2]
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    N = cu.shape[0] - 1
    assert cu[-1] == T
    h0a = None if h0 is None else _f64(h0).reshape(N, H, K, V)
    o = np.zeros((T, H, V), dtype=np.float64)
    ht = np.zeros((N, H, K, V), dtype=np.float64)
    rc = _load().kda_ref_prefill(cu.ctypes.data_as(_I64), N, H, K, V, _p(q),
                                 _p(k), _p(v), _p(g), _p(beta), float(scale),
                                 _p(h0a), _p(ht), _p(o), _threads(nthreads))
    if rc != 0:
        raise ValueError("cu_seqlens must start at 0 and be non-decreasing")
    return o, ht


def decode(q, k, v, g, beta, scale: float, pool, slot_idx,
           nthreads: int | None = None):
    """Single-token decode.  Returns (o [B,H,V], new_pool) without touching
    the caller's pool array."""
    q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    B, H, K = q.shape
    V = v.shape[2]
    pool = _f64(pool).copy()
    n_slots = pool.shape[0]
    idx = np.ascontiguousarray(np.asarray(slot_idx, dtype=np.int64))
    o = np.empty((B, H, V), dtype=np.float64)
    rc = _load().kda_ref_decode(_p(q), _p(k), _p(v), _p(g), _p(beta),
                                float(scale), _p(pool), n_slots,
                                idx.ctypes.data_as(_I64), B, H, K, V, _p(o),
                                _threads(nthreads))
    if rc != 0:
        raise ValueError("slot index out of range")
    return o, pool


def verify(q, k, v, g, beta, scale: float, pool, slot_idx,
           nthreads: int | None = None, inter_fill: float = 0.0):
    """Multi-token verify.  q,k,g [B,Tv,H,K]; v [B,Tv,H,V]; beta [B,Tv,H].

    Returns (o [B,Tv,H,V], inter [B,Tv,H,K,V]); the pool is only read.
    Rows of padding requests in inter keep ``inter_fill``.
    """
    q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    B, Tv, H, K = q.shape
    V = v.shape[3]
    pool = _f64(pool)
    n_slots = pool.shape[0]
    idx = np.ascontiguousarray(np.asarray(slot_idx, dtype=np.int64))
    o = np.empty((B, Tv, H, V), dtype=np.float64)
    inter = np.full((B, Tv, H, K, V), inter_fill, dtype=np.float64)
    rc = _load().kda_ref_verify(_p(q), _p(k), _p(v), _p(g), _p(beta),
                                float(scale), _p(pool), n_slots,
                                idx.ctypes.data_as(_I64), B, Tv, H, K, V,
                                _p(inter), _p(o), _threads(nthreads))
    if rc != 0:
        raise ValueError("slot index out of range")
    return o, inter


def l2norm(x, eps: float = 1e-6):
    """x / sqrt(sum x^2 + eps) over the last axis, float64: the in-kernel
    q/k normalisation (ReplaySSM analysis, section 3.10, eps 1e-6)."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def gated_rmsnorm(o, z, w, eps: float, act: str = "sigmoid"):
    """The layer's gated output norm ("Linear attention" tutorial, section
    "一层 GDN / KDA 的完整数据流"; the KDA form takes a sigmoid of the gate):
    o over the RMS of its last axis (plus eps), times the weight w and
    act(z), act = sigmoid or silu (z sigmoid(z)).  float64."""
    o, z, w = _f64(o), _f64(z), _f64(w)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    sg = 1.0 / (1.0 + np.exp(-z))
    return o / rms * w * (sg if act == "sigmoid" else z * sg)
