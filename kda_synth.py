"""Seeded synthetic inputs for the KDA path (tests, smoke check and bench).

This module holds none of the method's arithmetic: it only draws random
numbers, L2-normalises q and k (the inputs arrive normalised), and rounds
them to the dtype the GPU consumes.  The gate activation, the recurrence and
everything downstream live elsewhere (the HIP library and, separately, the
oracle).

Recipe (all draws fp64 from ``numpy.random.Generator(PCG64(seed))``, in this
order: q, k, v, a, b, A_log, dt_bias, initial state, slot permutation):
  q, k ~ N(0, 1), then L2-normalised per (token, head) in fp64;
  v ~ N(0, 1); a ~ N(0, 1) per key channel; b ~ N(0, 1);
  A_log ~ U(0, ln 16) per head; dt_bias ~ N(0, dt_bias_std) per channel;
  states ~ N(0, state_std);  q, k, v are rounded to the io dtype (RNE),
  a, b, A_log, dt_bias and the states to fp32.
``regime="long"`` replaces A_log by 0 and dt_bias by -8 (slow decay, so the
state carried between chunks and from the initial state stays visible).

Every array is returned as float32 numpy holding exactly representable values
of its dtype (bf16 values are exact in fp32).
"""
from __future__ import annotations

import math

import numpy as np
import torch

IO_DTYPES = ("f32", "bf16")


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _round(x: np.ndarray, io: str) -> np.ndarray:
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if io == "f32":
        return x32
    if io == "bf16":
        return torch.from_numpy(x32).to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(f"unknown io dtype {io!r}")


def _unit(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _gate_params(r: np.random.Generator, H: int, K: int, regime: str,
                 dt_bias_std: float):
    A_log = r.uniform(0.0, math.log(16.0), size=H)
    dt_bias = r.normal(0.0, 1.0, size=(H, K)) * dt_bias_std
    if regime == "long":
        A_log = np.zeros(H)
        dt_bias = np.full((H, K), -8.0)
    elif regime != "config":
        raise ValueError(f"unknown regime {regime!r}")
    return _round(A_log, "f32"), _round(dt_bias, "f32")


def prefill_case(seqlens, H: int, K: int, V: int, io: str, seed: int,
                 regime: str = "config", dt_bias_std: float = 0.5,
                 h0_std: float | None = 0.02) -> dict:
    """Packed varlen batch.  Shapes: q,k,a [T,H,K]; v [T,H,V]; b [T,H];
    A_log [H]; dt_bias [H,K]; h0 [N,H,K,V] or None; cu [N+1] int64."""
    seqlens = [int(s) for s in seqlens]
    T, N = sum(seqlens), len(seqlens)
    r = rng(seed)
    q = _round(_unit(r.standard_normal((T, H, K))), io)
    k = _round(_unit(r.standard_normal((T, H, K))), io)
    v = _round(r.standard_normal((T, H, V)), io)
    a = _round(r.standard_normal((T, H, K)), "f32")
    b = _round(r.standard_normal((T, H)), "f32")
    A_log, dt_bias = _gate_params(r, H, K, regime, dt_bias_std)
    h0 = None
    if h0_std is not None:
        h0 = _round(r.standard_normal((N, H, K, V)) * h0_std, "f32")
    cu = np.zeros(N + 1, dtype=np.int64)
    cu[1:] = np.cumsum(seqlens)
    return dict(q=q, k=k, v=v, a=a, b=b, A_log=A_log, dt_bias=dt_bias, h0=h0,
                cu=cu, io=io, T=T, N=N, H=H, K=K, V=V, seed=seed, regime=regime)


def decode_case(B: int, H: int, K: int, V: int, n_slots: int, io: str,
                seed: int, regime: str = "config", dt_bias_std: float = 0.5,
                state_std: float = 0.02, Tv: int | None = None,
                n_padding: int = 0) -> dict:
    """Single-token decode (Tv None) or multi-token verify (Tv = draft length).

    Shapes: q,k,a [B,(Tv,)H,K]; v [B,(Tv,)H,V]; b [B,(Tv,)H];
    pool [n_slots,H,K,V] fp32; slot_idx [B] int32 (distinct slots; the last
    ``n_padding`` rows get -1, the padding marker).
    """
    r = rng(seed)
    lead = (B,) if Tv is None else (B, Tv)
    q = _round(_unit(r.standard_normal(lead + (H, K))), io)
    k = _round(_unit(r.standard_normal(lead + (H, K))), io)
    v = _round(r.standard_normal(lead + (H, V)), io)
    a = _round(r.standard_normal(lead + (H, K)), "f32")
    b = _round(r.standard_normal(lead + (H,)), "f32")
    A_log, dt_bias = _gate_params(r, H, K, regime, dt_bias_std)
    pool = np.empty((n_slots, H, K, V), dtype=np.float32)
    for s in range(n_slots):  # slot by slot keeps the fp64 temporaries small
        pool[s] = r.standard_normal((H, K, V)) * state_std
    slot_idx = r.permutation(n_slots)[:B].astype(np.int32)
    if n_padding:
        slot_idx[B - n_padding:] = -1
    return dict(q=q, k=k, v=v, a=a, b=b, A_log=A_log, dt_bias=dt_bias,
                pool=pool, slot_idx=slot_idx, io=io, B=B, Tv=Tv, H=H, K=K,
                V=V, n_slots=n_slots, seed=seed, regime=regime)


def orthonormal_keys(n: int, K: int, seed: int) -> np.ndarray:
    """n <= K mutually orthonormal rows of length K (fp64, via QR)."""
    assert n <= K
    qm, _ = np.linalg.qr(rng(seed).standard_normal((K, K)))
    return np.ascontiguousarray(qm[:, :n].T)


# Named workloads (shapes and draw parameters); the seed of workload i is i.
WORKLOADS = {
    # B=1, T=64, H=2, K=V=16, fp32, chunk 16, dt_bias = 0, zero initial state
    "tiny_f32_prefill": dict(kind="prefill", seqlens=[64], H=2, K=16, V=16, io="f32",
                             chunk=16, dt_bias_std=0.0, h0_std=None, seed=0),
    # 4 sequences {512, 1024, 2048, 4096} packed, H=32, K=V=128, bf16, chunk 64
    "varlen_prefill_7680": dict(kind="prefill", seqlens=[512, 1024, 2048, 4096], H=32,
                                K=128, V=128, io="bf16", chunk=64, dt_bias_std=0.5,
                                h0_std=0.02, seed=1),
    # 256 single-token requests on a 512-slot fp32 pool, H=32, K=V=128, bf16
    "decode_256": dict(kind="decode", B=256, H=32, K=128, V=128, n_slots=512,
                       io="bf16", dt_bias_std=0.5, state_std=0.02, seed=2),
    # one 65536-token sequence, H=32, K=V=128, bf16, run as 16 x 4096 carried
    "long_prefill_65536": dict(kind="prefill", seqlens=[65536], H=32, K=128, V=128,
                               io="bf16", chunk=64, dt_bias_std=0.5, h0_std=0.02,
                               seed=3, segments=16),
    # 64 requests x 8 draft tokens on a 128-slot pool, H=32, K=V=128, bf16
    "verify_64x8": dict(kind="verify", B=64, Tv=8, H=32, K=128, V=128, n_slots=128,
                        io="bf16", dt_bias_std=0.5, state_std=0.02, seed=4),
}
