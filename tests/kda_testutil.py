"""Helpers shared by the tests: tolerances, gates from the oracle, devices."""
from __future__ import annotations

import numpy as np
import torch

import oracle

# Relative tolerances: fp32 inputs 1e-4, bf16 inputs (fp32 state) 2e-3, each
# applied per block (one (sequence|request, head) slice of an output) as
# ||x - ref||_2 <= tol * ||ref||_2.
TOL = {"f32": 1e-4, "bf16": 2e-3}
TORCH_IO = {"f32": torch.float32, "bf16": torch.bfloat16}


def rel_err_blocks(x, ref, block_ndim: int) -> float:
    """Largest per-block relative L2 error; blocks are the trailing
    ``block_ndim`` axes.  Blocks whose reference is exactly zero must match
    exactly (their error is reported as |x| then)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    bsz = int(np.prod(ref.shape[ref.ndim - block_ndim:])) if block_ndim else 1
    xb = x.reshape(-1, bsz)
    rb = ref.reshape(-1, bsz)
    num = np.linalg.norm(xb - rb, axis=1)
    den = np.linalg.norm(rb, axis=1)
    err = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return float(err.max()) if err.size else 0.0


def round_io(x, io: str) -> np.ndarray:
    """Round fp64 values to the io dtype (RNE) and back to fp64."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    return t.to(TORCH_IO[io]).to(torch.float64).numpy()


def half_ulp(ref, io: str) -> np.ndarray:
    """Half a unit in the last place of the io dtype at |ref| (the largest
    error of rounding ref to that dtype)."""
    _, e = np.frexp(np.asarray(ref, dtype=np.float64))  # ref = m 2^e, 0.5 <= |m| < 1
    mant = 8 if io == "bf16" else 24  # significand bits incl. the implicit one
    return np.where(ref == 0, 0.0, np.ldexp(1.0, e - mant - 1))


def io_output_errors(x, ref, io: str, block_ndim: int):
    """(per-block excess error, whole-tensor relative L2 error).

    An io-dtype output carries its own final rounding (in bf16 alone ~1.7e-3
    relative RMS).  Each element may therefore differ from the exact oracle
    value by half an io ulp plus the computation's own error; the per-block
    figure is the largest excess over that half ulp, relative to the RMS of
    the block's reference.  The whole-tensor figure is the plain relative L2
    error against the exact values."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    excess = np.maximum(np.abs(x - ref) - half_ulp(ref, io), 0.0)
    bsz = int(np.prod(ref.shape[ref.ndim - block_ndim:])) if block_ndim else 1
    eb = excess.reshape(-1, bsz).max(axis=1) if excess.size else np.zeros(0)
    rms = np.sqrt(np.mean(ref.reshape(-1, bsz) ** 2, axis=1)) if ref.size else np.zeros(0)
    per = np.where(rms > 0, eb / np.where(rms > 0, rms, 1.0), eb)
    per_block = float(per.max()) if per.size else 0.0
    den = np.linalg.norm(ref)
    whole = float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))
    return per_block, whole


def assert_io_output(x, ref, io: str, block_ndim: int, tol=None):
    tol = TOL[io] if tol is None else tol
    per_block, whole = io_output_errors(x, ref, io, block_ndim)
    assert per_block <= tol and whole <= tol, (per_block, whole, tol)
    return per_block, whole


def gates_f32(a, b, A_log, dt_bias, lower_bound=0.0):
    """Activated gates from the oracle (fp64), rounded to the fp32 the GPU
    consumes; both sides of a parity test take these same values."""
    lead = a.shape[:-2]
    H, K = a.shape[-2:]
    g, beta = oracle.gate(a.reshape(-1, H, K), b.reshape(-1, H), A_log, dt_bias,
                          lower_bound)
    return (g.astype(np.float32).reshape(lead + (H, K)),
            beta.astype(np.float32).reshape(lead + (H,)))


def dev(x, dtype=torch.float32, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device).to(dtype).contiguous()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()
