"""Python binding of libkda_probe (include/kda_probe.h): the plain streaming
and matrix-core kernels whose timed rates are the measured ceilings that
libkda's kernels are compared with.  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(_HERE, "libkda_probe.so")
EXPORTED = ("kda_probe_hbm", "kda_probe_mfma_bf16")
HBM_MODES = {"copy": 0, "rmw": 1, "read": 2, "write": 3}
MFMA_SHAPES = {"32x32x16": 0, "16x16x32": 1}
READ_SPAN = 16384  # bytes of source per partial sum of the "read" stream
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libkda_probe.so (built with libkda by ``kda_gated_delta_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(PROBE_LIB_PATH):
        raise ImportError(f"{PROBE_LIB_PATH} is missing: build it with "
                          "`python -m kda_gated_delta_amd.build`")
    L = ctypes.CDLL(PROBE_LIB_PATH)
    vp = ctypes.c_void_p
    L.kda_probe_hbm.argtypes = [ctypes.c_int, vp, vp, ctypes.c_size_t, vp]
    L.kda_probe_hbm.restype = ctypes.c_int
    L.kda_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int32, ctypes.c_int32, vp, vp]
    L.kda_probe_mfma_bf16.restype = ctypes.c_int
    _lib = L
    return L


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def read_partials(nbytes: int) -> int:
    """fp32 partial sums the "read" stream writes for ``nbytes`` of source."""
    return (int(nbytes) + READ_SPAN - 1) // READ_SPAN


def hbm(mode: str, src, dst, nbytes: int) -> None:
    """One streaming pass over ``nbytes`` bytes (see kda_probe_hbm)."""
    for t in (src, dst):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("probe buffers must be contiguous CUDA tensors")
    need = 4 * read_partials(nbytes) if mode == "read" else int(nbytes)
    if dst is None or dst.numel() * dst.element_size() < need:
        raise ValueError(f"dst must hold at least {need} bytes")
    if src is not None and src.numel() * src.element_size() < int(nbytes):
        raise ValueError(f"src must hold at least {nbytes} bytes")
    st = lib().kda_probe_hbm(HBM_MODES[mode], _ptr(src), _ptr(dst), int(nbytes), _stream())
    if st != 0:
        raise RuntimeError(f"kda_probe_hbm({mode}) failed with status {st}")


def mfma_bf16(shape: str, blocks: int, iters: int, out) -> None:
    """The bf16 matrix-core loop of one MFMA shape (see kda_probe_mfma_bf16);
    ``out`` holds 4 * blocks fp32."""
    if out.dtype != torch.float32 or out.numel() < 4 * blocks or not out.is_cuda:
        raise ValueError("out: float32 CUDA tensor of at least 4 * blocks elements")
    st = lib().kda_probe_mfma_bf16(MFMA_SHAPES[shape], int(blocks), int(iters), _ptr(out),
                                   _stream())
    if st != 0:
        raise RuntimeError(f"kda_probe_mfma_bf16 failed with status {st}")


def mfma_flops(shape: str, blocks: int, iters: int) -> int:
    """Flops of one kda_probe_mfma_bf16 launch: four waves per workgroup,
    eight products per wave and round (32x32x16: 32768 flops each,
    16x16x32: 16384)."""
    per = 32768 if MFMA_SHAPES[shape] == 0 else 16384
    return blocks * 4 * iters * 8 * per
