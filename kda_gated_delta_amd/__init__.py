"""Python binding of libkda (KDA gated delta rule, HIP kernels for gfx950).

Argument marshalling only: each function checks dtypes, shapes, devices and
contiguity of torch tensors, passes raw device pointers and the current HIP
stream to the C entry point of the same name (declared in include/kda.h), and
raises ``KdaError`` on a non-OK status.  Every step of the computation runs
in the library's kernels; there is no fallback of any kind.  PyTorch provides
device memory and streams.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_F32 = 0
KDA_BF16 = 1
_IO = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}

_lib = None


class PrefillSchedule(ctypes.Structure):
    """kda_prefill_schedule of include/kda_profile.h."""
    _fields_ = [(n, ctypes.c_int32) for n in ("n_waves", "segment_chunks", "uses_maps",
                                               "intra_launches", "state_launches",
                                               "other_launches")]


class PrefillOpts(ctypes.Structure):
    """kda_prefill_opts of include/kda.h (model-layer options of prefill)."""
    _fields_ = [("gate_mode", ctypes.c_int32), ("A_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p), ("lower_bound", ctypes.c_float),
                ("per_head_gate", ctypes.c_int32), ("qk_heads", ctypes.c_int32),
                ("snapshots", ctypes.c_void_p), ("snapshot_rows", ctypes.c_int64),
                ("snapshot_interval", ctypes.c_int32), ("qk_l2norm", ctypes.c_int32)]


class StepOpts(ctypes.Structure):
    """kda_step_opts of include/kda.h (model-layer options of decode/verify)."""
    _fields_ = [("gate_mode", ctypes.c_int32), ("A_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p), ("lower_bound", ctypes.c_float),
                ("per_head_gate", ctypes.c_int32), ("qk_l2norm", ctypes.c_int32),
                ("qk_heads", ctypes.c_int32), ("o_gate", ctypes.c_void_p),
                ("o_norm_w", ctypes.c_void_p), ("o_norm_eps", ctypes.c_float),
                ("o_gate_act", ctypes.c_int32)]


class KdaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libkda.so (built by ``kda_gated_delta_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m kda_gated_delta_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                             ctypes.c_float, ctypes.c_size_t)
    L.kda_status_string.argtypes = [ctypes.c_int]
    L.kda_status_string.restype = ctypes.c_char_p
    L.kda_gate_prep.argtypes = [vp, vp, vp, vp, i64, i32, i32, f32, vp, vp, vp]
    L.kda_gate_prep.restype = ctypes.c_int
    L.kda_chunk_prefill_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32,
                                                   ctypes.POINTER(sz)]
    L.kda_chunk_prefill_workspace_size.restype = ctypes.c_int
    L.kda_chunk_prefill.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, i32, i64,
                                    i32, i32, i32, i32, f32, vp, vp, vp, vp, sz, vp]
    L.kda_chunk_prefill.restype = ctypes.c_int
    L.kda_chunk_prefill_gated.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, f32, vp,
                                          i32, i64, i32, i32, i32, i32, f32, vp, vp, vp, vp,
                                          sz, vp]
    L.kda_chunk_prefill_gated.restype = ctypes.c_int
    L.kda_chunk_prefill_snapshots.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, i32, i64,
                                              i32, i32, i32, i32, f32, vp, vp, vp, vp, i64, i32,
                                              vp, sz, vp]
    L.kda_chunk_prefill_snapshots.restype = ctypes.c_int
    L.kda_chunk_prefill_marked.argtypes = L.kda_chunk_prefill_gated.argtypes + [vp]
    L.kda_chunk_prefill_marked.restype = ctypes.c_int
    L.kda_recurrent_decode.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, f32, vp, i64,
                                       vp, i32, i32, i32, i32, vp, vp]
    L.kda_recurrent_decode.restype = ctypes.c_int
    L.kda_verify.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, f32, vp, i64, vp, i32,
                             i32, i32, i32, i32, vp, vp, vp]
    L.kda_verify.restype = ctypes.c_int
    L.kda_chunk_prefill_ex.argtypes = L.kda_chunk_prefill.argtypes[:-1] + [
        ctypes.POINTER(PrefillOpts), vp]
    L.kda_chunk_prefill_ex.restype = ctypes.c_int
    L.kda_chunk_prefill_noalloc.argtypes = L.kda_chunk_prefill.argtypes[:-3] + [
        ctypes.POINTER(PrefillOpts), vp]
    L.kda_chunk_prefill_noalloc.restype = ctypes.c_int
    L.kda_recurrent_decode_ex.argtypes = L.kda_recurrent_decode.argtypes[:-1] + [
        ctypes.POINTER(StepOpts), vp]
    L.kda_recurrent_decode_ex.restype = ctypes.c_int
    L.kda_verify_ex.argtypes = L.kda_verify.argtypes[:-1] + [ctypes.POINTER(StepOpts), vp]
    L.kda_verify_ex.restype = ctypes.c_int
    L.kda_replay_decode.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, f32, vp, i64, vp, vp, vp,
                                    i32, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp]
    L.kda_replay_decode.restype = ctypes.c_int
    L.kda_replay_decode_ex.argtypes = L.kda_replay_decode.argtypes[:-1] + [
        ctypes.POINTER(StepOpts), vp]
    L.kda_replay_decode_ex.restype = ctypes.c_int
    L.kda_chunk_prefill_schedule.argtypes = [i64, i32, i32, i32, i32, i32,
                                             ctypes.POINTER(PrefillSchedule)]
    L.kda_chunk_prefill_schedule.restype = ctypes.c_int
    _lib = L
    return L


# every entry point declared in include/kda.h and include/kda_profile.h
EXPORTED = ("kda_status_string", "kda_gate_prep", "kda_chunk_prefill_workspace_size",
            "kda_chunk_prefill", "kda_chunk_prefill_marked", "kda_chunk_prefill_gated",
            "kda_chunk_prefill_snapshots",
            "kda_recurrent_decode", "kda_verify", "kda_replay_decode",
            "kda_recurrent_decode_ex", "kda_verify_ex", "kda_chunk_prefill_ex",
            "kda_replay_decode_ex", "kda_chunk_prefill_noalloc", "kda_chunk_prefill_schedule")

# Bytes of the static scratch array behind kda_chunk_prefill_noalloc
# (KDA_NOALLOC_SCRATCH_BYTES of include/kda.h).
NOALLOC_SCRATCH_BYTES = 256 << 20


def status_string(status: int) -> str:
    return lib().kda_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise KdaError(fn, status)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape, device) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _io_dtype(t: torch.Tensor) -> int:
    if t.dtype not in _IO:
        raise TypeError(f"io dtype must be float32 or bfloat16, got {t.dtype}")
    return _IO[t.dtype]


def kda_gate_prep(a, b, A_log, dt_bias=None, lower_bound: float = 0.0,
                  g=None, beta=None):
    """g [T,H,K], beta [T,H] (fp32) from a [T,H,K], b [T,H], A_log [H],
    dt_bias [H,K] (or None).  ``lower_bound < 0`` selects the safe gate."""
    T, H, K = a.shape
    dev = a.device
    _need(a, "a", torch.float32, (T, H, K), dev)
    _need(b, "b", torch.float32, (T, H), dev)
    _need(A_log, "A_log", torch.float32, (H,), dev)
    if dt_bias is not None:
        _need(dt_bias, "dt_bias", torch.float32, (H, K), dev)
    g = torch.empty_like(a) if g is None else g
    beta = torch.empty_like(b) if beta is None else beta
    _need(g, "g", torch.float32, (T, H, K), dev)
    _need(beta, "beta", torch.float32, (T, H), dev)
    _check("kda_gate_prep", lib().kda_gate_prep(
        _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), T, H, K, float(lower_bound),
        _ptr(g), _ptr(beta), _stream(dev)))
    return g, beta


def kda_chunk_prefill_workspace_size(T: int, N: int, H: int, K: int, V: int,
                                     chunk: int = 64) -> int:
    """Bytes of workspace kda_chunk_prefill needs (raises KdaError for a
    shape the prefill does not build)."""
    n = ctypes.c_size_t(0)
    _check("kda_chunk_prefill_workspace_size",
           lib().kda_chunk_prefill_workspace_size(T, N, H, K, V, chunk, ctypes.byref(n)))
    return int(n.value)


def kda_chunk_prefill_schedule(T: int, N: int, H: int, K: int, V: int,
                               chunk: int = 64) -> dict:
    """Kernels a prefill call of these sizes launches (include/kda_profile.h):
    n_waves, segment_chunks, uses_maps, intra_launches, state_launches,
    other_launches."""
    out = PrefillSchedule()
    _check("kda_chunk_prefill_schedule",
           lib().kda_chunk_prefill_schedule(T, N, H, K, V, chunk, ctypes.byref(out)))
    return {name: int(getattr(out, name)) for name, _ in PrefillSchedule._fields_}


def kda_chunk_prefill(q, k, v, g, beta, cu_seqlens, scale: float, h0=None,
                      output_final_state: bool = True, chunk: int = 64, o=None,
                      ht=None, workspace=None):
    """Varlen chunkwise prefill.  Returns (o [T,H,V], ht [N,H,K,V] or None).

    ``ht`` may be passed explicitly (it may be ``h0`` itself for an in-place
    update); ``workspace`` is a uint8 device tensor of at least
    ``kda_chunk_prefill_workspace_size`` bytes (allocated here if None).
    """
    return _prefill("kda_chunk_prefill", None, q, k, v, g, beta, cu_seqlens, scale, h0,
                    output_final_state, chunk, o, ht, workspace)


def kda_chunk_prefill_snapshots(q, k, v, g, beta, cu_seqlens, scale: float,
                                snapshot_interval: int, h0=None,
                                output_final_state: bool = True, chunk: int = 64, o=None,
                                ht=None, snapshots=None, workspace=None):
    """kda_chunk_prefill that also records each sequence's state after every
    ``snapshot_interval`` tokens (a multiple of ``chunk``) into
    ``snapshots`` [rows, H, K, V] fp32, sequence after sequence (allocated
    with T // snapshot_interval rows if None).  Returns (o, ht, snapshots)."""
    T, H, K = q.shape
    V = v.shape[2]
    dev = q.device
    if snapshots is None:
        snapshots = torch.empty((max(T // snapshot_interval, 1), H, K, V), dtype=torch.float32,
                                device=dev)
    _need(snapshots, "snapshots", torch.float32, (snapshots.shape[0], H, K, V), dev)
    o, ht = _prefill("kda_chunk_prefill_snapshots", None, q, k, v, g, beta, cu_seqlens, scale,
                     h0, output_final_state, chunk, o, ht, workspace,
                     snap=(snapshots, int(snapshot_interval)))
    return o, ht, snapshots


def kda_chunk_prefill_gated(q, k, v, a, b, A_log, dt_bias, cu_seqlens, scale: float,
                            lower_bound: float = 0.0, h0=None,
                            output_final_state: bool = True, chunk: int = 64, o=None,
                            ht=None, workspace=None):
    """kda_gate_prep + kda_chunk_prefill in one call: a [T,H,K] and b [T,H]
    are the raw gate inputs (A_log [H], dt_bias [H,K] or None)."""
    T, H, K = q.shape
    dev = q.device
    _need(a, "a", torch.float32, (T, H, K), dev)
    _need(b, "b", torch.float32, (T, H), dev)
    _need(A_log, "A_log", torch.float32, (H,), dev)
    if dt_bias is not None:
        _need(dt_bias, "dt_bias", torch.float32, (H, K), dev)
    return _prefill("kda_chunk_prefill_gated", None, q, k, v, a, b, cu_seqlens, scale, h0,
                    output_final_state, chunk, o, ht, workspace,
                    gate=(A_log, dt_bias, float(lower_bound)))


def kda_chunk_prefill_marked(marks, q, k, v, a, b, A_log, dt_bias, cu_seqlens,
                             scale: float, lower_bound: float = 0.0, h0=None,
                             output_final_state: bool = True, chunk: int = 64, o=None,
                             ht=None, workspace=None):
    """kda_chunk_prefill_gated that also records the four ``torch.cuda.Event``s
    in ``marks`` around its three kernels (chunk table, intra-chunk, state
    pass): ``marks[i].elapsed_time(marks[i + 1])`` is kernel i's duration."""
    if len(marks) != 4:
        raise ValueError("marks: expected 4 events")
    for m in marks:
        if not m.cuda_event:  # events are created lazily by their first record
            m.record()
    T, H, K = q.shape
    dev = q.device
    _need(a, "a", torch.float32, (T, H, K), dev)
    _need(b, "b", torch.float32, (T, H), dev)
    _need(A_log, "A_log", torch.float32, (H,), dev)
    if dt_bias is not None:
        _need(dt_bias, "dt_bias", torch.float32, (H, K), dev)
    return _prefill("kda_chunk_prefill_marked", marks, q, k, v, a, b, cu_seqlens, scale, h0,
                    output_final_state, chunk, o, ht, workspace,
                    gate=(A_log, dt_bias, float(lower_bound)))


def _prefill(fn, marks, q, k, v, g, beta, cu_seqlens, scale, h0, output_final_state,
             chunk, o, ht, workspace, gate=None, snap=None):
    T, H, K = q.shape
    V = v.shape[2]
    dev = q.device
    io = _io_dtype(q)
    N = cu_seqlens.shape[0] - 1
    _need(q, "q", q.dtype, (T, H, K), dev)
    _need(k, "k", q.dtype, (T, H, K), dev)
    _need(v, "v", q.dtype, (T, H, V), dev)
    _need(g, "g", torch.float32, (T, H, K), dev)
    _need(beta, "beta", torch.float32, (T, H), dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    if h0 is not None:
        _need(h0, "h0", torch.float32, (N, H, K, V), dev)
    if ht is None and output_final_state:
        ht = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
    if ht is not None:
        _need(ht, "ht", torch.float32, (N, H, K, V), dev)
    o = torch.empty((T, H, V), dtype=q.dtype, device=dev) if o is None else o
    _need(o, "o", q.dtype, (T, H, V), dev)
    need = kda_chunk_prefill_workspace_size(T, N, H, K, V, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    args = [io, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, T,
            H, K, V, chunk, float(scale), _ptr(h0), _ptr(ht), _ptr(o), _ptr(workspace),
            workspace.numel(), _stream(dev)]
    if gate is not None:
        A_log, dt_bias, lb = gate
        gargs = [io, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log), _ptr(dt_bias),
                 lb, _ptr(cu_seqlens), N, T, H, K, V, chunk, float(scale), _ptr(h0), _ptr(ht),
                 _ptr(o), _ptr(workspace), workspace.numel(), _stream(dev)]
        if marks is None:
            _check(fn, lib().kda_chunk_prefill_gated(*gargs))
        else:
            arr = (ctypes.c_void_p * 4)(*[m.cuda_event for m in marks])
            _check(fn, lib().kda_chunk_prefill_marked(*gargs, arr))
    elif snap is not None:
        snapshots, interval = snap
        sargs = args[:17] + [_ptr(snapshots), snapshots.shape[0], interval] + args[17:]
        _check(fn, lib().kda_chunk_prefill_snapshots(*sargs))
    else:
        _check(fn, lib().kda_chunk_prefill(*args))
    return o, ht


def kda_recurrent_decode(q, k, v, g, beta, scale: float, state_pool, slot_idx,
                         o=None):
    """Single-token decode; ``state_pool`` [n_slots,H,K,V] is updated in place.
    Returns o [B,H,V]."""
    B, H, K = q.shape
    V = v.shape[2]
    dev = q.device
    io = _io_dtype(q)
    n_slots = state_pool.shape[0]
    _need(k, "k", q.dtype, (B, H, K), dev)
    _need(v, "v", q.dtype, (B, H, V), dev)
    _need(g, "g", torch.float32, (B, H, K), dev)
    _need(beta, "beta", torch.float32, (B, H), dev)
    _need(state_pool, "state_pool", torch.float32, (n_slots, H, K, V), dev)
    _need(slot_idx, "slot_idx", torch.int32, (B,), dev)
    o = torch.empty((B, H, V), dtype=q.dtype, device=dev) if o is None else o
    _need(o, "o", q.dtype, (B, H, V), dev)
    _check("kda_recurrent_decode", lib().kda_recurrent_decode(
        io, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
        _ptr(state_pool), n_slots, _ptr(slot_idx), B, H, K, V, _ptr(o), _stream(dev)))
    return o


def kda_verify(q, k, v, g, beta, scale: float, state_pool, slot_idx,
               inter_states=None, o=None):
    """Multi-token verify; the pool is only read.  Returns (o [B,Tv,H,V],
    inter_states [B,Tv,H,K,V])."""
    B, Tv, H, K = q.shape
    V = v.shape[3]
    dev = q.device
    io = _io_dtype(q)
    n_slots = state_pool.shape[0]
    _need(k, "k", q.dtype, (B, Tv, H, K), dev)
    _need(v, "v", q.dtype, (B, Tv, H, V), dev)
    _need(g, "g", torch.float32, (B, Tv, H, K), dev)
    _need(beta, "beta", torch.float32, (B, Tv, H), dev)
    _need(state_pool, "state_pool", torch.float32, (n_slots, H, K, V), dev)
    _need(slot_idx, "slot_idx", torch.int32, (B,), dev)
    if inter_states is None:
        inter_states = torch.empty((B, Tv, H, K, V), dtype=torch.float32, device=dev)
    _need(inter_states, "inter_states", torch.float32, (B, Tv, H, K, V), dev)
    o = torch.empty((B, Tv, H, V), dtype=q.dtype, device=dev) if o is None else o
    _need(o, "o", q.dtype, (B, Tv, H, V), dev)
    _check("kda_verify", lib().kda_verify(
        io, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
        _ptr(state_pool), n_slots, _ptr(slot_idx), B, Tv, H, K, V,
        _ptr(inter_states), _ptr(o), _stream(dev)))
    return o, inter_states


def kda_replay_decode(q, k, v, g, beta, scale: float, state_pool, slot_idx, write_pos,
                      ring_d, ring_k, ring_g, force_flush=None, o=None, next_write_pos=None,
                      raw_gate=None, per_head_gate=False, qk_l2norm=False, o_gate=None,
                      o_norm_w=None, o_norm_eps: float = 1e-6, o_gate_act: str = "sigmoid"):
    """Buffered single-token decode.  ``state_pool`` [n_slots,H,K,V] holds the
    checkpoints; the rings ring_d [n_slots,H,L,V] fp32, ring_k [n_slots,H,L,K]
    (io dtype) and ring_g [n_slots,H,L,K] fp32 hold the steps since them;
    ``write_pos`` [B] int32 is each row's cursor.  ``raw_gate`` = (A_log,
    dt_bias, lower_bound) applies the gate to the raw a given as g (beta is
    then the raw b); ``per_head_gate`` takes g [B,H]; q, k may have fewer
    heads than v (grouped heads); ``qk_l2norm`` and ``o_gate`` (with
    ``o_norm_w``) as in kda_recurrent_decode_ex.  Returns (o [B,H,V],
    next_write_pos [B])."""
    B, HK, K = q.shape
    H, V = v.shape[1], v.shape[2]
    dev = q.device
    io = _io_dtype(q)
    n_slots = state_pool.shape[0]
    L = ring_d.shape[2]
    _need(k, "k", q.dtype, (B, HK, K), dev)
    _need(v, "v", q.dtype, (B, H, V), dev)
    _need(g, "g", torch.float32, (B, H) if per_head_gate else (B, H, K), dev)
    _need(beta, "beta", torch.float32, (B, H), dev)
    _need(state_pool, "state_pool", torch.float32, (n_slots, H, K, V), dev)
    _need(slot_idx, "slot_idx", torch.int32, (B,), dev)
    _need(write_pos, "write_pos", torch.int32, (B,), dev)
    if force_flush is not None:
        _need(force_flush, "force_flush", torch.int32, (B,), dev)
    _need(ring_d, "ring_d", torch.float32, (n_slots, H, L, V), dev)
    _need(ring_k, "ring_k", q.dtype, (n_slots, H, L, K), dev)
    _need(ring_g, "ring_g", torch.float32, (n_slots, H, L, K), dev)
    o = torch.empty((B, H, V), dtype=q.dtype, device=dev) if o is None else o
    _need(o, "o", q.dtype, (B, H, V), dev)
    if next_write_pos is None:
        next_write_pos = torch.empty((B,), dtype=torch.int32, device=dev)
    _need(next_write_pos, "next_write_pos", torch.int32, (B,), dev)
    args = [io, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(state_pool),
            n_slots, _ptr(slot_idx), _ptr(write_pos), _ptr(force_flush), L, _ptr(ring_d),
            _ptr(ring_k), _ptr(ring_g), B, H, K, V, _ptr(o), _ptr(next_write_pos)]
    if raw_gate is None and not per_head_gate and HK == H and not qk_l2norm and o_gate is None:
        _check("kda_replay_decode", lib().kda_replay_decode(*args, _stream(dev)))
    else:
        op = _step_opts(H, (B,), K, V, dev, q.dtype, raw_gate, per_head_gate, qk_l2norm, HK,
                        o_gate, o_norm_w, o_norm_eps, o_gate_act)
        _check("kda_replay_decode_ex", lib().kda_replay_decode_ex(*args, ctypes.byref(op),
                                                                  _stream(dev)))
    return o, next_write_pos


def _step_opts(H, lead, K, V, dev, dtype, raw_gate, per_head_gate, qk_l2norm, qk_heads, o_gate,
               o_norm_w, o_norm_eps, o_gate_act):
    """Checks the model-layer options and packs them (the tensors must stay
    alive during the call)."""
    op = StepOpts()
    if raw_gate is not None:
        A_log, dt_bias, lower_bound = raw_gate
        _need(A_log, "A_log", torch.float32, (H,), dev)
        if dt_bias is not None:
            _need(dt_bias, "dt_bias", torch.float32, (H,) if per_head_gate else (H, K), dev)
        op.gate_mode = 2 if lower_bound < 0 else 1
        op.A_log = A_log.data_ptr()
        op.dt_bias = None if dt_bias is None else dt_bias.data_ptr()
        op.lower_bound = float(lower_bound)
    op.per_head_gate = int(bool(per_head_gate))
    op.qk_l2norm = int(bool(qk_l2norm))
    op.qk_heads = int(qk_heads or 0)
    if o_gate is not None:
        _need(o_gate, "o_gate", dtype, lead + (H, V), dev)
        _need(o_norm_w, "o_norm_w", torch.float32, (V,), dev)
        op.o_gate = o_gate.data_ptr()
        op.o_norm_w = o_norm_w.data_ptr()
        op.o_norm_eps = float(o_norm_eps)
        op.o_gate_act = {"sigmoid": 0, "silu": 1}[o_gate_act]
    return op


def kda_recurrent_decode_ex(q, k, v, g, beta, scale: float, state_pool, slot_idx, *,
                            raw_gate=None, per_head_gate=False, qk_l2norm=False,
                            o_gate=None, o_norm_w=None, o_norm_eps: float = 1e-6,
                            o_gate_act: str = "sigmoid", o=None):
    """Decode with model-layer options: q, k [B,HK,K]; v [B,H,V]; g [B,H,K]
    (or [B,H] with per_head_gate), raw a when ``raw_gate`` = (A_log,
    dt_bias, lower_bound) is given (then beta holds the raw b); ``o_gate``
    [B,H,V] with ``o_norm_w`` [V] applies the gated RMSNorm to o."""
    B, HK, K = q.shape
    H, V = v.shape[1], v.shape[2]
    dev = q.device
    io = _io_dtype(q)
    n_slots = state_pool.shape[0]
    _need(k, "k", q.dtype, (B, HK, K), dev)
    _need(v, "v", q.dtype, (B, H, V), dev)
    _need(g, "g", torch.float32, (B, H) if per_head_gate else (B, H, K), dev)
    _need(beta, "beta", torch.float32, (B, H), dev)
    _need(state_pool, "state_pool", torch.float32, (n_slots, H, K, V), dev)
    _need(slot_idx, "slot_idx", torch.int32, (B,), dev)
    op = _step_opts(H, (B,), K, V, dev, q.dtype, raw_gate, per_head_gate, qk_l2norm, HK, o_gate,
                    o_norm_w, o_norm_eps, o_gate_act)
    o = torch.empty((B, H, V), dtype=q.dtype, device=dev) if o is None else o
    _need(o, "o", q.dtype, (B, H, V), dev)
    _check("kda_recurrent_decode_ex", lib().kda_recurrent_decode_ex(
        io, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
        _ptr(state_pool), n_slots, _ptr(slot_idx), B, H, K, V, _ptr(o), ctypes.byref(op),
        _stream(dev)))
    return o


def kda_verify_ex(q, k, v, g, beta, scale: float, state_pool, slot_idx, *, raw_gate=None,
                  per_head_gate=False, qk_l2norm=False, o_gate=None, o_norm_w=None,
                  o_norm_eps: float = 1e-6, o_gate_act: str = "sigmoid", inter_states=None,
                  o=None):
    """Verify with model-layer options (see kda_recurrent_decode_ex); q, k
    [B,Tv,HK,K], v [B,Tv,H,V].  Returns (o, inter_states)."""
    B, Tv, HK, K = q.shape
    H, V = v.shape[2], v.shape[3]
    dev = q.device
    io = _io_dtype(q)
    n_slots = state_pool.shape[0]
    _need(k, "k", q.dtype, (B, Tv, HK, K), dev)
    _need(v, "v", q.dtype, (B, Tv, H, V), dev)
    _need(g, "g", torch.float32, (B, Tv, H) if per_head_gate else (B, Tv, H, K), dev)
    _need(beta, "beta", torch.float32, (B, Tv, H), dev)
    _need(state_pool, "state_pool", torch.float32, (n_slots, H, K, V), dev)
    _need(slot_idx, "slot_idx", torch.int32, (B,), dev)
    op = _step_opts(H, (B, Tv), K, V, dev, q.dtype, raw_gate, per_head_gate, qk_l2norm, HK,
                    o_gate, o_norm_w, o_norm_eps, o_gate_act)
    if inter_states is None:
        inter_states = torch.empty((B, Tv, H, K, V), dtype=torch.float32, device=dev)
    _need(inter_states, "inter_states", torch.float32, (B, Tv, H, K, V), dev)
    o = torch.empty((B, Tv, H, V), dtype=q.dtype, device=dev) if o is None else o
    _need(o, "o", q.dtype, (B, Tv, H, V), dev)
    _check("kda_verify_ex", lib().kda_verify_ex(
        io, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(state_pool),
        n_slots, _ptr(slot_idx), B, Tv, H, K, V, _ptr(inter_states), _ptr(o),
        ctypes.byref(op), _stream(dev)))
    return o, inter_states


def _prefill_ex_args(q, k, v, g, beta, cu_seqlens, raw_gate, per_head_gate, h0, ht, o,
                     snapshots, snapshot_interval, qk_l2norm):
    """Checks the tensors of a prefill with options; returns (PrefillOpts,
    T, N, H, K, V, io)."""
    T, HK, K = q.shape
    H, V = v.shape[1], v.shape[2]
    dev = q.device
    io = _io_dtype(q)
    N = cu_seqlens.shape[0] - 1
    _need(k, "k", q.dtype, (T, HK, K), dev)
    _need(v, "v", q.dtype, (T, H, V), dev)
    _need(g, "g", torch.float32, (T, H) if per_head_gate else (T, H, K), dev)
    _need(beta, "beta", torch.float32, (T, H), dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    if h0 is not None:
        _need(h0, "h0", torch.float32, (N, H, K, V), dev)
    if ht is not None:
        _need(ht, "ht", torch.float32, (N, H, K, V), dev)
    _need(o, "o", q.dtype, (T, H, V), dev)
    op = PrefillOpts()
    if raw_gate is not None:
        A_log, dt_bias, lower_bound = raw_gate
        _need(A_log, "A_log", torch.float32, (H,), dev)
        if dt_bias is not None:
            _need(dt_bias, "dt_bias", torch.float32, (H,) if per_head_gate else (H, K), dev)
        op.gate_mode = 2 if lower_bound < 0 else 1
        op.A_log = A_log.data_ptr()
        op.dt_bias = None if dt_bias is None else dt_bias.data_ptr()
        op.lower_bound = float(lower_bound)
    op.per_head_gate = int(bool(per_head_gate))
    op.qk_heads = HK
    op.qk_l2norm = int(bool(qk_l2norm))
    if snapshots is not None:
        _need(snapshots, "snapshots", torch.float32, (snapshots.shape[0], H, K, V), dev)
        op.snapshots = snapshots.data_ptr()
        op.snapshot_rows = snapshots.shape[0]
        op.snapshot_interval = int(snapshot_interval)
    return op, T, N, H, K, V, io


def kda_chunk_prefill_ex(q, k, v, g, beta, cu_seqlens, scale: float, *, raw_gate=None,
                         per_head_gate=False, h0=None, output_final_state: bool = True,
                         chunk: int = 64, o=None, ht=None, snapshots=None,
                         snapshot_interval: int = 0, qk_l2norm: bool = False,
                         workspace=None):
    """Prefill with model-layer options: q, k [T,HK,K]; v [T,H,V]; g [T,H,K]
    (or [T,H] with per_head_gate), raw a when ``raw_gate`` = (A_log,
    dt_bias, lower_bound) is given (then beta holds the raw b); snapshots as
    in kda_chunk_prefill_snapshots; ``qk_l2norm``: q and k L2-normalised in
    the kernel.  Returns (o, ht)."""
    T, H, V = q.shape[0], v.shape[1], v.shape[2]
    K, N, dev = q.shape[2], cu_seqlens.shape[0] - 1, q.device
    if ht is None and output_final_state:
        ht = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
    o = torch.empty((T, H, V), dtype=q.dtype, device=dev) if o is None else o
    op, T, N, H, K, V, io = _prefill_ex_args(q, k, v, g, beta, cu_seqlens, raw_gate,
                                             per_head_gate, h0, ht, o, snapshots,
                                             snapshot_interval, qk_l2norm)
    need = kda_chunk_prefill_workspace_size(T, N, H, K, V, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check("kda_chunk_prefill_ex", lib().kda_chunk_prefill_ex(
        io, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, T, H, K, V,
        chunk, float(scale), _ptr(h0), _ptr(ht), _ptr(o), _ptr(workspace), workspace.numel(),
        ctypes.byref(op), _stream(dev)))
    return o, ht


def kda_chunk_prefill_noalloc(q, k, v, g, beta, cu_seqlens, scale: float, o, *, ht=None,
                              raw_gate=None, per_head_gate=False, h0=None, chunk: int = 64,
                              snapshots=None, snapshot_interval: int = 0,
                              qk_l2norm: bool = False):
    """kda_chunk_prefill_ex on the library's static scratch: allocates
    nothing.  The caller passes every output: ``o`` [T,H,V] and, to receive
    the final states, ``ht`` [N,H,K,V] (None: not written).  Raises KdaError
    with KDA_ERR_SCRATCH_LIMIT when the batch needs more workspace than
    KDA_NOALLOC_SCRATCH_BYTES.  Returns (o, ht)."""
    op, T, N, H, K, V, io = _prefill_ex_args(q, k, v, g, beta, cu_seqlens, raw_gate,
                                             per_head_gate, h0, ht, o, snapshots,
                                             snapshot_interval, qk_l2norm)
    _check("kda_chunk_prefill_noalloc", lib().kda_chunk_prefill_noalloc(
        io, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, T, H, K, V,
        chunk, float(scale), _ptr(h0), _ptr(ht), _ptr(o), ctypes.byref(op), _stream(q.device)))
    return o, ht
