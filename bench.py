"""Benchmark of the KDA hot path on one MI355X.

One step = gate activation + chunkwise prefill of the packed varlen batch of
four sequences {512, 1024, 2048, 4096} (H=32, K=V=128, bf16 q/k/v, fp32 raw
gate inputs and states, chunk 64), inputs resident in HBM, as one
kda_chunk_prefill_gated call (the gate evaluated inside the prefill; the
two-call sequence kda_gate_prep + kda_chunk_prefill is timed beside it).
``value`` is prefill tokens/s of that step.  The same run also measures, each on its own workload:
  decode  - 256 single-token requests on a 512-slot fp32 state pool
            (tokens/s and state GB/s against HBM peak);
  verify  - 64 requests x 8 draft tokens on a 128-slot pool;
  long    - one 65536-token sequence as 16 carried 4096-token segments;
and the fp64 CPU oracle on the prefill workload (``cpu_baseline``).

Timing uses HIP events on the stream the library launches on (torch's
current stream): W untimed warm-up steps, then K steps bracketed by
synchronisations.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import kda_gated_delta_amd as kda  # noqa: E402
import kda_synth  # noqa: E402
from kda_gated_delta_amd import ceilings  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published


def _dev(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda().to(dtype).contiguous()


SETTLE_S = 0.2  # --settle


def _time(fn, steps: int, warmup: int, settle_s: float | None = None) -> float:
    """Average milliseconds per call of fn over `steps` calls.  The `warmup`
    calls are followed by further untimed calls until `settle_s` seconds have
    passed: the GPU's clocks take tens of milliseconds to rise from idle, and
    a timed region that starts earlier measures that ramp, not the kernels."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    settle_s = SETTLE_S if settle_s is None else settle_s
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


# ------------------------------------------------------------ byte models

_FLUSH = None


def _fresh_memory():
    """Returns torch's cached device blocks to the driver before a workload
    allocates its own buffers, so that each workload's buffers are fresh
    allocations.  Without it, a buffered-decode run that followed the other
    workloads in one process, on a GPU that other processes had just used,
    was measured 7-8x slower (0.84-0.90 ms against 0.112 ms in every other
    arrangement) with unchanged kernels: the timing of its scattered
    per-slot reads depended on where the allocation history put them."""
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _time_flushed(fn, reps: int = 20) -> float:
    """Median milliseconds of single calls of fn, each timed alone between
    HIP events after a write and then a read of a 512 MiB scratch buffer
    (twice the 256 MB last-level cache): no input of fn is served from that
    cache, and the read leaves no dirty lines whose write-back would fall in
    the timed call."""
    global _FLUSH
    if _FLUSH is None:
        _FLUSH = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
    fn()
    times = []
    for _ in range(reps):
        _FLUSH.fill_(1.0)
        _FLUSH.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return float(np.median(times))


def prefill_bytes(T, N, H, K, V, io_bytes=2):
    """Algorithmic HBM bytes of one prefill call: q, k, v, o in the io dtype,
    g fp32, beta fp32 per token-head; h0 read and ht written per sequence."""
    per_tok_head = (2 * K + 2 * V) * io_bytes + 4 * K + 4
    return T * H * per_tok_head + 2 * N * H * K * V * 4


def intra_bytes(T, H, K, V, io_bytes=2):
    """Algorithmic bytes the intra-chunk kernel must move: it is the only
    reader of q, k, v and of the gate inputs (a and b, or the activated g and
    beta: the same sizes)."""
    return T * H * ((2 * K + V) * io_bytes + 4 * K + 4)


def state_bytes(T, N, H, K, V, io_bytes=2):
    """Algorithmic bytes the state kernel must move: o written, h0 read and
    ht written.  intra_bytes + state_bytes = prefill_bytes."""
    return T * H * V * io_bytes + 2 * N * H * K * V * 4


def intra_flops(T, H, K, V, C):
    """Algorithmic flops of the intra-chunk kernel per token-head: the
    strictly lower decayed K K^T ((C-1)/2 pairs per token), the lower decayed
    Q K^T with diagonal ((C+1)/2), and the two triangular products W = M (K e^G)
    and U = M V; 2 flops per multiply-add."""
    return T * H * ((C - 1) * K + (C + 1) * K + (C + 1) * K + (C + 1) * V)


def state_flops(T, H, K, V, C):
    """Algorithmic flops of the state kernel per token-head: W S, (Q e^G) S
    and (K e^{G_C - G})^T D (K V multiply-adds each) and the lower-triangular
    Aq D ((C+1)/2 V)."""
    return T * H * (6 * K * V + (C + 1) * V)


def gate_bytes(T, H, K):
    """a read, g written (fp32, per channel); b read, beta written."""
    return T * H * (8 * K + 8)


def prefill_flops(T, H, K, V, C):
    """Algorithmic flops per token-head of the chunk form (triangle-aware):
    2 (3 K V + C K + (C-1) K / 2 + C V)."""
    return T * H * 2 * (3 * K * V + C * K + (C - 1) * K / 2 + C * V)


def decode_bytes(B, H, K, V, io_bytes=2):
    """State read + write (fp32) plus q, k, v, o, g, beta per request-head."""
    return B * H * (2 * K * V * 4 + (2 * K + 2 * V) * io_bytes + 4 * K + 4)


def verify_bytes(B, Tv, H, K, V, io_bytes=2):
    """One state read, Tv state writes, and the per-token inputs/outputs."""
    return B * H * (K * V * 4 * (1 + Tv) + Tv * ((2 * K + 2 * V) * io_bytes + 4 * K + 4))


def replay_bytes(write_pos, flush, H, K, V, io_bytes=2):
    """Buffered decode: the checkpoint read, the ring entries read (m of
    them: k in the io dtype, g and d fp32), the checkpoint written by a
    flushing row or one ring entry appended by the others, and the token's
    q, k, v, o, g, beta, per request-head."""
    entry = K * io_bytes + 4 * K + 4 * V
    tok = (2 * K + 2 * V) * io_bytes + 4 * K + 4
    per_row = [K * V * 4 + m * entry + (K * V * 4 if f else entry) + tok
               for m, f in zip(write_pos, flush)]
    return int(H * sum(int(x) for x in per_row))


# -------------------------------------------------------------- workloads

def prefill_setup(name):
    w = kda_synth.WORKLOADS[name]
    c = kda_synth.prefill_case(w["seqlens"], w["H"], w["K"], w["V"], w["io"], seed=w["seed"],
                               dt_bias_std=w["dt_bias_std"], h0_std=w["h0_std"])
    io = torch.bfloat16 if w["io"] == "bf16" else torch.float32
    t = dict(q=_dev(c["q"], io), k=_dev(c["k"], io), v=_dev(c["v"], io), a=_dev(c["a"]),
             b=_dev(c["b"]), A_log=_dev(c["A_log"]), dt_bias=_dev(c["dt_bias"]),
             cu=_dev(c["cu"], torch.int32), h0=_dev(c["h0"]))
    return w, c, t


def bench_prefill(steps, warmup):
    w, c, t = prefill_setup("varlen_prefill_7680")
    T, N, H, K, V, C = c["T"], c["N"], w["H"], w["K"], w["V"], w["chunk"]
    scale = K ** -0.5
    g = torch.empty_like(t["a"])
    beta = torch.empty_like(t["b"])
    o = torch.empty_like(t["v"])
    ht = torch.empty_like(t["h0"])
    ws = torch.empty(kda.kda_chunk_prefill_workspace_size(T, N, H, K, V, C),
                     dtype=torch.uint8, device="cuda")

    # A plain elementwise copy (negation) of known size, 256 MiB read and
    # 256 MiB written, outside every timed region: the reference point that scales rocprofv3's FETCH_SIZE and
    # WRITE_SIZE counters to bytes.
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
    torch.neg(src, out=torch.empty_like(src))
    del src

    def gate():
        kda.kda_gate_prep(t["a"], t["b"], t["A_log"], t["dt_bias"], g=g, beta=beta)

    def prefill():
        kda.kda_chunk_prefill(t["q"], t["k"], t["v"], g, beta, t["cu"], scale, h0=t["h0"],
                              chunk=C, o=o, ht=ht, workspace=ws)

    def step():  # the gate applied inside the prefill: g and beta never hit HBM
        kda.kda_chunk_prefill_gated(t["q"], t["k"], t["v"], t["a"], t["b"], t["A_log"],
                                    t["dt_bias"], t["cu"], scale, h0=t["h0"], chunk=C, o=o,
                                    ht=ht, workspace=ws)

    def step_two_calls():
        gate()
        prefill()

    snaps = torch.empty((T // 256, H, K, V), device="cuda")

    def prefill_snapshots():  # the state after every 256 tokens kept as well
        kda.kda_chunk_prefill_snapshots(t["q"], t["k"], t["v"], g, beta, t["cu"], scale, 256,
                                        h0=t["h0"], chunk=C, o=o, ht=ht, snapshots=snaps,
                                        workspace=ws)

    ms_step = _time(step, steps, warmup)
    ms_step_two_calls = _time(step_two_calls, steps, warmup)
    ms_gate = _time(gate, steps, warmup)
    ms_prefill = _time(prefill, steps, warmup)
    ms_snapshots = _time(prefill_snapshots, steps, warmup)
    n_snaps = sum(int(c["cu"][i + 1] - c["cu"][i]) // 256 for i in range(N))
    kernels = kernel_times(t, o, ht, ws, scale, C, steps)
    pb = prefill_bytes(T, N, H, K, V)
    gb = gate_bytes(T, H, K)
    return dict(workload=w, T=T, N=N, ms_step=ms_step, ms_step_two_calls=ms_step_two_calls,
                ms_gate=ms_gate,
                ms_prefill=ms_prefill, prefill_bytes=pb, gate_bytes=gb,
                ms_snapshots=ms_snapshots, snapshot_bytes=n_snaps * H * K * V * 4,
                intra_bytes=intra_bytes(T, H, K, V), state_bytes=state_bytes(T, N, H, K, V),
                kernels=kernels, flops=prefill_flops(T, H, K, V, C), inputs=(c, g, beta))


def kernel_times(t, o, ht, ws, scale, C, steps):
    """Average duration (ms) of each of the step's three kernels, from HIP
    events that kda_chunk_prefill_marked (the gated call with marks) records
    between them on the launch stream, over `steps` back-to-back calls under
    the timed region's conditions (the same inputs, nothing flushed)."""
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    call = lambda m: kda.kda_chunk_prefill_marked(m, t["q"], t["k"], t["v"], t["a"], t["b"],
                                                  t["A_log"], t["dt_bias"], t["cu"], scale,
                                                  h0=t["h0"], chunk=C, o=o, ht=ht, workspace=ws)
    for m in marks[:2]:  # warm-up calls (their events are recorded again below)
        call(m)
    torch.cuda.synchronize()
    for m in marks:
        call(m)
    torch.cuda.synchronize()
    names = ("plan", "intra", "state")
    return {n: sum(m[i].elapsed_time(m[i + 1]) for m in marks) / steps
            for i, n in enumerate(names)}


def bench_decode(steps, warmup):
    w = kda_synth.WORKLOADS["decode_256"]
    c = kda_synth.decode_case(w["B"], w["H"], w["K"], w["V"], w["n_slots"], w["io"],
                              seed=w["seed"], dt_bias_std=w["dt_bias_std"],
                              state_std=w["state_std"])
    a, b = _dev(c["a"]), _dev(c["b"])
    g, beta = kda.kda_gate_prep(a, b, _dev(c["A_log"]), _dev(c["dt_bias"]))
    q, k, v = (_dev(c[x], torch.bfloat16) for x in "qkv")
    pool, idx = _dev(c["pool"]), _dev(c["slot_idx"], torch.int32)
    o = torch.empty_like(v)
    fn = lambda: kda.kda_recurrent_decode(q, k, v, g, beta, w["K"] ** -0.5, pool, idx, o=o)
    ms = _time(fn, max(steps, 20), warmup)
    ms_flushed = _time_flushed(fn)
    B, H, K, V = w["B"], w["H"], w["K"], w["V"]
    nbytes = decode_bytes(B, H, K, V)
    state = 2 * B * H * K * V * 4
    return dict(ms=ms, tokens_per_s=B / (ms * 1e-3), bytes=nbytes,
                gbs=nbytes / (ms * 1e-3) / 1e9, state_gbs=state / (ms * 1e-3) / 1e9,
                ms_flushed=ms_flushed, gbs_flushed=nbytes / (ms_flushed * 1e-3) / 1e9)


def bench_decode_layer(steps, warmup):
    """kda_recurrent_decode_ex on decode_256 with every layer option: gate
    from the raw a and b, in-kernel q/k L2 norm, gated RMSNorm of o."""
    w = kda_synth.WORKLOADS["decode_256"]
    c = kda_synth.decode_case(w["B"], w["H"], w["K"], w["V"], w["n_slots"], w["io"],
                              seed=w["seed"], dt_bias_std=w["dt_bias_std"],
                              state_std=w["state_std"])
    B, H, K, V = w["B"], w["H"], w["K"], w["V"]
    a, b = _dev(c["a"]), _dev(c["b"])
    q, k, v = (_dev(c[x], torch.bfloat16) for x in "qkv")
    pool, idx = _dev(c["pool"]), _dev(c["slot_idx"], torch.int32)
    z = torch.randn((B, H, V), device="cuda").to(torch.bfloat16)
    wn = torch.ones(V, device="cuda")
    o = torch.empty_like(v)
    raw = (_dev(c["A_log"]), _dev(c["dt_bias"]), 0.0)
    fn = lambda: kda.kda_recurrent_decode_ex(q, k, v, a, b, K ** -0.5, pool, idx, raw_gate=raw,
                                             qk_l2norm=True, o_gate=z, o_norm_w=wn, o=o)
    ms = _time(fn, max(steps, 20), warmup)
    nbytes = decode_bytes(B, H, K, V) + B * H * V * 2  # plus the output gate z
    return dict(ms=ms, tokens_per_s=B / (ms * 1e-3), bytes=nbytes,
                gbs=nbytes / (ms * 1e-3) / 1e9)


def bench_replay(steps, warmup, L=16):
    """kda_replay_decode on the decode_256 shapes with a ring of L: cursors
    staggered over the rows (row r at r % L, so 1/L of the rows write their
    checkpoint per call), rings filled by L earlier calls."""
    w = kda_synth.WORKLOADS["decode_256"]
    c = kda_synth.decode_case(w["B"], w["H"], w["K"], w["V"], w["n_slots"], w["io"],
                              seed=w["seed"], dt_bias_std=w["dt_bias_std"],
                              state_std=w["state_std"])
    B, H, K, V = w["B"], w["H"], w["K"], w["V"]
    a, b = _dev(c["a"]), _dev(c["b"])
    g, beta = kda.kda_gate_prep(a, b, _dev(c["A_log"]), _dev(c["dt_bias"]))
    q, k, v = (_dev(c[x], torch.bfloat16) for x in "qkv")
    pool, idx = _dev(c["pool"]), _dev(c["slot_idx"], torch.int32)
    n = w["n_slots"]
    ring_d = torch.zeros((n, H, L, V), device="cuda")
    ring_k = torch.zeros((n, H, L, K), dtype=torch.bfloat16, device="cuda")
    ring_g = torch.zeros((n, H, L, K), device="cuda")
    o = torch.empty_like(v)
    rows = torch.arange(B, device="cuda", dtype=torch.int32)
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    nxt = torch.empty_like(pos)
    for s in range(L):  # row r first writes its checkpoint at call r % L
        force = ((rows % L) == s).to(torch.int32)
        kda.kda_replay_decode(q, k, v, g, beta, K ** -0.5, pool, idx, pos, ring_d, ring_k,
                              ring_g, force_flush=force, o=o, next_write_pos=nxt)
        pos, nxt = nxt, pos
    wp = pos.cpu().numpy()
    fn = lambda: kda.kda_replay_decode(q, k, v, g, beta, K ** -0.5, pool, idx, pos, ring_d,
                                       ring_k, ring_g, o=o, next_write_pos=nxt)
    ms = _time(fn, max(steps, 20), warmup)
    nbytes = replay_bytes(wp, wp == L - 1, H, K, V)
    return dict(ms=ms, tokens_per_s=B / (ms * 1e-3), bytes=nbytes, L=L,
                mean_ring_entries=float(wp.mean()), flush_frac=float((wp == L - 1).mean()),
                gbs=nbytes / (ms * 1e-3) / 1e9)


def bench_verify(steps, warmup):
    w = kda_synth.WORKLOADS["verify_64x8"]
    c = kda_synth.decode_case(w["B"], w["H"], w["K"], w["V"], w["n_slots"], w["io"],
                              seed=w["seed"], dt_bias_std=w["dt_bias_std"],
                              state_std=w["state_std"], Tv=w["Tv"])
    B, Tv, H, K, V = w["B"], w["Tv"], w["H"], w["K"], w["V"]
    a, b = _dev(c["a"]).reshape(B * Tv, H, K), _dev(c["b"]).reshape(B * Tv, H)
    g, beta = kda.kda_gate_prep(a, b, _dev(c["A_log"]), _dev(c["dt_bias"]))
    g, beta = g.reshape(B, Tv, H, K), beta.reshape(B, Tv, H)
    q, k, v = (_dev(c[x], torch.bfloat16) for x in "qkv")
    pool, idx = _dev(c["pool"]), _dev(c["slot_idx"], torch.int32)
    inter = torch.empty((B, Tv, H, K, V), device="cuda")
    o = torch.empty_like(v)
    fn = lambda: kda.kda_verify(q, k, v, g, beta, K ** -0.5, pool, idx, inter_states=inter, o=o)
    ms = _time(fn, max(steps, 20), warmup)
    ms_flushed = _time_flushed(fn)
    nbytes = verify_bytes(B, Tv, H, K, V)
    return dict(ms=ms, tokens_per_s=B * Tv / (ms * 1e-3), bytes=nbytes,
                gbs=nbytes / (ms * 1e-3) / 1e9, ms_flushed=ms_flushed,
                gbs_flushed=nbytes / (ms_flushed * 1e-3) / 1e9)


def bench_long(steps, warmup):
    w = kda_synth.WORKLOADS["long_prefill_65536"]
    c = kda_synth.prefill_case(w["seqlens"], w["H"], w["K"], w["V"], w["io"], seed=w["seed"],
                               dt_bias_std=w["dt_bias_std"], h0_std=w["h0_std"])
    H, K, V, C, nseg = w["H"], w["K"], w["V"], w["chunk"], w["segments"]
    T = c["T"]
    seg = T // nseg
    q, k, v = (_dev(c[x], torch.bfloat16) for x in "qkv")
    g, beta = kda.kda_gate_prep(_dev(c["a"]), _dev(c["b"]), _dev(c["A_log"]),
                                _dev(c["dt_bias"]))
    h0 = _dev(c["h0"])
    state = torch.empty_like(h0)
    o = torch.empty_like(v)
    cu_seg = torch.tensor([0, seg], dtype=torch.int32, device="cuda")
    cu_full = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    ws = torch.empty(kda.kda_chunk_prefill_workspace_size(T, 1, H, K, V, C),
                     dtype=torch.uint8, device="cuda")

    def segmented():
        state.copy_(h0)
        for s in range(nseg):
            sl = slice(s * seg, (s + 1) * seg)
            kda.kda_chunk_prefill(q[sl], k[sl], v[sl], g[sl], beta[sl], cu_seg, K ** -0.5,
                                  h0=state, ht=state, chunk=C, o=o[sl], workspace=ws)

    def full():
        kda.kda_chunk_prefill(q, k, v, g, beta, cu_full, K ** -0.5, h0=h0, ht=state,
                              chunk=C, o=o, workspace=ws)

    n = max(2, steps // 10)
    ms_seg = _time(segmented, n, 1)
    ms_full = _time(full, n, 1)
    return dict(T=T, ms_segmented=ms_seg, ms_full=ms_full,
                tokens_per_s_segmented=T / (ms_seg * 1e-3),
                tokens_per_s_full=T / (ms_full * 1e-3),
                bytes=prefill_bytes(T, 1, H, K, V))


def _event_ms(fn, reps: int = 5) -> float:
    """Median milliseconds of one call of fn, each call between HIP events on
    the current stream (after two untimed calls)."""
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return float(np.median(times))


def measure_ceilings(nbytes: int = 2 << 30):
    """Rates that plain hand-written kernels (libkda_probe) reach on this GPU:
    HBM streams over `nbytes` per buffer in the access patterns of the paths
    (separate read + write, in-place read-modify-write, read only, write
    only), and loops of independent bf16 matrix-core products in the two MFMA
    shapes (32x32x16, and 16x16x32: the shape the prefill kernels use)."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    out = {}
    traffic = {"copy": 2 * nbytes, "rmw": 2 * nbytes, "read": nbytes, "write": nbytes}
    for mode, moved in traffic.items():
        ms = _event_ms(lambda: ceilings.hbm(mode, src if mode in ("copy", "read") else None,
                                            dst, nbytes))
        out[f"hbm_{mode}_gbs"] = moved / (ms * 1e-3) / 1e9
    del src, dst
    blocks, iters = 512, 20000
    res = torch.empty(4 * blocks, dtype=torch.float32, device="cuda")
    for shape in ("32x32x16", "16x16x32"):
        ms = _event_ms(lambda: ceilings.mfma_bf16(shape, blocks, iters, res))
        out[f"bf16_mfma_{shape}_tflops"] = ceilings.mfma_flops(shape, blocks, iters) / (ms * 1e-3) / 1e12
    out["what"] = (f"libkda_probe kernels timed in this run: HBM streams over {nbytes >> 30} GiB "
                   "per buffer (copy and rmw count read + write bytes; one 1024-thread "
                   "workgroup per 16 KiB, non-temporal); 512 workgroups of independent bf16 "
                   "MFMA chains per shape")
    return out


KERNEL_SYMBOL = {"intra": "intra_kernel", "state": "state_kernel"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_varlen_7680_traffic.md")
PREFILL_SOURCE = os.path.join(ROOT, "kda_gated_delta_amd", "csrc", "kda_prefill.hip")


def measured_counters(kernel):
    """The committed rocprofv3 counter record of `kernel` (HBM bytes per
    launch from FETCH_SIZE + WRITE_SIZE scaled by a copy kernel of known
    size; MFMA and VALU busy fractions), or None when there is none or the
    kernel source has changed since the counters were taken."""
    import hashlib

    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
        sha = hashlib.sha256(open(PREFILL_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    for ln in lines:
        if ln.startswith('{"traffic"'):
            rec = json.loads(ln)["traffic"].get(kernel)
            if rec and rec.get("source_sha256") == sha:
                return rec
    return None


def measured_traffic(kernel):
    rec = measured_counters(kernel)
    return None if rec is None else rec["bytes_per_launch"]


def roofline(p):
    """Roofline of the prefill's dominant kernel (the longer of the intra-chunk
    and state kernels by live HIP-event timing).  Its bound is the larger of
    algorithmic bytes / HBM peak and algorithmic flops / bf16 MFMA peak."""
    w, T, N = p["workload"], p["T"], p["N"]
    H, K, V, C = w["H"], w["K"], w["V"], w["chunk"]
    kern = max(("intra", "state"), key=lambda n: p["kernels"][n])
    nbytes = p["intra_bytes"] if kern == "intra" else p["state_bytes"]
    flops = (intra_flops if kern == "intra" else state_flops)(T, H, K, V, C)
    sec = p["kernels"][kern] * 1e-3
    if nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (BF16_MFMA_PEAK_TFLOPS * 1e12):
        bound, achieved, peak, unit = "hbm", nbytes / sec / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", flops / sec / 1e12, BF16_MFMA_PEAK_TFLOPS, "TFLOP/s"
    return {"bound": bound, "kernel": KERNEL_SYMBOL[kern], "achieved": achieved,
            "peak": peak, "unit": unit, "frac": achieved / peak,
            "traffic": measured_traffic(KERNEL_SYMBOL[kern]),
            "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
            "avg_ms": p["kernels"][kern]}


def cpu_baseline(inputs, workload):
    """The fp64 oracle on the whole prefill workload (gate + prefill), on all
    host cores, timed by wall clock."""
    import oracle  # test infrastructure: used only for this reported baseline

    c, _, _ = inputs
    nthreads = os.cpu_count() or 1
    t0 = time.time()
    g, beta = oracle.gate(c["a"], c["b"], c["A_log"], c["dt_bias"])
    oracle.prefill(c["q"], c["k"], c["v"], g.astype(np.float32), beta.astype(np.float32),
                   c["cu"], workload["K"] ** -0.5, c["h0"], nthreads=nthreads)
    dt = time.time() - t0
    # one thread on one head of the same batch: the per-core rate
    sub = lambda x: np.ascontiguousarray(x[:, :1])
    g1, b1 = sub(g).astype(np.float32), sub(beta).astype(np.float32)
    t1 = time.time()
    oracle.prefill(sub(c["q"]), sub(c["k"]), sub(c["v"]), g1, b1, c["cu"], workload["K"] ** -0.5,
                   np.ascontiguousarray(c["h0"][:, :1]), nthreads=1)
    dt1 = time.time() - t1
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return dict(value=c["T"] / dt, unit="tokens/s", cores=nthreads, kind="oracle",
                sample=f"whole varlen prefill batch ({c['T']} tokens x {workload['H']} heads, "
                       f"gate + token-serial fp64 recurrence), {dt:.1f} s wall, CPU: {cpu}",
                single_thread={"value": c["T"] / (dt1 * workload["H"]), "unit": "tokens/s",
                               "sample": f"one head of the same batch on one thread, "
                                         f"{dt1:.2f} s, scaled to {workload['H']} heads"})


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-long", action="store_true", help="skip the 65536-token workload")
    ap.add_argument("--only", choices=["prefill", "decode", "decode_layer", "replay", "verify",
                                       "long", "ceilings"],
                    default=None,
                    help="time a single workload (for profiler runs)")
    ap.add_argument("--settle", type=float, default=0.2,
                    help="seconds of untimed calls before each timed region (0 under a profiler)")
    args = ap.parse_args()
    global SETTLE_S
    SETTLE_S = args.settle
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the recurrence shards by head or request with no communication, "
              "but no multi-GPU path is built)", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    if args.only == "prefill":
        p = bench_prefill(args.steps, args.warmup)
        p.pop("inputs")
        p.pop("workload")
        print(json.dumps(p))
        return
    if args.only == "decode":
        print(json.dumps(bench_decode(args.steps, args.warmup)))
        return
    if args.only == "decode_layer":
        print(json.dumps(bench_decode_layer(args.steps, args.warmup)))
        return
    if args.only == "replay":
        print(json.dumps(bench_replay(args.steps, args.warmup)))
        return
    if args.only == "verify":
        print(json.dumps(bench_verify(args.steps, args.warmup)))
        return
    if args.only == "long":
        print(json.dumps(bench_long(args.steps, args.warmup)))
        return
    if args.only == "ceilings":
        print(json.dumps(measure_ceilings()))
        return

    p = bench_prefill(args.steps, args.warmup)
    w = p["workload"]
    tokens_per_s = p["T"] / (p["ms_step"] * 1e-3)
    achieved = p["prefill_bytes"] / (p["ms_prefill"] * 1e-3) / 1e9
    line = {
        "metric": "KDA prefill tokens/s; decode tokens/s + state HBM GB/s (% of peak), 1 GPU",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": p["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "varlen_prefill_7680: 4 packed sequences {512,1024,2048,4096}, "
                               "H=32, K=V=128, chunk 64, gate + prefill per step "
                               "(kda_chunk_prefill_gated)",
                   "global_batch": p["N"], "seq_len": p["T"], "parallelism": "none"},
        "roofline": roofline(p),
        "prefill": {"ms": p["ms_prefill"], "ms_gate": p["ms_gate"],
                    "ms_step_gate_prep_then_prefill": p["ms_step_two_calls"],
                    "kernel_ms": p["kernels"],
                    "tokens_per_s": p["T"] / (p["ms_prefill"] * 1e-3),
                    "algorithmic_bytes": p["prefill_bytes"],
                    "gbs": achieved, "frac_of_hbm_peak": achieved / HBM_PEAK_GBS,
                    "algorithmic_flops": p["flops"],
                    "tflops": p["flops"] / (p["ms_prefill"] * 1e-3) / 1e12,
                    "mfma_frac_of_bf16_peak": p["flops"] / (p["ms_prefill"] * 1e-3) / 1e12
                    / BF16_MFMA_PEAK_TFLOPS,
                    "gate_gbs": p["gate_bytes"] / (p["ms_gate"] * 1e-3) / 1e9,
                    "with_snapshots_every_256": {
                        "ms": p["ms_snapshots"],
                        "snapshot_bytes": p["snapshot_bytes"],
                        "gbs": (p["prefill_bytes"] + p["snapshot_bytes"])
                        / (p["ms_snapshots"] * 1e-3) / 1e9},
                    "counters": {n: ({x: r[x] for x in ("mfma_busy", "valu_busy") if x in r}
                                     if (r := measured_counters(n)) else None)
                                 for n in ("intra_kernel", "state_kernel")}},
    }
    _fresh_memory()
    d = bench_decode(args.steps, args.warmup)
    line["decode"] = {"workload": "decode_256: 256 requests, 512-slot fp32 pool, H=32, K=V=128",
                      "timing": "median of single calls, each after a 512 MiB write and read "
                                "that empty the last-level cache",
                      "tokens_per_s": 256 / (d["ms_flushed"] * 1e-3), "ms": d["ms_flushed"],
                      "state_gbs": d["state_gbs"] * d["ms"] / d["ms_flushed"],
                      "total_gbs": d["gbs_flushed"],
                      "frac_of_hbm_peak": d["gbs_flushed"] / HBM_PEAK_GBS,
                      "back_to_back": {"ms": d["ms"], "tokens_per_s": d["tokens_per_s"],
                                       "total_gbs": d["gbs"]}}
    _fresh_memory()
    dl = bench_decode_layer(args.steps, args.warmup)
    line["decode"]["with_layer_options"] = {
        "what": "raw gate in the kernel, q/k L2 norm, gated RMSNorm of o (kda_recurrent_decode_ex)",
        "ms": dl["ms"], "tokens_per_s": dl["tokens_per_s"], "total_gbs": dl["gbs"],
        "frac_of_hbm_peak": dl["gbs"] / HBM_PEAK_GBS}
    _fresh_memory()
    rp = bench_replay(args.steps, args.warmup)
    line["replay_decode"] = {"workload": "decode_256 with a 16-entry ring per slot, cursors "
                                         "staggered over the rows (kda_replay_decode)",
                             "tokens_per_s": rp["tokens_per_s"], "ms": rp["ms"],
                             "algorithmic_bytes": rp["bytes"], "total_gbs": rp["gbs"],
                             "frac_of_hbm_peak": rp["gbs"] / HBM_PEAK_GBS,
                             "mean_ring_entries": rp["mean_ring_entries"],
                             "flush_frac": rp["flush_frac"],
                             "speedup_vs_decode": d["ms"] / rp["ms"]}
    _fresh_memory()
    vr = bench_verify(args.steps, args.warmup)
    line["verify"] = {"workload": "verify_64x8: 64 requests x 8 draft tokens, 128-slot pool",
                      "timing": "median of single calls, each after a 512 MiB write and read "
                                "that empty the last-level cache (the 134 MB of pool a call "
                                "reads would otherwise stay cached between calls)",
                      "tokens_per_s": 512 / (vr["ms_flushed"] * 1e-3), "ms": vr["ms_flushed"],
                      "total_gbs": vr["gbs_flushed"],
                      "frac_of_hbm_peak": vr["gbs_flushed"] / HBM_PEAK_GBS,
                      "back_to_back": {"ms": vr["ms"], "tokens_per_s": vr["tokens_per_s"],
                                       "total_gbs": vr["gbs"]}}
    if not args.no_long:
        _fresh_memory()
        lg = bench_long(args.steps, args.warmup)
        line["long"] = {"workload": "long_prefill_65536: 16 carried 4096-token segments "
                                    "and one full run",
                        "tokens_per_s_segmented": lg["tokens_per_s_segmented"],
                        "tokens_per_s_full": lg["tokens_per_s_full"],
                        "ms_segmented": lg["ms_segmented"], "ms_full": lg["ms_full"]}
    _fresh_memory()
    cl = measure_ceilings()
    line["measured_ceilings"] = cl
    # each path against the measured stream of its access pattern: the decode
    # pool update is an in-place read-modify-write; verify, the buffered
    # decode and the prefill kernels read some buffers and write others
    line["roofline"]["frac_of_measured"] = line["roofline"]["achieved"] / (
        cl["hbm_copy_gbs"] if line["roofline"]["unit"] == "GB/s" else cl["bf16_mfma_32x32x16_tflops"])
    line["prefill"]["frac_of_measured_copy"] = achieved / cl["hbm_copy_gbs"]
    line["decode"]["frac_of_measured_rmw"] = d["gbs_flushed"] / cl["hbm_rmw_gbs"]
    line["replay_decode"]["frac_of_measured_copy"] = rp["gbs"] / cl["hbm_copy_gbs"]
    line["verify"]["frac_of_measured_copy"] = vr["gbs_flushed"] / cl["hbm_copy_gbs"]
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(p["inputs"], w)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
