"""Benchmark of the KDA hot path on one MI355X.

One step = gate activation + chunkwise prefill of one 65536-token sequence
(H=32, K=V=128, bf16 q/k/v, fp32 raw gate inputs and states, chunk 64: the
long-context workload, the largest of the five), inputs resident in HBM, as
one kda_chunk_prefill_gated call (the gate evaluated inside the prefill).
``value`` is prefill tokens/s of that step.  Every prefill workload is timed
as K single calls, each after a 512 MiB write and read that empty the 256 MB
last-level cache, between HIP events on the library's stream; the median is
the figure, the minimum and mean are reported beside it, and the per-kernel
durations come from events the same calls record between their kernels.
The same run also measures, each on its own workload:
  varlen  - the packed batch {512, 1024, 2048, 4096}, same shapes;
  share   - the 65536-token sequence at H = 4 (one GPU's heads under an
            8-way head split of H = 32);
  carried - the 65536-token sequence as 16 carried 4096-token calls;
  decode  - 256 single-token requests on a 512-slot fp32 state pool
            (tokens/s and state GB/s against HBM peak);
  verify  - 64 requests x 8 draft tokens on a 128-slot pool;
  replay  - the buffered decode on the decode shapes;
and the fp64 CPU oracle on bounded samples of the prefill, decode and verify
workloads (``cpu_baseline``).  Prints one JSON line.
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


def _time_rotating(fns, steps: int, warmup: int) -> float:
    """Mean milliseconds per call of a steady stream of calls that cycles
    over `fns`, one callable per private copy of a workload's buffers, the
    copies together several times larger than the last-level cache: each call
    finds none of its inputs cached (the calls in between moved far more
    bytes than the cache holds), and each call's write-backs of dirty lines
    fall inside the timed stream (in the next call) instead of after it, as
    they would after a single timed call with write-back stores."""
    n = len(fns)
    for i in range(max(warmup, n)):
        fns[i % n]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < SETTLE_S:  # clocks up from idle
        fns[i % n]()
        i += 1
        torch.cuda.synchronize()
    steps = max(steps, 4 * n)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for j in range(steps):
        fns[(i + j) % n]()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


ROTATE_SETS = 4  # private buffer copies per decode-family workload


# ------------------------------------------------------------ byte models

_FLUSH = None


def _time_flushed(fn, reps: int = 20) -> float:
    """Median milliseconds of single calls of fn, each timed alone between
    HIP events after a write and then a read of a 512 MiB scratch buffer
    (twice the 256 MB last-level cache): no input of fn is served from that
    cache, and the read leaves no dirty lines whose write-back would fall in
    the timed call."""
    fn()
    times = []
    for _ in range(reps):
        _flush()
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

def prefill_setup(name, seqlens=None, H=None):
    w = dict(kda_synth.WORKLOADS[name])
    if seqlens is not None:
        w["seqlens"] = seqlens
    if H is not None:
        w["H"] = H
    c = kda_synth.prefill_case(w["seqlens"], w["H"], w["K"], w["V"], w["io"], seed=w["seed"],
                               dt_bias_std=w["dt_bias_std"], h0_std=w["h0_std"])
    io = torch.bfloat16 if w["io"] == "bf16" else torch.float32
    t = dict(q=_dev(c["q"], io), k=_dev(c["k"], io), v=_dev(c["v"], io), a=_dev(c["a"]),
             b=_dev(c["b"]), A_log=_dev(c["A_log"]), dt_bias=_dev(c["dt_bias"]),
             cu=_dev(c["cu"], torch.int32), h0=_dev(c["h0"]))
    return w, c, t


def _flush():
    global _FLUSH
    if _FLUSH is None:
        _FLUSH = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
    _FLUSH.fill_(1.0)
    _FLUSH.sum()


def time_steps(step, steps, warmup, nmarks=0):
    """K single calls of step(marks), each after emptying the last-level
    cache, each between HIP events on the current stream (the library's
    stream).  Returns (list of per-call ms, list of per-call lists of ms
    between consecutive marks)."""
    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(nmarks)]
    for _ in range(warmup):
        step(mk() if nmarks else None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_S:  # clocks up from idle
        step(mk() if nmarks else None)
        torch.cuda.synchronize()
    calls, parts = [], []
    for _ in range(steps):
        _flush()
        m = mk() if nmarks else None
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step(m)
        e1.record()
        torch.cuda.synchronize()
        calls.append(e0.elapsed_time(e1))
        if nmarks:
            parts.append([m[i].elapsed_time(m[i + 1]) for i in range(nmarks - 1)])
    return calls, parts


def _stats(ms):
    return dict(ms_median=float(np.median(ms)), ms_min=float(np.min(ms)),
                ms_mean=float(np.mean(ms)), reps=len(ms))


def bench_prefill_workload(name, steps, warmup, seqlens=None, H=None, keep_inputs=False):
    """Gate + prefill as K cache-cold single calls of kda_chunk_prefill_gated
    (the step: with long chains the library overlaps the intra-chunk kernel
    of one wave of chunks with the state pass of the previous one, on a
    second stream).  The per-stage durations come from a further set of
    cache-cold calls of kda_chunk_prefill_marked, which runs the same kernels
    with the same plan on the caller's stream alone, stage after stage, with
    events between the stages."""
    w, c, t = prefill_setup(name, seqlens, H)
    T, N, H, K, V, C = c["T"], c["N"], w["H"], w["K"], w["V"], w["chunk"]
    scale = K ** -0.5
    o = torch.empty_like(t["v"])
    ht = torch.empty_like(t["h0"])
    ws = torch.empty(kda.kda_chunk_prefill_workspace_size(T, N, H, K, V, C),
                     dtype=torch.uint8, device="cuda")
    args = (t["q"], t["k"], t["v"], t["a"], t["b"], t["A_log"], t["dt_bias"], t["cu"], scale)
    kw = dict(h0=t["h0"], chunk=C, o=o, ht=ht, workspace=ws)

    def step(_):
        kda.kda_chunk_prefill_gated(*args, **kw)

    def marked(marks):
        kda.kda_chunk_prefill_marked(marks, *args, **kw)

    calls, _ = time_steps(step, steps, warmup)
    single, parts = time_steps(marked, max(10, steps // 2), 2, nmarks=4)
    names = ("plan", "intra", "state")
    kernel_ms = {n: float(np.mean([p[i] for p in parts])) for i, n in enumerate(names)}
    r = dict(workload=w, T=T, N=N, H=H, **_stats(calls), kernel_ms=kernel_ms,
             single_stream_ms=float(np.median(single)),
             prefill_bytes=prefill_bytes(T, N, H, K, V), intra_bytes=intra_bytes(T, H, K, V),
             state_bytes=state_bytes(T, N, H, K, V), flops=prefill_flops(T, H, K, V, C))
    r["tokens_per_s"] = T / (r["ms_median"] * 1e-3)
    if keep_inputs:
        r["inputs"] = c
    del t, o, ht, ws
    return r


def bench_carried(steps, warmup):
    """The 65536-token sequence as 16 consecutive 4096-token calls, each
    starting from the previous call's final state (in place), cache-cold."""
    w, c, t = prefill_setup("long_prefill_65536")
    H, K, V, C, nseg = w["H"], w["K"], w["V"], w["chunk"], w["segments"]
    T = c["T"]
    seg = T // nseg
    state = torch.empty_like(t["h0"])
    o = torch.empty_like(t["v"])
    cu_seg = torch.tensor([0, seg], dtype=torch.int32, device="cuda")
    ws = torch.empty(kda.kda_chunk_prefill_workspace_size(seg, 1, H, K, V, C),
                     dtype=torch.uint8, device="cuda")

    def step(_):
        state.copy_(t["h0"])
        for s in range(nseg):
            sl = slice(s * seg, (s + 1) * seg)
            kda.kda_chunk_prefill_gated(t["q"][sl], t["k"][sl], t["v"][sl], t["a"][sl],
                                        t["b"][sl], t["A_log"], t["dt_bias"], cu_seg, K ** -0.5,
                                        h0=state, ht=state, chunk=C, o=o[sl], workspace=ws)

    calls, _ = time_steps(step, max(steps // 5, 10), warmup)
    r = dict(T=T, **_stats(calls))
    r["tokens_per_s"] = T / (r["ms_median"] * 1e-3)
    return r


def bench_gate_and_snapshots(steps, warmup):
    """On the varlen batch: kda_gate_prep alone, the two-call sequence (gate
    prep then kda_chunk_prefill), and the prefill with a snapshot every 256
    tokens, cache-cold single calls."""
    w, c, t = prefill_setup("varlen_prefill_7680")
    T, N, H, K, V, C = c["T"], c["N"], w["H"], w["K"], w["V"], w["chunk"]
    scale = K ** -0.5
    g = torch.empty_like(t["a"])
    beta = torch.empty_like(t["b"])
    o = torch.empty_like(t["v"])
    ht = torch.empty_like(t["h0"])
    ws = torch.empty(kda.kda_chunk_prefill_workspace_size(T, N, H, K, V, C),
                     dtype=torch.uint8, device="cuda")
    snaps = torch.empty((T // 256, H, K, V), device="cuda")
    gate = lambda _: kda.kda_gate_prep(t["a"], t["b"], t["A_log"], t["dt_bias"], g=g, beta=beta)

    def two_calls(_):
        gate(None)
        kda.kda_chunk_prefill(t["q"], t["k"], t["v"], g, beta, t["cu"], scale, h0=t["h0"],
                              chunk=C, o=o, ht=ht, workspace=ws)

    def with_snaps(_):
        kda.kda_chunk_prefill_snapshots(t["q"], t["k"], t["v"], g, beta, t["cu"], scale, 256,
                                        h0=t["h0"], chunk=C, o=o, ht=ht, snapshots=snaps,
                                        workspace=ws)

    n_snaps = sum(int(c["cu"][i + 1] - c["cu"][i]) // 256 for i in range(N))
    ms_gate = float(np.median(time_steps(gate, steps, warmup)[0]))
    ms_two = float(np.median(time_steps(two_calls, steps, warmup)[0]))
    ms_snap = float(np.median(time_steps(with_snaps, steps, warmup)[0]))
    return dict(ms_gate=ms_gate, gate_gbs=gate_bytes(T, H, K) / (ms_gate * 1e-3) / 1e9,
                ms_gate_prep_then_prefill=ms_two, ms_with_snapshots_every_256=ms_snap,
                snapshot_bytes=n_snaps * H * K * V * 4)


def bench_decode(steps, warmup):
    """kda_recurrent_decode on decode_256: `ms` over a steady stream of calls
    rotating over ROTATE_SETS private copies of the buffers (cold inputs,
    write-backs paid); `ms_flushed` the median of single calls after emptying
    the cache; `ms_b2b` the same buffers back to back."""
    w = kda_synth.WORKLOADS["decode_256"]
    c = kda_synth.decode_case(w["B"], w["H"], w["K"], w["V"], w["n_slots"], w["io"],
                              seed=w["seed"], dt_bias_std=w["dt_bias_std"],
                              state_std=w["state_std"])
    B, H, K, V = w["B"], w["H"], w["K"], w["V"]

    def make(_):
        a, b = _dev(c["a"]), _dev(c["b"])
        g, beta = kda.kda_gate_prep(a, b, _dev(c["A_log"]), _dev(c["dt_bias"]))
        q, k, v = (_dev(c[x], torch.bfloat16) for x in "qkv")
        pool, idx = _dev(c["pool"]), _dev(c["slot_idx"], torch.int32)
        o = torch.empty_like(v)
        return lambda: kda.kda_recurrent_decode(q, k, v, g, beta, K ** -0.5, pool, idx, o=o)

    fns = [make(i) for i in range(ROTATE_SETS)]
    ms = _time_rotating(fns, steps, warmup)
    ms_flushed = _time_flushed(fns[0])
    ms_b2b = _time(fns[0], max(steps, 20), warmup)
    nbytes = decode_bytes(B, H, K, V)
    state = 2 * B * H * K * V * 4
    del fns
    return dict(ms=ms, tokens_per_s=B / (ms * 1e-3), bytes=nbytes,
                gbs=nbytes / (ms * 1e-3) / 1e9, state_gbs=state / (ms * 1e-3) / 1e9,
                ms_flushed=ms_flushed, gbs_flushed=nbytes / (ms_flushed * 1e-3) / 1e9,
                ms_b2b=ms_b2b, gbs_b2b=nbytes / (ms_b2b * 1e-3) / 1e9)


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
    checkpoint per call), rings filled by L earlier calls.  Timed as
    bench_decode (rotating copies, cache-cold single calls, back to back)."""
    w = kda_synth.WORKLOADS["decode_256"]
    c = kda_synth.decode_case(w["B"], w["H"], w["K"], w["V"], w["n_slots"], w["io"],
                              seed=w["seed"], dt_bias_std=w["dt_bias_std"],
                              state_std=w["state_std"])
    B, H, K, V = w["B"], w["H"], w["K"], w["V"]
    n = w["n_slots"]
    wps = []

    def make(_):
        a, b = _dev(c["a"]), _dev(c["b"])
        g, beta = kda.kda_gate_prep(a, b, _dev(c["A_log"]), _dev(c["dt_bias"]))
        q, k, v = (_dev(c[x], torch.bfloat16) for x in "qkv")
        pool, idx = _dev(c["pool"]), _dev(c["slot_idx"], torch.int32)
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
        wps.append(pos.cpu().numpy())
        return lambda: kda.kda_replay_decode(q, k, v, g, beta, K ** -0.5, pool, idx, pos, ring_d,
                                             ring_k, ring_g, o=o, next_write_pos=nxt)

    fns = [make(i) for i in range(ROTATE_SETS)]
    ms = _time_rotating(fns, steps, warmup)
    ms_flushed = _time_flushed(fns[0])
    ms_b2b = _time(fns[0], max(steps, 20), warmup)
    wp = wps[0]
    nbytes = replay_bytes(wp, wp == L - 1, H, K, V)
    del fns
    return dict(ms=ms, tokens_per_s=B / (ms * 1e-3), bytes=nbytes, L=L,
                mean_ring_entries=float(wp.mean()), flush_frac=float((wp == L - 1).mean()),
                gbs=nbytes / (ms * 1e-3) / 1e9, ms_flushed=ms_flushed,
                gbs_flushed=nbytes / (ms_flushed * 1e-3) / 1e9, ms_b2b=ms_b2b,
                gbs_b2b=nbytes / (ms_b2b * 1e-3) / 1e9)


def bench_verify(steps, warmup):
    """kda_verify on verify_64x8, timed as bench_decode."""
    w = kda_synth.WORKLOADS["verify_64x8"]
    c = kda_synth.decode_case(w["B"], w["H"], w["K"], w["V"], w["n_slots"], w["io"],
                              seed=w["seed"], dt_bias_std=w["dt_bias_std"],
                              state_std=w["state_std"], Tv=w["Tv"])
    B, Tv, H, K, V = w["B"], w["Tv"], w["H"], w["K"], w["V"]

    def make(_):
        a, b = _dev(c["a"]).reshape(B * Tv, H, K), _dev(c["b"]).reshape(B * Tv, H)
        g, beta = kda.kda_gate_prep(a, b, _dev(c["A_log"]), _dev(c["dt_bias"]))
        g, beta = g.reshape(B, Tv, H, K), beta.reshape(B, Tv, H)
        q, k, v = (_dev(c[x], torch.bfloat16) for x in "qkv")
        pool, idx = _dev(c["pool"]), _dev(c["slot_idx"], torch.int32)
        inter = torch.empty((B, Tv, H, K, V), device="cuda")
        o = torch.empty_like(v)
        return lambda: kda.kda_verify(q, k, v, g, beta, K ** -0.5, pool, idx, inter_states=inter,
                                      o=o)

    fns = [make(i) for i in range(ROTATE_SETS)]
    ms = _time_rotating(fns, steps, warmup)
    ms_flushed = _time_flushed(fns[0])
    ms_b2b = _time(fns[0], max(steps, 20), warmup)
    nbytes = verify_bytes(B, Tv, H, K, V)
    del fns
    return dict(ms=ms, tokens_per_s=B * Tv / (ms * 1e-3), bytes=nbytes,
                gbs=nbytes / (ms * 1e-3) / 1e9, ms_flushed=ms_flushed,
                gbs_flushed=nbytes / (ms_flushed * 1e-3) / 1e9, ms_b2b=ms_b2b,
                gbs_b2b=nbytes / (ms_b2b * 1e-3) / 1e9)


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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_long_65536_traffic.md")
PREFILL_SOURCE = os.path.join(ROOT, "kda_gated_delta_amd", "csrc", "kda_prefill.hip")


def _sha256(path):
    import hashlib

    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def measured_counters(kernel):
    """The committed rocprofv3 counter record of `kernel` on the headline
    workload (HBM bytes per call from FETCH_SIZE + WRITE_SIZE scaled by a
    copy kernel of known size; MFMA and VALU busy fractions), with the file
    it comes from and that file's hash; None when there is none or the
    kernel source has changed since the counters were taken."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
        sha = _sha256(PREFILL_SOURCE)
        file_sha = _sha256(TRAFFIC_FILE)
    except OSError:
        return None
    for ln in lines:
        if ln.startswith('{"traffic"'):
            rec = json.loads(ln)["traffic"].get(kernel)
            if rec and rec.get("source_sha256") == sha:
                return dict(rec, copied_from=os.path.relpath(TRAFFIC_FILE, ROOT),
                            copied_from_sha256=file_sha)
    return None


def roofline(r):
    """Roofline of the prefill's dominant stage (the longer of the intra-chunk
    kernel and the state pass by the live HIP-event timing of the timed
    calls).  Its bound is the larger of algorithmic bytes / HBM peak and
    algorithmic flops / bf16 MFMA peak; achieved = those algorithmic bytes
    (or flops) / the stage's mean duration per call."""
    w, T, N, H = r["workload"], r["T"], r["N"], r["H"]
    K, V, C = w["K"], w["V"], w["chunk"]
    sched = kda.kda_chunk_prefill_schedule(T, N, H, K, V, C)
    launches = {"intra": max(1, sched["intra_launches"]), "state": max(1, sched["state_launches"])}
    kern = max(("intra", "state"), key=lambda n: r["kernel_ms"][n])
    nbytes = r["intra_bytes"] if kern == "intra" else r["state_bytes"]
    flops = (intra_flops if kern == "intra" else state_flops)(T, H, K, V, C)
    sec = r["kernel_ms"][kern] * 1e-3
    if nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (BF16_MFMA_PEAK_TFLOPS * 1e12):
        bound, achieved, peak, unit = "hbm", nbytes / sec / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", flops / sec / 1e12, BF16_MFMA_PEAK_TFLOPS, "TFLOP/s"
    ctr = measured_counters(KERNEL_SYMBOL[kern])
    out = {"bound": bound, "kernel": KERNEL_SYMBOL[kern], "achieved": achieved,
           "peak": peak, "unit": unit, "frac": achieved / peak,
           "traffic": None if ctr is None else ctr["bytes_per_launch"],
           "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
           "stage_ms": r["kernel_ms"][kern], "launches": launches[kern],
           "avg_ms": r["kernel_ms"][kern] / launches[kern],
           "algorithmic_bytes_per_launch": nbytes / launches[kern],
           "schedule": sched}
    if ctr is not None:
        out["traffic_source"] = {"copied_from": ctr["copied_from"],
                                 "file_sha256": ctr["copied_from_sha256"],
                                 "kernel_source_sha256": ctr["source_sha256"]}
    # the other stage, by the same rule, for reference
    other = "state" if kern == "intra" else "intra"
    ob = r["intra_bytes"] if other == "intra" else r["state_bytes"]
    of = (intra_flops if other == "intra" else state_flops)(T, H, K, V, C)
    osec = r["kernel_ms"][other] * 1e-3
    out["other_stage"] = {"kernel": KERNEL_SYMBOL[other], "avg_ms": r["kernel_ms"][other],
                          "hbm_frac": ob / osec / 1e9 / HBM_PEAK_GBS,
                          "mfma_frac": of / osec / 1e12 / BF16_MFMA_PEAK_TFLOPS}
    return out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baselines(long_inputs, workload):
    """The fp64 oracle, as it stands, on bounded samples of the workloads, on
    all host cores (one thread per (sequence or request, head)), by wall
    clock: the 65536-token sequence on 16 of its 32 heads (gate +
    recurrence; tokens/s scaled to 32 heads), the varlen batch whole, the
    decode and verify workloads whole.  Each also gets a single-thread rate,
    from a smaller slice on one thread scaled to the whole workload."""
    import oracle  # test infrastructure: used only for these reported baselines

    nthreads = os.cpu_count() or 1
    cpu = _cpu_model()
    out = {}
    c = long_inputs
    Hs = 16
    sub = lambda x: np.ascontiguousarray(x[:, :Hs])
    t0 = time.time()
    g, beta = oracle.gate(sub(c["a"]), sub(c["b"]), c["A_log"][:Hs], c["dt_bias"][:Hs])
    oracle.prefill(sub(c["q"]), sub(c["k"]), sub(c["v"]), g.astype(np.float32),
                   beta.astype(np.float32), c["cu"], workload["K"] ** -0.5,
                   np.ascontiguousarray(c["h0"][:, :Hs]), nthreads=nthreads)
    dt = time.time() - t0
    H = workload["H"]
    out["long_prefill_65536"] = dict(
        value=c["T"] / (dt * H / Hs), unit="tokens/s", cores=nthreads, kind="oracle",
        sample=f"the 65536-token sequence on {Hs} of its {H} heads (gate + token-serial fp64 "
               f"recurrence), {dt:.1f} s wall, scaled to {H} heads; CPU: {cpu}")
    # one thread: head 0, the first quarter of the sequence
    Tq = c["T"] // 4
    one = lambda x: np.ascontiguousarray(x[:Tq, :1])
    t0 = time.time()
    g1, b1 = oracle.gate(one(c["a"]), one(c["b"]), c["A_log"][:1], c["dt_bias"][:1])
    oracle.prefill(one(c["q"]), one(c["k"]), one(c["v"]), g1.astype(np.float32),
                   b1.astype(np.float32), np.array([0, Tq]), workload["K"] ** -0.5,
                   np.ascontiguousarray(c["h0"][:, :1]), nthreads=1)
    dt1 = time.time() - t0
    out["long_prefill_65536"]["single_thread"] = dict(
        value=Tq / (dt1 * H), unit="tokens/s",
        sample=f"head 0 on its first {Tq} tokens on one thread, {dt1:.2f} s, scaled to {H} heads")
    del g, beta
    # varlen batch, whole
    _, cv, _ = prefill_setup("varlen_prefill_7680")
    t0 = time.time()
    g, beta = oracle.gate(cv["a"], cv["b"], cv["A_log"], cv["dt_bias"])
    oracle.prefill(cv["q"], cv["k"], cv["v"], g.astype(np.float32), beta.astype(np.float32),
                   cv["cu"], 128 ** -0.5, cv["h0"], nthreads=nthreads)
    dt = time.time() - t0
    out["varlen_prefill_7680"] = dict(value=cv["T"] / dt, unit="tokens/s", cores=nthreads,
                                      kind="oracle", sample=f"the whole batch, {dt:.2f} s wall")
    Hv = cv["q"].shape[1]
    one = lambda x: np.ascontiguousarray(x[:, :1])
    t0 = time.time()
    g1, b1 = oracle.gate(one(cv["a"]), one(cv["b"]), cv["A_log"][:1], cv["dt_bias"][:1])
    oracle.prefill(one(cv["q"]), one(cv["k"]), one(cv["v"]), g1.astype(np.float32),
                   b1.astype(np.float32), cv["cu"], 128 ** -0.5,
                   np.ascontiguousarray(cv["h0"][:, :1]), nthreads=1)
    dt1 = time.time() - t0
    out["varlen_prefill_7680"]["single_thread"] = dict(
        value=cv["T"] / (dt1 * Hv), unit="tokens/s",
        sample=f"head 0 of the batch on one thread, {dt1:.2f} s, scaled to {Hv} heads")
    # decode and verify workloads, whole
    wd = kda_synth.WORKLOADS["decode_256"]
    cd = kda_synth.decode_case(wd["B"], wd["H"], wd["K"], wd["V"], wd["n_slots"], wd["io"],
                               seed=wd["seed"], dt_bias_std=wd["dt_bias_std"],
                               state_std=wd["state_std"])
    gd, bd = oracle.gate(cd["a"], cd["b"], cd["A_log"], cd["dt_bias"])
    pool = cd["pool"].copy()
    t0 = time.time()
    oracle.decode(cd["q"], cd["k"], cd["v"], gd.astype(np.float32), bd.astype(np.float32),
                  wd["K"] ** -0.5, pool, cd["slot_idx"], nthreads=nthreads)
    dt = time.time() - t0
    out["decode_256"] = dict(value=wd["B"] / dt, unit="tokens/s", cores=nthreads, kind="oracle",
                             sample=f"one decode call of the workload, {dt:.3f} s wall")
    # (the single-thread samples take a pool of just their own slots: the
    # oracle converts the whole pool it is given, a cost per call, not per
    # request)
    Bs = 16
    pool_s = np.ascontiguousarray(cd["pool"][cd["slot_idx"][:Bs]])
    t0 = time.time()
    oracle.decode(cd["q"][:Bs], cd["k"][:Bs], cd["v"][:Bs], gd[:Bs].astype(np.float32),
                  bd[:Bs].astype(np.float32), wd["K"] ** -0.5, pool_s,
                  np.arange(Bs, dtype=np.int32), nthreads=1)
    dt1 = time.time() - t0
    out["decode_256"]["single_thread"] = dict(
        value=Bs / dt1, unit="tokens/s",
        sample=f"{Bs} of the {wd['B']} requests on one thread, {dt1:.3f} s")
    wv = kda_synth.WORKLOADS["verify_64x8"]
    cvv = kda_synth.decode_case(wv["B"], wv["H"], wv["K"], wv["V"], wv["n_slots"], wv["io"],
                                seed=wv["seed"], dt_bias_std=wv["dt_bias_std"],
                                state_std=wv["state_std"], Tv=wv["Tv"])
    B, Tv = wv["B"], wv["Tv"]
    gv, bv = oracle.gate(cvv["a"].reshape(B * Tv, wv["H"], wv["K"]),
                         cvv["b"].reshape(B * Tv, wv["H"]), cvv["A_log"], cvv["dt_bias"])
    t0 = time.time()
    oracle.verify(cvv["q"], cvv["k"], cvv["v"],
                  gv.astype(np.float32).reshape(B, Tv, wv["H"], wv["K"]),
                  bv.astype(np.float32).reshape(B, Tv, wv["H"]), wv["K"] ** -0.5, cvv["pool"],
                  cvv["slot_idx"], nthreads=nthreads)
    dt = time.time() - t0
    out["verify_64x8"] = dict(value=B * Tv / dt, unit="tokens/s", cores=nthreads, kind="oracle",
                              sample=f"one verify call of the workload, {dt:.3f} s wall")
    Bs = 8
    pool_s = np.ascontiguousarray(cvv["pool"][cvv["slot_idx"][:Bs]])
    t0 = time.time()
    oracle.verify(cvv["q"][:Bs], cvv["k"][:Bs], cvv["v"][:Bs],
                  gv.astype(np.float32).reshape(B, Tv, wv["H"], wv["K"])[:Bs],
                  bv.astype(np.float32).reshape(B, Tv, wv["H"])[:Bs], wv["K"] ** -0.5,
                  pool_s, np.arange(Bs, dtype=np.int32), nthreads=1)
    dt1 = time.time() - t0
    out["verify_64x8"]["single_thread"] = dict(
        value=Bs * Tv / dt1, unit="tokens/s",
        sample=f"{Bs} of the {B} requests on one thread, {dt1:.3f} s")
    head = dict(out["long_prefill_65536"])
    head["others"] = {k: v for k, v in out.items() if k != "long_prefill_65536"}
    return head


def _prefill_entry(r, what):
    w = r["workload"]
    out = {"workload": what, "tokens_per_s": r["tokens_per_s"], "ms": r["ms_median"],
           "ms_min": r["ms_min"], "ms_mean": r["ms_mean"], "reps": r["reps"],
           "kernel_ms": r["kernel_ms"], "single_stream_ms": r["single_stream_ms"],
           "kernel_ms_from": "kda_chunk_prefill_marked: the same kernels on one stream, "
                             "stage after stage, events between the stages",
           "algorithmic_bytes": r["prefill_bytes"],
           "gbs": r["prefill_bytes"] / (r["ms_median"] * 1e-3) / 1e9,
           "algorithmic_flops": r["flops"],
           "tflops": r["flops"] / (r["ms_median"] * 1e-3) / 1e12}
    out["frac_of_hbm_peak"] = out["gbs"] / HBM_PEAK_GBS
    out["roofline"] = roofline(r)
    del w
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--only", choices=["prefill", "varlen", "share", "carried", "decode",
                                       "decode_layer", "replay", "verify", "ceilings"],
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

    only = {
        "prefill": lambda: bench_prefill_workload("long_prefill_65536", args.steps, args.warmup),
        "varlen": lambda: bench_prefill_workload("varlen_prefill_7680", args.steps, args.warmup),
        "share": lambda: bench_prefill_workload("long_prefill_65536", args.steps, args.warmup,
                                                H=4),
        "carried": lambda: bench_carried(args.steps, args.warmup),
        "decode": lambda: bench_decode(args.steps, args.warmup),
        "decode_layer": lambda: bench_decode_layer(args.steps, args.warmup),
        "replay": lambda: bench_replay(args.steps, args.warmup),
        "verify": lambda: bench_verify(args.steps, args.warmup),
        "ceilings": measure_ceilings,
    }
    if args.only is not None:
        # one plain copy of known size first (64 Mi fp32 elements: 256 MiB
        # read, 256 MiB written), against which profiler byte counters of
        # the same run are scaled
        x = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        torch.neg(x)
        torch.cuda.synchronize()
        del x
        r = only[args.only]()
        if isinstance(r, dict):
            r.pop("workload", None)
        print(json.dumps(r))
        return

    lp = bench_prefill_workload("long_prefill_65536", args.steps, args.warmup,
                                keep_inputs=not args.no_cpu)
    long_inputs = lp.pop("inputs", None)
    line = {
        "metric": "KDA prefill tokens/s; decode tokens/s + state HBM GB/s (% of peak), 1 GPU",
        "value": lp["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": lp["ms_median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "long_prefill_65536: one 65536-token sequence, H=32, K=V=128, "
                               "chunk 64, gate + prefill per step (kda_chunk_prefill_gated)",
                   "global_batch": 1, "seq_len": lp["T"], "parallelism": "none",
                   "timing": "median of K single calls, each after a 512 MiB write and read "
                             "that empty the last-level cache"},
        "roofline": roofline(lp),
        "prefill": _prefill_entry(lp, "long_prefill_65536 (the step)"),
    }
    line["prefill_share"] = _prefill_entry(
        bench_prefill_workload("long_prefill_65536", args.steps, args.warmup, H=4),
        "one GPU's share of long_prefill_65536 under an 8-way head split: T=65536, H=4")
    cr = bench_carried(args.steps, args.warmup)
    line["prefill_carried"] = {"workload": "long_prefill_65536 as 16 consecutive 4096-token "
                                           "calls, the state carried in place",
                               "tokens_per_s": cr["tokens_per_s"], "ms": cr["ms_median"],
                               "ms_min": cr["ms_min"], "reps": cr["reps"]}
    vp = bench_prefill_workload("varlen_prefill_7680", args.steps, args.warmup)
    line["prefill_varlen"] = _prefill_entry(
        vp, "varlen_prefill_7680: 4 packed sequences {512,1024,2048,4096}, H=32, K=V=128")
    gs = bench_gate_and_snapshots(args.steps, args.warmup)
    line["prefill_varlen"].update(
        ms_gate_prep=gs["ms_gate"], gate_gbs=gs["gate_gbs"],
        ms_gate_prep_then_prefill=gs["ms_gate_prep_then_prefill"],
        with_snapshots_every_256={"ms": gs["ms_with_snapshots_every_256"],
                                  "snapshot_bytes": gs["snapshot_bytes"]})
    timing_rot = (f"mean over a steady stream of calls rotating over {ROTATE_SETS} private "
                  "copies of the buffers, each call's inputs cold in every cache and its "
                  "write-backs paid inside the stream")
    timing_cold = ("median of single calls, each after a 512 MiB write and read that empty "
                   "the last-level cache (dirty lines a call leaves in the caches are written "
                   "back after the timed region)")

    def family(r, what, n_tok, **extra):
        out = {"workload": what, "timing": timing_rot,
               "tokens_per_s": n_tok / (r["ms"] * 1e-3), "ms": r["ms"],
               "algorithmic_bytes": r["bytes"], "total_gbs": r["gbs"],
               "frac_of_hbm_peak": r["gbs"] / HBM_PEAK_GBS,
               "cache_cold_single_call": {"timing": timing_cold, "ms": r["ms_flushed"],
                                          "total_gbs": r["gbs_flushed"],
                                          "frac_of_hbm_peak": r["gbs_flushed"] / HBM_PEAK_GBS},
               "back_to_back_same_buffers": {"ms": r["ms_b2b"], "total_gbs": r["gbs_b2b"]}}
        out.update(extra)
        return out

    d = bench_decode(args.steps, args.warmup)
    line["decode"] = family(d, "decode_256: 256 requests, 512-slot fp32 pool, H=32, K=V=128",
                            256, state_gbs=d["state_gbs"])
    dl = bench_decode_layer(args.steps, args.warmup)
    line["decode"]["with_layer_options"] = {
        "what": "raw gate in the kernel, q/k L2 norm, gated RMSNorm of o (kda_recurrent_decode_ex), "
                "same buffers back to back",
        "ms": dl["ms"], "tokens_per_s": dl["tokens_per_s"], "total_gbs": dl["gbs"],
        "frac_of_hbm_peak": dl["gbs"] / HBM_PEAK_GBS}
    rp = bench_replay(args.steps, args.warmup)
    line["replay_decode"] = family(
        rp, "decode_256 with a 16-entry ring per slot, cursors staggered over the rows "
            "(kda_replay_decode)", 256, mean_ring_entries=rp["mean_ring_entries"],
        flush_frac=rp["flush_frac"], speedup_vs_decode=d["ms"] / rp["ms"])
    vr = bench_verify(args.steps, args.warmup)
    line["verify"] = family(vr, "verify_64x8: 64 requests x 8 draft tokens, 128-slot pool", 512)
    cl = measure_ceilings()
    line["measured_ceilings"] = cl
    # each path against the measured stream of its access pattern: the decode
    # pool update is an in-place read-modify-write; verify, the buffered
    # decode and the prefill kernels read some buffers and write others
    mf = cl["bf16_mfma_16x16x32_tflops"]
    line["roofline"]["frac_of_measured"] = line["roofline"]["achieved"] / (
        cl["hbm_copy_gbs"] if line["roofline"]["unit"] == "GB/s" else mf)
    line["decode"]["frac_of_measured_rmw"] = d["gbs"] / cl["hbm_rmw_gbs"]
    line["replay_decode"]["frac_of_measured_copy"] = rp["gbs"] / cl["hbm_copy_gbs"]
    line["verify"]["frac_of_measured_copy"] = vr["gbs"] / cl["hbm_copy_gbs"]
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baselines(long_inputs, lp["workload"])
    print(json.dumps(line))


if __name__ == "__main__":
    main()
