"""GPU parity of the chunkwise varlen prefill against the fp64 oracle.

The HIP path runs through the C ABI (thin binding); the oracle runs the
token-by-token recurrence on the same seeded inputs and on the same fp32
gates.  Besides the workloads' own gate distribution every shape is also run
in a slow-decay regime (A_log = 0, dt_bias = -8): with the workloads' gates
the state carried between chunks and the initial state decay below e^-38
within one chunk, so only slow decay makes those paths visible.
"""
import numpy as np
import pytest
import torch

import kda_gated_delta_amd as kda
import kda_synth
import oracle
from kda_testutil import TOL, TORCH_IO, assert_io_output, dev, gates_f32, host, rel_err_blocks

pytestmark = pytest.mark.gpu


def _inputs(c, g=None, beta=None):
    if g is None:
        g, beta = gates_f32(c["a"], c["b"], c["A_log"], c["dt_bias"])
    io = TORCH_IO[c["io"]]
    t = dict(q=dev(c["q"], io), k=dev(c["k"], io), v=dev(c["v"], io), g=dev(g),
             beta=dev(beta), cu=dev(c["cu"], torch.int32),
             h0=None if c["h0"] is None else dev(c["h0"]))
    return t, g, beta


def _check(c, chunk, heads=None, g=None, beta=None, scale=None):
    """Runs prefill on the GPU and compares o and ht with the oracle (all
    heads, or the listed ones)."""
    t, g, beta = _inputs(c, g, beta)
    K = c["K"]
    scale = K ** -0.5 if scale is None else scale
    o, ht = kda.kda_chunk_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"],
                                  scale, h0=t["h0"], chunk=chunk)
    torch.cuda.synchronize()
    o, ht = host(o), host(ht)
    hs = slice(None) if heads is None else heads
    sub = lambda x: None if x is None else np.ascontiguousarray(x[:, hs])
    o_ref, ht_ref = oracle.prefill(sub(c["q"]), sub(c["k"]), sub(c["v"]), sub(g),
                                   sub(beta), c["cu"], scale, sub(c["h0"]))
    assert_io_output(o[:, hs], o_ref, c["io"], 1)
    err_ht = rel_err_blocks(ht[:, hs], ht_ref, 2)
    assert err_ht <= TOL[c["io"]], err_ht
    return o, ht


# ------------------------------------------------------------ workloads

def test_tiny_f32_workload():
    w = kda_synth.WORKLOADS["tiny_f32_prefill"]
    for regime in ("config", "long"):
        c = kda_synth.prefill_case(w["seqlens"], w["H"], w["K"], w["V"], w["io"],
                                   seed=w["seed"], regime=regime,
                                   dt_bias_std=w["dt_bias_std"], h0_std=w["h0_std"])
        _check(c, w["chunk"])


def test_tiny_f32_zero_gate():
    """g = 0 (no decay) everywhere: the longest memory the recurrence has."""
    w = kda_synth.WORKLOADS["tiny_f32_prefill"]
    c = kda_synth.prefill_case(w["seqlens"], w["H"], w["K"], w["V"], w["io"], seed=5,
                               h0_std=0.5)
    _, beta = gates_f32(c["a"], c["b"], c["A_log"], c["dt_bias"])
    _check(c, w["chunk"], g=np.zeros_like(c["a"]), beta=beta)


@pytest.mark.parametrize("regime", ["config", "long"])
def test_varlen_workload(regime):
    w = kda_synth.WORKLOADS["varlen_prefill_7680"]
    c = kda_synth.prefill_case(w["seqlens"], w["H"], w["K"], w["V"], w["io"],
                               seed=w["seed"], regime=regime,
                               dt_bias_std=w["dt_bias_std"], h0_std=w["h0_std"])
    _check(c, w["chunk"])


def test_long_workload_segments_vs_full_vs_oracle():
    """65536 tokens: 16 carried segments of 4096 equal one full run bit for
    bit (the full run's state pass is cut into waves that hand the state on
    exactly, the 4096-token calls likewise), and both match the oracle
    (sampled heads)."""
    w = kda_synth.WORKLOADS["long_prefill_65536"]
    c = kda_synth.prefill_case(w["seqlens"], w["H"], w["K"], w["V"], w["io"],
                               seed=w["seed"], regime="long",
                               dt_bias_std=w["dt_bias_std"], h0_std=w["h0_std"])
    t, g, beta = _inputs(c)
    T, scale = c["T"], w["K"] ** -0.5
    o_full, ht_full = kda.kda_chunk_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                            t["cu"], scale, h0=t["h0"], chunk=w["chunk"])
    seg = T // w["segments"]
    state = t["h0"].clone()
    o_seg = torch.empty_like(o_full)
    cu1 = torch.tensor([0, seg], dtype=torch.int32, device="cuda")
    for s in range(w["segments"]):
        sl = slice(s * seg, (s + 1) * seg)
        o_s, _ = kda.kda_chunk_prefill(t["q"][sl], t["k"][sl], t["v"][sl], t["g"][sl],
                                       t["beta"][sl], cu1, scale, h0=state, ht=state,
                                       chunk=w["chunk"])  # in place: ht aliases h0
        o_seg[sl] = o_s
    torch.cuda.synchronize()
    # the segment boundaries coincide with chunk boundaries: identical arithmetic
    assert torch.equal(o_seg, o_full)
    assert torch.equal(state, ht_full)
    heads = [0, 13, 31]
    sub = lambda x: np.ascontiguousarray(x[:, heads])
    o_ref, ht_ref = oracle.prefill(sub(c["q"]), sub(c["k"]), sub(c["v"]), sub(g),
                                   sub(beta), c["cu"], scale, sub(c["h0"]))
    for o_, ht_ in ((o_full, ht_full), (o_seg, state)):
        assert_io_output(host(o_)[:, heads], o_ref, "bf16", 1)
        assert rel_err_blocks(host(ht_)[:, heads], ht_ref, 2) <= TOL["bf16"]


# ---------------------------------------------------------- shapes, edges

@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_head_dims_and_chunk_sizes(io, D, chunk):
    c = kda_synth.prefill_case([5, 17, 1, 41, 100], 3, D, D, io, seed=D + chunk,
                               regime="long")
    _check(c, chunk)


def _many_lengths(n):
    """n sequence lengths 0 .. 60 in a fixed scrambled order (zeros, ones and
    lengths on both sides of the 16-token chunk boundary included)."""
    return [(i * 37) % 61 for i in range(n)]


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_many_sequences_across_plan_blocks(io):
    # 700 sequences: the chunk-table kernel takes them 256 at a time and
    # carries the token, chunk and slot offsets from block to block; each
    # sequence has its own initial state
    c = kda_synth.prefill_case(_many_lengths(700), 2, 32, 32, io, seed=77, regime="long",
                               h0_std=0.1)
    assert len(c["cu"]) == 701 and int(c["cu"][-1]) > 16 * 700
    _check(c, 16)


@pytest.mark.parametrize("T", [1, 8, 64, 65, 128, 1024])
def test_single_sequence_lengths(T):
    for io in ("f32", "bf16"):
        c = kda_synth.prefill_case([T], 2, 128, 128, io, seed=T, regime="long")
        _check(c, 64)


@pytest.mark.parametrize("seqlens", [[32, 32, 32, 32], [5, 17, 1, 41], [128],
                                     [0, 70, 0, 3, 0]])
def test_varlen_edges_with_and_without_h0(seqlens):
    for h0_std in (None, 0.3):
        c = kda_synth.prefill_case(seqlens, 4, 64, 64, "bf16", seed=len(seqlens),
                                   regime="long", h0_std=h0_std)
        _, ht = _check(c, 32)
        for n, L in enumerate(seqlens):
            if L == 0:  # an empty sequence hands its initial state through
                exp = np.zeros_like(ht[n]) if c["h0"] is None else c["h0"][n]
                np.testing.assert_array_equal(ht[n], exp)


def test_result_does_not_depend_on_chunk_size():
    c = kda_synth.prefill_case([300, 77], 2, 128, 128, "f32", seed=9, regime="long")
    t, g, beta = _inputs(c)
    outs = [kda.kda_chunk_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"],
                                  0.1, h0=t["h0"], chunk=C) for C in (16, 32, 64)]
    torch.cuda.synchronize()
    for o, ht in outs[1:]:
        assert rel_err_blocks(host(o), host(outs[0][0]), 1) <= 5e-5
        assert rel_err_blocks(host(ht), host(outs[0][1]), 2) <= 5e-5


def test_no_final_state_and_empty_batch():
    c = kda_synth.prefill_case([40, 9], 2, 32, 32, "bf16", seed=3)
    t, g, beta = _inputs(c)
    o, ht = kda.kda_chunk_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"],
                                  0.2, h0=t["h0"], output_final_state=False, chunk=16)
    assert ht is None
    o_ref, _ = oracle.prefill(c["q"], c["k"], c["v"], g, beta, c["cu"], 0.2, c["h0"])
    torch.cuda.synchronize()
    assert_io_output(host(o), o_ref, "bf16", 1)
    # T = 0: only ht = h0 is written
    z = lambda *s: torch.zeros(*s, device="cuda")
    cu0 = torch.zeros(3, dtype=torch.int32, device="cuda")
    h0 = torch.randn(2, 2, 32, 32, device="cuda")
    o0, ht0 = kda.kda_chunk_prefill(z(0, 2, 32).bfloat16(), z(0, 2, 32).bfloat16(),
                                    z(0, 2, 32).bfloat16(), z(0, 2, 32), z(0, 2), cu0,
                                    0.2, h0=h0, chunk=16)
    torch.cuda.synchronize()
    assert o0.shape == (0, 2, 32) and torch.equal(ht0, h0)


def test_prefill_then_decodes_equals_longer_prefill():
    """prefill(seq[:T]) vs prefill(seq[:T-8]) followed by 8 decode steps."""
    c = kda_synth.prefill_case([200], 4, 128, 128, "bf16", seed=12, regime="long")
    t, g, beta = _inputs(c)
    T, kk, scale = 200, 8, 128 ** -0.5
    o_full, ht_full = kda.kda_chunk_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                            t["cu"], scale, h0=t["h0"])
    cu = torch.tensor([0, T - kk], dtype=torch.int32, device="cuda")
    pre = slice(0, T - kk)
    o_pre, ht_pre = kda.kda_chunk_prefill(t["q"][pre], t["k"][pre], t["v"][pre],
                                          t["g"][pre], t["beta"][pre], cu, scale,
                                          h0=t["h0"])
    pool = torch.cat([torch.zeros_like(ht_pre), ht_pre])  # slot 1
    idx = torch.ones(1, dtype=torch.int32, device="cuda")
    o_dec = []
    for i in range(T - kk, T):
        o_dec.append(kda.kda_recurrent_decode(t["q"][i:i + 1], t["k"][i:i + 1],
                                              t["v"][i:i + 1], t["g"][i:i + 1],
                                              t["beta"][i:i + 1], scale, pool, idx))
    torch.cuda.synchronize()
    o_dec = host(torch.cat(o_dec))
    # both routes are checked against the oracle, and against each other
    o_ref, ht_ref = oracle.prefill(c["q"], c["k"], c["v"], g, beta, c["cu"], scale, c["h0"])
    assert_io_output(o_dec, o_ref[T - kk:], "bf16", 1)
    assert rel_err_blocks(host(pool[1:]), ht_ref, 2) <= TOL["bf16"]
    assert rel_err_blocks(host(pool[1:]), host(ht_full), 2) <= TOL["bf16"]
    np.testing.assert_array_equal(host(o_pre), host(o_full[pre]))


def test_marked_prefill_equals_unmarked():
    """The timing-mark variant does the same work as the gated call:
    bit-identical results, and each mark pair brackets a kernel of positive
    duration."""
    c = kda_synth.prefill_case([300, 77, 640], 4, 128, 128, "bf16", seed=21, regime="long")
    io = TORCH_IO["bf16"]
    q, k, v = dev(c["q"], io), dev(c["k"], io), dev(c["v"], io)
    a, b, A_log, dt_bias = dev(c["a"]), dev(c["b"]), dev(c["A_log"]), dev(c["dt_bias"])
    cu, h0 = dev(c["cu"], torch.int32), dev(c["h0"])
    o1, ht1 = kda.kda_chunk_prefill_gated(q, k, v, a, b, A_log, dt_bias, cu, 0.1, h0=h0)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    o2, ht2 = kda.kda_chunk_prefill_marked(marks, q, k, v, a, b, A_log, dt_bias, cu, 0.1,
                                           h0=h0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(ht1, ht2)
    for i in range(3):
        assert marks[i].elapsed_time(marks[i + 1]) > 0


@pytest.mark.parametrize("lower_bound,with_bias,D,seqlens", [
    (0.0, True, 128, [300, 77, 640]),
    (-5.0, True, 128, [64, 1, 129]),
    (0.0, False, 64, [40, 9, 0, 100]),
])
def test_gated_prefill_equals_gate_prep_then_prefill(lower_bound, with_bias, D, seqlens):
    """The gate applied inside the prefill is the gate kernel's own: the
    fused call reproduces gate prep followed by prefill bit for bit, and
    both match the oracle."""
    c = kda_synth.prefill_case(seqlens, 4, D, D, "bf16", seed=31, h0_std=0.02)
    io = TORCH_IO["bf16"]
    q, k, v = dev(c["q"], io), dev(c["k"], io), dev(c["v"], io)
    a, b, A_log = dev(c["a"]), dev(c["b"]), dev(c["A_log"])
    dt_bias = dev(c["dt_bias"]) if with_bias else None
    cu, h0 = dev(c["cu"], torch.int32), dev(c["h0"])
    scale = D ** -0.5
    g, beta = kda.kda_gate_prep(a, b, A_log, dt_bias, lower_bound=lower_bound)
    o1, ht1 = kda.kda_chunk_prefill(q, k, v, g, beta, cu, scale, h0=h0)
    o2, ht2 = kda.kda_chunk_prefill_gated(q, k, v, a, b, A_log, dt_bias, cu, scale,
                                          lower_bound=lower_bound, h0=h0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(ht1, ht2)
    g_ref, b_ref = oracle.gate(c["a"], c["b"], c["A_log"],
                               c["dt_bias"] if with_bias else None, lower_bound)
    g32, b32 = g_ref.astype(np.float32), b_ref.astype(np.float32)
    o_ref, ht_ref = oracle.prefill(c["q"], c["k"], c["v"], g32, b32, c["cu"], scale, c["h0"])
    assert_io_output(host(o2), o_ref, "bf16", 1)
    assert rel_err_blocks(host(ht2), ht_ref, 2) <= TOL["bf16"]


@pytest.mark.parametrize("cu_bad,T", [([0, 200, 0, 200], 200),
                                      ([0, 150, 40, 300, 200, 300], 300),
                                      ([-7, 120, 999, 50, 300], 300)])
def test_malformed_cu_seqlens_stay_in_bounds(cu_bad, T):
    """cu_seqlens that decrease or leave [0, T] (no KDA_CHECK): the kernels
    take the disjoint clamped ranges (tests/test_plan_bounds.py), so the call
    equals the same call on that clamped array bit for bit, and matches the
    oracle there; snapshot rows stay within T // interval."""
    N = len(cu_bad) - 1
    p = np.maximum.accumulate(np.clip(np.asarray(cu_bad, dtype=np.int64), 0, T))
    assert p[0] == 0 and p[-1] == T
    c = kda_synth.prefill_case(list(np.diff(p)), 2, 64, 64, "bf16", seed=N, regime="long",
                               h0_std=0.1)
    t, g, beta = _inputs(c)
    bad = torch.tensor(cu_bad, dtype=torch.int32, device="cuda")
    outs = []
    for cu in (bad, t["cu"]):
        # rows past the batch's total are left untouched: start from zeros
        snaps = torch.zeros((T // 64, 2, 64, 64), device="cuda")
        o, ht, snaps = kda.kda_chunk_prefill_snapshots(
            t["q"], t["k"], t["v"], t["g"], t["beta"], cu, 0.125, 64, h0=t["h0"], chunk=32,
            snapshots=snaps)
        outs.append((o, ht, snaps))
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    o_ref, ht_ref = oracle.prefill(c["q"], c["k"], c["v"], g, beta, p, 0.125, c["h0"])
    assert_io_output(host(outs[1][0]), o_ref, "bf16", 1)
    assert rel_err_blocks(host(outs[1][1]), ht_ref, 2) <= TOL["bf16"]


def test_wave_schedule_equals_single_stream_and_oracle():
    """A batch of few sequences with at least 128 chunks in all runs its
    state pass in waves, the intra-chunk work of each wave on a second
    stream: the results equal the single-stream order (the timing-marks call
    runs every kernel on one stream) bit for bit, with and without the gate
    in the kernel and with snapshots, and match the oracle."""
    seqlens = [6000, 50, 2400, 0]
    assert kda.kda_chunk_prefill_schedule(sum(seqlens), len(seqlens), 32, 64, 64)["n_waves"] > 1
    c = kda_synth.prefill_case(seqlens, 32, 64, 64, "bf16", seed=51, regime="long", h0_std=0.05)
    t, g, beta = _inputs(c)
    a, b = dev(c["a"]), dev(c["b"])
    A_log, dt_bias = dev(c["A_log"]), dev(c["dt_bias"])
    o1, ht1 = kda.kda_chunk_prefill_gated(t["q"], t["k"], t["v"], a, b, A_log, dt_bias, t["cu"],
                                          0.125, h0=t["h0"], chunk=64)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    o2, ht2 = kda.kda_chunk_prefill_marked(marks, t["q"], t["k"], t["v"], a, b, A_log, dt_bias,
                                           t["cu"], 0.125, h0=t["h0"], chunk=64)
    o3, ht3, snaps = kda.kda_chunk_prefill_snapshots(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                                     t["cu"], 0.125, 256, h0=t["h0"], chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(ht1, ht2)
    heads = [0, 17, 31]
    sub = lambda x: None if x is None else np.ascontiguousarray(x[:, heads])
    o_ref, ht_ref = oracle.prefill(sub(c["q"]), sub(c["k"]), sub(c["v"]), sub(g), sub(beta),
                                   c["cu"], 0.125, sub(c["h0"]))
    assert_io_output(host(o3)[:, heads], o_ref, "bf16", 1)
    assert rel_err_blocks(host(ht3)[:, heads], ht_ref, 2) <= TOL["bf16"]
    # a snapshot deep in the first sequence (in a later wave): the final
    # state of a prefill of that prefix alone
    L = 256 * 9
    cu1 = torch.tensor([0, L], dtype=torch.int32, device="cuda")
    _, ht_pre = kda.kda_chunk_prefill(t["q"][:L], t["k"][:L], t["v"][:L], t["g"][:L],
                                      t["beta"][:L], cu1, 0.125, h0=t["h0"][:1], chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(snaps[8], ht_pre[0])


def test_wave_schedule_under_graph_capture():
    """A waved prefill captured into a HIP graph keeps to the capturing
    stream (the second stream is for eager calls only).  Every replay, with
    eager work and a cleared output between replays, equals the eager call
    bit for bit, and so does an eager call on a side stream."""
    seqlens = [6000, 50, 2400, 0]
    assert kda.kda_chunk_prefill_schedule(sum(seqlens), len(seqlens), 32, 64, 64)["n_waves"] > 1
    c = kda_synth.prefill_case(seqlens, 32, 64, 64, "bf16", seed=53, regime="long", h0_std=0.05)
    t, _, _ = _inputs(c)
    a, b = dev(c["a"]), dev(c["b"])
    A_log, dt_bias = dev(c["A_log"]), dev(c["dt_bias"])
    T, N = int(c["T"]), len(seqlens)
    o = torch.empty_like(t["v"])
    ht = torch.empty_like(t["h0"])
    ws = torch.empty(kda.kda_chunk_prefill_workspace_size(T, N, 32, 64, 64, 64),
                     dtype=torch.uint8, device="cuda")
    call = lambda: kda.kda_chunk_prefill_gated(t["q"], t["k"], t["v"], a, b, A_log, dt_bias,
                                               t["cu"], 0.125, h0=t["h0"], chunk=64, o=o, ht=ht,
                                               workspace=ws)
    call()
    torch.cuda.synchronize()
    o_ref, ht_ref = o.clone(), ht.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o.zero_()
        call()
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(ht, ht_ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for _ in range(3):
        o.zero_()
        ht.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(ht, ht_ref)
        call()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref)
