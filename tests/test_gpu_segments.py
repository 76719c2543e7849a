"""GPU parity of the state pass when long chains are cut into segments.

When a batch's (sequence, head) chains would leave most of the chip idle and
a sequence has at least 128 chunks, the state pass cuts it into segments:
the first runs from h0, the middle ones build their affine chunk maps
S -> M S + B side by side ("ReplaySSM" analysis, section 2.1: diagonal decays
compose), a scan chains the start states, and the later segments re-run from
them.  The result differs from the uncut chain only by rounding, so these
tests hold it to the oracle at the usual tolerances, in the slow-decay regime
where the carried state matters (A_log = 0, dt_bias = -8; "Linear attention"
tutorial, section "实例：Kimi K3"), and compare it with the same sequence run
as carried pieces short enough never to be cut.
"""
import numpy as np
import pytest
import torch

import kda_gated_delta_amd as kda
import kda_synth
import oracle
from kda_testutil import TOL, TORCH_IO, assert_io_output, dev, gates_f32, host, rel_err_blocks

pytestmark = pytest.mark.gpu


def _run(c, chunk, scale, **kw):
    g, beta = gates_f32(c["a"], c["b"], c["A_log"], c["dt_bias"])
    io = TORCH_IO[c["io"]]
    t = dict(q=dev(c["q"], io), k=dev(c["k"], io), v=dev(c["v"], io), g=dev(g), beta=dev(beta),
             cu=dev(c["cu"], torch.int32), h0=None if c["h0"] is None else dev(c["h0"]))
    return t, g, beta


def test_cut_chain_matches_oracle_and_carried_pieces():
    # one 16384-token sequence, H = 4: 256 chunks on 16 chains -> cut
    c = kda_synth.prefill_case([16384], 4, 128, 128, "bf16", seed=41, regime="long",
                               h0_std=0.05)
    t, g, beta = _run(c, 64, 128 ** -0.5)
    scale = 128 ** -0.5
    o, ht = kda.kda_chunk_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], scale,
                                  h0=t["h0"], chunk=64)
    # the same sequence as four carried pieces of 4096 tokens (64 chunks:
    # never cut), the state handed on in place
    state = t["h0"].clone()
    o_pc = torch.empty_like(o)
    cu1 = torch.tensor([0, 4096], dtype=torch.int32, device="cuda")
    for s in range(4):
        sl = slice(4096 * s, 4096 * (s + 1))
        o_s, _ = kda.kda_chunk_prefill(t["q"][sl], t["k"][sl], t["v"][sl], t["g"][sl],
                                       t["beta"][sl], cu1, scale, h0=state, ht=state, chunk=64)
        o_pc[sl] = o_s
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.prefill(c["q"], c["k"], c["v"], g, beta, c["cu"], scale, c["h0"])
    assert_io_output(host(o), o_ref, "bf16", 1)
    assert rel_err_blocks(host(ht), ht_ref, 2) <= TOL["bf16"]
    assert_io_output(host(o_pc), o_ref, "bf16", 1)
    # cut and uncut chains agree far inside the tolerance
    assert rel_err_blocks(host(ht), host(state), 2) <= 1e-4
    assert rel_err_blocks(host(o), host(o_pc), 1) <= 5e-3


def test_cut_chains_in_a_varlen_batch():
    # long and short sequences, an empty one: the long ones are cut, the
    # others run whole in the same launches
    seqlens = [5000, 17, 9000, 0, 4100]
    c = kda_synth.prefill_case(seqlens, 2, 64, 64, "bf16", seed=42, regime="long", h0_std=0.1)
    t, g, beta = _run(c, 32, 0.125)
    o, ht = kda.kda_chunk_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], 0.125,
                                  h0=t["h0"], chunk=32)
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.prefill(c["q"], c["k"], c["v"], g, beta, c["cu"], 0.125, c["h0"])
    assert_io_output(host(o), o_ref, "bf16", 1)
    assert rel_err_blocks(host(ht), ht_ref, 2) <= TOL["bf16"]
    np.testing.assert_array_equal(host(ht)[3], c["h0"][3])  # empty: h0 handed through


def test_cut_chain_fp32_inputs():
    # fp32 io at the 1e-4 bar: 256 chunks of 16 on 2 heads
    c = kda_synth.prefill_case([4096], 2, 32, 32, "f32", seed=43, regime="long", h0_std=0.1)
    t, g, beta = _run(c, 16, 32 ** -0.5)
    o, ht = kda.kda_chunk_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"],
                                  32 ** -0.5, h0=t["h0"], chunk=16)
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.prefill(c["q"], c["k"], c["v"], g, beta, c["cu"], 32 ** -0.5,
                                   c["h0"])
    assert_io_output(host(o), o_ref, "f32", 1)
    assert rel_err_blocks(host(ht), ht_ref, 2) <= TOL["f32"]


def test_cut_chain_snapshots():
    # snapshots every 256 tokens, inside the re-run segments too: each equals
    # the oracle's final state on that prefix
    seqlens = [9000, 3000]
    c = kda_synth.prefill_case(seqlens, 2, 64, 64, "bf16", seed=44, regime="long", h0_std=0.1)
    t, g, beta = _run(c, 32, 0.125)
    o, ht, snaps = kda.kda_chunk_prefill_snapshots(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                                   t["cu"], 0.125, 256, h0=t["h0"], chunk=32)
    torch.cuda.synchronize()
    snaps = host(snaps)
    rows0 = seqlens[0] // 256
    for n, j in [(0, 0), (0, 7), (0, 20), (0, rows0 - 1), (1, 5)]:
        L = 256 * (j + 1)
        s0 = 0 if n == 0 else seqlens[0]
        sl = slice(s0, s0 + L)
        cut = lambda x: np.ascontiguousarray(x[sl])
        _, st_ref = oracle.prefill(cut(c["q"]), cut(c["k"]), cut(c["v"]), cut(g), cut(beta),
                                   np.array([0, L]), 0.125, c["h0"][n:n + 1])
        row = j if n == 0 else rows0 + j
        assert rel_err_blocks(snaps[row:row + 1], st_ref, 2) <= TOL["bf16"], (n, j)


def test_cut_chain_long_memory_eight_heads():
    # one 16384-token sequence on 8 heads at K = V = 128 (affine maps, eight
    # segments of 32 chunks), every head against the oracle in the
    # slow-decay regime, whose carried state reaches across the cuts
    s = kda.kda_chunk_prefill_schedule(16384, 1, 8, 128, 128, 64)
    assert s["uses_maps"] == 1 and s["segment_chunks"] > 0
    c = kda_synth.prefill_case([16384], 8, 128, 128, "bf16", seed=45, regime="long",
                               h0_std=0.05)
    t, g, beta = _run(c, 64, 128 ** -0.5)
    scale = 128 ** -0.5
    o, ht = kda.kda_chunk_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], scale,
                                  h0=t["h0"], chunk=64)
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.prefill(c["q"], c["k"], c["v"], g, beta, c["cu"], scale, c["h0"])
    assert_io_output(host(o), o_ref, "bf16", 1)
    assert rel_err_blocks(host(ht), ht_ref, 2) <= TOL["bf16"]


@pytest.mark.parametrize("T,H,chunk,io", [(8192, 2, 16, "bf16"), (65536, 1, 16, "f32")])
def test_cut_chain_small_heads_long_scan(T, H, chunk, io):
    # K = V = 16: one V tile per head; the 65536-token case cuts 4096 chunks
    # into 64 segments, so the scan chains 62 maps
    s = kda.kda_chunk_prefill_schedule(T, 1, H, 16, 16, chunk)
    assert s["uses_maps"] == 1
    c = kda_synth.prefill_case([T], H, 16, 16, io, seed=46, regime="long", h0_std=0.1)
    t, g, beta = _run(c, chunk, 0.25)
    o, ht = kda.kda_chunk_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], 0.25,
                                  h0=t["h0"], chunk=chunk)
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.prefill(c["q"], c["k"], c["v"], g, beta, c["cu"], 0.25, c["h0"])
    assert_io_output(host(o), o_ref, io, 1)
    assert rel_err_blocks(host(ht), ht_ref, 2) <= TOL[io]
