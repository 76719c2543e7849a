"""Chunk-boundary state snapshots, kda_chunk_prefill_snapshots (tutorial,
sections "两种计算形态" and "prefix cache 与投机解码"): each snapshot must be
bit-identical to the final state of a prefill run on that prefix alone, o
and ht bit-identical to kda_chunk_prefill, and the snapshots must match the
oracle's state after the prefix."""
import numpy as np
import pytest
import torch

import kda_gated_delta_amd as kda
import kda_synth
import oracle
from kda_testutil import TOL, TORCH_IO, dev, gates_f32, host, rel_err_blocks

pytestmark = pytest.mark.gpu


def _inputs(c):
    g, beta = gates_f32(c["a"], c["b"], c["A_log"], c["dt_bias"])
    io = TORCH_IO[c["io"]]
    return dict(q=dev(c["q"], io), k=dev(c["k"], io), v=dev(c["v"], io), g=dev(g),
                beta=dev(beta), cu=dev(c["cu"], torch.int32),
                h0=None if c["h0"] is None else dev(c["h0"])), g, beta


def _prefixes(cu, interval):
    """(sequence, prefix length) of every snapshot row, in row order."""
    rows = []
    for n in range(len(cu) - 1):
        L = int(cu[n + 1] - cu[n])
        rows += [(n, (j + 1) * interval) for j in range(L // interval)]
    return rows


def _check(c, chunk, interval, against_oracle=True):
    t, g, beta = _inputs(c)
    K, H, V = c["K"], c["H"], c["V"]
    T = int(c["cu"][-1])
    scale = K ** -0.5
    rows = _prefixes(c["cu"], interval)
    cap = T // interval + 2
    snaps = torch.full((cap, H, K, V), float("nan"), device="cuda")
    o_s, ht_s, _ = kda.kda_chunk_prefill_snapshots(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                                   t["cu"], scale, interval, h0=t["h0"],
                                                   chunk=chunk, snapshots=snaps)
    o_p, ht_p = kda.kda_chunk_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"],
                                      scale, h0=t["h0"], chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_p) and torch.equal(ht_s, ht_p)
    assert torch.isnan(snaps[len(rows):]).all()  # rows past the total untouched
    if not rows:
        return
    # every prefix as a sequence of its own, in one batch
    cu = c["cu"]
    sel = np.concatenate([np.arange(cu[n], cu[n] + P) for n, P in rows])
    cu_p = np.concatenate([[0], np.cumsum([P for _, P in rows])]).astype(np.int32)
    h0_p = None if c["h0"] is None else t["h0"][[n for n, _ in rows]].contiguous()
    sel_d = torch.from_numpy(sel).cuda()
    _, ht_pre = kda.kda_chunk_prefill(t["q"][sel_d].contiguous(), t["k"][sel_d].contiguous(),
                                      t["v"][sel_d].contiguous(), t["g"][sel_d].contiguous(),
                                      t["beta"][sel_d].contiguous(), dev(cu_p, torch.int32),
                                      scale, h0=h0_p, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(snaps[:len(rows)], ht_pre)
    if against_oracle:
        h0 = None if c["h0"] is None else c["h0"][[n for n, _ in rows]]
        _, ht_ref = oracle.prefill(c["q"][sel], c["k"][sel], c["v"][sel], g[sel], beta[sel],
                                   cu_p, scale, h0)
        assert rel_err_blocks(host(snaps[:len(rows)]), ht_ref, 2) <= TOL[c["io"]]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("chunk,interval", [(64, 64), (64, 128), (32, 96), (16, 16)])
def test_snapshots_small_batches(io, chunk, interval):
    # ragged lengths, a zero-length sequence, sequences shorter than the interval
    c = kda_synth.prefill_case([200, 64, 5, 0, 384, 130], 3, 32, 32, io, seed=chunk + interval,
                               regime="long", h0_std=0.02)
    _check(c, chunk, interval)


@pytest.mark.parametrize("KV", [(16, 16), (64, 64), (128, 128)])
def test_snapshots_head_dims(KV):
    K, V = KV
    c = kda_synth.prefill_case([256, 193], 2, K, V, "bf16", seed=K, h0_std=None)
    _check(c, 64, 64)


def test_snapshots_varlen_workload():
    # the 7680-token batch {512, 1024, 2048, 4096}, H=32, K=V=128: a snapshot
    # every 1024 tokens (7 rows), checked bit for bit against the prefixes
    w = kda_synth.WORKLOADS["varlen_prefill_7680"]
    c = kda_synth.prefill_case(w["seqlens"], w["H"], w["K"], w["V"], w["io"], seed=w["seed"],
                               dt_bias_std=w["dt_bias_std"], h0_std=w["h0_std"])
    _check(c, w["chunk"], 1024, against_oracle=False)


def test_snapshots_many_sequences():
    # 700 sequences of 0 .. 60 tokens: snapshot rows are numbered across the
    # chunk-table kernel's blocks of 256 sequences
    lengths = [(i * 37) % 61 for i in range(700)]
    c = kda_synth.prefill_case(lengths, 2, 32, 32, "bf16", seed=78, h0_std=0.05)
    _check(c, 16, 16)
