"""The prefill at its largest offsets: one sequence of 2^23 + 37 tokens on 4
heads (bf16 io), whose q, k, v and o rows lie up to 8.6 GB into their buffers,
on the cut-chain schedule (few heads, a very long chain).

The sequence's gate resets the state at the last token of every chunk
(g = -1e4 on every channel, so exp(g) = 0 in fp32 and fp64 alike; by the
recurrence of the "Linear attention" tutorial, section "KDA", the state after
that token is beta k^T v whatever came before).  The outputs of a chunk then
depend only on the previous chunk's last token and on the chunk itself, and
any sampled chunk is checked against the oracle run on that 65-token window,
its inputs copied back from the device buffers the kernels read.
"""
import numpy as np
import pytest
import torch

import kda_gated_delta_amd as kda
import kda_synth
import oracle
from kda_testutil import TOL, assert_io_output, dev, gates_f32, host, rel_err_blocks

pytestmark = pytest.mark.gpu


def test_sequence_past_4gib_byte_offsets():
    T, H, K, V, C = (1 << 23) + 37, 4, 128, 128, 64
    P = 4099  # tokens of the seeded base block that is tiled over the sequence
    c = kda_synth.prefill_case([P], H, K, V, "bf16", seed=11, h0_std=0.02)
    g, beta = gates_f32(c["a"], c["b"], c["A_log"], c["dt_bias"])
    reps = (T + P - 1) // P

    def tile(x, dtype=torch.float32):  # [P, ...] on the host -> [T, ...] on the device
        d = dev(x, dtype)
        return d.repeat((reps,) + (1,) * (d.dim() - 1))[:T].contiguous()

    q, k = tile(c["q"], torch.bfloat16), tile(c["k"], torch.bfloat16)
    gg, bb = tile(g), tile(beta)
    # v plus a ramp of 2^-20 per token, rounded to bf16: rows 2^22 tokens
    # apart (4 GiB of q, k and v at this width) differ by 4, so a read from a
    # wrapped offset would show (q and k repeat with the odd period P)
    v = tile(c["v"])
    v += (torch.arange(T, device="cuda", dtype=torch.float32) * 2.0 ** -20)[:, None, None]
    v = v.to(torch.bfloat16)
    gg[C - 1::C] = -1.0e4
    cu = dev(np.array([0, T], np.int32), torch.int32)
    assert kda.kda_chunk_prefill_schedule(T, 1, H, K, V, C)["uses_maps"] == 1
    scale = K ** -0.5
    o, ht = kda.kda_chunk_prefill(q, k, v, gg, bb, cu, scale, h0=dev(c["h0"]), chunk=C)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(ht).all())

    nch = (T + C - 1) // C
    far = (5 << 20) // C  # rows about 5.4 GB into q, k, v and o
    assert far * C * H * K * 2 > (1 << 32)
    for ch in (0, 1, 2, nch // 2, far, nch - 2, nch - 1):
        t0 = 0 if ch == 0 else C * ch - 1
        t1 = min(C * (ch + 1), T)
        win = lambda x: np.ascontiguousarray(host(x[t0:t1]))
        o_ref, ht_ref = oracle.prefill(win(q), win(k), win(v), win(gg), win(bb),
                                       np.array([0, t1 - t0]), scale,
                                       c["h0"] if ch == 0 else None)
        skip = 0 if ch == 0 else 1  # the previous chunk's last token
        assert_io_output(host(o[t0 + skip:t1]), o_ref[skip:], "bf16", 1)
        if ch == nch - 1:
            err = rel_err_blocks(host(ht), ht_ref, 2)
            assert err <= TOL["bf16"], err
    # about 150 GB of device memory: hand it back before the next tests
    del q, k, v, gg, bb, o, ht
    torch.cuda.empty_cache()
