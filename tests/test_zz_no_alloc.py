"""kda_chunk_prefill_noalloc: the prefill on the library's static scratch
array (no allocation), called through the C ABI, against
kda_chunk_prefill_ex with its own workspace.  The two share every kernel, so
their outputs must be identical bit for bit: two calls in a row, the second
with a smaller batch (the scratch keeps the first call's contents), and the
model-layer options on the second."""
import numpy as np
import pytest
import torch

import kda_gated_delta_amd as kda
import kda_synth
from kda_testutil import dev, gates_f32

pytestmark = pytest.mark.gpu


def _case(seqlens, H, D, seed, io="bf16"):
    c = kda_synth.prefill_case(seqlens, H, D, D, io, seed=seed, regime="long", h0_std=0.05)
    g, beta = gates_f32(c["a"], c["b"], c["A_log"], c["dt_bias"])
    iot = torch.bfloat16 if io == "bf16" else torch.float32
    return dict(q=dev(c["q"], iot), k=dev(c["k"], iot), v=dev(c["v"], iot), g=dev(g),
                beta=dev(beta), cu=dev(c["cu"], torch.int32), h0=dev(c["h0"]),
                a=dev(c["a"]), b=dev(c["b"]), A_log=dev(c["A_log"]),
                dt_bias=dev(c["dt_bias"]))


def _outputs(t):
    T, H, V = t["v"].shape
    N = t["cu"].shape[0] - 1
    K = t["q"].shape[2]
    return (torch.full((T, H, V), float("nan"), dtype=t["q"].dtype, device="cuda"),
            torch.full((N, H, K, V), float("nan"), device="cuda"))


def test_noalloc_equals_prefill_ex_on_two_calls():
    big = _case([700, 1300, 64, 1], 32, 128, seed=21)
    small = _case([33, 200, 0, 91], 8, 64, seed=22)
    # first call: the plain prefill
    o1, ht1 = _outputs(big)
    kda.kda_chunk_prefill_noalloc(big["q"], big["k"], big["v"], big["g"], big["beta"],
                                  big["cu"], 0.088, o1, ht=ht1, h0=big["h0"], chunk=64)
    r1 = kda.kda_chunk_prefill_ex(big["q"], big["k"], big["v"], big["g"], big["beta"],
                                  big["cu"], 0.088, h0=big["h0"], chunk=64)
    # second call, a smaller batch with the gate applied in the kernel and
    # the in-kernel q/k norm
    o2, ht2 = _outputs(small)
    opts = dict(raw_gate=(small["A_log"], small["dt_bias"], 0.0), qk_l2norm=True,
                h0=small["h0"], chunk=32)
    kda.kda_chunk_prefill_noalloc(small["q"], small["k"], small["v"], small["a"], small["b"],
                                  small["cu"], 0.125, o2, ht=ht2, **opts)
    r2 = kda.kda_chunk_prefill_ex(small["q"], small["k"], small["v"], small["a"], small["b"],
                                  small["cu"], 0.125, **opts)
    torch.cuda.synchronize()
    assert torch.equal(o1, r1[0]) and torch.equal(ht1, r1[1])
    assert torch.equal(o2, r2[0]) and torch.equal(ht2, r2[1])
    assert not torch.isnan(o2.float()).any()


def test_noalloc_rejects_a_batch_beyond_the_scratch():
    # needs more workspace than the static array holds: refused before any
    # work is enqueued, and the outputs are left as they were
    H, D, T = 32, 128, 8192
    need = kda.kda_chunk_prefill_workspace_size(T, 1, H, D, D, 64)
    assert need > kda.NOALLOC_SCRATCH_BYTES
    z = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((T, H, D), device="cuda")
    beta = torch.zeros((T, H), device="cuda")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    o = torch.full((T, H, D), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kda.KdaError) as e:
        kda.kda_chunk_prefill_noalloc(z, z, z, g, beta, cu, 0.1, o)
    assert e.value.status == 5  # KDA_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
