"""Model-layer options of decode and verify (kda_recurrent_decode_ex,
kda_verify_ex): the gate applied in the kernel from raw inputs, the per-head
(Gated DeltaNet) gate, grouped q/k heads, in-kernel q/k L2 normalisation and
the gated RMSNorm of the output.  Options that restate another path exactly
are checked bit for bit against it; the rest against the oracle."""
import numpy as np
import pytest
import torch

import kda_gated_delta_amd as kda
import kda_synth
import oracle
from kda_testutil import TOL, TORCH_IO, assert_io_output, dev, gates_f32, host, rel_err_blocks

pytestmark = pytest.mark.gpu


def _case(io, B=6, H=4, K=64, V=64, n_slots=9, seed=0, Tv=None, regime="config"):
    c = kda_synth.decode_case(B, H, K, V, n_slots, io, seed=seed, regime=regime, Tv=Tv,
                              n_padding=1)
    return c


def _t(c):
    io = TORCH_IO[c["io"]]
    return {x: dev(c[x], io) for x in "qkv"}


def test_no_options_is_the_plain_step():
    for io in ("f32", "bf16"):
        c = _case(io, seed=1)
        t = _t(c)
        g, beta = gates_f32(c["a"], c["b"], c["A_log"], c["dt_bias"])
        pa, pb = dev(c["pool"]), dev(c["pool"])
        idx = dev(c["slot_idx"], torch.int32)
        o1 = kda.kda_recurrent_decode(t["q"], t["k"], t["v"], dev(g), dev(beta), 0.125, pa, idx)
        o2 = kda.kda_recurrent_decode_ex(t["q"], t["k"], t["v"], dev(g), dev(beta), 0.125, pb,
                                         idx)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(pa, pb)


@pytest.mark.parametrize("lb", [0.0, -5.0])
def test_raw_gate_in_decode_equals_gate_prep_then_decode(lb):
    c = _case("bf16", K=128, V=128, seed=2)
    t = _t(c)
    a, b = dev(c["a"]), dev(c["b"])
    A_log, dtb = dev(c["A_log"]), dev(c["dt_bias"])
    g, beta = kda.kda_gate_prep(a, b, A_log, dtb, lower_bound=lb)
    pa, pb = dev(c["pool"]), dev(c["pool"])
    idx = dev(c["slot_idx"], torch.int32)
    o1 = kda.kda_recurrent_decode(t["q"], t["k"], t["v"], g, beta, 0.09, pa, idx)
    o2 = kda.kda_recurrent_decode_ex(t["q"], t["k"], t["v"], a, b, 0.09, pb, idx,
                                     raw_gate=(A_log, dtb, lb))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(pa, pb)


def test_per_head_gate_equals_broadcast_gate():
    # the Gated DeltaNet gate: one decay per head, shared by every key channel
    c = _case("bf16", K=64, V=128, seed=3)
    t = _t(c)
    B, H, K = c["B"], c["H"], c["K"]
    r = np.random.default_rng(3)
    a_h = r.standard_normal((B, H)).astype(np.float32)
    dtb_h = (0.5 * r.standard_normal(H)).astype(np.float32)
    A_log = dev(c["A_log"])
    b = dev(c["b"])
    idx = dev(c["slot_idx"], torch.int32)
    # activated per-head g against the same g broadcast over K
    g_h = -np.abs(a_h)
    pa, pb = dev(c["pool"]), dev(c["pool"])
    o1 = kda.kda_recurrent_decode_ex(t["q"], t["k"], t["v"], dev(np.repeat(g_h[..., None], K, 2)),
                                     b, 0.1, pa, idx)
    o2 = kda.kda_recurrent_decode_ex(t["q"], t["k"], t["v"], dev(g_h), b, 0.1, pb, idx,
                                     per_head_gate=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(pa, pb)
    # raw per-head gate (a [B,H], dt_bias [H]) against the per-channel raw gate
    pa, pb = dev(c["pool"]), dev(c["pool"])
    o1 = kda.kda_recurrent_decode_ex(t["q"], t["k"], t["v"], dev(np.repeat(a_h[..., None], K, 2)),
                                     b, 0.1, pa, idx,
                                     raw_gate=(A_log, dev(np.repeat(dtb_h[:, None], K, 1)), 0.0))
    o2 = kda.kda_recurrent_decode_ex(t["q"], t["k"], t["v"], dev(a_h), b, 0.1, pb, idx,
                                     raw_gate=(A_log, dev(dtb_h), 0.0), per_head_gate=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(pa, pb)


def test_grouped_qk_heads_equal_repeated_heads():
    c = _case("bf16", H=8, K=128, V=64, seed=4)
    B, H, K = c["B"], c["H"], c["K"]
    io = TORCH_IO["bf16"]
    qg, kg = c["q"][:, :2], c["k"][:, :2]  # 2 q/k heads for 8 value heads
    rep = lambda x: np.repeat(x, 4, axis=1)
    g, beta = gates_f32(c["a"], c["b"], c["A_log"], c["dt_bias"])
    idx = dev(c["slot_idx"], torch.int32)
    pa, pb = dev(c["pool"]), dev(c["pool"])
    o1 = kda.kda_recurrent_decode(dev(rep(qg), io), dev(rep(kg), io), dev(c["v"], io), dev(g),
                                  dev(beta), 0.1, pa, idx)
    o2 = kda.kda_recurrent_decode_ex(dev(qg, io), dev(kg, io), dev(c["v"], io), dev(g), dev(beta),
                                     0.1, pb, idx)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(pa, pb)


def _raw_qk(c, seed):
    """Un-normalised q and k of the case's shape, rounded to its io dtype."""
    r = np.random.default_rng(seed)
    q = r.standard_normal(c["q"].shape) * 0.7
    k = r.standard_normal(c["k"].shape) * 1.3
    rt = lambda x: torch.from_numpy(x).to(TORCH_IO[c["io"]]).to(torch.float64).numpy()
    return rt(q), rt(k)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("act", ["sigmoid", "silu"])
def test_l2norm_and_output_norm_match_oracle(io, act):
    c = _case(io, K=128, V=128, seed=5, regime="long")
    B, H, K, V = c["B"], c["H"], c["K"], c["V"]
    q, k = _raw_qk(c, 5)
    r = np.random.default_rng(6)
    z = torch.from_numpy(r.standard_normal((B, H, V))).to(TORCH_IO[io])
    w = (1.0 + 0.1 * r.standard_normal(V)).astype(np.float32)
    g, beta = gates_f32(c["a"], c["b"], c["A_log"], c["dt_bias"])
    pool = dev(c["pool"])
    idx = dev(c["slot_idx"], torch.int32)
    o = kda.kda_recurrent_decode_ex(dev(q, TORCH_IO[io]), dev(k, TORCH_IO[io]),
                                    dev(c["v"], TORCH_IO[io]), dev(g), dev(beta), K ** -0.5, pool,
                                    idx, qk_l2norm=True, o_gate=z.cuda(), o_norm_w=dev(w),
                                    o_norm_eps=1e-6, o_gate_act=act)
    torch.cuda.synchronize()
    o_ref, pool_ref = oracle.decode(oracle.l2norm(q), oracle.l2norm(k), c["v"], g, beta,
                                    K ** -0.5, c["pool"], c["slot_idx"])
    o_ref = oracle.gated_rmsnorm(o_ref, z.to(torch.float64).numpy(), w, 1e-6, act)
    live = c["slot_idx"] >= 0
    assert_io_output(host(o)[live], o_ref[live], io, 1)
    np.testing.assert_array_equal(host(o)[~live], 0.0)
    lv = c["slot_idx"][live]
    assert rel_err_blocks(host(pool)[lv], pool_ref[lv], 2) <= TOL[io]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("Tv", [5, 11])
def test_verify_with_every_option(io, Tv):
    # raw safe gate, grouped heads, in-kernel L2 norm and the output norm,
    # against the oracle, and each step against the same options in decode;
    # 11 draft tokens span two staged batches of 8, the second ragged
    B, H, HK, K, V = 4, 4, 2, 64, 64
    c = _case(io, B=B, H=H, K=K, V=V, seed=7, Tv=Tv, regime="long")
    q, k = _raw_qk(c, 7)
    q, k = q[:, :, :HK], k[:, :, :HK]
    r = np.random.default_rng(8)
    z = r.standard_normal((B, Tv, H, V))
    z = torch.from_numpy(z).to(TORCH_IO[io])
    w = (1.0 + 0.1 * r.standard_normal(V)).astype(np.float32)
    lb = -4.0
    A_log, dtb = dev(c["A_log"]), dev(c["dt_bias"])
    io_t = TORCH_IO[io]
    qd, kd, vd = dev(q, io_t), dev(k, io_t), dev(c["v"], io_t)
    ad, bd = dev(c["a"]), dev(c["b"])
    pool = dev(c["pool"])
    idx = dev(c["slot_idx"], torch.int32)
    opts = dict(raw_gate=(A_log, dtb, lb), qk_l2norm=True, o_gate=z.cuda(), o_norm_w=dev(w),
                o_norm_eps=1e-6, o_gate_act="sigmoid")
    o, inter = kda.kda_verify_ex(qd, kd, vd, ad, bd, K ** -0.5, pool, idx, **opts)
    torch.cuda.synchronize()
    # oracle: gates, normalised q/k repeated over the value heads, recurrence, output norm
    g, beta = oracle.gate(c["a"].reshape(B * Tv, H, K), c["b"].reshape(B * Tv, H), c["A_log"],
                          c["dt_bias"], lb)
    g, beta = g.reshape(B, Tv, H, K), beta.reshape(B, Tv, H)
    rep = lambda x: np.repeat(x, H // HK, axis=2)
    o_ref, inter_ref = oracle.verify(rep(oracle.l2norm(q)), rep(oracle.l2norm(k)), c["v"], g, beta,
                                     K ** -0.5, c["pool"], c["slot_idx"])
    o_ref = oracle.gated_rmsnorm(o_ref, z.to(torch.float64).numpy(), w, 1e-6)
    live = c["slot_idx"] >= 0
    assert_io_output(host(o)[live], o_ref[live], io, 1)
    assert rel_err_blocks(host(inter)[live], inter_ref[live], 2) <= TOL[io]
    # every step equals the decode with the same options
    pool2 = dev(c["pool"])
    for s in range(Tv):
        sl = lambda x: x[:, s].contiguous()
        o_d = kda.kda_recurrent_decode_ex(sl(qd), sl(kd), sl(vd), sl(ad), sl(bd), K ** -0.5, pool2,
                                          idx, raw_gate=(A_log, dtb, lb), qk_l2norm=True,
                                          o_gate=sl(z.cuda()), o_norm_w=dev(w), o_norm_eps=1e-6)
        assert torch.equal(o_d, o[:, s]), s
        lvt = torch.from_numpy(live).cuda()
        assert torch.equal(pool2[idx[lvt].long()], inter[lvt, s]), s


# ------------------------------------------------------------- prefill

def _prefill_case(io, seqlens=(200, 64, 5, 130), H=4, K=64, V=64, seed=11):
    return kda_synth.prefill_case(list(seqlens), H, K, V, io, seed=seed, regime="long",
                                  h0_std=0.02)


def _pt(c):
    io = TORCH_IO[c["io"]]
    return {x: dev(c[x], io) for x in "qkv"}, dev(c["cu"], torch.int32), dev(c["h0"])


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [16, 64])
def test_prefill_per_head_gate_equals_broadcast_gate(io, chunk):
    c = _prefill_case(io)
    t, cu, h0 = _pt(c)
    T, H, K = c["q"].shape
    r = np.random.default_rng(12)
    a_h = r.standard_normal((T, H)).astype(np.float32)
    dtb_h = (0.5 * r.standard_normal(H) - 6.0).astype(np.float32)  # slow decay
    A_log, b = dev(c["A_log"]), dev(c["b"])
    g_h = -0.05 * np.abs(a_h)
    bc = lambda x: dev(np.repeat(x[..., None], K, -1))
    beta = torch.sigmoid(b)
    o1, h1 = kda.kda_chunk_prefill(t["q"], t["k"], t["v"], bc(g_h), beta, cu, 0.1, h0=h0,
                                   chunk=chunk)
    o2, h2 = kda.kda_chunk_prefill_ex(t["q"], t["k"], t["v"], dev(g_h), beta, cu, 0.1, h0=h0,
                                      chunk=chunk, per_head_gate=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    # raw per-head gate against the per-channel raw gate of the broadcast inputs
    o1, h1 = kda.kda_chunk_prefill_ex(t["q"], t["k"], t["v"], bc(a_h), b, cu, 0.1, h0=h0,
                                      chunk=chunk, raw_gate=(A_log, bc(dtb_h), 0.0))
    o2, h2 = kda.kda_chunk_prefill_ex(t["q"], t["k"], t["v"], dev(a_h), b, cu, 0.1, h0=h0,
                                      chunk=chunk, raw_gate=(A_log, dev(dtb_h), 0.0),
                                      per_head_gate=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    # and the per-head gate against the oracle (the Gated DeltaNet case)
    g_ref, beta_ref = oracle.gate(np.repeat(a_h[..., None], K, -1), c["b"], c["A_log"],
                                  np.repeat(dtb_h[:, None], K, 1))
    o_ref, ht_ref = oracle.prefill(c["q"], c["k"], c["v"], g_ref, beta_ref, c["cu"], 0.1,
                                   c["h0"])
    assert_io_output(host(o2), o_ref, io, 1)
    assert rel_err_blocks(host(h2), ht_ref, 2) <= TOL[io]


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefill_grouped_qk_heads_equal_repeated_heads(io):
    c = _prefill_case(io, H=8, K=64, V=64, seed=13)
    t, cu, h0 = _pt(c)
    iot = TORCH_IO[io]
    g, beta = gates_f32(c["a"], c["b"], c["A_log"], c["dt_bias"])
    qg, kg = c["q"][:, :2], c["k"][:, :2]  # 2 q/k heads for 8 value heads
    rep = lambda x: np.repeat(x, 4, axis=1)
    o1, h1 = kda.kda_chunk_prefill(dev(rep(qg), iot), dev(rep(kg), iot), t["v"], dev(g),
                                   dev(beta), cu, 0.125, h0=h0)
    o2, h2 = kda.kda_chunk_prefill_ex(dev(qg, iot), dev(kg, iot), t["v"], dev(g), dev(beta), cu,
                                      0.125, h0=h0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_prefill_options_snapshots_equal_snapshot_entry_point():
    c = _prefill_case("bf16", seqlens=(384, 130, 256), seed=14)
    t, cu, h0 = _pt(c)
    g, beta = gates_f32(c["a"], c["b"], c["A_log"], c["dt_bias"])
    s1 = torch.zeros((12, 4, 64, 64), device="cuda")
    s2 = torch.zeros_like(s1)
    o1, h1, _ = kda.kda_chunk_prefill_snapshots(t["q"], t["k"], t["v"], dev(g), dev(beta), cu,
                                                0.1, 128, h0=h0, snapshots=s1)
    o2, h2 = kda.kda_chunk_prefill_ex(t["q"], t["k"], t["v"], dev(g), dev(beta), cu, 0.1, h0=h0,
                                      snapshots=s2, snapshot_interval=128)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2) and torch.equal(s1, s2)


# ---------------------------------------------- in-kernel L2 norm in prefill

@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("D,chunk", [(128, 64), (64, 32), (32, 64), (16, 16)])
def test_prefill_l2norm_matches_oracle(io, D, chunk):
    """Un-normalised q and k, normalised in the kernel: the oracle runs on
    l2norm(q), l2norm(k) (fp64, eps 1e-6)."""
    c = _prefill_case(io, seqlens=(200, 64, 5, 130), K=D, V=D, seed=21)
    q, k = _raw_qk(c, 21)
    iot = TORCH_IO[io]
    g, beta = gates_f32(c["a"], c["b"], c["A_log"], c["dt_bias"])
    o, ht = kda.kda_chunk_prefill_ex(dev(q, iot), dev(k, iot), dev(c["v"], iot), dev(g),
                                     dev(beta), dev(c["cu"], torch.int32), D ** -0.5,
                                     h0=dev(c["h0"]), chunk=chunk, qk_l2norm=True)
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.prefill(oracle.l2norm(q), oracle.l2norm(k), c["v"], g, beta,
                                   c["cu"], D ** -0.5, c["h0"])
    assert_io_output(host(o), o_ref, io, 1)
    assert rel_err_blocks(host(ht), ht_ref, 2) <= TOL[io]


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefill_l2norm_with_grouped_heads_and_raw_gate(io):
    """Every prefill option at once: 2 q/k heads for 8 value heads, the
    softplus gate from raw a and b, and the in-kernel L2 norm."""
    c = _prefill_case(io, seqlens=(150, 1, 64, 97), H=8, K=64, V=64, seed=22)
    q, k = _raw_qk(c, 22)
    qg, kg = q[:, :2], k[:, :2]
    iot = TORCH_IO[io]
    o, ht = kda.kda_chunk_prefill_ex(dev(qg, iot), dev(kg, iot), dev(c["v"], iot),
                                     dev(c["a"]), dev(c["b"]), dev(c["cu"], torch.int32), 0.125,
                                     h0=dev(c["h0"]), chunk=32, qk_l2norm=True,
                                     raw_gate=(dev(c["A_log"]), dev(c["dt_bias"]), 0.0))
    torch.cuda.synchronize()
    g_ref, b_ref = oracle.gate(c["a"], c["b"], c["A_log"], c["dt_bias"])
    rep = lambda x: np.repeat(oracle.l2norm(x), 4, axis=1)
    o_ref, ht_ref = oracle.prefill(rep(qg), rep(kg), c["v"], g_ref, b_ref, c["cu"], 0.125,
                                   c["h0"])
    assert_io_output(host(o), o_ref, io, 1)
    assert rel_err_blocks(host(ht), ht_ref, 2) <= TOL[io]


def test_prefill_l2norm_varlen_workload_sampled_heads():
    """The varlen batch's shape ({512, 1024, 2048, 4096}, H = 32, K = V = 128,
    bf16, chunk 64, slow decay) with raw q and k, checked on three heads."""
    w = kda_synth.WORKLOADS["varlen_prefill_7680"]
    c = kda_synth.prefill_case(w["seqlens"], w["H"], w["K"], w["V"], "bf16", seed=23,
                               regime="long", dt_bias_std=w["dt_bias_std"], h0_std=w["h0_std"])
    q, k = _raw_qk(c, 23)
    g, beta = gates_f32(c["a"], c["b"], c["A_log"], c["dt_bias"])
    bf = torch.bfloat16
    o, ht = kda.kda_chunk_prefill_ex(dev(q, bf), dev(k, bf), dev(c["v"], bf), dev(g), dev(beta),
                                     dev(c["cu"], torch.int32), w["K"] ** -0.5,
                                     h0=dev(c["h0"]), chunk=w["chunk"], qk_l2norm=True)
    torch.cuda.synchronize()
    heads = [0, 17, 31]
    sub = lambda x: np.ascontiguousarray(x[:, heads])
    o_ref, ht_ref = oracle.prefill(oracle.l2norm(sub(q)), oracle.l2norm(sub(k)), sub(c["v"]),
                                   sub(g), sub(beta), c["cu"], w["K"] ** -0.5, sub(c["h0"]))
    assert_io_output(host(o)[:, heads], o_ref, "bf16", 1)
    assert rel_err_blocks(host(ht)[:, heads], ht_ref, 2) <= TOL["bf16"]
