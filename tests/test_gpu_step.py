"""GPU parity of gate prep, recurrent decode and verify against the oracle.

Every comparison runs the HIP path through the C ABI (via the thin binding)
and the fp64 oracle on the same seeded inputs; the oracle also supplies the
activated gates both sides consume (gates rounded to fp32).
"""
import numpy as np
import pytest
import torch

import kda_gated_delta_amd as kda
import kda_synth
import oracle
from kda_testutil import (TOL, TORCH_IO, assert_io_output, dev, gates_f32, host,
                          rel_err_blocks)

pytestmark = pytest.mark.gpu


def _scale(K):
    return K ** -0.5


# ------------------------------------------------------------------ gate

def _assert_gate_close(g, g_ref, a, dt_bias, A_log):
    """fp32 evaluation: the argument x = a + dt_bias and exp(A_log) * x are
    rounded to fp32, an error the gate amplifies by up to |exp(A_log) x|
    (its condition number); exp/log1p/division add a few ulp."""
    x = a.astype(np.float64) + (0.0 if dt_bias is None else dt_bias.astype(np.float64))
    arg = np.abs(np.exp(A_log.astype(np.float64))[:, None] * x)
    rtol = 2.0 ** -22 * (4.0 + arg)
    err = np.abs(g - g_ref)
    bad = err > rtol * np.abs(g_ref) + 1e-37
    assert not bad.any(), (err[bad][:5], g_ref[bad][:5])

@pytest.mark.parametrize("lower_bound", [0.0, -5.0])
def test_gate_prep_matches_oracle(lower_bound):
    w = kda_synth.WORKLOADS["varlen_prefill_7680"]
    c = kda_synth.prefill_case(w["seqlens"], w["H"], w["K"], w["V"], "bf16",
                               seed=w["seed"], h0_std=None)
    g_ref, b_ref = oracle.gate(c["a"], c["b"], c["A_log"], c["dt_bias"], lower_bound)
    g, beta = kda.kda_gate_prep(dev(c["a"]), dev(c["b"]), dev(c["A_log"]),
                                dev(c["dt_bias"]), lower_bound=lower_bound)
    torch.cuda.synchronize()
    g, beta = host(g), host(beta)
    _assert_gate_close(g, g_ref, c["a"], c["dt_bias"], c["A_log"])
    np.testing.assert_allclose(beta, b_ref, rtol=2e-6, atol=1e-30)


def test_gate_prep_edge_values_and_no_bias():
    # around the softplus threshold, far negative, large positive
    x = np.array([-100.0, -30.0, -1.0, 0.0, 19.99, 20.0, 20.01, 60.0], dtype=np.float32)
    a = np.tile(x, (5, 3, 2)).reshape(5, 3, 16).astype(np.float32)
    b = np.linspace(-30, 30, 15, dtype=np.float32).reshape(5, 3)
    A_log = np.array([0.0, 1.0, -2.0], dtype=np.float32)
    g_ref, b_ref = oracle.gate(a, b, A_log, None)
    g, beta = kda.kda_gate_prep(dev(a), dev(b), dev(A_log), None)
    torch.cuda.synchronize()
    _assert_gate_close(host(g), g_ref, a, None, A_log)
    np.testing.assert_allclose(host(beta), b_ref, rtol=2e-6, atol=1e-37)


# ---------------------------------------------------------------- decode

def _decode_inputs(c):
    g, beta = gates_f32(c["a"], c["b"], c["A_log"], c["dt_bias"])
    io = TORCH_IO[c["io"]]
    return dict(q=dev(c["q"], io), k=dev(c["k"], io), v=dev(c["v"], io), g=dev(g),
                beta=dev(beta)), g, beta


def _check_decode(c, steps=1):
    t, g, beta = _decode_inputs(c)
    K = c["K"]
    pool_d = dev(c["pool"])
    idx_d = dev(c["slot_idx"], torch.int32)
    pool_ref = c["pool"]
    tol = TOL[c["io"]]
    for _ in range(steps):
        o = kda.kda_recurrent_decode(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                     _scale(K), pool_d, idx_d)
        o_ref, pool_ref = oracle.decode(c["q"], c["k"], c["v"], g, beta, _scale(K),
                                        pool_ref, c["slot_idx"])
        torch.cuda.synchronize()
        assert_io_output(host(o), o_ref, c["io"], 1)
    pool = host(pool_d)
    live = c["slot_idx"][c["slot_idx"] >= 0]
    assert rel_err_blocks(pool[live], pool_ref[live], 2) <= tol
    dead = np.setdiff1d(np.arange(c["n_slots"]), live)
    np.testing.assert_array_equal(pool[dead], c["pool"][dead])  # untouched slots
    pad = c["slot_idx"] < 0
    if pad.any():
        np.testing.assert_array_equal(host(o)[pad], 0.0)


def test_decode_full_workload():
    w = kda_synth.WORKLOADS["decode_256"]
    c = kda_synth.decode_case(w["B"], w["H"], w["K"], w["V"], w["n_slots"], w["io"],
                              seed=w["seed"], dt_bias_std=w["dt_bias_std"],
                              state_std=w["state_std"])
    _check_decode(c)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("KV", [(16, 16), (32, 64), (64, 32), (128, 16), (16, 128), (128, 128)])
def test_decode_shapes(io, KV):
    K, V = KV
    c = kda_synth.decode_case(7, 3, K, V, n_slots=11, io=io, seed=K + V, n_padding=2)
    _check_decode(c, steps=3)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_long_memory_many_steps(io):
    c = kda_synth.decode_case(5, 4, 128, 128, n_slots=9, io=io, seed=21, regime="long")
    _check_decode(c, steps=12)


def test_pool_past_4gib_byte_offsets():
    """A 3000-slot pool at H = 32, K = V = 128 (6.3 GB, slot s at s x 2 MiB):
    decode, then verify, on slots past 4 GiB and near the start, against the
    oracle on copies of those slots; every other slot is left as it was."""
    H, K, V, n_pool = 32, 128, 128, 3000
    big = np.array([2999, 2048, 2500, 7, 2047, 2990, 0, 2049, 1500, 2995, 12, 2400])
    assert big.max() * H * K * V * 4 > (1 << 32)
    big_d = torch.from_numpy(big).cuda()
    c = kda_synth.decode_case(10, H, K, V, n_slots=len(big), io="bf16", seed=33, n_padding=1)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(34)
    pool = torch.empty((n_pool, H, K, V), device="cuda").normal_(0.0, 0.02, generator=gen)
    pool[big_d] = dev(c["pool"])  # the case's compact pool at the mapped slots
    before = pool.clone()
    to_big = lambda idx: np.where(idx >= 0, big[np.maximum(idx, 0)], -1).astype(np.int32)
    t, g, beta = _decode_inputs(c)
    o = kda.kda_recurrent_decode(t["q"], t["k"], t["v"], t["g"], t["beta"], _scale(K), pool,
                                 dev(to_big(c["slot_idx"]), torch.int32))
    o_ref, pool_ref = oracle.decode(c["q"], c["k"], c["v"], g, beta, _scale(K), c["pool"],
                                    c["slot_idx"])
    torch.cuda.synchronize()
    assert_io_output(host(o), o_ref, "bf16", 1)
    live = c["slot_idx"][c["slot_idx"] >= 0]
    live_d = torch.from_numpy(big[live]).cuda()
    assert rel_err_blocks(host(pool[live_d]), pool_ref[live], 2) <= TOL["bf16"]
    others = torch.ones(n_pool, dtype=torch.bool, device="cuda")
    others[live_d] = False
    assert torch.equal(pool[others], before[others])
    del before
    # verify from the updated pool: read only, each step against the oracle
    cv = kda_synth.decode_case(10, H, K, V, n_slots=len(big), io="bf16", seed=35, Tv=4,
                               n_padding=1)
    tv, gv, betav = _verify_inputs(cv)
    compact = host(pool[big_d]).astype(np.float32)
    before = pool.clone()
    inter = torch.full((10, 4, H, K, V), float("nan"), device="cuda")
    ov, inter = kda.kda_verify(tv["q"], tv["k"], tv["v"], tv["g"], tv["beta"], _scale(K), pool,
                               dev(to_big(cv["slot_idx"]), torch.int32), inter_states=inter)
    torch.cuda.synchronize()
    assert torch.equal(pool, before)
    ov_ref, inter_ref = oracle.verify(cv["q"], cv["k"], cv["v"], gv, betav, _scale(K), compact,
                                      cv["slot_idx"])
    lv = cv["slot_idx"] >= 0
    assert_io_output(host(ov)[lv], ov_ref[lv], "bf16", 1)
    assert rel_err_blocks(host(inter)[lv], inter_ref[lv], 2) <= TOL["bf16"]
    del pool, before, inter
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- verify

def _verify_inputs(c):
    B, Tv, H, K = c["q"].shape
    g, beta = gates_f32(c["a"], c["b"], c["A_log"], c["dt_bias"])
    io = TORCH_IO[c["io"]]
    return dict(q=dev(c["q"], io), k=dev(c["k"], io), v=dev(c["v"], io), g=dev(g),
                beta=dev(beta)), g, beta


def _check_verify(c, against_decode=True):
    t, g, beta = _verify_inputs(c)
    B, Tv, H, K = c["q"].shape
    pool_d = dev(c["pool"])
    idx_d = dev(c["slot_idx"], torch.int32)
    pool_before = pool_d.clone()
    inter_d = torch.full((B, Tv, H, K, c["V"]), float("nan"), device="cuda")
    o, inter = kda.kda_verify(t["q"], t["k"], t["v"], t["g"], t["beta"], _scale(K),
                              pool_d, idx_d, inter_states=inter_d)
    torch.cuda.synchronize()
    assert torch.equal(pool_d, pool_before)  # the pool is never written
    o_ref, inter_ref = oracle.verify(c["q"], c["k"], c["v"], g, beta, _scale(K),
                                     c["pool"], c["slot_idx"])
    tol = TOL[c["io"]]
    live = c["slot_idx"] >= 0
    assert_io_output(host(o)[live], o_ref[live], c["io"], 1)
    assert rel_err_blocks(host(inter)[live], inter_ref[live], 2) <= tol
    if (~live).any():
        np.testing.assert_array_equal(host(o)[~live], 0.0)
        assert torch.isnan(inter[torch.from_numpy(~live).cuda()]).all()  # not written
    if against_decode:
        # each verify step equals the same number of sequential decode calls
        pool2 = pool_d.clone()
        for s in range(Tv):
            o_d = kda.kda_recurrent_decode(
                t["q"][:, s].contiguous(), t["k"][:, s].contiguous(),
                t["v"][:, s].contiguous(), t["g"][:, s].contiguous(),
                t["beta"][:, s].contiguous(), _scale(K), pool2, idx_d)
            assert torch.equal(o_d, o[:, s]), s
            lv = torch.from_numpy(live).cuda()
            assert torch.equal(pool2[idx_d[lv].long()], inter[lv, s]), s


def test_verify_full_workload():
    w = kda_synth.WORKLOADS["verify_64x8"]
    c = kda_synth.decode_case(w["B"], w["H"], w["K"], w["V"], w["n_slots"], w["io"],
                              seed=w["seed"], dt_bias_std=w["dt_bias_std"],
                              state_std=w["state_std"], Tv=w["Tv"])
    _check_verify(c)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("Tv", [1, 3, 8, 11, 17])
def test_verify_draft_lengths(io, Tv):
    c = kda_synth.decode_case(6, 2, 64, 64, n_slots=9, io=io, seed=100 + Tv, Tv=Tv,
                              n_padding=1)
    _check_verify(c)


@pytest.mark.parametrize("KV", [(16, 16), (32, 128), (128, 32)])
def test_verify_shapes_long_memory(KV):
    K, V = KV
    c = kda_synth.decode_case(4, 3, K, V, n_slots=5, io="f32", seed=7, Tv=6, regime="long")
    _check_verify(c)


# ------------------------------------------- caller errors in device arrays

def _step_case(io="bf16", B=5, n_slots=6, Tv=None):
    c = kda_synth.decode_case(B, 2, 64, 64, n_slots, io, seed=91, Tv=Tv)
    lead = (B,) if Tv is None else (B * Tv,)
    g, beta = gates_f32(c["a"].reshape(lead + (2, 64)), c["b"].reshape(lead + (2,)),
                        c["A_log"], c["dt_bias"])
    shp = (B,) if Tv is None else (B, Tv)
    c["g"], c["beta"] = g.reshape(shp + (2, 64)), beta.reshape(shp + (2,))
    return c


def test_slot_past_the_pool_gives_nan_and_touches_nothing():
    """A live slot index >= n_slots is caught by the kernels' own bounds:
    that row's o is NaN, no state is read or written, and the other rows are
    computed as usual (decode, verify and the buffered decode)."""
    io = TORCH_IO["bf16"]
    c = _step_case()
    idx = c["slot_idx"].copy()
    idx[2] = c["n_slots"]  # one past the pool
    q, k, v = (dev(c[x], io) for x in "qkv")
    g, beta = dev(c["g"]), dev(c["beta"])
    pool = dev(c["pool"])
    o = kda.kda_recurrent_decode(q, k, v, g, beta, 0.125, pool, dev(idx, torch.int32))
    ref_pool = dev(c["pool"])
    o_ok = kda.kda_recurrent_decode(q, k, v, g, beta, 0.125, ref_pool,
                                    dev(c["slot_idx"], torch.int32))
    torch.cuda.synchronize()
    assert torch.isnan(o[2]).all()
    keep = [0, 1, 3, 4]
    assert torch.equal(o[keep], o_ok[keep])
    # the pool differs from the valid call only in the slot row 2 would have used
    s2 = int(c["slot_idx"][2])
    others = [s for s in range(c["n_slots"]) if s != s2]
    assert torch.equal(pool[others], ref_pool[others])
    assert torch.equal(pool[s2], dev(c["pool"])[s2])
    # verify: o NaN for the row, inter left as it was, pool untouched
    cv = _step_case(Tv=3)
    inter = torch.full((5, 3, 2, 64, 64), 7.0, device="cuda")
    pv = dev(cv["pool"])
    ov, inter = kda.kda_verify(*(dev(cv[x], io) for x in "qkv"), dev(cv["g"]), dev(cv["beta"]),
                               0.125, pv, dev(idx, torch.int32), inter_states=inter)
    torch.cuda.synchronize()
    assert torch.isnan(ov[2]).all() and (inter[2] == 7.0).all()
    assert torch.equal(pv, dev(cv["pool"]))
    # buffered decode: o NaN, cursor kept, pool and ring untouched
    ring = (torch.zeros((6, 2, 4, 64), device="cuda"),
            torch.zeros((6, 2, 4, 64), dtype=io, device="cuda"),
            torch.zeros((6, 2, 4, 64), device="cuda"))
    pos = torch.tensor([0, 1, 2, 3, 0], dtype=torch.int32, device="cuda")
    pr = dev(c["pool"])
    orp, nxt = kda.kda_replay_decode(q, k, v, g, beta, 0.125, pr, dev(idx, torch.int32), pos,
                                     *ring)
    torch.cuda.synchronize()
    assert torch.isnan(orp[2]).all() and int(nxt[2]) == 2
    assert torch.equal(pr[s2], dev(c["pool"])[s2])


def test_debug_checks_reject_bad_device_arrays(monkeypatch):
    """KDA_CHECK=1: bad cu_seqlens, slots past the pool, duplicate live slots
    and ring cursors outside the ring are rejected before anything runs; good
    arrays give the same results as without the checks."""
    io = TORCH_IO["bf16"]
    c = _step_case()
    q, k, v = (dev(c[x], io) for x in "qkv")
    g, beta = dev(c["g"]), dev(c["beta"])
    pool = dev(c["pool"])
    good = dev(c["slot_idx"], torch.int32)
    o_ref = kda.kda_recurrent_decode(q, k, v, g, beta, 0.125, dev(c["pool"]), good)
    monkeypatch.setenv("KDA_CHECK", "1")
    for bad in ([0, 1, 6, 2, 3], [0, 1, 1, 2, 3]):  # past the pool; slot 1 twice
        with pytest.raises(kda.KdaError) as e:
            kda.kda_recurrent_decode(q, k, v, g, beta, 0.125, pool,
                                     torch.tensor(bad, dtype=torch.int32, device="cuda"))
        assert e.value.status == 1
        with pytest.raises(kda.KdaError):
            kda.kda_verify(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None], 0.125,
                           pool, torch.tensor(bad, dtype=torch.int32, device="cuda"))
    assert torch.equal(pool, dev(c["pool"]))  # nothing ran
    o = kda.kda_recurrent_decode(q, k, v, g, beta, 0.125, pool, good)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    ring = (torch.zeros((6, 2, 4, 64), device="cuda"),
            torch.zeros((6, 2, 4, 64), dtype=io, device="cuda"),
            torch.zeros((6, 2, 4, 64), device="cuda"))
    with pytest.raises(kda.KdaError):
        kda.kda_replay_decode(q, k, v, g, beta, 0.125, pool, good,
                              torch.tensor([0, 1, 4, 0, 0], dtype=torch.int32, device="cuda"),
                              *ring)
    # prefill: cu must start at 0, end at T and never decrease
    pc = kda_synth.prefill_case([20, 12], 2, 64, 64, "bf16", seed=92)
    gp, bp = gates_f32(pc["a"], pc["b"], pc["A_log"], pc["dt_bias"])
    args = [dev(pc[x], io) for x in "qkv"] + [dev(gp), dev(bp)]
    for cu in ([0, 20, 31], [1, 20, 32], [0, 21, 20]):
        with pytest.raises(kda.KdaError):
            kda.kda_chunk_prefill(*args, torch.tensor(cu, dtype=torch.int32, device="cuda"), 0.125)
    o1, h1 = kda.kda_chunk_prefill(*args, dev(pc["cu"], torch.int32), 0.125)
    monkeypatch.delenv("KDA_CHECK")
    o2, h2 = kda.kda_chunk_prefill(*args, dev(pc["cu"], torch.int32), 0.125)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
