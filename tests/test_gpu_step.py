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
