"""Buffered ("replay") decode, kda_replay_decode ("ReplaySSM" analysis,
sections 2 and 3): against the plain decode kernel bit for bit where the ring
is empty, and against the oracle's token-by-token decode over many steps
with rings, flushes at the ring's end and forced flushes."""
import numpy as np
import pytest
import torch

import kda_gated_delta_amd as kda
import kda_synth
import oracle
from kda_testutil import TOL, TORCH_IO, assert_io_output, dev, gates_f32, host, rel_err_blocks

pytestmark = pytest.mark.gpu


def _scale(K):
    return K ** -0.5


def _case(B, H, K, V, n_slots, io, seed, steps, regime="config", n_padding=0):
    """decode_case with `steps` tokens per request ([B, steps, ...])."""
    c = kda_synth.decode_case(B, H, K, V, n_slots, io, seed=seed, regime=regime,
                              Tv=steps, n_padding=n_padding)
    g, beta = gates_f32(c["a"].reshape(B * steps, H, K), c["b"].reshape(B * steps, H),
                        c["A_log"], c["dt_bias"])
    c["g"], c["beta"] = g.reshape(B, steps, H, K), beta.reshape(B, steps, H)
    return c


def _step_inputs(c, s):
    io = TORCH_IO[c["io"]]
    return (dev(c["q"][:, s], io), dev(c["k"][:, s], io), dev(c["v"][:, s], io),
            dev(c["g"][:, s]), dev(c["beta"][:, s]))


def _rings(c, L):
    """Rings filled with NaN: an entry read before it was written shows."""
    n, H, K, V = c["n_slots"], c["H"], c["K"], c["V"]
    return (torch.full((n, H, L, V), float("nan"), device="cuda"),
            torch.full((n, H, L, K), float("nan"), dtype=TORCH_IO[c["io"]], device="cuda"),
            torch.full((n, H, L, K), float("nan"), device="cuda"))


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("KV", [(16, 16), (64, 32), (128, 128)])
def test_ring_of_one_is_the_plain_decode_bit_for_bit(io, KV):
    # L = 1: every step writes the checkpoint and the ring stays empty
    K, V = KV
    steps = 4
    c = _case(6, 3, K, V, 9, io, seed=K + V, steps=steps, n_padding=1)
    pool_a, pool_b = dev(c["pool"]), dev(c["pool"])
    idx = dev(c["slot_idx"], torch.int32)
    pos = torch.zeros(6, dtype=torch.int32, device="cuda")
    rd, rk, rg = _rings(c, 1)
    for s in range(steps):
        q, k, v, g, beta = _step_inputs(c, s)
        o_a = kda.kda_recurrent_decode(q, k, v, g, beta, _scale(K), pool_a, idx)
        o_b, nxt = kda.kda_replay_decode(q, k, v, g, beta, _scale(K), pool_b, idx, pos,
                                         rd, rk, rg)
        torch.cuda.synchronize()
        assert torch.equal(o_a, o_b), s
        assert torch.equal(pool_a, pool_b), s
        assert host(nxt).tolist() == [0] * 6  # flushed rows reset, padding keeps 0
    assert torch.isnan(rd).all() and torch.isnan(rg).all()  # nothing appended


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_forced_flush_at_cursor_zero_is_the_plain_decode(io):
    c = _case(5, 4, 128, 128, 8, io, seed=3, steps=3)
    pool_a, pool_b = dev(c["pool"]), dev(c["pool"])
    idx = dev(c["slot_idx"], torch.int32)
    pos = torch.zeros(5, dtype=torch.int32, device="cuda")
    force = torch.ones(5, dtype=torch.int32, device="cuda")
    rd, rk, rg = _rings(c, 16)
    for s in range(3):
        q, k, v, g, beta = _step_inputs(c, s)
        o_a = kda.kda_recurrent_decode(q, k, v, g, beta, _scale(128), pool_a, idx)
        o_b, nxt = kda.kda_replay_decode(q, k, v, g, beta, _scale(128), pool_b, idx, pos,
                                         rd, rk, rg, force_flush=force)
        torch.cuda.synchronize()
        assert torch.equal(o_a, o_b) and torch.equal(pool_a, pool_b), s
        assert host(nxt).tolist() == [0] * 5


def _run_against_oracle(c, L, steps, force_at=None):
    """Replay decode over `steps` tokens with cursors carried from call to
    call; force_at(s) gives the rows to flush at step s.  Every step's o is
    checked against the oracle's decode; at the end every live row is
    flushed and the pool is checked against the oracle's states."""
    B, K = c["B"], c["K"]
    tol = TOL[c["io"]]
    pool_d = dev(c["pool"])
    idx_d = dev(c["slot_idx"], torch.int32)
    live = c["slot_idx"] >= 0
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    rd, rk, rg = _rings(c, L)
    pool_ref = c["pool"].astype(np.float64)
    cursors = np.zeros(B, dtype=np.int64)
    for s in range(steps + 1):
        last = s == steps  # one extra step that flushes everything
        ss = min(s, steps - 1)
        q, k, v, g, beta = _step_inputs(c, ss)
        force = np.zeros(B, dtype=np.int32)
        if last:
            force[:] = 1
        elif force_at is not None:
            force[force_at(s)] = 1
        o, nxt = kda.kda_replay_decode(q, k, v, g, beta, _scale(K), pool_d, idx_d, pos,
                                       rd, rk, rg, force_flush=dev(force, torch.int32))
        o_ref, pool_ref = oracle.decode(c["q"][:, ss], c["k"][:, ss], c["v"][:, ss],
                                        c["g"][:, ss], c["beta"][:, ss], _scale(K),
                                        pool_ref, c["slot_idx"])
        torch.cuda.synchronize()
        assert_io_output(host(o)[live], o_ref[live], c["io"], 1)
        if (~live).any():
            np.testing.assert_array_equal(host(o)[~live], 0.0)
        flushed = (cursors == L - 1) | (force != 0)
        expect = np.where(live, np.where(flushed, 0, cursors + 1), cursors)
        np.testing.assert_array_equal(host(nxt), expect)
        cursors = expect
        pos = nxt
    pool = host(pool_d)
    lv = c["slot_idx"][live]
    assert rel_err_blocks(pool[lv], pool_ref[lv], 2) <= tol
    dead = np.setdiff1d(np.arange(c["n_slots"]), lv)
    np.testing.assert_array_equal(pool[dead], c["pool"][dead])


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("KV", [(16, 16), (32, 64), (128, 128)])
def test_ring_steps_match_oracle(io, KV):
    K, V = KV
    c = _case(7, 3, K, V, 11, io, seed=50 + K, steps=21, n_padding=2)
    # rows 0 and 3 are flushed early at different steps, so cursors differ
    _run_against_oracle(c, L=8, steps=21,
                        force_at=lambda s: {2: [0], 5: [3], 11: [0, 4]}.get(s, []))


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("L", [2, 16, 32])
def test_ring_lengths_long_memory(io, L):
    # weak decay: the ring's replayed terms carry most of the state
    c = _case(5, 4, 128, 128, 9, io, seed=60 + L, steps=40, regime="long", n_padding=1)
    _run_against_oracle(c, L=L, steps=40)


def test_full_decode_workload_staggered_cursors():
    # 256 requests, 512-slot pool, H=32, K=V=128, ring of 16: flushes spread
    # over the rows (row r first flushes at step r % 16)
    w = kda_synth.WORKLOADS["decode_256"]
    c = _case(w["B"], w["H"], w["K"], w["V"], w["n_slots"], w["io"], seed=w["seed"],
              steps=20)
    rows = np.arange(w["B"])
    _run_against_oracle(c, L=16, steps=20, force_at=lambda s: rows[rows % 16 == s])


def test_cursor_outside_ring_touches_nothing():
    c = _case(4, 2, 32, 32, 6, "f32", seed=9, steps=1)
    pool_d = dev(c["pool"])
    idx = dev(c["slot_idx"], torch.int32)
    pos = dev(np.array([0, 4, -1, 3], dtype=np.int32), torch.int32)  # L = 4
    rd, rk, rg = _rings(c, 4)
    q, k, v, g, beta = _step_inputs(c, 0)
    o, nxt = kda.kda_replay_decode(q, k, v, g, beta, 1.0, pool_d, idx, pos, rd, rk, rg)
    torch.cuda.synchronize()
    o = host(o)
    assert np.isfinite(o[0]).all() and np.isnan(o[1]).all() and np.isnan(o[2]).all()
    # row 3 at the ring's last position reads entries 0..2, which were never
    # written here (NaN): its output and flushed checkpoint are NaN, which
    # shows that the cursor decides what is read
    assert np.isnan(o[3]).all()
    assert host(nxt).tolist() == [1, 4, -1, 0]
    pool = host(pool_d)
    for r in (1, 2):
        s = c["slot_idx"][r]
        np.testing.assert_array_equal(pool[s], c["pool"][s])
    assert torch.isnan(rd[c["slot_idx"][1]]).all() and torch.isnan(rd[c["slot_idx"][2]]).all()


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_replay_options_equal_prepared_inputs(io):
    # raw per-head gate (Gated DeltaNet form) and grouped q/k heads against
    # the same steps with kda_gate_prep's per-channel g and repeated heads
    B, H, HK, K, V, L, steps = 6, 8, 2, 64, 64, 4, 9
    c = _case(B, H, K, V, 9, io, seed=70, steps=steps, regime="long", n_padding=1)
    r = np.random.default_rng(71)
    a_h = r.standard_normal((B, steps, H)).astype(np.float32)
    dtb_h = (0.5 * r.standard_normal(H) - 6.0).astype(np.float32)
    A_log = dev(c["A_log"])
    iot = TORCH_IO[io]
    idx = dev(c["slot_idx"], torch.int32)
    pool_a, pool_b = dev(c["pool"]), dev(c["pool"])
    ra, rb = _rings(c, L), _rings(c, L)
    pos_a = pos_b = torch.zeros(B, dtype=torch.int32, device="cuda")
    for s in range(steps):
        q = dev(c["q"][:, s, :HK], iot)
        k = dev(c["k"][:, s, :HK], iot)
        v = dev(c["v"][:, s], iot)
        b = dev(c["b"][:, s])
        force = dev(np.array([s == 5] + [False] * (B - 1), dtype=np.int32), torch.int32)
        a_bc = dev(np.repeat(a_h[:, s, :, None], K, -1))
        g_ch, beta = kda.kda_gate_prep(a_bc, b, A_log, dev(np.repeat(dtb_h[:, None], K, 1)))
        rep = lambda x: x.repeat_interleave(H // HK, dim=1).contiguous()
        o_a, pos_a = kda.kda_replay_decode(rep(q), rep(k), v, g_ch, beta, 0.1, pool_a, idx, pos_a,
                                           *ra, force_flush=force)
        o_b, pos_b = kda.kda_replay_decode(q, k, v, dev(a_h[:, s]), b, 0.1, pool_b, idx, pos_b,
                                           *rb, force_flush=force,
                                           raw_gate=(A_log, dev(dtb_h), 0.0), per_head_gate=True)
        torch.cuda.synchronize()
        assert torch.equal(o_a, o_b), s
        assert torch.equal(pos_a, pos_b) and torch.equal(pool_a, pool_b), s
    for x, y in zip(ra, rb):
        assert torch.equal(torch.nan_to_num(x, nan=7.0), torch.nan_to_num(y, nan=7.0))


# --------------------------------------------------- L2 norm and output norm

def _raw_qk(c, seed):
    """Un-normalised q and k of the case's shape, rounded to its io dtype."""
    r = np.random.default_rng(seed)
    rt = lambda x: torch.from_numpy(x).to(TORCH_IO[c["io"]]).to(torch.float64).numpy()
    return rt(r.standard_normal(c["q"].shape) * 0.7), rt(r.standard_normal(c["k"].shape) * 1.3)


def _norm_opts(c, seed):
    B, steps, H, V = c["B"], c["q"].shape[1], c["H"], c["V"]
    r = np.random.default_rng(seed)
    z = torch.from_numpy(r.standard_normal((B, steps, H, V))).to(TORCH_IO[c["io"]])
    w = (1.0 + 0.1 * r.standard_normal(V)).astype(np.float32)
    return z, w


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_ring_of_one_with_norms_is_the_plain_decode_with_norms(io):
    """Ring length 1 (every call flushes, nothing is replayed) with the q/k L2
    norm and the gated RMSNorm equals kda_recurrent_decode_ex with the same
    options, bit for bit, o and pool, over several steps."""
    c = _case(6, 4, 128, 128, 9, io, seed=71, steps=4, n_padding=1)
    q_raw, k_raw = _raw_qk(c, 71)
    z, w = _norm_opts(c, 72)
    iot = TORCH_IO[io]
    pool_a, pool_b = dev(c["pool"]), dev(c["pool"])
    idx = dev(c["slot_idx"], torch.int32)
    rd, rk, rg = _rings(c, 1)
    pos = torch.zeros(c["B"], dtype=torch.int32, device="cuda")
    for s in range(4):
        q, k = dev(q_raw[:, s], iot), dev(k_raw[:, s], iot)
        _, _, v, g, beta = _step_inputs(c, s)
        zz = z[:, s].contiguous().cuda()
        o_a = kda.kda_recurrent_decode_ex(q, k, v, g, beta, _scale(128), pool_a, idx,
                                          qk_l2norm=True, o_gate=zz, o_norm_w=dev(w),
                                          o_gate_act="silu")
        o_b, pos = kda.kda_replay_decode(q, k, v, g, beta, _scale(128), pool_b, idx, pos,
                                         rd, rk, rg, qk_l2norm=True, o_gate=zz,
                                         o_norm_w=dev(w), o_gate_act="silu")
        torch.cuda.synchronize()
        assert torch.equal(o_a, o_b) and torch.equal(pool_a, pool_b), s


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("L", [4, 16])
def test_ring_steps_with_norms_match_oracle(io, L):
    """Raw q and k normalised in the kernel, ring entries replayed from raw k
    rows, and the gated RMSNorm of o, against the oracle's decode on
    l2norm(q), l2norm(k) followed by its gated_rmsnorm; slow decay so that
    the replayed terms carry the state."""
    c = _case(5, 4, 128, 128, 9, io, seed=73 + L, steps=2 * L + 3, regime="long", n_padding=1)
    steps, B, K = 2 * L + 3, c["B"], c["K"]
    q_raw, k_raw = _raw_qk(c, 74)
    z, w = _norm_opts(c, 75)
    iot = TORCH_IO[io]
    pool_d, idx_d = dev(c["pool"]), dev(c["slot_idx"], torch.int32)
    live = c["slot_idx"] >= 0
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    rd, rk, rg = _rings(c, L)
    pool_ref = c["pool"].astype(np.float64)
    for s in range(steps):
        _, _, v, g, beta = _step_inputs(c, s)
        force = np.zeros(B, dtype=np.int32)
        if s == L // 2:
            force[1] = 1  # one row flushed early: its cursor runs apart
        o, pos = kda.kda_replay_decode(dev(q_raw[:, s], iot), dev(k_raw[:, s], iot), v, g, beta,
                                       _scale(K), pool_d, idx_d, pos, rd, rk, rg,
                                       force_flush=dev(force, torch.int32), qk_l2norm=True,
                                       o_gate=z[:, s].contiguous().cuda(), o_norm_w=dev(w))
        o_ref, pool_ref = oracle.decode(oracle.l2norm(q_raw[:, s]), oracle.l2norm(k_raw[:, s]),
                                        c["v"][:, s], c["g"][:, s], c["beta"][:, s], _scale(K),
                                        pool_ref, c["slot_idx"])
        o_ref = oracle.gated_rmsnorm(o_ref, z[:, s].to(torch.float64).numpy(), w, 1e-6)
        torch.cuda.synchronize()
        assert_io_output(host(o)[live], o_ref[live], io, 1)
