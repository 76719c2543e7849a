"""Pins of the fp64 oracle against facts the pages and mathematics fix.

Nothing here compares the oracle with itself: every expected value is a
closed form, a worked example printed on the pages, an invariant stated
there, or a brute-force evaluation of the recurrence in another form
(explicit transition matrices, the chunk-level triangular system).

Sources (page title, section):
  "Linear attention" tutorial -- sections "演化：从累加到 Gated Delta Rule"
  (unified recurrence, delta rule as overwrite, matrix form), "Gated DeltaNet"
  (scalar gate, partial Householder, five steps), "KDA：逐通道的遗忘门"
  (per-channel decay), "实例：Kimi K3" (beta as interpolation, safe-gate
  half-lives), "核心抽象" (prefix sum, associative read-back).
  sgl-jax "KDA inference components" design doc, section 2.3 (prefill then
  k >= 8 decodes equals the longer prefill).
  "PR #26888 report" (verify equals stepwise decode; the pool is untouched).
"""
import math
import os

import numpy as np
import pytest

import kda_synth
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(r, *shape):
    return r.standard_normal(shape)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# --------------------------------------------------------------------- gate

def _gate1(a, dt_bias=0.0, A_log=0.0, b=0.0, lb=0.0):
    g, beta = oracle.gate(np.array([[[a]]]), np.array([[b]]), np.array([A_log]),
                          np.array([[dt_bias]]), lower_bound=lb)
    return g[0, 0, 0], beta[0, 0]


def test_gate_softplus_closed_forms():
    # softplus(0) = ln 2; softplus(ln(e-1)) = 1; softplus(ln 3) = ln 4
    assert _gate1(0.0)[0] == pytest.approx(-math.log(2.0), rel=1e-15)
    assert _gate1(math.log(math.e - 1.0))[0] == pytest.approx(-1.0, rel=1e-14)
    # exp(A_log) multiplies: A_log = ln 2 doubles the decay rate
    assert _gate1(math.log(3.0), A_log=math.log(2.0))[0] == pytest.approx(
        -2.0 * math.log(4.0), rel=1e-14)
    # dt_bias adds to a before the softplus
    assert _gate1(-1.0, dt_bias=1.0 + math.log(math.e - 1.0))[0] == pytest.approx(
        -1.0, rel=1e-14)
    # softplus(ln(e^y - 1)) = y exactly, up to just below the threshold
    for y in (2.5, 5.0, 10.0, 19.0):
        assert _gate1(math.log(math.expm1(y)))[0] == pytest.approx(-y, rel=1e-13)
    # above the threshold 20 softplus(x) = x, within exp(-x) of the exact value
    assert _gate1(25.0)[0] == pytest.approx(-25.0, rel=1e-10)
    # far left: softplus(x) = e^x (1 - e^x / 2 + ...)
    x = -30.0
    assert _gate1(x)[0] == pytest.approx(-math.exp(x) * (1 - math.exp(x) / 2), rel=1e-14)
    # g <= 0 everywhere
    r = np.random.default_rng(0)
    g, _ = oracle.gate(r.normal(0, 5, (64, 3, 8)), r.normal(0, 1, (64, 3)),
                       r.uniform(-2, 3, 3), r.normal(0, 3, (3, 8)))
    assert np.all(g <= 0.0)


def test_gate_beta_sigmoid_closed_forms():
    assert _gate1(0.0, b=0.0)[1] == 0.5
    assert _gate1(0.0, b=math.log(3.0))[1] == pytest.approx(0.75, rel=1e-15)
    assert _gate1(0.0, b=-math.log(3.0))[1] == pytest.approx(0.25, rel=1e-15)


def test_safe_gate_closed_forms():
    assert _gate1(0.0, lb=-5.0)[0] == pytest.approx(-2.5, rel=1e-15)
    # exp(A_log) is the sigmoid's slope: 2 * (ln 3 / 2) = ln 3 -> sigmoid 0.75
    assert _gate1(math.log(3.0) / 2, A_log=math.log(2.0), lb=-5.0)[0] == \
        pytest.approx(-3.75, rel=1e-14)


def test_safe_gate_half_life_worked_example():
    rows = []
    with open(os.path.join(GOLDEN, "safe_gate_half_life.txt")) as f:
        for line in f:
            s = line.strip()
            if s and not s.startswith("#"):
                rows.append([float(x) for x in s.split()])
    assert len(rows) == 3
    for dt_bias, printed, prec in rows:
        g, _ = _gate1(0.0, dt_bias=dt_bias, A_log=0.0, lb=-5.0)
        half_life = math.log(2.0) / abs(g)
        assert abs(half_life - printed) <= prec, (dt_bias, half_life, printed)
    # floor of alpha and the largest one-step forgetting (g -> lower bound)
    g_min, _ = _gate1(1e3, A_log=0.0, lb=-5.0)
    assert abs(math.exp(g_min) - 0.0067) <= 0.00005
    assert abs((1.0 - math.exp(g_min)) * 100.0 - 99.3) <= 0.05


# ------------------------------------------------------ recurrence, brute

def _brute_prefill(q, k, v, g, beta, cu, scale, h0):
    """S_t = (I - b k^T k) Diag(exp g) S_{t-1} + b k^T v, o_t = scale q S_t,
    with the K x K transition matrix formed explicitly (the page's KDA form)."""
    T, H, K = q.shape
    V = v.shape[2]
    N = len(cu) - 1
    o = np.zeros((T, H, V))
    ht = np.zeros((N, H, K, V))
    for n in range(N):
        for h in range(H):
            S = h0[n, h].copy()
            for t in range(cu[n], cu[n + 1]):
                kk = k[t, h][None, :]  # row vector 1 x K
                M = (np.eye(K) - beta[t, h] * kk.T @ kk) @ np.diag(np.exp(g[t, h]))
                S = M @ S + beta[t, h] * kk.T @ v[t, h][None, :]
                o[t, h] = scale * (q[t, h][None, :] @ S)[0]
            ht[n, h] = S
    return o, ht


def _random_problem(seed, seqlens, H, K, V, unit_keys=False):
    r = np.random.default_rng(seed)
    T = sum(seqlens)
    q, k = _rand(r, T, H, K), _rand(r, T, H, K)
    if unit_keys:
        q, k = _unit(q), _unit(k)
    v = _rand(r, T, H, V)
    g = -r.exponential(0.3, (T, H, K))
    beta = r.uniform(0, 1, (T, H))
    h0 = _rand(r, len(seqlens), H, K, V)
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64)
    return q, k, v, g, beta, cu, h0


@pytest.mark.parametrize("seqlens", [[8], [3, 0, 5, 1]])
def test_recurrence_equals_explicit_transition_matrices(seqlens):
    # K != V so that a transposed state index cannot pass; raw (not unit)
    # q, k and scale != 1 so that no normalisation hides a dropped factor.
    q, k, v, g, beta, cu, h0 = _random_problem(1, seqlens, 2, 5, 7)
    o, ht = oracle.prefill(q, k, v, g, beta, cu, 0.37, h0)
    o_b, ht_b = _brute_prefill(q, k, v, g, beta, cu, 0.37, h0)
    np.testing.assert_allclose(o, o_b, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ht, ht_b, rtol=1e-12, atol=1e-12)


def _closed_form_chunk(q, k, v, g, beta, S0, scale):
    """One chunk of the recurrence as a unit lower-triangular system.

    G = inclusive cumulative sum of g over the chunk;
    A[t, j]  = sum_c k_t[c] k_j[c] exp(G_t[c] - G_j[c])   (j < t)
    Aq[t, j] = sum_c q_t[c] k_j[c] exp(G_t[c] - G_j[c])   (j <= t)
    (I + diag(beta) A) D = diag(beta) (V - (K * e^G) S0)
    O = scale [ (Q * e^G) S0 + Aq D ],  S_C = e^{G_C} S0 + (K * e^{G_C - G})^T D
    Solved with numpy's dense solver (no forward substitution of our own).
    """
    C, K = k.shape
    G = np.cumsum(g, axis=0)
    A = np.zeros((C, C))
    Aq = np.zeros((C, C))
    for t in range(C):
        for j in range(t + 1):
            w = np.exp(G[t] - G[j])
            if j < t:
                A[t, j] = np.sum(k[t] * k[j] * w)
            Aq[t, j] = np.sum(q[t] * k[j] * w)
    Tm = np.eye(C) + beta[:, None] * A
    rhs = beta[:, None] * (v - (k * np.exp(G)) @ S0)
    D = np.linalg.solve(Tm, rhs)
    O = scale * ((q * np.exp(G)) @ S0 + Aq @ D)
    S = np.exp(G[-1])[:, None] * S0 + (k * np.exp(G[-1] - G)).T @ D
    return O, S


@pytest.mark.parametrize("seed", [2, 3, 4])
def test_recurrence_equals_triangular_closed_form(seed):
    q, k, v, g, beta, cu, h0 = _random_problem(seed, [8], 1, 6, 4, unit_keys=True)
    o, ht = oracle.prefill(q, k, v, g, beta, cu, 0.5, h0)
    O, S = _closed_form_chunk(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], h0[0, 0], 0.5)
    np.testing.assert_allclose(o[:, 0], O, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ht[0, 0], S, rtol=1e-11, atol=1e-12)


# --------------------------------------------------- special cases, pages

def test_overwrite_reads_back_new_value():
    """beta = 1, g = 0, orthonormal keys: write (k1, v1), (k2, v2), then
    (k1, v3); reading k1 gives v3 and k2 gives v2, exactly."""
    K, V = 6, 5
    keys = kda_synth.orthonormal_keys(3, K, seed=7)
    r = np.random.default_rng(7)
    vals = _rand(r, 3, V)
    seq_k = np.stack([keys[0], keys[1], keys[0]])[:, None, :]
    seq_v = np.stack([vals[0], vals[1], vals[2]])[:, None, :]
    seq_q = np.stack([keys[0], keys[1], keys[0]])[:, None, :]  # read own key
    g = np.zeros((3, 1, K))
    beta = np.ones((3, 1))
    o, ht = oracle.prefill(seq_q, seq_k, seq_v, g, beta, [0, 3], 1.0)
    np.testing.assert_allclose(o[0, 0], vals[0], atol=1e-14)  # read after write
    np.testing.assert_allclose(o[2, 0], vals[2], atol=1e-14)  # overwritten
    np.testing.assert_allclose(keys[1] @ ht[0, 0], vals[1], atol=1e-14)
    np.testing.assert_allclose(keys[0] @ ht[0, 0], vals[2], atol=1e-14)
    # an orthogonal, never-written direction reads zero
    extra = kda_synth.orthonormal_keys(4, K, seed=7)[3]
    np.testing.assert_allclose(extra @ ht[0, 0], np.zeros(V), atol=1e-14)


def test_beta_zero_gate_zero_freezes_state():
    q, k, v, _, _, cu, h0 = _random_problem(5, [6, 3], 2, 4, 3)
    T = q.shape[0]
    g = np.zeros((T, 2, 4))
    beta = np.zeros((T, 2))
    o, ht = oracle.prefill(q, k, v, g, beta, cu, 0.7, h0)
    np.testing.assert_array_equal(ht, h0)
    for n in range(2):
        for t in range(cu[n], cu[n + 1]):
            for h in range(2):
                np.testing.assert_allclose(o[t, h], 0.7 * q[t, h] @ h0[n, h], rtol=1e-14)


def test_orthonormal_keys_give_linear_attention_prefix_sum():
    """beta = 1, g = 0, S0 = 0, mutually orthonormal keys: each read k_t S_{t-1}
    is 0, so S_t is the prefix sum of k^T v and o_t = q_t sum_{j<=t} k_j^T v_j."""
    K, V, T = 8, 5, 8
    keys = kda_synth.orthonormal_keys(T, K, seed=11)
    r = np.random.default_rng(11)
    v = _rand(r, T, 1, V)
    q = _rand(r, T, 1, K)
    o, ht = oracle.prefill(q, keys[:, None, :], v, np.zeros((T, 1, K)),
                           np.ones((T, 1)), [0, T], 1.0)
    for t in range(T):
        S_t = sum(np.outer(keys[j], v[j, 0]) for j in range(t + 1))
        np.testing.assert_allclose(o[t, 0], q[t, 0] @ S_t, atol=1e-13)
    np.testing.assert_allclose(ht[0, 0], S_t, atol=1e-13)


def _unified_step(S, q, k, v, gamma_diag, alpha_w, beta):
    """The tutorial's unified form: v_hat = k (gamma S); Delta = v - v_hat;
    S = gamma S + alpha k^T v + beta k^T Delta; o = q S (gamma as a diagonal)."""
    GS = gamma_diag[:, None] * S
    delta = v - k @ GS
    S = GS + alpha_w * np.outer(k, v) + beta * np.outer(k, delta)
    return S, q @ S


def test_unified_form_members():
    r = np.random.default_rng(13)
    K, V = 5, 4
    # (gamma = 1, alpha = 1, beta = 0) is plain linear attention's prefix sum
    S = np.zeros((K, V))
    ks, vs = _rand(r, 6, K), _rand(r, 6, V)
    for t in range(6):
        S, _ = _unified_step(S, ks[t], ks[t], vs[t], np.ones(K), 1.0, 0.0)
    np.testing.assert_allclose(S, ks.T @ vs, atol=1e-13)
    # (gamma = Diag(exp g), alpha = 0, beta) is the KDA step of the oracle
    for _ in range(5):
        S0 = _rand(r, K, V)
        q, k, v = _rand(r, K), _unit(_rand(r, K)), _rand(r, V)
        g = -r.exponential(0.5, K)
        b = r.uniform()
        S_u, o_u = _unified_step(S0, q, k, v, np.exp(g), 0.0, b)
        S_o, o_o = oracle.step(S0, q, k, v, g, b, 1.0)
        np.testing.assert_allclose(S_o, S_u, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(o_o, o_u, rtol=1e-13, atol=1e-14)


def test_scalar_gate_reproduces_gated_deltanet():
    """g[t, :] = gamma_t for every channel gives GDN's
    S_t = a_t S - a_t b_t k^T (k S) + b_t k^T v (the expanded GDN form)."""
    r = np.random.default_rng(17)
    T, K, V = 12, 6, 5
    q, k = _unit(_rand(r, T, K)), _unit(_rand(r, T, K))
    v = _rand(r, T, V)
    gam = -r.exponential(0.4, T)
    beta = r.uniform(0, 1, T)
    S0 = _rand(r, K, V)
    o, ht = oracle.prefill(q[:, None], k[:, None], v[:, None],
                           np.repeat(gam[:, None, None], K, axis=2), beta[:, None],
                           [0, T], 1.0, S0[None, None])
    S = S0.copy()
    for t in range(T):
        a = math.exp(gam[t])
        S = a * S - a * beta[t] * np.outer(k[t], k[t] @ S) + beta[t] * np.outer(k[t], v[t])
        np.testing.assert_allclose(o[t, 0], q[t] @ S, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(ht[0, 0], S, rtol=1e-13, atol=1e-13)


def test_beta_interpolates_between_old_and_new_value():
    """For a unit key: k S_t = (1 - beta) k S' + beta v, with S' the decayed
    state; any direction orthogonal to k reads the same as in S'."""
    r = np.random.default_rng(19)
    K, V = 7, 6
    for _ in range(10):
        S0 = _rand(r, K, V)
        k = _unit(_rand(r, K))
        v = _rand(r, V)
        g = -r.exponential(0.5, K)
        b = r.uniform()
        Sp = np.exp(g)[:, None] * S0
        S1, o = oracle.step(S0, k, k, v, g, b, 1.0)  # q = k reads k S_t
        np.testing.assert_allclose(o, (1 - b) * (k @ Sp) + b * v, rtol=1e-12, atol=1e-13)
        u = _rand(r, K)
        u -= (u @ k) * k
        np.testing.assert_allclose(u @ S1, u @ Sp, rtol=1e-12, atol=1e-13)


def test_state_norm_never_grows_without_writes():
    """With g <= 0, beta in [0, 1], |k| = 1 and v = 0 each step applies
    (I - b k^T k) Diag(a), spectral norm <= 1: |S|_F is non-increasing."""
    r = np.random.default_rng(23)
    K, V, T = 16, 8, 2000
    k = _unit(_rand(r, T, K))
    g = -r.exponential(0.01, (T, K))
    beta = r.uniform(0, 1, T)
    S = _rand(r, K, V)
    prev = np.linalg.norm(S)
    for t in range(0, T, 250):
        sl = slice(t, t + 250)
        _, ht = oracle.prefill(np.zeros((250, 1, K)), k[sl, None], np.zeros((250, 1, V)),
                               g[sl, None], beta[sl, None], [0, 250], 1.0, S[None, None])
        S = ht[0, 0]
        cur = np.linalg.norm(S)
        assert cur <= prev * (1 + 1e-14)
        prev = cur


# ------------------------------------------------------ varlen, decode, verify

def test_varlen_batch_equals_separate_runs_and_empty_sequence():
    q, k, v, g, beta, cu, h0 = _random_problem(29, [5, 0, 17, 1, 9], 3, 4, 6, True)
    o, ht = oracle.prefill(q, k, v, g, beta, cu, 0.3, h0)
    for n in range(5):
        s, e = cu[n], cu[n + 1]
        o_n, ht_n = oracle.prefill(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e],
                                   [0, e - s], 0.3, h0[n:n + 1])
        np.testing.assert_array_equal(o[s:e], o_n)
        np.testing.assert_array_equal(ht[n], ht_n[0])
    np.testing.assert_array_equal(ht[1], h0[1])  # zero-length sequence


def test_prefill_then_decodes_equals_longer_prefill():
    q, k, v, g, beta, cu, h0 = _random_problem(31, [40], 2, 8, 8, True)
    kk = 8
    o_full, ht_full = oracle.prefill(q, k, v, g, beta, cu, 0.25, h0)
    o_pre, ht_pre = oracle.prefill(q[:-kk], k[:-kk], v[:-kk], g[:-kk], beta[:-kk],
                                   [0, 40 - kk], 0.25, h0)
    pool = np.concatenate([np.zeros_like(ht_pre), ht_pre])  # slot 1 holds it
    for i in range(40 - kk, 40):
        o_d, pool = oracle.decode(q[i][None], k[i][None], v[i][None], g[i][None],
                                  beta[i][None], 0.25, pool, [1])
        np.testing.assert_allclose(o_d[0], o_full[i], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(pool[1], ht_full[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(pool[0], 0.0)


def test_decode_maps_slots_and_skips_padding():
    c = kda_synth.decode_case(6, 2, 8, 4, n_slots=10, io="f32", seed=3, n_padding=2)
    g, beta = oracle.gate(c["a"], c["b"], c["A_log"], c["dt_bias"])
    o, pool = oracle.decode(c["q"], c["k"], c["v"], g, beta, 0.5, c["pool"], c["slot_idx"])
    touched = set()
    for r in range(6):
        s = int(c["slot_idx"][r])
        if s < 0:
            np.testing.assert_array_equal(o[r], 0.0)
            continue
        touched.add(s)
        for h in range(2):
            S1, o1 = oracle.step(c["pool"][s, h], c["q"][r, h], c["k"][r, h],
                                 c["v"][r, h], g[r, h], beta[r, h], 0.5)
            np.testing.assert_array_equal(pool[s, h], S1)
            np.testing.assert_array_equal(o[r, h], o1)
    for s in range(10):
        if s not in touched:
            np.testing.assert_array_equal(pool[s], c["pool"][s])


def test_verify_equals_sequential_decodes_and_leaves_pool():
    c = kda_synth.decode_case(4, 3, 8, 8, n_slots=6, io="f32", seed=5, Tv=5, n_padding=1)
    B, Tv, H = 4, 5, 3
    g, beta = oracle.gate(c["a"].reshape(B * Tv, H, 8), c["b"].reshape(B * Tv, H),
                          c["A_log"], c["dt_bias"])
    g = g.reshape(B, Tv, H, 8)
    beta = beta.reshape(B, Tv, H)
    pool0 = c["pool"].copy()
    o, inter = oracle.verify(c["q"], c["k"], c["v"], g, beta, 0.5, c["pool"],
                             c["slot_idx"], inter_fill=np.nan)
    np.testing.assert_array_equal(c["pool"], pool0)
    pool = c["pool"]
    for s in range(Tv):
        o_d, pool = oracle.decode(c["q"][:, s], c["k"][:, s], c["v"][:, s], g[:, s],
                                  beta[:, s], 0.5, pool, c["slot_idx"])
        np.testing.assert_array_equal(o[:, s], o_d)
        for r in range(B):
            sl = int(c["slot_idx"][r])
            if sl < 0:
                assert np.all(np.isnan(inter[r, s]))
            else:
                np.testing.assert_array_equal(inter[r, s], pool[sl])


def test_thread_count_does_not_change_results():
    q, k, v, g, beta, cu, h0 = _random_problem(37, [33, 7, 20], 4, 8, 8, True)
    a = oracle.prefill(q, k, v, g, beta, cu, 0.3, h0, nthreads=1)
    b = oracle.prefill(q, k, v, g, beta, cu, 0.3, h0, nthreads=7)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_bad_cu_seqlens_rejected():
    q, k, v, g, beta, cu, h0 = _random_problem(41, [4, 4], 1, 4, 4)
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v, g, beta, [0, 5, 3, 8], 1.0)


# ------------------------------------------------- layer helpers (norms)

def test_l2norm_closed_forms():
    # (3, 4) has norm 5: with eps 0 the result is (0.6, 0.8); eps only
    # shrinks the norm to 5 / sqrt(25 + eps) and keeps the direction
    np.testing.assert_allclose(oracle.l2norm(np.array([3.0, 4.0]), eps=0.0), [0.6, 0.8],
                               rtol=0, atol=1e-15)
    y = oracle.l2norm(np.array([[3.0, 4.0], [0.0, 2e-3]]), eps=1e-6)
    np.testing.assert_allclose(np.linalg.norm(y[0]), 5.0 / np.sqrt(25.0 + 1e-6), rtol=1e-15)
    np.testing.assert_allclose(y[0] / np.linalg.norm(y[0]), [0.6, 0.8], rtol=1e-15)
    # a small row: |x|^2 = 4e-6, so |y| = 2e-3 / sqrt(5e-6)
    np.testing.assert_allclose(y[1], [0.0, 2e-3 / np.sqrt(5e-6)], rtol=1e-14)
    # rows are independent and eps = 0 is scale-free
    r = np.random.default_rng(4)
    x = r.standard_normal((5, 16))
    np.testing.assert_allclose(oracle.l2norm(7.5 * x, eps=0.0), oracle.l2norm(x, eps=0.0),
                               rtol=1e-14)


def test_gated_rmsnorm_closed_forms():
    w = np.array([1.0, 2.0, 3.0, 4.0])
    o = np.array([1.0, -1.0, 1.0, -1.0])  # RMS exactly 1
    z0 = np.zeros(4)
    # sigmoid(0) = 1/2; silu(0) = 0
    np.testing.assert_allclose(oracle.gated_rmsnorm(o, z0, w, 0.0), [0.5, -1.0, 1.5, -2.0],
                               rtol=0, atol=1e-15)
    np.testing.assert_array_equal(oracle.gated_rmsnorm(o, z0, w, 0.0, act="silu"), 0.0)
    # o = (2, 0): RMS sqrt(2); z = ln 3 gives sigmoid 3/4 and silu (3/4) ln 3
    o2, w2, z2 = np.array([2.0, 0.0]), np.array([1.0, 1.0]), np.full(2, np.log(3.0))
    np.testing.assert_allclose(oracle.gated_rmsnorm(o2, z2, w2, 0.0),
                               [np.sqrt(2.0) * 0.75, 0.0], rtol=1e-15)
    np.testing.assert_allclose(oracle.gated_rmsnorm(o2, z2, w2, 0.0, act="silu"),
                               [np.sqrt(2.0) * 0.75 * np.log(3.0), 0.0], rtol=1e-15)
    # eps enters under the root: RMS^2 = 2 + eps
    np.testing.assert_allclose(oracle.gated_rmsnorm(o2, z2, w2, 2.0)[0], 2.0 / 2.0 * 0.75,
                               rtol=1e-15)
    # invariant to the scale of o when eps = 0
    r = np.random.default_rng(5)
    x, z, ww = r.standard_normal((3, 8)), r.standard_normal((3, 8)), r.standard_normal(8)
    np.testing.assert_allclose(oracle.gated_rmsnorm(40.0 * x, z, ww, 0.0),
                               oracle.gated_rmsnorm(x, z, ww, 0.0), rtol=1e-13)
