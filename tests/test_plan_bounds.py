"""The prefill's rule for turning cu_seqlens into sequence ranges, checked on
the host (no GPU needed).

The chunk-table kernel never trusts cu_seqlens: with c'_m = cu[m] clamped
into [0, T] and p_n = max(c'_0 .. c'_n), sequence n covers tokens
p_n .. p_{n+1}-1.  This module restates that rule in numpy and checks the two
facts the kernels' bounds rest on, over adversarial arrays: the ranges are
disjoint and inside [0, T) (so the chunks number at most ceil(T/C) + N, the
workspace's chunk count, and the snapshot rows at most T // interval), and a
valid array is left unchanged.  tests/test_gpu_prefill.py runs the kernels on
such arrays and compares them with the same call on the clamped array.
"""
import numpy as np


def disjoint_bounds(cu, T):
    c = np.clip(np.asarray(cu, dtype=np.int64), 0, T)
    p = np.maximum.accumulate(c)
    return p[:-1], p[1:]


def _adversarial(rng, N, T):
    kind = rng.integers(4)
    if kind == 0:
        return rng.integers(-T - 1, 2 * T + 2, size=N + 1)
    if kind == 1:  # decreasing
        return np.sort(rng.integers(0, T + 1, size=N + 1))[::-1]
    if kind == 2:  # repeats of the whole range
        return np.array([0 if i % 2 == 0 else T for i in range(N + 1)])
    x = np.sort(rng.integers(0, T + 1, size=N + 1))
    x[0], x[-1] = 0, T
    return x


def test_ranges_are_disjoint_and_bounded():
    rng = np.random.default_rng(0)
    for _ in range(3000):
        N = int(rng.integers(1, 12))
        T = int(rng.integers(0, 500))
        C = int(rng.choice([16, 32, 64]))
        interval = C * int(rng.integers(1, 4))
        lo, hi = disjoint_bounds(_adversarial(rng, N, T), T)
        assert np.all(0 <= lo) and np.all(lo <= hi) and np.all(hi <= T)
        assert np.all(lo[1:] == hi[:-1])  # consecutive and non-overlapping
        chunks = int(np.sum((hi - lo + C - 1) // C))
        assert chunks <= (T + C - 1) // C + N
        assert int(np.sum((hi - lo) // interval)) <= T // interval


def test_valid_arrays_are_unchanged():
    rng = np.random.default_rng(1)
    for _ in range(500):
        N = int(rng.integers(1, 9))
        T = int(rng.integers(0, 400))
        cu = np.sort(rng.integers(0, T + 1, size=N + 1))
        cu[0], cu[-1] = 0, T
        lo, hi = disjoint_bounds(cu, T)
        np.testing.assert_array_equal(lo, cu[:-1])
        np.testing.assert_array_equal(hi, cu[1:])


def test_the_overlapping_example():
    # [0, T, 0, T]: the second pair would overlap the first; it becomes empty
    lo, hi = disjoint_bounds([0, 200, 0, 200], 200)
    np.testing.assert_array_equal(lo, [0, 200, 200])
    np.testing.assert_array_equal(hi, [200, 200, 200])
