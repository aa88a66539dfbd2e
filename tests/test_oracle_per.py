"""Pins of the oracle's prioritized-replay sampling and priority update
("GPU-Resident Prioritized Experience Replay", Sampling Kernels: proportional
sampling by prefix sum and search, IS weights; priority update and the
NaN/Inf clamp of Error Handling).

The sample is pinned by exact rational arithmetic on the same draws, by
frequencies against p_i / sum p (chi-square), and by its special cases; the
weights by their ratio and normalisation properties; the update by its
closed form and its rules for NaN, Inf, repeats (the largest new value) and
range.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def exact_index(p, u):
    """First k with sum_{j<=k} p_j > u * sum p, in exact rationals."""
    vals = [Fraction(float(x)) if x > 0 else Fraction(0) for x in p]
    total = sum(vals)
    target = Fraction(u) * total
    run = Fraction(0)
    for k, v in enumerate(vals):
        run += v
        if run > target:
            return k
    raise AssertionError("no index")


def test_uniform_draws_are_53_bit_and_in_range():
    us = np.array([oracle.per_uniform(12345, b) for b in range(2000)])
    assert np.all(us >= 0) and np.all(us < 1)
    assert np.all(np.floor(us * 2.0**53) == us * 2.0**53)  # on the 2^-53 grid
    assert abs(us.mean() - 0.5) < 5 * np.sqrt(1 / 12 / us.size)
    assert len(set(us.tolist())) == us.size


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_sample_matches_exact_prefix_search(seed):
    g = np.random.default_rng(seed)
    p = g.exponential(1.0, 37).astype(np.float32)
    p[[3, 9]] = 0.0
    p[5] = -2.0      # counts as zero
    p[11] = np.nan   # counts as zero
    idx, _, gap = oracle.per_sample(p, 400, seed, 0.4)
    for b in range(idx.size):
        u = oracle.per_uniform(seed, b)
        assert idx[b] == exact_index(p, u), b
    assert not np.isin(idx, [3, 5, 9, 11]).any()
    assert np.all(gap >= 0)


def test_sample_frequencies_follow_the_priorities():
    g = np.random.default_rng(7)
    p = g.uniform(0.05, 3.0, 20).astype(np.float32)
    draws = 200_000
    idx, _, _ = oracle.per_sample(p, draws, 99, 0.0)
    counts = np.bincount(idx, minlength=p.size)
    expected = p.astype(np.float64) / p.sum(dtype=np.float64) * draws
    chi2 = ((counts - expected) ** 2 / expected).sum()
    assert chi2 < 60.0  # df 19, p < 1e-6


def test_importance_weights():
    g = np.random.default_rng(4)
    p = g.uniform(0.1, 5.0, 64).astype(np.float32)
    beta = 0.4
    idx, w, _ = oracle.per_sample(p, 300, 5, beta)
    assert w.max() == np.float32(1.0)
    # w_a / w_b = (p_a / p_b)^(-beta)
    pa = p[idx].astype(np.float64)
    ratio = w.astype(np.float64) / w[0]
    assert np.allclose(ratio, (pa / pa[0]) ** -beta, rtol=1e-6)
    # the normaliser is the batch's largest weight: that of its smallest priority
    k = np.argmin(pa)
    assert w[k] == np.float32(1.0)
    _, w0, _ = oracle.per_sample(p, 50, 5, 0.0)
    assert np.all(w0 == 1.0)
    _, wu, _ = oracle.per_sample(np.full(64, 2.5, np.float32), 50, 5, 0.7)
    assert np.all(wu == 1.0)


def test_degenerate_total_falls_back_to_uniform():
    p = np.zeros(10, np.float32)
    idx, w, _ = oracle.per_sample(p, 100, 3, 0.4)
    want = [min(int(oracle.per_uniform(3, b) * 10), 9) for b in range(100)]
    assert idx.tolist() == want
    assert np.all(w == 1.0)


def test_sample_is_deterministic_per_seed():
    p = np.random.default_rng(1).exponential(1.0, 1000).astype(np.float32)
    a = oracle.per_sample(p, 256, 42, 0.4)
    b = oracle.per_sample(p, 256, 42, 0.4)
    c = oracle.per_sample(p, 256, 43, 0.4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert not np.array_equal(a[0], c[0])


def test_update_closed_form_and_clamps():
    p = np.linspace(0.5, 2.0, 8).astype(np.float32)
    alpha, eps, pmax = 0.6, 0.01, 5.0
    td = np.array([2.0, -0.5, 0.0, np.nan, np.inf, 1e6], np.float32)
    idx = np.array([0, 1, 2, 3, 4, 5], np.int32)
    q = oracle.per_update(p, idx, td, alpha, eps, pmax)
    assert abs(q[0] - (2.0 ** 0.6 + 0.01)) < 1e-6
    assert abs(q[1] - (0.5 ** 0.6 + 0.01)) < 1e-6
    assert q[2] == np.float32(eps)     # |0|^alpha + eps
    assert q[3] == np.float32(eps)     # NaN
    assert q[4] == np.float32(pmax)    # Inf
    assert q[5] == np.float32(pmax)    # clamped
    assert np.array_equal(q[6:], p[6:])  # untouched


def test_update_repeats_keep_the_largest_value():
    p = np.full(4, 50.0, np.float32)
    q = oracle.per_update(p, [2, 1, 2, 2], [3.0, 1.0, 0.25, 2.0], 1.0, 0.0, 100.0)
    assert q[2] == np.float32(3.0) and q[1] == np.float32(1.0)
    assert q[0] == 50.0 and q[3] == 50.0  # untouched; at 2 the old 50 gives way to 3
    q = oracle.per_update(p, [0, 0], [0.5, 0.25], 1.0, 0.0, 100.0)
    assert q[0] == np.float32(0.5)


def test_update_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.per_update(np.ones(4, np.float32), [4], [1.0], 0.6, 0.01, 5.0)
    with pytest.raises(ValueError):
        oracle.per_update(np.ones(4, np.float32), [-1], [1.0], 0.6, 0.01, 5.0)
