"""Pins for the oracle's softmax, CDF scan, inverse-CDF draw and log-prob
(PPO CUDA Pipeline Design, Kernel Phases, Phase A step 4)."""
import math

import numpy as np
import pytest
from scipy import stats

import oracle


def probs64(logits):
    x = np.asarray(logits, np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


@pytest.mark.parametrize("seed", range(5))
def test_cdf_ends_at_one_and_logp_matches(seed):
    g = np.random.default_rng(seed)
    for scale in (0.1, 1.0, 5.0, 30.0):
        lg = (g.standard_normal(45) * scale).astype(np.float32)
        u = float(g.random())
        a, lp, cdf, gap = oracle.softmax_sample(lg, u)
        p = probs64(lg)
        assert abs(cdf[-1] - 1.0) <= 45 * np.finfo(np.float32).eps
        np.testing.assert_allclose(cdf, np.cumsum(p), atol=1e-6)
        # log p[a] against an fp64 log-softmax
        assert abs(lp - math.log(p[a])) <= 1e-6 + 1e-6 * abs(math.log(p[a]))
        # the draw is the inverse CDF of the fp64 distribution (away from ties)
        c64 = np.cumsum(p)
        if np.min(np.abs(c64 - u)) > 1e-5:
            assert a == int(np.searchsorted(c64, u, side="right"))
        assert gap == pytest.approx(np.min(np.abs(cdf - u)), abs=1e-7)


def test_shift_invariance():
    """Logits on a 2^-10 grid stay exact under integer shifts, so the max-shifted
    exponentials and hence the CDF and log-probs are bit-identical."""
    g = np.random.default_rng(7)
    lg = (np.round(g.standard_normal(45) * 1024) / 1024).astype(np.float32)
    a0, lp0, c0, _ = oracle.softmax_sample(lg, 0.5)
    for shift in (-50.0, 3.0, 1000.0):
        a1, lp1, c1, _ = oracle.softmax_sample(lg + np.float32(shift), 0.5)
        assert np.array_equal(c0, c1) and a0 == a1 and lp0 == lp1


def test_uniform_logits_give_uniform_distribution():
    lg = np.full(45, 0.37, np.float32)
    _, lp, cdf, _ = oracle.softmax_sample(lg, 0.0)
    np.testing.assert_allclose(cdf, np.arange(1, 46) / 45.0, atol=1e-6)
    assert lp == pytest.approx(-math.log(45.0), abs=1e-6)
    for k in range(45):
        u = (k + 0.5) / 45.0
        assert oracle.softmax_sample(lg, u)[0] == k


def test_dominant_logit_is_deterministic():
    """Mass 1 - 44e^-60 on action 17; any u above the ~1e-25 mass in front of it
    draws 17 and log p = 0 to fp32 precision."""
    lg = np.full(45, -30.0, np.float32)
    lg[17] = 30.0
    for u in (1e-20, 0.3, 0.999999):
        a, lp, _, _ = oracle.softmax_sample(lg, u)
        assert a == 17 and abs(lp) < 1e-6


def test_boundary_rule_is_strict():
    """u exactly on a CDF value goes to the next action (a = min{k: u < CDF_k})."""
    lg = np.zeros(45, np.float32)
    lg[:2] = 10.0  # ~half the mass each on actions 0 and 1
    _, _, cdf, _ = oracle.softmax_sample(lg, 0.0)
    assert oracle.softmax_sample(lg, float(cdf[0]))[0] == 1
    assert oracle.softmax_sample(lg, float(np.nextafter(cdf[0], np.float32(0))))[0] == 0


def test_fallback_when_u_beyond_last_cdf():
    """If rounding leaves u >= CDF_44 the draw is the last action with weight."""
    lg = np.full(45, -200.0, np.float32)  # exp underflows to 0 for all but a few
    lg[3] = 0.0
    lg[9] = 0.0
    a = oracle.softmax_sample(lg, float(np.nextafter(np.float32(1), np.float32(0))))[0]
    assert a == 9


def test_chi_square_1e6_draws():
    """Empirical frequencies of 1e6 draws (u from the counter generator) match
    the fp64 softmax: reject at p < 1e-6."""
    g = np.random.default_rng(11)
    lg = (g.standard_normal(45) * 1.5).astype(np.float32)
    n = 1_000_000
    e = np.arange(n) % 1000
    t = np.arange(n) // 1000
    u = oracle.uniform(2024, e, t)
    a = oracle.sample_many(lg, u)
    counts = np.bincount(a, minlength=45).astype(np.float64)
    expected = probs64(lg) * n
    # merge classes with expected count < 5 into one bin
    small = expected < 5
    obs = np.append(counts[~small], counts[small].sum()) if small.any() else counts
    exp = np.append(expected[~small], expected[small].sum()) if small.any() else expected
    chi2 = ((obs - exp) ** 2 / exp).sum()
    df = obs.size - 1
    assert chi2 < stats.chi2.ppf(1 - 1e-6, df), (chi2, df)


def test_chi_square_detects_a_biased_sampler():
    """The same statistic rejects draws that follow a shifted distribution, so
    the bound above has power."""
    g = np.random.default_rng(11)
    lg = (g.standard_normal(45) * 1.5).astype(np.float32)
    lg2 = lg.copy()
    lg2[int(np.argmax(lg))] += 0.1
    n = 1_000_000
    e = np.arange(n) % 1000
    t = np.arange(n) // 1000
    a = oracle.sample_many(lg2, oracle.uniform(2024, e, t))
    counts = np.bincount(a, minlength=45).astype(np.float64)
    expected = probs64(lg) * n
    chi2 = ((counts - expected) ** 2 / expected).sum()
    assert chi2 > stats.chi2.ppf(1 - 1e-6, 44)
