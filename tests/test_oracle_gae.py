"""Pins for the oracle's GAE (PPO CUDA Pipeline Design, Kernel Phases, Phase B).

The oracle runs the pages' backward recurrence.  It is checked here against
things other than itself: the explicit O(L^2) discounted sum (brute force in
fp64), closed forms, a hand-worked example and the invariants the recurrence
implies (advantages reset across dones, returns = advantages + values).
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def brute_force(r, v, d, gamma, lam, last=None):
    """A_t = sum_{k>=t} (gamma lam)^{k-t} prod_{j=t}^{k-1}(1-d_j) delta_k, fp64."""
    L, N = r.shape
    r, v, d = r.astype(np.float64), v.astype(np.float64), d.astype(np.float64)
    vn = np.vstack([v[1:], (np.zeros(N) if last is None else last.astype(np.float64))[None]])
    delta = r + gamma * vn * (1 - d) - v
    A = np.zeros((L, N))
    for t in range(L):
        acc = np.zeros(N)
        keep = np.ones(N)
        for k in range(t, L):
            acc += (gamma * lam) ** (k - t) * keep * delta[k]
            keep = keep * (1 - d[k])
        A[t] = acc
    return A, A + v


@pytest.mark.parametrize("L,N", [(1, 1), (2, 3), (5, 8), (16, 4), (9, 7)])
@pytest.mark.parametrize("with_last", [False, True])
def test_gae_vs_bruteforce(L, N, with_last):
    g = np.random.default_rng(L * 100 + N + with_last)
    for gamma, lam in [(0.99, 0.95), (0.9, 0.5), (1.0, 1.0), (0.5, 0.0)]:
        r = g.standard_normal((L, N)).astype(np.float32)
        v = g.standard_normal((L, N)).astype(np.float32)
        d = (g.random((L, N)) < 0.2).astype(np.uint8)
        last = g.standard_normal(N).astype(np.float32) if with_last else None
        A, R = oracle.gae(r, v, d, gamma, lam, last_values=last)
        Ab, Rb = brute_force(r, v, d, gamma, lam, last)
        np.testing.assert_allclose(A, Ab, rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(R, Rb, rtol=1e-5, atol=1e-5)


def test_gae_hand_example():
    rows, params = [], {}
    for line in open(os.path.join(GOLDEN, "gae_hand.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        parts = line.split()
        if parts[0] in ("gamma", "lambda"):
            params[parts[0]] = float(parts[1])
        else:
            rows.append([float(x) for x in parts])
    rows = np.array(rows)
    r = rows[:, 1:2].astype(np.float32)
    v = rows[:, 2:3].astype(np.float32)
    d = rows[:, 3:4].astype(np.uint8)
    A, R = oracle.gae(r, v, d, params["gamma"], params["lambda"])
    assert np.array_equal(A[:, 0], rows[:, 4].astype(np.float32))
    assert np.array_equal(R[:, 0], rows[:, 5].astype(np.float32))


def test_lambda_zero_is_one_step_td():
    g = np.random.default_rng(1)
    L, N = 12, 5
    r = g.standard_normal((L, N)).astype(np.float32)
    v = g.standard_normal((L, N)).astype(np.float32)
    d = (g.random((L, N)) < 0.3).astype(np.uint8)
    A, _ = oracle.gae(r, v, d, 0.9, 0.0)
    vn = np.vstack([v[1:], np.zeros((1, N))]).astype(np.float64)
    delta = r + 0.9 * vn * (1 - d) - v
    np.testing.assert_allclose(A, delta, rtol=1e-6, atol=1e-6)


def test_lambda_one_zero_values_is_discounted_return():
    g = np.random.default_rng(2)
    L, N, gamma = 30, 3, 0.97
    r = g.standard_normal((L, N)).astype(np.float32)
    z = np.zeros((L, N), np.float32)
    _, R = oracle.gae(r, z, z.astype(np.uint8), gamma, 1.0)
    mc = np.zeros((L, N))
    for t in range(L):
        mc[t] = sum(gamma ** (k - t) * r[k].astype(np.float64) for k in range(t, L))
    np.testing.assert_allclose(R, mc, rtol=1e-5, atol=1e-5)


def test_unit_rewards_geometric_closed_form():
    L, gamma, lam = 200, 0.99, 0.95
    r = np.ones((L, 1), np.float32)
    z = np.zeros((L, 1), np.float32)
    A, _ = oracle.gae(r, z, z.astype(np.uint8), gamma, lam)
    gl = gamma * lam
    t = np.arange(L)
    closed = (1 - gl ** (L - t)) / (1 - gl)
    np.testing.assert_allclose(A[:, 0], closed, rtol=1e-5)


def test_done_gives_reward_minus_value():
    g = np.random.default_rng(3)
    L, N = 10, 6
    r = g.standard_normal((L, N)).astype(np.float32)
    v = g.standard_normal((L, N)).astype(np.float32)
    d = np.ones((L, N), np.uint8)
    A, _ = oracle.gae(r, v, d, 0.99, 0.95)
    assert np.array_equal(A, r - v)


def test_advantages_reset_across_dones():
    """With d_k = 1, A_t for t <= k is bit-identical after any change at t > k."""
    g = np.random.default_rng(4)
    L, N, k = 40, 8, 17
    r = g.standard_normal((L, N)).astype(np.float32)
    v = g.standard_normal((L, N)).astype(np.float32)
    d = (g.random((L, N)) < 0.1).astype(np.uint8)
    d[k] = 1
    A, R = oracle.gae(r, v, d, 0.99, 0.95)
    r2, v2, d2 = r.copy(), v.copy(), d.copy()
    r2[k + 1:] = g.standard_normal((L - k - 1, N))
    v2[k + 1:] = g.standard_normal((L - k - 1, N))
    d2[k + 1:] = (g.random((L - k - 1, N)) < 0.5)
    A2, R2 = oracle.gae(r2, v2, d2, 0.99, 0.95)
    assert np.array_equal(A[:k + 1], A2[:k + 1])
    assert np.array_equal(R[:k + 1], R2[:k + 1])
    assert not np.array_equal(A[k + 1:], A2[k + 1:])


def test_returns_are_advantages_plus_values_exactly():
    g = np.random.default_rng(5)
    r, v = (g.standard_normal((64, 33)).astype(np.float32) for _ in range(2))
    d = (g.random((64, 33)) < 0.05).astype(np.uint8)
    A, R = oracle.gae(r, v, d, 0.99, 0.95)
    assert np.array_equal(R, (A + v).astype(np.float32))


def test_fp32_within_rounding_of_fp64_mode():
    g = np.random.default_rng(6)
    r = g.standard_normal((2048, 16)).astype(np.float32)
    v = (0.5 * g.standard_normal((2048, 16))).astype(np.float32)
    d = (g.random((2048, 16)) < 0.005).astype(np.uint8)
    A32, _ = oracle.gae(r, v, d, 0.99, 0.95)
    A64, _ = oracle.gae(r, v, d, 0.99, 0.95, precision=oracle.FP64)
    np.testing.assert_allclose(A32, A64, rtol=1e-5, atol=1e-5)
