"""Pins of dynamic episode recycling in the oracle ("GPU Pipeline Phase 2b",
Future Phase 3 Optimization: an episode that ends restarts from a new random
bar instead of idling or running on).

Pinned by: identity with the plain run up to each episode's first done; the
restart bar is the defined draw (floor(x range / 2^32) of the independently
pinned Philox word); every later state row continues bar by bar from it;
restarts stay inside the market and are uniform over their range; the DQN's
next state of a done step is still the bar after the finished one.
"""
import numpy as np
import pytest

import oracle
import synthdata

N_BARS = 3000


def dqn(recycle, N=24, L=150, seed=13):
    inp = synthdata.dqn_inputs(dict(N=N, L=L, n_bars=N_BARS, seed=seed), bias_scale=0.1)
    inp["settings"] = dict(inp["settings"], recycle=recycle)
    return inp, oracle.dqn_rollout(inp, with_q=False)


def ppo(recycle, N=24, L=150, seed=14):
    inp = synthdata.ppo_inputs(dict(N=N, L=L, n_bars=N_BARS, seed=seed), bias_scale=0.1)
    inp["settings"] = dict(inp["settings"], recycle=recycle)
    return inp, oracle.rollout(inp, with_logits=False)


def bar_of_row(features, row):
    """The bar whose 51 features equal this state row (unique for AR(1) data)."""
    hits = np.nonzero((features == row[None, :51]).all(axis=1))[0]
    assert hits.size == 1
    return int(hits[0])


def test_recycle_draw_definition():
    seed = 123456789
    for (n, t, L, nb) in [(0, 0, 500, 10**6), (7, 499 - 1, 500, 10**6), (3, 10, 100, 200)]:
        x = int(oracle.philox([n, t, 5, 0], [seed & 0xFFFFFFFF, seed >> 32])[0])
        rng = nb - (L - t - 1)
        assert oracle.recycle_bar(seed, n, t, L, nb) == (x * rng) >> 32


@pytest.mark.parametrize("run", [dqn, ppo])
def test_recycled_run(run):
    inp0, plain = run(0)
    inp1, rec = run(1)
    F = inp1["features"]
    L, N = rec["actions"].shape
    seed = inp1["sampler_seed"]
    n_restarts = 0
    for n in range(N):
        d0 = np.nonzero(plain["dones"][:, n])[0]
        first = int(d0[0]) if d0.size else L - 1
        for k in ("actions", "rewards", "dones", "states"):
            assert np.array_equal(plain[k][: first + 1, n], rec[k][: first + 1, n]), (n, k)
        bar = int(inp1["starts"][n])
        for t in range(L):
            assert bar_of_row(F, rec["states"][t, n]) == bar, (n, t)
            if rec["dones"][t, n] and t + 1 < L:
                nb = oracle.recycle_bar(seed, n, t, L, N_BARS)
                assert 0 <= nb <= N_BARS - 1 - (L - t - 1)
                if "next_states" in rec and rec["next_states"] is not None:
                    assert bar_of_row(F, rec["next_states"][t, n]) == bar + 1
                bar = nb
                n_restarts += 1
            else:
                bar += 1
    assert n_restarts > 10


def test_restart_bars_are_uniform():
    seed, L, nb = 99, 500, 10_000
    draws = np.array([oracle.recycle_bar(seed, n, t, L, nb)
                      for n in range(200) for t in range(0, 400, 7)])
    top = np.array([nb - 1 - (L - t - 1) for n in range(200) for t in range(0, 400, 7)])
    assert np.all(draws >= 0) and np.all(draws <= top)
    frac = draws / (top + 1)
    assert abs(frac.mean() - 0.5) < 5 * np.sqrt(1 / 12 / frac.size)
    counts = np.histogram(frac, bins=20, range=(0, 1))[0]
    e = frac.size / 20
    assert ((counts - e) ** 2 / e).sum() < 54.0  # df 19, p < 1e-5
