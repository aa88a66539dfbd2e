"""Pins of the oracle's DQN collection ("GPU Pipeline Phase 2b", Data Flow and
Kernel Components 1, 7, 8; the priority rule of "GPU-Resident Prioritized
Experience Replay", Sampling Kernels).

The dueling network is pinned by properties of its aggregation
Q = V + (A - mean A) (each head isolated by zeroing the other's output
layer, identifiability shifts, the trunk feeding both heads); the random
action by exact integer arithmetic; the greedy action by argmax ties; the
environment and reward by the PPO oracle run on the same actions; the next
state by continuity with the following step's state; TD and priority by
their closed forms on the oracle's own outputs.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthdata


def small_inputs(N=8, L=120, seed=7, epsilon=None, bias_scale=0.1):
    return synthdata.dqn_inputs(dict(N=N, L=L, n_bars=3000, seed=seed), bias_scale=bias_scale,
                                epsilon=epsilon)


def net_and_state(seed=3):
    w = synthdata.dqn_weights(seed, bias_scale=0.2)["online"]
    g = np.random.default_rng(seed)
    s = g.standard_normal(54).astype(np.float32)
    return [x.copy() for x in w], s


def test_dueling_value_is_the_mean_of_q():
    """With the advantage output layer zeroed, Q_i = V for every i; the mean of
    the full Q over actions is that same V (the mean of A - mean A is 0)."""
    w, s = net_and_state()
    q = oracle.dueling_q(w, s)
    w0 = [x.copy() for x in w]
    w0[10][:] = 0.0
    w0[11][:] = 0.0
    qv = oracle.dueling_q(w0, s)
    assert np.all(qv == qv[0])
    assert abs(float(q.astype(np.float64).mean()) - float(qv[0])) <= 1e-5 * (1 + abs(qv[0]))


def test_dueling_advantage_differences():
    """Q_i - Q_j = A_i - A_j: with the value output layer zeroed the network
    gives A - mean A, whose differences equal those of the full Q."""
    w, s = net_and_state(5)
    q = oracle.dueling_q(w, s).astype(np.float64)
    w0 = [x.copy() for x in w]
    w0[6][:] = 0.0
    w0[7][:] = 0.0
    qa = oracle.dueling_q(w0, s).astype(np.float64)
    assert abs(qa.mean()) <= 1e-5 * np.abs(qa).max()
    d_full = q[:, None] - q[None, :]
    d_adv = qa[:, None] - qa[None, :]
    assert np.abs(d_full - d_adv).max() <= 1e-5 * (1 + np.abs(q).max())


def test_dueling_identifiability_shifts():
    """A constant added to every advantage bias leaves Q unchanged; a constant
    added to the value bias shifts every Q by it.  Both heads' outputs are
    linear: shifts of either sign, large enough to cross zero, carry through."""
    w, s = net_and_state(9)
    q = oracle.dueling_q(w, s).astype(np.float64)
    tol = 1e-5 * (1 + np.abs(q).max() + 50)
    for c in (3.0, -50.0):
        wa = [x.copy() for x in w]
        wa[11] += np.float32(c)
        assert np.abs(oracle.dueling_q(wa, s) - q).max() <= tol
        wv = [x.copy() for x in w]
        wv[7] += np.float32(c)
        assert np.abs(oracle.dueling_q(wv, s) - (q + c)).max() <= tol


def test_dueling_heads_read_the_trunk_output():
    """With the second trunk layer's weights zeroed its output is the ReLU of
    its bias for every state, so Q no longer depends on the state; with the
    first layer zeroed instead it does not either."""
    w, s = net_and_state(11)
    s2 = (s * -1.7 + 0.3).astype(np.float32)
    w2 = [x.copy() for x in w]
    w2[2][:] = 0.0
    assert np.array_equal(oracle.dueling_q(w2, s), oracle.dueling_q(w2, s2))
    w1 = [x.copy() for x in w]
    w1[0][:] = 0.0
    assert np.array_equal(oracle.dueling_q(w1, s), oracle.dueling_q(w1, s2))
    assert not np.array_equal(oracle.dueling_q(w, s), oracle.dueling_q(w, s2))


def test_argmax_ties_go_to_the_lowest_index():
    assert oracle.argmax_first([1.0, 3.0, 3.0, 2.0]) == 1
    assert oracle.argmax_first([5.0] * 45) == 0
    x = np.zeros(45, np.float32)
    x[44] = 1.0
    assert oracle.argmax_first(x) == 44
    x[7] = 1.0
    assert oracle.argmax_first(x) == 7
    assert oracle.argmax_first([-3.0, -1.0, -2.0]) == 1


def test_random_action_is_floor_45u_exactly():
    """u = m / 2^24: the random action is floor(45 m / 2^24), checked with exact
    rationals at every class boundary and on random grid points."""
    for k in range(1, 45):
        m = -(-k * 2**24 // 45)  # smallest m with 45 m / 2^24 >= k
        assert oracle.random_action(m / 2**24) == k
        assert oracle.random_action((m - 1) / 2**24) == k - 1
    g = np.random.default_rng(0)
    for m in list(g.integers(0, 2**24, 2000)) + [0, 2**24 - 1]:
        m = int(m)
        want = int(Fraction(45 * m, 2**24))  # floor of a positive rational
        assert oracle.random_action(m / 2**24) == want


@pytest.fixture(scope="module")
def run():
    inp = small_inputs()
    return inp, oracle.dqn_rollout(inp)


def test_next_state_is_the_following_state_unless_reset(run):
    inp, out = run
    L, N = out["actions"].shape
    S, NS, D = out["states"], out["next_states"], out["dones"]
    cont = D[:-1] == 0
    assert np.array_equal(NS[:-1][cont], S[1:][cont])
    reset = D[:-1] == 1
    assert reset.any(), "the run should hold some resets"
    assert np.all(S[1:][reset][:, 51] == 0.0) and np.all(S[1:][reset][:, 52] == 0.0)
    bars = inp["starts"][None, :] + np.arange(L)[:, None] + 1
    assert np.array_equal(NS[..., :51], inp["features"][bars])
    assert np.all(NS[..., 53] == np.float32(0.0005))


def test_actions_q_taken_and_exploration(run):
    inp, out = run
    Q, A, X = out["q_values"], out["actions"], out["explored"]
    L, N = A.shape
    qa = np.take_along_axis(Q, A[..., None].astype(np.int64), axis=2)[..., 0]
    assert np.array_equal(out["q_taken"], qa)
    greedy = X == 0
    assert greedy.any() and (~greedy).any()
    am = np.argmax(Q, axis=2)  # numpy's argmax also takes the first maximum
    assert np.array_equal(A[greedy], am[greedy])
    assert np.all(out["q_gap"] >= 0)
    t_idx, n_idx = np.nonzero(~greedy)
    u2 = oracle.uniform(inp["sampler_seed"], n_idx, t_idx, 2)
    assert np.array_equal(A[~greedy], [oracle.random_action(u) for u in u2])
    u1 = oracle.uniform(inp["sampler_seed"], np.tile(np.arange(N), L), np.repeat(np.arange(L), N), 1)
    assert np.array_equal(X.ravel() == 1, u1 < np.float32(inp["dqn"]["epsilon"]))


def test_target_max_td_and_priority_closed_forms(run):
    inp, out = run
    L, N = out["actions"].shape
    tw = inp["weights"]["target"]
    for t, n in [(0, 0), (5, 3), (L - 1, N - 1), (L // 2, 2)]:
        qt = oracle.dueling_q(tw, out["next_states"][t, n])
        assert out["q_next_max"][t, n] == qt.max()
    g = np.float32(inp["dqn"]["gamma"])
    r, qm, qa = out["rewards"], out["q_next_max"], out["q_taken"]
    d = out["dones"].astype(np.float32)
    td = (r + (g * qm) * (np.float32(1) - d)) - qa
    assert np.array_equal(out["td"], td.astype(np.float32))
    done = out["dones"] == 1
    assert np.array_equal(out["td"][done], (r - qa)[done])
    want = np.abs(out["td"].astype(np.float64)) ** 0.6
    assert np.allclose(out["priority"], want, rtol=2e-6, atol=0)


def test_environment_and_reward_match_the_ppo_oracle(run):
    """The same actions on the same market give the PPO collection's states,
    rewards, dones and barrier codes (its environment and reward are pinned on
    their own)."""
    inp, out = run
    ppo = dict(inp)
    ppo["weights"] = dict(synthdata.ppo_weights(1), curiosity=inp["weights"]["curiosity"])
    ref = oracle.rollout(ppo, forced_actions=out["actions"], with_logits=False)
    for k in ("rewards", "dones", "barrier", "states"):
        assert np.array_equal(out[k], ref[k]), k


def test_epsilon_extremes_and_rate():
    inp0 = small_inputs(N=6, L=60, seed=2, epsilon=0.0)
    o0 = oracle.dqn_rollout(inp0)
    assert not o0["explored"].any()
    assert np.array_equal(o0["actions"], np.argmax(o0["q_values"], axis=2))
    inp1 = small_inputs(N=6, L=60, seed=2, epsilon=1.0)
    o1 = oracle.dqn_rollout(inp1)
    assert o1["explored"].all()
    inp = small_inputs(N=64, L=200, seed=4)
    o = oracle.dqn_rollout(inp, with_q=False, with_next=False)
    rate = o["explored"].mean()
    sigma = np.sqrt(0.1 * 0.9 / o["explored"].size)
    assert abs(rate - 0.1) < 5 * sigma
    counts = np.bincount(o["actions"][o["explored"] == 1], minlength=45)
    expected = counts.sum() / 45
    chi2 = ((counts - expected) ** 2 / expected).sum()
    assert chi2 < 104.2  # df 44, p < 1e-6


def test_episodes_independent_and_deterministic(run):
    inp, out = run
    again = oracle.dqn_rollout(inp)
    for k in out:
        if out[k] is not None:
            assert np.array_equal(out[k], again[k]), k
    sub = oracle.dqn_rollout(inp, subset=[2, 5])
    for k in ("actions", "rewards", "td", "q_taken", "dones"):
        assert np.array_equal(sub[k][:, [2, 5]], out[k][:, [2, 5]]), k


def test_dqn_rejects_bad_arguments():
    inp = small_inputs(N=2, L=10)
    with pytest.raises(ValueError):
        oracle.dqn_rollout(inp, precision=oracle.BF16)
    bad = dict(inp)
    bad["starts"] = np.array([0, 2995], np.int32)
    with pytest.raises(ValueError):
        oracle.dqn_rollout(bad)
