"""Whole-rollout checks of the oracle (PPO CUDA Pipeline Design, Kernel Phases).

The composition of the steps (which bar each term reads, how the reward is
assembled) has no external worked example on the pages; it is checked here by
invariants (episode independence, determinism, teacher forcing) and by closed
forms on networks built to make the trajectory known in advance.
"""
import numpy as np
import pytest

import oracle
import synthdata

KEYS = ("states", "logits", "actions", "log_probs", "values", "rewards", "dones", "barrier",
        "adv", "ret", "u")


@pytest.fixture(scope="module")
def tiny():
    return synthdata.ppo_inputs("ppo_n16_l100")


@pytest.fixture(scope="module")
def tiny_out(tiny):
    return oracle.rollout(tiny)


def test_deterministic_and_thread_count_independent(tiny, tiny_out):
    o1 = oracle.rollout(tiny, n_threads=1)
    for k in KEYS:
        assert np.array_equal(o1[k], tiny_out[k]), k


def test_episode_subset_reproduces_columns(tiny, tiny_out):
    sub = [3, 11, 0]
    o = oracle.rollout(tiny, subset=sub)
    for k in KEYS:
        assert np.array_equal(o[k][:, sub], tiny_out[k][:, sub]), k


def test_teacher_forcing_with_own_actions_is_identity(tiny, tiny_out):
    o = oracle.rollout(tiny, forced_actions=tiny_out["actions"])
    for k in KEYS:
        assert np.array_equal(o[k], tiny_out[k]), k


def test_state_layout_and_draws(tiny, tiny_out):
    L, N = tiny["L"], tiny["N"]
    F = tiny["features"]
    bars = tiny["starts"][None, :] + np.arange(L)[:, None]
    assert np.array_equal(tiny_out["states"][:, :, :51], F[bars])
    assert np.all(tiny_out["states"][:, :, 53] == np.float32(0.0005))
    assert np.all(tiny_out["states"][0, :, 51:53] == 0)
    e, t = np.meshgrid(np.arange(N), np.arange(L))
    assert np.array_equal(tiny_out["u"], oracle.uniform(tiny["sampler_seed"], e, t).reshape(L, N))
    # exposure entering step t+1 is the one taken at step t unless the episode reset
    exp_tab = np.array([-1, -0.5, 0, 0.5, 1], np.float32)
    e_taken = exp_tab[tiny_out["actions"] // 9]
    nxt = tiny_out["states"][1:, :, 52]
    want = np.where(tiny_out["dones"][:-1] == 1, 0, e_taken[:-1])
    assert np.array_equal(nxt, want)
    assert np.all(tiny_out["states"][1:, :, 51][tiny_out["dones"][:-1] == 1] == 0)
    assert np.array_equal(tiny_out["dones"], (tiny_out["barrier"] > 0).astype(np.uint8))


def _flat_nets(seed=5, value_bias=0.7, action=22):
    """Actor: a dominant logit on `action`; critic: constant output; curiosity:
    all zero so the prediction is 0."""
    w = synthdata.ppo_weights(seed)
    for i in range(0, 6, 2):
        w["actor"][i] = np.zeros_like(w["actor"][i])
    b3 = np.full(45, -40.0, np.float32)
    b3[action] = 40.0
    w["actor"][5] = b3
    w["critic"] = [np.zeros_like(x) for x in w["critic"]]
    w["critic"][11] = np.array([value_bias], np.float32)
    w["curiosity"] = [np.zeros_like(x) for x in w["curiosity"]]
    return w


def test_closed_form_flat_policy(tiny):
    """Always flat: V == 1, no barrier, diversity entropy 0 (penalty -0.1),
    curiosity bonus = 0.01 mean_j F[bar+1][j]^2, value = critic bias; GAE of
    those rewards matches the explicit discounted sum."""
    inp = dict(tiny)
    inp["weights"] = _flat_nets()
    o = oracle.rollout(inp)
    L, N = inp["L"], inp["N"]
    assert np.all(o["actions"] == 22)
    assert np.all(o["log_probs"] == 0)
    assert np.all(o["states"][:, :, 51:53] == 0)
    assert np.all(o["dones"] == 0) and np.all(o["barrier"] == 0)
    assert np.all(o["values"] == np.float32(0.7))
    F = inp["features"].astype(np.float64)
    bars = inp["starts"][None, :] + np.arange(L)[:, None]
    bonus = 0.01 * (F[bars + 1] ** 2).mean(axis=2)
    np.testing.assert_allclose(o["rewards"], -0.1 + bonus, rtol=1e-5, atol=1e-6)
    gl = 0.99 * 0.95
    r = o["rewards"].astype(np.float64)
    delta = r + 0.99 * np.vstack([np.full((L - 1, N), 0.7), np.zeros((1, N))]) - 0.7
    A = np.zeros((L, N))
    for t in range(L):
        A[t] = sum(gl ** (k - t) * delta[k] for k in range(t, L))
    np.testing.assert_allclose(o["adv"], A, rtol=1e-5, atol=1e-5)


def test_closed_form_long_policy_bar_alignment(tiny):
    """Always long 1.0 with barriers out of reach: the normalised value feature
    at step t is prod_{k<t}(1 + P[b_k+1]/P[b_k] - 1) * (1 - open cost) - 1."""
    inp = dict(tiny)
    inp["weights"] = _flat_nets(action=36)
    st = dict(inp["settings"])
    st["profit_take"], st["stop_loss"], st["max_hold"] = 10.0, 0.99, 10**6
    o = oracle.rollout(inp, settings=st)
    L = inp["L"]
    P = inp["prices"].astype(np.float64)
    for n in range(inp["N"]):
        b = inp["starts"][n] + np.arange(L)
        g = P[b + 1] / P[b]
        V = np.cumprod(np.concatenate([[g[0] - 0.0002], g[1:]]))
        np.testing.assert_allclose(o["states"][1:, n, 51], V[:-1] - 1, rtol=1e-4, atol=2e-6)
        # reward = pnl - risk(0.01) + diversity (all long: -0.1) + bonus (prediction 0)
        pnl = np.concatenate([[g[0] - 1 - 0.0002], g[1:] - 1])
        F = inp["features"].astype(np.float64)
        bonus = 0.01 * (F[b + 1] ** 2).mean(axis=1)
        np.testing.assert_allclose(o["rewards"][:, n], pnl - 0.1 + bonus - 0.01, rtol=1e-5,
                                   atol=1e-6)


def test_precision_modes_agree_teacher_forced(tiny, tiny_out):
    o64 = oracle.rollout(tiny, precision=oracle.FP64, forced_actions=tiny_out["actions"])
    for k in ("logits", "values", "log_probs", "rewards", "adv", "ret"):
        np.testing.assert_allclose(o64[k], tiny_out[k], rtol=1e-4, atol=1e-5, err_msg=k)
    ob = oracle.rollout(tiny, precision=oracle.BF16, forced_actions=tiny_out["actions"])
    np.testing.assert_allclose(ob["values"], tiny_out["values"], rtol=0.1, atol=0.05)
    assert np.array_equal(ob["dones"], tiny_out["dones"])


def test_rejects_out_of_range_starts(tiny):
    inp = dict(tiny)
    inp["starts"] = tiny["starts"].copy()
    inp["starts"][2] = inp["n_bars"] - inp["L"]
    with pytest.raises(ValueError):
        oracle.rollout(inp)
