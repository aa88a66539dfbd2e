"""Pins of the oracle's networks as composed, not layer by layer.

Each network is rebuilt here as an fp64 numpy forward written from the shapes
the pages give, with nonzero biases:

* actor 54 -> 128 -> 64 -> 45, ReLU on both hidden layers, raw logits
  ("PPO CUDA Pipeline Design", Kernel Phases, Phase A step 3);
* critic 54 -> 512 -> 384 -> 256 -> 128 -> 64 -> 1, ReLU on every hidden
  layer, linear output (step 5);
* curiosity forward model on [state, one-hot(action)]: 99 -> 128 ReLU -> 51
  linear; bonus = 0.01 * mean squared error against the next bar's 51
  features (step 9; "GPU Pipeline Phase 2b", Kernel Components 2);
* dueling Q-network: trunk 54 -> 256 -> 128 (ReLU), value head 128 -> 64
  (ReLU) -> 1, advantage head 128 -> 64 (ReLU) -> 45,
  Q = V + (A - mean A) ("GPU Pipeline Phase 2b", Kernel Components 1).

The oracle evaluates each layer as a sequential fp32 sum.  Next to every fp64
reference value the forward carries a bound on the distance of an fp32
evaluation from it, by the probabilistic model of rounding errors (Higham and
Mary, "A New Approach to Probabilistic Rounding Error Analysis", SIAM J. Sci.
Comput. 41(5), 2019): every rounding is an independent, mean-zero error of at
most u |result| (u = 2^-24), so to first order the output error is a sum of
independent bounded terms and, by Hoeffding's inequality, lies within
lambda sqrt(sum of squared term bounds) except with probability
2 exp(-lambda^2 / 2).  The sum of squares is propagated layer by layer: a
layer maps it through W squared (errors of different inputs are
independent), adds (2K + 2) u^2 (sum |W x| + |b|)^2 for the 2K + 1 roundings
of a K-input sequential sum, and passes it through ReLU unchanged (ReLU is
1-Lipschitz); in the bf16 mode an input that carries an error may round to
the neighbouring bf16 value, one bf16 ulp (<= 2^-7 |x|) away.  lambda = 8
makes a false failure of any one output less likely than 3e-14.  The oracle
must lie inside the bound everywhere, and for every hidden ReLU the same
forward with that one ReLU removed must lie outside it somewhere, so a
dropped (or an added) activation anywhere in a network fails these tests.
"""
import numpy as np
import pytest

import oracle
import synthdata

from nets_ref import (ACTOR_RELU, CRITIC_RELU, CURIOSITY_RELU, LAMBDA, U, bf16, dense,  # noqa: F401
                      dueling, mlp, _chain)


def without(mask, l):
    m = list(mask)
    m[l] = not m[l]
    return tuple(m)


def bound(var):
    return LAMBDA * np.sqrt(var) + 1e-30


def check(name, got, ref, var):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref) - bound(var)
    assert not (err > 0).any(), (f"{name}: {int((err > 0).sum())} of {err.size} outside the "
                                 f"bound; worst excess {float(err.max()):.3g}")


def outside(got, ref, var):
    return bool((np.abs(np.asarray(got, np.float64) - ref) > bound(var)).any())


# ------------------------------------------------------------------ PPO rollout
def _ppo(bias, seed, precision=oracle.FP32, coef=None, N=8, L=60):
    inp = synthdata.ppo_inputs(dict(N=N, L=L, n_bars=4000, seed=seed), bias_scale=bias)
    if coef is not None:
        inp["settings"] = dict(inp["settings"], curiosity_coef=coef)
    out = oracle.rollout(inp, precision=precision)
    return inp, out


@pytest.mark.parametrize("precision", [oracle.FP32, oracle.BF16])
def test_actor_and_critic_inside_collect_match_fp64_forward(precision):
    """The logits and values the whole rollout stores are the actor and
    critic of its own stored states; each removed ReLU would be caught."""
    bf = precision == oracle.BF16
    inp, out = _ppo(0.2, 71, precision)
    s = out["states"].reshape(-1, 54).astype(np.float64)
    w = inp["weights"]
    logits, el = mlp(w["actor"], s, ACTOR_RELU, bf)
    check("logits", out["logits"].reshape(-1, 45), logits, el)
    v, ev = mlp(w["critic"], s, CRITIC_RELU, bf)
    check("values", out["values"].reshape(-1), v[:, 0], ev[:, 0])
    for l in range(2):
        lx, _ = mlp(w["actor"], s, without(ACTOR_RELU, l), bf)
        assert outside(out["logits"].reshape(-1, 45), lx, el), f"actor ReLU {l} has no effect"
    for l in range(6):
        vx, _ = mlp(w["critic"], s, without(CRITIC_RELU, l), bf)
        assert outside(out["values"].reshape(-1), vx[:, 0], ev[:, 0]), f"critic ReLU {l} not pinned"


def _env_terms(inp, out):
    """pnl, hit, diversity term and exposure of every step, from the (pinned)
    environment step driven by the oracle's own actions."""
    N, L = inp["N"], inp["L"]
    P = inp["prices"]
    terms = np.zeros((L, N, 4))
    for n in range(N):
        env = oracle.Env(inp["settings"])
        bar = int(inp["starts"][n])
        for t in range(L):
            r = env.step(int(out["actions"][t, n]), t, P[bar], P[bar + 1])
            terms[t, n] = (r["pnl"], r["hit"], r["div"], r["exposure"])
            if r["done"]:
                env.reset()
            bar += 1
    return terms


def _bonus(inp, out, relu=CURIOSITY_RELU, bf=False):
    """Curiosity bonus of every step and its bound (fp64 reference)."""
    L, N = out["actions"].shape
    s = out["states"].reshape(-1, 54).astype(np.float64)
    onehot = np.eye(45)[out["actions"].reshape(-1)]
    x = np.concatenate([s, onehot], axis=1)
    pred, vp = mlp(inp["weights"]["curiosity"], x, relu, bf)
    bars = inp["starts"][None, :].astype(np.int64) + np.arange(L)[:, None]
    target = inp["features"][(bars + 1).reshape(-1)].astype(np.float64)
    d = pred - target
    vd = vp + U * U * d * d                      # the subtraction's rounding
    se = (d * d).sum(axis=1)
    # d^2 has sensitivity 2 d; the 51 squares and 50 sums round once each
    vse = (4 * d * d * vd).sum(axis=1) + 102 * U * U * se * se
    coef = inp["settings"]["curiosity_coef"]
    bonus = coef * se / 51.0
    vb = (coef / 51.0) ** 2 * vse + 4 * U * U * bonus * bonus
    return bonus.reshape(L, N), vb.reshape(L, N)


def _reward_check(inp, out, bf=False):
    terms = _env_terms(inp, out)
    pnl, hit, div, ex = (terms[..., i] for i in range(4))
    st = inp["settings"]
    bonus, vb = _bonus(inp, out, bf=bf)
    t1 = pnl * (1.0 + st["barrier_scale"] * hit)
    t4 = np.float32(st["risk_coef"]) * np.abs(ex)
    ref = t1 + div + bonus - t4
    # the left-to-right fp32 combination of the five terms: 6 roundings
    var = vb + 6 * U * U * (np.abs(t1) + np.abs(div) + np.abs(bonus) + np.abs(t4)) ** 2
    return ref, var


@pytest.mark.parametrize("coef", [None, 1.0])
def test_curiosity_bonus_inside_collect_matches_fp64_forward(coef):
    """The reward minus its environment terms is the curiosity bonus of the
    forward model on [state, one-hot(action)] against the next bar; with the
    coefficient raised to 1 the bonus dominates the reward."""
    inp, out = _ppo(0.2, 72, coef=coef)
    ref, var = _reward_check(inp, out)
    check("rewards", out["rewards"], ref, var)
    terms = _env_terms(inp, out)
    st = inp["settings"]
    base = (terms[..., 0] * (1.0 + st["barrier_scale"] * terms[..., 1]) + terms[..., 2]
            - np.float32(st["risk_coef"]) * np.abs(terms[..., 3]))
    for l in range(2):
        bx, _ = _bonus(inp, out, relu=without(CURIOSITY_RELU, l))
        assert outside(out["rewards"], base + bx, var), f"curiosity ReLU {l} not pinned"


def test_curiosity_bonus_inside_collect_bf16():
    inp, out = _ppo(0.2, 73, precision=oracle.BF16, coef=1.0)
    ref, var = _reward_check(inp, out, bf=True)
    check("rewards (bf16)", out["rewards"], ref, var)


def test_values_reach_negative_and_hidden_units_are_cut():
    """The pins have power only if the ReLUs cut: the reference's hidden
    pre-activations are negative for a good share of units, and the value
    output takes both signs (a ReLU on the output would show)."""
    inp, out = _ppo(0.2, 74)
    s = out["states"].reshape(-1, 54).astype(np.float64)
    x = s
    w = inp["weights"]["critic"]
    for l in range(5):
        pre = x @ w[2 * l].astype(np.float64).T + w[2 * l + 1]
        assert 0.2 < (pre < 0).mean() < 0.8, l
        x = np.maximum(pre, 0)
    assert (out["values"] < 0).any() and (out["values"] > 0).any()


# -------------------------------------------------------------------------- DQN
def _qnets(seed, bias=0.2):
    return synthdata.dqn_weights(seed, bias_scale=bias)


def test_dueling_q_matches_fp64_forward():
    w = _qnets(81)["online"]
    g = np.random.default_rng(5)
    s = (g.standard_normal((200, 54)) * 2.0).astype(np.float32)
    s[:, 53] = 0.0005
    got = np.stack([oracle.dueling_q(w, row) for row in s])
    ref, bound = dueling(w, s.astype(np.float64))
    check("dueling Q", got, ref, bound)
    for l in range(2):
        rx, _ = dueling(w, s.astype(np.float64), trunk_relu=without((True, True), l))
        assert outside(got, rx, bound), f"trunk ReLU {l} not pinned"
    for l in range(2):
        rx, _ = dueling(w, s.astype(np.float64), head_relu=without((True, True), l))
        assert outside(got, rx, bound), f"head ReLU {l} not pinned"


def test_dqn_collect_q_values_and_target_max_match_fp64_forward():
    """Inside the DQN collection: the online Q of every stored state, the
    Q of the action taken, and the largest target Q of every stored next
    state."""
    inp = synthdata.dqn_inputs(dict(N=6, L=50, n_bars=3000, seed=82), bias_scale=0.2)
    out = oracle.dqn_rollout(inp)
    s = out["states"].reshape(-1, 54).astype(np.float64)
    q, eq = dueling(inp["weights"]["online"], s)
    check("q_values", out["q_values"].reshape(-1, 45), q, eq)
    a = out["actions"].reshape(-1)
    rows = np.arange(a.size)
    check("q_taken", out["q_taken"].reshape(-1), q[rows, a], eq[rows, a])
    sn = out["next_states"].reshape(-1, 54).astype(np.float64)
    qt, et = dueling(inp["weights"]["target"], sn)
    # max is 1-Lipschitz in the largest error of its arguments
    check("q_next_max", out["q_next_max"].reshape(-1), qt.max(axis=1), et.max(axis=1))
    qo, _ = dueling(inp["weights"]["online"], sn)
    assert outside(out["q_next_max"].reshape(-1), qo.max(axis=1), et.max(axis=1)), \
        "the target net is not the online net"
