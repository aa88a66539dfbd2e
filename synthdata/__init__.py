"""Seeded synthetic inputs for PPO and DQN experience collection.

This module only *generates inputs*: market features and prices, network
weights, episode start bars, GAE test streams and the scalar settings of a
collection run.  It holds no step of the method (no network evaluation, no
sampling, no portfolio or reward arithmetic), so the CPU oracle and the HIP
library can both be fed from it without sharing any of the method's code.

Input recipe (the pages' own market data and trained weights are private;
these stand in for them at the pages' shapes: 51 features per bar, 45 actions,
bars in the 10^4..10^6 range):

* features: each of the 51 columns is an independent AR(1) process
  x_b = 0.9 x_{b-1} + eps_b with eps ~ N(0, 1), started from its stationary
  law N(0, 1 / (1 - 0.9^2)).
* prices: geometric random walk P_0 = 100, P_b = P_{b-1} exp(0.01 z_b).
* weights: He-normal N(0, 2 / fan_in) for every layer, [out, in] row-major,
  zero biases (``bias_scale`` > 0 adds N(0, bias_scale^2) biases so bias
  handling can be exercised).
* episode starts: uniform integers in [0, n_bars - L).
* GAE streams: rewards ~ N(0, 1), values ~ N(0, 0.5^2), dones ~ Bernoulli(0.005).

All randomness comes from numpy's PCG64 keyed by (seed, stream id), so every
array is a deterministic function of its seed.
"""
from __future__ import annotations

import numpy as np
from scipy.signal import lfilter

N_FEATURES = 51
STATE_DIM = 54
N_ACTIONS = 45
ACTOR_DIMS = (54, 128, 64, 45)
CRITIC_DIMS = (54, 512, 384, 256, 128, 64, 1)
CURIOSITY_DIMS = (STATE_DIM + N_ACTIONS, 128, N_FEATURES)
# dueling Q-network of the DQN collection: trunk, value head, advantage head
Q_TRUNK_DIMS = (54, 256, 128)
Q_VALUE_DIMS = (128, 64, 1)
Q_ADV_DIMS = (128, 64, 45)

# Named workloads: sizes and master seeds.
WORKLOADS = {
    "ppo_n16_l100": dict(N=16, L=100, n_bars=20_000, seed=0),
    "ppo_n128_l500": dict(N=128, L=500, n_bars=200_000, seed=1),
    "gae_n4096_l2048": dict(N=4096, L=2048, seed=2),
    "ppo_n8192_l500": dict(N=8192, L=500, n_bars=1_000_000, seed=3),
    "dqn_n16384_l500": dict(N=16384, L=500, n_bars=1_000_000, seed=4),
}

_STREAM_MARKET = 1
_STREAM_WEIGHTS = 2
_STREAM_STARTS = 3
_STREAM_GAE = 4
_STREAM_SAMPLER = 5


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(seed), int(stream)]))


def settings() -> dict:
    """Scalar settings of a collection run (reward, barrier, diversity, GAE)."""
    return dict(
        gamma=0.99,
        lam=0.95,
        profit_take=0.02,
        stop_loss=0.01,
        max_hold=50,
        div_window=20,
        div_threshold=1.0,
        div_penalty=-0.1,
        curiosity_coef=0.01,
        risk_coef=0.01,
        spread=0.0005,
        barrier_scale=0.5,
        exposure=(-1.0, -0.5, 0.0, 0.5, 1.0),
        cost=(0.0002, 0.0005, 0.001),
        urgency_mult=0.5,
    )


def market(n_bars: int, seed: int, rho: float = 0.9, sigma: float = 0.01, p0: float = 100.0):
    """(features [n_bars, 51] f32, prices [n_bars] f32)."""
    g = _rng(seed, _STREAM_MARKET)
    eps = g.standard_normal((n_bars, N_FEATURES))
    eps[0] /= np.sqrt(1.0 - rho * rho)
    # filter each feature's series along contiguous memory, then back to [bars, 51]
    feats = lfilter([1.0], [1.0, -rho], np.ascontiguousarray(eps.T), axis=1).T.astype(np.float32)
    z = g.standard_normal(n_bars)
    z[0] = 0.0
    prices = (p0 * np.exp(sigma * np.cumsum(z))).astype(np.float32)
    return np.ascontiguousarray(feats), np.ascontiguousarray(prices)


def _he_layer(g, fan_in, fan_out, bias_scale):
    w = (g.standard_normal((fan_out, fan_in)) * np.sqrt(2.0 / fan_in)).astype(np.float32)
    if bias_scale > 0:
        b = (g.standard_normal(fan_out) * bias_scale).astype(np.float32)
    else:
        b = np.zeros(fan_out, np.float32)
    return w, b


def _mlp(g, dims, bias_scale):
    out = []
    for i in range(len(dims) - 1):
        w, b = _he_layer(g, dims[i], dims[i + 1], bias_scale)
        out += [w, b]
    return out


def ppo_weights(seed: int, bias_scale: float = 0.0) -> dict:
    """{'actor': [W1,b1,W2,b2,W3,b3], 'critic': [12 arrays], 'curiosity': [4 arrays]}."""
    g = _rng(seed, _STREAM_WEIGHTS)
    return dict(
        actor=_mlp(g, ACTOR_DIMS, bias_scale),
        critic=_mlp(g, CRITIC_DIMS, bias_scale),
        curiosity=_mlp(g, CURIOSITY_DIMS, bias_scale),
    )


def q_net_weights(g, bias_scale: float) -> list:
    """12 arrays: trunk 1, trunk 2, value 1, value 2, advantage 1, advantage 2
    (weight [out, in], then bias)."""
    return (_mlp(g, Q_TRUNK_DIMS, bias_scale) + _mlp(g, Q_VALUE_DIMS, bias_scale)
            + _mlp(g, Q_ADV_DIMS, bias_scale))


def dqn_weights(seed: int, bias_scale: float = 0.0) -> dict:
    """{'online': [12], 'target': [12], 'curiosity': [4]}: online and target
    nets initialised independently."""
    g = _rng(seed, _STREAM_WEIGHTS)
    return dict(online=q_net_weights(g, bias_scale), target=q_net_weights(g, bias_scale),
                curiosity=_mlp(g, CURIOSITY_DIMS, bias_scale))


def dqn_settings() -> dict:
    """Scalars of the DQN collection: exploration rate, TD discount, priority
    exponent."""
    return dict(epsilon=0.1, gamma=0.99, alpha=0.6)


def episode_starts(N: int, L: int, n_bars: int, seed: int) -> np.ndarray:
    g = _rng(seed, _STREAM_STARTS)
    return g.integers(0, n_bars - L, size=N, dtype=np.int64).astype(np.int32)


def sampler_seed(seed: int) -> int:
    """64-bit key for the per-(episode, step) draws of one collection."""
    g = _rng(seed, _STREAM_SAMPLER)
    return int(g.integers(0, 2**63 - 1, dtype=np.int64)) * 2 + 1


def gae_inputs(N: int, L: int, seed: int, p_done: float = 0.005):
    """(rewards, values, dones) of shape [L, N]: f32, f32, u8."""
    g = _rng(seed, _STREAM_GAE)
    r = g.standard_normal((L, N)).astype(np.float32)
    v = (0.5 * g.standard_normal((L, N))).astype(np.float32)
    d = (g.random((L, N)) < p_done).astype(np.uint8)
    return r, v, d


def ppo_inputs(name_or_spec, bias_scale: float = 0.0) -> dict:
    """Everything one PPO collection needs, for a named workload or a spec dict."""
    spec = WORKLOADS[name_or_spec] if isinstance(name_or_spec, str) else dict(name_or_spec)
    N, L, nb, seed = spec["N"], spec["L"], spec["n_bars"], spec["seed"]
    feats, prices = market(nb, seed)
    return dict(
        N=N, L=L, n_bars=nb, seed=seed,
        features=feats, prices=prices,
        weights=ppo_weights(seed, bias_scale),
        starts=episode_starts(N, L, nb, seed),
        sampler_seed=sampler_seed(seed),
        settings=settings(),
    )


def dqn_inputs(name_or_spec, bias_scale: float = 0.0, epsilon: float | None = None) -> dict:
    """Everything one DQN collection needs, for a named workload or a spec dict."""
    spec = WORKLOADS[name_or_spec] if isinstance(name_or_spec, str) else dict(name_or_spec)
    N, L, nb, seed = spec["N"], spec["L"], spec["n_bars"], spec["seed"]
    feats, prices = market(nb, seed)
    dq = dqn_settings()
    if epsilon is not None:
        dq["epsilon"] = epsilon
    return dict(
        N=N, L=L, n_bars=nb, seed=seed,
        features=feats, prices=prices,
        weights=dqn_weights(seed, bias_scale),
        starts=episode_starts(N, L, nb, seed),
        sampler_seed=sampler_seed(seed),
        settings=settings(),
        dqn=dq,
    )
