"""Pins for the oracle's environment step: 45-action factorisation, portfolio,
triple barrier and diversity entropy (GPU Pipeline Phase 2b, Kernel Components
2-6; PPO CUDA Pipeline Design, Phase A steps 6-8; Fused CUDA Training Kernel,
Task 1 step 3)."""
import itertools
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
EXP = (-1.0, -0.5, 0.0, 0.5, 1.0)
COST = (0.0002, 0.0005, 0.001)


def test_factorisation_round_trip(settings):
    rows = oracle.action_maps(settings)
    assert len(rows) == 45
    seen = set()
    for a, (x, o, u, cat, e, c) in enumerate(rows):
        assert 0 <= x < 5 and 0 <= o < 3 and 0 <= u < 3
        assert a == 9 * x + 3 * o + u
        seen.add((x, o, u))
        assert e == np.float32(EXP[x])
        assert c == pytest.approx(COST[o] * (1 + 0.5 * u), rel=1e-7)
        assert cat == (0 if x <= 1 else (1 if x == 2 else 2))
    assert len(seen) == 45


def test_constant_price_pays_only_costs(settings):
    g = np.random.default_rng(0)
    env = oracle.Env(settings)
    V = 1.0
    e_prev = 0.0
    for t, a in enumerate(g.integers(0, 45, 200)):
        out = env.step(int(a), t, 123.25, 123.25)
        e = EXP[a // 9]
        c = np.float32(np.float32(COST[(a % 9) // 3]) * np.float32(1 + 0.5 * (a % 3)))
        assert out["pnl"] == -np.float32(c * np.float32(abs(e - e_prev)))
        V = np.float32(V * np.float32(1 + out["pnl"]))
        assert out["V"] == V
        e_prev = e
        if out["done"]:  # only time exits can fire at a constant price
            assert out["code"] == 3
            env.reset()
            V, e_prev = 1.0, 0.0


def test_always_flat_keeps_value_one(settings):
    g = np.random.default_rng(1)
    env = oracle.Env(settings)
    p = 100 * np.exp(np.cumsum(0.01 * g.standard_normal(300))).astype(np.float32)
    for t in range(299):
        out = env.step(18 + t % 9, t, p[t], p[t + 1])
        assert out["pnl"] == 0.0 and out["V"] == 1.0 and not out["done"]


def test_long_path_value_closed_form():
    """Long 1.0 held with profit/stop far away: V = prod(1 + (m_k - 1)) - first cost,
    computed in fp64 and compared to the fp32 oracle."""
    st = dict(oracle_settings())
    st["profit_take"], st["stop_loss"], st["max_hold"] = 10.0, 0.99, 10**6
    env = oracle.Env(st)
    g = np.random.default_rng(2)
    p = (100 * np.exp(np.cumsum(0.01 * g.standard_normal(120)))).astype(np.float32)
    V = 1.0
    for t in range(119):
        a = 36 + (t % 3)  # long 1.0, varying urgency (cost only paid on the open)
        out = env.step(a, t, p[t], p[t + 1])
        cost = COST[0] * (1 + 0.5 * (a % 3)) if t == 0 else 0.0
        V *= 1 + (float(p[t + 1]) / float(p[t]) - 1) - cost
        assert out["V"] == pytest.approx(V, rel=2e-6)


def oracle_settings():
    import synthdata
    return synthdata.settings()


def _scenarios():
    scen, cur = [], None
    for line in open(os.path.join(GOLDEN, "barrier_paths.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        parts = line.split()
        if parts[0] == "scenario":
            cur = (parts[1], [])
            scen.append(cur)
        else:
            reps = 1
            if parts[0] == "repeat":
                reps = int(parts[1])
                parts = parts[2:]
            assert parts[0] == "step"
            a, p0, p1, code, hit, done = parts[1:]
            cur[1].extend([(int(a), float(p0), float(p1), int(code), int(hit), int(done))] * reps)
    return scen


@pytest.mark.parametrize("name,steps", _scenarios(), ids=[s[0] for s in _scenarios()])
def test_barrier_paths(settings, name, steps):
    env = oracle.Env(settings)
    for t, (a, p0, p1, code, hit, done) in enumerate(steps):
        out = env.step(a, t, p0, p1)
        assert (out["code"], out["hit"], int(out["done"])) == (code, hit, done), (name, t)
        if out["done"]:
            env.reset()


def entropy64(counts):
    n = sum(counts)
    return -sum(c / n * math.log(c / n) for c in counts if c > 0)


def test_entropy_all_triples_and_threshold_margin():
    worst = 1.0
    for n0, n1, n2 in itertools.product(range(21), repeat=3):
        n = n0 + n1 + n2
        if n < 1 or n > 20:
            continue
        h = oracle.entropy3(n0, n1, n2)
        h64 = entropy64((n0, n1, n2))
        assert abs(h - h64) <= 1e-6
        assert (h < 1.0) == (h64 < 1.0)
        worst = min(worst, abs(h64 - 1.0))
    # no count triple of a 20-wide window lies within 1.4e-3 nat of the threshold
    assert worst > 1.4e-3
    assert entropy64((3, 7, 10)) == pytest.approx(0.99858, abs=1e-5)


def test_diversity_window_slides(settings):
    """The penalty follows the entropy of the classes of the last <= 20 actions
    since the last reset (fp64 recomputation from the action list)."""
    g = np.random.default_rng(3)
    st = dict(settings)
    st["max_hold"] = 10**6
    st["profit_take"] = st["stop_loss"] = 0.9
    env = oracle.Env(st)
    hist = []
    for t in range(400):
        a = int(g.choice([0, 9, 18, 27, 36], p=[0.1, 0.1, 0.5, 0.15, 0.15]) + g.integers(0, 9))
        out = env.step(a, t, 100.0, 100.0)
        hist.append(0 if a // 9 <= 1 else (1 if a // 9 == 2 else 2))
        win = hist[-20:]
        h = entropy64([win.count(c) for c in range(3)])
        assert out["div"] == (np.float32(-0.1) if h < 1.0 else 0.0), t
    assert out["done"] is False
