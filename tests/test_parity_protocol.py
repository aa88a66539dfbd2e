"""The GPU-vs-oracle comparison protocol (tests/parity.py), checked on the
CPU: the oracle stands in for the GPU, and mistakes are planted in its
outputs, so each rule of the protocol is seen to pass what it must pass and
to fail what it must fail."""
import copy

import numpy as np
import pytest

import oracle
import synthdata
from parity import (ATOL, BF16_RTOL, RTOL, bf16_floors, compare_bf16, compare_dqn,
                    compare_rollout)


@pytest.fixture(scope="module")
def run():
    inp = synthdata.ppo_inputs(dict(N=12, L=70, n_bars=3000, seed=91), bias_scale=0.1)
    return inp, oracle.rollout(inp)


def _swapped(inp, orc, n, t):
    """A trajectory that differs from the oracle's at (t, n) only by the next
    action, with every output the oracle gives for it."""
    a = orc["actions"].copy()
    a0 = int(a[t, n])
    a[t, n] = a0 + 1 if a0 < 44 else a0 - 1
    return oracle.rollout(inp, forced_actions=a), a0, int(a[t, n])


def test_identical_outputs_pass(run):
    inp, orc = run
    rep = {}
    assert compare_rollout(inp, copy.deepcopy(orc), orc, report=rep) == []
    assert rep["flagged"] == [] and rep["draws"] == 12 * 70


def test_near_tie_swap_is_flagged_and_passes_teacher_forced(run):
    inp, orc = run
    n, t = 5, 17
    gpu, a0, a1 = _swapped(inp, orc, n, t)
    o = copy.deepcopy(orc)
    _, _, cdf, _ = oracle.softmax_sample(orc["logits"][t, n], orc["u"][t, n])
    o["u"][t, n] = cdf[min(a0, a1)]  # the draw sits on the boundary between the two
    rep = {}
    assert compare_rollout(inp, gpu, o, report=rep) == []
    assert [(f[0], f[1]) for f in rep["flagged"]] == [(n, t)]


def test_far_from_tie_swap_fails(run):
    inp, orc = run
    n, t = 5, 17
    gpu, _, _ = _swapped(inp, orc, n, t)
    _, _, cdf, gap = oracle.softmax_sample(orc["logits"][t, n], orc["u"][t, n])
    assert gap > 1e-6  # this seed's draw is not near a boundary
    fails = compare_rollout(inp, gpu, orc)
    assert len(fails) == 1 and f"episode {n} step {t}" in fails[0] and "gap" in fails[0]


@pytest.mark.parametrize("key", ["values", "logits", "advantages", "states", "rewards"])
def test_float_tolerance_edges(run, key):
    inp, orc = run
    ok = orc["adv" if key == "advantages" else key]
    gpu = copy.deepcopy(orc)
    gpu["advantages"], gpu["returns"] = orc["adv"].copy(), orc["ret"].copy()
    g = gpu[key]
    idx = (33, 7) + ((3,) if g.ndim == 3 else ())
    tol = ATOL + RTOL * abs(float(ok[idx]))
    g[idx] = np.float32(float(ok[idx]) + 0.5 * tol)
    assert compare_rollout(inp, gpu, orc) == []
    g[idx] = np.float32(float(ok[idx]) + 3.0 * tol)
    fails = compare_rollout(inp, gpu, orc)
    assert len(fails) == 1 and key in fails[0] and "episode 7" in fails[0]


@pytest.mark.parametrize("key", ["dones", "barrier"])
def test_integer_mismatch_fails(run, key):
    inp, orc = run
    gpu = copy.deepcopy(orc)
    gpu["advantages"], gpu["returns"] = orc["adv"], orc["ret"]
    gpu[key][40, 2] ^= 1
    fails = compare_rollout(inp, gpu, orc)
    assert any(key in f and "episode 2" in f for f in fails)


# ----------------------------------------------------------------------- bf16
@pytest.fixture(scope="module")
def bf16_run():
    inp = synthdata.ppo_inputs(dict(N=16, L=100, n_bars=3000, seed=92), bias_scale=0.1)
    forced = oracle.rollout(inp, precision=oracle.BF16)
    gpu = copy.deepcopy(forced)
    gpu["advantages"], gpu["returns"] = forced["adv"].copy(), forced["ret"].copy()
    cols = list(range(16))
    return inp, gpu, forced, cols, bf16_floors(inp, forced, cols)


def test_bf16_floors_are_far_below_the_scale(bf16_run):
    """The floor is one rounding decision's effect: far below 2e-2 of an
    output's rms, and above zero."""
    inp, _, forced, _, fl = bf16_run
    for k, ko in (("values", "values"), ("logits", "logits"), ("advantages", "adv")):
        rms = float(np.sqrt((forced[ko].astype(np.float64) ** 2).mean()))
        assert 0 < fl[k] < 0.25 * BF16_RTOL * rms, (k, fl[k], rms)


def test_bf16_identical_passes(bf16_run):
    inp, gpu, forced, cols, fl = bf16_run
    fails, st = compare_bf16(inp, gpu, forced, cols, fl)
    assert fails == [] and all(v["outliers"] == 0 for v in st.values())


def test_bf16_outlier_budget(bf16_run):
    """Outliers (beyond floor + 2e-2 |o|, within the cap 2e-2 max(|o|, rms))
    can only sit where |o| is below the rms: up to the budget they pass, one
    more fails."""
    inp, gpu0, forced, cols, fl = bf16_run
    o = forced["values"].astype(np.float64).ravel()
    rms = np.sqrt((o * o).mean())
    budget = max(2, int(np.ceil(1e-3 * o.size)))
    small = np.argsort(np.abs(o))[: budget + 1]
    gpu = copy.deepcopy(gpu0)
    v = gpu["values"].reshape(-1)

    def plant(i):
        tol = fl["values"] + BF16_RTOL * abs(o[i])
        cap = fl["values"] + BF16_RTOL * max(abs(o[i]), rms)
        v[i] = np.float32(o[i] + 0.5 * (tol + cap))

    for i in small[:budget]:
        plant(i)
    fails, st = compare_bf16(inp, gpu, forced, cols, fl)
    assert fails == [] and st["values"]["outliers"] == budget
    plant(small[budget])
    fails, _ = compare_bf16(inp, gpu, forced, cols, fl)
    assert len(fails) == 1 and "values" in fails[0] and "budget" in fails[0]


def test_bf16_hard_cap(bf16_run):
    inp, gpu0, forced, cols, fl = bf16_run
    gpu = copy.deepcopy(gpu0)
    o = forced["values"].astype(np.float64)
    rms = np.sqrt((o * o).mean())
    i = int(np.argmin(np.abs(o).ravel()))
    gpu["values"].reshape(-1)[i] = np.float32(o.ravel()[i] + 1.1 * (BF16_RTOL * rms + fl["values"]))
    fails, _ = compare_bf16(inp, gpu, forced, cols, fl)
    assert any("cap" in f for f in fails)


def test_bf16_advantage_takes_return_and_value_tolerance(bf16_run):
    """An advantage is its return minus its value, so its error may reach
    the return's and the value's tolerances together: at the element where
    the value is largest against the advantage such an error passes (though
    it is beyond 2e-2 |A| plus the advantages' own floor), and budget + 1
    errors of 1.5 times that tolerance fail."""
    inp, gpu0, forced, cols, fl = bf16_run
    A = forced["adv"].astype(np.float64).ravel()
    R = forced["ret"].astype(np.float64).ravel()
    V = forced["values"].astype(np.float64).ravel()
    tol = (fl["returns"] + BF16_RTOL * np.abs(R)) + (fl["values"] + BF16_RTOL * np.abs(V))
    order = np.argsort(-(np.abs(V) / (np.abs(A) + 1e-6)))
    budget = max(2, int(np.ceil(1e-3 * A.size)))
    gpu = copy.deepcopy(gpu0)
    a = gpu["advantages"].reshape(-1)
    i = order[0]
    a[i] = np.float32(A[i] + 0.9 * tol[i])
    assert 0.9 * tol[i] > fl["advantages"] + BF16_RTOL * abs(A[i])
    fails, st = compare_bf16(inp, gpu, forced, cols, fl)
    assert fails == [] and st["advantages"]["outliers"] == 0
    for j in order[: budget + 1]:
        a[j] = np.float32(A[j] + 1.5 * tol[j])
    fails, _ = compare_bf16(inp, gpu, forced, cols, fl)
    assert any("advantages" in f and "budget" in f for f in fails)


def test_bf16_integer_and_state_mismatch(bf16_run):
    inp, gpu0, forced, cols, fl = bf16_run
    gpu = copy.deepcopy(gpu0)
    gpu["barrier"][10, 3] = 3 - gpu["barrier"][10, 3]
    gpu["states"][20, 4, 51] += 1e-3
    fails, _ = compare_bf16(inp, gpu, forced, cols, fl)
    assert any("barrier" in f for f in fails) and any("states" in f for f in fails)


# ------------------------------------------------------------------------ DQN
@pytest.fixture(scope="module")
def dqn_run():
    inp = synthdata.dqn_inputs(dict(N=10, L=40, n_bars=3000, seed=93), bias_scale=0.1)
    return inp, oracle.dqn_rollout(inp)


def _as_gpu(o):
    """An oracle DQN output under the GPU binding's names."""
    g = copy.deepcopy(o)
    g["priorities"] = g.pop("priority")
    return g


def test_dqn_identical_passes(dqn_run):
    inp, orc = dqn_run
    rep = {}
    assert compare_dqn(inp, _as_gpu(orc), orc, report=rep) == []
    assert rep["flagged"] == []


def _dqn_swap(inp, orc):
    """First greedy step of episode 3 with the second-best action forced."""
    n = 3
    t = int(np.nonzero(orc["explored"][:, n] == 0)[0][0])
    q = orc["q_values"][t, n]
    a = orc["actions"].copy()
    a[t, n] = int(np.argsort(-q, kind="stable")[1])
    return n, t, _as_gpu(oracle.dqn_rollout(inp, forced_actions=a))


def test_dqn_near_tie_is_flagged_and_passes(dqn_run):
    inp, orc = dqn_run
    n, t, gpu = _dqn_swap(inp, orc)
    gpu["explored"] = orc["explored"].copy()
    o = copy.deepcopy(orc)
    o["q_gap"][t, n] = 0.0  # the two largest Q values coincide
    rep = {}
    assert compare_dqn(inp, gpu, o, report=rep) == []
    assert [(f[0], f[1]) for f in rep["flagged"]] == [(n, t)]


def test_dqn_far_swap_and_td_and_priority_fail(dqn_run):
    inp, orc = dqn_run
    n, t, gpu = _dqn_swap(inp, orc)
    gpu["explored"] = orc["explored"].copy()
    assert orc["q_gap"][t, n] > 1e-3
    fails = compare_dqn(inp, gpu, orc)
    assert any(f"episode {n} step {t}" in f for f in fails)
    g = _as_gpu(orc)
    g["td"][5, 1] += 1e-2
    fails = compare_dqn(inp, g, orc)
    assert any("td" in f for f in fails) and any("priorities" in f for f in fails)
    g = _as_gpu(orc)
    g["priorities"][5, 1] *= 1.001
    assert any("priorities" in f for f in compare_dqn(inp, g, orc))
