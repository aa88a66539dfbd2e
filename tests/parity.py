"""The comparison protocol of the GPU parity tests (test infrastructure): run
the HIP path and the oracle on the same seeded inputs and compare them.

PPO collection, fp32 (the stated tolerances):
* integer outputs (actions, dones, barrier codes) bit-exact;
* fp32 outputs within |g - o| <= 1e-5 + 1e-4 |o|;
* at the first action mismatch of an episode, the oracle's distance from u to
  the CDF boundary between the two actions decides: below 1e-6 the draw is a
  near tie, and the episode is re-run in the oracle with the GPU's actions
  teacher-forced and compared again by the rules above; otherwise it fails.

PPO collection, bf16 (the GPU's bf16 run against the oracle's bf16 mode with
the GPU's actions teacher-forced):
* integers bit-exact, states within the fp32 tolerance (the portfolio
  features are fp32 arithmetic on both sides);
* every other float within |g - o| <= floor + 2e-2 |o| element by element,
  where the floor of an output is the median change of that output when one
  hidden-layer input of its network moves to a neighbouring bf16 value (the
  GPU and the oracle sum in different orders, so a layer input that sits at
  a bf16 rounding boundary may round the other way on one side); elements
  beyond it are outliers, held to a fixed budget per output (at most
  max(2, 1e-3 of the elements)) and to a hard cap of 2e-2 max(|o|, rms(o))
  each;
* advantages are returns minus values (A = R - V, exact in fp32 up to one
  rounding), so an advantage's error is at most its return's plus its
  value's: its tolerance and cap are the sums of theirs at the same element
  (where |V| is much larger than |A|, a value's bf16 error within its own
  tolerance is a large fraction of the advantage).

DQN collection: integers (actions, explore flags, dones, barrier codes)
bit-exact; states, next states, Q values, Q(s,a), max Q_target and rewards
within the fp32 tolerance; the TD error, a difference of terms that each carry
that tolerance, within 1e-5 + 1e-4 (|r| + gamma |max Q_t| + |Q(s,a)|); the
priority as |td|^alpha of the GPU's own td; at the first action mismatch a
greedy step whose oracle gap between its two largest Q values is below
1e-5 (1 + max |Q|) is a near tie and the episode is re-run teacher-forced.

Every comparison appends what it saw (near-tie flags, near-boundary draws,
outlier counts, agreement) to a JSON-lines record at the path in the
environment variable PARITY_RECORD, when it is set.
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle

ATOL, RTOL = 1e-5, 1e-4
NEAR_TIE = 1e-6
FLOAT_KEYS = ("states", "logits", "log_probs", "values", "rewards", "advantages", "returns")
INT_KEYS = ("actions", "dones", "barrier")
ORACLE_NAME = {"advantages": "adv", "returns": "ret"}

BF16_RTOL = 2e-2
BF16_BUDGET_FRAC = 1e-3
BF16_BUDGET_MIN = 2

DQN_INT_KEYS = ("actions", "explored", "dones", "barrier")
DQN_FLOAT_KEYS = ("states", "next_states", "q_values", "q_taken", "q_next_max", "rewards")
DQN_TIE = 1e-5


def record(name: str, **data):
    """Append one JSON line describing a comparison to the parity record
    (the file PARITY_RECORD names; nothing when it is unset)."""
    path = os.environ.get("PARITY_RECORD")
    if not path:
        return
    try:
        os.makedirs(os.path.dirname(path), exist_ok=True)
        with open(path, "a") as f:
            f.write(json.dumps(dict(test=name, **data), default=float) + "\n")
    except OSError:
        pass


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def to_device(inputs: dict, device="cuda"):
    import torch
    w = inputs["weights"]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return dict(
        weights=dict(actor=[dev(x) for x in w["actor"]], critic=[dev(x) for x in w["critic"]],
                     curiosity=[dev(x) for x in w["curiosity"]]),
        features=dev(inputs["features"]), prices=dev(inputs["prices"]),
        starts=dev(inputs["starts"].astype(np.int32)),
    )


def run_gpu(inputs: dict, logits: bool = True, settings: dict | None = None, precision: int = 0,
            seed: int | None = None):
    import torch
    import rl_experience_collection_amd as rx
    d = to_device(inputs)
    col = rx.Collector(inputs["N"], inputs["L"], d["weights"], d["features"], d["prices"],
                       settings=settings or inputs["settings"], precision=precision)
    out = col.collect(d["starts"], inputs["sampler_seed"] if seed is None else seed, logits=logits)
    torch.cuda.synchronize()
    res = {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}
    col.close()
    return res


def close_mask(g, o, rtol=RTOL, atol=ATOL):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    return np.abs(g - o) <= atol + rtol * np.abs(o)


def boundary_gap(logits, u, a_gpu, a_orc) -> float:
    _, _, cdf, _ = oracle.softmax_sample(logits, u)
    lo, hi = min(a_gpu, a_orc), max(a_gpu, a_orc)
    return float(np.min(np.abs(cdf[lo:hi].astype(np.float64) - float(u))))


def _first_float_failure(g, o, cols, rtol, atol):
    """(episode, index within the episode) of the first element outside the
    tolerance, or None; g and o are [L, N, ...] arrays restricted to cols."""
    ok = close_mask(g, o, rtol, atol)
    if ok.all():
        return None
    idx = np.argwhere(~ok)
    j = int(np.argmin(idx[:, 1]))  # the lowest compared episode position
    t = tuple(int(x) for x in idx[j])
    return cols[t[1]], (t[0],) + t[2:]


def compare_rollout(inputs: dict, gpu: dict, orc: dict, episodes=None, rtol=RTOL, atol=ATOL,
                    precision: int = 0, settings: dict | None = None, report: dict | None = None):
    """Compare the given episode columns; returns the list of failure strings.
    report (optional) receives the near-tie flags and the number of oracle
    draws that lay within NEAR_TIE of a CDF boundary."""
    L, N = gpu["actions"].shape
    cols = list(range(N)) if episodes is None else list(episodes)
    c = np.asarray(cols, np.int64)
    fails, flagged = [], []
    mism_cols = np.nonzero((gpu["actions"][:, c] != orc["actions"][:, c]).any(axis=0))[0]
    rerun = {}
    for pos in mism_cols:
        n = cols[pos]
        t = int(np.nonzero(gpu["actions"][:, n] != orc["actions"][:, n])[0][0])
        gap = boundary_gap(orc["logits"][t, n], orc["u"][t, n], int(gpu["actions"][t, n]),
                           int(orc["actions"][t, n]))
        if gap >= NEAR_TIE:
            fails.append(f"episode {n} step {t}: action {gpu['actions'][t, n]} vs "
                         f"{orc['actions'][t, n]}, gap {gap:.3g} >= {NEAR_TIE}")
            continue
        flagged.append((n, t, gap))
        forced = np.zeros((L, N), np.int32)
        forced[:, n] = gpu["actions"][:, n]
        rerun[n] = oracle.rollout(inputs, precision=precision, forced_actions=forced, subset=[n],
                                  settings=settings)
    bad_pos = set(int(p) for p in mism_cols if cols[p] not in rerun)
    plain = np.asarray([p for p in range(len(cols)) if p not in bad_pos and cols[p] not in rerun],
                       np.int64)
    pc = c[plain] if plain.size else plain
    groups = [(pc, orc)] + [(np.asarray([n]), o) for n, o in rerun.items()]
    for cc, o in groups:
        if cc.size == 0:
            continue
        cl = [int(x) for x in cc]
        for k in INT_KEYS:
            d = gpu[k][:, cc] != o[k][:, cc]
            if d.any():
                t, p = (int(x) for x in np.argwhere(d)[0])
                fails.append(f"episode {cl[p]}: {k} differs first at step {t}")
        for k in FLOAT_KEYS:
            if gpu.get(k) is None:
                continue
            ok = ORACLE_NAME.get(k, k)
            r = _first_float_failure(gpu[k][:, cc], o[ok][:, cc], cl, rtol, atol)
            if r is not None:
                n, idx = r
                p = cl.index(n)
                g = gpu[k][:, cc][(idx[0], p) + idx[1:]]
                v = o[ok][:, cc][(idx[0], p) + idx[1:]]
                fails.append(f"episode {n}: {k} at {idx}: gpu {g!r} oracle {v!r}")
    if report is not None:
        report["flagged"] = flagged
        if orc.get("cdf_gap") is not None:
            report["near_boundary_draws"] = int((orc["cdf_gap"][:, c] < NEAR_TIE).sum())
        report["draws"] = int(L * len(cols))
    return fails


# ----------------------------------------------------------------------- bf16
def bf16_floors(inputs: dict, forced: dict, cols, rows: int = 600, seed: int = 0) -> dict:
    """Absolute floor of the bf16 gate per output: the median change of that
    output when one nonzero hidden-layer input of its network, chosen at
    random in each of up to `rows` compared rows, moves to a neighbouring bf16
    value.  Advantages and returns take (1 + gamma) times the values' floor
    (one value enters two TD residuals); log-probabilities twice the logits'
    (log p_a = l_a - log sum exp l)."""
    from nets_ref import ACTOR_RELU, CRITIC_RELU, CURIOSITY_RELU, flip_effects
    rng = np.random.default_rng(seed)
    L = forced["actions"].shape[0]
    c = np.asarray(list(cols), np.int64)
    s = forced["states"][:, c].reshape(-1, 54).astype(np.float64)
    pick = rng.choice(s.shape[0], size=min(rows, s.shape[0]), replace=False)
    w = inputs["weights"]
    dv = flip_effects(w["critic"], s[pick], CRITIC_RELU, rng)[:, 0]
    dl = flip_effects(w["actor"], s[pick], ACTOR_RELU, rng)
    # curiosity: rows whose next state is the next bar (no done, not the last step)
    a = forced["actions"][:, c].reshape(-1)
    done = forced["dones"][:, c].reshape(-1)
    tt = np.repeat(np.arange(L), c.size)
    ok = np.nonzero((tt < L - 1) & (done == 0))[0]
    dr = np.zeros(1)
    if ok.size:
        sel = rng.choice(ok, size=min(rows, ok.size), replace=False)
        x = np.concatenate([s[sel], np.eye(45)[a[sel]]], axis=1)
        nxt = forced["states"][:, c].reshape(-1, 54)[sel + c.size, :51].astype(np.float64)
        from nets_ref import forward_inputs
        _, pred = forward_inputs(w["curiosity"], x, CURIOSITY_RELU)
        dp = flip_effects(w["curiosity"], x, CURIOSITY_RELU, rng)
        d = pred - nxt
        coef = inputs["settings"]["curiosity_coef"]
        # the signed change of each prediction is not kept; |d| |dp| bounds
        # the first-order change of each squared error
        dr = coef * (2 * np.abs(d) * dp + dp * dp).sum(axis=1) / 51.0
    gamma = inputs["settings"]["gamma"]
    fv = float(np.median(dv))
    fl = float(np.median(dl))
    return dict(values=fv, logits=fl, log_probs=2 * fl, rewards=float(np.median(dr)),
                advantages=(1 + gamma) * fv, returns=(1 + gamma) * fv)


def compare_bf16(inputs: dict, gpu: dict, forced: dict, cols, floors: dict):
    """The bf16 gate over the given episode columns.  Returns (fails, stats):
    stats[k] = dict(n, outliers, budget, worst_excess, max_err_over_cap,
    floor)."""
    c = np.asarray(list(cols), np.int64)
    fails, stats = [], {}
    for k in ("dones", "barrier"):
        if not np.array_equal(gpu[k][:, c], forced[k][:, c]):
            fails.append(f"bf16: {k} differs")
    g, o = gpu["states"][:, c], forced["states"][:, c]
    if not close_mask(g, o).all():
        fails.append("bf16: states outside the fp32 tolerance")
    def tol_cap(k):
        o = forced[ORACLE_NAME.get(k, k)][:, c].astype(np.float64)
        if k == "advantages":  # A = R - V: the sums of the return's and the value's
            tr, cr = tol_cap("returns")
            tv, cv = tol_cap("values")
            return tr + tv, cr + cv
        rms = float(np.sqrt((o * o).mean())) if o.size else 0.0
        return (floors[k] + BF16_RTOL * np.abs(o),
                BF16_RTOL * np.maximum(np.abs(o), rms) + floors[k])

    for k in ("logits", "log_probs", "values", "rewards", "advantages", "returns"):
        if gpu.get(k) is None:
            continue
        g = gpu[k][:, c].astype(np.float64)
        o = forced[ORACLE_NAME.get(k, k)][:, c].astype(np.float64)
        err = np.abs(g - o)
        tol, cap = tol_cap(k)
        out = err > tol
        nout = int(out.sum())
        budget = max(BF16_BUDGET_MIN, int(np.ceil(BF16_BUDGET_FRAC * err.size)))
        over_cap = float((err / cap).max()) if err.size else 0.0
        stats[k] = dict(n=int(err.size), outliers=nout, budget=budget,
                        worst_excess=float((err - tol).max()) if err.size else 0.0,
                        max_err_over_cap=over_cap, floor=floors[k])
        if nout > budget:
            fails.append(f"bf16: {k}: {nout} of {err.size} outside floor + 2e-2 |o| "
                         f"(budget {budget})")
        if over_cap > 1.0:
            fails.append(f"bf16: {k}: an error reaches {over_cap:.3g} x the cap "
                         f"2e-2 max(|o|, rms) + floor")
    return fails, stats


# ------------------------------------------------------------------------ DQN
def compare_dqn(inputs: dict, gpu: dict, orc: dict, episodes=None, report=None):
    L, N = gpu["actions"].shape
    gamma, alpha = inputs["dqn"]["gamma"], inputs["dqn"]["alpha"]
    fails, flagged = [], []
    for n in (range(N) if episodes is None else episodes):
        o = orc
        mism = np.nonzero(gpu["actions"][:, n] != orc["actions"][:, n])[0]
        if mism.size:
            t = int(mism[0])
            q = orc["q_values"][t, n] if orc.get("q_values") is not None else None
            scale = 1.0 + (float(np.abs(q).max()) if q is not None
                           else abs(float(orc["q_taken"][t, n])))
            tie = (orc["explored"][t, n] == 0 and gpu["explored"][t, n] == 0
                   and orc["q_gap"][t, n] < DQN_TIE * scale)
            if not tie:
                fails.append(f"episode {n} step {t}: action {gpu['actions'][t, n]} vs "
                             f"{orc['actions'][t, n]} (gap {orc['q_gap'][t, n]:.3g})")
                continue
            flagged.append((n, t, float(orc["q_gap"][t, n])))
            forced = np.zeros((L, N), np.int32)
            forced[:, n] = gpu["actions"][:, n]
            o = oracle.dqn_rollout(inputs, forced_actions=forced, subset=[n])
        for k in DQN_INT_KEYS:
            if gpu.get(k) is None:
                continue
            if not np.array_equal(gpu[k][:, n], o[k][:, n]):
                t = int(np.nonzero(gpu[k][:, n] != o[k][:, n])[0][0])
                fails.append(f"episode {n}: {k} differs first at step {t}")
        for k in DQN_FLOAT_KEYS:
            if gpu.get(k) is None or o.get(k) is None:
                continue
            ok = close_mask(gpu[k][:, n], o[k][:, n])
            if not ok.all():
                idx = tuple(np.argwhere(~ok)[0])
                fails.append(f"episode {n}: {k} at {idx}: gpu {gpu[k][:, n][idx]!r} "
                             f"oracle {o[k][:, n][idx]!r}")
        scale = (np.abs(o["rewards"][:, n]) + gamma * np.abs(o["q_next_max"][:, n])
                 + np.abs(o["q_taken"][:, n])).astype(np.float64)
        err = np.abs(gpu["td"][:, n].astype(np.float64) - o["td"][:, n])
        if not (err <= 1e-5 + 1e-4 * scale).all():
            t = int(np.argmax(err - 1e-4 * scale))
            fails.append(f"episode {n}: td at {t}: gpu {gpu['td'][t, n]!r} oracle {o['td'][t, n]!r}")
    # the priority is |td|^alpha of the GPU's own td, everywhere
    want = np.abs(gpu["td"].astype(np.float64)) ** alpha
    if not np.allclose(gpu["priorities"], want, rtol=5e-6, atol=1e-30):
        fails.append("priorities differ from |td|^alpha")
    if report is not None:
        report["flagged"] = flagged
    return fails
