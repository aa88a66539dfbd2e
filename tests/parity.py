"""Shared helpers of the GPU parity tests: run the HIP path and the oracle on
the same seeded inputs and compare them by the protocol

* integer outputs (actions, dones, barrier codes) bit-exact;
* fp32 outputs within |g - o| <= 1e-5 + 1e-4 |o| (bf16: 1e-5 + 2e-2 |o|);
* at the first action mismatch of an episode, the oracle's distance from u to
  the CDF boundary between the two actions decides: below 1e-6 the draw is a
  near tie, and the episode is re-run in the oracle with the GPU's actions
  teacher-forced and compared again by the rules above; otherwise it fails.
"""
from __future__ import annotations

import numpy as np

import oracle

ATOL, RTOL = 1e-5, 1e-4
NEAR_TIE = 1e-6
FLOAT_KEYS = ("states", "logits", "log_probs", "values", "rewards", "advantages", "returns")
INT_KEYS = ("actions", "dones", "barrier")
ORACLE_NAME = {"advantages": "adv", "returns": "ret"}


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


def compare_rollout(inputs: dict, gpu: dict, orc: dict, episodes=None, rtol=RTOL, atol=ATOL,
                    precision: int = 0, settings: dict | None = None, report: dict | None = None):
    """Compare the given episode columns; returns the list of failure strings."""
    L, N = gpu["actions"].shape
    cols = range(N) if episodes is None else episodes
    fails = []
    flagged = []
    for n in cols:
        o = orc
        mism = np.nonzero(gpu["actions"][:, n] != orc["actions"][:, n])[0]
        if mism.size:
            t = int(mism[0])
            gap = boundary_gap(orc["logits"][t, n], orc["u"][t, n], int(gpu["actions"][t, n]),
                               int(orc["actions"][t, n]))
            if gap >= NEAR_TIE:
                fails.append(f"episode {n} step {t}: action {gpu['actions'][t, n]} vs "
                             f"{orc['actions'][t, n]}, gap {gap:.3g} >= {NEAR_TIE}")
                continue
            flagged.append((n, t, gap))
            forced = np.zeros((L, N), np.int32)
            forced[:, n] = gpu["actions"][:, n]
            o = oracle.rollout(inputs, precision=precision, forced_actions=forced, subset=[n],
                               settings=settings)
        for k in INT_KEYS:
            if not np.array_equal(gpu[k][:, n], o[k][:, n]):
                t = int(np.nonzero(gpu[k][:, n] != o[k][:, n])[0][0])
                fails.append(f"episode {n}: {k} differs first at step {t}")
        for k in FLOAT_KEYS:
            if gpu.get(k) is None:
                continue
            ok = close_mask(gpu[k][:, n], o[ORACLE_NAME.get(k, k)][:, n], rtol, atol)
            if not ok.all():
                idx = np.argwhere(~ok)[0]
                g = gpu[k][:, n][tuple(idx)]
                r = o[ORACLE_NAME.get(k, k)][:, n][tuple(idx)]
                fails.append(f"episode {n}: {k} at {tuple(idx)}: gpu {g!r} oracle {r!r}")
    if report is not None:
        report["flagged"] = flagged
    return fails
