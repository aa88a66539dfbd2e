"""GPU parity of the whole collection (rollout_collect) against the oracle,
through the C ABI, on the seeded workloads and edge cases."""
import numpy as np
import pytest

import oracle
import synthdata
from parity import (bf16_floors, close_mask, compare_bf16, compare_rollout, gpu_available,
                    record, run_gpu)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]


def _assert_parity(inp, gpu, orc, episodes=None, name=None, **kw):
    """The fp32 protocol; the near-tie flags and the oracle's near-boundary
    draws go to the parity record.  A flagged episode's first mismatch lies
    within 1e-6 of a CDF boundary by construction, so flags never exceed the
    near-boundary draws."""
    rep = {}
    fails = compare_rollout(inp, gpu, orc, episodes=episodes, report=rep, **kw)
    record(name or "rollout", N=inp["N"], L=inp["L"], episodes=rep["draws"] // inp["L"],
           flagged=len(rep["flagged"]), near_boundary_draws=rep.get("near_boundary_draws"),
           draws=rep["draws"], first_flags=rep["flagged"][:5], failures=len(fails))
    assert not fails, "\n".join(fails[:20])
    if rep.get("near_boundary_draws") is not None:
        assert len(rep["flagged"]) <= rep["near_boundary_draws"]
    return rep


def test_tiny_workload_n16_l100():
    inp = synthdata.ppo_inputs("ppo_n16_l100")
    _assert_parity(inp, run_gpu(inp), oracle.rollout(inp))


def test_tiny_workload_with_random_biases():
    inp = synthdata.ppo_inputs("ppo_n16_l100", bias_scale=0.2)
    _assert_parity(inp, run_gpu(inp), oracle.rollout(inp))


@pytest.mark.parametrize("N,L", [(1, 1), (1, 7), (19, 37), (33, 64), (47, 3)])
def test_ragged_sizes(N, L):
    spec = dict(N=N, L=L, n_bars=3000, seed=100 + N + L)
    inp = synthdata.ppo_inputs(spec, bias_scale=0.1)
    _assert_parity(inp, run_gpu(inp), oracle.rollout(inp))


def test_default_workload_n128_l500():
    inp = synthdata.ppo_inputs("ppo_n128_l500")
    rep = _assert_parity(inp, run_gpu(inp), oracle.rollout(inp), name="ppo_n128_l500_fp32")
    assert len(rep["flagged"]) <= 64


def test_chip_workload_n8192_l500_all_episodes():
    """Full-size launch, every one of the 8192 episodes against the oracle
    (the oracle on all host cores: about 35 s on 16).  Near-boundary draws
    expected: 4,096,000 draws x 44 boundaries x 2e-6 = about 360."""
    inp = synthdata.ppo_inputs("ppo_n8192_l500")
    gpu = run_gpu(inp, logits=True)
    orc = oracle.rollout(inp)
    rep = _assert_parity(inp, gpu, orc, name="ppo_n8192_l500_fp32_all")
    assert 100 < rep["near_boundary_draws"] < 1000
    # every (t, n): integer codes consistent, finite floats
    assert np.array_equal(gpu["dones"], (gpu["barrier"] > 0).astype(np.uint8))
    for k in ("values", "rewards", "advantages", "returns", "log_probs"):
        assert np.isfinite(gpu[k]).all(), k
    assert np.array_equal(gpu["returns"], (gpu["advantages"] + gpu["values"]).astype(np.float32))
    assert int(gpu["counters"][0]) == 0 and int(gpu["counters"][2]) == 0


def test_gae_inside_collect_matches_oracle_gae_on_gpu_streams():
    inp = synthdata.ppo_inputs("ppo_n128_l500")
    gpu = run_gpu(inp, logits=False)
    A, R = oracle.gae(gpu["rewards"], gpu["values"], gpu["dones"], 0.99, 0.95)
    assert close_mask(gpu["advantages"], A).all()
    assert close_mask(gpu["returns"], R).all()


def test_deterministic_and_episode_independent():
    inp = synthdata.ppo_inputs(dict(N=48, L=80, n_bars=5000, seed=7))
    g1 = run_gpu(inp)
    g2 = run_gpu(inp)
    for k in g1:
        if g1[k] is not None and k != "counters":
            assert np.array_equal(g1[k], g2[k]), k
    sub = dict(inp)
    sub["N"] = 16
    sub["starts"] = inp["starts"][:16]
    g3 = run_gpu(sub)
    for k in ("states", "actions", "log_probs", "values", "rewards", "dones", "barrier",
              "advantages", "returns"):
        assert np.array_equal(g3[k], g1[k][:, :16]), k


def test_clamped_starts_are_counted_and_match_clamped_oracle():
    inp = synthdata.ppo_inputs(dict(N=20, L=30, n_bars=400, seed=11))
    bad = inp["starts"].copy()
    bad[3] = -5
    bad[7] = 400 - 30  # one past the last valid start
    bad[8] = 10**6
    gin = dict(inp)
    gin["starts"] = bad
    gpu = run_gpu(gin)
    assert int(gpu["counters"][1]) == 3
    fixed = dict(inp)
    fixed["starts"] = np.clip(bad, 0, 400 - 30 - 1).astype(np.int32)
    _assert_parity(fixed, gpu, oracle.rollout(fixed))


def test_set_weights_takes_effect():
    import torch
    import rl_experience_collection_amd as rx
    from parity import to_device
    a = synthdata.ppo_inputs(dict(N=32, L=40, n_bars=3000, seed=21))
    b = dict(a)
    b["weights"] = synthdata.ppo_weights(99, bias_scale=0.1)
    da, db = to_device(a), to_device(b)
    col = rx.Collector(32, 40, da["weights"], da["features"], da["prices"], settings=a["settings"])
    col.set_weights(db["weights"])
    out = col.collect(da["starts"], a["sampler_seed"], logits=True)
    torch.cuda.synchronize()
    gpu = {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}
    col.close()
    _assert_parity(b, gpu, oracle.rollout(b))


def test_sampler_chi_square_on_gpu():
    """1e6 GPU draws from one fixed logit vector (constant actor output)."""
    from scipy import stats
    inp = synthdata.ppo_inputs(dict(N=8192, L=123, n_bars=2000, seed=5))
    w = inp["weights"]
    g = np.random.default_rng(0)
    logits = (g.standard_normal(45) * 1.5).astype(np.float32)
    w["actor"][4] = np.zeros_like(w["actor"][4])
    w["actor"][5] = logits
    gpu = run_gpu(inp, logits=False)
    n = gpu["actions"].size
    counts = np.bincount(gpu["actions"].ravel(), minlength=45).astype(np.float64)
    p = np.exp(logits.astype(np.float64) - logits.max())
    p /= p.sum()
    exp = p * n
    small = exp < 5
    obs = np.append(counts[~small], counts[small].sum()) if small.any() else counts
    ex = np.append(exp[~small], exp[small].sum()) if small.any() else exp
    chi2 = ((obs - ex) ** 2 / ex).sum()
    assert chi2 < stats.chi2.ppf(1 - 1e-6, obs.size - 1)


# --------------------------------------------------------------------------- bf16
def _bf16_compare(inp, episodes=None, name="bf16"):
    """GPU bf16 collection vs the oracle's bf16 mode with the GPU's actions
    teacher-forced, by the bf16 gate of tests/parity.py: integers bit-exact,
    states at the fp32 tolerance, every other float element-wise within
    floor + 2e-2 |o| up to a fixed outlier budget, the floor being the
    measured effect of one bf16 rounding decision taken the other way.  The
    free-running action agreement is recorded, not gated."""
    gpu = run_gpu(inp, precision=1)
    free = oracle.rollout(inp, precision=oracle.BF16, subset=episodes)
    cols = list(range(inp["N"])) if episodes is None else list(episodes)
    agree = float((free["actions"][:, cols] == gpu["actions"][:, cols]).mean())
    forced = oracle.rollout(inp, precision=oracle.BF16, forced_actions=gpu["actions"], subset=episodes)
    floors = bf16_floors(inp, forced, cols)
    fails, stats = compare_bf16(inp, gpu, forced, cols, floors)
    record(name, N=inp["N"], L=inp["L"], episodes=len(cols), action_agreement=agree,
           outputs=stats, failures=fails)
    assert not fails, "\n".join(fails)
    return agree


def test_bf16_tiny_teacher_forced():
    inp = synthdata.ppo_inputs("ppo_n16_l100", bias_scale=0.1)
    assert _bf16_compare(inp, name="bf16_n16_l100") > 0.5


@pytest.mark.parametrize("N,L", [(1, 1), (47, 3), (33, 64), (129, 9)])
def test_bf16_ragged_sizes(N, L):
    """Row counts below one 128-row work item, ragged tails, several items."""
    spec = dict(N=N, L=L, n_bars=3000, seed=200 + N + L)
    _bf16_compare(synthdata.ppo_inputs(spec, bias_scale=0.1), name=f"bf16_n{N}_l{L}")


def test_bf16_episodes_reaching_the_last_bar():
    """Every episode starts at the last valid start, so the curiosity target
    of the final step is the market's last feature row (the row-end loads)."""
    inp = synthdata.ppo_inputs(dict(N=40, L=30, n_bars=400, seed=17), bias_scale=0.1)
    inp["starts"] = np.full(40, 400 - 30 - 1, dtype=np.int32)
    _bf16_compare(inp)


def test_bf16_chip_workload_sampled_episodes():
    inp = synthdata.ppo_inputs("ppo_n8192_l500")
    sub = sorted(set(list(range(0, 8192, 97)) + [8191]))
    assert _bf16_compare(inp, episodes=sub, name="bf16_n8192_l500_sampled") > 0.9


# ----------------------------------------------------------------- recycling
def _recycled(spec, **kw):
    inp = synthdata.ppo_inputs(spec, **kw)
    inp["settings"] = dict(inp["settings"], recycle=1)
    return inp


@pytest.mark.parametrize("N,L,n_bars", [(16, 100, 3000), (33, 64, 3000), (1, 7, 3000),
                                        (20, 60, 61)])
def test_recycling_matches_oracle(N, L, n_bars):
    """Dynamic episode recycling ("GPU Pipeline Phase 2b", Future Phase 3
    Optimization): same protocol as the plain run; n_bars = L + 1 leaves
    restarts only t + 2 valid bars."""
    inp = _recycled(dict(N=N, L=L, n_bars=n_bars, seed=300 + N + L), bias_scale=0.1)
    gpu = run_gpu(inp)
    _assert_parity(inp, gpu, oracle.rollout(inp))
    if N * L >= 1000:
        assert gpu["dones"][:-1].sum() > 0


def test_recycling_changes_the_run_after_a_done():
    inp = _recycled(dict(N=32, L=120, n_bars=3000, seed=8), bias_scale=0.1)
    plain = dict(inp, settings=dict(inp["settings"], recycle=0))
    g1, g0 = run_gpu(inp), run_gpu(plain)
    d = g0["dones"]
    first = np.where(d.any(axis=0), d.argmax(axis=0), inp["L"])
    moved = 0
    for n in range(inp["N"]):
        f = int(first[n])
        assert np.array_equal(g1["states"][: f + 1, n], g0["states"][: f + 1, n]), n
        if f + 1 < inp["L"]:
            moved += int(not np.array_equal(g1["states"][f + 1, n], g0["states"][f + 1, n]))
    assert moved > 10


def test_recycling_chip_workload_n8192_l500_sampled_episodes():
    inp = _recycled("ppo_n8192_l500")
    gpu = run_gpu(inp, logits=True)
    sub = sorted(set(list(range(0, 8192, 331)) + [8191, 8190, 15, 16]))
    _assert_parity(inp, gpu, oracle.rollout(inp, subset=sub), episodes=sub)
    assert np.array_equal(gpu["dones"], (gpu["barrier"] > 0).astype(np.uint8))
    for k in ("values", "rewards", "advantages", "returns", "log_probs"):
        assert np.isfinite(gpu[k]).all(), k


def test_recycling_bf16_teacher_forced():
    assert _bf16_compare(_recycled("ppo_n16_l100", bias_scale=0.1), name="bf16_recycle_n16_l100") > 0.5


@pytest.mark.parametrize("precision", [0, 1])
def test_wide_collection_n65536_l64_sampled_episodes(precision):
    """N = 65536: the actor launches 4096 workgroups, eight times the resident
    ones, and the value kernel runs 4.2 M rows; a spread of episodes against
    the oracle (fp32 by the parity protocol, bf16 teacher-forced)."""
    inp = synthdata.ppo_inputs(dict(N=65536, L=64, n_bars=200_000, seed=31), bias_scale=0.1)
    sub = sorted(set(list(range(0, 65536, 4093)) + [65535, 32768, 17]))
    if precision == 0:
        gpu = run_gpu(inp, logits=True)
        _assert_parity(inp, gpu, oracle.rollout(inp, subset=sub), episodes=sub)
    else:
        _bf16_compare(inp, episodes=sub, name="bf16_n65536_l64_sampled")


# ------------------------------------- split rollout, overlapped value pass
@pytest.mark.parametrize("N,L,precision,recycle",
                         [(16, 100, 0, 0), (40, 37, 0, 1), (128, 300, 1, 0), (33, 130, 0, 0),
                          (8192, 64, 0, 0), (128, 500, 1, 1)])
def test_split_rollout_equals_one_launch(N, L, precision, recycle):
    """The rollout split into launches of consecutive steps (the episode
    state carried between them), each part's value pass on the handle's
    second stream, gives the single launch's outputs bit for bit."""
    inp = synthdata.ppo_inputs(dict(N=N, L=L, n_bars=3000, seed=300 + N + L), bias_scale=0.1)
    base = dict(inp["settings"], recycle=recycle)
    one = run_gpu(inp, settings=dict(base, overlap=0), precision=precision)
    split = run_gpu(inp, settings=dict(base, overlap=1), precision=precision)
    for k, v in one.items():
        if v is not None:
            assert v.tobytes() == split[k].tobytes(), k


def test_split_rollout_matches_oracle():
    """Parity of the split rollout (3 parts of 45, 45 and 46 steps) with
    the oracle, clamped starts included."""
    inp = synthdata.ppo_inputs(dict(N=24, L=136, n_bars=400, seed=41))
    inp["starts"][5] = 400 - 136 - 1
    gpu = run_gpu(inp, settings=dict(inp["settings"], overlap=1))
    _assert_parity(inp, gpu, oracle.rollout(inp))


# -------------------------------------------------------- failure reporting
def _nan_planted(which):
    inp = synthdata.ppo_inputs(dict(N=40, L=50, n_bars=3000, seed=51), bias_scale=0.1)
    w = inp["weights"]
    if which == "critic":
        w["critic"][11] = np.array([np.nan], np.float32)  # the output bias
    else:
        w["actor"][4] = w["actor"][4].copy()
        w["actor"][4][7, 3] = np.nan  # one weight of the logit layer
    return inp


@pytest.mark.parametrize("which", ["critic", "actor"])
@pytest.mark.parametrize("precision", [0, 1])
def test_nonfinite_weights_are_counted_and_the_collection_completes(which, precision):
    """A NaN in the critic's output bias makes every value non-finite; a NaN
    in one weight of the actor's logit layer makes logit 7 of every step
    non-finite.  The collection completes with valid actions and codes, and
    counters[0] reports the steps (every one of the L x N)."""
    inp = _nan_planted(which)
    gpu = run_gpu(inp, precision=precision)
    L, N = inp["L"], inp["N"]
    assert int(gpu["counters"][0]) == L * N
    assert ((gpu["actions"] >= 0) & (gpu["actions"] < 45)).all()
    assert np.isin(gpu["barrier"], [0, 1, 2, 3]).all()
    if which == "critic":
        assert np.isnan(gpu["values"]).all() and np.isnan(gpu["advantages"]).all()
        assert np.isfinite(gpu["log_probs"]).all()
    else:
        assert np.isnan(gpu["logits"][:, :, 7]).all()
        assert np.isfinite(gpu["values"]).all()
        # a NaN logit weighs nothing in the draw: action 7 is never taken
        assert not (gpu["actions"] == 7).any()
    record(f"nonfinite_{which}_{'bf16' if precision else 'fp32'}", counters=gpu["counters"].tolist())


def test_gae_lookback_give_up_is_reported_not_silent(monkeypatch):
    """Rollouts longer than 512 steps chain 512-step GAE chunks through
    bounded waits.  With the bound set to zero polls from the host (so every
    kernel still ends normally), every chunk but the latest gives up: each
    episode counts one event per such chunk in counters[2], and its
    advantages and returns before the latest chunk are NaN, never silently
    wrong; the latest chunk needs no carry and matches the oracle.  Then the
    standalone scan on the same streams, and the default bound again."""
    import torch
    import rl_experience_collection_amd as rx
    N, L = 300, 1300
    nk, last = -(-L // 512), (L - 1) // 512 * 512
    monkeypatch.setenv("ROLLOUT_GAE_SPIN_LIMIT", "0")
    inp = synthdata.ppo_inputs(dict(N=N, L=L, n_bars=5000, seed=52), bias_scale=0.1)
    gpu = run_gpu(inp, logits=False)
    A, R = oracle.gae(gpu["rewards"], gpu["values"], gpu["dones"], 0.99, 0.95)
    assert int(gpu["counters"][2]) == N * (nk - 1)
    assert np.isnan(gpu["advantages"][:last]).all() and np.isnan(gpu["returns"][:last]).all()
    assert close_mask(gpu["advantages"][last:], A[last:]).all()
    assert close_mask(gpu["returns"][last:], R[last:]).all()
    dev = {k: torch.from_numpy(gpu[k]).cuda() for k in ("rewards", "values", "dones")}
    Ag, Rg = torch.empty_like(dev["rewards"]), torch.empty_like(dev["rewards"])
    rx.gae_scan(dev["rewards"], dev["values"], dev["dones"], None, 0.99, 0.95, Ag, Rg)
    torch.cuda.synchronize()
    Ag = Ag.cpu().numpy()
    assert np.isnan(Ag[:last]).all() and close_mask(Ag[last:], A[last:]).all()
    record("gae_give_up_zero_polls", N=N, L=L, gave_up=int(gpu["counters"][2]),
           nan_rows=int(last))
    monkeypatch.delenv("ROLLOUT_GAE_SPIN_LIMIT")
    gpu2 = run_gpu(inp, logits=False)
    assert int(gpu2["counters"][2]) == 0
    assert close_mask(gpu2["advantages"], A).all() and close_mask(gpu2["returns"], R).all()


@pytest.mark.parametrize("precision,recycle", [(0, 0), (1, 1)])
def test_instrumented_step_kernel_gives_the_same_collection(precision, recycle):
    """rollout_phase_cycles switches in a build of the step kernel that reads
    the clock at every phase boundary: the collection it produces is bit for
    bit the plain kernel's (N=128 is split into several launches with value
    passes beside them), every wave counts all L steps, and the phases add
    up to no more than the loop's cycles."""
    import torch
    import rl_experience_collection_amd as rx
    from parity import to_device
    inp = synthdata.ppo_inputs(dict(N=128, L=500, n_bars=3000, seed=61), bias_scale=0.1)
    d = to_device(inp)
    settings = dict(inp["settings"], recycle=recycle)
    col = rx.Collector(inp["N"], inp["L"], d["weights"], d["features"], d["prices"],
                       settings=settings, precision=precision)
    plain = {k: v.clone() for k, v in col.collect(d["starts"], inp["sampler_seed"]).items()
             if v is not None}
    col.phase_cycles(True)
    stamped = col.collect(d["starts"], inp["sampler_seed"])
    st = col.phase_cycles(False)
    torch.cuda.synchronize()
    for k, v in plain.items():
        assert torch.equal(v, stamped[k]), k
    assert st.shape == (4 * 128 // 16, rx.STAMP_WORDS)
    assert (st[:, 11] == inp["L"]).all()
    assert (st[:, :11].sum(axis=1) <= st[:, 12]).all() and (st[:, 12] > 0).all()
    # switched off again: the plain kernel counts nothing
    col.collect(d["starts"], inp["sampler_seed"])
    assert (col.phase_cycles(False) == 0).all()
    col.close()


@pytest.mark.parametrize("precision,recycle", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_feature_table_gives_the_same_collection(monkeypatch, precision, recycle):
    """Without recycling and with few workgroups, the actor's first-layer
    feature part (bias plus the k-steps that read only market features)
    comes by default from a per-step table computed at each collection;
    with ROLLOUT_FEATURE_TABLE=0 at create the step computes it itself.
    Both use the same MFMA instructions on the same operands, so the
    collections match bit for bit (N=40 leaves a ragged workgroup; N=128 is
    split into launches; recycled collections always compute in the
    step)."""
    import torch
    import rl_experience_collection_amd as rx
    from parity import to_device
    for N, L in ((40, 130), (128, 300)):
        inp = synthdata.ppo_inputs(dict(N=N, L=L, n_bars=2000, seed=71 + N), bias_scale=0.1)
        d = to_device(inp)
        settings = dict(inp["settings"], recycle=recycle)
        outs = []
        for table in (True, False):
            if not table:
                monkeypatch.setenv("ROLLOUT_FEATURE_TABLE", "0")
            col = rx.Collector(N, L, d["weights"], d["features"], d["prices"], settings=settings,
                               precision=precision)
            outs.append(col.collect(d["starts"], inp["sampler_seed"], logits=True))
            torch.cuda.synchronize()
            col.close()
            monkeypatch.delenv("ROLLOUT_FEATURE_TABLE", raising=False)
        for k, v in outs[0].items():
            if v is not None:
                assert torch.equal(v, outs[1][k]), (N, k)
        assert int(outs[0]["dones"].sum()) > 0


# ---------------------------------------------------- sizes and modes mixed
def _mixed_cases(seed, count):
    """Deterministic mixes of the sizes that cut tiles, work items and
    launch parts unevenly, precisions, recycling, the split rollout forced
    on or off or left to the default, and markets from the minimum
    n_bars = L + 1 up."""
    import random
    rng = random.Random(seed)
    for _ in range(count):
        N = rng.choice([1, 2, 15, 16, 17, 31, 33, 64, 100, 127, 129, 200, 257])
        L = rng.choice([1, 2, 3, 15, 16, 17, 63, 64, 65, 100, 130, 199])
        yield (N, L, rng.choice([0, 1]), rng.choice([0, 1]), rng.choice([-1, 0, 1]),
               rng.choice([L + 1, L + 5, 3000]), rng.randrange(1, 10**6))


@pytest.mark.parametrize("N,L,precision,recycle,overlap,n_bars,seed", list(_mixed_cases(7, 24)))
def test_mixed_sizes_and_modes(N, L, precision, recycle, overlap, n_bars, seed):
    """Each case against the oracle by its precision's protocol; a case with
    the rollout split (overlap 1) also equals the single launch bit for bit."""
    inp = synthdata.ppo_inputs(dict(N=N, L=L, n_bars=n_bars, seed=seed), bias_scale=0.1)
    inp["settings"] = dict(inp["settings"], recycle=recycle, overlap=overlap)
    gpu = run_gpu(inp, settings=inp["settings"], precision=precision)
    if overlap == 1:
        one = run_gpu(inp, settings=dict(inp["settings"], overlap=0), precision=precision)
        for k, v in one.items():
            if v is not None:
                assert v.tobytes() == gpu[k].tobytes(), k
    if precision == 0:
        _assert_parity(inp, gpu, oracle.rollout(inp), name=f"mixed_n{N}_l{L}")
    else:
        forced = oracle.rollout(inp, precision=oracle.BF16, forced_actions=gpu["actions"])
        cols = list(range(N))
        fails, stats = compare_bf16(inp, gpu, forced, cols, bf16_floors(inp, forced, cols))
        record(f"mixed_bf16_n{N}_l{L}", N=N, L=L, episodes=N, outputs=stats, failures=fails)
        assert not fails, "\n".join(fails)
