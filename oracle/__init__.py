"""ctypes wrapper of the CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the package smoke check and the CPU-baseline leg of the
benchmark may import this module.  It wraps oracle/liboracle.so (plain C, see
oracle.h for the pages each function follows) and shares nothing with the HIP
library.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

FP32, BF16, FP64 = 0, 1, 2
N_ACTIONS = 45
STATE_DIM = 54
MAX_WINDOW = 256


class Params(C.Structure):
    _fields_ = [
        ("n_episodes", C.c_int32), ("n_steps", C.c_int32), ("precision", C.c_int32),
        ("gamma", C.c_float), ("lam", C.c_float),
        ("profit_take", C.c_float), ("stop_loss", C.c_float),
        ("max_hold", C.c_int32), ("div_window", C.c_int32),
        ("div_threshold", C.c_float), ("div_penalty", C.c_float),
        ("curiosity_coef", C.c_float), ("risk_coef", C.c_float),
        ("spread", C.c_float), ("barrier_scale", C.c_float),
        ("exposure", C.c_float * 5), ("cost", C.c_float * 3),
        ("urgency_mult", C.c_float), ("recycle", C.c_int32),
    ]


class Nets(C.Structure):
    _fields_ = [
        ("aw", C.c_void_p * 3), ("ab", C.c_void_p * 3),
        ("vw", C.c_void_p * 6), ("vb", C.c_void_p * 6),
        ("cw", C.c_void_p * 2), ("cb", C.c_void_p * 2),
    ]


class Outputs(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "states", "logits", "u", "cdf_gap", "actions", "log_probs", "values",
        "rewards", "dones", "barrier", "adv", "ret")]


class QNet(C.Structure):
    _fields_ = [("w", C.c_void_p * 6), ("b", C.c_void_p * 6)]


class DqnNets(C.Structure):
    _fields_ = [("online", QNet), ("target", QNet),
                ("cw", C.c_void_p * 2), ("cb", C.c_void_p * 2)]


class DqnParams(C.Structure):
    _fields_ = [("epsilon", C.c_float), ("alpha", C.c_float)]


class DqnOutputs(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "states", "next_states", "q_values", "actions", "explored", "q_gap", "q_taken",
        "q_next_max", "rewards", "dones", "barrier", "td", "priority")]


class Episode(C.Structure):
    _fields_ = [
        ("V", C.c_float), ("e_prev", C.c_float),
        ("armed", C.c_int32), ("side", C.c_int32), ("t_open", C.c_int32),
        ("entry", C.c_float), ("cnt", C.c_int32 * 3), ("pushed", C.c_int32),
        ("ring", C.c_uint8 * MAX_WINDOW),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(LIB_PATH)
        vp, f32, i32 = C.c_void_p, C.c_float, C.c_int32
        L.orc_philox4x32_10.argtypes = [vp, vp, vp]
        L.orc_uniform.argtypes = [C.c_uint64, C.c_uint32, C.c_uint32, C.c_uint32]
        L.orc_uniform.restype = f32
        L.orc_uniform_many.argtypes = [C.c_uint64, vp, vp, C.c_uint32, C.c_int64, vp]
        L.orc_bf16_round.argtypes = [f32]
        L.orc_bf16_round.restype = f32
        L.orc_linear.argtypes = [vp, vp, vp, C.c_int, C.c_int, C.c_int, C.c_int, vp]
        L.orc_softmax_sample.argtypes = [vp, C.c_int, f32, vp, vp, vp]
        L.orc_softmax_sample.restype = C.c_int
        L.orc_sample_many.argtypes = [vp, C.c_int, vp, C.c_int64, vp]
        L.orc_log_softmax_at.argtypes = [vp, C.c_int, C.c_int]
        L.orc_log_softmax_at.restype = f32
        L.orc_entropy3.argtypes = [C.c_int, C.c_int, C.c_int]
        L.orc_entropy3.restype = f32
        for fn in ("orc_action_exp_index", "orc_action_ord_index", "orc_action_urg_index",
                   "orc_action_category"):
            getattr(L, fn).argtypes = [C.c_int]
            getattr(L, fn).restype = C.c_int
        L.orc_action_exposure.argtypes = [C.POINTER(Params), C.c_int]
        L.orc_action_exposure.restype = f32
        L.orc_action_cost.argtypes = [C.POINTER(Params), C.c_int]
        L.orc_action_cost.restype = f32
        L.orc_episode_reset.argtypes = [C.POINTER(Episode)]
        L.orc_env_step.argtypes = [C.POINTER(Params), C.POINTER(Episode), C.c_int, C.c_int,
                                   f32, f32, vp, vp, vp, vp, vp]
        L.orc_env_step.restype = C.c_int
        L.orc_gae.argtypes = [vp, vp, vp, vp, i32, i32, f32, f32, C.c_int, vp, vp]
        L.orc_rollout.argtypes = [C.POINTER(Params), C.POINTER(Nets), vp, vp, C.c_int64, vp,
                                  C.c_uint64, vp, vp, i32, C.POINTER(Outputs), i32]
        L.orc_rollout.restype = C.c_int
        L.orc_dueling_q.argtypes = [C.POINTER(QNet), vp, C.c_int, vp]
        L.orc_argmax_first.argtypes = [vp, C.c_int]
        L.orc_argmax_first.restype = C.c_int
        L.orc_random_action.argtypes = [f32]
        L.orc_random_action.restype = C.c_int
        L.orc_dqn_rollout.argtypes = [C.POINTER(Params), C.POINTER(DqnParams), C.POINTER(DqnNets),
                                      vp, vp, C.c_int64, vp, C.c_uint64, vp, vp, i32,
                                      C.POINTER(DqnOutputs), i32]
        L.orc_dqn_rollout.restype = C.c_int
        L.orc_recycle_bar.argtypes = [C.c_uint64, C.c_uint32, i32, i32, C.c_int64]
        L.orc_recycle_bar.restype = C.c_int64
        L.orc_per_uniform.argtypes = [C.c_uint64, C.c_uint32]
        L.orc_per_uniform.restype = C.c_double
        L.orc_per_sample.argtypes = [vp, C.c_int64, i32, C.c_uint64, f32, vp, vp, vp]
        L.orc_per_sample.restype = C.c_int
        L.orc_per_update.argtypes = [vp, C.c_int64, vp, vp, i32, f32, f32, f32]
        L.orc_per_update.restype = C.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def make_params(settings: dict, N: int = 1, L: int = 1, precision: int = FP32) -> Params:
    p = Params()
    p.n_episodes, p.n_steps, p.precision = N, L, precision
    p.gamma, p.lam = settings["gamma"], settings["lam"]
    p.profit_take, p.stop_loss = settings["profit_take"], settings["stop_loss"]
    p.max_hold, p.div_window = settings["max_hold"], settings["div_window"]
    p.div_threshold, p.div_penalty = settings["div_threshold"], settings["div_penalty"]
    p.curiosity_coef, p.risk_coef = settings["curiosity_coef"], settings["risk_coef"]
    p.spread, p.barrier_scale = settings["spread"], settings["barrier_scale"]
    p.exposure = (C.c_float * 5)(*settings["exposure"])
    p.cost = (C.c_float * 3)(*settings["cost"])
    p.urgency_mult = settings["urgency_mult"]
    p.recycle = int(settings.get("recycle", 0))
    return p


# --------------------------------------------------------------------------- RNG
def philox(ctr, key) -> np.ndarray:
    c = np.asarray(ctr, np.uint32).copy()
    k = np.asarray(key, np.uint32).copy()
    o = np.zeros(4, np.uint32)
    lib().orc_philox4x32_10(_p(c), _p(k), _p(o))
    return o


def uniform(seed: int, episode, step, stream: int = 0) -> np.ndarray:
    e = np.ascontiguousarray(episode, np.uint32).ravel()
    t = np.ascontiguousarray(step, np.uint32).ravel()
    assert e.shape == t.shape
    u = np.zeros(e.shape, np.float32)
    lib().orc_uniform_many(C.c_uint64(seed), _p(e), _p(t), stream, e.size, _p(u))
    return u


# ---------------------------------------------------------------- building blocks
def bf16_round(x: float) -> float:
    return lib().orc_bf16_round(float(x))


def linear(W, b, x, relu: bool, precision: int = FP32) -> np.ndarray:
    W, b, x = _f32(W), _f32(b), _f32(x)
    out_dim, in_dim = W.shape
    y = np.zeros(out_dim, np.float32)
    lib().orc_linear(_p(W), _p(b), _p(x), in_dim, out_dim, int(relu), precision, _p(y))
    return y


def softmax_sample(logits, u: float):
    """(action, logp, cdf[45], gap)."""
    lg = _f32(logits)
    lp = np.zeros(1, np.float32)
    cdf = np.zeros(lg.size, np.float32)
    gap = np.zeros(1, np.float32)
    a = lib().orc_softmax_sample(_p(lg), lg.size, float(u), _p(lp), _p(cdf), _p(gap))
    return a, float(lp[0]), cdf, float(gap[0])


def sample_many(logits, u) -> np.ndarray:
    lg = _f32(logits)
    uu = _f32(u).ravel()
    a = np.zeros(uu.size, np.int32)
    lib().orc_sample_many(_p(lg), lg.size, _p(uu), uu.size, _p(a))
    return a


def log_softmax_at(logits, a: int) -> float:
    lg = _f32(logits)
    return lib().orc_log_softmax_at(_p(lg), lg.size, int(a))


def entropy3(n0: int, n1: int, n2: int) -> float:
    return lib().orc_entropy3(n0, n1, n2)


def action_maps(settings: dict):
    """Per-action (exp index, ord index, urg index, category, exposure, cost)."""
    p = make_params(settings)
    L = lib()
    rows = []
    for a in range(N_ACTIONS):
        rows.append((L.orc_action_exp_index(a), L.orc_action_ord_index(a),
                     L.orc_action_urg_index(a), L.orc_action_category(a),
                     L.orc_action_exposure(C.byref(p), a), L.orc_action_cost(C.byref(p), a)))
    return rows


class Env:
    """One episode's environment state, stepped by the oracle's env step."""

    def __init__(self, settings: dict):
        self.p = make_params(settings)
        self.s = Episode()
        lib().orc_episode_reset(C.byref(self.s))

    def reset(self):
        lib().orc_episode_reset(C.byref(self.s))

    def step(self, a: int, t: int, p0: float, p1: float) -> dict:
        pnl = np.zeros(1, np.float32); div = np.zeros(1, np.float32)
        e = np.zeros(1, np.float32)
        hit = np.zeros(1, np.int32); code = np.zeros(1, np.int32)
        done = lib().orc_env_step(C.byref(self.p), C.byref(self.s), a, t, float(p0), float(p1),
                                  _p(pnl), _p(hit), _p(code), _p(div), _p(e))
        return dict(pnl=float(pnl[0]), hit=int(hit[0]), code=int(code[0]), div=float(div[0]),
                    exposure=float(e[0]), done=bool(done), V=self.s.V)


# -------------------------------------------------------------------------- GAE
def gae(rewards, values, dones, gamma: float, lam: float, last_values=None,
        precision: int = FP32):
    r, v = _f32(rewards), _f32(values)
    d = np.ascontiguousarray(dones, np.uint8)
    L_, N_ = r.shape
    lv = None if last_values is None else _f32(last_values)
    adv = np.zeros_like(r)
    ret = np.zeros_like(r)
    lib().orc_gae(_p(r), _p(v), _p(d), _p(lv), L_, N_, gamma, lam, precision, _p(adv), _p(ret))
    return adv, ret


# ---------------------------------------------------------------------- rollout
def rollout(inputs: dict, precision: int = FP32, forced_actions=None, subset=None,
            n_threads: int = 0, with_logits: bool = True, settings: dict | None = None) -> dict:
    """Run the oracle on host arrays from synthdata.ppo_inputs(); returns [L][N] arrays."""
    N, L = inputs["N"], inputs["L"]
    st = settings or inputs["settings"]
    p = make_params(st, N, L, precision)
    w = inputs["weights"]
    keep = [_f32(x) for x in w["actor"] + w["critic"] + w["curiosity"]]
    nets = Nets()
    for i in range(3):
        nets.aw[i], nets.ab[i] = keep[2 * i].ctypes.data, keep[2 * i + 1].ctypes.data
    for i in range(6):
        nets.vw[i], nets.vb[i] = keep[6 + 2 * i].ctypes.data, keep[6 + 2 * i + 1].ctypes.data
    for i in range(2):
        nets.cw[i], nets.cb[i] = keep[18 + 2 * i].ctypes.data, keep[18 + 2 * i + 1].ctypes.data
    feats, prices = _f32(inputs["features"]), _f32(inputs["prices"])
    starts = np.ascontiguousarray(inputs["starts"], np.int32)
    out = dict(
        states=np.zeros((L, N, STATE_DIM), np.float32),
        logits=np.zeros((L, N, N_ACTIONS), np.float32) if with_logits else None,
        u=np.zeros((L, N), np.float32),
        cdf_gap=np.zeros((L, N), np.float32),
        actions=np.zeros((L, N), np.int32),
        log_probs=np.zeros((L, N), np.float32),
        values=np.zeros((L, N), np.float32),
        rewards=np.zeros((L, N), np.float32),
        dones=np.zeros((L, N), np.uint8),
        barrier=np.zeros((L, N), np.uint8),
        adv=np.zeros((L, N), np.float32),
        ret=np.zeros((L, N), np.float32),
    )
    o = Outputs()
    for k, arr in out.items():
        setattr(o, k, None if arr is None else arr.ctypes.data)
    fa = None if forced_actions is None else np.ascontiguousarray(forced_actions, np.int32)
    sub = None if subset is None else np.ascontiguousarray(subset, np.int32)
    rc = lib().orc_rollout(C.byref(p), C.byref(nets), _p(feats), _p(prices), feats.shape[0],
                           _p(starts), C.c_uint64(inputs["sampler_seed"]), _p(fa), _p(sub),
                           0 if sub is None else sub.size, C.byref(o), n_threads)
    if rc != 0:
        raise ValueError("oracle rollout rejected its arguments")
    return out


# -------------------------------------------------------------------------- DQN
def _qnet(arrays, keep):
    """QNet struct over 12 [out, in] arrays (trunk 1, trunk 2, value 1, value 2,
    advantage 1, advantage 2; weight then bias)."""
    net = QNet()
    for i in range(6):
        w, b = _f32(arrays[2 * i]), _f32(arrays[2 * i + 1])
        keep += [w, b]
        net.w[i], net.b[i] = w.ctypes.data, b.ctypes.data
    return net


def dueling_q(arrays, s, precision: int = FP32) -> np.ndarray:
    keep = []
    net = _qnet(arrays, keep)
    x = _f32(s)
    q = np.zeros(N_ACTIONS, np.float32)
    lib().orc_dueling_q(C.byref(net), _p(x), precision, _p(q))
    return q


def argmax_first(x) -> int:
    x = _f32(x)
    return lib().orc_argmax_first(_p(x), x.size)


def random_action(u: float) -> int:
    return lib().orc_random_action(float(u))


def dqn_rollout(inputs: dict, precision: int = FP32, forced_actions=None, subset=None,
                n_threads: int = 0, with_q: bool = True, with_next: bool = True) -> dict:
    """Run the DQN oracle on host arrays from synthdata.dqn_inputs(); [L][N] arrays."""
    N, L = inputs["N"], inputs["L"]
    p = make_params(inputs["settings"], N, L, precision)
    p.gamma = inputs["dqn"]["gamma"]
    dq = DqnParams()
    dq.epsilon, dq.alpha = inputs["dqn"]["epsilon"], inputs["dqn"]["alpha"]
    w = inputs["weights"]
    keep = []
    nets = DqnNets()
    nets.online = _qnet(w["online"], keep)
    nets.target = _qnet(w["target"], keep)
    for i in range(2):
        cw, cb = _f32(w["curiosity"][2 * i]), _f32(w["curiosity"][2 * i + 1])
        keep += [cw, cb]
        nets.cw[i], nets.cb[i] = cw.ctypes.data, cb.ctypes.data
    feats, prices = _f32(inputs["features"]), _f32(inputs["prices"])
    starts = np.ascontiguousarray(inputs["starts"], np.int32)
    out = dict(
        states=np.zeros((L, N, STATE_DIM), np.float32),
        next_states=np.zeros((L, N, STATE_DIM), np.float32) if with_next else None,
        q_values=np.zeros((L, N, N_ACTIONS), np.float32) if with_q else None,
        actions=np.zeros((L, N), np.int32),
        explored=np.zeros((L, N), np.uint8),
        q_gap=np.zeros((L, N), np.float32),
        q_taken=np.zeros((L, N), np.float32),
        q_next_max=np.zeros((L, N), np.float32),
        rewards=np.zeros((L, N), np.float32),
        dones=np.zeros((L, N), np.uint8),
        barrier=np.zeros((L, N), np.uint8),
        td=np.zeros((L, N), np.float32),
        priority=np.zeros((L, N), np.float32),
    )
    o = DqnOutputs()
    for k, arr in out.items():
        setattr(o, k, None if arr is None else arr.ctypes.data)
    fa = None if forced_actions is None else np.ascontiguousarray(forced_actions, np.int32)
    sub = None if subset is None else np.ascontiguousarray(subset, np.int32)
    rc = lib().orc_dqn_rollout(C.byref(p), C.byref(dq), C.byref(nets), _p(feats), _p(prices),
                               feats.shape[0], _p(starts), C.c_uint64(inputs["sampler_seed"]),
                               _p(fa), _p(sub), 0 if sub is None else sub.size, C.byref(o),
                               n_threads)
    if rc != 0:
        raise ValueError("oracle DQN rollout rejected its arguments")
    return out


def recycle_bar(seed: int, episode: int, t: int, n_steps: int, n_bars: int) -> int:
    return lib().orc_recycle_bar(C.c_uint64(seed), episode, t, n_steps, n_bars)


# ---------------------------------------------------------------- prioritized replay
def per_uniform(seed: int, draw: int) -> float:
    return lib().orc_per_uniform(C.c_uint64(seed), draw)


def per_sample(priorities, batch: int, seed: int, beta: float):
    """(indices [B] i32, weights [B] f32, gap [B] f64) by proportional sampling."""
    p = _f32(priorities).ravel()
    idx = np.zeros(batch, np.int32)
    w = np.zeros(batch, np.float32)
    gap = np.zeros(batch, np.float64)
    rc = lib().orc_per_sample(_p(p), p.size, batch, C.c_uint64(seed), float(beta), _p(idx), _p(w),
                              _p(gap))
    if rc != 0:
        raise ValueError("oracle PER sample rejected its arguments")
    return idx, w, gap


def per_update(priorities, indices, td, alpha: float, epsilon: float, max_priority: float):
    """A new priority array after the batch's update (the input is not modified)."""
    p = _f32(priorities).ravel().copy()
    idx = np.ascontiguousarray(indices, np.int32)
    t = _f32(td)
    rc = lib().orc_per_update(_p(p), p.size, _p(idx), _p(t), idx.size, float(alpha),
                              float(epsilon), float(max_priority))
    if rc != 0:
        raise ValueError("oracle PER update rejected its arguments")
    return p
