"""Benchmark of fused PPO experience collection on one MI355X.

One step = one rollout_collect: actor rollout over L steps, batched critic +
curiosity + reward over the L*N stored states, GAE scan.  The headline
workload is the chip-filling PPO collection (N=8192 episodes x L=500 steps,
fp32); the pages' default N=128 x L=500 collection and the standalone GAE
scan (N=4096 x L=2048) are measured in the same run and reported beside it.

Prints ONE JSON line.  Every input is synthetic and seeded (synthdata), and
resident in HBM before the timed region starts.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_MFMA = 157.3e12   # MI355X dense fp32 matrix, FLOP/s
PEAK_BF16_MFMA = 2.5e15     # MI355X dense bf16 matrix, FLOP/s
PEAK_HBM = 8.0e12           # MI355X HBM3E, B/s
METRIC = "experiences/sec at N=128,L=500 and N=8192; MFMA util %; GAE scan HBM GB/s"

# algorithmic work per unit (2 flops per multiply-add; biases not counted)
ACTOR_FLOP = 2 * (54 * 128 + 128 * 64 + 64 * 45)                                  # 35,968
CRITIC_FLOP = 2 * (54 * 512 + 512 * 384 + 384 * 256 + 256 * 128 + 128 * 64 + 64)  # 727,168
CURIOSITY_FLOP = 2 * (54 * 128 + 128 * 51) + 128                                  # 27,008
VALUE_KERNEL_FLOP = CRITIC_FLOP + CURIOSITY_FLOP                                  # 754,176
MLP_FLOP = ACTOR_FLOP + VALUE_KERNEL_FLOP                                         # 790,144
# DQN collection: online and target dueling nets (trunk 54-256-128, value
# head 128-64-1, advantage head 128-64-45) and the curiosity model
Q_NET_FLOP = 2 * (54 * 256 + 256 * 128 + 128 * 64 + 64 * 1 + 128 * 64 + 64 * 45)   # 131,840
DQN_FLOP = 2 * Q_NET_FLOP + CURIOSITY_FLOP                                          # 290,688
GAE_BYTES = 17   # read r 4, V 4, d 1; write A 4, R 4


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(name, files):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != source_hash(files):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


_SLEEP_PER_MS = None


def gpu_lead(ms):
    """Occupy the device for about `ms` with a spin kernel that touches no
    memory, so that the host enqueues the timed launches ahead of it: events
    between short launches then time device work, not Python call overhead."""
    global _SLEEP_PER_MS
    import torch
    import rl_experience_collection_amd as rx
    if _SLEEP_PER_MS is None:  # spin cycles per millisecond on this device
        ev = rx.HipEvents(2)
        n = 1 << 20
        torch.cuda._sleep(n)  # first launch outside the measurement
        ev.record(0)
        torch.cuda._sleep(n)
        ev.record(1)
        torch.cuda.synchronize()
        _SLEEP_PER_MS = n / max(ev.elapsed_ms(0, 1), 1e-3)
        ev.close()
    torch.cuda._sleep(int(ms * _SLEEP_PER_MS))


def time_collect(inp, steps, warmup, precision=0):
    import torch
    import numpy as np
    import rl_experience_collection_amd as rx

    N, L = inp["N"], inp["L"]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    w = inp["weights"]
    weights = dict(actor=[dev(x) for x in w["actor"]], critic=[dev(x) for x in w["critic"]],
                   curiosity=[dev(x) for x in w["curiosity"]])
    feats, prices, starts = dev(inp["features"]), dev(inp["prices"]), dev(inp["starts"])
    col = rx.Collector(N, L, weights, feats, prices, settings=inp["settings"], precision=precision)
    outs = rx.alloc_outputs(N, L, "cuda")
    ev = rx.HipEvents(4 * steps)
    seed = inp["sampler_seed"]
    for i in range(warmup):
        col.collect(starts, seed + i, outputs=outs)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        col.collect(starts, seed + warmup + i, outputs=outs, phase_events=ev.handles[4 * i:4 * i + 4])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ph = np.array([[ev.elapsed_ms(4 * i + j, 4 * i + j + 1) for j in range(3)] for i in range(steps)])
    per_step = np.array([ev.elapsed_ms(4 * i, 4 * i + 3) for i in range(steps)])
    bad = int(outs["counters"][0].item())
    ev.close()
    col.close()
    return dict(N=N, L=L, wall_s=wall, step_ms_events=per_step, phases_ms=ph.mean(axis=0),
                nonfinite=bad)


def time_gemm_reference(dtype_name, n=8192, reps=10):
    """A square n x n x n matrix product in torch (the vendor GEMM library)
    on random operands, timed with events around `reps` products: what the
    matrix cores sustain on this device, at the clock they then run at, for
    a large dense product with no data movement of its own (bf16: the faster
    of 8192 and 16384 is reported)."""
    import torch
    dt = dict(bf16=torch.bfloat16, fp32=torch.float32)[dtype_name]
    g = torch.Generator(device="cuda").manual_seed(7)
    a = torch.randn(n, n, device="cuda", dtype=dt, generator=g)
    b = torch.randn(n, n, device="cuda", dtype=dt, generator=g)
    for _ in range(3):
        c = a @ b
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        c = a @ b
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del a, b, c
    return dict(op=f"torch.matmul {dtype_name} {n}x{n}x{n}, random operands", ms=ms,
                TFLOPs=2.0 * n ** 3 / (ms * 1e-3) / 1e12)


def zero_value_weights(inp):
    """The same inputs with the critic and curiosity weights zeroed: the value
    kernel then does identical work on zero operands."""
    w = dict(inp["weights"])
    w["critic"] = [x * 0 for x in w["critic"]]
    w["curiosity"] = [x * 0 for x in w["curiosity"]]
    return dict(inp, weights=w)


def smi_sample():
    """Socket power (W) and the shader clocks (MHz) of every XCD from
    amd-smi, or None where the tool is missing or fails."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True,
                           text=True, timeout=10)
        if r.returncode:
            return None
        d = json.loads(r.stdout)
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clocks = [v["clk"]["value"] for k, v in g["clock"].items()
                  if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
        return dict(power_W=g["power"]["socket_power"]["value"], gfx_MHz=clocks)
    except Exception:
        return None


def value_power(inp, seconds=3.0):
    """The N=8192 L=500 collection back to back for about `seconds` each in
    bf16, in bf16 with the critic and curiosity weights zeroed (the same
    instructions on zero operands) and in fp32, with the board's socket
    power and shader clocks read from amd-smi while the device is busy, and
    the value kernel's time from phase events."""
    import numpy as np
    import torch
    import rl_experience_collection_amd as rx

    N, L = inp["N"], inp["L"]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    res = []
    for name, prec, src in (("bf16", 1, inp), ("bf16, zeroed critic and curiosity weights", 1,
                                                zero_value_weights(inp)), ("fp32", 0, inp)):
        w = src["weights"]
        weights = dict(actor=[dev(x) for x in w["actor"]], critic=[dev(x) for x in w["critic"]],
                       curiosity=[dev(x) for x in w["curiosity"]])
        col = rx.Collector(N, L, weights, dev(src["features"]), dev(src["prices"]),
                           settings=src["settings"], precision=prec)
        starts, outs = dev(src["starts"]), rx.alloc_outputs(N, L, "cuda")
        ev = rx.HipEvents(4)
        col.collect(starts, 1, outputs=outs, phase_events=ev.handles)
        torch.cuda.synchronize()
        per = ev.elapsed_ms(0, 3)
        reps = max(3, int(seconds * 1e3 / per))
        samples, stop = [], threading.Event()

        def sampler():
            while not stop.is_set():
                x = smi_sample()
                if x:
                    samples.append(x)
                stop.wait(0.25)
        th = threading.Thread(target=sampler)
        th.start()
        for i in range(reps):
            col.collect(starts, 2 + i, outputs=outs,
                        phase_events=ev.handles if i == reps // 2 else None)
        torch.cuda.synchronize()
        stop.set()
        th.join()
        value_ms = ev.elapsed_ms(1, 2)
        ev.close()
        col.close()
        busy = samples[1:-1]  # (the first and last may fall outside the busy span)
        p = [x["power_W"] for x in busy]
        c = [float(np.mean(x["gfx_MHz"])) for x in busy]
        res.append(dict(run=name, collections=reps, value_kernel_ms=value_ms,
                        samples=len(p), power_W_median=float(np.median(p)) if p else None,
                        power_W_max=float(max(p)) if p else None,
                        gfx_MHz_median=float(np.median(c)) if c else None))
    return res


def actor_phase_stamps(inp, reps, precision=0):
    """Per-phase shader-clock cycles of one sequential step (the instrumented
    step kernel, rollout_phase_cycles), averaged over every wave and step of
    `reps` collections, beside the plain kernel's step time from the same
    handle (phase events of as many plain collections)."""
    import torch
    import numpy as np
    import rl_experience_collection_amd as rx

    N, L = inp["N"], inp["L"]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    w = inp["weights"]
    weights = dict(actor=[dev(x) for x in w["actor"]], critic=[dev(x) for x in w["critic"]],
                   curiosity=[dev(x) for x in w["curiosity"]])
    feats, prices, starts = dev(inp["features"]), dev(inp["prices"]), dev(inp["starts"])
    col = rx.Collector(N, L, weights, feats, prices, settings=inp["settings"], precision=precision)
    outs = rx.alloc_outputs(N, L, "cuda")
    seed = inp["sampler_seed"]
    ev = rx.HipEvents(4 * reps)

    def run(tag):
        for i in range(reps):
            col.collect(starts, seed + i, outputs=outs, phase_events=ev.handles[4 * i:4 * i + 4])
        torch.cuda.synchronize()
        return float(np.mean([ev.elapsed_ms(4 * i, 4 * i + 1) for i in range(reps)]))

    col.collect(starts, seed, outputs=outs)
    plain_ms = run("plain")
    col.phase_cycles(True)
    col.collect(starts, seed, outputs=outs)  # warm the instrumented kernel
    col.phase_cycles(True)                   # drop its counts
    stamped_ms = run("stamped")
    st = col.phase_cycles(False).astype(np.float64)
    ev.close()
    col.close()
    real = st[:, 11] > 0  # waves that counted steps
    steps = st[real, 11]
    per = st[real, :11].sum(axis=0) / steps.sum()
    loop = st[real, 12].sum() / steps.sum()
    names = [f"{k:02d} {n}" for k, n in enumerate(rx.STAMP_PHASES)]
    return dict(N=N, L=L, precision="bf16" if precision else "fp32", collections=reps,
                waves=int(real.sum()), cycles_per_step=dict(zip(names, [round(x, 1) for x in per])),
                phase_sum_cycles_per_step=round(float(per.sum()), 1),
                loop_cycles_per_step=round(float(loop), 1),
                # the stamped kernel's rollout phase (events) against its own loop cycles
                clock_GHz=round(float(loop * L / (stamped_ms * 1e-3) / 1e9), 3),
                plain_rollout_ms=round(plain_ms, 4), stamped_rollout_ms=round(stamped_ms, 4),
                plain_us_per_step=round(plain_ms * 1e3 / L, 3),
                stamped_us_per_step=round(stamped_ms * 1e3 / L, 3))


def time_dqn(inp, steps, warmup):
    """DQN collections at the input's size; events around each launch."""
    import torch
    import numpy as np
    import rl_experience_collection_amd as rx

    N, L = inp["N"], inp["L"]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    w = inp["weights"]
    weights = {k: [dev(x) for x in w[k]] for k in ("online", "target", "curiosity")}
    feats, prices, starts = dev(inp["features"]), dev(inp["prices"]), dev(inp["starts"])
    col = rx.DqnCollector(N, L, weights, feats, prices, settings=inp["settings"], dqn=inp["dqn"])
    outs = rx.alloc_dqn_outputs(N, L, "cuda")
    ev = rx.HipEvents(2 * steps)
    seed = inp["sampler_seed"]
    for i in range(warmup):
        col.collect(starts, seed + i, outputs=outs)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        col.collect(starts, seed + warmup + i, outputs=outs, phase_events=ev.handles[2 * i:2 * i + 2])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(steps)])
    bad = int(outs["counters"][0].item())
    ev.close()
    col.close()
    return dict(N=N, L=L, wall_s=wall, kernel_ms=float(per.mean()), nonfinite=bad)


def time_per(n, batch, reps):
    """Prioritized replay on n priorities: per_sample (batch draws), the
    gather of the drawn rows of a replay of n transitions, per_update.
    Priorities ~ Exp(1) with 2% zeros (synthetic)."""
    import numpy as np
    import torch
    import rl_experience_collection_amd as rx
    g = np.random.default_rng(9)
    p = g.exponential(1.0, n).astype(np.float32)
    p[g.integers(0, n, n // 50)] = 0.0
    pd = torch.from_numpy(p).cuda()
    states = torch.randn((n, 54), device="cuda")
    acts = torch.zeros(n, dtype=torch.int32, device="cuda")
    rew = torch.randn(n, device="cuda")
    dn = torch.zeros(n, dtype=torch.uint8, device="cuda")
    td = torch.randn(batch, device="cuda")
    s = rx.PerSampler(n, batch)
    idx = torch.empty(batch, dtype=torch.int32, device="cuda")
    w = torch.empty(batch, dtype=torch.float32, device="cuda")
    out = dict(states=torch.empty((batch, 54), device="cuda"),
               next_states=torch.empty((batch, 54), device="cuda"),
               actions=torch.empty(batch, dtype=torch.int32, device="cuda"),
               rewards=torch.empty(batch, device="cuda"),
               dones=torch.empty(batch, dtype=torch.uint8, device="cuda"))
    def step(r, e0=None, ev=None):
        if ev: ev.record(e0)
        rx.per_sample(s.handle, pd, batch, 1000 + r, 0.4, idx, w)
        if ev: ev.record(e0 + 1)
        rx.per_gather(idx, n, states, states, acts, rew, dn, out=out)
        if ev: ev.record(e0 + 2)
        rx.per_update(pd, idx, td, 0.6, 1e-3, 100.0)
        if ev: ev.record(e0 + 3)
    for r in range(2):
        step(r)
    torch.cuda.synchronize()
    # all timed steps enqueued behind a device-side lead: the events time the
    # device, with the host ahead of it as in a training loop
    ev = rx.HipEvents(4 * reps)
    gpu_lead(2.0 + 0.2 * reps)
    for r in range(reps):
        step(2 + r, 4 * r, ev)
    torch.cuda.synchronize()
    t = np.zeros(3)
    for r in range(reps):
        t += [ev.elapsed_ms(4 * r, 4 * r + 1), ev.elapsed_ms(4 * r + 1, 4 * r + 2),
              ev.elapsed_ms(4 * r + 2, 4 * r + 3)]
    ev.close()
    s.close()
    t = t / reps
    return dict(n=n, batch=batch, sample_ms=float(t[0]), gather_ms=float(t[1]),
                update_ms=float(t[2]))


def probe_lib():
    """Measurement kernels (weight-stream and GAE-traffic ceilings), built
    beside the collection library."""
    import ctypes as C
    import torch  # noqa: F401  (the HIP runtime must be loaded through torch first)
    lib = C.CDLL(os.path.join(ROOT, "rl_experience_collection_amd", "libbenchprobes.so"))
    P = C.c_void_p
    lib.bench_value_stream_shape.argtypes = [C.c_int, C.POINTER(C.c_longlong), C.POINTER(C.c_int)]
    lib.bench_weight_stream.argtypes = [P, C.c_longlong, C.c_longlong, P, P]
    lib.bench_gae_traffic.argtypes = [P, P, P, P, P, C.c_longlong, P]
    lib.bench_lds_activation.argtypes = [C.c_longlong, P, C.POINTER(C.c_longlong), P]
    return lib


def time_gae(spec, reps, traffic_only=False):
    """Cold: a 512 MiB read sweep evicts the 256 MB infinity cache with clean
    lines before each timed launch.  Warm: back-to-back launches.  With
    traffic_only, the element-wise kernel that moves the same bytes is timed
    instead of the scan (the copy ceiling at this size)."""
    import numpy as np
    import torch
    import synthdata
    import rl_experience_collection_amd as rx

    r, v, d = synthdata.gae_inputs(spec["N"], spec["L"], spec["seed"])
    R, V, D = (torch.from_numpy(x).cuda() for x in (r, v, d))
    A, Rt = torch.empty_like(R), torch.empty_like(R)
    flush = torch.ones(512 * 2**20 // 4, dtype=torch.float32, device="cuda")
    if traffic_only:
        lib, st = probe_lib(), torch.cuda.current_stream().cuda_stream

        def launch():
            rc = lib.bench_gae_traffic(R.data_ptr(), V.data_ptr(), D.data_ptr(), A.data_ptr(),
                                       Rt.data_ptr(), R.numel(), st)
            if rc:
                raise RuntimeError(f"bench_gae_traffic: {rc}")
    else:
        def launch():
            rx.gae_scan(R, V, D, None, 0.99, 0.95, A, Rt)
    ev = rx.HipEvents(2)
    cold = []
    for i in range(reps + 2):
        flush.sum()
        ev.record(0)
        launch()
        ev.record(1)
        torch.cuda.synchronize()
        if i >= 2:
            cold.append(ev.elapsed_ms(0, 1))
    launch()
    gpu_lead(1.0 + 0.1 * reps)  # the host enqueues the warm launches ahead
    ev.record(0)
    for i in range(reps):
        launch()
    ev.record(1)
    torch.cuda.synchronize()
    warm = ev.elapsed_ms(0, 1) / reps
    ev.close()
    n = spec["N"] * spec["L"]
    return dict(elements=n, cold_ms=float(np.median(cold)), warm_ms=float(warm))


def time_vendor_copy(nbytes, reps=12):
    """torch's device copy of nbytes / 2 bytes (so nbytes cross HBM: half read,
    half written), cold as in time_gae: what the vendor's own streaming
    kernel reaches for a transfer of that size."""
    import numpy as np
    import torch
    import rl_experience_collection_amd as rx
    a = torch.ones(max(nbytes // 8, 1), device="cuda")
    b = torch.empty_like(a)
    flush = torch.ones(512 * 2**20 // 4, dtype=torch.float32, device="cuda")
    ev = rx.HipEvents(2)
    out = []
    for i in range(reps + 2):
        flush.sum()
        ev.record(0)
        b.copy_(a)
        ev.record(1)
        torch.cuda.synchronize()
        if i >= 2:
            out.append(ev.elapsed_ms(0, 1))
    ev.close()
    ms = float(np.median(out))
    moved = 2 * 4 * a.numel()
    return dict(bytes=moved, cold_ms=ms, TBps=moved / (ms * 1e-3) / 1e12)


def time_weight_stream(rows, bf16, reps):
    """The value kernel's weight stream alone (no arithmetic) for `rows`
    stored states: the L2-to-register bound of that kernel."""
    import ctypes as C
    import torch
    import rl_experience_collection_amd as rx
    lib = probe_lib()
    nbytes, per = C.c_longlong(), C.c_int()
    if lib.bench_value_stream_shape(int(bf16), C.byref(nbytes), C.byref(per)):
        raise RuntimeError("bench_value_stream_shape failed")
    groups = -(-rows // per.value)
    blob = torch.randn(nbytes.value // 4, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream

    def launch():
        rc = lib.bench_weight_stream(blob.data_ptr(), nbytes.value, groups, sink.data_ptr(), st)
        if rc:
            raise RuntimeError(f"bench_weight_stream: {rc}")
    for _ in range(2):
        launch()
    ev = rx.HipEvents(2)
    ev.record(0)
    for _ in range(reps):
        launch()
    ev.record(1)
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(0, 1) / reps
    ev.close()
    total = nbytes.value * groups
    return dict(ms=ms, block_bytes=nbytes.value, rows_per_item=per.value, items=groups,
                bytes_per_launch=total, TBps=total / (ms * 1e-3) / 1e12)


def _host_cpu():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def device_info():
    """The GPU the figures come from: name, architecture, compute units (from
    torch) and the engine clock limit rocminfo reports (None if unavailable):
    the published peaks assume 256 CUs at 2.4 GHz."""
    import subprocess
    import torch
    p = torch.cuda.get_device_properties(0)
    info = dict(name=p.name, arch=getattr(p, "gcnArchName", None), cus=p.multi_processor_count,
                max_clock_MHz=None)
    try:
        r = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30)
        gpu = False
        for line in r.stdout.splitlines():
            t = line.strip()
            if t.startswith("Device Type:"):
                gpu = t.endswith("GPU")
            elif gpu and t.startswith("Max Clock Freq. (MHz):"):
                info["max_clock_MHz"] = int(t.split(":", 1)[1].split()[0])
                break
    except Exception:
        pass
    return info


def _threads():
    return int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1)


def time_lds_activation(rows, reps):
    """The bf16 value kernel's LDS activation traffic alone (reads of every
    layer's B operands, the ReLU/pack stores, the barriers) for `rows`
    stored states: the LDS bound of that kernel."""
    import ctypes as C
    import torch
    import rl_experience_collection_amd as rx
    lib = probe_lib()
    groups = -(-rows // 128)
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    per = C.c_longlong()
    st = torch.cuda.current_stream().cuda_stream

    def launch():
        rc = lib.bench_lds_activation(groups, sink.data_ptr(), C.byref(per), st)
        if rc:
            raise RuntimeError(f"bench_lds_activation: {rc}")
    for _ in range(2):
        launch()
    ev = rx.HipEvents(2)
    ev.record(0)
    for _ in range(reps):
        launch()
    ev.record(1)
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(0, 1) / reps
    ev.close()
    return dict(ms=ms, items=groups, bytes_per_item=per.value,
                TBps=per.value * groups / (ms * 1e-3) / 1e12)


def cpu_baseline(inp, n_episodes, precision=0, dqn=False):
    """The oracle as it stands on a bounded episode subset of the same
    workload (all of it when n_episodes >= N)."""
    import numpy as np
    import oracle

    n_episodes = min(n_episodes, inp["N"])
    sub = None if n_episodes == inp["N"] else np.linspace(0, inp["N"] - 1, n_episodes).astype(np.int32)
    threads = _threads()
    t0 = time.perf_counter()
    if dqn:
        oracle.dqn_rollout(inp, subset=sub, n_threads=threads, with_q=False, with_next=False)
    else:
        oracle.rollout(inp, precision=precision, subset=sub, n_threads=threads, with_logits=False)
    dt = time.perf_counter() - t0
    exp = n_episodes * inp["L"]
    part = ("all" if sub is None else f"{n_episodes} of") + f" {inp['N']} episodes"
    return dict(value=exp / dt, unit="transitions/s" if dqn else "experiences/s", cores=threads,
                kind="oracle",
                sample=f"{part} x {inp['L']} steps ({exp} {'transitions' if dqn else 'experiences'}, "
                       f"{dt:.1f} s) of the N={inp['N']} L={inp['L']} "
                       f"{'DQN ' if dqn else ''}workload{' in the bf16 mode' if precision else ''}"
                       f"; episodes are independent; host CPU: {_host_cpu()}")


def cpu_baseline_gae(spec):
    """The oracle's GAE scan (one host thread: it is a plain loop) on the
    whole standalone workload."""
    import oracle
    import synthdata
    r, v, d = synthdata.gae_inputs(spec["N"], spec["L"], spec["seed"])
    t0 = time.perf_counter()
    oracle.gae(r, v, d, 0.99, 0.95)
    dt = time.perf_counter() - t0
    n = spec["N"] * spec["L"]
    return dict(value=GAE_BYTES * n / dt / 1e9, unit="GB/s", elements_per_s=n / dt, cores=1,
                kind="oracle", sample=f"all {n} elements (N={spec['N']} L={spec['L']}, {dt:.3f} s); "
                                      f"host CPU: {_host_cpu()}")


def recycled(inp):
    """The same workload with dynamic episode recycling on."""
    return dict(inp, settings=dict(inp["settings"], recycle=1))


def run_single(name, steps, warmup):
    """One workload, for profiler counter passes."""
    import torch
    import synthdata
    if name.startswith("collect"):
        inp = synthdata.ppo_inputs("ppo_n128_l500" if name == "collect_n128_fp32" else "ppo_n8192_l500")
        if name.endswith("recycle"):
            inp = recycled(inp)
        r = time_collect(inp, steps, warmup, precision=1 if name.endswith("bf16") else 0)
        return dict(workload=name, ms_per_step=r["wall_s"] * 1000 / steps,
                    phases_ms=[float(x) for x in r["phases_ms"]])
    if name.startswith("gae"):
        spec = (synthdata.WORKLOADS["gae_n4096_l2048"] if name.endswith("n4096_l2048")
                else dict(N=8192, L=500, seed=synthdata.WORKLOADS["ppo_n8192_l500"]["seed"]))
        r = time_gae(spec, steps, traffic_only=name.startswith("gae_traffic"))
        return dict(workload=name, cold_ms=r["cold_ms"], warm_ms=r["warm_ms"])
    if name.startswith("dqn"):
        inp = synthdata.dqn_inputs("dqn_n16384_l500")
        r = time_dqn(recycled(inp) if name.endswith("recycle") else inp, steps, warmup)
        return dict(workload=name, ms_per_step=r["wall_s"] * 1000 / steps, kernel_ms=r["kernel_ms"],
                    exp_per_s=r["N"] * r["L"] * steps / r["wall_s"],
                    TFLOPs=DQN_FLOP * r["N"] * r["L"] / (r["kernel_ms"] * 1e-3) / 1e12,
                    nonfinite=r["nonfinite"])
    if name.startswith("per"):
        return dict(workload=name, **time_per(16384 * 500, 4096, steps))
    if name == "lds_activation_bf16":
        return dict(workload=name, **time_lds_activation(8192 * 500, steps))
    if name.startswith("weight_stream"):
        return dict(workload=name, **time_weight_stream(8192 * 500, name.endswith("bf16"), steps))
    a = torch.ones(1 << 28, device="cuda")  # copy_1gib: 1 GiB read + 1 GiB written per copy
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    return dict(workload=name, copies=steps, bytes_each_way=1 << 30)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-episodes", type=int, default=2560)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="all",
                    choices=("all", "collect_n8192_fp32", "collect_n8192_bf16", "collect_n128_fp32",
                             "collect_n8192_fp32_recycle", "dqn_n16384_l500_recycle",
                             "gae_n4096_l2048", "gae_n8192_l500", "gae_traffic_n4096_l2048",
                             "gae_traffic_n8192_l500", "weight_stream_fp32", "weight_stream_bf16",
                             "lds_activation_bf16",
                             "dqn_n16384_l500", "per_n8192000_b4096",
                             "copy_1gib"),
                    help="one workload only (for profiler counter passes); prints its own "
                         "JSON line instead of the benchmark line")
    ap.add_argument("--value-power", action="store_true",
                    help="socket power and shader clock (amd-smi) while the N=8192 L=500 "
                         "collection runs back to back in bf16, bf16 with zeroed value weights "
                         "and fp32, one JSON line each, instead of the benchmark line")
    ap.add_argument("--actor-stamps", action="store_true",
                    help="per-phase cycles of the sequential step (instrumented kernel) at "
                         "N=128 L=500 and N=8192 L=500, fp32 and bf16, one JSON line each, "
                         "instead of the benchmark line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the collection shards by episode and runs with no "
              f"communication; --gpus {args.gpus} is not supported (one GPU per process).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synthdata
    assert torch.cuda.is_available(), "bench.py needs the GPU"

    if args.workload != "all":
        print(json.dumps(run_single(args.workload, args.steps, args.warmup)), flush=True)
        return
    if args.value_power:
        for r in value_power(synthdata.ppo_inputs("ppo_n8192_l500")):
            print(json.dumps(r), flush=True)
        return
    if args.actor_stamps:
        for name, prec in (("ppo_n128_l500", 0), ("ppo_n128_l500", 1), ("ppo_n8192_l500", 0),
                           ("ppo_n8192_l500", 1)):
            r = actor_phase_stamps(synthdata.ppo_inputs(name), max(3, min(args.steps, 10)), prec)
            print(json.dumps(dict(workload=name, **r)), flush=True)
        return

    spec = dict(synthdata.WORKLOADS["ppo_n8192_l500"])
    log("generating inputs ...")
    big_inp = synthdata.ppo_inputs(spec)
    log("timing N=8192 L=500 fp32 ...")
    big = time_collect(big_inp, args.steps, args.warmup)
    N, L = big["N"], big["L"]
    ms = big["wall_s"] * 1000 / args.steps
    exps = N * L * args.steps / big["wall_s"]
    t_roll, t_val, t_gae = big["phases_ms"]
    log("timing N=8192 L=500 bf16 ...")
    bfr = time_collect(big_inp, args.steps, args.warmup, precision=1)
    log("timing N=8192 L=500 bf16 with zeroed critic and curiosity weights ...")
    bfz = time_collect(zero_value_weights(big_inp), args.steps, args.warmup, precision=1)
    log("timing N=8192 L=500 fp32 with episode recycling ...")
    rec = time_collect(recycled(big_inp), args.steps, args.warmup)
    log("timing N=128 L=500 fp32 ...")
    small = time_collect(synthdata.ppo_inputs("ppo_n128_l500"), args.steps, args.warmup)
    log("timing GAE N=4096 L=2048 and N=8192 L=500 ...")
    gae = time_gae(synthdata.WORKLOADS["gae_n4096_l2048"], max(args.steps, 20))
    gae_c = time_gae(dict(N=N, L=L, seed=spec["seed"]), max(args.steps, 20))
    log("timing the ceilings: GAE traffic element-wise, value-kernel weight stream ...")
    gae_x = time_gae(synthdata.WORKLOADS["gae_n4096_l2048"], max(args.steps, 20), traffic_only=True)
    gae_cx = time_gae(dict(N=N, L=L, seed=spec["seed"]), max(args.steps, 20), traffic_only=True)
    log("timing the vendor copy at the scans' byte counts and at 1 GiB ...")
    cp_c = time_vendor_copy(GAE_BYTES * N * L)
    cp_x = time_vendor_copy(GAE_BYTES * gae["elements"])
    cp_g = time_vendor_copy(1 << 31, reps=5)
    ws_f = time_weight_stream(N * L, False, 5)
    ws_b = time_weight_stream(N * L, True, 5)
    lds_b = time_lds_activation(N * L, 5)
    log("timing the vendor GEMM references (bf16, fp32) ...")
    gemm_b = max((time_gemm_reference("bf16"), time_gemm_reference("bf16", 16384, reps=3)),
                 key=lambda r: r["TFLOPs"])
    gemm_f = time_gemm_reference("fp32", reps=3)
    log("timing the DQN collection N=16384 L=500 ...")
    dq_inp = synthdata.dqn_inputs("dqn_n16384_l500")
    dq = time_dqn(dq_inp, args.steps, args.warmup)
    dq_exp = dq["N"] * dq["L"]
    log("timing the DQN collection N=16384 L=500 with episode recycling ...")
    dqr = time_dqn(recycled(dq_inp), args.steps, args.warmup)
    log("timing prioritized replay on 8,192,000 priorities ...")
    per = time_per(dq_exp, 4096, max(args.steps, 20))
    per_step = per["sample_ms"] + per["gather_ms"] + per["update_ms"]

    value_files = ["rl_experience_collection_amd/csrc/value.hip",
                   "rl_experience_collection_amd/csrc/nets.hpp",
                   "rl_experience_collection_amd/csrc/device.hpp"]
    traffic = load_traffic("value_kernel_n8192_l500_traffic.txt", value_files)
    achieved = VALUE_KERNEL_FLOP * N * L / (t_val * 1e-3)
    roofline = dict(bound="mfma", achieved=achieved / 1e12, peak=PEAK_FP32_MFMA / 1e12,
                    unit="TFLOP/s", frac=achieved / PEAK_FP32_MFMA, traffic=traffic,
                    traffic_unit="HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                 "copy-calibrated; null if the kernel changed since)",
                    algorithmic_bytes_per_launch=4096000 * 436,
                    kernel="value_kernel (critic + curiosity, fp32 MFMA 16x16x4)",
                    flop_per_launch=VALUE_KERNEL_FLOP * N * L, avg_launch_ms=t_val,
                    weight_stream_bound=dict(ms=ws_f["ms"], TBps=ws_f["TBps"],
                                             bytes_per_launch=ws_f["bytes_per_launch"]),
                    gemm_reference=dict(gemm_f, frac_of_fp32_peak=gemm_f["TFLOPs"] * 1e12 / PEAK_FP32_MFMA,
                                        value_kernel_frac_of_gemm=achieved / 1e12 / gemm_f["TFLOPs"]))
    mlp_util = MLP_FLOP * N * L / ((t_roll + t_val) * 1e-3) / PEAK_FP32_MFMA
    # N=128: 8 workgroups of 16 episodes hold 8 CUs through the sequential
    # chain; the actor's work against the fp32 MFMA peak of those CUs
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    active = -(-128 // 16)
    t_small_actor = float(small["phases_ms"][0])
    small_achieved = ACTOR_FLOP * 128 * 500 / (t_small_actor * 1e-3)
    small_roof = dict(bound="mfma", kernel="actor_rollout_kernel (sequential chain, 8 workgroups)",
                      achieved=small_achieved / 1e12, unit="TFLOP/s",
                      peak=PEAK_FP32_MFMA * active / cus / 1e12, active_cus=active,
                      frac=small_achieved / (PEAK_FP32_MFMA * active / cus),
                      actor_ms=t_small_actor, flop_per_launch=ACTOR_FLOP * 128 * 500,
                      note="peak = the fp32 MFMA peak scaled to the CUs the rollout occupies")
    gae_in = 17 * N * L / (t_gae * 1e-3)

    line = dict(
        metric=METRIC, value=exps, unit="experiences/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=ms, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="f32", data="synthetic",
        config=dict(workload="ppo_collect_n8192_l500_fp32", episodes=N, steps_per_episode=L,
                    bars=spec["n_bars"], experiences_per_step=N * L, precision="fp32"),
        roofline=roofline,
        phases_ms=dict(actor_rollout=t_roll, value_critic_curiosity=t_val, gae_scan=t_gae),
        mlp_mfma_util=mlp_util,
        gae_in_collect_GBps=gae_in / 1e9,
        nonfinite_events=big["nonfinite"],
        device=device_info(),
        also=dict(
            ppo_collect_n8192_l500_bf16=dict(
                value=N * L * args.steps / bfr["wall_s"], unit="experiences/s",
                ms_per_step=bfr["wall_s"] * 1000 / args.steps,
                phases_ms=dict(zip(("actor_rollout", "value_critic_curiosity", "gae_scan"),
                                   map(float, bfr["phases_ms"]))),
                value_kernel_TFLOPs=VALUE_KERNEL_FLOP * N * L / (bfr["phases_ms"][1] * 1e-3) / 1e12,
                value_kernel_frac_of_bf16_peak=VALUE_KERNEL_FLOP * N * L /
                (bfr["phases_ms"][1] * 1e-3) / PEAK_BF16_MFMA,
                # the value kernel streams its weights from L2 once per work item:
                # the bound is the slower of the MFMA peak and that stream alone
                weight_stream_bound_ms=ws_b["ms"], weight_stream_TBps=ws_b["TBps"],
                weight_stream_bytes_per_launch=ws_b["bytes_per_launch"],
                # its activation operands cross the CU's LDS once per wave and layer:
                # that traffic alone, with the kernel's barriers
                lds_stream_bound_ms=lds_b["ms"], lds_stream_TBps=lds_b["TBps"],
                lds_bytes_per_item=lds_b["bytes_per_item"],
                value_kernel_frac_of_bound=max(ws_b["ms"], lds_b["ms"], VALUE_KERNEL_FLOP * N * L /
                                               PEAK_BF16_MFMA * 1e3) / float(bfr["phases_ms"][1]),
                # what the matrix cores sustain here on random bf16 operands (a
                # large square product in the vendor library), and the value
                # kernel on zero operands: the bf16 rate is bounded by power,
                # and so the clock, not by the published peak
                gemm_reference=dict(gemm_b, frac_of_bf16_peak=gemm_b["TFLOPs"] * 1e12 / PEAK_BF16_MFMA,
                                    value_kernel_frac_of_gemm=VALUE_KERNEL_FLOP * N * L /
                                    (bfr["phases_ms"][1] * 1e-3) / 1e12 / gemm_b["TFLOPs"]),
                value_kernel_ms_zero_weights=float(bfz["phases_ms"][1])),
            dqn_collect_n16384_l500_fp32=dict(
                value=dq_exp * args.steps / dq["wall_s"], unit="experiences/s",
                ms_per_step=dq["wall_s"] * 1000 / args.steps, kernel_ms=dq["kernel_ms"],
                flop_per_experience=DQN_FLOP,
                TFLOPs=DQN_FLOP * dq_exp / (dq["kernel_ms"] * 1e-3) / 1e12,
                frac_of_fp32_peak=DQN_FLOP * dq_exp / (dq["kernel_ms"] * 1e-3) / PEAK_FP32_MFMA,
                nonfinite_events=dq["nonfinite"]),
            ppo_collect_n8192_l500_fp32_recycle=dict(
                value=N * L * args.steps / rec["wall_s"], unit="experiences/s",
                ms_per_step=rec["wall_s"] * 1000 / args.steps,
                phases_ms=dict(zip(("actor_rollout", "value_critic_curiosity", "gae_scan"),
                                   map(float, rec["phases_ms"]))),
                nonfinite_events=rec["nonfinite"]),
            dqn_collect_n16384_l500_fp32_recycle=dict(
                value=dq_exp * args.steps / dqr["wall_s"], unit="experiences/s",
                ms_per_step=dqr["wall_s"] * 1000 / args.steps, kernel_ms=dqr["kernel_ms"],
                frac_of_fp32_peak=DQN_FLOP * dq_exp / (dqr["kernel_ms"] * 1e-3) / PEAK_FP32_MFMA,
                nonfinite_events=dqr["nonfinite"]),
            per_n8192000_b4096=dict(
                value=per["batch"] / (per_step * 1e-3), unit="sampled transitions/s",
                step_ms=per_step, sample_ms=per["sample_ms"], gather_ms=per["gather_ms"],
                update_ms=per["update_ms"],
                priority_read_GBps=4 * per["n"] / (per["sample_ms"] * 1e-3) / 1e9,
                note="one replay step: draw 4096 of 8,192,000 (one DQN collection), gather "
                     "their rows, update their priorities"),
            ppo_collect_n128_l500_fp32=dict(
                value=128 * 500 * args.steps / small["wall_s"], unit="experiences/s",
                ms_per_step=small["wall_s"] * 1000 / args.steps,
                phases_ms=dict(zip(("actor_rollout", "value_critic_curiosity", "gae_scan"),
                                   map(float, small["phases_ms"]))),
                roofline=small_roof,
                note="the rollout runs as a few launches of consecutive steps (4 on 256 CUs: "
                     "3 of 145-146 steps, then 64); the value pass of each finished part "
                     "overlaps the next part on the CUs the rollout leaves free, so "
                     "value_critic_curiosity is only the pass after the rollout"),
            gae_scan_n4096_l2048=dict(
                value=GAE_BYTES * gae["elements"] / (gae["cold_ms"] * 1e-3) / 1e9, unit="GB/s",
                frac_of_hbm_peak=GAE_BYTES * gae["elements"] / (gae["cold_ms"] * 1e-3) / PEAK_HBM,
                cold_ms=gae["cold_ms"], warm_ms=gae["warm_ms"],
                warm_GBps=GAE_BYTES * gae["elements"] / (gae["warm_ms"] * 1e-3) / 1e9,
                copy_ceiling_cold_ms=gae_x["cold_ms"], copy_ceiling_warm_ms=gae_x["warm_ms"],
                frac_of_copy_ceiling_cold=gae_x["cold_ms"] / gae["cold_ms"],
                vendor_copy_same_bytes_cold_ms=cp_x["cold_ms"],
                frac_of_vendor_copy_cold=cp_x["cold_ms"] / gae["cold_ms"]),
            gae_scan_n8192_l500=dict(
                value=GAE_BYTES * gae_c["elements"] / (gae_c["cold_ms"] * 1e-3) / 1e9, unit="GB/s",
                frac_of_hbm_peak=GAE_BYTES * gae_c["elements"] / (gae_c["cold_ms"] * 1e-3) / PEAK_HBM,
                cold_ms=gae_c["cold_ms"], warm_ms=gae_c["warm_ms"],
                warm_GBps=GAE_BYTES * gae_c["elements"] / (gae_c["warm_ms"] * 1e-3) / 1e9,
                warm_frac_of_hbm_peak=GAE_BYTES * gae_c["elements"] / (gae_c["warm_ms"] * 1e-3)
                / PEAK_HBM,
                copy_ceiling_cold_ms=gae_cx["cold_ms"], copy_ceiling_warm_ms=gae_cx["warm_ms"],
                frac_of_copy_ceiling_cold=gae_cx["cold_ms"] / gae_c["cold_ms"],
                # torch's own device copy moving the same bytes, and a 1 GiB
                # copy: what HBM streaming reaches here at this size and at
                # a size where launch and drain no longer count
                vendor_copy_same_bytes_cold_ms=cp_c["cold_ms"],
                frac_of_vendor_copy_cold=cp_c["cold_ms"] / gae_c["cold_ms"],
                vendor_copy_1gib_each_way=dict(cold_ms=cp_g["cold_ms"], TBps=cp_g["TBps"],
                                               frac_of_hbm_peak=cp_g["TBps"] * 1e12 / PEAK_HBM))),
    )
    if not args.no_cpu_baseline:
        log("timing the oracle on the host ...")
        line["cpu_baseline"] = cpu_baseline(big_inp, args.cpu_episodes)
        also = line["also"]
        also["ppo_collect_n128_l500_fp32"]["cpu_baseline"] = cpu_baseline(
            synthdata.ppo_inputs("ppo_n128_l500"), 128)
        also["ppo_collect_n8192_l500_bf16"]["cpu_baseline"] = cpu_baseline(
            big_inp, max(args.cpu_episodes // 4, 16), precision=1)
        also["gae_scan_n4096_l2048"]["cpu_baseline"] = cpu_baseline_gae(
            synthdata.WORKLOADS["gae_n4096_l2048"])
        also["gae_scan_n8192_l500"]["cpu_baseline"] = cpu_baseline_gae(
            dict(N=N, L=L, seed=spec["seed"]))
        also["dqn_collect_n16384_l500_fp32"]["cpu_baseline"] = cpu_baseline(
            dq_inp, max(args.cpu_episodes // 2, 16), dqn=True)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
