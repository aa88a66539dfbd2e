"""Build librollout.so (HIP, gfx950) in-tree with hipcc."""
import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(os.path.dirname(PKG), "_build", "rollout")
LIB = os.path.join(PKG, "librollout.so")
SOURCES = ["abi.hip", "pack.hip", "rollout.hip", "value.hip", "gae.hip", "dqn.hip", "per.hip"]
# measurement kernels used by bench.py only, in a library of their own
PROBE_LIB = os.path.join(PKG, "libbenchprobes.so")
PROBE_SOURCES = ["bench_probes.hip"]
ARCH = os.environ.get("ROLLOUT_OFFLOAD_ARCH", "gfx950")
# The device compiler's atomic optimizer turns an atomic that one lane
# issues into a wave-aggregated one whose returned value is broadcast at once,
# which waits for every load the wave has in flight (the value kernel's work
# ticket, taken while its next layer's weights stream in); none of the
# library's atomics gains from aggregation, so it is off.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xarch_device", "-mllvm=-amdgpu-atomic-optimizer-strategy=None",
]


def _hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _compile(src):
    obj = os.path.join(OBJ, src.replace(".hip", ".o"))
    cmd = [_hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return obj, err


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        results = list(ex.map(_compile, srcs))
    for _, err in results:
        if verbose and err.strip():
            print(err)
    objs = [o for o, _ in results]
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
