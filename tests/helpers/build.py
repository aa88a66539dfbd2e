"""Build test helpers (host-only programs; no GPU is touched)."""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PHILOX_REF = os.path.join(HERE, "philox_ref")
SAN_DIR = os.path.join(ROOT, "_build", "sanitize")


def build_philox_ref() -> str:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    src = os.path.join(HERE, "philox_ref.cpp")
    subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", src, "-o",
                    PHILOX_REF + ".tmp"], check=True, stdout=subprocess.DEVNULL,
                   stderr=subprocess.DEVNULL)
    os.replace(PHILOX_REF + ".tmp", PHILOX_REF)
    return PHILOX_REF


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stderr[-4000:]}")


def build_sanitized_oracle(planted: bool = False) -> str:
    """The oracle and its driver under AddressSanitizer + UBSan (gcc, host);
    planted=True adds an out-of-bounds call to the driver."""
    os.makedirs(SAN_DIR, exist_ok=True)
    exe = os.path.join(SAN_DIR, "sanitize_oracle" + ("_planted" if planted else ""))
    _run(["gcc", "-O1", "-g", "-std=c99", "-fno-omit-frame-pointer", "-ffp-contract=off",
          *(["-DPLANT_OUT_OF_BOUNDS"] if planted else []),
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fopenmp",
          os.path.join(HERE, "sanitize_oracle.c"), os.path.join(ROOT, "oracle", "oracle.c"),
          "-o", exe, "-lm"])
    return exe


def build_sanitized_abi() -> str:
    """The library's C-ABI translation unit with its host code under
    AddressSanitizer + UBSan, linked with the other (unchanged) objects of the
    library and the driver.  The device code is built as usual."""
    from rl_experience_collection_amd import build as hip_build
    os.makedirs(SAN_DIR, exist_ok=True)
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clangxx = "/opt/rocm/llvm/bin/clang++"
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    objs = [os.path.join(hip_build.OBJ, s.replace(".hip", ".o")) for s in hip_build.SOURCES
            if s != "abi.hip"]
    if not all(os.path.exists(o) for o in objs):
        hip_build.build()
    abi = os.path.join(SAN_DIR, "abi_san.o")
    _run([hipcc, *hip_build.FLAGS, "-O1", "-g", "-fno-omit-frame-pointer", *san, "-c",
          os.path.join(hip_build.CSRC, "abi.hip"), "-o", abi])
    drv = os.path.join(SAN_DIR, "sanitize_abi.o")
    _run([clangxx, "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-c",
          os.path.join(HERE, "sanitize_abi.cpp"), "-o", drv])
    exe = os.path.join(SAN_DIR, "sanitize_abi")
    _run([hipcc, f"--offload-arch={hip_build.ARCH}", *san, drv, abi, *objs, "-o", exe])
    return exe


if __name__ == "__main__":
    print(build_philox_ref())
