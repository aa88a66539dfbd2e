"""Build test helpers (host-only programs; no GPU is touched)."""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
PHILOX_REF = os.path.join(HERE, "philox_ref")


def build_philox_ref() -> str:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    src = os.path.join(HERE, "philox_ref.cpp")
    subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", src, "-o",
                    PHILOX_REF + ".tmp"], check=True, stdout=subprocess.DEVNULL,
                   stderr=subprocess.DEVNULL)
    os.replace(PHILOX_REF + ".tmp", PHILOX_REF)
    return PHILOX_REF


if __name__ == "__main__":
    print(build_philox_ref())
