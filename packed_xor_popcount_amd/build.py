"""Build libbnn.so (the HIP library behind include/bnn.h) in-tree for gfx950.

    python -m packed_xor_popcount_amd.build        # or: python packed_xor_popcount_amd/build.py

One hipcc invocation compiles every translation unit under csrc/ for
gfx950 only.  Packed-fp32 instruction selection is disabled
(-packed-fp32-ops); no fast-math.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbnn.so")
ROOT = os.path.dirname(HERE)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def hipcc_cmd(out: str = LIB, extra=()):
    return [
        HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-fno-fast-math", "-ffp-contract=off", "-Wall",
        "-I", os.path.join(ROOT, "include"),
        *extra, *sources(), "-o", out,
    ]


def build(verbose: bool = False) -> str:
    cmd = hipcc_cmd()
    if verbose:
        print(" ".join(cmd), flush=True)
    tmp = LIB + ".tmp"
    cmd[-1] = tmp
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = sources() + glob.glob(os.path.join(CSRC, "*.h")) + [os.path.join(ROOT, "include", "bnn.h")]
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
