"""Build libbnn.so (the HIP library behind include/bnn.h) and libbnn_calib.so
(the rate probes behind include/bnn_calib.h) in-tree for gfx950.

    python -m packed_xor_popcount_amd.build        # or: python packed_xor_popcount_amd/build.py

Every translation unit is compiled to its own object for gfx950 only (in
parallel, under _build/), then the objects are linked into the shared
libraries.  Packed-fp32 instruction selection is disabled (-packed-fp32-ops);
no fast-math.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
CALIB_SRC = os.path.join(CSRC, "calib")
LIB = os.path.join(HERE, "libbnn.so")
CALIB_LIB = os.path.join(HERE, "libbnn_calib.so")
ROOT = os.path.dirname(HERE)
OBJ = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-ffp-contract=off", "-Wall",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def calib_sources():
    return sorted(glob.glob(os.path.join(CALIB_SRC, "*.hip")))


def _compile(src: str, verbose: bool) -> str:
    rel = os.path.relpath(src, CSRC).replace(os.sep, "_")
    obj = os.path.join(OBJ, rel + ".o")
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return obj


def _link(objs, out: str, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every translation unit and link both libraries; returns the
    path of libbnn.so."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    csrcs = calib_sources()
    jobs = int(os.environ.get("MAX_JOBS", "8"))
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, 16))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs + csrcs))
    _link(objs[: len(srcs)], LIB, verbose)
    if csrcs:
        _link(objs[len(srcs):], CALIB_LIB, verbose)
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
