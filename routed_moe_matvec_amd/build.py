"""Build libqgemv.so (HIP, gfx950) in-tree with hipcc.

Each source is compiled to an object on its own (in parallel), then the
objects are linked into the shared library.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqgemv.so")
OBJDIR = os.path.join(ROOT, "_build", "qgemv")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no v_pk_*_f32 generation on this target.
# -ffp-contract=off: every fused multiply-add is an explicit fmaf, so kernels
#  that share a decoder round identically.
# correctly rounded fp32 division: the activation quantizer is bit-exact.
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Wall",
]
LINK_FLAGS = ["--offload-arch=gfx950", "-shared", "-fPIC"]

# the host pass does not know the target feature; that warning is expected
_NOISE = "is not a recognized feature for this target"


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in proc.stderr.splitlines() if _NOISE not in l)
    if proc.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError("hipcc failed (%d): %s" % (proc.returncode, " ".join(cmd[-3:])))
    if err.strip() and verbose:
        sys.stderr.write(err + "\n")


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJDIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cmds = [[HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, *LINK_FLAGS, *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
