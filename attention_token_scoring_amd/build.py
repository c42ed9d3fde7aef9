"""Builds libspecprefill.so in-tree from csrc/*.hip with hipcc for gfx950.

Each source compiles to its own object (in parallel), then one link step.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libspecprefill.so")
OBJ = os.path.join(HERE, "_obj")
ARCH = os.environ.get("SP_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # selection must reproduce IEEE single/double steps exactly: no FMA contraction
    "-ffp-contract=off",
    # no packed fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# The scoring kernels assume finite inputs: without NaN semantics the compiler
# folds the DPP lane moves into the v_max that consumes them.
SCORE_FLAGS = ["-fno-honor-nans"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _flags_for(src: str) -> list[str]:
    base = os.path.basename(src)
    return FLAGS + (SCORE_FLAGS if base.startswith("sp_score") else [])


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{errs}")


def build(force: bool = True, verbose: bool = False, jobs: int | None = None) -> str:
    if not force and os.path.exists(LIB):
        return LIB
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJ, os.path.basename(s)[:-4] + ".o") for s in srcs]
    if jobs is None:
        jobs = max(1, min(len(srcs), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_run, [_hipcc(), *_flags_for(s), "-c", s, "-o", o], verbose)
                for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
    tmp = LIB + ".tmp"
    _run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
