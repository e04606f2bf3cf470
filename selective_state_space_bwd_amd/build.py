"""Build the gfx950 HIP library in place: ``python -m selective_state_space_bwd_amd.build``.

Compiles every ``csrc/*.hip`` with hipcc for gfx950 (one process per source,
in parallel, into a build folder beside the sources) and links them into
``libssmbwd.so`` next to this file.  Packed fp32 instructions are switched off
for all device code.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libssmbwd.so")
ARCH = os.environ.get("SSMBWD_ARCH", "gfx950")

OBJ_DIR = os.path.join(HERE, "_build")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-function",
]
NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in res.stderr.splitlines() if NOISE not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    cc = hipcc()
    objs = [os.path.join(OBJ_DIR, os.path.basename(src)[:-4] + ".o") for src in sources()]
    jobs = [[cc, *FLAGS, *extra_flags, "-c", src, "-o", obj] for src, obj in zip(sources(), objs)]
    workers = max(1, min(len(jobs), len(os.sched_getaffinity(0))))
    with concurrent.futures.ThreadPoolExecutor(workers) as pool:
        for f in [pool.submit(_run, cmd, verbose) for cmd in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-fno-gpu-rdc", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
