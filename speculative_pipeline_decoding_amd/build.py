"""Build libspd.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

Usage: python -m speculative_pipeline_decoding_amd.build [-v]
The library lands next to this file; object files go to <repo>/_build/.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libspd.so")
ARCH = os.environ.get("SPD_OFFLOAD_ARCH", "gfx950")

SOURCES = ["spd_api.hip", "gemv.hip", "attention.hip", "linear.hip", "vocab.hip", "small.hip", "gemm.hip"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernel arguments arrive preloaded in SGPRs (gfx950): a kernel's first dependent
    # load, the descriptor address, needs no round trip (0.3-1 us per launch)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wno-unused-result",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int = 8) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for s in SOURCES:
        obj = os.path.join(BUILD, s.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *FLAGS, "-c", os.path.join(CSRC, s), "-o", obj])
    with ThreadPoolExecutor(min(jobs, len(cmds))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
