"""Build libeplb.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python moe_expert_load_eplb_amd/build.py

Compiles every source under csrc/ with hipcc (one object per source, in
parallel, under _build/) and links them into one shared library next to this
file.  Always recompiles.  Run it by path (not as ``-m``): importing the
package would load the library being rebuilt.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libeplb.so")
# the benchmark's reference streams (copy / read-only), not part of the library
REF_LIB = os.path.join(PKG, "libeplb_ref.so")
REF_SOURCES = [os.path.join("ref", "stream_ref.hip")]
ARCH = "gfx950"

SOURCES = ["api.hip", "hist.hip", "rebalance.hip", "redirect.hip", "fused.hip", "quality.hip", "rearrange.hip", "lp.hip",
           "lp_noalloc.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the EPLB library needs ROCm's hipcc")


BUILD = os.path.join(PKG, "_build")
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         # packed-FP32 instructions are kept out of every kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         f"-I{INCLUDE}", f"-I{CSRC}"]


def compile_command(src: str, obj: str) -> list[str]:
    return [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]


def link_command(objs: list[str], out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared", *objs, "-o", out]


def _run(cmd: list[str]) -> tuple[int, str]:
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    return res.returncode, "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + REF_SOURCES
    objs = [os.path.join(BUILD, os.path.basename(os.path.splitext(s)[0]) + ".o") for s in srcs]
    cmds = [compile_command(s, o) for s, o in zip(srcs, objs)]
    jobs = max(1, min(len(cmds), len(os.sched_getaffinity(0)), 16))
    with ThreadPoolExecutor(jobs) as pool:
        results = list(pool.map(_run, cmds))
    for cmd, (rc, err) in zip(cmds, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError(f"hipcc failed ({rc}):\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
    for lib, part in ((LIB, objs[:len(SOURCES)]), (REF_LIB, objs[len(SOURCES):])):
        tmp = lib + ".tmp"
        cmd = link_command(part, tmp)
        if verbose:
            print(" ".join(cmd), flush=True)
        rc, err = _run(cmd)
        if rc != 0:
            raise RuntimeError(f"hipcc link failed ({rc}):\n{err}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
