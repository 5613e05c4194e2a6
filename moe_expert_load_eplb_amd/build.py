"""Build libeplb.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python moe_expert_load_eplb_amd/build.py

Compiles every source under csrc/ with hipcc into one shared library next to
this file.  Always recompiles.  Run it by path (not as ``-m``): importing the
package would load the library being rebuilt.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libeplb.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "hist.hip", "rebalance.hip", "redirect.hip", "fused.hip", "quality.hip", "rearrange.hip", "lp.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the EPLB library needs ROCm's hipcc")


def command(out: str = LIB) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-function",
            # packed-FP32 instructions are kept out of every kernel
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{INCLUDE}", f"-I{CSRC}",
            *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
