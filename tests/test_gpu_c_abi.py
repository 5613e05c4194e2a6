"""The C ABI driven from a plain C program (HIP runtime for device memory,
no Python in between): the pages' worked example through eplb_rebalance
(needs an MI355X)."""
from __future__ import annotations

import os
import subprocess

import pytest

from test_abi_cpu import ROOT, _cc

pytestmark = pytest.mark.gpu


def test_worked_example_from_c(tmp_path):
    exe = _cc(os.path.join(ROOT, "tests", "c", "abi_gpu.c"), str(tmp_path / "abi_gpu"),
              ("-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include"),
              ("-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"))
    print("[c-abi] running the worked example from C", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "abi_gpu ok" in r.stdout
