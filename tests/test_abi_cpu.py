"""The C ABI on a machine without a GPU: the library loads, exports every
function include/eplb.h declares, and rejects bad arguments on the host with
the documented codes before touching the device."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import eplb_oracle as ora

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "eplb.h")
LIB = os.path.join(ROOT, "moe_expert_load_eplb_amd", "libeplb.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libeplb.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(eplb_[a-z_0-9]+)\s*\(", text, flags=re.M)


def header_constants():
    return {m.group(1): int(m.group(2)) for m in
            re.finditer(r"#define\s+(EPLB_[A-Z_]+)\s+(-?\d+)", open(HEADER).read())}


@pytest.fixture(scope="module")
def lib():
    lib = ctypes.CDLL(LIB)
    p, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.eplb_load_hist.argtypes = [p, i64, i64, i32, i32, p, i32, i64, p, p, p]
    lib.eplb_rebalance.argtypes = [p, i64, i32, i32, i32, i32, i32, i32, p, p, p, p, p]
    lib.eplb_redirect.argtypes = [p, i64, i64, i32, i32, p, p, i32, p, p]
    lib.eplb_hist_redirect.argtypes = [p, i64, i64, i32, i32, p, i32, i64, p, p, p, p, i32, p, p]
    lib.eplb_load_ema.argtypes = [p, i64, i64, i32, i32, p, i32, p, p, p]
    lib.eplb_placement_load.argtypes = [p, p, p, i64, i32, i32, i32, p, p, p]
    lib.eplb_ema_redirect.argtypes = [p, i64, i64, i32, i32, p, i32, p, p, p, p, i32, p, p]
    lib.eplb_rearrange.argtypes = [p, p, p, i64, i32, i32, i32, i32, i32, p, p, p, p, p, p]
    lib.eplb_lp_solve.argtypes = [p, p, p, i64, i32, i32, i32, p, p, p, p, p]
    lib.eplb_lp_redirect.argtypes = [p, i64, i64, i32, i32, p, p, i32, i32, p, i64, p, p]
    lib.eplb_lp_redirect_workspace_bytes.argtypes = [i64, i64, i32, i32]
    lib.eplb_lp_redirect_workspace_bytes.restype = i64
    lib.eplb_status_string.restype = ctypes.c_char_p
    lib.eplb_rebalance_lds_bytes.argtypes = [i32] * 6
    lib.eplb_rebalance_lds_bytes.restype = i64
    lib.eplb_rebalance_max_count.argtypes = [i32] * 4
    lib.eplb_rebalance_max_count.restype = i32
    return lib


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) >= {"eplb_load_hist", "eplb_rebalance", "eplb_redirect", "eplb_status_string",
                          "eplb_rebalance_lds_bytes", "eplb_hist_redirect", "eplb_load_ema",
                          "eplb_placement_load", "eplb_rearrange", "eplb_lp_solve", "eplb_lp_redirect", "eplb_ema_redirect",
                          "eplb_lp_redirect_workspace_bytes", "eplb_rebalance_max_count",
                          "eplb_lp_redirect_noalloc"}
    for n in names:
        assert hasattr(lib, n), f"{n} declared in eplb.h but not exported"


def test_codes_match_binding_and_oracle():
    c = header_constants()
    assert c["EPLB_OK"] == 0 and len({v for k, v in c.items() if k.startswith("EPLB_E_")}) == 7
    assert c["EPLB_S_BAD_LOAD"] == ora.STATUS_BAD_LOAD and c["EPLB_S_OVERFLOW"] == ora.STATUS_OVERFLOW
    assert c["EPLB_S_BAD_MAP"] == ora.STATUS_BAD_MAP and c["EPLB_S_BAD_TOPOLOGY"] == ora.STATUS_BAD_TOPOLOGY
    src = open(os.path.join(ROOT, "moe_expert_load_eplb_amd", "__init__.py")).read()
    for k, v in c.items():
        if k.startswith("EPLB_"):
            assert re.search(rf"^{k} = {v}$", src, flags=re.M), k


def test_status_strings(lib):
    for code in range(8):
        assert lib.eplb_status_string(code)
    assert b"unknown" in lib.eplb_status_string(99)
    assert lib.eplb_status_string(16) != lib.eplb_status_string(99)


FAKE = 0x1000   # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("E,P,G,N,RK,X", [
    (16, 24, 4, 2, 8, 5), (15, 24, 4, 2, 8, 5), (16, 24, 4, 2, 7, 5), (16, 25, 4, 2, 8, 5),
    (16, 8, 4, 2, 8, 5), (16, 24, 4, 2, 8, 4), (15, 24, 3, 2, 8, 10), (15, 24, 3, 2, 8, 9),
    (0, 24, 4, 2, 8, 3), (16, 24, 0, 2, 8, 5), (16, 24, 4, 2, 8, 0), (256, 288, 8, 4, 32, 9),
    (256, 320, 8, 5, 40, 65), (12, 16, 4, 2, 8, 2), (12, 16, 4, 2, 8, 3),
])
def test_rebalance_validation_matches_oracle_rules(lib, E, P, G, N, RK, X):
    """The library's argument rules are the pages' (as the oracle states them)."""
    want = {None: 0, "arg": 1, "div": 2, "redundancy": 3, "capacity": 4}[ora.argument_error(E, P, G, N, RK, X)]
    got = lib.eplb_rebalance_lds_bytes(E, P, G, N, RK, X)
    if want == 0:
        assert got > 0
    else:
        assert got == -want
        assert lib.eplb_rebalance(FAKE, 1, E, P, G, N, RK, X, FAKE, FAKE, FAKE, FAKE, None) == want


def test_rebalance_limits_and_nulls(lib):
    assert lib.eplb_rebalance(FAKE, -1, 16, 24, 4, 2, 8, 5, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.eplb_rebalance(None, 1, 16, 24, 4, 2, 8, 5, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.eplb_rebalance(FAKE, 1, 16, 24, 4, 2, 8, 5, FAKE, FAKE, FAKE, None, None) == 1
    assert lib.eplb_rebalance(FAKE, 1, 8192, 8192, 1, 1, 1, 1, FAKE, FAKE, FAKE, FAKE, None) == 5
    assert lib.eplb_rebalance_lds_bytes(4096, 8192, 1, 1, 8, 4097) == -5        # LDS budget
    assert lib.eplb_rebalance_lds_bytes(1024, 1024, 1, 1, 8, 1) == -5          # 1024 experts on one node
    assert lib.eplb_rebalance_lds_bytes(512, 512, 1, 1, 8, 1) > 0               # 512 fit
    assert lib.eplb_rebalance_lds_bytes(1024, 1024, 2, 2, 8, 1) > 0             # 512 per node
    # up to 160 KiB (the LDS of one gfx950 compute unit), not beyond
    assert 64 * 1024 < lib.eplb_rebalance_lds_bytes(2560, 3072, 8, 8, 64, 65) <= 160 * 1024
    assert lib.eplb_rebalance_lds_bytes(3072, 4096, 8, 8, 64, 129) == -5
    # the documented workloads fit
    for args in [(16, 24, 4, 2, 8, 5), (256, 288, 8, 4, 32, 9), (256, 320, 8, 5, 40, 65),
                 (512, 640, 16, 8, 64, 17), (256, 288, 8, 18, 144, 33), (60, 1830, 1, 1, 10, 1771)]:
        assert 0 < lib.eplb_rebalance_lds_bytes(*args) <= 64 * 1024, args


def test_gpu_test_shapes_fit(lib):
    """Every placement shape the GPU parity tests use passes host validation."""
    import ast
    src = open(os.path.join(ROOT, "tests", "test_gpu_parity.py")).read()
    block = src[src.index("@pytest.mark.parametrize(\"shape\", [") + len("@pytest.mark.parametrize(\"shape\", "):]
    block = block[:block.index("])") + 1]
    for E, G, N, RK, P in ast.literal_eval(block):
        X = 1 + (P - E) // (N if G % N == 0 else 1)
        assert lib.eplb_rebalance_lds_bytes(E, P, G, N, RK, X) > 0, (E, G, N, RK, P)


def test_stream_validation(lib):
    ok = dict(idx=FAKE, L=2, T=10, K=8, E=256)
    # hist: bad sizes, null buffers, id count per layer >= 2^31
    assert lib.eplb_load_hist(FAKE, -1, 10, 8, 256, FAKE, 4, 0, FAKE, FAKE, None) == 1
    assert lib.eplb_load_hist(FAKE, 2, 10, 0, 256, FAKE, 4, 0, FAKE, FAKE, None) == 1
    assert lib.eplb_load_hist(FAKE, 2, 10, 8, 0, FAKE, 4, 0, FAKE, FAKE, None) == 1
    assert lib.eplb_load_hist(FAKE, 2, 10, 8, 256, FAKE, 0, 0, FAKE, FAKE, None) == 1
    assert lib.eplb_load_hist(FAKE, 2, 10, 8, 256, FAKE, 4, -1, FAKE, FAKE, None) == 1
    assert lib.eplb_load_hist(None, 2, 10, 8, 256, FAKE, 4, 0, FAKE, FAKE, None) == 1
    assert lib.eplb_load_hist(FAKE, 2, 10, 8, 256, None, 4, 0, FAKE, FAKE, None) == 1
    assert lib.eplb_load_hist(FAKE, 2, 10, 8, 4097, FAKE, 4, 0, FAKE, FAKE, None) == 5
    assert lib.eplb_load_hist(FAKE, 2, 1 << 28, 8, 256, FAKE, 4, 0, FAKE, FAKE, None) == 6
    # redirect
    assert lib.eplb_redirect(FAKE, 2, 10, 8, 256, FAKE, FAKE, 0, FAKE, None) == 1
    assert lib.eplb_redirect(FAKE, 2, 10, 8, 256, FAKE, FAKE, 70000, FAKE, None) == 5
    assert lib.eplb_redirect(FAKE, 2, 10, 8, 256, None, FAKE, 9, FAKE, None) == 1
    assert lib.eplb_redirect(FAKE, 2, 10, 8, 256, FAKE, FAKE, 9, FAKE, None) == 1     # out == idx
    assert lib.eplb_redirect(FAKE, 2, (1 << 31) // 8, 8, 256, FAKE, FAKE, 9, FAKE + 64, None) == 6
    # fused: the union of both calls' rules
    hr = lambda *a: lib.eplb_hist_redirect(*a)
    good = [FAKE, 2, 10, 8, 256, FAKE, 4, 0, FAKE, FAKE, FAKE, FAKE, 9, FAKE + 64, None]
    for pos, bad, code in [(1, -1, 1), (3, 0, 1), (4, 0, 1), (6, 0, 1), (7, -1, 1), (12, 0, 1), (12, 70000, 5),
                           (4, 4097, 5), (2, 1 << 28, 6), (0, None, 1), (5, None, 1), (8, None, 1), (9, None, 1),
                           (10, None, 1), (11, None, 1), (13, None, 1), (13, FAKE, 1)]:
        args = list(good)
        args[pos] = bad
        assert hr(*args) == code, (pos, bad)
    assert ok


def test_ema_and_quality_validation(lib):
    good = [FAKE, 2, 10, 8, 256, FAKE, 4, FAKE, FAKE, None]
    for pos, bad, code in [(1, -1, 1), (3, 0, 1), (4, 0, 1), (4, 4097, 5), (2, 1 << 28, 6), (6, -1, 1),
                           (6, 63, 1), (0, None, 1), (5, None, 1), (7, None, 1), (8, None, 1)]:
        args = list(good)
        args[pos] = bad
        assert lib.eplb_load_ema(*args) == code, (pos, bad)
    assert lib.eplb_load_ema(None, 0, 10, 8, 256, None, 62, None, None, None) == 0   # L = 0: nothing to do
    good = [FAKE, FAKE, FAKE, 58, 256, 288, 32, FAKE, FAKE, None]
    for pos, bad, code in [(3, -1, 1), (3, (1 << 22) + 1, 5), (4, 0, 1), (4, 4097, 5), (5, 0, 1), (6, 0, 1),
                           (6, 5, 2), (0, None, 1), (1, None, 1), (2, None, 1), (7, None, 1), (8, None, 1),
                           (7, FAKE + 8, 1), (8, FAKE + 58 * 32 * 8 - 8, 1)]:
        args = list(good)
        args[pos] = bad
        assert lib.eplb_placement_load(*args) == code, (pos, bad)
    assert lib.eplb_placement_load(None, None, None, 0, 256, 288, 32, None, None, None) == 0


def test_fastdiv_magic_numbers():
    """The exact-division magic used for t mod c and t / K: for every divisor
    up to 2^16 and dividends near the 31-bit edge and near multiples of the
    divisor, floor(n/d) == (n * m >> 32) >> (l - 1), m = floor(2^(31+l)/d) + 1,
    l = ceil(log2 d) (Granlund & Montgomery 1994, Thm 4.2, N = 31)."""
    rng = np.random.default_rng(3)
    top = (1 << 31) - 1
    for d in range(2, 1 << 16):
        l = (d - 1).bit_length()
        m = (1 << (31 + l)) // d + 1
        assert m < (1 << 32)
        k = top // d
        ns = [0, 1, d - 1, d, d + 1, top, top - 1, k * d, k * d - 1, (k - 1) * d - 1]
        ns += [int(x) for x in rng.integers(0, top, 4)]
        for n in ns:
            assert ((n * m) >> 32) >> (l - 1) == n // d, (d, n)


def test_rearrange_validation(lib):
    F = [FAKE + 64 * i for i in range(8)]
    good = [F[0], F[1], F[2], 58, 256, 288, 32, 4, 9, F[3], F[4], F[5], F[6], F[7], None]
    for pos, bad, code in [(3, -1, 1), (4, 0, 1), (5, 0, 1), (6, 0, 1), (7, 0, 1), (8, 0, 1),
                           (6, 5, 2), (7, 5, 2), (4, 4097, 5), (5, 8192 * 2, 5), (8, 70000, 5),
                           (0, None, 1), (1, None, 1), (2, None, 1), (9, None, 1), (13, None, 1),
                           (9, F[1], 1), (10, F[2], 1), (12, F[0], 1)]:
        args = list(good)
        args[pos] = bad
        if pos == 5 and bad == 8192 * 2:
            args[6] = 32                                # keep P % RK == 0
        assert lib.eplb_rearrange(*args) == code, (pos, bad)
    assert lib.eplb_rearrange(None, None, None, 0, 256, 288, 32, 4, 9, None, None, None, None, None, None) == 0


def test_lp_solve_validation(lib):
    F = [FAKE + 64 * i for i in range(8)]
    good = [F[0], F[1], F[2], 58, 256, 8, 2, F[3], F[4], F[5], F[6], None]
    for pos, bad, code in [(3, -1, 1), (4, 0, 1), (5, 0, 1), (6, 0, 1), (4, 4097, 5), (5, 65, 5), (6, 65, 5),
                           (0, None, 1), (1, None, 1), (2, None, 1), (7, None, 1), (8, None, 1), (9, None, 1),
                           (10, None, 1), (9, F[0], 1), (7, F[2], 1)]:         # outputs equal to inputs
        args = list(good)
        args[pos] = bad
        assert lib.eplb_lp_solve(*args) == code, (pos, bad)
    assert lib.eplb_lp_solve(None, None, None, 0, 256, 8, 2, None, None, None, None, None) == 0


def test_lp_redirect_validation(lib):
    F = [FAKE + 64 * i for i in range(8)]
    need = lib.eplb_lp_redirect_workspace_bytes(58, 16384, 8, 256)
    assert need == 58 * 64 * 256 * 4
    assert lib.eplb_lp_redirect_workspace_bytes(58, 1 << 28, 8, 256) == -6
    assert lib.eplb_lp_redirect_workspace_bytes(-1, 10, 8, 256) == -1
    good = [F[0], 58, 16384, 8, 256, F[1], F[2], 8, 2, F[3], need, F[4], None]
    for pos, bad, code in [(1, -1, 1), (3, 0, 1), (4, 0, 1), (4, 4097, 5), (2, 1 << 28, 6), (7, 0, 1), (8, 0, 1),
                           (7, 65, 5), (8, 65, 5), (0, None, 1), (5, None, 1), (6, None, 1), (9, None, 1),
                           (11, None, 1), (11, F[0], 1), (10, need - 1, 1)]:
        args = list(good)
        args[pos] = bad
        assert lib.eplb_lp_redirect(*args) == code, (pos, bad)
    assert lib.eplb_lp_redirect(None, 0, 16384, 8, 256, None, None, 8, 2, None, 0, None, None) == 0


def _cc(src, out, extra=(), libs=()):
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lib_dir = os.path.dirname(LIB)
    cmd = [cc, *extra, "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), src,
           "-L", lib_dir, "-leplb", f"-Wl,-rpath,{lib_dir}", *libs, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def test_header_is_c99_and_every_entry_point_links(tmp_path):
    """The boundary from plain C: eplb.h compiles under ISO C99 -pedantic,
    every declared function links against libeplb.so, and the host-only
    calls answer (no GPU touched)."""
    import subprocess
    exe = _cc(os.path.join(ROOT, "tests", "c", "abi_host.c"), str(tmp_path / "abi_host"), ("-std=c99", "-pedantic"))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "abi_host ok: 15 entry points" in r.stdout
    assert len(declared_functions()) == 15


def test_ema_redirect_validation(lib):
    F = [FAKE + 64 * i for i in range(8)]
    good = [F[0], 2, 10, 8, 256, F[1], 4, F[2], F[3], F[4], F[5], 9, F[6], None]
    for pos, bad, code in [(1, -1, 1), (3, 0, 1), (4, 0, 1), (4, 4097, 5), (2, 1 << 28, 6), (6, -1, 1), (6, 63, 1),
                           (11, 0, 1), (11, 70000, 5), (0, None, 1), (5, None, 1), (7, None, 1), (8, None, 1),
                           (9, None, 1), (10, None, 1), (12, None, 1), (12, F[0], 1)]:
        args = list(good)
        args[pos] = bad
        assert lib.eplb_ema_redirect(*args) == code, (pos, bad)


@pytest.mark.parametrize("seed", range(4))
def test_max_count_matches_oracle(lib, seed):
    """eplb_rebalance_max_count is the oracle's capacity bound on random
    shapes of both policies, and the least X eplb_rebalance accepts."""
    rng = np.random.default_rng(seed)
    for _ in range(200):
        N = int(rng.integers(1, 9))
        G = int(rng.integers(1, 17))
        E = G * int(rng.integers(1, 9)) if rng.random() < 0.8 else int(rng.integers(1, 100))
        P = E + int(rng.integers(-3, 200))
        Np = ora.policy(G, N)[1]
        if P < 1 or P % Np:
            continue                                   # (the GPU count rules are not this call's)
        RK = Np
        err = ora.argument_error(E, P, G, N, RK, 1 << 20)
        got = lib.eplb_rebalance_max_count(E, P, G, N)
        if err is not None:
            assert got == -{"arg": 1, "div": 2, "redundancy": 3}[err], (E, P, G, N)
            continue
        want = ora.max_count(E, P, G, N)
        assert got == want, (E, P, G, N)
        if want > 1 and lib.eplb_rebalance_lds_bytes(E, P, G, N, RK, want) > 0:
            assert lib.eplb_rebalance_lds_bytes(E, P, G, N, RK, want - 1) == -4
    assert lib.eplb_rebalance_max_count(0, 24, 4, 2) == -1


def test_launch_size_limits(lib):
    """Calls that would launch 2^32 work-items or more are refused on the
    host, before any kernel (and before a window or moving average is
    touched)."""
    big = (1 << 22) + 1
    assert lib.eplb_load_hist(FAKE, big, 1, 1, 8, FAKE, 2, 0, FAKE + 64, FAKE + 128, None) == 5
    assert lib.eplb_redirect(FAKE, big, 1, 1, 8, FAKE + 64, FAKE + 128, 2, FAKE << 30, None) == 5
    assert lib.eplb_hist_redirect(FAKE, big, 1, 1, 8, FAKE, 2, 0, FAKE, FAKE, FAKE, FAKE, 2, FAKE << 20, None) == 5
    assert lib.eplb_load_ema(FAKE, big, 1, 1, 8, FAKE, 2, FAKE, FAKE, None) == 5
    assert lib.eplb_ema_redirect(FAKE, big, 1, 1, 8, FAKE, 2, FAKE, FAKE, FAKE, FAKE, 2, FAKE << 20, None) == 5
    F = [FAKE << (4 * i + 4) for i in range(8)]
    assert lib.eplb_rebalance(F[0], big, 16, 24, 4, 2, 8, 5, F[1], F[2], F[3], F[4], None) == 5
    assert lib.eplb_rearrange(F[0], F[1], F[2], big, 16, 24, 8, 2, 5, F[3], F[4], F[5], F[6], F[7], None) == 5
    assert lib.eplb_lp_solve(F[0], F[1], F[2], 1 << 20, 16, 8, 2, F[3], F[4], F[5], F[6], None) == 5
    # 2^25 segments of 2048 ids: the most one redirect by flows takes
    assert lib.eplb_lp_redirect(F[0], 1 << 14, 2048 * 2048 + 1, 1, 8, F[1], F[2], 8, 2, F[3], 1 << 62, F[4],
                                None) == 5


def test_overlapping_buffers_rejected(lib):
    """An output that shares any byte with an input (not only the same
    pointer) is refused."""
    n = 2 * 10 * 8 * 4
    assert lib.eplb_redirect(FAKE, 2, 10, 8, 256, FAKE << 8, FAKE << 9, 9, FAKE + n - 4, None) == 1
    assert lib.eplb_redirect(FAKE + 4, 2, 10, 8, 256, FAKE << 8, FAKE << 9, 9, FAKE + 4 - n + 4, None) == 1
    F = [FAKE << (4 * i + 4) for i in range(8)]
    # rebalance: status inside log2phy
    assert lib.eplb_rebalance(F[0], 2, 16, 24, 4, 2, 8, 5, F[1], F[2], F[3], F[2] + 8, None) == 1
    # lp_solve: flow overlapping rep
    assert lib.eplb_lp_solve(F[0], F[1], F[2], 2, 16, 8, 2, F[3], F[2] + 4, F[5], F[6], None) == 1
    # lp_redirect: workspace inside out; out over flow
    need = lib.eplb_lp_redirect_workspace_bytes(2, 5000, 2, 64)
    assert lib.eplb_lp_redirect(F[0], 2, 5000, 2, 64, F[1], F[2], 8, 2, F[4] + 16, need, F[4], None) == 1
    assert lib.eplb_lp_redirect(F[0], 2, 5000, 2, 64, F[1], F[2], 8, 2, F[3], need, F[2] + 8, None) == 1
    # streaming calls: in/out buffers (ring, ema), loads, counters and tables
    L, T, K, E, W, X = 2, 10, 8, 256, 4, 9
    ring_b, load_b = W * L * E * 4, L * E * 8
    assert lib.eplb_load_hist(F[0], L, T, K, E, F[1], W, 0, F[1] + ring_b - 8, F[3], None) == 1   # load in ring
    assert lib.eplb_load_hist(F[0], L, T, K, E, F[1], W, 0, F[2], F[2] + load_b - 8, None) == 1  # n_invalid in load
    assert lib.eplb_load_hist(F[0], L, T, K, E, F[0] + 4, W, 0, F[2], F[3], None) == 1          # ring over idx
    # a ring whose byte count (2^31 - 1 steps x 2^22 layers x 4096 experts x 4 B)
    # does not fit in 63 bits still holds the load placed 2^60 bytes into it
    assert lib.eplb_load_hist(FAKE << 4, 1 << 22, 1, 1, 4096, 1 << 44, (1 << 31) - 1, 0, (1 << 44) + (1 << 60),
                              1 << 36, None) == 1
    assert lib.eplb_redirect(F[0], L, T, K, E, F[1], F[2], X, F[1] + L * E * X * 4 - 4, None) == 1  # out over log2phy
    assert lib.eplb_redirect(F[0], L, T, K, E, F[1], F[2], X, F[2] - 4, None) == 1                # out over logcnt
    good = [F[0], L, T, K, E, F[1], W, 0, F[2], F[3], F[4], F[5], X, F[6], None]
    for pos, bad in [(8, F[1] + 8), (9, F[2]), (13, F[4]), (13, F[5] + 4), (5, F[6]), (9, F[0])]:
        args = list(good)
        args[pos] = bad
        assert lib.eplb_hist_redirect(*args) == 1, (pos, bad)
    assert lib.eplb_load_ema(F[0], L, T, K, E, F[1], 4, F[1] + 16, F[3], None) == 1                # ema over count
    assert lib.eplb_ema_redirect(F[0], L, T, K, E, F[1], 4, F[2], F[3], F[4], F[5], X, F[2] + 8, None) == 1


def test_lp_redirect_noalloc_validation(lib):
    """The no-allocation redirect applies eplb_lp_redirect's rules and refuses
    inputs whose counts need more than its fixed array, before any GPU call."""
    f = lib.eplb_lp_redirect_noalloc
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    F = [FAKE << (4 * i + 4) for i in range(6)]
    limit = header_constants().get("EPLB_NOALLOC_SCRATCH_BYTES")
    assert limit is None                                  # a parenthesised expression, checked below
    assert "#define EPLB_NOALLOC_SCRATCH_BYTES (4 * 1024 * 1024)" in open(HEADER).read()
    good = [F[0], 58, 16384, 8, 256, F[1], F[2], 16, 4, F[3], None]
    for pos, bad, code in [(1, -1, 1), (3, 0, 1), (4, 0, 1), (4, 4097, 5), (2, 1 << 28, 6), (7, 0, 1), (8, 0, 1),
                           (7, 65, 5), (8, 65, 5), (0, None, 1), (5, None, 1), (6, None, 1), (9, None, 1),
                           (9, F[0] + 64, 1)]:
        args = list(good)
        args[pos] = bad
        assert f(*args) == code, (pos, bad)
    # 58 x 64 segments x 64 counts = 950,272 bytes fit; 4x the tokens do not
    big = list(good)
    big[2] = 16384 * 5
    assert f(*big) == 5
    assert f(None, 0, 16384, 8, 256, None, None, 16, 4, None, None) == 0      # nothing to do
