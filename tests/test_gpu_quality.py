"""Moving-average load estimate and placement quality: HIP path vs the CPU
oracle, through the C ABI (needs an MI355X).

The moving average is integer work and is compared bit for bit.  Rank loads
are double precision on the device and exact rationals in the oracle; the
bound the arithmetic gives is checked exactly (in rationals): a rank load of
P/RK terms is within (P/RK + 1) units of 2^-53 of the exact value, the
max / mean ratio within (P/RK + 3).
"""
from __future__ import annotations

import sys
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle_pins
import workloads as wl
from oracle import eplb_oracle as ora

pytestmark = pytest.mark.gpu

eplb = pytest.importorskip("moe_expert_load_eplb_amd")
DEV = torch.device("cuda:0")
U = Fraction(1, 1 << 53)


def note(msg: str) -> None:
    print(f"[quality] {msg}", flush=True)
    sys.stdout.flush()


def gpu(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def host(t):
    return t.cpu().numpy()


def assert_same(name, got, want):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, f"{name}: shape {got.shape} vs {want.shape}"
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{name}: {len(bad)} mismatches, first at {i}: got {got[i]} want {want[i]}")


def within(got: float, exact: Fraction, units: int) -> bool:
    if exact == 0:
        return got == 0.0
    return abs(Fraction(got) - exact) <= units * U * exact


def check_quality(load, phy2log, logcnt, RK, rows=None):
    """GPU placement_load on all rows; every row in `rows` (default: all)
    checked against the oracle within the stated bound, NaN where the
    oracle has no result."""
    load = np.asarray(load, dtype=np.int64)
    B, E = load.shape
    P = phy2log.shape[1]
    ppr = P // RK
    note(f"placement_load B={B} E={E} P={P} RK={RK}")
    rank_d, imb_d = eplb.placement_load(gpu(load), gpu(phy2log), gpu(logcnt), RK)
    torch.cuda.synchronize()
    rank_h, imb_h = host(rank_d), host(imb_d)
    rows = list(range(B)) if rows is None else list(rows)
    ranks, imb = ora.placement_load(load[rows], phy2log[rows], logcnt[rows], RK)
    for i, b in enumerate(rows):
        if ranks[i] is None:
            assert np.isnan(rank_h[b]).all() and np.isnan(imb_h[b]), f"row {b}: expected NaN"
            continue
        for r in range(RK):
            assert within(float(rank_h[b, r]), ranks[i][r], ppr + 1), \
                f"row {b} rank {r}: {rank_h[b, r]!r} vs {float(ranks[i][r])!r}"
        assert within(float(imb_h[b]), imb[i], ppr + 3), f"row {b} imbalance {imb_h[b]!r} vs {float(imb[i])!r}"
    return rank_h, imb_h


# ---------------------------------------------------------------- placement quality

def test_quality_worked_example():
    """GPU loads of the pages' example: 86.5 .. 156 (hierarchical) and
    95.5 .. 138.5 with three groups (global)."""
    g = oracle_pins.GOLDEN
    w = np.array(g["inputs"]["weight"], dtype=np.int64)
    for groups, X, key in ((4, 3, "layer0_gpu_load_hierarchical"), (3, 5, "layer0_gpu_load_global_groups3")):
        phy2log, _, logcnt, status = (host(t) for t in eplb.rebalance(gpu(w), 16, groups, 2, 8, X))
        assert (status == 0).all()
        rank_h, imb_h = check_quality(w, phy2log, logcnt, 8)
        assert rank_h[0].min() == float(Fraction(g[key]["min"])) and rank_h[0].max() == float(Fraction(g[key]["max"]))
        assert np.isclose(rank_h.sum(axis=1), w.sum(axis=1), rtol=1e-15).all()


@pytest.mark.parametrize("case", ["dsv3", "global", "decode144", "skewed"])
def test_quality_after_rebalance(case):
    if case == "skewed":
        pl = wl.SKEWED_1024.placement
        load = wl.skewed_loads()
        rows = list(range(0, load.shape[0], 37)) + [1023]
    else:
        pl = {"dsv3": wl.DSV3_PREFILL.placement, "global": wl.GLOBAL_DECODE.placement,
              "decode144": wl.DSV3_DECODE_144}[case]
        load = wl.zipf_loads(58, pl.E, 1.1, 1 << 20)
        rows = None
    phy2log, _, logcnt, status = (host(t) for t in eplb.rebalance(gpu(load), pl.P, pl.G, pl.N, pl.RK))
    assert (status == 0).all()
    _, imb_h = check_quality(load, phy2log, logcnt, pl.RK, rows)
    assert (imb_h >= 1.0 - 1e-12).all()


def test_quality_of_old_placement_under_new_load():
    """The use that decides whether to rebalance: yesterday's placement
    judged by today's loads, next to today's placement."""
    pl = wl.DSV3_PREFILL.placement
    old = wl.zipf_loads(58, pl.E, 1.1, 1 << 20, wid=11)
    new = wl.zipf_loads(58, pl.E, 1.1, 1 << 20, wid=12)
    p_old, _, c_old, _ = (host(t) for t in eplb.rebalance(gpu(old), pl.P, pl.G, pl.N, pl.RK))
    p_new, _, c_new, _ = (host(t) for t in eplb.rebalance(gpu(new), pl.P, pl.G, pl.N, pl.RK))
    _, imb_stale = check_quality(new, p_old, c_old, pl.RK)
    _, imb_fresh = check_quality(new, p_new, c_new, pl.RK)
    assert imb_fresh.mean() < imb_stale.mean()


def test_quality_edge_cases():
    rng = np.random.default_rng(5)
    # one rank holds everything: its load is the total, max / mean = 1
    E, P = 12, 16
    load = rng.integers(0, 1000, size=(3, E)).astype(np.int64)
    phy2log, _, logcnt, _ = (host(t) for t in eplb.rebalance(gpu(load), P, 1, 1, 1))
    _, imb = check_quality(load, phy2log, logcnt, 1)
    assert (imb == 1.0).all()
    # one slot per rank, several ranks per lane (RK > 64), ragged against 64
    E, P = 150, 200
    load = rng.integers(0, 1 << 40, size=(5, E), endpoint=True).astype(np.int64)
    phy2log, _, logcnt, _ = (host(t) for t in eplb.rebalance(gpu(load), P, 1, 1, 200))
    check_quality(load, phy2log, logcnt, 200)
    # arbitrary maps: invalid entries, counts that do not match phy2log, zero loads
    B, E, P, RK = 9, 40, 96, 12
    load = rng.integers(0, 5000, size=(B, E)).astype(np.int64)
    phy2log = rng.integers(0, E, size=(B, P)).astype(np.int32)
    logcnt = rng.integers(1, 7, size=(B, E)).astype(np.int32)
    load[0] = 0                                  # all zero: ratio 1
    phy2log[1, 7] = E                            # out of range
    phy2log[2, 95] = -1
    logcnt[3, phy2log[3, 0]] = 0                 # a referenced count of 0
    unused = sorted(set(range(E)) - set(phy2log[4].tolist()))
    if unused:
        logcnt[4, unused[0]] = 0                 # an unreferenced count of 0 is harmless
    load[5, 3] = -1
    load[6, 3] = (1 << 40) + 1
    load[7, 3] = 1 << 40                         # the largest accepted load
    _, imb = check_quality(load, phy2log, logcnt, RK)
    assert imb[0] == 1.0 and np.isnan(imb[[1, 2, 3, 5, 6]]).all() and not np.isnan(imb[[4, 7, 8]]).any()
    # no problems
    r, i = eplb.placement_load(torch.zeros((0, E), dtype=torch.int64, device=DEV),
                               torch.zeros((0, P), dtype=torch.int32, device=DEV),
                               torch.zeros((0, E), dtype=torch.int32, device=DEV), RK)
    assert r.shape == (0, RK) and i.shape == (0,)


# ---------------------------------------------------------------- moving average

def _ema_chain(work, steps_h, shift, ema0=None):
    pl = work.placement
    L, E = work.layers, pl.E
    ema_ref = np.zeros((L, E), dtype=np.int64) if ema0 is None else ema0.copy()
    ema = gpu(ema_ref)
    for s, idx_h in enumerate(steps_h):
        note(f"ema {work.name} shift {shift} step {s}")
        _, cnt, bad = eplb.load_ema(gpu(idx_h), E, ema, shift)
        torch.cuda.synchronize()
        c, invl = ora.load_hist(idx_h, E)
        ema_ref = ora.ema_update(ema_ref, c, shift).reshape(L, E)
        assert_same(f"step {s} counts", host(cnt).astype(np.int64), c)
        assert_same(f"step {s} invalid", host(bad), invl)
        assert_same(f"step {s} ema", host(ema), ema_ref)
    return host(ema), ema_ref


@pytest.mark.parametrize("shift", [0, 1, 3, 7])
def test_ema_tiny_with_invalid_ids(shift):
    work = wl.TINY_HIER
    steps = [wl.routing_step(work, s) for s in range(5)]
    rng = np.random.default_rng(shift)
    for idx_h in steps[1:3]:
        m = rng.random(idx_h.shape) < 0.01
        idx_h[m] = rng.choice(np.array([-1, -7, work.placement.E, 1 << 30], dtype=np.int32), size=int(m.sum()))
    _ema_chain(work, steps, shift)


def test_ema_dsv3_feeds_rebalance():
    """Ten DeepSeek-V3 prefill steps into the moving average (shift 3, from a
    nonzero start), then the rebalance of the estimate: bit-exact."""
    work = wl.DSV3_PREFILL
    pl = work.placement
    steps = [wl.routing_step(work, s) for s in range(work.window)]
    ema0 = np.random.default_rng(3).integers(0, 1 << 20, size=(work.layers, pl.E)).astype(np.int64)
    ema_h, ema_ref = _ema_chain(work, steps, 3, ema0)
    outs = [host(t) for t in eplb.rebalance(gpu(ema_h), pl.P, pl.G, pl.N, pl.RK)]
    ref = ora.rebalance(ema_ref, pl.P, pl.G, pl.N, pl.RK, ora.max_count(pl.E, pl.P, pl.G, pl.N))
    for name, g in zip(("phy2log", "log2phy", "logcnt", "status"), outs):
        assert_same(name, g, ref[name])


def test_ema_ragged_and_large():
    """Layers off 16-byte boundaries, E = 1 and 4096, negative and large
    starting values (floor of a negative value rounds down)."""
    rng = np.random.default_rng(8)
    for (L, T, K, E, shift) in ((3, 20001, 3, 16, 2), (2, 7, 1, 1, 0), (1, 33333, 2, 4096, 9), (4, 1, 3, 3, 62)):
        note(f"ema ragged L={L} T={T} K={K} E={E} shift={shift}")
        idx_h = rng.integers(-2, E + 2, size=(L, T, K)).astype(np.int32)
        ema_ref = rng.integers(-(1 << 61), 1 << 61, size=(L, E)).astype(np.int64)
        ema = gpu(ema_ref)
        _, cnt, bad = eplb.load_ema(gpu(idx_h), E, ema, shift)
        torch.cuda.synchronize()
        c, invl = ora.load_hist(idx_h, E)
        assert_same("counts", host(cnt).astype(np.int64), c)
        assert_same("invalid", host(bad), invl)
        assert_same("ema", host(ema), ora.ema_update(ema_ref, c, shift).reshape(L, E))


def test_ema_full_size():
    """58 x 2^20 x 8 ids per step (the streaming workload), three steps,
    shift 4: whole histograms and estimates compared."""
    work = wl.STREAM_1M
    L, T, K, E = work.layers, work.tokens, work.topk, work.placement.E
    idx = torch.empty((L, T, K), dtype=torch.int32, device=DEV)
    ema = torch.zeros((L, E), dtype=torch.int64, device=DEV)
    ema_ref = np.zeros((L, E), dtype=np.int64)
    for s in range(3):
        note(f"ema full size step {s}")
        wl.routing_step_device(work, s, DEV, out=idx)
        _, cnt, bad = eplb.load_ema(idx, E, ema, 4)
        torch.cuda.synchronize()
        c, invl = ora.load_hist(host(idx), E)
        ema_ref = ora.ema_update(ema_ref, c, 4).reshape(L, E)
        assert_same(f"step {s} counts", host(cnt).astype(np.int64), c)
        assert int(host(bad).sum()) == 0 and int(invl.sum()) == 0
        assert_same(f"step {s} ema", host(ema), ema_ref)


# ---------------------------------------------------------------- moving average + redirect in one pass

@pytest.mark.parametrize("L,T,K,E,shift", [(3, 20001, 3, 16, 2), (2, 7, 1, 5, 0), (5, 4097, 8, 256, 4),
                                           (2, 70000, 5, 1, 7), (1, 33333, 2, 4096, 9)])
def test_ema_redirect_ragged(L, T, K, E, shift):
    """Counts, moving average, invalid ids and redirected ids of the fused
    pass against the oracle: ragged tails, several workgroups per layer,
    out-of-range ids and counts."""
    rng = np.random.default_rng(L * T + K + shift)
    idx_h = rng.integers(-3, E + 3, size=(L, T, K)).astype(np.int32)
    X = 4
    logcnt = rng.integers(-1, X + 2, size=(L, E)).astype(np.int32)
    log2phy = rng.integers(0, 1000, size=(L, E, X)).astype(np.int32)
    ema0 = rng.integers(0, 1 << 30, size=(L, E)).astype(np.int64)
    ema = gpu(ema0)
    note(f"ema_redirect L={L} T={T} K={K} E={E} shift={shift}")
    _, cnt, bad, out = eplb.ema_redirect(gpu(idx_h), E, ema, shift, gpu(log2phy), gpu(logcnt))
    torch.cuda.synchronize()
    c, invl = ora.load_hist(idx_h, E)
    assert_same("count", host(cnt).astype(np.int64), c)
    assert_same("invalid", host(bad), invl)
    assert_same("ema", host(ema), ora.ema_update(ema0, c, shift).reshape(L, E))
    assert_same("redirect", host(out), ora.redirect(idx_h, log2phy, logcnt))


def test_ema_redirect_full_size():
    """One step of the streaming workload (58 x 2^20 x 8 ids) with its
    placement: identical to eplb_load_ema followed by eplb_redirect, and to
    the oracle on every layer."""
    work = wl.STREAM_1M
    pl = work.placement
    L, E = work.layers, pl.E
    idx = wl.routing_step_device(work, 0, DEV)
    ema_a = torch.zeros((L, E), dtype=torch.int64, device=DEV)
    _, cnt_a, bad_a = eplb.load_ema(idx, E, ema_a, 4)
    placement = eplb.rebalance(ema_a, pl.P, pl.G, pl.N, pl.RK)
    out_a = eplb.redirect(idx, placement[1], placement[2])
    ema_b = torch.zeros((L, E), dtype=torch.int64, device=DEV)
    _, cnt_b, bad_b, out_b = eplb.ema_redirect(idx, E, ema_b, 4, placement[1], placement[2])
    torch.cuda.synchronize()
    for name, a, b in (("ema", ema_a, ema_b), ("count", cnt_a, cnt_b), ("invalid", bad_a, bad_b), ("out", out_a, out_b)):
        assert bool(torch.equal(a, b)), f"{name}: fused differs from the two separate calls"
    idx_h = host(idx)
    l2p_h, cnt_h, out_h = host(placement[1]), host(placement[2]), host(out_b)
    c, _ = ora.load_hist(idx_h, E)
    assert_same("counts", host(cnt_b).astype(np.int64), c)
    for l in range(L):
        assert_same(f"redirect layer {l}", out_h[l:l + 1],
                    ora.redirect(idx_h[l:l + 1], l2p_h[l:l + 1], cnt_h[l:l + 1]))
