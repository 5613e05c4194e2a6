"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

Integer work throughout, so every comparison is bit-exact.  Small and
mid-size inputs are compared element by element; the full-size streaming
workload (58 layers x 2^20 tokens x top-8) is compared on whole per-step
histograms, on sampled layers and positions of the redirect, and through
properties that hold at any size.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

import invariants as inv
import oracle_pins
import workloads as wl
from oracle import eplb_oracle as ora

pytestmark = pytest.mark.gpu

eplb = pytest.importorskip("moe_expert_load_eplb_amd")
DEV = torch.device("cuda:0")


def note(msg: str) -> None:
    print(f"[parity] {msg}", flush=True)
    sys.stdout.flush()


def gpu(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def host(t):
    return t.cpu().numpy()


def assert_same(name, got, want):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, f"{name}: shape {got.shape} vs {want.shape}"
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{name}: {len(bad)} mismatches, first at {i}: got {got[i]} want {want[i]}")


def rebalance_both(load, P, G, N, RK, X=None):
    load = np.asarray(load, dtype=np.int64)
    B, E = load.shape
    if X is None:
        X = eplb.max_count(E, P, G, N)
    note(f"rebalance B={B} E={E} P={P} G={G} N={N} RK={RK} X={X}")
    outs = eplb.rebalance(gpu(load), P, G, N, RK, X)
    torch.cuda.synchronize()
    got = [host(t) for t in outs]
    ref = ora.rebalance(load, P, G, N, RK, X)
    for name, g in zip(("phy2log", "log2phy", "logcnt", "status"), got):
        assert_same(name, g, ref[name])
    return got, ref


# ---------------------------------------------------------------- the pages' example

def test_worked_example_gpu():
    g = oracle_pins.GOLDEN
    w = np.array(g["inputs"]["weight"], dtype=np.int64)
    (phy2log, log2phy, logcnt, status), _ = rebalance_both(w, 16, 4, 2, 8, 3)
    assert phy2log.tolist() == g["phy2log"]["value"]
    assert logcnt[0].tolist() == g["layer0_logcnt"]["value"]
    assert log2phy[0, 0, :2].tolist() == g["layer0_log2phy"]["expert0"]
    assert log2phy[0, 1, :2].tolist() == g["layer0_log2phy"]["expert1"]
    assert (log2phy[:, :, 2] == -1).all()
    # global policy (num_groups = 3)
    rebalance_both(w, 16, 3, 2, 8, 5)


# ---------------------------------------------------------------- the five workloads

def _routing_steps(work, steps, tokens=None):
    return [wl.routing_step(work, s, tokens=tokens) for s in range(steps)]


def _hist_window_check(work, steps_h, ring_steps=None):
    """Run eplb_load_hist over the steps; compare each step's counts, the
    invalid counts and the window load with the oracle."""
    pl = work.placement
    L = work.layers
    W = work.window
    ring = torch.zeros((W, L, pl.E), dtype=torch.int32, device=DEV)
    hists = []
    for s, idx_h in enumerate(steps_h):
        note(f"hist {work.name} step {s}")
        load, bad = eplb.load_hist(gpu(idx_h), pl.E, ring, step=s)
        torch.cuda.synchronize()
        cnt, invl = ora.load_hist(idx_h, pl.E)
        hists.append(cnt)
        assert_same(f"step {s} counts", host(ring[s % W]).astype(np.int64), cnt)
        assert_same(f"step {s} invalid", host(bad), invl)
        assert_same(f"step {s} window", host(load), ora.window_load(hists, W))
    return host(load)


def test_tiny_hier_full_path():
    work = wl.TINY_HIER
    pl = work.placement
    steps = _routing_steps(work, 3)
    load = _hist_window_check(work, steps)
    (phy2log, log2phy, logcnt, status), ref = rebalance_both(load, pl.P, pl.G, pl.N, pl.RK)
    out = host(eplb.redirect(gpu(steps[-1]), gpu(log2phy), gpu(logcnt)))
    assert_same("redirect", out, ora.redirect(steps[-1], ref["log2phy"], ref["logcnt"]))


@pytest.fixture(scope="module")
def dsv3_steps():
    return _routing_steps(wl.DSV3_PREFILL, wl.DSV3_PREFILL.window)


def test_dsv3_prefill_full_path(dsv3_steps):
    work = wl.DSV3_PREFILL
    pl = work.placement
    load = _hist_window_check(work, dsv3_steps)
    (phy2log, log2phy, logcnt, status), ref = rebalance_both(load, pl.P, pl.G, pl.N, pl.RK)
    assert (status == 0).all()
    for b in range(0, work.layers, 7):
        inv.check_placement(load[b], phy2log[b], log2phy[b], logcnt[b], pl.E, pl.P, pl.G, pl.N, pl.RK)
    idx = dsv3_steps[-1]
    out = host(eplb.redirect(gpu(idx), gpu(log2phy), gpu(logcnt)))
    assert_same("redirect", out, ora.redirect(idx, ref["log2phy"], ref["logcnt"]))


def test_global_decode_full_path():
    work = wl.GLOBAL_DECODE
    pl = work.placement
    steps = _routing_steps(work, work.window)
    load = _hist_window_check(work, steps)
    (phy2log, log2phy, logcnt, status), ref = rebalance_both(load, pl.P, pl.G, pl.N, pl.RK)
    assert (status == 0).all()
    out = host(eplb.redirect(gpu(steps[-1]), gpu(log2phy), gpu(logcnt)))
    assert_same("redirect", out, ora.redirect(steps[-1], ref["log2phy"], ref["logcnt"]))


def test_skewed_1024_rebalance():
    work = wl.SKEWED_1024
    pl = work.placement
    load = wl.skewed_loads()
    X = pl.max_count
    note(f"rebalance skewed B={load.shape[0]}")
    outs = eplb.rebalance(gpu(load), pl.P, pl.G, pl.N, pl.RK, X)
    torch.cuda.synchronize()
    phy2log, log2phy, logcnt, status = (host(t) for t in outs)
    assert (status == 0).all()
    assert (logcnt.sum(axis=1) == pl.P).all() and (logcnt >= 1).all()
    sample = list(range(0, work.layers, 16)) + [1, 17, 1023]
    ref = ora.rebalance(load[sample], pl.P, pl.G, pl.N, pl.RK, X)
    for name, g in (("phy2log", phy2log), ("log2phy", log2phy), ("logcnt", logcnt), ("status", status)):
        assert_same(name, g[sample], ref[name])
    for b in sample[:8]:
        inv.check_placement(load[b], phy2log[b], log2phy[b], logcnt[b], pl.E, pl.P, pl.G, pl.N, pl.RK)


def test_stream_1m_full_size():
    """58 x 2^20 x 8 ids per step, 10-step window, C1-shaped placement,
    redirect of the last step: whole histograms compared per step; the
    redirect compared on sampled layers in full and by properties on all."""
    work = wl.STREAM_1M
    pl = work.placement
    L, T, K, E, W = work.layers, work.tokens, work.topk, pl.E, work.window
    idx = torch.empty((L, T, K), dtype=torch.int32, device=DEV)
    ring = torch.zeros((W, L, E), dtype=torch.int32, device=DEV)
    hists = []
    for s in range(W):
        note(f"stream step {s}: generate + hist")
        wl.routing_step_device(work, s, DEV, out=idx)
        load, bad = eplb.load_hist(idx, E, ring, step=s)
        torch.cuda.synchronize()
        # oracle counts of this step, from the same bytes
        idx_h = host(idx)
        cnt, invl = ora.load_hist(idx_h, E)
        hists.append(cnt)
        assert_same(f"step {s} counts", host(ring[s]).astype(np.int64), cnt)
        assert int(invl.sum()) == 0 and int(host(bad).sum()) == 0
    load_h = host(load)
    assert_same("window", load_h, ora.window_load(hists, W))
    (phy2log, log2phy, logcnt, status), ref = rebalance_both(load_h, pl.P, pl.G, pl.N, pl.RK)
    note("stream redirect")
    out = eplb.redirect(idx, gpu(log2phy), gpu(logcnt))
    torch.cuda.synchronize()
    # properties on every id: the replica serves the routed expert, and it is
    # replica (t mod logcnt) of it
    p2l = gpu(phy2log).long()
    cnt_t = gpu(logcnt).long()
    l2p = gpu(log2phy).long()
    for l in range(L):
        o = out[l].long()
        e = idx[l].long()
        assert bool((p2l[l][o] == e).all()), f"layer {l}: a redirected id serves another expert"
        t = torch.arange(T, device=DEV).unsqueeze(1)
        r = t % cnt_t[l][e]
        assert bool((l2p[l][e, r] == o).all()), f"layer {l}: replica is not t mod logcnt"
    # element-by-element on sampled layers
    out_h = host(out)
    for l in (0, 29, 57):
        assert_same(f"redirect layer {l}", out_h[l:l + 1],
                    ora.redirect(idx_h[l:l + 1], ref["log2phy"][l:l + 1], ref["logcnt"][l:l + 1]))


# ---------------------------------------------------------------- edge cases

def test_decode_144_global():
    pl = wl.DSV3_DECODE_144
    load = wl.zipf_loads(6, pl.E, 1.2, 1 << 18)
    rebalance_both(load, pl.P, pl.G, pl.N, pl.RK)


@pytest.mark.parametrize("shape", [
    (16, 4, 4, 8, 24),        # G == N: groups stay in place
    (16, 4, 2, 24, 24),       # one physical expert per GPU
    (16, 4, 2, 16, 16),       # no redundancy, one per GPU
    (64, 4, 1, 8, 80),        # one node, hierarchical with 4 groups
    (64, 1, 1, 4, 64),        # one group, no replicas
    (1, 1, 1, 1, 1),          # one expert
    (1, 1, 1, 3, 9),          # one expert, many replicas
    (24, 6, 4, 8, 32),        # global: 6 % 4 != 0
    (20, 5, 5, 10, 30),
    (18, 9, 3, 3, 27),
    (96, 12, 4, 16, 160),
    (200, 8, 2, 100, 400),    # 50 GPUs per node (>= 64 packs would need >1 pack per lane)
    (130, 2, 1, 130, 260),    # 130 packs: two packs per lane
    (64, 1, 1, 16, 64),       # 16 packs: the run-at-once packing, smallest case
    (51, 1, 1, 17, 68),       # 17 packs
    (100, 3, 2, 64, 256),     # global, 64 packs: runs can span the whole wave
    (300, 3, 1, 60, 600),     # global, 60 packs of 10
    (64, 32, 16, 32, 96),     # 32 groups onto 16 nodes: step 1 packs with runs
    (100, 5, 1, 12, 144),     # 12 packs of 12: register runs, three item chunks
    (45, 3, 1, 9, 90),        # 9 packs
    (40, 8, 4, 20, 60),       # 5 packs per node, 8 groups onto 4 nodes
    (100, 4, 1, 100, 300),    # 100 packs: runs over two registers of positions
    (90, 1, 1, 90, 180),
    (256, 8, 1, 200, 800),    # 200 packs of 4 over four registers
    (256, 1, 1, 256, 512),    # 256 packs: every pack index of the one-word form
])
def test_shapes_random(shape):
    E, G, N, RK, P = shape
    rng = np.random.default_rng(E * 1000 + P)
    load = rng.integers(0, 1000, size=(12, E)) * rng.integers(0, 2, size=(12, E))
    load[0] = 0
    load[1] = 7
    load[2] = rng.integers(0, 3, size=E)
    rebalance_both(load, P, G, N, RK)


def _fuzz_shapes(rng, count):
    """Valid placement shapes of every kind: hierarchical and global, 1 to 200
    GPUs per node (the sequential, register-run and LDS-run packing forms, one
    to four registers of packs), one to eight registers of experts per node."""
    shapes = []
    while len(shapes) < count:
        N = int(rng.choice([1, 1, 2, 3, 4, 5, 8]))
        hier = rng.random() < 0.6
        G = N * int(rng.integers(1, 5)) if hier else int(rng.choice([g for g in range(2, 13) if g % N]) if N > 1 else 1)
        if not hier and N == 1:
            hier = True
        Np = N if hier else 1
        S = int(rng.integers(1, 9))
        E = G * S if hier else int(rng.integers(2, 80))
        RKn = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 9, 12, 16, 17, 24, 33, 40, 64, 80, 130, 200]))
        RK = RKn * Np
        ppr = int(rng.integers(1, 6))
        P = RK * ppr
        if P < E or E > 512 or E // Np > 512 or RK > 512:
            continue
        if hier and E % G:
            continue
        shapes.append((E, G, N, RK, P))
    return shapes


def test_random_shapes_fuzz():
    """300 random valid shapes, 3 problems each (zero, tied, skewed and large
    loads), element by element against the oracle."""
    rng = np.random.default_rng(20251203)
    for E, G, N, RK, P in _fuzz_shapes(rng, 300):
        kind = rng.integers(0, 4)
        if kind == 0:
            load = rng.integers(0, 5, size=(3, E))
        elif kind == 1:
            load = rng.integers(0, 1 << 20, size=(3, E))
        elif kind == 2:
            load = (rng.zipf(1.3, size=(3, E)) * 1000).clip(0, 1 << 40)
        else:
            load = rng.integers((1 << 40) - 100, (1 << 40) + 1, size=(3, E))
        load[0, : E // 2] = 0
        rebalance_both(load.astype(np.int64), P, G, N, RK)


def test_large_loads_and_exactness():
    rng = np.random.default_rng(5)
    load = rng.integers((1 << 40) - 5000, (1 << 40) + 1, size=(16, 64))
    load[:, ::7] = rng.integers(0, 1 << 40, size=(16, 10))
    rebalance_both(load, 96, 8, 2, 16)
    rebalance_both(load, 96, 3, 2, 16, 33)
    # cases where float32 would tie but exact values differ
    for hi in (1 << 30, (1 << 40) - 4096):
        w = np.array([[hi - 64, hi - 32, 5, 3], [hi - 32, hi - 64, 3, 5]], dtype=np.int64)
        rebalance_both(w, 4, 1, 1, 2, 1)
    w = np.array([[(1 << 30) + 1, 3 * (1 << 30) + 4, 1, 1]], dtype=np.int64)
    rebalance_both(w, 6, 1, 1, 3, 3)


def test_status_cases():
    w = np.array([[1, 2, 3, 4], [1, -1, 3, 4], [1, 2, 3, (1 << 40) + 1], [1, 2, 3, 1 << 40]], dtype=np.int64)
    (_, _, _, status), _ = rebalance_both(w, 6, 2, 1, 2, 3)
    assert status.tolist() == [0, eplb.EPLB_S_BAD_LOAD, eplb.EPLB_S_BAD_LOAD, 0]
    E = 60
    P = E + sum(range(E))
    for V, want in (((1 << 40) // 60, eplb.EPLB_S_OVERFLOW), (1 << 30, 0)):
        w = np.array([[(i + 1) * V for i in range(E)]], dtype=np.int64)
        (_, _, logcnt, status), _ = rebalance_both(w, P, 1, 1, 10)
        assert status.tolist() == [want]
        if want == 0:
            assert logcnt[0].tolist() == list(range(1, E + 1))


def test_counts_with_large_prime_factors():
    """Replica counts 131, 137 (primes above the trial-division table) and
    mixes with small ones: the lcm of the counts is still exact.  Loads
    u_i = c_i * V make c_i the final counts (every pick is above V)."""
    V = 1 << 20
    for counts, RK in (([131, 5, 3, 1], 10), ([131, 137, 2], 10), ([262, 131, 1, 1, 1], 4)):
        E = len(counts)
        P = sum(counts)
        w = np.array([[c * V for c in counts]], dtype=np.int64)
        (_, _, logcnt, status), _ = rebalance_both(w, P, 1, 1, RK)
        assert logcnt[0].tolist() == counts and status.tolist() == [0]


def test_empty_inputs():
    E, P = 16, 24
    outs = eplb.rebalance(torch.zeros((0, E), dtype=torch.int64, device=DEV), P, 4, 2, 8, 5)
    assert all(t.shape[0] == 0 for t in outs)
    ring = torch.zeros((2, 3, E), dtype=torch.int32, device=DEV)
    ring[1] = 5
    load, bad = eplb.load_hist(torch.zeros((3, 0, 2), dtype=torch.int32, device=DEV), E, ring, step=0)
    torch.cuda.synchronize()
    assert (host(ring[0]) == 0).all() and (host(load) == 5).all() and (host(bad) == 0).all()
    out = eplb.redirect(torch.zeros((3, 0, 2), dtype=torch.int32, device=DEV),
                        torch.zeros((3, E, 2), dtype=torch.int32, device=DEV),
                        torch.ones((3, E), dtype=torch.int32, device=DEV))
    assert out.shape == (3, 0, 2)


@pytest.mark.parametrize("L,T,K,E", [(3, 20001, 3, 16), (2, 7, 1, 5), (5, 4097, 8, 256),
                                     (2, 70000, 5, 1), (1, 33333, 2, 4096), (4, 1, 3, 3)])
def test_hist_redirect_ragged(L, T, K, E):
    """Layers that start off 16-byte boundaries, ragged tails, several
    workgroups per layer, out-of-range ids, invalid counts."""
    rng = np.random.default_rng(L * T + K)
    idx_h = rng.integers(-3, E + 3, size=(L, T, K)).astype(np.int32)
    W = 3
    ring = torch.zeros((W, L, E), dtype=torch.int32, device=DEV)
    ring[2] = 1
    load, bad = eplb.load_hist(gpu(idx_h), E, ring, step=4)     # slot 1
    torch.cuda.synchronize()
    cnt, invl = ora.load_hist(idx_h, E)
    assert_same("counts", host(ring[1]).astype(np.int64), cnt)
    assert_same("invalid", host(bad), invl)
    assert_same("window", host(load), cnt + 1)
    X = 4
    logcnt = rng.integers(-1, X + 2, size=(L, E)).astype(np.int32)
    log2phy = rng.integers(0, 1000, size=(L, E, X)).astype(np.int32)
    out = host(eplb.redirect(gpu(idx_h), gpu(log2phy), gpu(logcnt)))
    assert_same("redirect", out, ora.redirect(idx_h, log2phy, logcnt))
    # an output buffer on a different 16-byte phase than the input
    big = torch.empty(L * T * K + 1, dtype=torch.int32, device=DEV)
    out2 = big[1:].view(L, T, K)
    idx_d, l2p_d, cnt_d = gpu(idx_h), gpu(log2phy), gpu(logcnt)     # kept alive across the launch
    rc = eplb.lib.eplb_redirect(idx_d.data_ptr(), L, T, K, E, l2p_d.data_ptr(), cnt_d.data_ptr(), X,
                                out2.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert_same("redirect misaligned out", host(out2), ora.redirect(idx_h, log2phy, logcnt))


def test_repeatable():
    load = wl.zipf_loads(58, 256, 1.1, 1 << 20)
    a = [host(t) for t in eplb.rebalance(gpu(load), 288, 8, 4, 32)]
    b = [host(t) for t in eplb.rebalance(gpu(load), 288, 8, 4, 32)]
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ---------------------------------------------------------------- fused statistics + redirect

@pytest.mark.parametrize("L,T,K,E", [(3, 20001, 3, 16), (2, 7, 1, 5), (5, 4097, 8, 256),
                                     (1, 33333, 2, 4096), (4, 1, 3, 3)])
def test_fused_ragged(L, T, K, E):
    """One pass gives the oracle's counts, window, invalid counts and
    redirect, on misaligned layers, ragged tails, invalid ids and counts."""
    rng = np.random.default_rng(L * T + K + 7)
    idx_h = rng.integers(-3, E + 3, size=(L, T, K)).astype(np.int32)
    X = 4
    logcnt = rng.integers(-1, X + 2, size=(L, E)).astype(np.int32)
    log2phy = rng.integers(0, 1000, size=(L, E, X)).astype(np.int32)
    W = 3
    ring = torch.zeros((W, L, E), dtype=torch.int32, device=DEV)
    ring[0] = 2
    note(f"hist_redirect L={L} T={T} K={K} E={E}")
    load, bad, out = eplb.hist_redirect(gpu(idx_h), E, ring, 7, gpu(log2phy), gpu(logcnt))   # slot 1
    torch.cuda.synchronize()
    cnt, invl = ora.load_hist(idx_h, E)
    assert_same("counts", host(ring[1]).astype(np.int64), cnt)
    assert_same("invalid", host(bad), invl)
    assert_same("window", host(load), cnt + 2)
    assert_same("redirect", host(out), ora.redirect(idx_h, log2phy, logcnt))
    # an output buffer on a different 16-byte phase than the input
    big = torch.empty(L * T * K + 1, dtype=torch.int32, device=DEV)
    out2 = big[1:].view(L, T, K)
    eplb.hist_redirect(gpu(idx_h), E, ring, 7, gpu(log2phy), gpu(logcnt), out=out2)
    torch.cuda.synchronize()
    assert_same("redirect misaligned out", host(out2), ora.redirect(idx_h, log2phy, logcnt))
    assert_same("counts again", host(ring[1]).astype(np.int64), cnt)


def test_stream_entries_fuzz():
    """40 random shapes through every streaming entry (histogram + window,
    redirect, fused histogram + redirect, moving average, fused moving
    average + redirect): ragged and empty layers, ids out of range, stale
    ring slots, odd window positions, against the oracle."""
    rng = np.random.default_rng(99)
    for case in range(40):
        L = int(rng.integers(1, 7))
        T = int(rng.choice([0, 1, 3, int(rng.integers(1, 6000))]))
        K = int(rng.integers(1, 10))
        E = int(rng.choice([1, 2, 7, 64, 256, int(rng.integers(1, 700))]))
        W = int(rng.integers(1, 6))
        step = int(rng.integers(0, 50))
        X = int(rng.integers(1, 6))
        shift = int(rng.integers(0, 8))
        note(f"stream fuzz {case}: L={L} T={T} K={K} E={E} W={W} step={step} X={X}")
        idx_h = rng.integers(-2, E + 2, size=(L, T, K)).astype(np.int32)
        logcnt = rng.integers(-1, X + 2, size=(L, E)).astype(np.int32)
        log2phy = rng.integers(0, 5000, size=(L, E, X)).astype(np.int32)
        ring_h = rng.integers(0, 1000, size=(W, L, E)).astype(np.int32)        # stale slots
        cnt, invl = ora.load_hist(idx_h, E)
        others = ring_h.astype(np.int64).sum(axis=0) - ring_h[step % W]
        idx_d, l2p_d, cnt_d = gpu(idx_h), gpu(log2phy), gpu(logcnt)
        ring = gpu(ring_h)
        load, bad = eplb.load_hist(idx_d, E, ring, step)
        torch.cuda.synchronize()
        assert_same("slot", host(ring[step % W]).astype(np.int64), cnt)
        assert_same("window", host(load), others + cnt)
        assert_same("invalid", host(bad), invl)
        want = ora.redirect(idx_h, log2phy, logcnt)
        assert_same("redirect", host(eplb.redirect(idx_d, l2p_d, cnt_d)), want)
        ring = gpu(ring_h)
        load, bad, out = eplb.hist_redirect(idx_d, E, ring, step, l2p_d, cnt_d)
        torch.cuda.synchronize()
        assert_same("fused window", host(load), others + cnt)
        assert_same("fused redirect", host(out), want)
        ema_h = rng.integers(-(1 << 40), 1 << 40, size=(L, E)).astype(np.int64)
        ema = gpu(ema_h)
        ema, count, bad = eplb.load_ema(idx_d, E, ema, shift)
        torch.cuda.synchronize()
        assert_same("ema", host(ema), ora.ema_update(ema_h, cnt, shift).reshape(L, E))
        assert_same("ema count", host(count).astype(np.int64), cnt)
        ema = gpu(ema_h)
        ema, count, bad, out = eplb.ema_redirect(idx_d, E, ema, shift, l2p_d, cnt_d)
        torch.cuda.synchronize()
        assert_same("fused ema", host(ema), ora.ema_update(ema_h, cnt, shift).reshape(L, E))
        assert_same("fused ema redirect", host(out), want)


@pytest.mark.parametrize("work", [wl.TINY_HIER, wl.DSV3_PREFILL], ids=lambda w: w.name)
def test_fused_serving_loop(work):
    """A serving loop: step s is redirected with the placement from the window
    before s (step 0 with the identity placement of the first rebalance of an
    all-zero window) and counted into the window; the placement is then
    recomputed.  Every output matches the oracle run the same way."""
    pl = work.placement
    L, E, W = work.layers, pl.E, work.window
    X = pl.max_count
    nsteps = 3
    steps = [wl.routing_step(work, s, tokens=min(work.tokens, 4096)) for s in range(nsteps)]
    ring = torch.zeros((W, L, E), dtype=torch.int32, device=DEV)
    load = torch.zeros((L, E), dtype=torch.int64, device=DEV)
    hists = []
    ref_load = np.zeros((L, E), dtype=np.int64)
    for s, idx_h in enumerate(steps):
        note(f"serving loop {work.name} step {s}")
        phy2log, log2phy, logcnt, status = eplb.rebalance(load, pl.P, pl.G, pl.N, pl.RK, X)
        ref = ora.rebalance(ref_load, pl.P, pl.G, pl.N, pl.RK, X)
        assert_same(f"step {s} log2phy", host(log2phy), ref["log2phy"])
        load, bad, out = eplb.hist_redirect(gpu(idx_h), E, ring, s, log2phy, logcnt)
        torch.cuda.synchronize()
        cnt, invl = ora.load_hist(idx_h, E)
        hists.append(cnt)
        ref_load = ora.window_load(hists, W)
        assert_same(f"step {s} window", host(load), ref_load)
        assert_same(f"step {s} redirect", host(out), ora.redirect(idx_h, ref["log2phy"], ref["logcnt"]))


def test_fused_full_size():
    """58 x 2^20 x 8 ids: whole-step counts against the oracle, redirect on
    sampled layers against the oracle and by its properties on every id."""
    work = wl.STREAM_1M
    pl = work.placement
    L, T, K, E, W = work.layers, work.tokens, work.topk, pl.E, work.window
    idx = torch.empty((L, T, K), dtype=torch.int32, device=DEV)
    wl.routing_step_device(work, 0, DEV, out=idx)
    idx_h = host(idx)
    cnt0, _ = ora.load_hist(idx_h, E)
    (phy2log, log2phy, logcnt, status), ref = rebalance_both(cnt0, pl.P, pl.G, pl.N, pl.RK)
    wl.routing_step_device(work, 1, DEV, out=idx)
    idx_h = host(idx)
    ring = torch.zeros((W, L, E), dtype=torch.int32, device=DEV)
    ring[0] = gpu(cnt0.astype(np.int32))
    note("stream hist_redirect step 1")
    load, bad, out = eplb.hist_redirect(idx, E, ring, 1, gpu(log2phy), gpu(logcnt))
    torch.cuda.synchronize()
    cnt1, invl = ora.load_hist(idx_h, E)
    assert_same("counts", host(ring[1]).astype(np.int64), cnt1)
    assert_same("window", host(load), cnt0 + cnt1)
    assert int(host(bad).sum()) == 0
    p2l = gpu(phy2log).long()
    cnt_t = gpu(logcnt).long()
    l2p = gpu(log2phy).long()
    t = torch.arange(T, device=DEV).unsqueeze(1)
    for l in range(L):
        o = out[l].long()
        e = idx[l].long()
        assert bool((p2l[l][o] == e).all())
        assert bool((l2p[l][e, t % cnt_t[l][e]] == o).all())
    out_h = host(out)
    for l in (0, 31, 57):
        assert_same(f"redirect layer {l}", out_h[l:l + 1],
                    ora.redirect(idx_h[l:l + 1], ref["log2phy"][l:l + 1], ref["logcnt"][l:l + 1]))


@pytest.mark.parametrize("T,K", [(2048, 8), (70000, 5)], ids=["one-workgroup-per-layer", "several-per-layer"])
def test_slot_and_invalid_overwritten(T, K):
    """The slot of this step, n_invalid and the count buffer of the moving
    average are written whatever they held before the call."""
    rng = np.random.default_rng(T)
    L, E, W = 3, 40, 4
    idx_h = rng.integers(-2, E + 2, size=(L, T, K)).astype(np.int32)
    for fused in (False, True):
        note(f"slot overwrite T={T} K={K} fused={fused}")
        ring = torch.full((W, L, E), 7, dtype=torch.int32, device=DEV)
        load = torch.full((L, E), -5, dtype=torch.int64, device=DEV)
        bad = torch.full((L,), 123, dtype=torch.int64, device=DEV)
        if fused:
            l2p = torch.zeros((L, E, 1), dtype=torch.int32, device=DEV)
            cnt1 = torch.ones((L, E), dtype=torch.int32, device=DEV)
            eplb.hist_redirect(gpu(idx_h), E, ring, 6, l2p, cnt1, load, bad)
        else:
            eplb.load_hist(gpu(idx_h), E, ring, 6, load, bad)
        torch.cuda.synchronize()
        cnt, invl = ora.load_hist(idx_h, E)
        assert_same("slot", host(ring[2]).astype(np.int64), cnt)
        assert_same("invalid", host(bad), invl)
        assert_same("window", host(load), cnt + 7 * (W - 1))
    ema = torch.full((L, E), 1000, dtype=torch.int64, device=DEV)
    count = torch.full((L, E), 9, dtype=torch.int32, device=DEV)
    bad = torch.full((L,), 123, dtype=torch.int64, device=DEV)
    eplb.load_ema(gpu(idx_h), E, ema, 2, count, bad)
    torch.cuda.synchronize()
    assert_same("ema count", host(count).astype(np.int64), cnt)
    assert_same("ema invalid", host(bad), invl)
    assert_same("ema", host(ema), ora.ema_update(np.full((L, E), 1000), cnt, 2).reshape(L, E))
