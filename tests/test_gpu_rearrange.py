"""Rearrangement plan: HIP path vs the CPU oracle, through the C ABI (needs an
MI355X).  Integer work: every output is compared bit for bit."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle_pins
import workloads as wl
from oracle import eplb_oracle as ora

pytestmark = pytest.mark.gpu

eplb = pytest.importorskip("moe_expert_load_eplb_amd")
DEV = torch.device("cuda:0")
KEYS = ("phy2log", "log2phy", "src", "moves", "status")


def note(msg: str) -> None:
    print(f"[rearrange] {msg}", flush=True)
    sys.stdout.flush()


def gpu(x):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.int32))).to(DEV)


def assert_same(name, got, want):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, f"{name}: shape {got.shape} vs {want.shape}"
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{name}: {len(bad)} mismatches, first at {i}: got {got[i]} want {want[i]}")


def plan_both(old, new, l2p, RK, N, rows=None):
    old, new, l2p = (np.asarray(a) for a in (old, new, l2p))
    B, P = new.shape
    note(f"rearrange B={B} P={P} E={l2p.shape[1]} X={l2p.shape[2]} RK={RK} N={N}")
    got = [t.cpu().numpy() for t in eplb.rearrange(gpu(old), gpu(new), gpu(l2p), RK, N)]
    rows = list(range(B)) if rows is None else list(rows)
    ref = ora.rearrange_plan(old[rows], new[rows], l2p[rows], RK, N)
    for k, g in zip(KEYS, got):
        assert_same(k, g[rows], ref[k])
    return dict(zip(KEYS, got))


def check_properties(old, new, RK, q):
    """Cheap checks at any size: within-rank permutation, kept slots hold the
    old expert, sources hold the expert, fewest copies."""
    B, P = new.shape
    ppr = P // RK
    E = q["log2phy"].shape[1]
    assert (q["status"] == 0).all()
    plan = q["phy2log"]
    assert (np.sort(plan.reshape(B, RK, ppr), axis=2) == np.sort(new.reshape(B, RK, ppr), axis=2)).all()
    kept = q["src"] < 0
    assert (plan[kept] == old[kept]).all()
    rows, cols = np.nonzero(~kept)
    assert (old[rows, q["src"][rows, cols]] == plan[rows, cols]).all()
    for b in range(B):
        least = 0
        for r in range(RK):
            a = np.bincount(old[b, r * ppr:(r + 1) * ppr], minlength=E)
            c = np.bincount(new[b, r * ppr:(r + 1) * ppr], minlength=E)
            least += ppr - int(np.minimum(a, c).sum())
        assert int(q["moves"][b].sum()) == least == int((~kept[b]).sum())


def test_rearrange_hand_cases():
    plan_both([[0, 1, 2, 3, 4, 0]], [[2, 0, 0, 4, 1, 3]], [[[1, 2], [4, -1], [0, -1], [5, -1], [3, -1]]], 2, 2)
    for N in (1, 2):
        plan_both([[0, 1, 2, 3, 4, 1]], [[3, 4, 0, 1, 2, 0]], [[[2, 5], [3, -1], [4, -1], [0, -1], [1, -1]]], 2, N)


def test_rearrange_worked_example():
    """Layer 0's printed placement in force, layer 1's as the new one (and
    the reverse), on the example's 2 nodes x 4 GPUs."""
    g = oracle_pins.GOLDEN
    p2l = np.array(g["phy2log"]["value"], dtype=np.int64)
    l2p = oracle_pins._valid_l2p(p2l, 12, 3)
    plan_both(p2l[[0, 1]], p2l[[1, 0]], l2p[[1, 0]], 8, 2)


@pytest.mark.parametrize("case", ["dsv3", "global", "decode144", "skewed"])
def test_rearrange_between_rebalances(case):
    """The serving use: the placement from one window's loads in force, the
    next window's placement computed; both from the GPU rebalance."""
    if case == "skewed":
        pl = wl.SKEWED_1024.placement
        a = wl.skewed_loads()
        b = np.roll(a, 1, axis=1)
        rows = [0, 1, 511, 1023]
        nodes = pl.N
    else:
        pl = {"dsv3": wl.DSV3_PREFILL.placement, "global": wl.GLOBAL_DECODE.placement,
              "decode144": wl.DSV3_DECODE_144}[case]
        a = wl.zipf_loads(58, pl.E, 1.1, 1 << 20, wid=21)
        b = wl.zipf_loads(58, pl.E, 1.1, 1 << 20, wid=22)
        rows = None
        nodes = pl.N
    old = [t.cpu().numpy() for t in eplb.rebalance(torch.from_numpy(a).to(DEV), pl.P, pl.G, pl.N, pl.RK)]
    new = [t.cpu().numpy() for t in eplb.rebalance(torch.from_numpy(b).to(DEV), pl.P, pl.G, pl.N, pl.RK)]
    q = plan_both(old[0], new[0], new[1], pl.RK, nodes, rows)
    check_properties(old[0], new[0], pl.RK, q)


@pytest.mark.parametrize("B,E,RK,ppr,N", [(7, 5, 3, 2, 3), (4, 40, 8, 9, 2), (3, 300, 64, 5, 8), (2, 70, 1, 100, 1),
                                          (5, 1, 4, 3, 2), (2, 1000, 2, 2048, 1), (3, 13, 13, 1, 13)])
def test_rearrange_random(B, E, RK, ppr, N):
    """Random placements (every expert has a replica), ragged against the
    workgroup size, one slot per rank, one rank, many slots per thread."""
    rng = np.random.default_rng(B * 1000 + E)
    P = RK * ppr
    E = min(E, P)

    def placement():
        return np.stack([rng.permutation(np.concatenate([np.arange(E), rng.integers(0, E, P - E)]))
                         for _ in range(B)])
    old = placement()
    new = old.copy()
    new[: B // 2] = placement()[: B // 2]                     # half fresh, half a small change
    for b in range(B // 2, B):
        i = rng.integers(0, P, size=max(1, P // 10))
        new[b, i] = new[b, rng.permutation(i)]
    X = max(int(np.bincount(new[b], minlength=E).max()) for b in range(B)) + 1
    q = plan_both(old, new, oracle_pins._valid_l2p(new, E, X), RK, N)
    check_properties(old, new, RK, q)


def _oracle_check(job):
    """In a worker process (numpy and the oracle only): the first output of
    one case that differs from the oracle's, or None."""
    i, old, new, l2p, RK, N, got = job
    ref = ora.rearrange_plan(old, new, l2p, RK, N)
    for k, g in zip(KEYS, got):
        if not np.array_equal(g, ref[k]):
            return i, k
    return None


def test_rearrange_wide_fuzz():
    """1500 random cases of three problems: 1 to 256 ranks, any node count
    dividing them, 1 to 9 slots per rank, fresh or slightly changed
    placements, log2phy wider than needed, and one problem in eight with a
    bad entry; every output against the oracle (on a pool of forked worker
    processes, which touch no GPU)."""
    import multiprocessing
    import os
    rng = np.random.default_rng(20261206)
    jobs = []
    for i in range(1500):
        RK = int(rng.choice([1, 2, 3, 4, 5, 8, 13, 16, 32, 64, 100, 256]))
        N = int(rng.choice([d for d in range(1, RK + 1) if RK % d == 0]))
        ppr = int(rng.integers(1, 10))
        P = RK * ppr
        E = int(rng.integers(1, P + 1))
        B = 3

        def placement():
            return np.stack([rng.permutation(np.concatenate([np.arange(E), rng.integers(0, E, P - E)]))
                             for _ in range(B)])
        old = placement()
        new = placement() if rng.random() < 0.5 else old.copy()
        if rng.random() < 0.5:
            for b in range(B):
                j = rng.integers(0, P, size=max(1, P // 8))
                new[b, j] = new[b, rng.permutation(j)]
        X = max(int(np.bincount(new[b], minlength=E).max()) for b in range(B)) + int(rng.integers(0, 3))
        l2p = oracle_pins._valid_l2p(new, E, X)
        if rng.random() < 0.125:
            b = int(rng.integers(0, B))
            which = int(rng.integers(0, 3))
            if which == 0:
                old[b, int(rng.integers(0, P))] = E
            elif which == 1:
                new[b, int(rng.integers(0, P))] = -1
            else:
                l2p[b, int(rng.integers(0, E)), 0] = P
        got = [t.cpu().numpy() for t in eplb.rearrange(gpu(old), gpu(new), gpu(l2p), RK, N)]
        jobs.append((i, old, new, l2p, RK, N, got))
        if i % 500 == 0:
            note(f"wide fuzz: {i} cases on the GPU")
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    note(f"wide fuzz: oracle on {workers} processes")
    with multiprocessing.get_context("fork").Pool(workers) as pool:
        bad = [r for r in pool.imap_unordered(_oracle_check, jobs, chunksize=4) if r is not None]
    assert not bad, f"{len(bad)} cases differ from the oracle, first: {bad[0]}"


def test_rearrange_many_problems():
    """100,000 problems in one call (a grid past 65,535 workgroups); every
    997th against the oracle."""
    rng = np.random.default_rng(8)
    B, E, RK, ppr, N = 100_000, 6, 4, 2, 2
    P = RK * ppr

    def placement():
        base = np.concatenate([np.arange(E), rng.integers(0, E, size=(P - E,))])
        return np.stack([rng.permutation(base) for _ in range(B)])
    old, new = placement(), placement()
    X = max(int(np.bincount(r, minlength=E).max()) for r in new[::1000]) + 3
    # log2phy of every problem, vectorised: slot of the r-th copy of each expert
    l2p = np.full((B, E, X), -1, dtype=np.int64)
    order = np.argsort(new, axis=1, kind="stable")
    sorted_e = np.take_along_axis(new, order, axis=1)
    first = np.zeros((B, P), dtype=np.int64)
    for j in range(1, P):
        first[:, j] = np.where(sorted_e[:, j] == sorted_e[:, j - 1], first[:, j - 1] + 1, 0)
    l2p[np.repeat(np.arange(B), P), sorted_e.ravel(), first.ravel()] = order.ravel()
    rows = list(range(0, B, 997)) + [B - 1]
    plan_both(old, new, l2p, RK, N, rows=rows)


def test_rearrange_max_size():
    """P = 8192 on one rank (the longest scans) and on 512 ranks; E = 4096;
    checked by properties."""
    rng = np.random.default_rng(77)
    E, P = 4096, 8192
    old = np.stack([rng.permutation(np.concatenate([np.arange(E), rng.integers(0, E, P - E)])) for _ in range(2)])
    new = np.stack([rng.permutation(np.concatenate([np.arange(E), rng.integers(0, E, P - E)])) for _ in range(2)])
    X = max(int(np.bincount(new[b], minlength=E).max()) for b in range(2))
    l2p = oracle_pins._valid_l2p(new, E, X)
    for RK, N in ((1, 1), (512, 64)):
        note(f"rearrange max size RK={RK}")
        q = dict(zip(KEYS, (t.cpu().numpy() for t in eplb.rearrange(gpu(old), gpu(new), gpu(l2p), RK, N))))
        check_properties(old, new, RK, q)


def test_rearrange_bad_maps_and_empty():
    old = np.array([[0, 1, 2, 3]] * 5)
    new = np.array([[1, 0, 3, 2]] * 5)
    l2p = oracle_pins._valid_l2p(new, 4, 1)
    old[1, 2] = 4
    new[2, 0] = -1
    l2p[3, 0, 0] = 4
    new[4, 0] = 1
    old[4, 1] = 0
    q = plan_both(old, new, l2p, 2, 1)
    assert q["status"].tolist() == [0, 18, 18, 18, 18]
    z = torch.zeros((0, 4), dtype=torch.int32, device=DEV)
    outs = eplb.rearrange(z, z, torch.zeros((0, 4, 1), dtype=torch.int32, device=DEV), 2, 1)
    assert [tuple(t.shape) for t in outs] == [(0, 4), (0, 4, 1), (0, 4), (0, 3), (0,)]
