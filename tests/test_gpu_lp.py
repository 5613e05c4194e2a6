"""Per-batch redistribution over replica edges (LPLB-style): HIP path vs the
CPU oracle, through the C ABI (needs an MI355X).  Integer work: every output
is compared bit for bit."""
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
SOLVE_KEYS = ("lam", "flow", "rank_load", "status")


def note(msg: str) -> None:
    print(f"[lp] {msg}", flush=True)
    sys.stdout.flush()


def gpu(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x))).to(dtype).to(DEV)


def assert_same(name, got, want):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, f"{name}: shape {got.shape} vs {want.shape}"
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{name}: {len(bad)} mismatches, first at {i}: got {got[i]} want {want[i]}")


def solve_both(cnt, home, rep, rows=None):
    cnt, home, rep = (np.asarray(a) for a in (cnt, home, rep))
    B, E = cnt.shape
    RK = rep.shape[1]
    note(f"lp_solve B={B} E={E} RK={RK} R={rep.shape[2]}")
    got = [t.cpu().numpy() for t in eplb.lp_solve(gpu(cnt, torch.int64), gpu(home, torch.int32),
                                                  gpu(rep, torch.int32))]
    rows = list(range(B)) if rows is None else list(rows)
    ref = ora.lp_solve(cnt[rows], home[rows], rep[rows], RK)
    for k, g in zip(SOLVE_KEYS, got):
        assert_same(k, g[rows], ref[k])
    return dict(zip(SOLVE_KEYS, got))


def check_solution(cnt, home, rep, q):
    """Any size: flows within capacity, loads consistent, max load = lam."""
    B, RK = q["rank_load"].shape
    for b in range(B):
        assert q["status"][b] == 0
        load = oracle_pins._lp_loads(cnt[b], home[b], rep[b], q["flow"][b], RK)
        assert load.tolist() == q["rank_load"][b].tolist()
        assert load.max() == q["lam"][b]
        f = q["flow"][b]
        assert (f >= 0).all() and (f[rep[b] < 0] == 0).all()
        ok = rep[b] >= 0
        assert (f[ok] <= cnt[b][rep[b][ok]]).all()


@pytest.mark.parametrize("RK,R,E,top", [(1, 1, 3, 10), (2, 1, 5, 10), (3, 2, 9, 50), (5, 3, 40, 1000),
                                        (8, 2, 256, 10**5), (8, 4, 64, 7), (11, 2, 100, 10**6),
                                        (12, 3, 200, 10**5), (13, 2, 300, 10**3),
                                        (16, 4, 256, 10**4), (16, 1, 4096, 1 << 40)])
def test_lp_solve_random(RK, R, E, top):
    rng = np.random.default_rng(RK * 100 + R)
    cnt, home, rep = oracle_pins._lp_random(rng, RK, R, E, B=6, top=top, fill=0.8)
    if top == 1 << 40:
        cnt = rng.integers(0, (1 << 40) + 1, size=cnt.shape).astype(np.int64)
    q = solve_both(cnt, home, rep)
    check_solution(cnt, home, rep, q)


@pytest.mark.parametrize("work", [wl.LPLB_CUBE, wl.LPLB_HYPERCUBE], ids=lambda w: w.name)
def test_lp_solve_topologies(work):
    """Batches of 16384 tokens x top-8 on the 8-GPU cube (the pages' r2o)
    and the 16-GPU hypercube: all 58 layers checked, 12 against the oracle."""
    idx, home, rep = wl.lp_inputs(work)
    cnt = np.stack([np.bincount(idx[l].ravel(), minlength=work.E) for l in range(work.layers)]).astype(np.int64)
    q = solve_both(cnt, home, rep, rows=range(0, work.layers, 5))
    check_solution(cnt, home, rep, q)
    base = np.stack([np.bincount(home[l], weights=cnt[l], minlength=work.RK) for l in range(work.layers)])
    assert (q["lam"] <= base.max(axis=1)).all() and (q["lam"] < base.max(axis=1)).any()


def test_lp_solve_degenerate_and_bad():
    # no replicas, zero counts, already even loads, and each invalid input
    cnt = np.array([[5, 9, 1, 7]] * 3 + [[5, 1, 2, 0]] * 6, dtype=np.int64)
    home = np.array([[0, 1, 1, 2]] * 3 + [[0, 1, 1, 0]] * 6)
    rep = np.full((9, 3, 2), -1)
    rep[1, 0, 0], rep[1, 1, 0] = 1, 0
    cnt[2] = 0
    rep[3:, 0, 0], rep[3:, 1, 0] = 1, 0
    cnt[4, 2] = -1
    cnt[5, 2] = (1 << 40) + 1
    home[6, 0] = 3
    rep[7, 0, 1] = 4
    rep[8, 2, 1] = 0                                   # expert 0 twice
    q = solve_both(cnt, home, rep)
    assert q["status"].tolist() == [0, 0, 0, 0, 19, 19, 19, 19, 19]
    z = eplb.lp_solve(torch.zeros((0, 4), dtype=torch.int64, device=DEV),
                      torch.zeros((0, 4), dtype=torch.int32, device=DEV),
                      torch.zeros((0, 3, 2), dtype=torch.int32, device=DEV))
    assert [tuple(t.shape) for t in z] == [(0,), (0, 3, 2), (0, 3), (0,)]


# ---------------------------------------------------------------- redirect by the flows

@pytest.mark.parametrize("L,T,K,E,RK,R", [(2, 5000, 8, 64, 8, 2), (3, 1, 3, 5, 2, 1), (1, 2048, 1, 256, 8, 2),
                                          (2, 4097, 2, 1, 1, 1), (1, 33333, 3, 4096, 16, 4),
                                          (4, 700, 7, 300, 11, 3)])
def test_lp_redirect_random(L, T, K, E, RK, R):
    """Segments of 2048 ids cut anywhere (ragged tails, one id, several
    segments), out-of-range ids, flows of 0, above the count and negative,
    a workspace holding garbage."""
    rng = np.random.default_rng(L * T + E)
    idx_h = rng.integers(-2, E + 2, size=(L, T, K)).astype(np.int32)
    rep = np.full((L, RK, R), -1, dtype=np.int32)
    for l in range(L):
        pool = list(rng.permutation(E))
        for g in range(RK):
            for j in range(R):
                if pool and rng.random() < 0.8:
                    rep[l, g, j] = pool.pop()
    flow = rng.integers(-3, max(4, T * K // max(E, 1) * 2), size=(L, RK, R)).astype(np.int64)
    flow[0, 0, 0] = 1 << 40
    need = eplb.lp_redirect_workspace_bytes(L, T, K, E)
    ws = torch.randint(-1000, 1000, (max(need // 4, 1),), dtype=torch.int32, device=DEV)
    note(f"lp_redirect L={L} T={T} K={K} E={E} RK={RK} R={R}")
    got = eplb.lp_redirect(gpu(idx_h, torch.int32), E, gpu(rep, torch.int32), gpu(flow, torch.int64), ws)
    torch.cuda.synchronize()
    assert_same("lp_redirect", got.cpu().numpy(), ora.lp_redirect(idx_h, rep, flow, E))


def test_lp_redirect_bad_layers():
    rng = np.random.default_rng(2)
    E, RK, R = 20, 4, 2
    idx_h = rng.integers(0, E, size=(3, 3000, 2)).astype(np.int32)
    rep = np.array([[[0, 1], [2, 3], [4, 5], [6, 7]]] * 3, dtype=np.int32)
    rep[1, 3, 1] = 0                                   # expert 0 twice
    rep[2, 0, 0] = E + 4                               # out of range
    flow = np.full((3, RK, R), 100, dtype=np.int64)
    got = eplb.lp_redirect(gpu(idx_h, torch.int32), E, gpu(rep, torch.int32), gpu(flow, torch.int64)).cpu().numpy()
    assert_same("lp_redirect", got, ora.lp_redirect(idx_h, rep, flow, E))
    assert (got[1:] == -1).all() and (got[0] >= 0).all()


@pytest.mark.parametrize("work", [wl.LPLB_CUBE, wl.LPLB_HYPERCUBE], ids=lambda w: w.name)
def test_lp_batch_end_to_end(work):
    """One batch through the whole LPLB-style path on the GPU: per-layer
    counts (eplb_load_hist, W = 1), the solve, the redirect; the redirect
    matches the oracle on sampled layers, and on every layer the ids each
    rank ends up serving add up to the solve's rank loads."""
    idx_h, home, rep = wl.lp_inputs(work)
    L, E, RK = work.layers, work.E, work.RK
    R = rep.shape[2]
    idx = gpu(idx_h, torch.int32)
    ring = torch.zeros((1, L, E), dtype=torch.int32, device=DEV)
    cnt, bad = eplb.load_hist(idx, E, ring, 0)
    lam, flow, rank_load, status = eplb.lp_solve(cnt, gpu(home, torch.int32), gpu(rep, torch.int32))
    out = eplb.lp_redirect(idx, E, gpu(rep, torch.int32), flow)
    torch.cuda.synchronize()
    assert int(status.abs().sum()) == 0 and int(bad.sum()) == 0
    out_h, flow_h, load_h = out.cpu().numpy(), flow.cpu().numpy(), rank_load.cpu().numpy()
    for l in (0, 29, 57):
        assert_same(f"layer {l}", out_h[l:l + 1], ora.lp_redirect(idx_h[l:l + 1], rep[l:l + 1], flow_h[l:l + 1], E))
    rank_of = np.empty((L, E + RK * R), dtype=np.int64)
    rank_of[:, :E] = home
    rank_of[:, E:] = np.repeat(np.arange(RK), R)[None, :]
    for l in range(L):
        served = np.bincount(rank_of[l][out_h[l].ravel()], minlength=RK)
        assert served.tolist() == load_h[l].tolist(), f"layer {l}"
