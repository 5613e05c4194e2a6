"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

Integer work throughout, so every comparison is bit-exact.  Small and
mid-size inputs are compared element by element; so is the full-size
streaming workload (58 layers x 2^20 tokens x top-8): whole per-step
histograms and the redirect of every layer, with properties that hold at
any size checked on the device besides.
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
        X = ora.max_count(E, P, G, N)
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


def test_rebalance_experts_interface():
    """The pages' call on their example (float weights on the host, as the
    pages pass them, and int64 on the GPU): int64 maps on the weight's
    device, log2phy as wide as the largest count, the printed values."""
    g = oracle_pins.GOLDEN
    inp = g["inputs"]
    args = (inp["num_replicas"], inp["num_groups"], inp["num_nodes"], inp["num_gpus"])
    w = torch.tensor(inp["weight"], dtype=torch.float32)
    for weight in (w, w.to(torch.int64).to(DEV)):
        phy2log, log2phy, logcnt = eplb.rebalance_experts(weight, *args)
        assert all(t.dtype == torch.int64 and t.device == weight.device for t in (phy2log, log2phy, logcnt))
        assert phy2log.tolist() == g["phy2log"]["value"]
        assert logcnt[0].tolist() == g["layer0_logcnt"]["value"]
        assert log2phy.shape == (2, 12, 2)
        assert log2phy[0, 0].tolist() == g["layer0_log2phy"]["expert0"]
        assert log2phy[0, 1].tolist() == g["layer0_log2phy"]["expert1"]
    with pytest.raises(ValueError):
        eplb.rebalance_experts(w + 0.5, *args)
    with pytest.raises(ValueError):
        eplb.rebalance_experts(w * 2.0 ** 70, *args)            # beyond int64
    with pytest.raises(eplb.EplbError):
        eplb.rebalance_experts(-w, *args)                       # negative loads: the problem's status
    with pytest.raises(eplb.EplbError):
        eplb.rebalance_experts(w, 16, 4, 2, 7)                  # 16 slots do not divide over 7 GPUs


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


def _oracle_rows(args):
    load, P, G, N, RK, X = args
    return ora.rebalance(load, P, G, N, RK, X)


def _oracle_rebalance_pool(load, P, G, N, RK, X, parts=16):
    """The oracle on every row of ``load``, the rows split over a pool of
    forked host processes (they run Python only and touch no GPU)."""
    import multiprocessing
    nw = max(1, min(parts, len(os.sched_getaffinity(0))))
    chunks = [c for c in np.array_split(np.arange(load.shape[0]), nw) if len(c)]
    with multiprocessing.get_context("fork").Pool(len(chunks)) as pool:
        parts_out = pool.map(_oracle_rows, [(load[c], P, G, N, RK, X) for c in chunks])
    return {k: np.concatenate([r[k] for r in parts_out]) for k in ("phy2log", "log2phy", "logcnt", "status")}


def test_skewed_1024_rebalance():
    """All 1024 problems of the skewed batch, element by element."""
    work = wl.SKEWED_1024
    pl = work.placement
    load = wl.skewed_loads()
    X = ora.max_count(pl.E, pl.P, pl.G, pl.N)
    note(f"rebalance skewed B={load.shape[0]}")
    outs = eplb.rebalance(gpu(load), pl.P, pl.G, pl.N, pl.RK, X)
    torch.cuda.synchronize()
    phy2log, log2phy, logcnt, status = (host(t) for t in outs)
    assert (status == 0).all()
    note("oracle on all 1024 skewed problems")
    ref = _oracle_rebalance_pool(load, pl.P, pl.G, pl.N, pl.RK, X)
    for name, g in (("phy2log", phy2log), ("log2phy", log2phy), ("logcnt", logcnt), ("status", status)):
        assert_same(name, g, ref[name])
    for b in range(0, work.layers, 128):
        inv.check_placement(load[b], phy2log[b], log2phy[b], logcnt[b], pl.E, pl.P, pl.G, pl.N, pl.RK)


def test_stream_1m_full_size():
    """58 x 2^20 x 8 ids per step, 10-step window, C1-shaped placement,
    redirect of the last step: whole histograms compared per step; the
    redirect compared element by element on every layer, and by its
    properties on the device."""
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
    # element by element on every layer, one layer at a time
    out_h = host(out)
    for l in range(L):
        assert_same(f"redirect layer {l}", out_h[l:l + 1],
                    ora.redirect(idx_h[l:l + 1], ref["log2phy"][l:l + 1], ref["logcnt"][l:l + 1]))


def test_stream_1m_global_placement():
    """One step of the streaming workload (58 x 2^20 x 8 ids) through the
    global-policy decode placement (E = 256, P = 320 on 5 nodes x 8 GPUs,
    X = 65), the launch bench.py times for the wide-table redirect: the
    placement from the step's own histogram against the oracle, then the
    redirect and the fused pass element by element on every layer."""
    work, pl = wl.STREAM_1M, wl.GLOBAL_DECODE.placement
    L, T, K, E = work.layers, work.tokens, work.topk, pl.E
    idx = torch.empty((L, T, K), dtype=torch.int32, device=DEV)
    note("global placement stream: generate + hist")
    wl.routing_step_device(work, 3, DEV, out=idx)
    ring = torch.zeros((2, L, E), dtype=torch.int32, device=DEV)
    load, bad = eplb.load_hist(idx, E, ring, step=0)
    torch.cuda.synchronize()
    (phy2log, log2phy, logcnt, status), ref = rebalance_both(host(load), pl.P, pl.G, pl.N, pl.RK)
    assert log2phy.shape[2] == 65 and int(logcnt.max()) > 1
    l2p, cnt = gpu(log2phy), gpu(logcnt)
    note("global placement stream: redirect + fused pass")
    out = eplb.redirect(idx, l2p, cnt)
    _, _, fused = eplb.hist_redirect(idx, E, ring, 1, l2p, cnt)
    torch.cuda.synchronize()
    assert bool(torch.equal(out, fused)), "fused pass and redirect differ"
    assert bool(torch.equal(ring[1], ring[0])), "the fused pass counted other totals"
    idx_h, out_h = host(idx), host(out)
    for l in range(L):
        assert_same(f"redirect layer {l}", out_h[l:l + 1],
                    ora.redirect(idx_h[l:l + 1], ref["log2phy"][l:l + 1], ref["logcnt"][l:l + 1]))


def test_layer_beyond_2gib():
    """One layer of 2^29 + 24 ids (just over 2 GiB): the redirect and the
    fused pass store through global stores instead of the buffer stores of
    smaller layers.  Every id is checked by the redirect's definition and the
    counts against a bincount; a slice of tokens element by element against
    the oracle."""
    pl = wl.DSV3_PREFILL.placement
    E, T, K = pl.E, (1 << 26) + 3, 8
    load = wl.zipf_loads(1, E, 1.1, 1 << 20)
    (phy2log, log2phy, logcnt, status), ref = rebalance_both(load, pl.P, pl.G, pl.N, pl.RK)
    g = torch.Generator(device=DEV)
    g.manual_seed(2026)
    note("layer beyond 2 GiB: generate")
    idx = torch.randint(0, E, (1, T, K), dtype=torch.int32, device=DEV, generator=g)
    l2p, cnt = gpu(log2phy), gpu(logcnt)
    note("layer beyond 2 GiB: redirect")
    out = eplb.redirect(idx, l2p, cnt)
    W = 2
    ring = torch.zeros((W, 1, E), dtype=torch.int32, device=DEV)
    note("layer beyond 2 GiB: hist_redirect")
    wload, bad, fused = eplb.hist_redirect(idx, E, ring, 0, l2p, cnt)
    torch.cuda.synchronize()
    assert bool(torch.equal(out, fused)), "fused pass and redirect differ"
    e = idx[0].long()
    t = torch.arange(T, device=DEV).unsqueeze(1)
    want = l2p[0].long()[e, t % cnt[0].long()[e]]
    assert bool((out[0].long() == want).all()), "a redirected id is not log2phy[e][t mod logcnt[e]]"
    del e, want
    counts = torch.bincount(idx.view(-1).long(), minlength=E)
    assert bool(torch.equal(ring[0, 0].long(), counts)) and bool(torch.equal(wload[0], counts))
    assert int(bad.sum()) == 0
    # the last 5000 tokens against the oracle: their rows start at T0, so
    # T0 mod lcm(counts) rows of padding in front give every count the same
    # row residues
    T0 = T - 5000
    pad = T0 % int(np.lcm.reduce(ref["logcnt"][0].astype(np.int64)))
    idx_h = np.concatenate([np.zeros((1, pad, K), np.int32), host(idx[:, T0:])], axis=1)
    want_h = ora.redirect(idx_h, ref["log2phy"], ref["logcnt"])[:, pad:]
    assert_same("last 5000 tokens", host(out[:, T0:]), want_h)


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
    (65, 5, 1, 5, 70),        # replication on the first 64 experts, one expert behind them
    (128, 1, 1, 16, 160),     # 32 replicas among 128 experts
    (512, 1, 1, 8, 576),      # 64 replicas among 512 experts (eight registers)
    (384, 6, 2, 16, 512),     # two nodes of 192 experts, 64 replicas each
    (256, 8, 3, 40, 320),     # global: 64 replicas among 256 (the decode shape)
])
def test_shapes_random(shape):
    E, G, N, RK, P = shape
    rng = np.random.default_rng(E * 1000 + P)
    load = rng.integers(0, 1000, size=(12, E)) * rng.integers(0, 2, size=(12, E))
    load[0] = 0
    load[1] = 7
    load[2] = rng.integers(0, 3, size=E)
    rebalance_both(load, P, G, N, RK)


def _selection_loads(E, seed):
    """Load patterns that stress the replicas-at-once form of step 2: zeros,
    equal loads, small-integer ties, exact ratio ties (multiples of one
    base), loads near 2^40, Zipf, one hot expert, and the heaviest expert
    holding the highest index (it loses every tie of value)."""
    rng = np.random.default_rng(seed)
    rows = [
        np.zeros(E),
        np.full(E, 7),
        rng.integers(0, 4, size=E),
        rng.integers(1, 30) * rng.choice([1, 2, 3, 4, 6, 12, 60], size=E),
        rng.integers((1 << 40) - 64, (1 << 40) + 1, size=E),
        (rng.zipf(1.2, size=E) * 1000).clip(0, 1 << 40),
        np.where(np.arange(E) == rng.integers(0, E), 1 << 40, 1),
        np.arange(E) * 3,
        (E - np.arange(E)) * 5,
        rng.integers(0, 1000, size=E) * rng.integers(0, 2, size=E),
        np.where(np.arange(E) % 2 == 0, 12, 0),
        np.where(np.arange(E) >= E - 2, 360, rng.choice([0, 40, 60, 90, 120, 180], size=E)),
    ]
    return np.stack(rows).astype(np.int64)


@pytest.mark.parametrize("shape", [
    (64, 1, 1, 8, 88),          # 24 replicas among 64 experts (the smallest count taken at once)
    (40, 1, 1, 8, 104),         # 64 replicas among 40 experts
    (33, 3, 1, 11, 66),         # 33 among 33
    (128, 2, 2, 16, 192),       # two nodes of 64 experts, 32 replicas each
    (100, 4, 2, 10, 150),       # two nodes of 50, 25 each
    (512, 8, 8, 64, 1024),      # eight nodes of 64, 64 each
    (1, 1, 1, 1, 25),           # one expert, 24 replicas
    (2, 1, 1, 2, 66),           # two experts, 64 replicas
    (130, 2, 2, 26, 234),       # two nodes of 65: one expert behind the first 64
    (200, 8, 1, 8, 264),        # 64 replicas among 200 experts
    (256, 8, 18, 144, 288),     # global: 32 replicas among 256 (the 144-GPU decode shape)
    (256, 8, 3, 40, 320),       # global: 64 among 256 (the decode shape)
])
def test_replication_by_selection(shape):
    """Nodes with 24 to 64 replicas, where step 2 takes its replicas at once
    instead of one by one, against the oracle's one-by-one greedy."""
    E, G, N, RK, P = shape
    rebalance_both(_selection_loads(E, E * 7 + P), P, G, N, RK)


@pytest.mark.parametrize("shape", [
    (256, 8, 4, 32, 288),       # DeepSeek-V3 prefill: 8 GPUs per node, 9 slots each
    (128, 4, 2, 32, 160),       # 16 GPUs per node, 5 slots each
    (96, 4, 4, 16, 128),        # 4 GPUs per node, 8 slots each
    (64, 2, 1, 8, 112),         # 8 GPUs, 14 slots each (the 32-bit form's largest pack)
    (64, 2, 1, 8, 120),         # 8 GPUs, 15 slots each (beyond it: the 64-bit words)
])
def test_step3_word_widths(shape):
    """The same shapes with loads scaled so that the node totals (times the
    lcm of the counts) fall below 2^24, below 2^48 and above it: step 3
    packs with 32-bit words, 64-bit words and wider sums, each against the
    oracle."""
    E, G, N, RK, P = shape
    rng = np.random.default_rng(E + P)
    base = (rng.zipf(1.3, size=(4, E)) * 7).clip(0, 1000)
    base[1] = rng.integers(0, 1000, size=E)
    base[2] = np.arange(E) % 13
    base[3, : E // 2] = 0
    for scale in (1, 1 << 11, 1 << 12, 1 << 22, 1 << 30):
        rebalance_both((base * scale).clip(0, 1 << 40).astype(np.int64), P, G, N, RK)


@pytest.mark.parametrize("shape", [
    (8, 8, 8, 504, 3528),       # one expert per node, 441 copies of it (counts past 128: the general lcm)
    (24, 24, 8, 432, 3456),     # three experts per node on 54 GPUs of 8 slots
    (1152, 4, 4, 240, 1200),    # 288 experts per node on 60 GPUs (64,312 B of LDS, at the budget)
])
def test_shapes_at_the_lds_budget(shape):
    """Shapes whose working set is just below the 64 KB LDS budget (17 to 64
    GPUs per node need no packing scratch), with zero, equal, skewed and
    large loads, against the oracle."""
    E, G, N, RK, P = shape
    rng = np.random.default_rng(E + P)
    load = rng.integers(0, 1000, size=(4, E)).astype(np.int64)
    load[0] = 0
    load[1] = 5
    load[2] = (rng.zipf(1.2, size=E) * 100).clip(0, 1 << 40)
    load[3] = rng.integers((1 << 40) - 1000, (1 << 40) + 1, size=E)
    rebalance_both(load, P, G, N, RK)


@pytest.mark.parametrize("shape,rows", [
    ((3, 1, 1, 3, 300), [[5, 4, 3], [1, 1, 1], [0, 0, 0], [7, 0, 3], [9, 6, 2]]),
    ((4, 1, 1, 4, 400), [[5, 4, 3, 2], [1, 1, 1, 1], [8, 0, 6, 3], [100, 99, 98, 97]]),
])
def test_counts_above_64(shape, rows):
    """Replica counts between 65 and 128 (several distinct ones: the lcm of
    the counts up to 64 by prime powers, then each larger count by Euclid)
    and beyond 128 (the general prime-power table), against the oracle."""
    E, G, N, RK, P = shape
    rebalance_both(np.array(rows, dtype=np.int64), P, G, N, RK)


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


def _wide_fuzz_shapes(rng, count):
    """Valid shapes over a wider range than _fuzz_shapes: up to 16 nodes and
    1024 experts, 1 to 256 GPUs per node, 1 to 8 experts per GPU, group
    sizes up to 16."""
    out = []
    while len(out) < count:
        N = int(rng.choice([1, 1, 2, 3, 4, 5, 6, 8, 16]))
        hier = N == 1 or rng.random() < 0.6
        G = N * int(rng.integers(1, 5)) if hier else int(rng.choice([g for g in range(2, 20) if g % N]))
        Np = N if hier else 1
        E = G * int(rng.integers(1, 17)) if hier else int(rng.integers(2, 300))
        RK = Np * int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 12, 15, 16, 17, 20, 24, 31, 32, 33, 40, 48, 63,
                                  64, 65, 80, 100, 128, 130, 200, 256]))
        P = RK * int(rng.integers(1, 9))
        if P < E or E > 1024 or P > 2048 or E // Np > 512 or RK > 512 or (hier and E % G):
            continue
        out.append((E, G, N, RK, P))
    return out


def _fuzz_loads(rng, E, B):
    """B load rows of one of ten kinds: ties of small values, uniform, Zipf,
    near 2^40, one hot expert, all equal, powers of two, values whose ratios
    to replica counts tie, mostly zero, all zero."""
    rows = []
    for _ in range(B):
        k = int(rng.integers(0, 10))
        if k == 0:
            r = rng.integers(0, 3, size=E)
        elif k == 1:
            r = rng.integers(0, 1 << 20, size=E)
        elif k == 2:
            r = (rng.zipf(1.2, size=E) * 997).clip(0, 1 << 40)
        elif k == 3:
            r = rng.integers((1 << 40) - 50, (1 << 40) + 1, size=E)
        elif k == 4:
            r = rng.integers(0, 100, size=E)
            r[rng.integers(0, E)] = int(rng.integers(1 << 20, 1 << 40))
        elif k == 5:
            r = np.full(E, int(rng.integers(0, 1 << 40)))
        elif k == 6:
            r = 1 << rng.integers(0, 41, size=E)
        elif k == 7:
            r = rng.choice([0, 6, 12, 18, 24, 36, 60, 120, 360, 720], size=E)
        elif k == 8:
            r = np.where(rng.random(E) < 0.8, 0, rng.integers(1, 1000, size=E))
        else:
            r = np.zeros(E)
        rows.append(np.asarray(r, dtype=np.int64))
    return np.stack(rows)


def _oracle_check(job):
    """In a worker process (numpy and the oracle only): the first output of
    one shape that differs from the oracle's, or None."""
    shape, X, load, got = job
    E, G, N, RK, P = shape
    ref = ora.rebalance(load, P, G, N, RK, X)
    for name, g in zip(("phy2log", "log2phy", "logcnt", "status"), got):
        if not np.array_equal(g, ref[name]):
            return shape, name, tuple(np.argwhere(g != ref[name])[0])
    return None


def test_wide_random_fuzz():
    """3000 random shapes of _wide_fuzz_shapes, four load rows each of the
    ten kinds of _fuzz_loads, every output against the oracle (the oracle on
    a pool of forked worker processes, which touch no GPU)."""
    import multiprocessing
    import os
    rng = np.random.default_rng(20261204)
    jobs = []
    for i, (E, G, N, RK, P) in enumerate(_wide_fuzz_shapes(rng, 3000)):
        X = ora.max_count(E, P, G, N)
        load = _fuzz_loads(rng, E, 4)
        outs = eplb.rebalance(gpu(load), P, G, N, RK, X)
        torch.cuda.synchronize()
        jobs.append(((E, G, N, RK, P), X, load, [host(t) for t in outs]))
        if i % 500 == 0:
            note(f"wide fuzz: {i} shapes on the GPU")
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    note(f"wide fuzz: oracle on {workers} processes")
    with multiprocessing.get_context("fork").Pool(workers) as pool:
        bad = [r for r in pool.imap_unordered(_oracle_check, jobs, chunksize=8) if r is not None]
    assert not bad, f"{len(bad)} shapes differ from the oracle, first: {bad[0]}"


@pytest.mark.parametrize("shape", [
    (512, 16, 8, 64, 640),       # 16 groups onto 8 nodes; totals of 2^48 and above take the 64-bit sums
    (128, 64, 32, 32, 160),      # 64 groups onto 32 nodes: runs found in LDS (17 to 64 nodes)
    (128, 128, 64, 64, 192),     # 128 groups onto 64 nodes: more than 64 groups ranked by the whole workgroup
    (256, 256, 128, 128, 384),   # 256 groups onto 128 nodes: eight registers of node packs
    (1024, 256, 128, 128, 1280),  # the same with 8 experts per node
])
def test_step1_packing_forms(shape):
    """Every form of the groups-onto-nodes packing, including the general
    one for total loads of 2^48 and above, against the oracle."""
    E, G, N, RK, P = shape
    rng = np.random.default_rng(E + G + N)
    top = 1 << 40
    load = np.stack([
        rng.integers(top - (1 << 30), top + 1, size=E),          # sums far above 2^48
        rng.integers(0, 1 << 20, size=E),                         # small: the one-word form
        rng.integers(0, 4, size=E),                               # many ties
        np.zeros(E, dtype=np.int64),
        (rng.zipf(1.2, size=E) * 4096).clip(0, top),
        np.full(E, top),
    ]).astype(np.int64)
    if E >= 256:                                                  # the last row's total is E * 2^40
        assert int(load[5].sum()) >= (1 << 48) - 1
    rebalance_both(load, P, G, N, RK)


@pytest.mark.parametrize("shape", [
    (1164, 12, 6, 186, 1302),    # 66 KiB
    (600, 8, 4, 512, 3072),      # 80 KiB: 128 GPUs per node, counts up to 619
    (1860, 20, 5, 500, 2000),    # 114 KiB, global policy
    (2048, 8, 4, 32, 2304),      # 116 KiB
    (2048, 16, 8, 256, 4096),    # 144 KiB
    (2560, 8, 8, 64, 3072),      # 148 KiB
])
def test_shapes_beyond_64k_lds(shape):
    """Shapes whose working set is between 64 and 160 KiB of LDS (one
    workgroup per compute unit), zero, tied, skewed and 2^40-scale loads,
    against the oracle."""
    E, G, N, RK, P = shape
    X = ora.max_count(E, P, G, N)
    assert eplb.lib.eplb_rebalance_lds_bytes(E, P, G, N, RK, X) > 64 * 1024
    rng = np.random.default_rng(E + P)
    load = np.stack([
        rng.integers(0, 3, size=E),
        (rng.zipf(1.2, size=E) * 1000).clip(0, 1 << 40),
        rng.integers((1 << 40) - 1000, (1 << 40) + 1, size=E),
        np.where(np.arange(E) % 7 == 0, rng.integers(0, 1 << 30, size=E), 0),
    ]).astype(np.int64)
    rebalance_both(load, P, G, N, RK, X)


def test_wide_shape_many_problems():
    """300 problems of a shape above 64 KiB of LDS with one register of
    experts and of GPUs per node (the form held to 64 registers for batches
    beyond one workgroup per compute unit); every 7th against the oracle."""
    E, G, N, RK, P = 2048, 64, 32, 64, 2304                  # 32 nodes of 64 experts, 2 GPUs each
    X = ora.max_count(E, P, G, N)
    assert eplb.lib.eplb_rebalance_lds_bytes(E, P, G, N, RK, X) > 64 * 1024
    rng = np.random.default_rng(17)
    load = (rng.zipf(1.2, size=(300, E)) * 100).clip(0, 1 << 40).astype(np.int64)
    load[::5] = rng.integers(0, 3, size=(60, E))
    got = [host(t) for t in eplb.rebalance(gpu(load), P, G, N, RK, X)]
    rows = list(range(0, 300, 7)) + [299]
    ref = ora.rebalance(load[rows], P, G, N, RK, X)
    for name, g in zip(("phy2log", "log2phy", "logcnt", "status"), got):
        assert_same(name, g[rows], ref[name])


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


def test_many_problems_and_layers():
    """Grids far past 65,535 workgroups: 200,000 small rebalance problems
    (every 997th against the oracle, all by the invariants) and 70,000
    streaming layers through the fused pass (all against the oracle)."""
    rng = np.random.default_rng(31)
    B, E, P, G, N, RK = 200_000, 16, 24, 4, 2, 8
    load = rng.integers(0, 1 << 20, size=(B, E)).astype(np.int64)
    note(f"rebalance B={B}")
    phy2log, log2phy, logcnt, status = (host(t) for t in eplb.rebalance(gpu(load), P, G, N, RK))
    rows = list(range(0, B, 997)) + [B - 1]
    ref = ora.rebalance(load[rows], P, G, N, RK, ora.max_count(E, P, G, N))
    for name, got in zip(("phy2log", "log2phy", "logcnt", "status"), (phy2log, log2phy, logcnt, status)):
        assert_same(name, got[rows], ref[name])
    assert (status == 0).all() and (logcnt.sum(axis=1) == P).all() and (logcnt >= 1).all()
    placed = np.zeros((B, E), dtype=np.int64)                          # each expert's slots = its count
    np.add.at(placed, (np.repeat(np.arange(B), P), phy2log.ravel()), 1)
    assert (placed == logcnt).all()
    L, T, K = 70_000, 3, 2
    idx_h = rng.integers(-1, E + 1, size=(L, T, K)).astype(np.int32)
    X = 4
    cnt_h = rng.integers(1, X + 1, size=(L, E)).astype(np.int32)
    l2p_h = rng.integers(0, 1000, size=(L, E, X)).astype(np.int32)
    ring = torch.zeros((2, L, E), dtype=torch.int32, device=DEV)
    note(f"hist_redirect L={L}")
    load_w, bad, out = eplb.hist_redirect(gpu(idx_h), E, ring, 1, gpu(l2p_h), gpu(cnt_h))
    torch.cuda.synchronize()
    cnt, invl = ora.load_hist(idx_h, E)
    assert_same("counts", host(ring[1]).astype(np.int64), cnt)
    assert_same("window", host(load_w), cnt)
    assert_same("invalid", host(bad), invl)
    assert_same("redirect", host(out), ora.redirect(idx_h, l2p_h, cnt_h))


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


def test_stream_entries_wide_fuzz():
    """300 more random cases through the redirect, the fused pass and the
    fused moving average over a wider range: up to 4096 experts and log2phy
    widths up to 70 (placements whose replica lists exceed the workgroup's
    staged table read the global rows), outputs on every 4-byte phase
    against the input, against the oracle."""
    rng = np.random.default_rng(2026)
    for case in range(300):
        L = int(rng.integers(1, 5))
        T = int(rng.choice([1, 5, int(rng.integers(1, 3000))]))
        K = int(rng.integers(1, 9))
        E = int(rng.choice([3, 64, 256, 1000, 4096, int(rng.integers(1, 4097))]))
        X = int(rng.choice([1, 2, 9, 33, 65, 70]))
        W = int(rng.integers(1, 4))
        step = int(rng.integers(0, 9))
        shift = int(rng.integers(0, 8))
        phase = int(rng.integers(0, 4))
        idx_h = rng.integers(-2, E + 2, size=(L, T, K)).astype(np.int32)
        if rng.random() < 0.5:                        # mostly valid counts, many replicas
            logcnt = rng.integers(1, X + 1, size=(L, E)).astype(np.int32)
        else:
            logcnt = rng.integers(-1, X + 2, size=(L, E)).astype(np.int32)
        log2phy = rng.integers(0, 1 << 20, size=(L, E, X)).astype(np.int32)
        ring_h = rng.integers(0, 1000, size=(W, L, E)).astype(np.int32)
        cnt, invl = ora.load_hist(idx_h, E)
        want = ora.redirect(idx_h, log2phy, logcnt)
        idx_d, l2p_d, cnt_d = gpu(idx_h), gpu(log2phy), gpu(logcnt)
        n = L * T * K
        big = torch.empty(n + 4, dtype=torch.int32, device=DEV)
        out = big[phase:phase + n].view(L, T, K)
        eplb.redirect(idx_d, l2p_d, cnt_d, out=out)
        torch.cuda.synchronize()
        assert_same(f"case {case} redirect", host(out), want)
        ring = gpu(ring_h)
        others = ring_h.astype(np.int64).sum(axis=0) - ring_h[step % W]
        load, bad, _ = eplb.hist_redirect(idx_d, E, ring, step, l2p_d, cnt_d, out=out)
        torch.cuda.synchronize()
        assert_same(f"case {case} fused redirect", host(out), want)
        assert_same(f"case {case} fused window", host(load), others + cnt)
        assert_same(f"case {case} fused invalid", host(bad), invl)
        ema_h = rng.integers(0, 1 << 40, size=(L, E)).astype(np.int64)
        ema, count, bad, _ = eplb.ema_redirect(idx_d, E, gpu(ema_h), shift, l2p_d, cnt_d, out=out)
        torch.cuda.synchronize()
        assert_same(f"case {case} fused ema redirect", host(out), want)
        assert_same(f"case {case} fused ema", host(ema), ora.ema_update(ema_h, cnt, shift).reshape(L, E))


@pytest.mark.parametrize("work", [wl.TINY_HIER, wl.DSV3_PREFILL], ids=lambda w: w.name)
def test_fused_serving_loop(work):
    """A serving loop: step s is redirected with the placement from the window
    before s (step 0 with the identity placement of the first rebalance of an
    all-zero window) and counted into the window; the placement is then
    recomputed.  Every output matches the oracle run the same way."""
    pl = work.placement
    L, E, W = work.layers, pl.E, work.window
    X = ora.max_count(pl.E, pl.P, pl.G, pl.N)
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
    """58 x 2^20 x 8 ids: whole-step counts against the oracle, and the
    redirect element by element against it on every layer."""
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
    for l in range(L):
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
