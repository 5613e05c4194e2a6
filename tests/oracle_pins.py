"""Checks that pin the oracle to facts outside itself.

Each ``pin_*`` function raises AssertionError (or any exception) when the
oracle module ``o`` disagrees with what the pages print, with a closed form,
with brute force, or with an invariant.  ``test_oracle_pins.py`` runs them on
the real oracle; ``test_oracle_mutations.py`` plants plausible mistakes in the
oracle and shows that at least one pin fails for each.
"""
from __future__ import annotations

import itertools
import json
import os
from fractions import Fraction

import numpy as np

import invariants as inv

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))


def _example(o, groups=None, X=2):
    g = GOLDEN["inputs"]
    w = np.array(g["weight"], dtype=np.int64)
    return w, o.rebalance(w, g["num_replicas"], groups or g["num_groups"], g["num_nodes"], g["num_gpus"], X)


# ---------------------------------------------------------------- worked example

def pin_golden_phy2log(o):
    """The printed phy2log of both layers (hierarchical policy)."""
    _, r = _example(o)
    assert (r["status"] == 0).all()
    assert r["phy2log"].tolist() == GOLDEN["phy2log"]["value"]


def pin_golden_layer0(o):
    """Layer 0 walk-through: node contents, replicated experts, logcnt, log2phy."""
    w, r = _example(o)
    logcnt = r["logcnt"][0].tolist()
    assert logcnt == GOLDEN["layer0_logcnt"]["value"]
    assert r["maxlogcnt"] == 2
    phy = r["phy2log"][0]
    node0 = set(phy[:8].tolist())
    node1 = set(phy[8:].tolist())
    S = 3
    assert node0 == {e for g in GOLDEN["layer0_node_groups"]["node0_groups"] for e in range(g * S, g * S + S)}
    assert node1 == {e for g in GOLDEN["layer0_node_groups"]["node1_groups"] for e in range(g * S, g * S + S)}
    assert sorted(w[0][sorted(node0)].tolist()) and int(w[0][sorted(node0)].sum()) == 446
    assert int(w[0][sorted(node1)].sum()) == 587
    rep = GOLDEN["layer0_replicated"]
    assert {e for e in node0 if logcnt[e] == 2} == set(rep["node0"])
    assert {e for e in node1 if logcnt[e] == 2} == set(rep["node1"])
    l2p = GOLDEN["layer0_log2phy"]
    assert r["log2phy"][0, 0].tolist() == l2p["expert0"]
    assert r["log2phy"][0, 1].tolist() == l2p["expert1"]


def pin_golden_gpu_loads(o):
    """Per-GPU loads of layer 0: hierarchical 86.5..156 (mean ~129); global
    (num_groups = 3) 95.5..138.5."""
    w, r = _example(o)
    loads = inv.gpu_loads(w[0], r["phy2log"][0], r["logcnt"][0], 8)
    g = GOLDEN["layer0_gpu_load_hierarchical"]
    assert min(loads) == Fraction(g["min"]) and max(loads) == Fraction(g["max"])
    assert round(sum(loads) / len(loads)) == g["mean_rounded"]
    gg = GOLDEN["layer0_gpu_load_global_groups3"]
    w, r = _example(o, groups=gg["num_groups"], X=5)
    loads = inv.gpu_loads(w[0], r["phy2log"][0], r["logcnt"][0], 8)
    assert min(loads) == Fraction(gg["min"]) and max(loads) == Fraction(gg["max"])
    # without replication the hottest expert alone exceeds the balanced maximum
    hot = GOLDEN["layer0_no_replica_hot_gpu"]
    assert int(w[0][hot["expert"]]) == hot["load"] > max(loads)


def pin_dsv3_shape(o):
    """DeepSeek-V3 scale: 256 + 32 = 288 physical experts, 9 per GPU on 32 GPUs
    (hierarchical prefill); 144 GPUs on 18 nodes takes the global policy."""
    d = GOLDEN["dsv3_shape"]
    E, G, P = d["E"], d["G"], d["P"]
    assert E + d["redundant"] == P
    pre, dec = d["prefill"], d["decode"]
    assert P // pre["RK"] == pre["per_gpu"]
    assert o.policy(G, pre["N"])[2] == pre["hierarchical"]
    assert o.policy(G, dec["N"])[2] == dec["hierarchical"]
    rng = np.random.default_rng(7)
    w = rng.zipf(1.5, size=(2, E)).astype(np.int64) * 3
    for N, RK in ((pre["N"], pre["RK"]), (dec["N"], dec["RK"])):
        X = 1 + (P - E) // (N if G % N == 0 else 1)
        r = o.rebalance(w, P, G, N, RK, X)
        for b in range(2):
            inv.check_placement(w[b], r["phy2log"][b], r["log2phy"][b], r["logcnt"][b], E, P, G, N, RK)
            phy = r["phy2log"][b]
            assert all(len(phy[k * (P // RK):(k + 1) * (P // RK)]) == P // RK for k in range(RK))


# ---------------------------------------------------------------- replication

def pin_replication_bruteforce(o):
    """Greedy replication reaches the smallest possible max load per replica:
    brute force over every count vector for up to 5 experts and 6 replicas."""
    rng = np.random.default_rng(11)
    for trial in range(150):
        En = int(rng.integers(1, 6))
        Rn = int(rng.integers(0, 7))
        u = [int(x) for x in rng.integers(0, 40, size=En)]
        if trial % 5 == 0:
            u = [int(x) for x in rng.integers(0, 3, size=En)]     # many ties
        _, _, count = o.replicate(u, En + Rn)
        got = max(Fraction(u[i], count[i]) for i in range(En))
        best = None
        for extra in itertools.product(range(Rn + 1), repeat=En):
            if sum(extra) != Rn:
                continue
            m = max(Fraction(u[i], 1 + extra[i]) for i in range(En))
            best = m if best is None else min(best, m)
        assert got == best, (u, Rn, count)
        assert sum(count) == En + Rn and min(count) >= 1


def pin_replication_dhondt(o):
    """Closed form: the replicas are the Rn largest of the merged sequences
    {u_i / k : k >= 1} (D'Hondt apportionment), created in that order, with
    ties by lower expert index then lower k; replica rank is k."""
    rng = np.random.default_rng(12)
    for trial in range(200):
        En = int(rng.integers(1, 12))
        Rn = int(rng.integers(0, 20))
        hi = [3, 50, 10**6, 1 << 40][trial % 4]
        u = [int(x) for x in rng.integers(0, hi, size=En)]
        phy, rank, count = o.replicate(u, En + Rn)
        cands = [(Fraction(u[i], k), i, k) for i in range(En) for k in range(1, Rn + 1)]
        cands.sort(key=lambda c: (-c[0], c[1], c[2]))
        top = cands[:Rn]
        assert phy[En:] == [c[1] for c in top]
        assert rank[En:] == [c[2] for c in top]
        assert phy[:En] == list(range(En)) and rank[:En] == [0] * En
        assert count == [1 + sum(1 for c in top if c[1] == i) for i in range(En)]


# ---------------------------------------------------------------- packing

def pin_packing_closed_forms(o):
    """Special cases with closed forms.

    * one item per pack: identity;
    * one pack: everything in pack 0, positions in heaviest-first order;
    * m packs of q equal positive weights: item t -> pack t % m, position
      t // m; all-zero weights: item t -> pack t // q, position t % q;
    * 2m distinct positive weights into m packs of 2: the pack that takes the
      r-th heaviest item also takes the (2m-1-r)-th ("snake" pairing), and the
      r-th heaviest goes to pack r.
    """
    rng = np.random.default_rng(13)
    for n in (1, 3, 8):
        assert o.balanced_packing([int(x) for x in rng.integers(0, 9, n)], n) == (list(range(n)), [0] * n)
    ws = [5, 9, 9, 1, 7]
    pack, pos = o.balanced_packing(ws, 1)
    assert pack == [0] * 5 and pos == [3, 0, 1, 4, 2]
    for m, q in ((2, 2), (3, 4), (4, 3), (5, 5)):
        for val in (1, Fraction(7, 3)):
            pack, pos = o.balanced_packing([val] * (m * q), m)
            assert pack == [t % m for t in range(m * q)] and pos == [t // m for t in range(m * q)]
        # all-zero weights never separate the packs: each fills before the next
        pack, pos = o.balanced_packing([0] * (m * q), m)
        assert pack == [t // q for t in range(m * q)] and pos == [t % q for t in range(m * q)]
    for m in (2, 3, 5, 8):
        for _ in range(20):
            ws = [int(x) for x in rng.choice(10**6, size=2 * m, replace=False) + 1]
            pack, pos = o.balanced_packing(ws, m)
            order = sorted(range(2 * m), key=lambda i: -ws[i])
            for r in range(m):
                assert pack[order[r]] == r and pos[order[r]] == 0
                assert pack[order[2 * m - 1 - r]] == r and pos[order[2 * m - 1 - r]] == 1


def pin_identity_cases(o):
    """One item per pack is the identity, not a greedy pass.

    * G == N: group g goes to node g whatever its load;
    * P == RK (one physical expert per GPU): GPU k of a node holds the node's
      k-th physical expert: first the node's experts group by group in slot
      order, then the replicas in creation order (per-replica value
      non-increasing)."""
    rng = np.random.default_rng(14)
    w = rng.integers(0, 100, size=(3, 16))
    w[:, 12:] += 1000                                # group 3 heaviest: greedy would move it
    r = o.rebalance(w, 24, 4, 4, 8, 3)
    for b in range(3):
        for g in range(4):
            assert set(r["phy2log"][b][g * 6:(g + 1) * 6].tolist()) == set(range(g * 4, g * 4 + 4))
    r = o.rebalance(w, 24, 4, 2, 24, 5)
    for b in range(3):
        phy, cnt = r["phy2log"][b], r["logcnt"][b]
        inv.check_placement(w[b], phy, r["log2phy"][b], cnt, 16, 24, 4, 2, 24)
        for n in range(2):
            node = phy[n * 12:(n + 1) * 12].tolist()
            for s in range(2):
                blk = node[s * 4:(s + 1) * 4]
                assert blk[0] % 4 == 0 and blk == list(range(blk[0], blk[0] + 4))
            reps = node[8:]
            seen = {}
            vals = []
            for e in reps:
                seen[e] = seen.get(e, 0) + 1
                vals.append(Fraction(int(w[b][e]), seen[e]))
            assert vals == sorted(vals, reverse=True)
            assert all(cnt[e] == 1 + reps.count(e) for e in set(node))


def pin_degenerate_loads(o):
    """All-zero loads: every comparison ties, so groups fill node 0 first
    (groups 0, 1 on node 0; 2, 3 on node 1) and all redundant slots of a node
    go to its lowest node-local expert (experts 0 and 8).  All-equal positive loads: the first
    replica halves an expert's share, so the extras go one each to the lowest
    node-local experts; with 4 equal groups on 2 nodes, groups 0 and 2 land on
    node 0 and groups 1 and 3 on node 1 (ties to the lower node), so experts
    0-3 and 4-7 are the ones copied."""
    w = np.zeros((1, 16), dtype=np.int64)
    r = o.rebalance(w, 24, 4, 2, 8, 5)
    inv.check_placement(w[0], r["phy2log"][0], r["log2phy"][0], r["logcnt"][0], 16, 24, 4, 2, 8)
    assert r["logcnt"][0].tolist() == [5] + [1] * 7 + [5] + [1] * 7
    w = np.full((1, 16), 5, dtype=np.int64)
    r = o.rebalance(w, 24, 4, 2, 8, 5)
    inv.check_placement(w[0], r["phy2log"][0], r["log2phy"][0], r["logcnt"][0], 16, 24, 4, 2, 8)
    assert r["logcnt"][0].tolist() == [2] * 8 + [1] * 8
    w = np.zeros((1, 8), dtype=np.int64)
    r = o.rebalance(w, 12, 3, 2, 4, 5)                # global: expert 0 gets all 4 extras
    assert r["logcnt"][0].tolist() == [5, 1, 1, 1, 1, 1, 1, 1]


def pin_exact_arithmetic(o):
    """Loads near 2^30-2^40 that float32 cannot tell apart must still be
    ordered exactly.

    * 4 experts, one node, 2 GPUs of 2, no replicas: the snake pairing puts the
      heaviest and the lightest on GPU 0, the 2nd and 3rd on GPU 1, so
      phy2log = [1st, 4th, 2nd, 3rd] by exact weight;
    * 2 experts, 3 physical: the only replica goes to the exactly heavier one.
    """
    for hi in (1 << 30, (1 << 40) - 4096):
        w = np.array([[hi - 64, hi - 32, 5, 3], [hi - 32, hi - 64, 3, 5]], dtype=np.int64)
        r = o.rebalance(w, 4, 1, 1, 2, 1)
        assert r["phy2log"][0].tolist() == [1, 3, 0, 2]
        assert r["phy2log"][1].tolist() == [0, 2, 1, 3]
        w = np.array([[hi - 64, hi - 32], [hi - 32, hi - 64]], dtype=np.int64)
        r = o.rebalance(w, 3, 1, 1, 1, 2)
        assert r["logcnt"].tolist() == [[1, 2], [2, 1]]
    # replica loads w/3 vs w': (3*2^30 + 4)/3 > 2^30 + 1 exactly; in float32
    # both round to 2^30 and the lower index would win.
    w = np.array([[(1 << 30) + 1, 3 * (1 << 30) + 4, 1, 1]], dtype=np.int64)
    _, _, count = o.replicate([int(x) for x in w[0]], 6)
    assert count == [1, 3, 1, 1]
    r = o.rebalance(w, 6, 1, 1, 3, 3)
    # replica loads: e1 x3 at (3*2^30+4)/3 each, e0 at 2^30+1, e2 and e3 at 1;
    # heaviest-first: e1, e1, e1, e0, e2, e3.  The copies of e1 open GPUs 0,
    # 1, 2; e0 joins GPU 0 (three equal sums, lowest index); e2 and e3 fill
    # GPUs 1 and 2.
    assert r["phy2log"][0].tolist() == [1, 0, 1, 2, 1, 3]


def pin_invariants_random(o):
    """Structural invariants on random problems of many shapes, both policies."""
    rng = np.random.default_rng(15)
    shapes = [(16, 4, 2, 8, 24), (12, 4, 2, 8, 16), (12, 3, 2, 8, 16), (32, 8, 4, 8, 48),
              (24, 6, 4, 8, 32), (64, 4, 1, 8, 80), (20, 5, 5, 10, 30), (18, 9, 3, 3, 27)]
    for (E, G, N, RK, P) in shapes:
        Np = N if G % N == 0 else 1
        X = 1 + (P - E) // Np
        w = rng.integers(0, 1000, size=(4, E)) * rng.integers(0, 2, size=(4, E))
        r = o.rebalance(w, P, G, N, RK, X)
        assert (r["status"] == 0).all()
        for b in range(4):
            inv.check_placement(w[b], r["phy2log"][b], r["log2phy"][b], r["logcnt"][b], E, P, G, N, RK)


def pin_status_rules(o):
    """Loads outside [0, 2^40] mark the problem; so does a node whose exact
    common-denominator pack sums need 127 bits or more.  Marked problems are
    all -1.  The argument rules follow the pages' divisibility requirements."""
    w = np.array([[1, 2, 3, 4], [1, -1, 3, 4], [1, 2, 3, (1 << 40) + 1], [1, 2, 3, 1 << 40]], dtype=np.int64)
    r = o.rebalance(w, 6, 2, 1, 2, 3)
    assert r["status"].tolist() == [0, o.STATUS_BAD_LOAD, o.STATUS_BAD_LOAD, 0]
    assert (r["phy2log"][1] == -1).all() and (r["log2phy"][2] == -1).all() and (r["logcnt"][1] == -1).all()
    # Loads u_i = (i + 1) * V give final counts exactly i + 1 (every pick has
    # a value above V, every unpicked candidate equals V), so the node's
    # denominator is lcm(1..60) and its load sum is 1830 V.
    for V, want in (((1 << 40) // 60, o.STATUS_OVERFLOW), (1 << 30, 0)):
        from math import lcm
        E = 60
        P = E + sum(range(E))
        assert (lcm(*range(1, E + 1)) * V * P >= (1 << 127)) == (want != 0)
        w = np.array([[(i + 1) * V for i in range(E)]], dtype=np.int64)
        r = o.rebalance(w, P, 1, 1, 10, E)
        assert r["status"].tolist() == [want]
        if want == 0:
            assert r["logcnt"][0].tolist() == list(range(1, E + 1))
    assert o.argument_error(16, 24, 4, 2, 8, 5) is None
    assert o.argument_error(15, 24, 4, 2, 8, 5) == "div"        # groups do not divide experts
    assert o.argument_error(16, 24, 4, 2, 7, 5) == "div"        # GPUs not a multiple of nodes
    assert o.argument_error(16, 25, 4, 2, 8, 5) == "div"        # physical not a multiple of GPUs
    assert o.argument_error(16, 8, 4, 2, 8, 5) == "redundancy"
    assert o.argument_error(16, 24, 4, 2, 8, 4) == "capacity"   # 1 + (24 - 16) / 2 = 5 needed
    assert o.argument_error(15, 24, 3, 2, 8, 10) is None        # global path: E % G not required
    assert o.argument_error(15, 24, 3, 2, 8, 9) == "capacity"
    assert o.argument_error(0, 24, 4, 2, 8, 3) == "arg"


# ---------------------------------------------------------------- hist / window / redirect

def pin_hist_bruteforce(o):
    """Counts equal a plain loop's on small inputs, including out-of-range ids;
    per layer, counts plus invalid ids equal T*K."""
    rng = np.random.default_rng(16)
    for (L, T, K, E) in ((1, 1, 1, 1), (2, 7, 3, 5), (3, 50, 4, 16), (2, 0, 2, 4)):
        idx = rng.integers(-2, E + 2, size=(L, T, K)).astype(np.int32)
        cnt, bad = o.load_hist(idx, E)
        ref = [[0] * E for _ in range(L)]
        refbad = [0] * L
        for l in range(L):
            for t in range(T):
                for k in range(K):
                    e = int(idx[l, t, k])
                    if 0 <= e < E:
                        ref[l][e] += 1
                    else:
                        refbad[l] += 1
        assert cnt.tolist() == ref and bad.tolist() == refbad
        assert (cnt.sum(axis=1) + bad == T * K).all()


def pin_window(o):
    """The window is the sum of the last W per-step histograms (all of them
    while fewer than W exist)."""
    rng = np.random.default_rng(17)
    hs = [rng.integers(0, 9, size=(2, 5)) for _ in range(7)]
    for W in (1, 3, 7, 10):
        for s in range(1, 8):
            got = o.window_load(hs[:s], W)
            want = np.zeros((2, 5), dtype=np.int64)
            for h in hs[max(0, s - W):s]:
                want = want + h
            assert (got == want).all()


def pin_redirect(o):
    """Redirect: every output names a replica of the routed expert; replica r
    of expert e receives exactly the token rows t with t mod logcnt = r; the
    loop form and the vectorised form agree; invalid ids give -1."""
    w = np.array(GOLDEN["inputs"]["weight"], dtype=np.int64)
    r = o.rebalance(w, 16, 4, 2, 8, 3)
    rng = np.random.default_rng(18)
    idx = rng.integers(-1, 13, size=(2, 40, 3)).astype(np.int32)
    out = o.redirect(idx, r["log2phy"], r["logcnt"])
    assert out.tolist() == o.redirect_loop(idx.tolist(), r["log2phy"].tolist(), r["logcnt"].tolist())
    for l in range(2):
        for t in range(40):
            for k in range(3):
                e = int(idx[l, t, k])
                if not 0 <= e < 12:
                    assert out[l, t, k] == -1
                    continue
                p = int(out[l, t, k])
                assert r["phy2log"][l, p] == e
                c = int(r["logcnt"][l, e])
                assert list(r["log2phy"][l, e, :c]).index(p) == t % c


def pin_ema(o):
    """EMA: shift 0 keeps the latest counts; a plain loop agrees; from zero
    with constant counts c the estimate rises monotonically and settles where
    floor(e / 2^s) = c, i.e. in [c * 2^s, c * 2^s + 2^s); a hand-worked
    sequence for shift 2."""
    rng = np.random.default_rng(19)
    cnt = rng.integers(0, 1000, size=(3, 7))
    ema = rng.integers(0, 10**6, size=(3, 7))
    assert (o.ema_update(ema, cnt, 0).reshape(3, 7) == cnt).all()
    for s in (1, 3, 10):
        got = o.ema_update(ema, cnt, s).reshape(3, 7)
        want = [[int(ema[i, j]) - (int(ema[i, j]) >> s) + int(cnt[i, j]) for j in range(7)] for i in range(3)]
        assert got.tolist() == want
    for c, s in ((5, 2), (1000, 4), (0, 3), (1, 1)):
        e = np.zeros(1, dtype=np.int64)
        prev = -1
        for _ in range(400):
            e = o.ema_update(e, np.array([c]), s)
            assert int(e[0]) >= prev
            prev = int(e[0])
        assert c << s <= int(e[0]) < (c << s) + (1 << s) or (c == 0 and int(e[0]) == 0)
    e = np.zeros(1, dtype=np.int64)
    seq = []
    for c in (8, 8, 0, 4):
        e = o.ema_update(e, np.array([c]), 2)
        seq.append(int(e[0]))
    assert seq == [8, 14, 11, 13]      # 0-0+8; 8-2+8; 14-3+0; 11-2+4


def pin_placement_load(o):
    """Per-GPU loads of the worked example's layer 0: range 86.5..156, mean
    ~129 (hierarchical); 95.5..138.5 with num_groups = 3 (global); the sum of
    rank loads equals the total load; a bad map gives None."""
    w, r = _example(o)
    ranks, imb = o.placement_load(w, r["phy2log"], r["logcnt"], 8)
    g = GOLDEN["layer0_gpu_load_hierarchical"]
    assert min(ranks[0]) == Fraction(g["min"]) and max(ranks[0]) == Fraction(g["max"])
    assert round(sum(ranks[0]) / 8) == g["mean_rounded"]
    assert imb[0] == Fraction(g["max"]) / (Fraction(int(w[0].sum()), 8))
    for b in range(2):
        assert sum(ranks[b]) == int(w[b].sum())
    gg = GOLDEN["layer0_gpu_load_global_groups3"]
    w, r = _example(o, groups=gg["num_groups"], X=5)
    ranks, _ = o.placement_load(w, r["phy2log"], r["logcnt"], 8)
    assert min(ranks[0]) == Fraction(gg["min"]) and max(ranks[0]) == Fraction(gg["max"])
    bad = r["phy2log"].copy()
    bad[1, 3] = 12
    ranks, imb = o.placement_load(w, bad, r["logcnt"], 8)
    assert ranks[1] is None and imb[1] is None and ranks[0] is not None
    cnt0 = r["logcnt"].copy()
    cnt0[0, int(r["phy2log"][0, 0])] = 0
    assert o.placement_load(w, r["phy2log"], cnt0, 8)[1][0] is None
    for v in (-1, (1 << 40) + 1):
        wb = w.copy()
        wb[0, 5] = v
        assert o.placement_load(wb, r["phy2log"], r["logcnt"], 8)[1][0] is None
    wb = w.copy()
    wb[0, 5] = 1 << 40
    assert o.placement_load(wb, r["phy2log"], r["logcnt"], 8)[1][0] is not None
    z = np.zeros((1, 12), dtype=np.int64)
    rz = o.rebalance(z, 16, 4, 2, 8, 3)
    _, imb = o.placement_load(z, rz["phy2log"], rz["logcnt"], 8)
    assert imb[0] == 1


def _valid_l2p(new, E, X):
    """log2phy of a placement: slots of each expert in ascending order."""
    B, P = new.shape
    l2p = np.full((B, E, X), -1, dtype=np.int64)
    for b in range(B):
        seen = [0] * E
        for s in range(P):
            e = int(new[b, s])
            l2p[b, e, seen[e]] = s
            seen[e] += 1
    return l2p


def pin_rearrange_hand(o):
    """Two cases worked by hand.  (a) P=6, 2 ranks of 3, 2 nodes:
    old [0 1 2 | 3 4 0], new [2 0 0 | 4 1 3].  Rank 0 keeps 0 (slot 0, matched
    to new slot 1) and 2 (slot 2, new slot 0); the second 0 (new slot 2) goes
    to the freed slot 1 and is copied from slot 0 on the same rank.  Rank 1
    keeps 4 and 3; expert 1 goes to slot 5, copied from slot 1 on the other
    node.  (b) old [0 1 2 | 3 4 1], new [3 4 0 | 1 2 0]: two freed slots per
    rank, filled in ascending order (rank 0: 3 then 4 into slots 1, 2)."""
    r = o.rearrange_plan(np.array([[0, 1, 2, 3, 4, 0]]), np.array([[2, 0, 0, 4, 1, 3]]),
                         np.array([[[1, 2], [4, -1], [0, -1], [5, -1], [3, -1]]]), 2, 2)
    assert r["status"].tolist() == [0]
    assert r["phy2log"].tolist() == [[0, 0, 2, 3, 4, 1]]
    assert r["src"].tolist() == [[-1, 0, -1, -1, -1, 1]]
    assert r["moves"].tolist() == [[1, 0, 1]]
    assert r["log2phy"].tolist() == [[[0, 1], [5, -1], [2, -1], [3, -1], [4, -1]]]
    old, new = np.array([[0, 1, 2, 3, 4, 1]]), np.array([[3, 4, 0, 1, 2, 0]])
    l2p = np.array([[[2, 5], [3, -1], [4, -1], [0, -1], [1, -1]]])
    for N, moves in ((1, [0, 4, 0]), (2, [0, 0, 4])):
        r = o.rearrange_plan(old, new, l2p, 2, N)
        assert r["phy2log"].tolist() == [[0, 3, 4, 2, 0, 1]]
        assert r["src"].tolist() == [[-1, 3, 4, 2, 0, -1]]
        assert r["moves"].tolist() == [moves]
        assert r["log2phy"].tolist() == [[[0, 4], [5, -1], [3, -1], [1, -1], [2, -1]]]


def pin_rearrange_identity_and_permutation(o):
    """A placement against itself moves nothing; against a shuffle of its
    slots within each rank it moves nothing and the plan is the old one."""
    w, r = _example(o)
    p2l, l2p = r["phy2log"], r["log2phy"]
    q = o.rearrange_plan(p2l, p2l, l2p, 8, 2)
    assert (q["phy2log"] == p2l).all() and (q["log2phy"] == l2p).all()
    assert (q["src"] == -1).all() and (q["moves"] == 0).all() and (q["status"] == 0).all()
    rng = np.random.default_rng(4)
    shuf = p2l.copy()
    for b in range(2):
        for g in range(8):
            shuf[b, 2 * g:2 * g + 2] = rng.permutation(shuf[b, 2 * g:2 * g + 2])
    q = o.rearrange_plan(p2l, shuf, _valid_l2p(shuf, 12, 3), 8, 2)
    assert (q["phy2log"] == p2l).all() and (q["moves"] == 0).all() and (q["src"] == -1).all()


def _check_plan(o, old, new, RK, N, q):
    """Properties any correct plan has, each checked by brute force."""
    import itertools
    B, P = new.shape
    E = q["log2phy"].shape[1]
    ppr, per_node = P // RK, P // N
    for b in range(B):
        plan = q["phy2log"][b]
        for r in range(RK):
            sl = slice(r * ppr, (r + 1) * ppr)
            assert sorted(plan[sl].tolist()) == sorted(new[b, sl].tolist())      # within-rank permutation
        for e in range(E):
            got = sorted(x for x in q["log2phy"][b, e].tolist() if x >= 0)
            assert got == [s for s in range(P) if plan[s] == e]
        fetch = [0, 0, 0]
        for s in range(P):
            if q["src"][b, s] < 0:
                assert plan[s] == old[b, s]
                continue
            src = int(q["src"][b, s])
            holders = [x for x in range(P) if old[b, x] == plan[s]]
            assert src in holders
            classes = [[x for x in holders if x // ppr == s // ppr],
                       [x for x in holders if x // per_node == s // per_node], holders]
            cls = next(i for i, c in enumerate(classes) if c)
            assert src == min(classes[cls])
            fetch[cls] += 1
            if cls == 0:
                assert q["src"][b, src] == -1          # a same-rank source is kept, never overwritten
        assert q["moves"][b].tolist() == fetch
        # fewest fetches: ppr minus the multiset overlap of each rank
        from collections import Counter
        least = sum(ppr - sum((Counter(old[b, r * ppr:(r + 1) * ppr].tolist())
                               & Counter(new[b, r * ppr:(r + 1) * ppr].tolist())).values()) for r in range(RK))
        assert sum(fetch) == least
        if ppr <= 3 and RK <= 3:                       # and no within-rank permutation does better
            best = min(sum(int(a != c) for a, c in zip(sum((list(x) for x in combo), []), old[b].tolist()))
                       for combo in itertools.product(*[itertools.permutations(new[b, r * ppr:(r + 1) * ppr].tolist())
                                                       for r in range(RK)]))
            assert best == sum(fetch)


def pin_rearrange_properties(o):
    """Random old/new placements (every new expert present in the old one):
    within-rank permutation, consistent log2phy, sources hold the expert and
    are the lowest of the nearest class, fewest fetches (closed form, and
    brute force over all within-rank permutations on tiny cases)."""
    rng = np.random.default_rng(12)
    for trial in range(40):
        RK = int(rng.integers(1, 4)) if trial < 25 else int(rng.integers(2, 9))
        ppr = int(rng.integers(1, 4)) if trial < 25 else int(rng.integers(1, 7))
        N = int(rng.choice([d for d in range(1, RK + 1) if RK % d == 0]))
        P = RK * ppr
        E = int(rng.integers(1, P + 1))
        B = 3
        old = np.stack([rng.permutation(np.concatenate([np.arange(E), rng.integers(0, E, P - E)]))
                        for _ in range(B)])
        new = np.stack([rng.permutation(np.concatenate([np.arange(E), rng.integers(0, E, P - E)]))
                        for _ in range(B)])
        X = max(int(np.bincount(new[b], minlength=E).max()) for b in range(B))
        q = o.rearrange_plan(old, new, _valid_l2p(new, E, X), RK, N)
        assert (q["status"] == 0).all()
        _check_plan(o, old, new, RK, N, q)


def pin_rearrange_bad_maps(o):
    """Entries outside their ranges, or a new expert with no old replica:
    status 18 and every output of that problem -1; other problems unaffected."""
    old = np.array([[0, 1, 2, 3]] * 5)
    new = np.array([[1, 0, 3, 2]] * 5)
    l2p = _valid_l2p(new, 4, 1)
    old[1, 2] = 4
    new[2, 0] = -1
    l2p[3, 0, 0] = 4
    new[4, 0] = 1
    old[4, 1] = 0                                      # expert 1 no longer in the old placement
    q = o.rearrange_plan(old, new, l2p, 2, 1)
    assert q["status"].tolist() == [0, 18, 18, 18, 18]
    for k in ("phy2log", "log2phy", "src", "moves"):
        assert (q[k][1:] == -1).all()
    assert q["phy2log"][0].tolist() == [0, 1, 2, 3] and (q["src"][0] == -1).all()


def _lp_random(rng, RK, R, E, B=1, top=50, fill=0.7):
    """A random topology: home ranks, and replica slots filled with distinct
    experts (not on their own home rank, mostly)."""
    cnt = rng.integers(0, top, size=(B, E)).astype(np.int64)
    home = rng.integers(0, RK, size=(B, E)).astype(np.int64)
    rep = np.full((B, RK, R), -1, dtype=np.int64)
    for b in range(B):
        pool = list(rng.permutation(E))
        for g in range(RK):
            for j in range(R):
                if pool and rng.random() < fill:
                    rep[b, g, j] = pool.pop()
    return cnt, home, rep


def _lp_loads(cnt, home, rep, flow, RK):
    load = np.zeros(RK, dtype=np.int64)
    for e, c in enumerate(cnt):
        load[home[e]] += c
    for g in range(RK):
        for j in range(rep.shape[1]):
            x = rep[g, j]
            if x >= 0:
                load[home[x]] -= flow[g, j]
                load[g] += flow[g, j]
    return load


def pin_lp_closed_forms(o):
    """No replica: the largest home load.  Zero counts: 0.  Two ranks joined
    by one replica of rank 0's expert: ceil((a + b) / 2) when a >= b, else b.
    A capacity too small to balance: base minus the capacity.  Already even
    loads: no flow."""
    cnt = np.array([[5, 9, 1, 7]])
    home = np.array([[0, 1, 1, 2]])
    r = o.lp_solve(cnt, home, np.full((1, 3, 2), -1), 3)
    assert r["lam"].tolist() == [10] and (r["flow"] == 0).all() and r["rank_load"].tolist() == [[5, 10, 7]]
    r = o.lp_solve(np.zeros((1, 4), dtype=np.int64), home, np.array([[[1, -1], [0, -1], [2, -1]]]), 3)
    assert r["lam"].tolist() == [0] and (r["flow"] == 0).all()
    for a, b in ((10, 2), (11, 2), (3, 3), (2, 10), (0, 0), (1, 0), (7, 6)):
        r = o.lp_solve(np.array([[a, b]]), np.array([[0, 1]]), np.array([[[-1], [0]]]), 2)
        want = -(-(a + b) // 2) if a >= b else b
        assert r["lam"].tolist() == [want], (a, b, r["lam"])
        assert r["rank_load"].max() == want
    r = o.lp_solve(np.array([[10, 90, 0]]), np.array([[0, 0, 1]]), np.array([[[-1], [0]]]), 2)
    assert r["lam"].tolist() == [90] and r["flow"][0, 1, 0] == 10
    cnt = np.full((1, 8), 4)
    home = np.array([[0, 0, 1, 1, 2, 2, 3, 3]])
    rep = np.array([[[2, 5], [4, 7], [6, 1], [0, 3]]])
    r = o.lp_solve(cnt, home, rep, 4)
    assert r["lam"].tolist() == [8] and (r["flow"] == 0).all()


def pin_lp_subset_bound(o):
    """The optimum equals the supply-demand bound (Gale, 1957): the largest,
    over nonempty sets S of ranks, of ceil((load of S - capacity leaving S)
    / |S|) -- computed here by enumerating every S."""
    import itertools
    rng = np.random.default_rng(31)
    for trial in range(60):
        RK = int(rng.integers(1, 7))
        R = int(rng.integers(1, 4))
        E = int(rng.integers(RK, 4 * RK + 2))
        cnt, home, rep = _lp_random(rng, RK, R, E, top=int(rng.choice([3, 50, 10**6])))
        r = o.lp_solve(cnt, home, rep, RK)
        base = np.zeros(RK, dtype=np.int64)
        np.add.at(base, home[0], cnt[0])
        best = 0
        for k in range(1, RK + 1):
            for S in itertools.combinations(range(RK), k):
                S = set(S)
                out_cap = sum(int(cnt[0, x]) for g in range(RK) if g not in S for x in rep[0, g]
                              if x >= 0 and home[0, x] in S)
                v = sum(int(base[i]) for i in S) - out_cap
                best = max(best, -(-v // k))
        assert r["lam"][0] == best, (trial, r["lam"][0], best)


def pin_lp_linprog(o):
    """The same linear program in real numbers (scipy's HiGHS): its optimum
    lies within one token below the integer optimum."""
    from scipy.optimize import linprog
    rng = np.random.default_rng(32)
    for trial in range(30):
        RK = int(rng.integers(2, 9))
        R = int(rng.integers(1, 3))
        E = 4 * RK
        cnt, home, rep = _lp_random(rng, RK, R, E, top=1000)
        r = o.lp_solve(cnt, home, rep, RK)
        edges = [(int(home[0, x]), g, int(cnt[0, x])) for g in range(RK) for x in rep[0, g] if x >= 0]
        base = np.zeros(RK)
        np.add.at(base, home[0], cnt[0])
        n = len(edges)
        c = np.zeros(n + 1)
        c[-1] = 1.0
        A = np.zeros((RK, n + 1))
        for i, (src, dst, _) in enumerate(edges):
            A[src, i] -= 1.0
            A[dst, i] += 1.0
        A[:, -1] = -1.0
        bounds = [(0, cap) for _, _, cap in edges] + [(0, None)]
        res = linprog(c, A_ub=A, b_ub=-base, bounds=bounds, method="highs")
        assert res.status == 0
        lam_f = res.fun
        assert lam_f - 1e-6 <= r["lam"][0] < lam_f + 1 + 1e-6, (trial, lam_f, r["lam"][0])


def pin_lp_bruteforce(o):
    """Tiny cases: every integer flow tried; the least largest load matches,
    and the returned flows reach it within their capacities."""
    import itertools
    rng = np.random.default_rng(33)
    for trial in range(40):
        RK = int(rng.integers(2, 4))
        cnt, home, rep = _lp_random(rng, RK, 1, RK + 2, top=6, fill=0.8)
        r = o.lp_solve(cnt, home, rep, RK)
        slots = [(g, j) for g in range(RK) for j in range(1) if rep[0, g, j] >= 0]
        best = None
        for fl in itertools.product(*[range(int(cnt[0, rep[0, g, j]]) + 1) for g, j in slots]):
            flow = np.zeros((RK, 1), dtype=np.int64)
            for (g, j), f in zip(slots, fl):
                flow[g, j] = f
            m = int(_lp_loads(cnt[0], home[0], rep[0], flow, RK).max())
            best = m if best is None else min(best, m)
        assert r["lam"][0] == best


def pin_lp_flows_valid(o):
    """Flows between 0 and the replicated expert's count (0 on empty slots),
    loads recomputed from them equal the returned ones, and the largest is
    the optimum; several replicas per rank pair share the pair's flow."""
    rng = np.random.default_rng(34)
    for trial in range(40):
        RK = int(rng.integers(2, 9))
        R = int(rng.integers(1, 5))
        cnt, home, rep = _lp_random(rng, RK, R, 6 * RK, B=2, top=int(rng.choice([5, 1000])), fill=0.9)
        r = o.lp_solve(cnt, home, rep, RK)
        for b in range(2):
            f = r["flow"][b]
            assert (f >= 0).all() and (f[rep[b] < 0] == 0).all()
            assert all(f[g, j] <= cnt[b, rep[b, g, j]] for g in range(RK) for j in range(R) if rep[b, g, j] >= 0)
            load = _lp_loads(cnt[b], home[b], rep[b], f, RK)
            assert load.tolist() == r["rank_load"][b].tolist()
            assert load.max() == r["lam"][b] and load.sum() == cnt[b].sum()


def pin_lp_redirect(o):
    """Against a plain loop: occurrences of an expert counted in (token, k)
    order, the first f to the replica; exactly min(f, count) ids move."""
    rng = np.random.default_rng(35)
    E, RK, R = 12, 3, 2
    rep = np.array([[[4, -1], [0, 7], [-1, 11]], [[-1, -1], [3, -1], [5, 2]]])
    flow = np.array([[[3, 0], [5, 0], [0, 100]], [[0, 0], [1, 0], [0, 2]]])
    idx = rng.integers(-1, E + 1, size=(2, 50, 3)).astype(np.int32)
    got = o.lp_redirect(idx, rep, flow, E)
    for l in range(2):
        seen = {}
        slot = {int(rep[l, g, j]): (g, j) for g in range(RK) for j in range(R) if rep[l, g, j] >= 0}
        for t in range(50):
            for k in range(3):
                e = int(idx[l, t, k])
                if not (0 <= e < E):
                    assert got[l, t, k] == -1
                    continue
                i = seen.get(e, 0)
                seen[e] = i + 1
                if e in slot and i < flow[l][slot[e]]:
                    assert got[l, t, k] == E + slot[e][0] * R + slot[e][1]
                else:
                    assert got[l, t, k] == e
        for x, (g, j) in slot.items():
            moved = int((got[l] == E + g * R + j).sum())
            assert moved == min(int(flow[l, g, j]), int((idx[l] == x).sum()))
    bad = rep.copy()
    bad[0, 0, 1] = 0                                  # expert 0 twice in layer 0
    bad[1, 0, 0] = E                                  # an id out of range in layer 1
    got = o.lp_redirect(idx, bad, flow, E)
    assert (got == -1).all()


def pin_lp_status(o):
    """An id, home or count out of range, or an expert with two replicas:
    status 19 and every output -1; other problems unaffected."""
    cnt = np.array([[5, 1, 2, 0]] * 6)
    home = np.array([[0, 1, 1, 0]] * 6)
    rep = np.array([[[1, -1], [0, -1]]] * 6)
    cnt[1, 2] = -1
    cnt[2, 2] = (1 << 40) + 1
    home[3, 0] = 2
    rep[4, 0, 1] = 4
    rep[5, 0, 1] = 0                                    # expert 0 twice
    r = o.lp_solve(cnt, home, rep, 2)
    assert r["status"].tolist() == [0, 19, 19, 19, 19, 19]
    assert (r["lam"][1:] == -1).all() and (r["flow"][1:] == -1).all() and (r["rank_load"][1:] == -1).all()
    assert r["lam"][0] == 4


ALL_PINS = [pin_golden_phy2log, pin_golden_layer0, pin_golden_gpu_loads, pin_dsv3_shape,
            pin_replication_bruteforce, pin_replication_dhondt, pin_packing_closed_forms,
            pin_identity_cases, pin_degenerate_loads, pin_exact_arithmetic, pin_invariants_random,
            pin_status_rules,
            pin_hist_bruteforce, pin_window, pin_redirect, pin_ema, pin_placement_load,
            pin_rearrange_hand, pin_rearrange_identity_and_permutation, pin_rearrange_properties,
            pin_rearrange_bad_maps, pin_lp_closed_forms, pin_lp_subset_bound, pin_lp_linprog, pin_lp_bruteforce,
            pin_lp_flows_valid, pin_lp_redirect, pin_lp_status]
