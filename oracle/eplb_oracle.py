"""Plain CPU oracle for the EPLB hot path.  TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call this module.  The product path (the HIP library
and its Python binding) never does, and this module imports nothing from it.

What it computes, and where the pages define it.  "The pages" are the web pages
on DeepSeek's Expert Parallelism Load Balancer; the authority is the Russian
translation page «DualPipe и EPLB: конвейер в обе стороны и балансировщик
экспертов» (ai.flicky.cc), Part 2 "EPLB", cited below as [EPLB-ru] plus the
section name:

* ``load_hist`` / ``window_load`` -- the load of a logical expert is the number
  of tokens the router sent to it during the observation period ([EPLB-ru],
  translator's glossary box "термины"); the predicted load is built from
  historical statistics over a window of steps ([EPLB-ru], opening section,
  "moving average" remark).  Here: integer counts, summed over the last W steps.
* ``balanced_packing``, ``replicate``, ``rebalance`` -- the three-step
  hierarchical policy and the global policy ([EPLB-ru] sections "Алгоритм",
  "Иерархическая балансировка", "Глобальная балансировка", the flowchart, and
  the appendix's three functions and entry point as described there), taken in
  the pages' order: groups -> nodes, replicas within a node, replicas -> GPUs.
* ``redirect`` -- each routed (token, k) goes to one physical replica of its
  logical expert; replica ``t mod logcnt`` of token row t.
* ``ema_update`` -- an integer exponential moving average of the per-step
  counts, the other reading of the opening section's "moving average".
* ``placement_load`` -- per-GPU load of a placement and its max / mean
  ([EPLB-ru], the translator's hands-on exercise 2 and the worked example).
* ``rearrange_plan`` -- the weight copies that turn one placement into the
  next; the pages are silent, so this follows a stated plain rule.
* ``lp_solve`` / ``lp_redirect`` -- LPLB-style per-batch redistribution of
  tokens over replica edges, and the redirect by its flows (the two LPLB
  pages; exact integer reading stated in ``lp_solve``).

Arithmetic: every value is an exact Python integer or ``fractions.Fraction``.
The pages compute replica loads and pack sums in float32; this oracle uses
exact rationals instead (readings R1 and R5 in the design notes), so the result
is the one the greedy procedure defines, with no rounding at all.

Readings of points the pages leave open (each is a design decision, stated once
more where it is used):
  * sorts are stable: equal weights keep ascending item index;
  * a tie between packs of equal sum goes to the lowest pack index;
  * a tie in "highest load per replica" goes to the lowest node-local index;
  * one item per pack is the identity assignment, not a greedy pass;
  * the global policy is the hierarchical one with one group and one node;
  * loads must lie in [0, 2**40]; outside that, the problem's status is
    STATUS_BAD_LOAD and all its outputs are -1;
  * if lcm(replica counts of a node) * (sum of that node's loads) >= 2**127 the
    problem's status is STATUS_OVERFLOW and all its outputs are -1 (the exact
    common-denominator pack sums would not fit 127 bits).
"""
from __future__ import annotations

from fractions import Fraction
from math import lcm

import numpy as np

LOAD_MAX = 1 << 40          # largest accepted load (tokens) of one logical expert
SUM_LIMIT = 1 << 127        # bound on lcm(counts) * node load sum

# Per-problem status values (the C header documents the same numbers).
STATUS_OK = 0
STATUS_BAD_LOAD = 16
STATUS_OVERFLOW = 17


# --------------------------------------------------------------------------
# Policy selection and argument rules
# --------------------------------------------------------------------------

def policy(num_groups: int, num_nodes: int) -> tuple[int, int, bool]:
    """Return (groups, nodes, hierarchical) for the policy the pages select.

    [EPLB-ru] "Алгоритм": the hierarchical policy is used when the number of
    nodes divides the number of expert groups; otherwise the global policy,
    which the flowchart and appendix entry point describe as the same routine
    run with a single group on a single node.
    """
    if num_groups % num_nodes == 0:
        return num_groups, num_nodes, True
    return 1, 1, False


def max_count(E: int, P: int, G: int, N: int) -> int:
    """Largest replica count the policy can give one logical expert.

    Within a node the replication step adds Pn - En = (P - E) / nodes
    replicas; at most all of them go to one expert, which then has 1 + that
    many copies ([EPLB-ru] appendix: the replication function's output width,
    and the entry point's log2phy sized by the largest count).  ``nodes`` is
    the policy's node count (1 on the global path).
    """
    _, Np, _ = policy(G, N)
    return 1 + (P - E) // Np


def argument_error(E: int, P: int, G: int, N: int, RK: int, X: int) -> str | None:
    """Name the first argument rule a rebalance call breaks, or None.

    Rules: every size positive; the divisibility requirements stated in the
    appendix functions' docstrings and checks (groups divide the experts on the
    hierarchical path, nodes divide the GPUs, GPUs divide the physical experts);
    no fewer physical than logical experts (the replication step adds a
    non-negative number of replicas); and a log2phy capacity X that can hold
    the largest count the policy can produce, 1 + (P - E) / nodes.
    """
    if min(E, P, G, N, RK, X) < 1:
        return "arg"
    Gp, Np, hier = policy(G, N)
    if hier and E % G != 0:
        return "div"
    if RK % Np != 0 or P % RK != 0:
        return "div"
    if P < E:
        return "redundancy"
    if X < 1 + (P - E) // Np:
        return "capacity"
    return None


# --------------------------------------------------------------------------
# The two greedy building blocks
# --------------------------------------------------------------------------

def balanced_packing(weights, num_packs: int) -> tuple[list[int], list[int]]:
    """Greedy balanced packing of n weighted items into num_packs packs.

    [EPLB-ru] appendix, first function as described in the translator's
    summary above it: every pack ends with exactly n / num_packs items; items
    are visited heaviest first and each goes into the lightest pack that still
    has room.  When each pack holds one item the assignment is the identity.

    ``weights`` are exact numbers (int or Fraction).  Returns, per item, the
    pack it went to and its position (arrival order) inside that pack.

    Readings: the heaviest-first order is a stable sort (equal weights keep
    ascending item index); among packs with room and equal sums the lowest
    pack index wins.
    """
    n = len(weights)
    assert num_packs >= 1 and n % num_packs == 0
    per_pack = n // num_packs
    if per_pack == 1:
        return list(range(n)), [0] * n

    order = sorted(range(n), key=lambda i: weights[i], reverse=True)
    # ``sorted(reverse=True)`` keeps equal keys in their original order, which
    # is the stable descending order used here.
    pack_sum = [0] * num_packs
    pack_len = [0] * num_packs
    pack_of = [-1] * n
    slot_of = [-1] * n
    for item in order:
        open_packs = [p for p in range(num_packs) if pack_len[p] < per_pack]
        target = min(open_packs, key=lambda p: (pack_sum[p], p))
        pack_of[item] = target
        slot_of[item] = pack_len[target]
        pack_sum[target] += weights[item]
        pack_len[target] += 1
    return pack_of, slot_of


def replicate(loads: list[int], num_phy: int) -> tuple[list[int], list[int], list[int]]:
    """Grow ``len(loads)`` logical experts to ``num_phy`` physical ones.

    [EPLB-ru] appendix, second function as summarised by the translator: each
    added replica goes to the expert whose load per replica (load / count) is
    currently highest.  Physical slot j < num_log is the original of expert j;
    slot num_log + r is the r-th replica created.  A replica's rank is the
    expert's count just before it was added (the original has rank 0).

    Reading: a tie in load per replica goes to the lowest index.
    Returns (phy2log, rank, count) for this subproblem.
    """
    num_log = len(loads)
    assert num_phy >= num_log
    count = [1] * num_log
    phy2log = list(range(num_log))
    rank = [0] * num_log
    for _ in range(num_phy - num_log):
        best = 0
        best_val = Fraction(loads[0], count[0])
        for i in range(1, num_log):
            val = Fraction(loads[i], count[i])
            if val > best_val:
                best, best_val = i, val
        phy2log.append(best)
        rank.append(count[best])
        count[best] += 1
    return phy2log, rank, count


# --------------------------------------------------------------------------
# One rebalance problem (one MoE layer or one load snapshot)
# --------------------------------------------------------------------------

def rebalance_problem(w: list[int], P: int, G: int, N: int, RK: int) -> dict:
    """Run the policy on one problem's logical loads ``w``.

    Returns a dict with ``status``, and for STATUS_OK also ``phy2log`` (P ints),
    ``phyrank`` (P ints) and ``logcnt`` (E ints).

    Steps, in the order [EPLB-ru] "Иерархическая балансировка" gives them:
      1. sum each group's loads and pack the groups onto the nodes, balanced;
         the experts are renumbered node by node ("mlog" order): expert
         g*S + j of a group placed on node n at slot s gets node-local index
         s*S + j;
      2. within each node, replicate experts greedily;
      3. the node's physical experts, each carrying its expert's load divided
         by the expert's final count, are packed onto the node's GPUs,
         balanced; physical id = node*Pn + gpu*ppr + position on the GPU.
    """
    E = len(w)
    if any((x < 0 or x > LOAD_MAX) for x in w):
        return {"status": STATUS_BAD_LOAD}
    Gp, Np, _ = policy(G, N)
    S = E // Gp                 # experts per group
    En = E // Np                # logical experts per node
    Pn = P // Np                # physical experts per node
    RKn = RK // Np              # GPUs per node
    ppr = P // RK               # physical experts per GPU
    groups_per_node = Gp // Np

    # Step 1: groups -> nodes.
    group_load = [sum(w[g * S:(g + 1) * S]) for g in range(Gp)]
    node_of_group, slot_of_group = balanced_packing(group_load, Np)
    mlog2log = [-1] * E
    for g in range(Gp):
        base = (node_of_group[g] * groups_per_node + slot_of_group[g]) * S
        for j in range(S):
            mlog2log[base + j] = g * S + j

    phy2log = [-1] * P
    phyrank = [-1] * P
    logcnt = [-1] * E
    for n in range(Np):
        # Step 2: replicas within node n.
        u = [w[mlog2log[n * En + i]] for i in range(En)]
        local_phy, local_rank, count = replicate(u, Pn)

        if lcm(*count) * sum(u) >= SUM_LIMIT:
            return {"status": STATUS_OVERFLOW}

        # Step 3: physical experts of node n -> its GPUs.
        per_replica = [Fraction(u[local_phy[j]], count[local_phy[j]]) for j in range(Pn)]
        gpu_of, pos_of = balanced_packing(per_replica, RKn)
        for j in range(Pn):
            pid = n * Pn + gpu_of[j] * ppr + pos_of[j]
            phy2log[pid] = mlog2log[n * En + local_phy[j]]
            phyrank[pid] = local_rank[j]
        for i in range(En):
            logcnt[mlog2log[n * En + i]] = count[i]
    return {"status": STATUS_OK, "phy2log": phy2log, "phyrank": phyrank, "logcnt": logcnt}


def rebalance(load, P: int, G: int, N: int, RK: int, X: int):
    """Batched rebalance: every row of ``load`` ([B, E] integers) is a problem.

    Returns numpy int32 arrays ``phy2log`` [B, P], ``log2phy`` [B, E, X],
    ``logcnt`` [B, E] and ``status`` [B], plus ``maxlogcnt`` (the largest
    count over all problems, the width the pages give log2phy).

    log2phy[b, e, r] is the physical id of the rank-r replica of expert e, and
    -1 for r >= logcnt[b, e] ([EPLB-ru] appendix entry point, and the
    translator's exercise on layer 0 of the example).  A problem whose status
    is not STATUS_OK has every output entry set to -1.
    """
    arr = np.asarray(load)
    B, E = arr.shape
    load = [[int(x) for x in row] for row in arr.tolist()]
    phy2log = np.full((B, P), -1, dtype=np.int32)
    log2phy = np.full((B, E, X), -1, dtype=np.int32)
    logcnt = np.full((B, E), -1, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    maxlogcnt = 0
    for b in range(B):
        res = rebalance_problem(load[b], P, G, N, RK)
        status[b] = res["status"]
        if res["status"] != STATUS_OK:
            continue
        phy2log[b] = res["phy2log"]
        logcnt[b] = res["logcnt"]
        maxlogcnt = max(maxlogcnt, max(res["logcnt"]))
        for pid in range(P):
            log2phy[b, res["phy2log"][pid], res["phyrank"][pid]] = pid
    return {"phy2log": phy2log, "log2phy": log2phy, "logcnt": logcnt,
            "status": status, "maxlogcnt": maxlogcnt}


# --------------------------------------------------------------------------
# Load statistics and redirect
# --------------------------------------------------------------------------

def load_hist(idx: np.ndarray, E: int) -> tuple[np.ndarray, np.ndarray]:
    """Per-layer token counts from top-k routing ids.

    ``idx`` is [L, T, K] (any integer dtype).  cnt[l, e] is the number of
    (t, k) with idx[l, t, k] == e, for 0 <= e < E ([EPLB-ru] glossary: the load
    is the tokens routed to the expert).  Ids outside [0, E) are not counted;
    invalid[l] says how many there were in layer l.
    """
    idx = np.asarray(idx)
    L = idx.shape[0]
    cnt = np.zeros((L, E), dtype=np.int64)
    invalid = np.zeros(L, dtype=np.int64)
    for l in range(L):
        flat = idx[l].reshape(-1).astype(np.int64)
        ok = (flat >= 0) & (flat < E)
        cnt[l] = np.bincount(flat[ok], minlength=E)
        invalid[l] = flat.size - int(ok.sum())
    return cnt, invalid


def window_load(step_hists: list[np.ndarray], W: int) -> np.ndarray:
    """Sum of the last W per-step histograms (fewer while fewer exist).

    The pages predict load from a moving average over history ([EPLB-ru]
    opening section); the placement only compares loads, and every comparison
    is unchanged by a common positive factor, so the windowed sum is used.
    """
    assert W >= 1 and len(step_hists) >= 1
    recent = step_hists[-W:]
    total = np.zeros_like(np.asarray(recent[0], dtype=np.int64))
    for h in recent:
        total += np.asarray(h, dtype=np.int64)
    return total


def redirect(idx: np.ndarray, log2phy: np.ndarray, logcnt: np.ndarray) -> np.ndarray:
    """Logical -> physical expert ids for every routed (token, k).

    out[l, t, k] = log2phy[l, e, t mod logcnt[l, e]] with e = idx[l, t, k], so
    the tokens of an expert with c replicas are spread over the c replicas by
    token row ([EPLB-ru] glossary: with two copies each gets about half).
    An id outside [0, E), or a count outside [1, X], gives -1.
    """
    idx = np.asarray(idx)
    L, T, K = idx.shape
    E, X = log2phy.shape[1], log2phy.shape[2]
    out = np.full((L, T, K), -1, dtype=np.int32)
    t = np.arange(T, dtype=np.int64)[:, None]
    for l in range(L):
        e = idx[l].astype(np.int64)
        ok_e = (e >= 0) & (e < E)
        e_safe = np.where(ok_e, e, 0)
        c = logcnt[l].astype(np.int64)[e_safe]
        ok = ok_e & (c >= 1) & (c <= X)
        r = np.where(ok, t % np.where(ok, c, 1), 0)
        vals = log2phy[l][e_safe, r]
        out[l] = np.where(ok, vals, -1)
    return out


def redirect_loop(idx, log2phy, logcnt) -> list:
    """Same as :func:`redirect`, as plain Python loops (for small inputs)."""
    L, T, K = len(idx), len(idx[0]), len(idx[0][0])
    E, X = len(log2phy[0]), len(log2phy[0][0])
    out = [[[-1] * K for _ in range(T)] for _ in range(L)]
    for l in range(L):
        for t in range(T):
            for k in range(K):
                e = int(idx[l][t][k])
                if 0 <= e < E:
                    c = int(logcnt[l][e])
                    if 1 <= c <= X:
                        out[l][t][k] = int(log2phy[l][e][t % c])
    return out


# --------------------------------------------------------------------------
# Load estimate by exponential moving average, and placement quality
# --------------------------------------------------------------------------

def ema_update(ema: np.ndarray, cnt: np.ndarray, shift: int) -> np.ndarray:
    """One step of an integer exponential moving average of the load.

    The pages predict load with a moving average over history ([EPLB-ru],
    opening section).  This variant keeps, per (layer, expert), an integer
    ema <- ema - floor(ema / 2^shift) + cnt, a decay of 1 - 2^-shift per step
    in exact integer arithmetic (steady state: about 2^shift x the per-step
    count).  shift = 0 keeps only the latest step.
    """
    ema = [int(x) for x in np.asarray(ema, dtype=np.int64).ravel().tolist()]
    cnt = [int(x) for x in np.asarray(cnt, dtype=np.int64).ravel().tolist()]
    out = [e - (e >> shift) + c for e, c in zip(ema, cnt)]
    return np.array(out, dtype=np.int64)


def placement_load(load, phy2log, logcnt, RK: int):
    """Exact load of every rank (GPU) under a placement, and max / mean.

    A rank's load is the sum over its physical experts of load[e] / logcnt[e]
    (each replica takes an equal share of its expert's tokens; [EPLB-ru]
    glossary), as in the translator's hands-on exercise 2 after the annotated
    source (add up weight / logcnt per GPU, compare max / mean between the
    policies) and the check of the worked example under "Интерфейс и пример".
    Returns (rank_loads as Fractions [B][RK], imbalance [B] as Fractions
    max / mean, 1 when every load is 0; both None for a problem whose maps name
    an expert outside [0, E) or a count below 1, or with a load outside
    [0, 2^40] as for the rebalance).
    """
    load = np.asarray(load)
    phy2log = np.asarray(phy2log)
    logcnt = np.asarray(logcnt)
    B, E = load.shape
    P = phy2log.shape[1]
    ppr = P // RK
    ranks, imb = [], []
    for b in range(B):
        w = [int(x) for x in load[b].tolist()]
        c = [int(x) for x in logcnt[b].tolist()]
        phy = [int(x) for x in phy2log[b].tolist()]
        if any(x < 0 or x > LOAD_MAX for x in w) or any(not (0 <= e < E) or c[e] < 1 for e in phy):
            ranks.append(None)
            imb.append(None)
            continue
        r = [sum((Fraction(w[phy[g * ppr + s]], c[phy[g * ppr + s]]) for s in range(ppr)), Fraction(0))
             for g in range(RK)]
        mean = Fraction(sum(w), RK)
        ranks.append(r)
        imb.append(Fraction(1) if mean == 0 else max(r) / mean)
    return ranks, imb


# --------------------------------------------------------------------------
# Rearrangement plan: from the placement in force to a new one
# --------------------------------------------------------------------------

STATUS_BAD_MAP = 18


def rearrange_plan(old_phy2log, new_phy2log, new_log2phy, RK: int, N: int) -> dict:
    """Which expert weights to copy where when a new placement replaces the
    one in force, keeping in place every replica that can stay.

    The pages stop at the placement: the rebalance assigns replicas to GPUs
    ([EPLB-ru], opening section and "Алгоритм") and says nothing of moving
    weights.  This plan takes the plainest route.  Positions within a rank
    (GPU) are interchangeable, so the new placement is kept rank for rank and
    only permuted inside each rank:

    * rank r holds slots [r*ppr, (r+1)*ppr), ppr = P / RK;
    * for each expert e, the first m old slots of the rank holding e stay
      (kept), m = min(copies of e in the old rank, copies in the new rank),
      matched in order to the first m new slots of the rank holding e;
    * the other new slots of the rank, in ascending order, take the other old
      slots of the rank (the freed ones), in ascending order;
    * a freed slot then fetches its new expert from an old slot holding it:
      one on the same rank if any (kept, so never overwritten), else one on
      the same node (node of slot s = s // (P / N)), else any; the lowest
      slot in that class.  Every source refers to the OLD placement.

    The number of fetches, ppr minus the multiset overlap per rank, is the
    least any within-rank permutation of the new placement allows.

    Returns int32 arrays: phy2log [B][P] (the new placement, permuted within
    ranks), log2phy [B][E][X] (the new log2phy through the same permutation,
    replica order kept), src [B][P] (old slot to copy from, -1 when the slot is
    kept), moves [B][3] (fetches from the same rank, the same node, another
    node), status [B] (STATUS_OK, or STATUS_BAD_MAP when an old or new entry
    lies outside [0, E), a log2phy entry outside [-1, P), or a new expert has
    no old replica; all outputs of such a problem are -1).
    """
    old_phy2log = np.asarray(old_phy2log)
    new_phy2log = np.asarray(new_phy2log)
    new_log2phy = np.asarray(new_log2phy)
    B, P = new_phy2log.shape
    E, X = new_log2phy.shape[1], new_log2phy.shape[2]
    ppr = P // RK
    per_node = P // N
    out = {"phy2log": np.full((B, P), -1, dtype=np.int32),
           "log2phy": np.full((B, E, X), -1, dtype=np.int32),
           "src": np.full((B, P), -1, dtype=np.int32),
           "moves": np.full((B, 3), -1, dtype=np.int32),
           "status": np.zeros(B, dtype=np.int32)}
    for b in range(B):
        old = [int(x) for x in old_phy2log[b].tolist()]
        new = [int(x) for x in new_phy2log[b].tolist()]
        l2p = [[int(x) for x in row] for row in new_log2phy[b].tolist()]
        if (any(not (0 <= e < E) for e in old + new) or any(not (-1 <= s < P) for row in l2p for s in row)
                or not set(new) <= set(old)):
            out["status"][b] = STATUS_BAD_MAP
            continue
        perm = [None] * P                       # new slot -> slot in the plan
        kept = [False] * P                      # old slot stays as it is
        for r in range(RK):
            slots = range(r * ppr, (r + 1) * ppr)
            used_old = set()
            matched_new = set()
            for e in sorted(set(new[s] for s in slots)):
                old_e = [s for s in slots if old[s] == e]
                new_e = [s for s in slots if new[s] == e]
                for q, p in zip(old_e, new_e):
                    perm[p] = q
                    kept[q] = True
                    used_old.add(q)
                    matched_new.add(p)
            freed = [s for s in slots if s not in used_old]
            waiting = [s for s in slots if s not in matched_new]
            for q, p in zip(freed, waiting):
                perm[p] = q
        plan = [None] * P
        for p in range(P):
            plan[perm[p]] = new[p]
        src = [-1] * P
        moves = [0, 0, 0]
        for s in range(P):
            if kept[s]:
                continue
            holders = [q for q in range(P) if old[q] == plan[s]]
            same_rank = [q for q in holders if q // ppr == s // ppr]
            same_node = [q for q in holders if q // per_node == s // per_node]
            if same_rank:
                src[s], cls = same_rank[0], 0
            elif same_node:
                src[s], cls = same_node[0], 1
            else:
                src[s], cls = holders[0], 2
            moves[cls] += 1
        out["phy2log"][b] = plan
        out["log2phy"][b] = [[perm[s] if s >= 0 else -1 for s in row] for row in l2p]
        out["src"][b] = src
        out["moves"][b] = moves
    return out


# --------------------------------------------------------------------------
# Per-batch redistribution over a fixed replica topology (LPLB-style)
# --------------------------------------------------------------------------

STATUS_BAD_TOPOLOGY = 19


def _lp_graph(cnt, home, rep, RK):
    """Rank loads before any move, and the capacity between ranks: a replica
    on rank g of expert x (home rank o) is an edge o -> g that can carry up
    to cnt[x] of x's tokens."""
    base = [0] * RK
    for e, c in enumerate(cnt):
        base[home[e]] += c
    cap = [[0] * RK for _ in range(RK)]
    for g in range(RK):
        for x in rep[g]:
            if x >= 0 and home[x] != g:
                cap[home[x]][g] += cnt[x]
    return base, cap


def _lp_network(base, cap, lam):
    """Residual capacities of the feasibility network for a bound lam:
    source -> r carries what r must shed (base - lam), r -> sink what r may
    still take (lam - base), and the rank edges their capacities."""
    RK = len(base)
    V = RK + 2
    s, t = RK, RK + 1
    r = [[0] * V for _ in range(V)]
    for v in range(RK):
        r[s][v] = max(0, base[v] - lam)
        r[v][t] = max(0, lam - base[v])
        for g in range(RK):
            if g != v:
                r[v][g] = cap[v][g]
    return r, s, t


def _max_flow(r, s, t):
    """Shortest augmenting paths (Edmonds and Karp, J. ACM 1972) on the
    residual matrix r, in place.  The search goes level by level from the
    source; a node's predecessor is the lowest-numbered node of the previous
    level with residual capacity to it, so the paths, and the flow, are one
    definite choice among the optimal ones.  Returns the flow value."""
    V = len(r)
    total = 0
    while True:
        parent = [-1] * V
        seen = [False] * V
        seen[s] = True
        frontier = [s]
        while frontier and not seen[t]:
            nxt = []
            for v in range(V):
                if seen[v]:
                    continue
                for u in frontier:                          # ascending
                    if r[u][v] > 0:
                        parent[v] = u
                        nxt.append(v)
                        break
            for v in nxt:
                seen[v] = True
            frontier = nxt
        if not seen[t]:
            return total
        b = None
        v = t
        while v != s:
            u = parent[v]
            b = r[u][v] if b is None else min(b, r[u][v])
            v = u
        v = t
        while v != s:
            u = parent[v]
            r[u][v] -= b
            r[v][u] += b
            v = u
        total += b


def lp_solve(cnt, home, rep, RK: int) -> dict:
    """Per-batch token redistribution over replica edges, exact.

    Two pages describe LPLB: «DeepSeek开源LPLB：基于线性规划的MoE负载均衡器…»
    (2048ai.net; items 4, 5 and 7: the replica topology r2o, the LP model and
    the typical topologies) and the Machine Heart report on LPLB
    (wwwcj777.com; section «LPLB 的工作原理»).  Each redundant expert links
    the GPU of its original to its own GPU; that edge can carry at most the
    tokens routed to the expert in the current batch; a linear program moves
    tokens along the edges to make the loads of the expert-parallel group as
    even as possible.  The pages do not write the program out; this reading
    minimises the largest rank load with whole tokens:

        minimise  lam  over integer flows 0 <= f[g][j] <= cnt[rep[g][j]]
        subject to  base[r] - (flows out of r) + (flows into r) <= lam

    where base[r] sums the batch counts of the experts whose original lives
    on rank r (home), and slot j of rank g holds a replica of rep[g][j]
    (-1: empty).  lam is the least integer for which a feasible flow exists
    (binary search, each bound tested by a maximum flow); the flows are those
    of the shortest-augmenting-path maximum flow at that lam, split over the
    replica slots of each rank pair in ascending slot order.

    cnt [B][E] int64 (0 .. 2^40), home [B][E] int32 in [0, RK), rep [B][RK][R]
    int32 (-1 or an expert id; an expert has at most one replica).
    Returns lam [B] int64, flow [B][RK][R] int64, rank_load [B][RK] int64,
    status [B] (STATUS_OK, or STATUS_BAD_TOPOLOGY for an id or count out of
    range or an expert replicated twice; outputs -1).
    """
    cnt = np.asarray(cnt)
    home = np.asarray(home)
    rep = np.asarray(rep)
    B, E = cnt.shape
    R = rep.shape[2]
    out = {"lam": np.full(B, -1, dtype=np.int64), "flow": np.full((B, RK, R), -1, dtype=np.int64),
           "rank_load": np.full((B, RK), -1, dtype=np.int64), "status": np.zeros(B, dtype=np.int32)}
    for b in range(B):
        c = [int(x) for x in cnt[b].tolist()]
        h = [int(x) for x in home[b].tolist()]
        rp = [[int(x) for x in row] for row in rep[b].tolist()]
        reps = [x for row in rp for x in row if x != -1]
        if (any(x < 0 or x > LOAD_MAX for x in c) or any(not (0 <= x < RK) for x in h)
                or any(not (0 <= x < E) for x in reps) or len(set(reps)) != len(reps)):
            out["status"][b] = STATUS_BAD_TOPOLOGY
            continue
        base, cap = _lp_graph(c, h, rp, RK)

        def feasible(lam):
            r, s, t = _lp_network(base, cap, lam)
            need = sum(r[s])
            return _max_flow(r, s, t) == need

        lo, hi = 0, max(base)                   # hi: no move needed
        while lo < hi:
            mid = (lo + hi) // 2
            if feasible(mid):
                hi = mid
            else:
                lo = mid + 1
        lam = lo
        r, s, t = _lp_network(base, cap, lam)
        _max_flow(r, s, t)
        # net flow on each rank pair, split over that pair's replica slots
        flow = [[0] * R for _ in range(RK)]
        load = list(base)
        for o in range(RK):
            for g in range(RK):
                if o == g:
                    continue
                net = max(0, cap[o][g] - r[o][g])
                for j in range(R):
                    x = rp[g][j]
                    if x >= 0 and h[x] == o and net > 0:
                        f = min(net, c[x])
                        flow[g][j] = f
                        net -= f
                        load[o] -= f
                        load[g] += f
        out["lam"][b] = lam
        out["flow"][b] = flow
        out["rank_load"][b] = load
    return out


def lp_redirect(idx, rep, flow, E: int) -> np.ndarray:
    """Physical expert of every routed (token, k) under the batch's flows.

    Physical ids: expert e's original is e; slot j of rank g is E + g*R + j
    (the LPLB planner of the usage example on «DeepSeek开源LPLB…» counts
    the logical experts plus the redundant ones per rank times the ranks).
    The occurrences of expert x in a layer, counted in (token, k) order, are
    numbered 0, 1, ...; the first f of them go to x's replica, f being that
    replica's flow, the rest stay with the original.  Ids outside [0, E)
    give -1, and so does every id of a layer whose rep names an id outside
    [0, E) or an expert twice (the topologies eplb_lp_solve rejects; the
    pages' planner never builds one).
    """
    idx = np.asarray(idx)
    rep = np.asarray(rep)
    flow = np.asarray(flow)
    L = idx.shape[0]
    RK, R = rep.shape[1], rep.shape[2]
    out = np.empty(idx.shape, dtype=np.int32)
    for l in range(L):
        named = [int(x) for x in rep[l].ravel().tolist() if x != -1]
        if any(not (0 <= x < E) for x in named) or len(set(named)) != len(named):
            out[l] = -1
            continue
        slot = np.full(E, -1, dtype=np.int64)
        fx = np.zeros(E, dtype=np.int64)
        for g in range(RK):
            for j in range(R):
                x = int(rep[l, g, j])
                if x >= 0:
                    slot[x] = E + g * R + j
                    fx[x] = int(flow[l, g, j])
        flat = idx[l].ravel().astype(np.int64)
        valid = (flat >= 0) & (flat < E)
        key = np.where(valid, flat, E)
        order = np.argsort(key, kind="stable")           # positions grouped by expert, in order
        sk = key[order]
        first = np.searchsorted(sk, sk, side="left")
        occ = np.empty_like(flat)
        occ[order] = np.arange(flat.size) - first
        e = np.where(valid, flat, 0)
        to_rep = valid & (slot[e] >= 0) & (occ < fx[e])
        res = np.where(to_rep, slot[e], flat)
        out[l] = np.where(valid, res, -1).reshape(idx.shape[1:])
    return out
