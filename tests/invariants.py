"""Properties every valid EPLB placement has, at any size.

Used on the oracle's output (to pin it) and on the HIP path's output at sizes
where the oracle is not run on every problem.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def effective(E, G, N):
    """(groups, nodes) the policy works with: (G, N) if N divides G, else (1, 1)."""
    return (G, N) if G % N == 0 else (1, 1)


def check_placement(w, phy2log, log2phy, logcnt, E, P, G, N, RK):
    """Assert the structural invariants of one problem's placement.

    * every logical expert has at least one replica and the counts sum to P;
    * phy2log holds every logical expert exactly logcnt[e] times;
    * log2phy[e, r] for r < logcnt[e] are e's physical ids, each once, and -1
      beyond the count;
    * per node: En originals' worth of experts and Pn physical slots; in the
      hierarchical case all experts of a group (and every replica of them) sit
      on one node, and each node holds exactly G/N groups;
    * replication within each node minimises the largest load per replica:
      max_e w[e]/logcnt[e] over the node equals the smallest M for which
      sum_e max(1, ceil(w[e]/M)) physical slots fit in the node (a feasibility
      threshold computed by bisection, independent of the greedy procedure).
    """
    Gp, Np = effective(E, G, N)
    phy2log = np.asarray(phy2log)
    log2phy = np.asarray(log2phy)
    logcnt = np.asarray(logcnt)
    X = log2phy.shape[1]
    assert phy2log.shape == (P,) and logcnt.shape == (E,)
    assert (logcnt >= 1).all(), "an expert lost all replicas"
    assert int(logcnt.sum()) == P
    assert ((phy2log >= 0) & (phy2log < E)).all()
    assert (np.bincount(phy2log, minlength=E) == logcnt).all()
    for e in range(E):
        c = int(logcnt[e])
        pids = log2phy[e, :c]
        assert (pids >= 0).all() and (pids < P).all()
        assert len(set(pids.tolist())) == c
        assert (phy2log[pids] == e).all()
        assert (log2phy[e, c:] == -1).all()
    Pn, En = P // Np, E // Np
    node_of_pid = np.arange(P) // Pn
    S = E // Gp
    nodes_of_expert = [set(node_of_pid[log2phy[e, :logcnt[e]]].tolist()) for e in range(E)]
    for e in range(E):
        assert len(nodes_of_expert[e]) == 1, "replicas of one expert span nodes"
    expert_node = np.array([next(iter(s)) for s in nodes_of_expert])
    for n in range(Np):
        assert int((expert_node == n).sum()) == En
    if Np > 1:
        per_node_groups = np.zeros(Np, dtype=int)
        for g in range(Gp):
            ns = set(expert_node[g * S:(g + 1) * S].tolist())
            assert len(ns) == 1, "a group spans nodes"
            per_node_groups[ns.pop()] += 1
        assert (per_node_groups == Gp // Np).all()
    # Replication optimality within a node (minimax threshold form).
    w = [int(x) for x in np.asarray(w).tolist()]
    for n in range(Np):
        members = [e for e in range(E) if expert_node[e] == n]
        got = max(Fraction(w[e], int(logcnt[e])) for e in members)
        assert got == minimax_load([w[e] for e in members], Pn)


def minimax_load(u, slots):
    """Smallest achievable max_i u_i / c_i over integer c_i >= 1, sum c_i = slots."""
    if all(x == 0 for x in u):
        return Fraction(0)
    extra = slots - len(u)
    cands = sorted({Fraction(x, k) for x in u if x > 0 for k in range(1, extra + 2)})

    def need(M):
        return sum(1 if x == 0 else max(1, -(-x * M.denominator // M.numerator)) for x in u)

    lo, hi = 0, len(cands) - 1          # cands[hi] (the largest u) is always feasible
    while lo < hi:
        mid = (lo + hi) // 2
        if need(cands[mid]) <= slots:
            hi = mid
        else:
            lo = mid + 1
    return cands[lo]


def gpu_loads(w, phy2log, logcnt, RK):
    """Exact load of each GPU: sum over its physical experts of load/count."""
    P = len(phy2log)
    ppr = P // RK
    return [sum(Fraction(int(w[phy2log[g * ppr + s]]), int(logcnt[phy2log[g * ppr + s]]))
                for s in range(ppr)) for g in range(RK)]
