"""The serving step captured in HIP graphs and replayed (needs an MI355X).

The library allocates nothing and never synchronises, so its calls can be
recorded in a graph.  One graph per ring slot holds a serving step: count
step s into slot s % W and redirect it with the placement in force
(eplb_hist_redirect), then the rebalance that overwrites that placement for
the next step.  Every replay, with fresh ids copied into the captured input
buffer by ordinary eager work in between, must give outputs identical to the
same calls made eagerly on separate buffers, and to the oracle.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import eplb_oracle as ora

pytestmark = pytest.mark.gpu

eplb = pytest.importorskip("moe_expert_load_eplb_amd")
DEV = torch.device("cuda:0")


def note(msg: str) -> None:
    print(f"[graph] {msg}", flush=True)
    sys.stdout.flush()


class Loop:
    """Buffers of one serving loop (the placement is updated in place)."""

    def __init__(self, work, tokens, W):
        pl = work.placement
        L, K, E = work.layers, work.topk, pl.E
        self.E, self.pl, self.W = E, pl, W
        self.idx = torch.zeros((L, tokens, K), dtype=torch.int32, device=DEV)
        self.ring = torch.zeros((W, L, E), dtype=torch.int32, device=DEV)
        self.load = torch.zeros((L, E), dtype=torch.int64, device=DEV)
        self.bad = torch.zeros((L,), dtype=torch.int64, device=DEV)
        self.out = torch.zeros_like(self.idx)
        X = ora.max_count(pl.E, pl.P, pl.G, pl.N)
        # the placement in force before the first step: every expert once, in order, on a uniform load
        self.placement = eplb.rebalance(torch.ones((L, E), dtype=torch.int64, device=DEV), pl.P, pl.G, pl.N, pl.RK, X)

    def step(self, s):
        pl = self.pl
        eplb.hist_redirect(self.idx, self.E, self.ring, s, self.placement[1], self.placement[2],
                           self.load, self.bad, self.out)
        eplb.rebalance(self.load, pl.P, pl.G, pl.N, pl.RK, out=self.placement)

    def state(self):
        return [t.cpu().numpy().copy() for t in (self.out, self.load, self.bad, *self.placement)]


@pytest.mark.parametrize("work,tokens,W", [(wl.TINY_HIER, 4096, 3), (wl.DSV3_PREFILL, 2000, 4)],
                         ids=["tiny", "dsv3"])
def test_graph_replay_matches_eager(work, tokens, W):
    graph_loop = Loop(work, tokens, W)
    eager_loop = Loop(work, tokens, W)
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    graphs = []
    for slot in range(W):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            graph_loop.step(slot)
        graphs.append(g)
    torch.cuda.synchronize()
    # capture records the calls without running them: both loops start alike

    hists = []
    prev = [t.cpu().numpy().copy() for t in eager_loop.placement]
    for s in range(2 * W + 3):
        note(f"{work.name} step {s} (slot {s % W})")
        idx_h = wl.routing_step(work, s, tokens=tokens)
        graph_loop.idx.copy_(torch.from_numpy(idx_h))
        eager_loop.idx.copy_(torch.from_numpy(idx_h))
        graphs[s % W].replay()
        eager_loop.step(s)
        torch.cuda.synchronize()
        g, e = graph_loop.state(), eager_loop.state()
        for name, a, b in zip(("out", "load", "n_invalid", "phy2log", "log2phy", "logcnt", "status"), g, e):
            assert np.array_equal(a, b), f"step {s}: {name} differs between graph replay and eager"
        # and both against the oracle: redirect with the placement in force, window, new placement
        cnt, inv = ora.load_hist(idx_h, work.placement.E)
        hists.append(cnt)
        assert np.array_equal(g[0], ora.redirect(idx_h, prev[1], prev[2]))
        assert np.array_equal(g[1], ora.window_load(hists, W))
        ref = ora.rebalance(g[1], work.placement.P, work.placement.G, work.placement.N, work.placement.RK,
                            ora.max_count(work.placement.E, work.placement.P, work.placement.G, work.placement.N))
        assert np.array_equal(g[3], ref["phy2log"]) and np.array_equal(g[5], ref["logcnt"])
        prev = g[3:]


def test_concurrent_streams():
    """Calls on three streams at once (disjoint buffers; the library keeps no
    state) give the outputs of the same calls made one after another."""
    work = wl.DSV3_PREFILL
    pl = work.placement
    idx = torch.from_numpy(wl.routing_step(work, 0, tokens=2048)).to(DEV)
    loads = torch.from_numpy(wl.zipf_loads(58, pl.E, 1.1, 1 << 20)).to(DEV)
    sk = wl.SKEWED_1024.placement
    sk_loads = torch.from_numpy(wl.skewed_loads(wl.SKEWED_1024, range(256))).to(DEV)
    base = eplb.rebalance(loads, pl.P, pl.G, pl.N, pl.RK)

    def calls(ring):
        return eplb.hist_redirect(idx, pl.E, ring, 0, base[1], base[2])

    # one after another on the current stream
    ring0 = torch.zeros((2, 58, pl.E), dtype=torch.int32, device=DEV)
    want_a = [t.clone() for t in calls(ring0)]
    want_b = [t.clone() for t in eplb.rebalance(loads, pl.P, pl.G, pl.N, pl.RK)]
    want_c = [t.clone() for t in eplb.rebalance(sk_loads, sk.P, sk.G, sk.N, sk.RK)]
    torch.cuda.synchronize()
    for rep in range(5):
        note(f"three streams, round {rep}")
        streams = [torch.cuda.Stream(DEV) for _ in range(3)]
        for s in streams:
            s.wait_stream(torch.cuda.current_stream(DEV))
        ring = torch.zeros((2, 58, pl.E), dtype=torch.int32, device=DEV)
        torch.cuda.synchronize()
        with torch.cuda.stream(streams[0]):
            got_a = calls(ring)
        with torch.cuda.stream(streams[1]):
            got_b = eplb.rebalance(loads, pl.P, pl.G, pl.N, pl.RK)
        with torch.cuda.stream(streams[2]):
            got_c = eplb.rebalance(sk_loads, sk.P, sk.G, sk.N, sk.RK)
        torch.cuda.synchronize()
        for w, g in zip(want_a + want_b + want_c, list(got_a) + list(got_b) + list(got_c)):
            assert torch.equal(w, g)


def test_resume_from_saved_state():
    """The window ring, the step number and the placement in force are all
    the state a serving loop keeps (the library keeps none): saving them
    after step 3 and resuming in fresh buffers gives the outputs of the
    uninterrupted loop, step for step."""
    work, tokens, W = wl.DSV3_PREFILL, 3000, 4
    steps = [wl.routing_step(work, s, tokens=tokens) for s in range(8)]
    run = Loop(work, tokens, W)
    outs = []
    saved = None
    for s, idx_h in enumerate(steps):
        run.idx.copy_(torch.from_numpy(idx_h))
        run.step(s)
        torch.cuda.synchronize()
        outs.append(run.state())
        if s == 3:                              # checkpoint: host copies of the loop's state
            saved = (run.ring.cpu().clone(), [t.cpu().clone() for t in run.placement])
    resumed = Loop(work, tokens, W)
    resumed.ring.copy_(saved[0].to(DEV))
    for t, h in zip(resumed.placement, saved[1]):
        t.copy_(h.to(DEV))
    for s in range(4, len(steps)):
        note(f"resumed step {s}")
        resumed.idx.copy_(torch.from_numpy(steps[s]))
        resumed.step(s)
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "load", "n_invalid", "phy2log", "log2phy", "logcnt", "status"),
                              resumed.state(), outs[s]):
            assert np.array_equal(a, b), f"step {s}: {name} differs after resuming"
