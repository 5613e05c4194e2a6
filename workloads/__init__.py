"""Seeded synthetic workloads for the EPLB hot path.

This module only draws inputs: routing ids and load vectors.  It holds none of
the load balancer's arithmetic, and both the oracle's tests and the HIP path's
tests and benchmark read the same bytes from it.

Seeds: every buffer comes from ``numpy.random.SeedSequence(ROOT_SEED,
spawn_key=(workload_id, layer, step))`` with the PCG64 bit generator (or, for
the device-generated streaming workload, a torch generator seeded from that
same sequence), so a (workload, layer, step) triple always yields the same
bytes.

Shapes follow the DeepSeek-V3 deployment the pages describe (256 routed
experts per layer in 8 groups, 32 redundant experts, 4 prefill nodes of 8 GPUs,
a decode deployment that takes the global policy) and the worked example of
the EPLB README translation.  There are no routing traces in this repository;
these distributions stand in for them.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

ROOT_SEED = 0xE91B


@dataclass(frozen=True)
class Placement:
    """Placement shape: logical experts E in G groups, P physical experts on
    RK ranks (EP GPUs) spread over N nodes."""
    E: int
    G: int
    N: int
    RK: int
    P: int


@dataclass(frozen=True)
class Workload:
    """One named workload.  ``routing`` selects the id distribution."""
    name: str
    wid: int                       # seed namespace
    layers: int                    # problems for the rebalance
    placement: Placement
    tokens: int = 0                # T per step
    topk: int = 0                  # K
    window: int = 1                # W steps summed into the load
    routing: str = ""              # "dirichlet", "zipf_distinct", "zipf_iid", "hot_zipf"
    param: float = 0.0             # Dirichlet alpha or Zipf exponent
    extra: dict = field(default_factory=dict)


# The five workloads the hot path is measured and checked on.
TINY_HIER = Workload(
    name="tiny_hier_e16_p24_2x4", wid=0, layers=2,
    placement=Placement(E=16, G=4, N=2, RK=8, P=24),
    tokens=4096, topk=2, window=1, routing="dirichlet", param=0.5)

DSV3_PREFILL = Workload(
    name="dsv3_prefill_58L_e256_p288_4x8", wid=1, layers=58,
    placement=Placement(E=256, G=8, N=4, RK=32, P=288),
    tokens=16384, topk=8, window=10, routing="zipf_distinct", param=1.1)

GLOBAL_DECODE = Workload(
    name="global_decode_58L_e256_p320_5x8", wid=2, layers=58,
    placement=Placement(E=256, G=8, N=5, RK=40, P=320),
    tokens=2048, topk=8, window=32, routing="zipf_distinct", param=1.3)

STREAM_1M = Workload(
    name="stream_58L_1Mtok_top8_e256_p288", wid=3, layers=58,
    placement=Placement(E=256, G=8, N=4, RK=32, P=288),
    tokens=1 << 20, topk=8, window=10, routing="zipf_iid", param=1.1)

SKEWED_1024 = Workload(
    name="skewed_1024x_e512_p640_8x8", wid=4, layers=1024,
    placement=Placement(E=512, G=16, N=8, RK=64, P=640),
    routing="hot_zipf", param=1.0,
    extra={"model_layers": 64, "snapshots": 16, "tokens": 1 << 20, "hot_share": 0.3})

WORKLOADS = {w.name: w for w in (TINY_HIER, DSV3_PREFILL, GLOBAL_DECODE, STREAM_1M, SKEWED_1024)}

# Extra placement shapes used by the parity tests.
DSV3_DECODE_144 = Placement(E=256, G=8, N=18, RK=144, P=288)   # global policy, 2 per GPU
WORKED_EXAMPLE = Placement(E=12, G=4, N=2, RK=8, P=16)


def rng_for(wid: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(ROOT_SEED, spawn_key=(wid, *key))))


def seed64(wid: int, *key: int) -> int:
    """A 63-bit seed for a non-numpy generator, from the same seed tree."""
    ss = np.random.SeedSequence(ROOT_SEED, spawn_key=(wid, *key))
    return int(ss.generate_state(1, np.uint64)[0]) & ((1 << 63) - 1)


def zipf_probs(E: int, s: float, perm: np.ndarray) -> np.ndarray:
    """p[e] proportional to (perm[e] + 1) ** -s: expert e has popularity rank perm[e]."""
    ranks = perm.astype(np.float64) + 1.0
    p = ranks ** (-s)
    return p / p.sum()


def layer_probs(wl: Workload, layer: int) -> np.ndarray:
    """The per-layer expert popularity of a routing workload (fixed across steps)."""
    E = wl.placement.E
    rng = rng_for(wl.wid, layer)
    if wl.routing == "dirichlet":
        return rng.dirichlet(np.full(E, wl.param))
    perm = rng.permutation(E)
    return zipf_probs(E, wl.param, perm)


def draw_ids(rng: np.random.Generator, p: np.ndarray, T: int, K: int, distinct: bool) -> np.ndarray:
    """T x K int32 expert ids from categorical p.

    With ``distinct`` every token's K ids differ (top-k routing never picks an
    expert twice for one token): ids are drawn i.i.d., and an id equal to one
    at an earlier position of its token is drawn again, round after round,
    until the token has no repeat.
    """
    cdf = np.cumsum(p)
    cdf[-1] = 1.0
    E = p.size

    def sample(n):
        u = rng.random(n)
        return np.minimum(np.searchsorted(cdf, u, side="right"), E - 1).astype(np.int32)

    ids = sample(T * K).reshape(T, K)
    if distinct:
        assert K <= int((p > 0).sum())
        rows = np.arange(T)
        while rows.size:
            sub = ids[rows]
            dup = np.zeros(sub.shape, dtype=bool)
            for k in range(1, K):
                dup[:, k] = (sub[:, :k] == sub[:, k:k + 1]).any(axis=1)
            n = int(dup.sum())
            if n == 0:
                break
            sub[dup] = sample(n)
            ids[rows] = sub
            rows = rows[dup.any(axis=1)]
    return ids


def routing_step(wl: Workload, step: int, layers: range | None = None, tokens: int | None = None) -> np.ndarray:
    """Routing ids [L, T, K] int32 of one step (host, numpy)."""
    layers = range(wl.layers) if layers is None else layers
    T = wl.tokens if tokens is None else tokens
    out = np.empty((len(layers), T, wl.topk), dtype=np.int32)
    distinct = wl.routing in ("dirichlet", "zipf_distinct")
    for i, l in enumerate(layers):
        p = layer_probs(wl, l)
        out[i] = draw_ids(rng_for(wl.wid, l, step), p, T, wl.topk, distinct)
    return out


def routing_step_device(wl: Workload, step: int, device, out=None):
    """Routing ids [L, T, K] int32 of one step, drawn on the GPU with torch.

    Used for the streaming workload (58 x 2^20 x 8 ids per step), too large to
    draw on the host at benchmark speed.  Ids are i.i.d. per (token, k) (repeats
    allowed), by inverse-CDF lookup of uniform draws in the layer's Zipf CDF.
    """
    import torch
    L, T, K, E = wl.layers, wl.tokens, wl.topk, wl.placement.E
    if out is None:
        out = torch.empty((L, T, K), dtype=torch.int32, device=device)
    for l in range(L):
        p = layer_probs(wl, l)
        cdf = torch.tensor(np.cumsum(p), dtype=torch.float64, device=device)
        cdf[-1] = 1.0
        g = torch.Generator(device=device)
        g.manual_seed(seed64(wl.wid, l, step))
        u = torch.rand(T * K, generator=g, device=device, dtype=torch.float64)
        r = torch.searchsorted(cdf, u, right=True).clamp_(max=E - 1)
        out[l].view(-1).copy_(r.to(torch.int32))
    return out


def skewed_loads(wl: Workload = SKEWED_1024, problems: range | None = None) -> np.ndarray:
    """Loads [B, E] int64 of the skewed batch.

    Problem b is snapshot b % 16 of model layer b // 16.  Each layer has one hot
    expert holding round(0.3 * 2^20) tokens in every snapshot; the other
    2^20 - that tokens fall multinomially on the remaining experts with Zipf(1.0)
    popularity over a per-layer permutation.
    """
    E = wl.placement.E
    snaps = wl.extra["snapshots"]
    total = wl.extra["tokens"]
    hot_tok = int(round(wl.extra["hot_share"] * total))
    problems = range(wl.layers) if problems is None else problems
    out = np.zeros((len(problems), E), dtype=np.int64)
    for i, b in enumerate(problems):
        layer, snap = divmod(b, snaps)
        lrng = rng_for(wl.wid, layer)
        hot = int(lrng.integers(E))
        others = np.array([e for e in range(E) if e != hot])
        p = zipf_probs(E - 1, wl.param, lrng.permutation(E - 1))
        counts = rng_for(wl.wid, layer, snap).multinomial(total - hot_tok, p)
        out[i, others] = counts
        out[i, hot] = hot_tok
    return out


# ---------------------------------------------------------------- LPLB-style redistribution
# The 8-GPU cube of the LPLB usage example (its r2o table): slot j of rank g
# holds a replica of an expert whose original lives on rank CUBE_R2O[g][j].
CUBE_R2O = ((3, 6), (0, 7), (1, 4), (2, 5), (7, 0), (4, 1), (5, 2), (6, 3))


def hypercube_r2o(RK: int) -> tuple:
    """Rank g's slot d replicates an expert of rank g xor 2^d (no diagonals)."""
    dims = RK.bit_length() - 1
    assert 1 << dims == RK
    return tuple(tuple(g ^ (1 << d) for d in range(dims)) for g in range(RK))


def torus_r2o(nodes: int, per_node: int) -> tuple:
    """Torus over `nodes` nodes of `per_node` GPUs (rank n * per_node + g):
    slot 0 of a rank replicates an expert of the previous GPU of its node,
    slot 1 one of the same GPU of the previous node, so every GPU has one
    expert copied onto a neighbour in its node and one onto a GPU of the
    next node."""
    out = []
    for n in range(nodes):
        for g in range(per_node):
            out.append((n * per_node + (g - 1) % per_node, ((n - 1) % nodes) * per_node + g))
    return tuple(out)


@dataclass
class LpWorkload:
    """Per-batch redistribution inputs: ids of one batch per layer, experts
    in contiguous blocks per rank, replica slots named by an r2o table."""
    name: str
    wid: int
    layers: int
    E: int
    RK: int
    r2o: tuple
    tokens: int
    topk: int
    param: float                   # Zipf exponent of the per-layer popularity


LPLB_CUBE = LpWorkload(name="lplb_cube_58L_e256_8x2", wid=5, layers=58, E=256, RK=8, r2o=CUBE_R2O,
                       tokens=16384, topk=8, param=1.1)
LPLB_HYPERCUBE = LpWorkload(name="lplb_hypercube_58L_e256_16x4", wid=6, layers=58, E=256, RK=16,
                            r2o=hypercube_r2o(16), tokens=16384, topk=8, param=1.1)
LPLB_TORUS = LpWorkload(name="lplb_torus_58L_e256_4x8x2", wid=7, layers=58, E=256, RK=32, r2o=torus_r2o(4, 8),
                        tokens=16384, topk=8, param=1.1)


def lp_inputs(w: LpWorkload, layers: range | None = None, tokens: int | None = None):
    """(idx [L][T][K] int32, home [L][E] int32, rep [L][RK][R] int32).

    Per layer: a Zipf popularity over a random permutation of the experts,
    T tokens x K distinct ids drawn from it; expert e's original on rank
    e // (E / RK); the slots that name rank o in r2o (in (g, j) order) take
    o's experts in order of decreasing popularity (ties: lower id), so the
    most popular experts of each rank have the replicas.
    """
    layers = range(w.layers) if layers is None else layers
    T = w.tokens if tokens is None else tokens
    per = w.E // w.RK
    R = len(w.r2o[0])
    idx = np.empty((len(layers), T, w.topk), dtype=np.int32)
    home = np.empty((len(layers), w.E), dtype=np.int32)
    rep = np.full((len(layers), w.RK, R), -1, dtype=np.int32)
    for i, l in enumerate(layers):
        rng = rng_for(w.wid, l)
        p = zipf_probs(w.E, w.param, rng.permutation(w.E))
        idx[i] = draw_ids(rng_for(w.wid, l, 1), p, T, w.topk, distinct=True)
        home[i] = np.arange(w.E) // per
        nxt = {o: 0 for o in range(w.RK)}
        for g in range(w.RK):
            for j in range(R):
                o = w.r2o[g][j]
                mine = sorted(range(o * per, (o + 1) * per), key=lambda e: (-p[e], e))
                rep[i, g, j] = mine[nxt[o]]
                nxt[o] += 1
    return idx, home, rep


def zipf_loads(B: int, E: int, s: float, tokens: int, wid: int = 9) -> np.ndarray:
    """Generic loads [B, E] int64: multinomial token counts, Zipf(s) popularity."""
    out = np.zeros((B, E), dtype=np.int64)
    for b in range(B):
        rng = rng_for(wid, b)
        p = zipf_probs(E, s, rng.permutation(E))
        out[b] = rng.multinomial(tokens, p)
    return out


def sha256(a) -> str:
    """Digest of a buffer's bytes (logged next to every generated input)."""
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
