"""The seeded input generators: determinism and the stated shapes (CPU only)."""
import numpy as np

import workloads as wl


def test_routing_deterministic_and_distinct():
    a = wl.routing_step(wl.TINY_HIER, 0)
    b = wl.routing_step(wl.TINY_HIER, 0)
    c = wl.routing_step(wl.TINY_HIER, 1)
    assert a.shape == (2, 4096, 2) and a.dtype == np.int32
    assert wl.sha256(a) == wl.sha256(b) != wl.sha256(c)
    assert ((a >= 0) & (a < 16)).all()
    assert (a[..., 0] != a[..., 1]).all()


def test_zipf_distinct_rows():
    x = wl.routing_step(wl.DSV3_PREFILL, 3, layers=range(2), tokens=512)
    s = np.sort(x, axis=2)
    assert not (s[..., 1:] == s[..., :-1]).any()
    # popularity follows the per-layer permutation: the most frequent expert is rank 0
    p = wl.layer_probs(wl.DSV3_PREFILL, 0)
    cnt = np.bincount(wl.routing_step(wl.DSV3_PREFILL, 0, layers=range(1), tokens=4096).ravel(), minlength=256)
    assert int(np.argmax(cnt)) == int(np.argmax(p))


def test_skewed_loads():
    x = wl.skewed_loads(problems=range(40))
    assert x.shape == (40, 512) and x.dtype == np.int64
    assert (x.sum(axis=1) == 1 << 20).all()
    hot = int(round(0.3 * (1 << 20)))
    assert ((x == hot).sum(axis=1) >= 1).all()
    # the 16 snapshots of one layer share the hot expert
    assert len({int(np.argmax(x[i])) for i in range(16)}) == 1


def test_placement_shapes():
    """The workloads' shapes take the policies the configurations name: the
    prefill shape hierarchical with up to 9 copies of an expert, the decode
    shapes global (8 groups on 5 and on 18 nodes), the skewed batch
    hierarchical with up to 17."""
    from oracle import eplb_oracle as ora
    pre, dec, d144, sk = (wl.DSV3_PREFILL.placement, wl.GLOBAL_DECODE.placement, wl.DSV3_DECODE_144,
                          wl.SKEWED_1024.placement)
    assert ora.policy(pre.G, pre.N)[2] and ora.max_count(pre.E, pre.P, pre.G, pre.N) == 9
    assert not ora.policy(dec.G, dec.N)[2] and ora.max_count(dec.E, dec.P, dec.G, dec.N) == 65
    assert not ora.policy(d144.G, d144.N)[2]
    assert ora.policy(sk.G, sk.N)[2] and ora.max_count(sk.E, sk.P, sk.G, sk.N) == 17


def test_lplb_topologies():
    """The r2o tables: the cube of the pages' usage example, the hypercube
    (slot d of rank g on rank g xor 2^d) and the torus (slot 0 on the
    previous GPU of the node, slot 1 on the same GPU of the previous node)."""
    assert wl.CUBE_R2O[0] == (3, 6) and len(wl.CUBE_R2O) == 8
    h = wl.hypercube_r2o(16)
    assert all(h[g][d] == g ^ (1 << d) for g in range(16) for d in range(4))
    t = wl.torus_r2o(4, 8)
    assert len(t) == 32
    for r, (a, b) in enumerate(t):
        n, g = divmod(r, 8)
        assert a == n * 8 + (g + 7) % 8 and b == ((n + 3) % 4) * 8 + g
    # every rank's experts are replicated once inside its node and once on the next node
    for o in range(32):
        names = [(r, j) for r in range(32) for j in range(2) if t[r][j] == o]
        assert sorted(j for _, j in names) == [0, 1]
