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
    assert wl.DSV3_PREFILL.placement.hierarchical and wl.DSV3_PREFILL.placement.max_count == 9
    assert not wl.GLOBAL_DECODE.placement.hierarchical and wl.GLOBAL_DECODE.placement.max_count == 65
    assert not wl.DSV3_DECODE_144.hierarchical
    assert wl.SKEWED_1024.placement.max_count == 17
