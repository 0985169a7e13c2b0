"""CPU checks of the seeded input recipes (replicated_fp8_sparse_amd.workloads).

The generators hold none of the method's arithmetic; these tests pin what the
parity and bench runs rely on: the same seed gives the same bytes, and each
workload has the shape, padding, slot structure and value features it is
documented to have.
"""
import hashlib

import numpy as np
import pytest

from replicated_fp8_sparse_amd import workloads as W


def digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def layer_digest(x):
    return digest(x.latent, x.rope, x.indexer, x.slots)


def values(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("name", ["tiny", "prefill", "heavy"])
def test_single_layer_generators_are_deterministic(name):
    fn = getattr(W, name)
    _, a = fn()
    _, b = fn()
    assert layer_digest(a) == layer_digest(b)
    _, c = fn(seed=101)
    assert layer_digest(c) != layer_digest(a)


def test_decode_and_graph_generators_are_deterministic():
    _, a = W.decode(layers=4)
    _, b = W.decode(layers=4)
    assert [layer_digest(x) for x in a] == [layer_digest(x) for x in b]
    assert len({layer_digest(x) for x in a}) == 4          # fresh rows per layer
    assert digest(W.graph_slots()) == digest(W.graph_slots())
    assert digest(W.graph_slots(seed=6)) != digest(W.graph_slots())


def valid_slots(x, layout):
    s = x.slots[x.slots >= 0]
    assert np.all(s < layout.capacity)
    assert np.unique(s).size == s.size, "valid slots must be distinct"
    return s


def test_tiny_recipe():
    layout, x = W.tiny()
    assert (layout.replicas, layout.layers, layout.num_pages, layout.guard) == (1, 1, 16, 64)
    assert x.latent.shape == (256, 512) and x.rope.shape == (256, 64) and x.indexer.shape == (256, 128)
    assert int((x.slots == -1).sum()) == 25                 # about 10 % padded
    valid_slots(x, layout)
    zero = [t for t in range(256) if not x.latent[t].any() and not x.rope[t].any() and not x.indexer[t].any()]
    assert len(zero) == 2
    big = np.abs(values(x.latent)).max(axis=1)
    outliers = np.nonzero(big > 1000)[0]
    assert outliers.size == 2 and not set(outliers) & set(zero)
    for t in outliers:        # one element of each tile scaled by 1e4: at most one large value per tile
        tiles = np.abs(values(x.latent[t])).reshape(4, 128)
        assert np.all((tiles > 10).sum(axis=1) <= 1) and (tiles > 10).sum() >= 2
    assert np.abs(values(x.latent[np.setdiff1d(np.arange(256), outliers)])).max() < 10


def test_decode_recipe():
    layout, layers = W.decode()
    assert (layout.replicas, layout.layers, layout.num_pages) == (2, 61, 4096)
    assert len(layers) == 61
    for x in layers:
        assert x.slots.shape == (64,) and x.latent.shape == (64, 512)
        assert np.array_equal(x.slots, layers[0].slots)     # one slot mapping for all layers
    assert int((layers[0].slots == -1).sum()) == 3           # about 5 % padded
    valid_slots(layers[0], layout)


def test_prefill_recipe():
    layout, x = W.prefill()
    assert (layout.replicas, layout.num_pages) == (4, 16384)
    T = x.slots.size
    assert T == 8192
    assert np.all(x.slots[-37:] == -1) and np.all(x.slots[:-37] >= 0)   # padded tail of 37
    valid_slots(x, layout)
    s = x.slots[:-37]
    starts = np.concatenate([[0], np.nonzero(np.diff(s) != 1)[0] + 1])
    assert np.all(s[starts] % 64 == 0), "every run starts on a page boundary"
    lengths = np.diff(np.concatenate([starts, [s.size]]))
    assert np.all(lengths[:-1] >= 64) and lengths.sum() == 8155
    # a run never shares a page with another run
    page_of_run = {}
    for i, (a, n) in enumerate(zip(starts, lengths)):
        for p in np.unique(s[a:a + n] // 64):
            assert page_of_run.setdefault(int(p), i) == i


def test_heavy_recipe():
    layout, x = W.heavy()
    assert (layout.replicas, layout.num_pages) == (4, 16384)
    T = x.slots.size
    assert T == 32768 and np.all(x.slots >= 0)
    valid_slots(x, layout)
    t = np.arange(T)
    assert np.all(x.slots % 64 == t % 64)                    # whole pages, in a permuted order
    pages = x.slots[::64] // 64
    assert np.unique(pages).size == pages.size and not np.array_equal(pages, np.sort(pages))
    tiles = np.concatenate([x.latent.reshape(T, 4, 128), x.indexer.reshape(T, 1, 128)], axis=1)
    zero_tiles = int((~tiles.any(axis=2)).sum())
    assert zero_tiles == 5 * T // 100                        # 1 % of the tiles all-zero
    amax = np.abs(values(tiles)).max(axis=2)
    nz = amax[amax > 0]
    assert nz.max() / nz.min() > 1e6                         # tile scales span 20+ binades
    assert (amax > 448).any() and (amax[amax > 0] < 1e-2).any()


def test_graph_slots_recipe():
    s = W.graph_slots()
    layout = W.graph_layout()
    assert s.size == W.GRAPH_T and np.all(s >= 0) and np.all(s < layout.capacity)
    assert np.unique(s).size == s.size
    assert np.all(s % 64 == np.arange(s.size) % 64)


def test_layout_fill_and_guards():
    layout = W.CacheLayout(replicas=1, layers=2, num_pages=3, guard=64)
    m, i = layout.fill_host()
    assert m.size == 2 * 3 * (64 * 656 + 64) + W.CANARY_BYTES
    pages = m[:-W.CANARY_BYTES].reshape(6, 64 * 656 + 64)
    assert np.all(pages[:, :64 * 656] == W.FILL) and np.all(pages[:, 64 * 656:] == W.GUARD)
    assert np.all(m[-W.CANARY_BYTES:] == W.GUARD)
    ipages = i[:-W.CANARY_BYTES].reshape(6, 64 * 132 + 64)
    assert np.all(ipages[:, :64 * 132] == W.FILL) and np.all(ipages[:, 64 * 132:] == W.GUARD)


def test_rotation_slots_write_disjoint_pages():
    """The benchmark's warm prefill and heavy-tail figures rotate over slot mappings that
    write disjoint page sets; each mapping keeps its workload's recipe."""
    from replicated_fp8_sparse_amd import workloads as W
    _, hx = W.heavy()
    heavy = W.heavy_rotation_slots(8)
    assert np.array_equal(heavy[0], hx.slots)                       # the heavy workload's own mapping first
    prefill = W.prefill_rotation_slots(16)
    for maps, pages_per_map in ((heavy, 512), (prefill, None)):
        seen = set()
        for s in maps:
            valid = s[s >= 0]
            assert np.unique(valid).size == valid.size              # distinct slots
            pages = set((valid // 64).tolist())
            assert not (pages & seen), "two mappings share a page"
            seen |= pages
            if pages_per_map:
                assert len(pages) == pages_per_map and np.array_equal(valid % 64, np.arange(valid.size) % 64)
    for j, s in enumerate(prefill):
        assert s.size == 8192 and np.all(s[8155:] == -1) and np.all(s[:8155] >= 0)
        assert np.all(s[:8155] // 64 // 1024 == j)                  # inside the mapping's own window
        runs = np.split(s[:8155], np.nonzero(np.diff(s[:8155]) != 1)[0] + 1)
        assert all(r[0] % 64 == 0 for r in runs)                    # runs start at page boundaries
        assert sum(r.size for r in runs) == 8155


def test_topk_slots_recipe():
    """Each request's k slots are distinct, lie in its own context's pages, and the
    contexts of the default recipe cover the graph layer's pages once."""
    s = W.topk_slots()
    assert s.dtype == np.int64 and s.shape == (16 * 2048,)
    assert digest(s) == digest(W.topk_slots()) and digest(s) != digest(W.topk_slots(seed=7))
    cap = W.graph_layout().capacity
    assert s.min() >= 0 and s.max() < cap
    for q, r in enumerate(s.reshape(16, 2048)):
        assert np.unique(r).size == r.size
        pages = r // 64
        assert pages.min() >= q * 512 and pages.max() < (q + 1) * 512
        assert not np.all(np.diff(r) > 0), "a request's slots come in random order"
    small = W.topk_slots(requests=3, k=100, context_pages=4, num_pages=10)
    assert set((small // 64).tolist()) <= set(range(10))
    assert set((small[200:] // 64).tolist()) <= {8, 9, 0, 1}   # request 2 wraps around
