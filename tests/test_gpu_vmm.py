"""Replica storage at stable virtual addresses (kvpub_vmm_*): stores and gathers
into VMM-backed replicas are byte-exact against the oracle, growing the storage
keeps every written byte and every address, and the grown capacity becomes
usable.  Only backed ranges are ever touched by the test (slots beyond the
context's capacity are skipped and counted by the kernels)."""
import numpy as np
import pytest

from replicated_fp8_sparse_amd import kvpub, workloads as W
import gpu_util as G

pytestmark = pytest.mark.gpu

MAIN_PAGE, IDX_PAGE = 64 * 656, 64 * 132


def _ptr(a):
    return a.ctypes.data


class Mirror:
    """Host replicas with the VMM layout, initialised like the device's backed pages."""

    def __init__(self, cfg, layers):
        self.cfg, self.L = cfg, layers
        self.main = [np.full(layers * cfg.main_layer_stride, W.FILL, np.uint8) for _ in range(cfg.num_replicas)]
        self.idx = [np.full(layers * cfg.idx_layer_stride, W.FILL, np.uint8) for _ in range(cfg.num_replicas)]

    def store(self, orc, pages, layer, x):
        c = self.cfg
        return orc.store(self.main, self.idx, num_pages=pages, main_page_stride=c.main_page_stride,
                         main_layer_stride=c.main_layer_stride, idx_page_stride=c.idx_page_stride,
                         idx_layer_stride=c.idx_layer_stride, layer=layer, latent=x.latent, rope=x.rope,
                         indexer=x.indexer, slot_mapping=x.slots)


def fill_pages(hip, cfg, mb, ib, p0, p1, layers):
    for r in range(cfg.num_replicas):
        for l in range(layers):
            assert hip.hipMemset(mb[r] + l * cfg.main_layer_stride + p0 * MAIN_PAGE, W.FILL, (p1 - p0) * MAIN_PAGE) == 0
            assert hip.hipMemset(ib[r] + l * cfg.idx_layer_stride + p0 * IDX_PAGE, W.FILL, (p1 - p0) * IDX_PAGE) == 0
    assert hip.hipDeviceSynchronize() == 0


def compare_backed(hip, cfg, mb, ib, mirror, pages, layers, what):
    for r in range(cfg.num_replicas):
        for l in range(layers):
            for base, stride, page, host in ((mb[r], cfg.main_layer_stride, MAIN_PAGE, mirror.main[r]),
                                             (ib[r], cfg.idx_layer_stride, IDX_PAGE, mirror.idx[r])):
                n = pages * page
                got = np.empty(n, np.uint8)
                assert hip.hipMemcpy(_ptr(got), base + l * stride, n, G.HIP_MEMCPY_DEVICE_TO_HOST) == 0
                want = host[l * stride:l * stride + n]
                bad = np.nonzero(got != want)[0]
                assert bad.size == 0, f"{what}: replica {r} layer {l}: {bad.size} bytes differ, first at {bad[0]}"


def test_vmm_store_grow_gather(orc):
    G.log("vmm: R=2, L=3, 40 pages backed of 1000 reserved, grow to 300")
    t = G.torch()
    hip = G.hip_runtime()
    R, L, P0, PMAX, P1 = 2, 3, 40, 1000, 300
    cfg = kvpub.kvpub_config_init(R, L, P0)
    st, vmm, mb, ib = kvpub.kvpub_vmm_create(cfg, PMAX)
    kvpub.check(st, "kvpub_vmm_create")
    try:
        assert cfg.main_layer_stride >= PMAX * MAIN_PAGE and cfg.idx_layer_stride >= PMAX * IDX_PAGE
        assert all(b % 16 == 0 for b in mb + ib)
        assert kvpub.kvpub_vmm_pages(vmm) == (kvpub.KVPUB_OK, P0)
        fill_pages(hip, cfg, mb, ib, 0, P0, L)
        st, ctx = kvpub.kvpub_create(cfg, mb, ib)
        kvpub.check(st, "kvpub_create")
        mirror = Mirror(cfg, L)
        rng = np.random.default_rng(51)
        s = t.cuda.current_stream().cuda_stream

        def store(layer, slots):
            x = W.LayerInputs(*W._normal_rows(rng, slots.size), slots.astype(np.int64))
            d = G.DeviceInputs(x)
            kvpub.check(kvpub.kvpub_store(ctx, layer, d.T, d.latent.data_ptr(), 512, d.rope.data_ptr(), 64,
                                          d.indexer.data_ptr(), 128, d.slots.data_ptr(), s))
            t.cuda.synchronize()
            return x

        # before growing: slots in the backed pages, plus pads and slots beyond the capacity
        slots = rng.permutation(P0 * 64)[:1500]
        slots = np.concatenate([slots, [-1, -1, P0 * 64, PMAX * 64 - 1, P1 * 64]])
        x1 = store(1, slots)
        assert mirror.store(orc, P0, 1, x1) == 3
        st, invalid, _ = kvpub.kvpub_error_read(ctx, True)
        assert invalid == 3
        compare_backed(hip, cfg, mb, ib, mirror, P0, L, "before growing")

        # grow: same bases, more pages; the context's capacity follows
        kvpub.check(kvpub.kvpub_vmm_grow(vmm, P1, ctx), "kvpub_vmm_grow")
        assert kvpub.kvpub_vmm_pages(vmm) == (kvpub.KVPUB_OK, P1)
        fill_pages(hip, cfg, mb, ib, P0, P1, L)
        compare_backed(hip, cfg, mb, ib, mirror, P0, L, "after growing, old pages")
        slots = np.concatenate([rng.permutation(np.arange(P0 * 64, P1 * 64))[:3000], [P1 * 64, -1]])
        x2 = store(2, slots)
        slots = rng.permutation(np.setdiff1d(np.arange(P1 * 64), x1.slots))[:2000]
        x3 = store(1, slots)
        assert mirror.store(orc, P1, 2, x2) == 1
        assert mirror.store(orc, P1, 1, x3) == 0
        compare_backed(hip, cfg, mb, ib, mirror, P1, L, "after growing")

        # the reader side over old and new pages
        want_slots = np.concatenate([x1.slots[:200], x2.slots[:200], x3.slots[:200]]).astype(np.int64)
        T = want_slots.size
        outs = [t.zeros((T, w), dtype=t.int16, device="cuda") for w in (512, 64, 128)]
        sd = G.to_dev_i64(want_slots)
        for layer in (1, 2):
            kvpub.check(kvpub.kvpub_gather(ctx, 1, layer, T, sd.data_ptr(), outs[0].data_ptr(), 512,
                                           outs[1].data_ptr(), 64, outs[2].data_ptr(), 128, s))
            t.cuda.synchronize()
            c = cfg
            want = orc.gather(mirror.main[1], mirror.idx[1], num_pages=P1, main_page_stride=c.main_page_stride,
                              main_layer_stride=c.main_layer_stride, idx_page_stride=c.idx_page_stride,
                              idx_layer_stride=c.idx_layer_stride, layer=layer, slot_mapping=want_slots)
            for got, w, name in zip(outs, want[:3], ("latent", "rope", "indexer")):
                assert np.array_equal(got.cpu().numpy().view(np.uint16), w), f"vmm gather {name} layer {layer}"
        kvpub.check(kvpub.kvpub_destroy(ctx))
    finally:
        kvpub.check(kvpub.kvpub_vmm_destroy(vmm), "kvpub_vmm_destroy")


def test_vmm_bad_arguments():
    bad = kvpub.KVPUB_ERR_INVALID_ARG
    cfg = kvpub.kvpub_config_init(1, 2, 8)
    st, vmm, _, _ = kvpub.kvpub_vmm_create(cfg, 4)                # max below the initial pages
    assert st == bad and vmm is None
    cfg = kvpub.kvpub_config_init(9, 2, 8)                        # too many replicas
    assert kvpub.kvpub_vmm_create(cfg, 16)[0] == bad
    cfg = kvpub.kvpub_config_init(1, 2, 8)
    st, vmm, mb, ib = kvpub.kvpub_vmm_create(cfg, 16)
    kvpub.check(st)
    try:
        assert kvpub.kvpub_vmm_grow(vmm, 17) == bad                # beyond the reservation
        other = G.DeviceCache(W.CacheLayout(replicas=1, layers=2, num_pages=8))
        assert kvpub.kvpub_vmm_grow(vmm, 12, other.ctx) == bad     # a context over other storage
        other.free()
        assert kvpub.kvpub_vmm_pages(vmm) == (kvpub.KVPUB_OK, 8)
        assert kvpub.kvpub_vmm_grow(vmm, 4) == kvpub.KVPUB_OK      # never shrinks
        assert kvpub.kvpub_vmm_pages(vmm) == (kvpub.KVPUB_OK, 8)
    finally:
        kvpub.check(kvpub.kvpub_vmm_destroy(vmm))


def _grow_forced_to_fail(mode, vmm, pages, ctx, monkeypatch):
    monkeypatch.setenv("KVPUB_TEST_VMM_GROW_FAIL", mode)
    try:
        return kvpub.kvpub_vmm_grow(vmm, pages, ctx)
    finally:
        monkeypatch.delenv("KVPUB_TEST_VMM_GROW_FAIL")


def test_vmm_failed_grow_keeps_the_storage(orc, monkeypatch):
    """Mapping the bigger chunk fails (forced from the host): the old chunk is put
    back, the page count and every written byte stay, and the storage grows later."""
    G.log("vmm: forced swap failure, R=1, L=2, 16 -> 64 pages")
    t = G.torch()
    hip = G.hip_runtime()
    R, L, P0, P1 = 1, 2, 16, 64
    cfg = kvpub.kvpub_config_init(R, L, P0)
    st, vmm, mb, ib = kvpub.kvpub_vmm_create(cfg, 128)
    kvpub.check(st, "kvpub_vmm_create")
    try:
        fill_pages(hip, cfg, mb, ib, 0, P0, L)
        st, ctx = kvpub.kvpub_create(cfg, mb, ib)
        kvpub.check(st)
        mirror = Mirror(cfg, L)
        rng = np.random.default_rng(52)
        x = W.LayerInputs(*W._normal_rows(rng, 300), rng.permutation(P0 * 64)[:300].astype(np.int64))
        d = G.DeviceInputs(x)
        s = t.cuda.current_stream().cuda_stream
        kvpub.check(kvpub.kvpub_store(ctx, 1, d.T, d.latent.data_ptr(), 512, d.rope.data_ptr(), 64,
                                      d.indexer.data_ptr(), 128, d.slots.data_ptr(), s))
        t.cuda.synchronize()
        mirror.store(orc, P0, 1, x)
        assert _grow_forced_to_fail("swap", vmm, P1, ctx, monkeypatch) == kvpub.KVPUB_ERR_HIP
        assert kvpub.kvpub_vmm_pages(vmm) == (kvpub.KVPUB_OK, P0)
        compare_backed(hip, cfg, mb, ib, mirror, P0, L, "after a failed grow")
        kvpub.check(kvpub.kvpub_vmm_grow(vmm, P1, ctx), "kvpub_vmm_grow")
        assert kvpub.kvpub_vmm_pages(vmm) == (kvpub.KVPUB_OK, P1)
        compare_backed(hip, cfg, mb, ib, mirror, P0, L, "after growing")
        kvpub.check(kvpub.kvpub_destroy(ctx))
    finally:
        kvpub.check(kvpub.kvpub_vmm_destroy(vmm))


def test_vmm_broken_storage_fails_closed(monkeypatch):
    """Mapping the bigger chunk and putting the old one back both fail (forced from
    the host): the storage and its context report 0 pages, stores count every slot
    as invalid and write nothing, gathers are refused, and destroy still works."""
    G.log("vmm: forced swap + restore failure, R=2, L=2, 8 -> 32 pages")
    t = G.torch()
    R, L, P0 = 2, 2, 8
    cfg = kvpub.kvpub_config_init(R, L, P0)
    st, vmm, mb, ib = kvpub.kvpub_vmm_create(cfg, 64)
    kvpub.check(st, "kvpub_vmm_create")
    try:
        st, ctx = kvpub.kvpub_create(cfg, mb, ib)
        kvpub.check(st)
        assert _grow_forced_to_fail("restore", vmm, 32, ctx, monkeypatch) == kvpub.KVPUB_ERR_HIP
        assert kvpub.kvpub_vmm_pages(vmm) == (kvpub.KVPUB_OK, 0)
        assert kvpub.kvpub_vmm_grow(vmm, 32, ctx) == kvpub.KVPUB_ERR_HIP     # stays broken
        rng = np.random.default_rng(53)
        x = W.LayerInputs(*W._normal_rows(rng, 100), rng.permutation(P0 * 64)[:100].astype(np.int64))
        d = G.DeviceInputs(x)
        s = t.cuda.current_stream().cuda_stream
        for layer in range(L):
            kvpub.check(kvpub.kvpub_store(ctx, layer, d.T, d.latent.data_ptr(), 512, d.rope.data_ptr(), 64,
                                          d.indexer.data_ptr(), 128, d.slots.data_ptr(), s))
        t.cuda.synchronize()
        st, invalid, _ = kvpub.kvpub_error_read(ctx, True)
        kvpub.check(st)
        assert invalid == L * 100
        out = [t.zeros((100, w), dtype=t.int16, device="cuda") for w in (512, 64, 128)]
        assert kvpub.kvpub_gather(ctx, 0, 0, 100, d.slots.data_ptr(), out[0].data_ptr(), 512, out[1].data_ptr(),
                                  64, out[2].data_ptr(), 128, s) == kvpub.KVPUB_ERR_INVALID_ARG
        kvpub.check(kvpub.kvpub_destroy(ctx))
    finally:
        kvpub.check(kvpub.kvpub_vmm_destroy(vmm))


def test_vmm_repeated_growth(orc):
    """Grow 8 -> 16 -> 40 -> 64 pages (the reserved maximum): after each step the
    bases are unchanged, every byte written before is still there, and slots of
    the new pages can be stored."""
    G.log("vmm: repeated growth, R=2, L=2, 8 -> 16 -> 40 -> 64 pages")
    t = G.torch()
    hip = G.hip_runtime()
    R, L = 2, 2
    steps = [8, 16, 40, 64]
    cfg = kvpub.kvpub_config_init(R, L, steps[0])
    st, vmm, mb, ib = kvpub.kvpub_vmm_create(cfg, steps[-1])
    kvpub.check(st, "kvpub_vmm_create")
    try:
        fill_pages(hip, cfg, mb, ib, 0, steps[0], L)
        st, ctx = kvpub.kvpub_create(cfg, mb, ib)
        kvpub.check(st)
        mirror = Mirror(cfg, L)
        rng = np.random.default_rng(54)
        s = t.cuda.current_stream().cuda_stream
        prev = 0
        for i, pages in enumerate(steps):
            if i:
                kvpub.check(kvpub.kvpub_vmm_grow(vmm, pages, ctx), "kvpub_vmm_grow")
                assert kvpub.kvpub_vmm_pages(vmm) == (kvpub.KVPUB_OK, pages)
                fill_pages(hip, cfg, mb, ib, prev, pages, L)
            # new rows in the pages this step added, in both layers
            new = rng.permutation(np.arange(prev * 64, pages * 64))[:200].astype(np.int64)
            for layer in range(L):
                x = W.LayerInputs(*W._normal_rows(rng, new.size), new)
                d = G.DeviceInputs(x)
                kvpub.check(kvpub.kvpub_store(ctx, layer, d.T, d.latent.data_ptr(), 512, d.rope.data_ptr(), 64,
                                              d.indexer.data_ptr(), 128, d.slots.data_ptr(), s))
                t.cuda.synchronize()
                assert mirror.store(orc, pages, layer, x) == 0
            compare_backed(hip, cfg, mb, ib, mirror, pages, L, f"after growing to {pages} pages")
            prev = pages
        st, invalid, _ = kvpub.kvpub_error_read(ctx, False)
        assert invalid == 0
        kvpub.check(kvpub.kvpub_destroy(ctx))
    finally:
        kvpub.check(kvpub.kvpub_vmm_destroy(vmm))


def test_vmm_graphs_follow_growth(orc):
    """Graphs captured before growing see the grown capacity: a store + fence
    graph and a gather graph are captured while 8 of 40 pages are backed; before
    growing, slots in the other pages are skipped and counted (and gathered as
    zero rows); after growing to 40 pages the same graphs store and gather them."""
    G.log("vmm: graphs captured before growing, R=2, L=2, 8 -> 40 pages")
    t = G.torch()
    hip = G.hip_runtime()
    R, L, P0, P1, T = 2, 2, 8, 40, 300
    cfg = kvpub.kvpub_config_init(R, L, P0)
    st, vmm, mb, ib = kvpub.kvpub_vmm_create(cfg, P1)
    kvpub.check(st, "kvpub_vmm_create")
    graph = None
    try:
        fill_pages(hip, cfg, mb, ib, 0, P0, L)
        st, ctx = kvpub.kvpub_create(cfg, mb, ib)
        kvpub.check(st)
        mirror = Mirror(cfg, L)
        rng = np.random.default_rng(55)
        slots = rng.permutation(P1 * 64)[:T].astype(np.int64)
        slots[::29] = -1
        assert (slots >= P0 * 64).sum() > 200                      # most slots are beyond the backed pages
        lat = t.empty((L, T, 512), dtype=t.int16, device="cuda")
        rope = t.empty((L, T, 64), dtype=t.int16, device="cuda")
        ind = t.empty((L, T, 128), dtype=t.int16, device="cuda")
        ds = G.to_dev_i64(slots)
        ios = [kvpub.layer_io(lat[l].data_ptr(), rope[l].data_ptr(), ind[l].data_ptr(), ds.data_ptr(), T, l)
               for l in range(L)]
        st, graph = kvpub.kvpub_graph_create(ctx, ios, 0)
        kvpub.check(st, "kvpub_graph_create")
        stream = t.cuda.Stream()
        outs = [t.zeros((T, w), dtype=t.int16, device="cuda") for w in (512, 64, 128)]
        g_gather = t.cuda.CUDAGraph()
        with t.cuda.stream(stream):
            with t.cuda.graph(g_gather, stream=stream):
                kvpub.check(kvpub.kvpub_gather(ctx, 1, 1, T, ds.data_ptr(), outs[0].data_ptr(), 512,
                                               outs[1].data_ptr(), 64, outs[2].data_ptr(), 128,
                                               stream.cuda_stream))
        t.cuda.synchronize()

        def replay(pages, what):
            xs = []
            for l in range(L):
                x = W.LayerInputs(*W._normal_rows(rng, T), slots)
                for dst, src in ((lat, x.latent), (rope, x.rope), (ind, x.indexer)):
                    dst[l].copy_(t.from_numpy(src.view(np.int16)))
                xs.append(x)
            t.cuda.synchronize()
            kvpub.check(kvpub.kvpub_graph_replay(graph, stream.cuda_stream))
            t.cuda.synchronize()
            want_invalid = sum(mirror.store(orc, pages, l, xs[l]) for l in range(L))
            st, invalid, flags = kvpub.kvpub_error_read(ctx, True)
            kvpub.check(st)
            assert invalid == want_invalid and flags == 0, (what, invalid, want_invalid)
            compare_backed(hip, cfg, mb, ib, mirror, pages, L, what)
            g_gather.replay()
            t.cuda.synchronize()
            c = cfg
            want = orc.gather(mirror.main[1], mirror.idx[1], num_pages=pages, main_page_stride=c.main_page_stride,
                              main_layer_stride=c.main_layer_stride, idx_page_stride=c.idx_page_stride,
                              idx_layer_stride=c.idx_layer_stride, layer=1, slot_mapping=slots)
            for got, w, name in zip(outs, want[:3], ("latent", "rope", "indexer")):
                assert np.array_equal(got.cpu().numpy().view(np.uint16), w), f"{what}: gathered {name}"
            kvpub.check(kvpub.kvpub_error_read(ctx, True)[0])
            return want_invalid

        assert replay(P0, "before growing") > 0
        kvpub.check(kvpub.kvpub_vmm_grow(vmm, P1, ctx), "kvpub_vmm_grow")
        fill_pages(hip, cfg, mb, ib, P0, P1, L)
        assert replay(P1, "after growing") == 0
        assert kvpub.kvpub_epoch_read(ctx, 0) == (kvpub.KVPUB_OK, 2 * L)
        del g_gather
        kvpub.check(kvpub.kvpub_graph_destroy(graph))
        graph = None
        kvpub.check(kvpub.kvpub_destroy(ctx))
    finally:
        if graph is not None:
            kvpub.kvpub_graph_destroy(graph)
        kvpub.check(kvpub.kvpub_vmm_destroy(vmm))


def test_vmm_gather_graph_replayed_on_broken_storage(monkeypatch):
    """A gather captured while the storage is fine and replayed after it broke
    (capacity 0 in the context's device words) reads nothing from the cache:
    every output row is zero and every non-padded slot is counted."""
    G.log("vmm: gather graph replayed on a broken storage, R=1, L=1, 8 pages")
    t = G.torch()
    cfg = kvpub.kvpub_config_init(1, 1, 8)
    st, vmm, mb, ib = kvpub.kvpub_vmm_create(cfg, 32)
    kvpub.check(st, "kvpub_vmm_create")
    try:
        st, ctx = kvpub.kvpub_create(cfg, mb, ib)
        kvpub.check(st)
        T = 37
        slots = np.arange(T, dtype=np.int64) * 7
        slots[::5] = -1
        ds = G.to_dev_i64(slots)
        outs = [t.full((T, w), 0x3F80, dtype=t.int16, device="cuda") for w in (512, 64, 128)]
        stream = t.cuda.Stream()
        g = t.cuda.CUDAGraph()
        with t.cuda.stream(stream):
            with t.cuda.graph(g, stream=stream):
                kvpub.check(kvpub.kvpub_gather(ctx, 0, 0, T, ds.data_ptr(), outs[0].data_ptr(), 512,
                                               outs[1].data_ptr(), 64, outs[2].data_ptr(), 128, stream.cuda_stream))
        t.cuda.synchronize()
        monkeypatch.setenv("KVPUB_TEST_VMM_GROW_FAIL", "restore")
        assert kvpub.kvpub_vmm_grow(vmm, 16, ctx) == kvpub.KVPUB_ERR_HIP
        monkeypatch.delenv("KVPUB_TEST_VMM_GROW_FAIL")
        assert kvpub.kvpub_vmm_pages(vmm) == (kvpub.KVPUB_OK, 0)
        kvpub.check(kvpub.kvpub_error_read(ctx, True)[0])
        g.replay()
        t.cuda.synchronize()
        for o in outs:
            assert not o.any(), "rows gathered from a storage with no backed page must be zero"
        st, invalid, _ = kvpub.kvpub_error_read(ctx, False)
        kvpub.check(st)
        assert invalid == int((slots != -1).sum())
        del g
        kvpub.check(kvpub.kvpub_destroy(ctx))
    finally:
        kvpub.check(kvpub.kvpub_vmm_destroy(vmm))


def test_vmm_one_layer_write_through_graph_follows_growth(orc):
    """One-layer storage, a launch large enough for the write-through store path
    (R=4, T=12288: 38.7 MB written), captured before growing: the stores' buffer
    range covers the layer's whole reserved span, so after growing the same graph
    writes the new pages (a range sized to the pages backed at capture would drop
    those stores without a trace)."""
    G.log("vmm: one layer, write-through launch in a graph captured before growing, R=4, 64 -> 256 pages")
    t = G.torch()
    hip = G.hip_runtime()
    R, L, P0, P1, T = 4, 1, 64, 256, 12288
    assert T * R * 788 > 32 << 20                                 # takes the write-through path
    cfg = kvpub.kvpub_config_init(R, L, P0)
    st, vmm, mb, ib = kvpub.kvpub_vmm_create(cfg, P1)
    kvpub.check(st, "kvpub_vmm_create")
    graph = None
    try:
        fill_pages(hip, cfg, mb, ib, 0, P0, L)
        st, ctx = kvpub.kvpub_create(cfg, mb, ib)
        kvpub.check(st)
        mirror = Mirror(cfg, L)
        rng = np.random.default_rng(56)
        slots = rng.permutation(P1 * 64)[:T].astype(np.int64)
        assert (slots >= P0 * 64).sum() > T // 2
        lat = t.empty((T, 512), dtype=t.int16, device="cuda")
        rope = t.empty((T, 64), dtype=t.int16, device="cuda")
        ind = t.empty((T, 128), dtype=t.int16, device="cuda")
        ds = G.to_dev_i64(slots)
        st, graph = kvpub.kvpub_graph_create(
            ctx, [kvpub.layer_io(lat.data_ptr(), rope.data_ptr(), ind.data_ptr(), ds.data_ptr(), T, 0)], 0)
        kvpub.check(st, "kvpub_graph_create")
        stream = t.cuda.Stream()

        def replay(pages, what):
            x = W.LayerInputs(*W._normal_rows(rng, T), slots)
            for dst, src in ((lat, x.latent), (rope, x.rope), (ind, x.indexer)):
                dst.copy_(t.from_numpy(src.view(np.int16)))
            t.cuda.synchronize()
            kvpub.check(kvpub.kvpub_graph_replay(graph, stream.cuda_stream))
            t.cuda.synchronize()
            want_invalid = mirror.store(orc, pages, 0, x)
            st, invalid, flags = kvpub.kvpub_error_read(ctx, True)
            kvpub.check(st)
            assert invalid == want_invalid and flags == 0, (what, invalid, want_invalid)
            compare_backed(hip, cfg, mb, ib, mirror, pages, L, what)
            return want_invalid

        assert replay(P0, "before growing") > 0
        kvpub.check(kvpub.kvpub_vmm_grow(vmm, P1, ctx), "kvpub_vmm_grow")
        fill_pages(hip, cfg, mb, ib, P0, P1, L)
        assert replay(P1, "after growing") == 0
        assert kvpub.kvpub_epoch_read(ctx, 0) == (kvpub.KVPUB_OK, 2)
        kvpub.check(kvpub.kvpub_graph_destroy(graph))
        graph = None
        kvpub.check(kvpub.kvpub_destroy(ctx))
    finally:
        if graph is not None:
            kvpub.kvpub_graph_destroy(graph)
        kvpub.check(kvpub.kvpub_vmm_destroy(vmm))


def test_vmm_heavy_full_size(orc):
    """The heavy-tail store shape on VMM-backed replicas, as the benchmark times it
    (T=32,768 tokens, R=4, 16,384 pages, one launch on the write-through path):
    every backed byte of every replica against the oracle."""
    layout, x = W.heavy()
    R, P = layout.replicas, layout.num_pages
    G.log(f"vmm heavy full size: T={x.slots.size} R={R} pages={P}")
    t = G.torch()
    hip = G.hip_runtime()
    cfg = kvpub.kvpub_config_init(R, 1, P)
    st, vmm, mb, ib = kvpub.kvpub_vmm_create(cfg, P)
    kvpub.check(st, "kvpub_vmm_create")
    try:
        fill_pages(hip, cfg, mb, ib, 0, P, 1)
        st, ctx = kvpub.kvpub_create(cfg, mb, ib)
        kvpub.check(st)
        d = G.DeviceInputs(x)
        assert d.T * R * 788 > 32 << 20                            # the write-through path
        kvpub.check(kvpub.kvpub_store(ctx, 0, d.T, d.latent.data_ptr(), 512, d.rope.data_ptr(), 64,
                                      d.indexer.data_ptr(), 128, d.slots.data_ptr(),
                                      t.cuda.current_stream().cuda_stream), "kvpub_store")
        t.cuda.synchronize()
        st, invalid, flags = kvpub.kvpub_error_read(ctx, False)
        kvpub.check(st)
        assert invalid == 0 and flags == 0
        G.log("vmm heavy full size: oracle")
        mirror = Mirror(cfg, 1)
        assert mirror.store(orc, P, 0, x) == 0
        G.log("vmm heavy full size: compare every backed byte")
        compare_backed(hip, cfg, mb, ib, mirror, P, 1, "heavy on VMM-backed replicas")
        kvpub.check(kvpub.kvpub_destroy(ctx))
    finally:
        kvpub.check(kvpub.kvpub_vmm_destroy(vmm))
