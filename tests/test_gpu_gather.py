"""GPU parity of the reader side: kvpub_gather against the oracle's gather.

The replicas are written on the GPU by kvpub_store (byte-exact against the
oracle, see test_gpu_store.py), copied to the host, and the oracle's
dequantizing gather of the host copy is compared bit for bit with the GPU's
gather of the device replica: latent and indexer bf16 values, RoPE bits, zero
rows for padded and out-of-range slots, and the out-of-range count.  Output
rows beyond T and the gaps of strided outputs must stay untouched.
"""
import numpy as np
import pytest

from replicated_fp8_sparse_amd import kvpub, workloads as W
from gpu_util import DeviceCache, DeviceInputs, log, torch, to_dev_i64

pytestmark = pytest.mark.gpu

CANARY = 0x5A5A


class Outputs:
    """Device output buffers with row strides (elements) and canary rows after T."""

    def __init__(self, T, ls=512, rs=64, is_=128, extra_rows=2):
        t = torch()
        self.T, self.ls, self.rs, self.is_ = T, ls, rs, is_
        n = T + extra_rows
        self.lat = t.full((n, ls), CANARY, dtype=t.int16, device="cuda")
        self.rope = t.full((n, rs), CANARY, dtype=t.int16, device="cuda")
        self.idx = t.full((n, is_), CANARY, dtype=t.int16, device="cuda")

    def host(self):
        torch().cuda.synchronize()
        return tuple(b.cpu().numpy().view(np.uint16) for b in (self.lat, self.rope, self.idx))


def gather(dev, out, replica, layer, slots_dev, T):
    t = torch()
    return kvpub.kvpub_gather(dev.ctx, replica, layer, T, slots_dev.data_ptr(), out.lat.data_ptr(), out.ls,
                              out.rope.data_ptr(), out.rs, out.idx.data_ptr(), out.is_,
                              t.cuda.current_stream().cuda_stream)


def oracle_gather(orc, dev, replica, layer, slots):
    L = dev.layout
    mains, idxs = dev.host()
    return orc.gather(mains[replica], idxs[replica], num_pages=L.num_pages, main_page_stride=L.main_page_stride,
                      main_layer_stride=L.main_layer_stride, idx_page_stride=L.idx_page_stride,
                      idx_layer_stride=L.idx_layer_stride, layer=layer, slot_mapping=slots)


def check(out, want, what):
    g_lat, g_rope, g_idx = out.host()
    w_lat, w_rope, w_idx, _ = want
    T = out.T
    for name, g, w, width in (("latent", g_lat, w_lat, 512), ("rope", g_rope, w_rope, 64),
                              ("indexer", g_idx, w_idx, 128)):
        diff = np.nonzero(g[:T, :width] != w)
        assert diff[0].size == 0, (f"{what}: {name} differs at {diff[0].size} elements, first "
                                   f"token {diff[0][0]} elem {diff[1][0]}: got {g[diff[0][0], diff[1][0]]:#06x} "
                                   f"want {w[diff[0][0], diff[1][0]]:#06x}")
        assert np.all(g[T:] == CANARY), f"{what}: {name} rows after T written"
        assert np.all(g[:T, width:] == CANARY), f"{what}: {name} stride gap written"


def test_gather_tiny_every_replica(orc):
    log("gather tiny: T=256, R=1 and R=3, pads / invalid / zero rows")
    for R in (1, 3):
        layout, x = W.tiny()
        layout = W.CacheLayout(replicas=R, layers=layout.layers, num_pages=layout.num_pages,
                               guard=layout.guard) if R != layout.replicas else layout
        dev = DeviceCache(layout)
        xin = DeviceInputs(x)
        kvpub.check(dev.store(0, xin))
        dev.errors(clear=True)
        # gather the stored slots, the pads and 3 out-of-range slots, in shuffled order
        rng = np.random.default_rng(31)
        slots = np.concatenate([x.slots, [layout.capacity, layout.capacity + 7, -5]]).astype(np.int64)
        slots = slots[rng.permutation(slots.size)]
        sd = to_dev_i64(slots)
        for r in range(R):
            out = Outputs(slots.size)
            kvpub.check(gather(dev, out, r, 0, sd, slots.size))
            want = oracle_gather(orc, dev, r, 0, slots)
            check(out, want, f"tiny R={R} replica {r}")
        st, invalid, flags = dev.errors()
        assert invalid == 3 * R, invalid          # only the out-of-range ones, once per gather
        dev.free()


def test_gather_roundtrip_of_exact_tiles():
    """Tiles of e4m3 values with amax 448 * 2^k come back bit for bit."""
    log("gather exact round trip")
    rng = np.random.default_rng(32)
    T = 256
    codes = np.array([c for c in range(1, 0x7F)], np.int64)
    e = (codes >> 3) & 15
    m = codes & 7
    vals = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    lat = rng.choice(vals, (T, 4, 128)) * rng.choice([-1.0, 1.0], (T, 4, 128))
    lat[:, :, 0] = 448.0
    lat *= np.exp2(rng.integers(-30, 31, (T, 4, 1)).astype(np.float64))
    idx = rng.choice(vals, (T, 1, 128))
    idx[:, :, 5] = -448.0
    idx *= np.exp2(rng.integers(-30, 31, (T, 1, 1)).astype(np.float64))
    to_bf16 = lambda a: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    latent, indexer = to_bf16(lat.reshape(T, 512)), to_bf16(idx.reshape(T, 128))
    rope = to_bf16(rng.standard_normal((T, 64)))
    layout = W.CacheLayout(replicas=2, layers=2, num_pages=8)
    slots = rng.permutation(layout.capacity)[:T].astype(np.int64)
    x = W.LayerInputs(latent, rope, indexer, slots)
    dev = DeviceCache(layout)
    kvpub.check(dev.store(1, DeviceInputs(x)))
    out = Outputs(T)
    kvpub.check(gather(dev, out, 1, 1, to_dev_i64(slots), T))
    g_lat, g_rope, g_idx = out.host()
    assert np.array_equal(g_lat[:T], latent) and np.array_equal(g_idx[:T], indexer)
    assert np.array_equal(g_rope[:T], rope)
    dev.free()


@pytest.mark.parametrize("T", [1, 3, 4, 5, 17, 63, 64, 65, 255, 1001])
def test_gather_ragged_strided_repeated(orc, T):
    """Ragged T, strided outputs, repeated and unordered slots (a reader may ask
    for the same slot twice)."""
    rng = np.random.default_rng(100 + T)
    layout = W.CacheLayout(replicas=2, layers=1, num_pages=32)
    n = min(layout.capacity, 1500)
    xs = W.LayerInputs(*W._normal_rows(rng, n), rng.permutation(layout.capacity)[:n].astype(np.int64))
    dev = DeviceCache(layout)
    kvpub.check(dev.store(0, DeviceInputs(xs)))
    slots = rng.choice(xs.slots, T).astype(np.int64)
    if T > 3:
        slots[rng.choice(T, 2, replace=False)] = -1
    out = Outputs(T, ls=520, rs=72, is_=136)
    kvpub.check(gather(dev, out, 1, 0, to_dev_i64(slots), T))
    check(out, oracle_gather(orc, dev, 1, 0, slots), f"ragged T={T}")
    dev.free()


def test_gather_heavy_tail_values(orc):
    """The heavy-tail workload's value range (tiny and saturating tiles, all-zero
    tiles) through store and gather, every token."""
    log("gather heavy: T=32768, R=4 store, gather from replica 2")
    layout, x = W.heavy()
    dev = DeviceCache(layout)
    kvpub.check(dev.store(0, DeviceInputs(x)))
    T = x.slots.size
    out = Outputs(T)
    kvpub.check(gather(dev, out, 2, 0, to_dev_i64(x.slots), T))
    check(out, oracle_gather(orc, dev, 2, 0, x.slots), "heavy")
    dev.free()


def test_gather_bad_arguments():
    layout = W.CacheLayout(replicas=2, layers=2, num_pages=4)
    dev = DeviceCache(layout)
    out = Outputs(8)
    sd = to_dev_i64(np.arange(8))
    s = torch().cuda.current_stream().cuda_stream
    bad = kvpub.KVPUB_ERR_INVALID_ARG
    g = lambda **k: kvpub.kvpub_gather(dev.ctx, k.get("r", 0), k.get("l", 0), k.get("T", 8), k.get("sl", sd.data_ptr()),
                                      k.get("lat", out.lat.data_ptr()), k.get("ls", 512), out.rope.data_ptr(),
                                      k.get("rs", 64), out.idx.data_ptr(), 128, s)
    assert g(r=2) == bad and g(l=2) == bad and g(T=-1) == bad
    assert g(sl=0) == bad and g(lat=0) == bad and g(lat=out.lat.data_ptr() + 2) == bad
    assert g(ls=511) == bad and g(ls=500) == bad and g(rs=60) == bad
    assert g(ls=1 << 31) == bad and g(rs=1 << 31) == bad                    # strides above 2^31 - 1
    assert g(T=0) == kvpub.KVPUB_OK
    torch().cuda.synchronize()
    assert np.all(out.host()[0] == CANARY), "a rejected call wrote output"
    dev.free()


def _random_cache_bytes(rng, layout):
    """One replica's Main-KV and Indexer-K buffers holding arbitrary bytes of the
    documented format: any e4m3 code but the NaN ones, tile scales drawn from zero,
    binary32 subnormals and normal values from 2^-126 to 2^100, any RoPE bits."""
    L = layout
    m = rng.integers(0, 256, size=L.main_bytes, dtype=np.uint8)
    i = rng.integers(0, 256, size=L.idx_bytes, dtype=np.uint8)

    def scales(n):
        e = rng.uniform(-149, 100, size=n)
        v = (2.0 ** e * rng.uniform(1, 2, size=n)).astype(np.float32)
        v[rng.random(n) < 0.05] = 0.0
        return v.view(np.uint8).reshape(n, 4)

    for l in range(L.layers):
        for p in range(L.num_pages):
            base = l * L.main_layer_stride + p * L.main_page_stride
            rows = m[base:base + 64 * 656].reshape(64, 656)
            codes = rows[:, :512]
            codes[(codes & 0x7F) == 0x7F] &= 0xFE
            rows[:, 512:528] = scales(64 * 4).reshape(64, 16)
            ib = l * L.idx_layer_stride + p * L.idx_page_stride
            icodes = i[ib:ib + 8192]
            icodes[(icodes & 0x7F) == 0x7F] &= 0xFE
            i[ib + 8192:ib + 8448] = scales(64).reshape(-1)
    return m, i


@pytest.mark.parametrize("seed", range(24))
def test_gather_random_caches(orc, seed):
    """Seeded random layouts (replicas, layers, pages, guard bytes) filled with
    arbitrary bytes of the documented format, gathered from a random replica and
    layer with repeated, unordered, padded and out-of-range slots into strided
    outputs, bit for bit against the oracle's gather of the same bytes."""
    t = torch()
    rng = np.random.default_rng(7000 + seed)
    layout = W.CacheLayout(replicas=int(rng.integers(1, 5)), layers=int(rng.integers(1, 4)),
                           num_pages=int(rng.integers(2, 40)), guard=int(rng.choice([0, 16, 64])))
    T = int(rng.integers(1, 3000))
    replica, layer = int(rng.integers(0, layout.replicas)), int(rng.integers(0, layout.layers))
    log(f"gather random cache {seed}: R={layout.replicas} L={layout.layers} pages={layout.num_pages} "
        f"guard={layout.guard} T={T} replica={replica} layer={layer}")
    dev = DeviceCache(layout)
    try:
        host = [_random_cache_bytes(rng, layout) for _ in range(layout.replicas)]
        for r, (m, i) in enumerate(host):
            dev.main[r].copy_(t.from_numpy(m))
            dev.idx[r].copy_(t.from_numpy(i))
        slots = rng.integers(0, layout.capacity, size=T).astype(np.int64)
        if T > 4:
            slots[rng.choice(T, T // 6, replace=False)] = -1
            bad = rng.choice(T, max(1, T // 40), replace=False)
            slots[bad] = np.where(rng.random(bad.size) < 0.5, layout.capacity + rng.integers(0, 99, bad.size),
                                  -2 - rng.integers(0, 99, bad.size))
        out = Outputs(T, ls=512 + 8 * int(rng.integers(0, 3)), rs=64 + 8 * int(rng.integers(0, 3)),
                      is_=128 + 8 * int(rng.integers(0, 3)))
        kvpub.check(gather(dev, out, replica, layer, to_dev_i64(slots), T), "kvpub_gather")
        L = layout
        want = orc.gather(host[replica][0], host[replica][1], num_pages=L.num_pages,
                          main_page_stride=L.main_page_stride, main_layer_stride=L.main_layer_stride,
                          idx_page_stride=L.idx_page_stride, idx_layer_stride=L.idx_layer_stride, layer=layer,
                          slot_mapping=slots)
        check(out, want, f"random cache {seed}")
        st, invalid, _ = dev.errors(clear=True)
        kvpub.check(st)
        assert invalid == want[3]
    finally:
        dev.free()


def test_gather_graph_layer_full_size(orc):
    """The reader side at the size the benchmark times: one layer of the graph
    workload (R=2, 8,192 pages; T=4,096 tokens at page-permuted slots) stored with
    kvpub_store, then all 4,096 rows gathered from each replica, bit for bit
    against the oracle's gather of the same replica bytes."""
    rng = np.random.default_rng(808)
    layout = W.CacheLayout(replicas=2, layers=1, num_pages=W.graph_layout().num_pages)
    slots = W.graph_slots()
    T = slots.size
    x = W.LayerInputs(*W._normal_rows(rng, T), slots)
    log(f"gather, graph layer full size: T={T}, R=2, pages={layout.num_pages}")
    dev = DeviceCache(layout)
    try:
        kvpub.check(dev.store(0, DeviceInputs(x)), "kvpub_store")
        sd = to_dev_i64(slots)
        for replica in range(layout.replicas):
            out = Outputs(T)
            kvpub.check(gather(dev, out, replica, 0, sd, T), "kvpub_gather")
            check(out, oracle_gather(orc, dev, replica, 0, slots), f"graph layer, replica {replica}")
    finally:
        dev.free()


def test_gather_topk_pattern(orc):
    """The decode-time read pattern at the size the benchmark times it: 16 requests,
    each selecting 2,048 distinct slots of its own 512-page context, gathered as one
    launch of 32,768 slots from one layer of the graph workload's cache (R=2, 8,192
    pages).  Half of the selected slots hold rows stored by kvpub_store, the rest the
    fill bytes (valid codes and scales all the same); bit for bit against the
    oracle's gather of the same replica bytes."""
    rng = np.random.default_rng(909)
    layout = W.CacheLayout(replicas=2, layers=1, num_pages=W.graph_layout().num_pages)
    slots = W.topk_slots()
    T = slots.size
    stored = rng.permutation(slots)[:T // 2]
    x = W.LayerInputs(*W._normal_rows(rng, stored.size), stored)
    log(f"gather, top-k pattern: T={T} (16 x 2048), stored {stored.size}, R=2, pages={layout.num_pages}")
    dev = DeviceCache(layout)
    try:
        kvpub.check(dev.store(0, DeviceInputs(x)), "kvpub_store")
        out = Outputs(T)
        kvpub.check(gather(dev, out, 1, 0, to_dev_i64(slots), T), "kvpub_gather")
        check(out, oracle_gather(orc, dev, 1, 0, slots), "top-k pattern, replica 1")
        st, invalid, _ = dev.errors(clear=True)
        kvpub.check(st)
        assert invalid == 0
    finally:
        dev.free()
