"""Helpers for the GPU tests: device caches, calls through the C ABI, comparisons.

Everything that computes cache bytes on the GPU goes through libkvpub.so
(``replicated_fp8_sparse_amd.kvpub``); torch only allocates device memory,
fills it with the harness patterns, moves bytes and compares them.
"""
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from replicated_fp8_sparse_amd import kvpub
from replicated_fp8_sparse_amd.workloads import CacheLayout, FILL, GUARD, LayerInputs


def log(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def torch():
    import torch as t
    return t


def to_dev_u16(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")


def to_dev_i64(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to("cuda")


class DeviceInputs:
    def __init__(self, x: LayerInputs):
        self.host = x
        self.T = x.slots.shape[0]
        self.latent = to_dev_u16(x.latent)
        self.rope = to_dev_u16(x.rope)
        self.indexer = to_dev_u16(x.indexer)
        self.slots = to_dev_i64(x.slots)


class DeviceCache:
    """R replicas of `layout` on cuda:0 plus a kvpub context over them."""

    def __init__(self, layout: CacheLayout, lanes=1, participants=1, timeout_ns=0, create=True):
        t = torch()
        self.layout = layout
        self.main = [t.empty(layout.main_bytes, dtype=t.uint8, device="cuda") for _ in range(layout.replicas)]
        self.idx = [t.empty(layout.idx_bytes, dtype=t.uint8, device="cuda") for _ in range(layout.replicas)]
        for b in self.main:
            layout.fill_device(b, "main")
        for b in self.idx:
            layout.fill_device(b, "idx")
        t.cuda.synchronize()
        self.ctx = None
        if create:
            st, self.ctx = self.create(lanes, participants, timeout_ns)
            kvpub.check(st, "kvpub_create")

    def config(self, lanes=1, participants=1, timeout_ns=0):
        L = self.layout
        cfg = kvpub.kvpub_config_init(L.replicas, L.layers, L.num_pages)
        cfg.main_page_stride = L.main_page_stride
        cfg.idx_page_stride = L.idx_page_stride
        cfg.main_layer_stride = L.main_layer_stride
        cfg.idx_layer_stride = L.idx_layer_stride
        cfg.num_lanes = lanes
        cfg.num_participants = participants
        cfg.fence_timeout_ns = timeout_ns
        return cfg

    def create(self, lanes=1, participants=1, timeout_ns=0):
        cfg = self.config(lanes, participants, timeout_ns)
        return kvpub.kvpub_create(cfg, [b.data_ptr() for b in self.main], [b.data_ptr() for b in self.idx])

    def store(self, layer, x: DeviceInputs, stream=None, T=None):
        t = torch()
        s = stream if stream is not None else t.cuda.current_stream()
        return kvpub.kvpub_store(self.ctx, layer, x.T if T is None else T, x.latent.data_ptr(), 512,
                                 x.rope.data_ptr(), 64, x.indexer.data_ptr(), 128,
                                 x.slots.data_ptr(), s.cuda_stream)

    def fence(self, lane=0, stream=None):
        t = torch()
        s = stream if stream is not None else t.cuda.current_stream()
        return kvpub.kvpub_fence(self.ctx, lane, s.cuda_stream)

    def epoch(self, lane=0):
        st, v = kvpub.kvpub_epoch_read(self.ctx, lane)
        kvpub.check(st, "kvpub_epoch_read")
        return v

    def errors(self, clear=False):
        return kvpub.kvpub_error_read(self.ctx, clear)

    def destroy(self):
        if self.ctx is not None:
            st = kvpub.kvpub_destroy(self.ctx)
            self.ctx = None
            kvpub.check(st, "kvpub_destroy")

    def host(self):
        torch().cuda.synchronize()
        return ([b.cpu().numpy() for b in self.main], [b.cpu().numpy() for b in self.idx])

    def free(self):
        self.destroy()
        self.main = self.idx = None
        torch().cuda.empty_cache()


def oracle_replicas(orc, layout, layer_inputs):
    """Host replicas after applying [(layer, LayerInputs), ...] with the oracle.
    Returns (main list, idx list, total invalid)."""
    m0, i0 = layout.fill_host()
    mains = [m0.copy() for _ in range(layout.replicas)]
    idxs = [i0.copy() for _ in range(layout.replicas)]
    invalid = 0
    for layer, x in layer_inputs:
        invalid += orc.store(mains, idxs, num_pages=layout.num_pages,
                             main_page_stride=layout.main_page_stride,
                             main_layer_stride=layout.main_layer_stride,
                             idx_page_stride=layout.idx_page_stride,
                             idx_layer_stride=layout.idx_layer_stride, layer=layer,
                             latent=x.latent, rope=x.rope, indexer=x.indexer,
                             slot_mapping=x.slots)
    return mains, idxs, invalid


def describe_diff(got, want, layout, which):
    bad = np.nonzero(got != want)[0]
    if bad.size == 0:
        return "identical"
    stride = layout.main_page_stride if which == "main" else layout.idx_page_stride
    lstride = layout.main_layer_stride if which == "main" else layout.idx_layer_stride
    out = []
    for off in bad[:6]:
        l, rem = divmod(int(off), lstride)
        p, b = divmod(rem, stride)
        out.append(f"off {off} (layer {l} page {p} byte {b}): got {got[off]:#04x} want {want[off]:#04x}")
    return f"{bad.size} bytes differ: " + "; ".join(out)


def assert_full_parity(dev: DeviceCache, mains, idxs):
    gm, gi = dev.host()
    for r in range(dev.layout.replicas):
        assert np.array_equal(gm[r], mains[r]), "main replica %d: %s" % (
            r, describe_diff(gm[r], mains[r], dev.layout, "main"))
        assert np.array_equal(gi[r], idxs[r]), "indexer replica %d: %s" % (
            r, describe_diff(gi[r], idxs[r], dev.layout, "idx"))


def oracle_rows_parallel(orc, x: LayerInputs, workers=16, chunk=2048):
    """Oracle rows of every token of x, computed in parallel chunks."""
    T = x.slots.shape[0]
    main = np.empty((T, 656), np.uint8)
    codes = np.empty((T, 128), np.uint8)
    scales = np.empty((T, 4), np.uint8)

    def run(lo):
        hi = min(T, lo + chunk)
        m, c, s = orc.encode_rows(x.latent[lo:hi], x.rope[lo:hi], x.indexer[lo:hi])
        main[lo:hi], codes[lo:hi], scales[lo:hi] = m, c, s

    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(run, range(0, T, chunk)))
    return main, codes, scales


def written_offsets(layout, layer, slots):
    """Device int64 byte offsets of the rows written for the valid slots of one layer:
    (main [n,656], idx codes [n,128], idx scale [n,4], valid mask numpy)."""
    t = torch()
    valid = (slots >= 0) & (slots < layout.capacity)
    s = t.from_numpy(slots[valid]).to("cuda")
    p, o = s // 64, s % 64
    mb = layer * layout.main_layer_stride + p * layout.main_page_stride + o * 656
    ib = layer * layout.idx_layer_stride + p * layout.idx_page_stride
    ar = lambda n: t.arange(n, device="cuda", dtype=t.int64)
    main = mb[:, None] + ar(656)[None, :]
    codes = (ib + o * 128)[:, None] + ar(128)[None, :]
    scale = (ib + 8192 + o * 4)[:, None] + ar(4)[None, :]
    return main, codes, scale, valid


def assert_gathered_parity(dev: DeviceCache, layer, x: LayerInputs, rows, what=""):
    """Every written byte of `layer` in every replica equals the oracle's rows."""
    main_o, codes_o, scale_o, valid = written_offsets(dev.layout, layer, x.slots)
    m_want, c_want, s_want = (r[valid] for r in rows)
    for r in range(dev.layout.replicas):
        gm = dev.main[r][main_o].cpu().numpy()
        gc = dev.idx[r][codes_o].cpu().numpy()
        gs = dev.idx[r][scale_o].cpu().numpy()
        for name, got, want in (("main row", gm, m_want), ("indexer codes", gc, c_want),
                                ("indexer scale", gs, s_want)):
            if not np.array_equal(got, want):
                bad = np.argwhere(got != want)
                tok = np.nonzero(valid)[0][bad[0, 0]]
                raise AssertionError(f"{what} layer {layer} replica {r} {name}: {len(bad)} bytes "
                                     f"differ; first at token {tok} byte {bad[0, 1]}: got "
                                     f"{got[tuple(bad[0])]:#04x} want {want[tuple(bad[0])]:#04x}")


def assert_untouched(dev: DeviceCache, layers_slots):
    """Bytes outside the rows written for [(layer, slots), ...] still hold the fill
    and guard patterns, in every replica (checked one layer at a time)."""
    t = torch()
    L = dev.layout
    by_layer = {}
    for layer, slots in layers_slots:
        by_layer.setdefault(layer, []).append(slots)
    for which, bufs, lstride, pstride, used in (
            ("main", dev.main, L.main_layer_stride, L.main_page_stride, 64 * 656),
            ("idx", dev.idx, L.idx_layer_stride, L.idx_page_stride, 64 * 132)):
        for r, buf in enumerate(bufs):
            for layer in range(L.layers):
                sl = buf[layer * lstride:(layer + 1) * lstride].clone()
                for slots in by_layer.get(layer, []):
                    mo, co, so, _ = written_offsets(L, 0, slots)
                    if which == "main":
                        sl[mo.reshape(-1)] = FILL
                    else:
                        sl[co.reshape(-1)] = FILL
                        sl[so.reshape(-1)] = FILL
                pages = sl.view(L.num_pages, pstride)
                ok = bool((pages[:, :used] == FILL).all())
                if L.guard:
                    ok = ok and bool((pages[:, used:] == GUARD).all())
                assert ok, f"{which} replica {r} layer {layer}: a byte outside the written rows changed"
                del sl
            assert bool((buf[L.layers * lstride:] == GUARD).all()), f"{which} replica {r}: canary overwritten"


def assert_replicas_identical(dev: DeviceCache):
    t = torch()
    for r in range(1, dev.layout.replicas):
        assert t.equal(dev.main[r], dev.main[0]), f"main replica {r} differs from replica 0"
        assert t.equal(dev.idx[r], dev.idx[0]), f"indexer replica {r} differs from replica 0"


def hip_runtime():
    """The HIP runtime library already loaded in this process (the one torch and
    libkvpub share), for raw-address copies and fills in tests."""
    import ctypes
    path = None
    with open("/proc/self/maps") as fh:
        for line in fh:
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
    assert path, "HIP runtime not loaded"
    lib = ctypes.CDLL(path)
    lib.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    lib.hipMemcpy.restype = ctypes.c_int
    lib.hipMemset.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t]
    lib.hipMemset.restype = ctypes.c_int
    lib.hipDeviceSynchronize.restype = ctypes.c_int
    return lib


HIP_MEMCPY_HOST_TO_DEVICE = 1
HIP_MEMCPY_DEVICE_TO_HOST = 2
