"""kvpub_create_static (the entry point that allocates nothing) against kvpub_create.

Two calls in a row through the C ABI, the second with a smaller input: each
time a static context and an ordinary one store the same rows into their own
buffers and fence; the buffers must be byte-identical (and equal the
oracle's), and the epochs and invalid-slot counts equal -- the second static
context starts from cleared words although it reuses the first one's array.
"""
import numpy as np
import pytest

from replicated_fp8_sparse_amd import kvpub, workloads as W
from replicated_fp8_sparse_amd.workloads import CacheLayout

import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    kvpub.load()
    yield
    torch.cuda.empty_cache()


def _inputs(seed, T, capacity, n_invalid):
    rng = np.random.default_rng(seed)
    slots = rng.choice(capacity, size=T, replace=False).astype(np.int64)
    pos = rng.permutation(T)
    slots[pos[:T // 20]] = -1
    slots[pos[T // 20:T // 20 + n_invalid]] = capacity + rng.integers(0, 1000, n_invalid)
    lat = W.bf16_bits(rng.standard_normal((T, 512), dtype=np.float32))
    rp = W.bf16_bits(rng.standard_normal((T, 64), dtype=np.float32))
    ix = W.bf16_bits(rng.standard_normal((T, 128), dtype=np.float32))
    return W.LayerInputs(lat, rp, ix, slots)


def _one_call(orc, layout, x, n_fences, n_invalid):
    import torch
    ref = G.DeviceCache(layout)
    sta = G.DeviceCache(layout, create=False)
    try:
        stream = torch.cuda.current_stream()
        st, sta.ctx = kvpub.kvpub_create_static(sta.config(), [b.data_ptr() for b in sta.main],
                                                [b.data_ptr() for b in sta.idx], stream.cuda_stream)
        kvpub.check(st, "kvpub_create_static")
        # one static context per GPU at a time
        st2, other = kvpub.kvpub_create_static(ref.config(), [b.data_ptr() for b in ref.main],
                                               [b.data_ptr() for b in ref.idx], stream.cuda_stream)
        assert st2 == kvpub.KVPUB_ERR_IN_USE and other is None
        dx = G.DeviceInputs(x)
        for dev in (ref, sta):
            kvpub.check(dev.store(0, dx), "kvpub_store")
            for _ in range(n_fences):
                kvpub.check(dev.fence(0), "kvpub_fence")
        torch.cuda.synchronize()
        for r in range(layout.replicas):
            assert torch.equal(sta.main[r], ref.main[r]), f"main replica {r} differs"
            assert torch.equal(sta.idx[r], ref.idx[r]), f"indexer replica {r} differs"
        assert sta.epoch(0) == ref.epoch(0) == n_fences
        st_s, inv_s, fl_s = sta.errors()
        st_r, inv_r, fl_r = ref.errors()
        assert (st_s, inv_s, fl_s) == (st_r, inv_r, fl_r) == (kvpub.KVPUB_OK, n_invalid, 0)
        mains, idxs, inv = G.oracle_replicas(orc, layout, [(0, x)])
        assert inv == n_invalid
        G.assert_full_parity(sta, mains, idxs)
    finally:
        sta.free()
        ref.free()


def test_static_context_matches_ordinary_context_twice(orc):
    # first call: the main store kernel (T > 2048 with two replicas), 3 fences
    layout = CacheLayout(replicas=2, layers=1, num_pages=64)
    G.log("no-alloc: call 1, T=3000 R=2 64 pages, 7 invalid slots, 3 fences")
    _one_call(orc, layout, _inputs(41, 3000, layout.capacity, 7), 3, 7)
    # second call, smaller: the small-batch kernel, 1 fence; the words must start cleared
    layout = CacheLayout(replicas=2, layers=1, num_pages=16)
    G.log("no-alloc: call 2, T=100 R=2 16 pages, 2 invalid slots, 1 fence")
    _one_call(orc, layout, _inputs(42, 100, layout.capacity, 2), 1, 2)


def test_static_context_limits():
    layout = CacheLayout(replicas=1, layers=1, num_pages=4)
    dev = G.DeviceCache(layout, create=False)
    try:
        mb, ib = [b.data_ptr() for b in dev.main], [b.data_ptr() for b in dev.idx]
        st, ctx = kvpub.kvpub_create_static(dev.config(participants=2), mb, ib)
        assert st == kvpub.KVPUB_ERR_UNSUPPORTED and ctx is None
        cfg = dev.config()
        cfg.num_lanes = 65
        st, ctx = kvpub.kvpub_create_static(cfg, mb, ib)
        assert st == kvpub.KVPUB_ERR_INVALID_ARG and ctx is None
        # all 64 lanes fit; destroy frees the device's static context for the next call
        st, dev.ctx = kvpub.kvpub_create_static(dev.config(lanes=64), mb, ib)
        kvpub.check(st, "kvpub_create_static (64 lanes)")
        kvpub.check(dev.fence(63))
        assert dev.epoch(63) == 1 and dev.epoch(0) == 0
        dev.destroy()
        st, dev.ctx = kvpub.kvpub_create_static(dev.config(lanes=64), mb, ib)
        kvpub.check(st, "kvpub_create_static (again)")
        assert dev.epoch(63) == 0, "a new static context must start with cleared epochs"
    finally:
        dev.free()
