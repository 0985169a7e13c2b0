"""GPU tests of the fence, lanes, host-driven peers, graph capture and replay,
and context lifetime -- all through the C ABI."""
import os
import threading
import time

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


def test_decode_61_layers_eager(orc):
    """61 x (store layer l, fence): epoch +61, every layer byte-exact, replicas identical."""
    layout, xs = W.decode()
    G.log(f"decode eager: 61 layers T=64 R=2 pages={layout.num_pages}")
    dev = G.DeviceCache(layout)
    try:
        dxs = [G.DeviceInputs(x) for x in xs]
        for l, dx in enumerate(dxs):
            kvpub.check(dev.store(l, dx), "kvpub_store")
            kvpub.check(dev.fence(0), "kvpub_fence")
        assert dev.epoch(0) == orc_epoch(orc, 0, 61)
        st, invalid, flags = dev.errors()
        assert st == kvpub.KVPUB_OK and invalid == 0 and flags == 0
        for l, x in enumerate(xs):
            rows = orc.encode_rows(x.latent, x.rope, x.indexer)
            G.assert_gathered_parity(dev, l, x, rows, "decode")
        G.assert_replicas_identical(dev)
        G.log("decode eager: untouched bytes")
        G.assert_untouched(dev, [(l, x.slots) for l, x in enumerate(xs)])
    finally:
        dev.free()


def orc_epoch(orc, e0, n):
    return orc.epoch_after(e0, n)


def test_lanes_advance_independently():
    import torch
    layout = CacheLayout(replicas=1, layers=1, num_pages=1)
    dev = G.DeviceCache(layout, lanes=64)
    try:
        G.log("lanes: 64 lanes; 10 fences on lane 0 (stream A), 7 on lane 2 (stream B), 3 on lane 63")
        a, b = torch.cuda.Stream(), torch.cuda.Stream()
        for _ in range(10):
            kvpub.check(dev.fence(0, a))
        for _ in range(7):
            kvpub.check(dev.fence(2, b))
        for _ in range(3):
            kvpub.check(dev.fence(63, b))
        torch.cuda.synchronize()
        want = {0: 10, 2: 7, 63: 3}
        assert [dev.epoch(l) for l in range(64)] == [want.get(l, 0) for l in range(64)]
        assert dev.fence(64, a) == kvpub.KVPUB_ERR_INVALID_ARG
    finally:
        dev.free()


def test_host_peer_released_fences_complete():
    """Two participants; the second is a host thread that publishes epochs late."""
    import torch
    layout = CacheLayout(replicas=1, layers=1, num_pages=1)
    dev = G.DeviceCache(layout, participants=2, timeout_ns=5_000_000_000)
    try:
        st, sig = kvpub.kvpub_participant_signal(dev.ctx, 0, 1)
        kvpub.check(st)
        G.log("host peer: 5 fences, peer publishes 1..5 with 20 ms gaps")
        for _ in range(5):
            kvpub.check(dev.fence(0))

        def peer():
            for k in range(1, 6):
                time.sleep(0.02)
                sig[0] = k

        th = threading.Thread(target=peer)
        th.start()
        torch.cuda.synchronize()
        th.join()
        assert dev.epoch(0) == 5
        st, _, flags = dev.errors()
        assert st == kvpub.KVPUB_OK and flags == 0
    finally:
        dev.free()


def test_fence_timeout_fails_closed(orc):
    """A peer that never publishes: the bounded wait gives up, the context is
    poisoned, and later stores write nothing (the kernels all exit normally)."""
    layout, x = W.tiny()
    dev = G.DeviceCache(layout, participants=2, timeout_ns=2_000_000)
    try:
        G.log("fence timeout: peer never signals, 2 ms limit")
        kvpub.check(dev.fence(0))
        st, invalid, flags = dev.errors()
        assert st == kvpub.KVPUB_ERR_FENCE_TIMEOUT
        assert flags == kvpub.KVPUB_FLAG_FENCE_TIMEOUT | kvpub.KVPUB_FLAG_POISONED
        before = dev.host()
        kvpub.check(dev.store(0, G.DeviceInputs(x)), "kvpub_store")
        kvpub.check(dev.fence(0))
        after = dev.host()
        for a, b in zip(before[0] + before[1], after[0] + after[1]):
            assert np.array_equal(a, b), "a poisoned context still wrote"
        assert dev.epoch(0) == 1, "a poisoned fence advanced the epoch"
    finally:
        dev.free()


def test_graph_replay_61_layers_x100(orc):
    """Capture 61 x (store, fence) once; replay 100 times with new inputs each time.
    The epoch reaches 6100, replicas stay identical after every replay, and
    replays 0 and 99 match the oracle on every written byte."""
    import torch
    layout = W.graph_layout()
    L, T = W.GRAPH_LAYERS, W.GRAPH_T
    slots = W.graph_slots()
    G.log(f"graph: {L} layers x T={T}, R=2, pages={layout.num_pages}, 100 replays")
    dev = G.DeviceCache(layout)
    graph = None
    try:
        lat = torch.empty((L, T, 512), dtype=torch.bfloat16, device="cuda")
        rope = torch.empty((L, T, 64), dtype=torch.bfloat16, device="cuda")
        idx = torch.empty((L, T, 128), dtype=torch.bfloat16, device="cuda")
        dslots = G.to_dev_i64(slots)
        ios = [kvpub.layer_io(lat[l].data_ptr(), rope[l].data_ptr(), idx[l].data_ptr(),
                              dslots.data_ptr(), T, l) for l in range(L)]
        st, graph = kvpub.kvpub_graph_create(dev.ctx, ios, 0)
        kvpub.check(st, "kvpub_graph_create")
        assert dev.epoch(0) == 0, "capturing must not execute anything"
        stream = torch.cuda.current_stream()
        for rep in range(100):
            W.graph_fill_inputs_device(lat, rope, idx, seed=5, replay=rep)
            kvpub.check(kvpub.kvpub_graph_replay(graph, stream.cuda_stream), "kvpub_graph_replay")
            torch.cuda.synchronize()
            G.assert_replicas_identical(dev)
            if rep in (0, 99):
                G.log(f"graph: oracle check of replay {rep}")
                hl = lat.view(torch.int16).cpu().numpy().view(np.uint16)
                hr = rope.view(torch.int16).cpu().numpy().view(np.uint16)
                hi = idx.view(torch.int16).cpu().numpy().view(np.uint16)
                for l in range(L):
                    x = W.LayerInputs(hl[l], hr[l], hi[l], slots)
                    rows = G.oracle_rows_parallel(orc, x)
                    G.assert_gathered_parity(dev, l, x, rows, f"graph replay {rep}")
        assert dev.epoch(0) == orc.epoch_after(0, L * 100)
        st, invalid, flags = dev.errors()
        assert st == kvpub.KVPUB_OK and invalid == 0 and flags == 0
        G.log("graph: untouched bytes")
        G.assert_untouched(dev, [(l, slots) for l in range(L)])
    finally:
        if graph is not None:
            kvpub.kvpub_graph_destroy(graph)
        dev.free()


def test_store_and_fence_under_torch_graph_capture(orc):
    """kvpub_store and kvpub_fence are capture-safe inside an external torch CUDA graph."""
    import torch
    layout, x = W.tiny()
    dev = G.DeviceCache(layout)
    try:
        G.log("torch graph capture of store + fence, 5 replays")
        dx = G.DeviceInputs(x)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                kvpub.check(dev.store(0, dx, stream=s), "kvpub_store (capture)")
                kvpub.check(dev.fence(0, stream=s), "kvpub_fence (capture)")
        torch.cuda.synchronize()
        assert dev.epoch(0) == 0
        for i in range(5):
            g.replay()
            torch.cuda.synchronize()
            assert dev.epoch(0) == i + 1
        mains, idxs, _ = G.oracle_replicas(orc, layout, [(0, x)])
        G.assert_full_parity(dev, mains, idxs)
        del g
    finally:
        dev.free()


@pytest.mark.parametrize("fail_at", [1, 2, 3])
def test_create_is_all_or_nothing(fail_at):
    import torch
    layout = CacheLayout(replicas=2, layers=1, num_pages=2)
    dev = G.DeviceCache(layout, create=False)
    try:
        G.log(f"allocation failure injected at allocation {fail_at}")
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        os.environ["KVPUB_TEST_FAIL_ALLOC_AT"] = str(fail_at)
        try:
            st, ctx = dev.create(participants=2)
        finally:
            del os.environ["KVPUB_TEST_FAIL_ALLOC_AT"]
        assert st == kvpub.KVPUB_ERR_OUT_OF_MEMORY and ctx is None
        assert torch.cuda.mem_get_info()[0] == free0
        st, ctx = dev.create(participants=2)
        kvpub.check(st)
        dev.ctx = ctx
    finally:
        dev.free()


def test_create_rejects_bad_config():
    layout = CacheLayout(replicas=2, layers=2, num_pages=4)
    dev = G.DeviceCache(layout, create=False)
    try:
        G.log("bad configs")
        mb = [b.data_ptr() for b in dev.main]
        ib = [b.data_ptr() for b in dev.idx]
        for field, val in (("num_replicas", 0), ("num_replicas", 9), ("block_size", 32),
                           ("main_page_stride", 41983), ("idx_page_stride", 8440),
                           ("main_layer_stride", 3 * 41984), ("num_lanes", 0),
                           ("num_lanes", 65), ("num_participants", 9), ("flags", 2),
                           ("struct_size", 8)):
            cfg = dev.config()
            setattr(cfg, field, val)
            st, ctx = kvpub.kvpub_create(cfg, mb, ib)
            assert st == kvpub.KVPUB_ERR_INVALID_ARG and ctx is None, (field, val, st)
        st, ctx = kvpub.kvpub_create(dev.config(), [mb[0] + 8, mb[1]], ib)
        assert st == kvpub.KVPUB_ERR_INVALID_ARG
        cfg = dev.config()
        cfg.device = 64
        st, ctx = kvpub.kvpub_create(cfg, mb, ib)
        assert st == kvpub.KVPUB_ERR_INVALID_ARG
    finally:
        dev.free()


def test_graph_with_empty_and_mixed_layers(orc):
    """A captured sequence whose layers hold 0, 5, 300 and 2500 tokens (no store,
    the small-batch mapping, and the main kernel): every layer still fences once
    per replay, and the written bytes equal the oracle's after two replays."""
    import torch
    layout = CacheLayout(replicas=2, layers=4, num_pages=64, guard=64)
    sizes = [0, 5, 300, 2500]
    rng = np.random.default_rng(77)
    dev = G.DeviceCache(layout)
    graph = None
    try:
        xs, keep = [], []
        for layer, T in enumerate(sizes):
            slots = rng.permutation(layout.capacity)[:T].astype(np.int64)
            if T > 10:
                slots[::13] = -1
            xs.append(W.LayerInputs(*W._normal_rows(rng, T), slots))
        ios = []
        for layer, x in enumerate(xs):
            d = G.DeviceInputs(x)
            keep.append(d)
            ios.append(kvpub.layer_io(d.latent.data_ptr() if x.slots.size else 0,
                                      d.rope.data_ptr() if x.slots.size else 0,
                                      d.indexer.data_ptr() if x.slots.size else 0,
                                      d.slots.data_ptr() if x.slots.size else 0, x.slots.size, layer))
        st, graph = kvpub.kvpub_graph_create(dev.ctx, ios, 0)
        kvpub.check(st, "kvpub_graph_create")
        s = torch.cuda.current_stream().cuda_stream
        for _ in range(2):
            kvpub.check(kvpub.kvpub_graph_replay(graph, s))
        torch.cuda.synchronize()
        assert dev.epoch(0) == 2 * len(sizes)
        mains, idxs, want_invalid = G.oracle_replicas(orc, layout, list(enumerate(xs)))
        G.assert_full_parity(dev, mains, idxs)
        st, invalid, flags = dev.errors()
        assert invalid == 2 * want_invalid and flags == 0
    finally:
        if graph is not None:
            kvpub.kvpub_graph_destroy(graph)
        dev.free()


def test_two_lanes_two_graphs_replayed_concurrently(orc):
    """Two overlapped micro-batches (one fence lane each): graph A stores 3000
    tokens per layer (main kernel) and fences lane 0, graph B stores 500 other
    tokens per layer (small-batch kernel) into the same layers and fences lane 1;
    they are replayed five times each, concurrently on two streams.  Every byte
    of every replica equals the oracle applying both micro-batches (their slots
    are disjoint, so the order between them does not matter), and each lane's
    epoch counts exactly its own fences."""
    import torch
    L, TA, TB, reps = 4, 3000, 500, 5
    layout = CacheLayout(replicas=2, layers=L, num_pages=64)
    rng = np.random.default_rng(404)
    G.log(f"two lanes: graphs of {L} x (store, fence), T={TA} on lane 0 and T={TB} on lane 1, {reps} concurrent replays")
    dev = G.DeviceCache(layout, lanes=2)
    graphs = []
    try:
        perm = rng.permutation(layout.capacity)
        sa = perm[:TA].astype(np.int64)
        sb = perm[TA:TA + TB].astype(np.int64)
        sa[::97] = -1
        sb[::31] = -1
        xa = [W.LayerInputs(*W._normal_rows(rng, TA), sa) for _ in range(L)]
        xb = [W.LayerInputs(*W._normal_rows(rng, TB), sb) for _ in range(L)]
        da = [G.DeviceInputs(x) for x in xa]
        db = [G.DeviceInputs(x) for x in xb]
        for lane, ds in ((0, da), (1, db)):
            ios = [kvpub.layer_io(d.latent.data_ptr(), d.rope.data_ptr(), d.indexer.data_ptr(),
                                  d.slots.data_ptr(), d.T, l) for l, d in enumerate(ds)]
            st, g = kvpub.kvpub_graph_create(dev.ctx, ios, lane)
            kvpub.check(st, "kvpub_graph_create")
            graphs.append(g)
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
        for _ in range(reps):
            kvpub.check(kvpub.kvpub_graph_replay(graphs[0], s0.cuda_stream), "replay A")
            kvpub.check(kvpub.kvpub_graph_replay(graphs[1], s1.cuda_stream), "replay B")
        torch.cuda.synchronize()
        assert (dev.epoch(0), dev.epoch(1)) == (reps * L, reps * L)
        st, invalid, flags = dev.errors()
        assert st == kvpub.KVPUB_OK and invalid == 0 and flags == 0
        mains, idxs, want_invalid = G.oracle_replicas(orc, layout, [(l, x) for l, x in enumerate(xa)] +
                                                      [(l, x) for l, x in enumerate(xb)])
        assert want_invalid == 0
        G.assert_full_parity(dev, mains, idxs)
    finally:
        for g in graphs:
            kvpub.kvpub_graph_destroy(g)
        dev.free()


def test_graph_replays_wait_for_a_host_peer_at_each_epoch(orc):
    """Two participants under graph replay: 4 x (store, fence) captured once and
    replayed 3 times; a host thread stands in for the peer and publishes epochs
    1..12 one at a time, 3 ms apart.  Each replayed fence waits for the peer's
    signal to reach the epoch it has just advanced to (read from the device, not
    fixed at capture), so the replays can finish only after the last
    publication -- with an expected value frozen at capture, replays 2 and 3
    would pass as soon as the peer had published 4.  The epoch ends at 12, no
    timeout is recorded, and the stored bytes equal the oracle's."""
    import torch
    L, reps, gap = 4, 3, 0.003
    layout = CacheLayout(replicas=2, layers=L, num_pages=8)
    rng = np.random.default_rng(505)
    G.log(f"host peer under graph replay: {L} x (store, fence), {reps} replays, peer publishes 1..{L * reps}")
    dev = G.DeviceCache(layout, participants=2, timeout_ns=10_000_000_000)
    graph = None
    try:
        xs = [W.LayerInputs(*W._normal_rows(rng, 32), rng.permutation(layout.capacity)[:32].astype(np.int64))
              for _ in range(L)]
        ds = [G.DeviceInputs(x) for x in xs]
        ios = [kvpub.layer_io(d.latent.data_ptr(), d.rope.data_ptr(), d.indexer.data_ptr(), d.slots.data_ptr(),
                              d.T, l) for l, d in enumerate(ds)]
        st, graph = kvpub.kvpub_graph_create(dev.ctx, ios, 0)
        kvpub.check(st, "kvpub_graph_create")
        st, sig = kvpub.kvpub_participant_signal(dev.ctx, 0, 1)
        kvpub.check(st)
        torch.cuda.synchronize()
        stream = torch.cuda.Stream()
        published = []

        def peer():
            for k in range(1, L * reps + 1):
                time.sleep(gap)
                published.append(time.perf_counter())   # before the write the GPU may act on
                sig[0] = k

        t0 = time.perf_counter()
        for _ in range(reps):
            kvpub.check(kvpub.kvpub_graph_replay(graph, stream.cuda_stream), "kvpub_graph_replay")
        th = threading.Thread(target=peer)
        th.start()
        stream.synchronize()
        done = time.perf_counter()
        th.join()
        assert len(published) == L * reps
        assert done >= published[-1], "the replays finished before the peer published the last epoch"
        assert done - t0 >= (L * reps - 1) * gap
        assert dev.epoch(0) == L * reps
        st, invalid, flags = dev.errors()
        assert st == kvpub.KVPUB_OK and invalid == 0 and flags == 0
        mains, idxs, _ = G.oracle_replicas(orc, layout, list(enumerate(xs)))
        G.assert_full_parity(dev, mains, idxs)
    finally:
        if graph is not None:
            kvpub.kvpub_graph_destroy(graph)
        dev.free()


def _layered_inputs(seed, layers, T, capacity):
    """Per-layer N(0,1) rows sharing one slot mapping of T distinct slots (a few padded)."""
    rng = np.random.default_rng(seed)
    slots = rng.choice(capacity, size=T, replace=False).astype(np.int64)
    slots[rng.choice(T, size=T // 50, replace=False)] = -1
    xs = []
    for _ in range(layers):
        lat = W.bf16_bits(rng.standard_normal((T, 512), dtype=np.float32))
        rp = W.bf16_bits(rng.standard_normal((T, 64), dtype=np.float32))
        ix = W.bf16_bits(rng.standard_normal((T, 128), dtype=np.float32))
        xs.append(W.LayerInputs(lat, rp, ix, slots))
    return xs


def test_release_only_fence_eager_and_replayed(orc):
    """The one-participant fence with the release-only option: eager fences and a
    replayed store + fence graph advance the epoch once per fence, and the stores
    are the oracle's bytes."""
    import torch
    layout = CacheLayout(replicas=2, layers=6, num_pages=64)
    xs = _layered_inputs(31, layout.layers, 3000, layout.capacity)
    dev = G.DeviceCache(layout, create=False)
    graph = None
    try:
        cfg = dev.config()
        cfg.flags = kvpub.KVPUB_CONFIG_FENCE_RELEASE_ONLY
        st, dev.ctx = kvpub.kvpub_create(cfg, [b.data_ptr() for b in dev.main], [b.data_ptr() for b in dev.idx])
        kvpub.check(st, "kvpub_create (release only)")
        G.log("release-only fence: 5 eager fences, then 6 layers x T=3000 R=2 captured, 40 replays")
        for _ in range(5):
            kvpub.check(dev.fence(0))
        assert dev.epoch(0) == 5
        dxs = [G.DeviceInputs(x) for x in xs]
        ios = [kvpub.layer_io(d.latent.data_ptr(), d.rope.data_ptr(), d.indexer.data_ptr(),
                              d.slots.data_ptr(), d.T, l) for l, d in enumerate(dxs)]
        st, graph = kvpub.kvpub_graph_create(dev.ctx, ios, 0)
        kvpub.check(st, "kvpub_graph_create")
        s = torch.cuda.current_stream().cuda_stream
        for _ in range(40):
            kvpub.check(kvpub.kvpub_graph_replay(graph, s))
        assert dev.epoch(0) == orc.epoch_after(5, 40 * layout.layers)
        st, invalid, flags = dev.errors()
        assert st == kvpub.KVPUB_OK and invalid == 0 and flags == 0
        mains, idxs, _ = G.oracle_replicas(orc, layout, list(enumerate(xs)))
        G.assert_full_parity(dev, mains, idxs)
    finally:
        if graph is not None:
            kvpub.kvpub_graph_destroy(graph)
        dev.free()


def test_host_epoch_fence_does_not_advance_under_replay(orc):
    """The pages' two-launch fence with a host-held epoch (lane 0) beside the
    single-launch device-epoch fence (lane 1), each captured after the same
    stores: eagerly both count every fence; replayed, lane 1 advances by the
    layer count on every replay while lane 0 stays at the value published at
    capture.  Both graphs leave the oracle's bytes."""
    import torch
    layout = CacheLayout(replicas=2, layers=4, num_pages=32)
    xs = _layered_inputs(32, layout.layers, 1500, layout.capacity)
    dev = G.DeviceCache(layout, lanes=2)
    try:
        G.log("host-epoch fence: 3 eager, then 4 layers captured with each fence, 10 replays each")
        for _ in range(3):
            kvpub.check(kvpub.kvpub_fence_host_epoch(dev.ctx, 0, torch.cuda.current_stream().cuda_stream))
            kvpub.check(dev.fence(1))
        assert (dev.epoch(0), dev.epoch(1)) == (3, 3)
        dxs = [G.DeviceInputs(x) for x in xs]
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        graphs = []
        for lane in (0, 1):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(s):
                with torch.cuda.graph(g, stream=s):
                    for l, d in enumerate(dxs):
                        kvpub.check(dev.store(l, d, stream=s), "kvpub_store (capture)")
                        if lane == 0:
                            kvpub.check(kvpub.kvpub_fence_host_epoch(dev.ctx, 0, s.cuda_stream))
                        else:
                            kvpub.check(dev.fence(1, stream=s))
            graphs.append(g)
        torch.cuda.synchronize()
        assert (dev.epoch(0), dev.epoch(1)) == (3, 3), "capturing must not execute anything"
        n = layout.layers
        for rep in range(10):
            graphs[0].replay()
            graphs[1].replay()
            torch.cuda.synchronize()
            assert dev.epoch(0) == 3 + n, f"replay {rep}: the host-held epoch moved ({dev.epoch(0)})"
            assert dev.epoch(1) == orc.epoch_after(3, n * (rep + 1)), f"replay {rep}: device epoch"
        st, invalid, flags = dev.errors()
        assert st == kvpub.KVPUB_OK and invalid == 0 and flags == 0
        mains, idxs, _ = G.oracle_replicas(orc, layout, list(enumerate(xs)))
        G.assert_full_parity(dev, mains, idxs)
        del graphs
    finally:
        dev.free()


def test_host_epoch_fence_needs_one_participant():
    layout = CacheLayout(replicas=1, layers=1, num_pages=1)
    dev = G.DeviceCache(layout, participants=2)
    try:
        assert kvpub.kvpub_fence_host_epoch(dev.ctx, 0, 0) == kvpub.KVPUB_ERR_UNSUPPORTED
        assert kvpub.kvpub_fence_host_epoch(dev.ctx, 1, 0) == kvpub.KVPUB_ERR_INVALID_ARG
    finally:
        dev.free()
