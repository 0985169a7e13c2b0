"""GPU parity of kvpub_store against the CPU oracle, byte for byte.

Every test calls the HIP path through the C ABI (libkvpub.so) and compares
every byte of every replica with the oracle run on the same input bytes.
Small cases compare whole buffers; the full-size prefill and heavy-tail
workloads compare every written row (gathered on the GPU) and check on the
GPU that every other byte still holds the fill / guard pattern.
"""
import numpy as np
import pytest

from replicated_fp8_sparse_amd import kvpub, workloads as W
from replicated_fp8_sparse_amd.workloads import CacheLayout, LayerInputs, bf16_bits

import gpu_util as G
import pins

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' on CPU-only machines)")
    kvpub.load()
    yield
    torch.cuda.empty_cache()


def run_full(orc, layout, layer_inputs, label):
    """Store [(layer, LayerInputs)] on the GPU and compare whole buffers with the oracle."""
    G.log(f"{label}: R={layout.replicas} pages={layout.num_pages} layers={layout.layers}")
    dev = G.DeviceCache(layout)
    try:
        for layer, x in layer_inputs:
            dx = G.DeviceInputs(x)
            kvpub.check(dev.store(layer, dx), "kvpub_store")
        st, invalid, flags = dev.errors()
        kvpub.check(st, "kvpub_error_read")
        mains, idxs, want_invalid = G.oracle_replicas(orc, layout, layer_inputs)
        G.assert_full_parity(dev, mains, idxs)
        assert invalid == want_invalid, f"invalid slots {invalid} != {want_invalid}"
        assert flags == 0
    finally:
        dev.free()


# Batches of up to 1024 tokens (2048 with one or two replicas) take the
# small-batch mapping (one wave per group and round); larger ones the main
# kernel.  Appending this many padded tokens (slot -1: nothing written) runs a
# small case through the main kernel with the same expected bytes.
MAIN_KERNEL_PADS = 2100
MAPPINGS = ["small", "main"]


def with_pads(x, n, rng):
    """x followed by n padded tokens with random rows."""
    if n == 0:
        return x
    extra = lambda w: bf16_bits(rng.standard_normal((n, w)).astype(np.float32))
    return LayerInputs(np.concatenate([x.latent, extra(512)]), np.concatenate([x.rope, extra(64)]),
                       np.concatenate([x.indexer, extra(128)]),
                       np.concatenate([x.slots, np.full(n, -1, np.int64)]))


def pads_for(mapping):
    return MAIN_KERNEL_PADS if mapping == "main" else 0


@pytest.mark.parametrize("mapping", MAPPINGS)
def test_tiny_parity(orc, mapping):
    layout, x = W.tiny()
    x = with_pads(x, pads_for(mapping), np.random.default_rng(7))
    run_full(orc, layout, [(0, x)], f"tiny T=256 ({mapping} mapping)")


def _hand_rows(rng):
    """Tokens that reach the corners of the quantizer."""
    rows = []
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])

    def token(lat, idx):
        rows.append((lat.astype(np.uint16), idx.astype(np.uint16)))

    # e4m3-exact tiles with amax 448 (scale exactly 1.0) and the same pattern x 2^k
    for k in (0, -20, 20):
        codes = rng.choice(finite, size=640)
        codes[::128] = 0x7E
        vals = pins.e4m3_decode(codes) * 2.0 ** k
        b = bf16_bits(vals.astype(np.float32))
        token(b[:512], b[512:])
    # smallest bf16 subnormal as amax (the scale is a binary32 subnormal)
    b = np.zeros(640, np.uint16)
    b[rng.choice(640, 100, replace=False)] = 0x0001
    b[rng.choice(640, 100, replace=False)] = 0x8001
    b[rng.choice(640, 50, replace=False)] = 0x8000
    b[0::128] = 0x0001
    token(b[:512], b[512:])
    # -0.0 inside non-zero tiles, alternating signs, all elements equal to amax
    b = bf16_bits(rng.standard_normal(640).astype(np.float32))
    b[1::3] = 0x8000
    token(b[:512], b[512:])
    b = bf16_bits((np.where(np.arange(640) % 2, -1.0, 1.0) * 3.25).astype(np.float32))
    token(b[:512], b[512:])
    # tiles far below / around the fast-division threshold, and near the bf16 maximum
    for mag in (1e-20, 448.0 * 2.0 ** -64, 448.0 * 2.0 ** -64 * (1 - 2 ** -8), 1e-37, 1e30, 3.0e38):
        v = rng.standard_normal(640)
        v = v / np.abs(v).max() * mag
        token(bf16_bits(v[:512].astype(np.float32)), bf16_bits(v[512:].astype(np.float32)))
    b = np.full(640, 0x7F7F, np.uint16)
    b[1::2] = 0xFF7F
    token(b[:512], b[512:])
    # one element per tile much larger than the rest (the other codes underflow)
    v = rng.standard_normal(640) * 1e-3
    v[::128] = 1e4
    token(bf16_bits(v[:512].astype(np.float32)), bf16_bits(v[512:].astype(np.float32)))
    return rows


@pytest.mark.parametrize("mapping", MAPPINGS)
def test_hand_cases_parity(orc, mapping):
    rng = np.random.default_rng(101)
    rows = _hand_rows(rng)
    n = len(rows)
    layout = CacheLayout(replicas=2, layers=2, num_pages=16, guard=64)
    T = n + 8
    latent = bf16_bits(rng.standard_normal((T, 512)).astype(np.float32))
    rope = rng.integers(0, 65536, size=(T, 64), dtype=np.uint16)   # any bit pattern passes through
    indexer = bf16_bits(rng.standard_normal((T, 128)).astype(np.float32))
    for t, (lat, idx) in enumerate(rows):
        latent[t], indexer[t] = lat, idx
    slots = rng.permutation(layout.capacity)[:T].astype(np.int64)
    # 3 slots >= capacity, one negative invalid slot, padded tokens
    slots[n + 0] = layout.capacity
    slots[n + 1] = layout.capacity + 12345
    slots[n + 2] = 2 ** 40
    slots[n + 3] = -7
    slots[n + 4:] = -1
    x = with_pads(LayerInputs(latent, rope, indexer, slots), pads_for(mapping), rng)
    run_full(orc, layout, [(1, x)], f"hand cases T={T} ({mapping} mapping)")


@pytest.mark.parametrize("path", ["small", "main", "write_through"])
def test_skipped_tokens_with_non_finite_rows(orc, path):
    """Padded and invalid tokens may carry anything in their rows (NaN, infinities,
    the largest values): the kernels load those rows with their group but no byte
    they store depends on them.  Skipped tokens are interleaved with valid ones so
    that they share groups (waves) and tiles' neighbours; the oracle never reads
    their rows."""
    rng = np.random.default_rng(202)
    R, T = (4, 11000) if path == "write_through" else (2, 300 if path == "small" else 2300)
    skipped = np.zeros(T, bool)
    skipped[rng.choice(T, T // 3, replace=False)] = True
    skipped[1::7] = True
    nvalid = int((~skipped).sum())
    layout = CacheLayout(replicas=R, layers=1, num_pages=(nvalid + 63) // 64 + 3)
    latent = bf16_bits(rng.standard_normal((T, 512)).astype(np.float32))
    rope = rng.integers(0, 65536, size=(T, 64), dtype=np.uint16)
    indexer = bf16_bits(rng.standard_normal((T, 128)).astype(np.float32))
    bad = np.array([0x7FC0, 0xFFC0, 0x7F80, 0xFF80, 0x7FA0, 0x7F7F, 0xFF7F], np.uint16)
    ns = int(skipped.sum())
    latent[skipped] = rng.choice(bad, size=(ns, 512))
    indexer[skipped] = rng.choice(bad, size=(ns, 128))
    latent[skipped, ::5] = 0x7FC0                     # a NaN in every tile of every skipped row
    slots = np.full(T, -1, np.int64)
    slots[~skipped] = rng.permutation(layout.capacity)[:nvalid]
    inval = np.flatnonzero(skipped)[::4]              # a quarter of the skipped tokens: invalid slots
    slots[inval] = layout.capacity + rng.integers(0, 1000, inval.size)
    x = LayerInputs(latent, rope, indexer, slots)
    written = T * R * 788
    assert (T <= 2048) == (path == "small") and (written > 32 << 20) == (path == "write_through")
    run_full(orc, layout, [(0, x)], f"non-finite skipped rows, T={T}, R={R} ({path})")


@pytest.mark.parametrize("mapping", MAPPINGS)
def test_encoder_sweep_parity(orc, mapping):
    """Tiles with amax 448 have scale 1.0, so every bf16 value in [-448, 448] is
    fed to the e4m3 conversion exactly once."""
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = pins.bf16_to_f32(b)
    vals = b[np.isfinite(v) & (np.abs(v) <= 448.0)]
    per_tile = 127
    n_tiles = -(-vals.size // per_tile)
    tiles = np.zeros((n_tiles, 128), np.uint16)
    flat = np.zeros(n_tiles * per_tile, np.uint16)
    flat[:vals.size] = vals
    tiles[:, :per_tile] = flat.reshape(n_tiles, per_tile)
    tiles[:, per_tile] = 0x43E0  # 448.0
    n_tok = -(-n_tiles // 5)
    allt = np.zeros((n_tok * 5, 128), np.uint16)
    allt[:n_tiles] = tiles
    allt[n_tiles:, 0] = 0x43E0
    allt = allt.reshape(n_tok, 5, 128)
    latent = allt[:, :4].reshape(n_tok, 512)
    indexer = allt[:, 4].copy()
    rng = np.random.default_rng(102)
    rope = rng.integers(0, 65536, size=(n_tok, 64), dtype=np.uint16)
    layout = CacheLayout(replicas=1, layers=1, num_pages=4)
    slots = rng.permutation(layout.capacity)[:n_tok].astype(np.int64)
    x = with_pads(LayerInputs(latent, rope, indexer, slots), pads_for(mapping), rng)
    run_full(orc, layout, [(0, x)], f"encoder sweep T={n_tok} ({mapping} mapping)")


@pytest.mark.parametrize("mapping", MAPPINGS)
@pytest.mark.parametrize("T", [1, 2, 3, 5, 7, 13, 17, 31, 33, 63, 65, 100, 1001])
def test_ragged_and_strided(orc, T, mapping):
    """Token counts that leave partial waves and blocks; inputs with row strides
    wider than the rows; three replicas.  With the main mapping, padded tokens
    follow the T real ones (the same partial groups, in a larger launch)."""
    import torch
    rng = np.random.default_rng(200 + T)
    layout = CacheLayout(replicas=3, layers=1, num_pages=32)
    LS, RS, IS = 520, 72, 136
    T_real = T
    T = T_real + pads_for(mapping)
    wide_l = bf16_bits(rng.standard_normal((T, LS)).astype(np.float32))
    wide_r = bf16_bits(rng.standard_normal((T, RS)).astype(np.float32))
    wide_i = bf16_bits(rng.standard_normal((T, IS)).astype(np.float32))
    slots = np.full(T, -1, np.int64)
    slots[:T_real] = rng.permutation(layout.capacity)[:T_real]
    if T_real > 4:
        slots[rng.choice(T_real, T_real // 5, replace=False)] = -1
    x = LayerInputs(np.ascontiguousarray(wide_l[:, :512]), np.ascontiguousarray(wide_r[:, :64]),
                    np.ascontiguousarray(wide_i[:, :128]), slots)
    G.log(f"ragged T={T_real} strides {LS}/{RS}/{IS} ({mapping} mapping, launch of {T})")
    dev = G.DeviceCache(layout)
    try:
        dl, dr, di = G.to_dev_u16(wide_l), G.to_dev_u16(wide_r), G.to_dev_u16(wide_i)
        ds = G.to_dev_i64(slots)
        st = kvpub.kvpub_store(dev.ctx, 0, T, dl.data_ptr(), LS, dr.data_ptr(), RS, di.data_ptr(),
                               IS, ds.data_ptr(), torch.cuda.current_stream().cuda_stream)
        kvpub.check(st, "kvpub_store")
        mains, idxs, _ = G.oracle_replicas(orc, layout, [(0, x)])
        G.assert_full_parity(dev, mains, idxs)
    finally:
        dev.free()


@pytest.mark.parametrize("R,T", [(1, 2049), (2, 2050), (2, 2051), (1, 3003), (2, 4095)])
def test_streamed_launch_ragged_real_tokens(orc, R, T):
    """Streamed launches (at most 16 MB written, 32-bit offsets: the graph layer's
    path, whose row loads use per-group bases and 32-bit lane offsets) with a
    token count that leaves the last group short, every token real (no padding
    after it), rows wider than their data, into the second of two layers; a few
    pads and invalid slots among them."""
    import torch
    rng = np.random.default_rng(700 + T)
    layout = CacheLayout(replicas=R, layers=2, num_pages=72)
    LS, RS, IS = 528, 80, 144
    wide_l = bf16_bits(rng.standard_normal((T, LS)).astype(np.float32))
    wide_r = bf16_bits(rng.standard_normal((T, RS)).astype(np.float32))
    wide_i = bf16_bits(rng.standard_normal((T, IS)).astype(np.float32))
    slots = rng.permutation(layout.capacity)[:T].astype(np.int64)
    slots[rng.choice(T - 8, T // 20, replace=False)] = -1               # pads, not in the last group
    slots[rng.choice(T - 8, 3, replace=False)] = layout.capacity + 5    # invalid, counted
    assert (slots[-(T % 4):] >= 0).all()
    x = LayerInputs(np.ascontiguousarray(wide_l[:, :512]), np.ascontiguousarray(wide_r[:, :64]),
                    np.ascontiguousarray(wide_i[:, :128]), slots)
    G.log(f"streamed ragged R={R} T={T} strides {LS}/{RS}/{IS}, layer 1 of 2")
    assert T * R * 788 <= 16 << 20
    dev = G.DeviceCache(layout)
    try:
        dl, dr, di = G.to_dev_u16(wide_l), G.to_dev_u16(wide_r), G.to_dev_u16(wide_i)
        ds = G.to_dev_i64(slots)
        kvpub.check(kvpub.kvpub_store(dev.ctx, 1, T, dl.data_ptr(), LS, dr.data_ptr(), RS, di.data_ptr(),
                                      IS, ds.data_ptr(), torch.cuda.current_stream().cuda_stream), "kvpub_store")
        st, invalid, flags = dev.errors()
        kvpub.check(st, "kvpub_error_read")
        mains, idxs, want_invalid = G.oracle_replicas(orc, layout, [(1, x)])
        assert invalid == want_invalid == 3 and flags == 0
        G.assert_full_parity(dev, mains, idxs)
    finally:
        dev.free()


def test_empty_store_is_noop(orc):
    layout = CacheLayout(replicas=2, layers=1, num_pages=2)
    dev = G.DeviceCache(layout)
    try:
        G.log("empty store T=0")
        before = dev.host()
        st = kvpub.kvpub_store(dev.ctx, 0, 0, 0, 512, 0, 64, 0, 128, 0, 0)
        assert st == kvpub.KVPUB_OK
        after = dev.host()
        for a, b in zip(before[0] + before[1], after[0] + after[1]):
            assert np.array_equal(a, b)
    finally:
        dev.free()


def test_bad_arguments_write_nothing(orc):
    import torch
    layout, x = W.tiny()
    dev = G.DeviceCache(layout)
    try:
        G.log("bad arguments")
        dx = G.DeviceInputs(x)
        s = torch.cuda.current_stream().cuda_stream
        p = (dx.latent.data_ptr(), dx.rope.data_ptr(), dx.indexer.data_ptr(), dx.slots.data_ptr())
        bad = [
            (dev.ctx, 1, x.slots.size, p[0], 512, p[1], 64, p[2], 128, p[3], s),      # layer >= L
            (dev.ctx, 0, -1, p[0], 512, p[1], 64, p[2], 128, p[3], s),                # T < 0
            (dev.ctx, 0, 16, p[0] + 2, 512, p[1], 64, p[2], 128, p[3], s),            # misaligned
            (dev.ctx, 0, 16, p[0], 511, p[1], 64, p[2], 128, p[3], s),                # stride < row
            (dev.ctx, 0, 16, p[0], 516, p[1], 64, p[2], 128, p[3], s),                # stride % 8
            (dev.ctx, 0, 16, p[0], 1 << 31, p[1], 64, p[2], 128, p[3], s),            # stride >= 2^31
            (dev.ctx, 0, 16, p[0], 512, p[1], 1 << 31, p[2], 128, p[3], s),
            (dev.ctx, 0, 16, p[0], 512, p[1], 64, p[2], 1 << 31, p[3], s),
            (dev.ctx, 0, 16, p[0], 512, p[1], 64, p[2], 128, 0, s),                   # null slots
            (None, 0, 16, p[0], 512, p[1], 64, p[2], 128, p[3], s),                   # null ctx
        ]
        before = dev.host()
        for args in bad:
            assert kvpub.kvpub_store(*args) == kvpub.KVPUB_ERR_INVALID_ARG, args
        assert kvpub.kvpub_fence(dev.ctx, 1, s) == kvpub.KVPUB_ERR_INVALID_ARG
        after = dev.host()
        for a, b in zip(before[0] + before[1], after[0] + after[1]):
            assert np.array_equal(a, b)
        assert dev.epoch(0) == 0
    finally:
        dev.free()


def _big_parity(orc, layout, x, label):
    G.log(f"{label}: T={x.slots.size} R={layout.replicas} pages={layout.num_pages}")
    dev = G.DeviceCache(layout)
    try:
        dx = G.DeviceInputs(x)
        kvpub.check(dev.store(0, dx), "kvpub_store")
        st, invalid, flags = dev.errors()
        kvpub.check(st, "kvpub_error_read")
        assert invalid == 0 and flags == 0
        G.log(f"{label}: oracle rows")
        rows = G.oracle_rows_parallel(orc, x)
        G.log(f"{label}: compare written rows")
        G.assert_gathered_parity(dev, 0, x, rows, label)
        G.assert_replicas_identical(dev)
        G.log(f"{label}: untouched bytes")
        G.assert_untouched(dev, [(0, x.slots)])
    finally:
        dev.free()


def test_prefill_full_size(orc):
    layout, x = W.prefill()
    _big_parity(orc, layout, x, "prefill")


def test_heavy_full_size(orc):
    layout, x = W.heavy()
    _big_parity(orc, layout, x, "heavy-tail")


def _run_slots(rng, T, capacity, kind):
    if kind == "from0":
        return np.arange(T, dtype=np.int64)
    if kind == "offset3":
        return 3 + np.arange(T, dtype=np.int64)
    if kind == "offset61":               # every unit straddles a page boundary somewhere
        return 61 + np.arange(T, dtype=np.int64)
    if kind == "reversed":
        return (T - 1 - np.arange(T, dtype=np.int64))
    if kind == "holes":                  # runs broken by pads and invalid slots inside units
        s = 8 + np.arange(T, dtype=np.int64)
        s[5::23] = -1
        s[11::37] = capacity + 5
        return s
    if kind == "pages":                  # whole pages in random order, tail partial
        return W.perm_page_slots(rng, T, capacity // 64)
    raise ValueError(kind)


@pytest.mark.parametrize("mapping", MAPPINGS)
@pytest.mark.parametrize("T", [8, 16, 17, 40, 63, 1000])
@pytest.mark.parametrize("kind", ["from0", "offset3", "offset61", "reversed", "holes", "pages"])
def test_consecutive_slot_runs(orc, T, kind, mapping):
    """Slot runs (the main kernel's row-image path) and broken runs (its
    piece-by-piece path) in the same launch, two replicas, page guards; run
    through both mappings (padded tokens appended for the main one)."""
    rng = np.random.default_rng(300 + T)
    layout = CacheLayout(replicas=2, layers=1, num_pages=24, guard=64)
    slots = _run_slots(rng, T, layout.capacity, kind)
    latent = bf16_bits(rng.standard_normal((T, 512)).astype(np.float32))
    rope = bf16_bits(rng.standard_normal((T, 64)).astype(np.float32))
    indexer = bf16_bits(rng.standard_normal((T, 128)).astype(np.float32))
    latent[T // 2] = 0                   # an all-zero row inside a run
    x = with_pads(LayerInputs(latent, rope, indexer, slots), pads_for(mapping), rng)
    run_full(orc, layout, [(0, x)], f"runs {kind} T={T} ({mapping} mapping)")


def test_store_across_the_launch_split(orc):
    """More than 2^24 tokens in one call: the host splits the batch into several
    launches.  Inputs are drawn on the GPU; the tokens around the split and a
    random sample elsewhere are gathered on the GPU and compared with the oracle
    row by row; every other row's bytes must still hold the fill pattern there."""
    t = G.torch()
    T = (1 << 24) + 37
    G.log(f"store across the launch split: T={T}, R=2 (about 24 GB of inputs, 26 GB of cache)")
    layout = W.CacheLayout(replicas=2, layers=1, num_pages=(T + 63) // 64 + 2)
    dev = G.DeviceCache(layout)
    g = t.Generator(device="cuda").manual_seed(41)
    lat = t.randn((T, 512), device="cuda", generator=g, dtype=t.bfloat16)
    rope = t.randn((T, 64), device="cuda", generator=g, dtype=t.bfloat16)
    ind = t.randn((T, 128), device="cuda", generator=g, dtype=t.bfloat16)
    # consecutive slots shifted by one page: token t -> slot t + 64, so rows of the two
    # launches interleave with nothing else
    slots = t.arange(64, T + 64, dtype=t.int64, device="cuda")
    s = t.cuda.current_stream().cuda_stream
    kvpub.check(kvpub.kvpub_store(dev.ctx, 0, T, lat.data_ptr(), 512, rope.data_ptr(), 64, ind.data_ptr(), 128,
                                  slots.data_ptr(), s))
    t.cuda.synchronize()
    rng = np.random.default_rng(42)
    split = 1 << 24
    sample = np.unique(np.concatenate([np.arange(split - 40, split + 37), np.arange(0, 40),
                                       rng.integers(0, T, 2000)])).astype(np.int64)
    idx_t = t.from_numpy(sample).to("cuda")
    x = W.LayerInputs(lat[idx_t].view(t.int16).cpu().numpy().view(np.uint16),
                      rope[idx_t].view(t.int16).cpu().numpy().view(np.uint16),
                      ind[idx_t].view(t.int16).cpu().numpy().view(np.uint16), sample + 64)
    rows = orc.encode_rows(x.latent, x.rope, x.indexer)
    G.assert_gathered_parity(dev, 0, x, rows, "split")
    del lat, rope, ind
    # the reader side across the same split: gather every slot from replica 1
    # and compare the sampled rows with the oracle's decode of the oracle's rows
    g_lat = t.empty((T, 512), dtype=t.int16, device="cuda")
    g_rope = t.empty((T, 64), dtype=t.int16, device="cuda")
    g_idx = t.empty((T, 128), dtype=t.int16, device="cuda")
    kvpub.check(kvpub.kvpub_gather(dev.ctx, 1, 0, T, slots.data_ptr(), g_lat.data_ptr(), 512, g_rope.data_ptr(),
                                   64, g_idx.data_ptr(), 128, s))
    t.cuda.synchronize()
    got_lat = g_lat[idx_t].cpu().numpy().view(np.uint16)
    got_rope = g_rope[idx_t].cpu().numpy().view(np.uint16)
    got_idx = g_idx[idx_t].cpu().numpy().view(np.uint16)
    main_rows, icodes, iscale = rows
    for i in range(sample.size):
        sc = main_rows[i, 512:528].view(np.float32)
        want = np.concatenate([orc.dequant_tile(main_rows[i, 128 * j:128 * (j + 1)], sc[j]) for j in range(4)])
        assert np.array_equal(got_lat[i], want), f"split gather latent, token {sample[i]}"
        assert np.array_equal(got_rope[i], x.rope[i]), f"split gather rope, token {sample[i]}"
        want_i = orc.dequant_tile(icodes[i], iscale[i].view(np.float32)[0])
        assert np.array_equal(got_idx[i], want_i), f"split gather indexer, token {sample[i]}"
    del g_lat, g_rope, g_idx
    dev.free()


@pytest.mark.parametrize("R,T", [(3, 15003), (4, 13001)])
def test_write_through_scattered_slots(orc, R, T):
    """A launch that writes more than 32 MB takes the write-through store path.
    Most slots are scattered (no row runs, so every piece goes through the
    per-token stores), 40 pages are filled by consecutive runs, and there are
    pads, invalid slots, all-zero rows and a ragged tail.  Every written row,
    the invalid count, and every byte outside the rows (guards included) are
    checked against the oracle."""
    rng = np.random.default_rng(61 + R)
    layout = CacheLayout(replicas=R, layers=1, num_pages=4096, guard=64)
    assert T * R * 788 > 32 << 20
    pages = rng.permutation(layout.num_pages)
    run_slots = (64 * pages[:40, None] + np.arange(64)).reshape(-1)
    rest = (64 * pages[40:, None] + np.arange(64)).reshape(-1)
    scattered = rng.choice(rest, size=T - run_slots.size, replace=False)
    slots = np.concatenate([run_slots, scattered]).astype(np.int64)
    slots[::23] = -1
    slots[[7, 1001, T - 2]] = [layout.capacity + 3, 2 * layout.capacity, -9]
    lat, rope, ind = W._normal_rows(rng, T)
    lat[[11, 2600]] = 0
    ind[[12, T - 1]] = 0
    x = LayerInputs(lat, rope, ind, slots)
    G.log(f"write-through scattered: R={R} T={T}")
    dev = G.DeviceCache(layout)
    try:
        kvpub.check(dev.store(0, G.DeviceInputs(x)), "kvpub_store")
        st, invalid, flags = dev.errors()
        kvpub.check(st, "kvpub_error_read")
        assert invalid == 3 and flags == 0
        rows = G.oracle_rows_parallel(orc, x)
        G.assert_gathered_parity(dev, 0, x, rows, "write-through scattered")
        G.assert_replicas_identical(dev)
        G.assert_untouched(dev, [(0, x.slots)])
    finally:
        dev.free()


def _mixed_slots(rng, T, num_pages):
    """Half the tokens fill whole pages in a permuted order (row runs), the rest
    take scattered slots of other pages; every 17th token is padded and two
    slots are invalid."""
    pages = rng.permutation(num_pages)
    n_run = (T // 2) // 64 * 64
    run = (64 * pages[:n_run // 64, None] + np.arange(64)).reshape(-1)
    rest = (64 * pages[n_run // 64:, None] + np.arange(64)).reshape(-1)
    slots = np.concatenate([run, rng.choice(rest, size=T - n_run, replace=False)]).astype(np.int64)
    slots[3::17] = -1
    slots[[1, T - 3]] = [64 * num_pages + 9, -2]
    return slots


@pytest.mark.parametrize("path", ["small", "small_max", "main", "write_back", "write_through"])
@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 6, 7, 8])
def test_every_replica_count(orc, R, path):
    """R = 1..8 through each store path: the small-batch mapping (300 tokens, and
    just below its size limit), the main kernel with streamed whole lines (the same tokens behind padded
    ones), with write-back stores (a batch writing about 24 MB) and with
    write-through stores (just over 32 MB).  Whole buffers against the oracle."""
    rng = np.random.default_rng(500 + R)
    T = {"small": 300, "small_max": 2047 if R <= 2 else 1023, "main": 300, "write_back": (24 << 20) // (R * 788),
         "write_through": (32 << 20) // (R * 788) + 97}[path]
    num_pages = max(16, 2 * ((T + 63) // 64))
    layout = CacheLayout(replicas=R, layers=1, num_pages=num_pages, guard=64)
    slots = _mixed_slots(rng, T, num_pages)
    lat, rope, ind = W._normal_rows(rng, T)
    x = LayerInputs(lat, rope, ind, slots)
    if path == "main":
        x = with_pads(x, MAIN_KERNEL_PADS, rng)
    run_full(orc, layout, [(0, x)], f"R={R} {path} T={x.slots.size}")


def _random_rows(rng, T, width):
    """bf16 rows from a mix of distributions, chosen per token: normal, heavy-tailed
    with a wide per-token magnitude, all zero, subnormal-only, or with one large
    element per row."""
    kind = rng.integers(0, 5, size=T)
    x = rng.standard_normal((T, width))
    heavy = kind == 1
    x[heavy] = (rng.standard_t(3, size=(int(heavy.sum()), width)) *
                np.exp(rng.normal(0, 3, size=(int(heavy.sum()), 1))))
    x[kind == 2] = 0.0
    sub = kind == 3
    x[sub] = rng.standard_normal((int(sub.sum()), width)) * 1e-39
    big = np.flatnonzero(kind == 4)
    x[big, rng.integers(0, width, size=big.size)] *= 1e4
    x = np.clip(x, -3.0e38, 3.0e38)
    return bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("seed", range(48))
def test_random_configurations(orc, seed):
    """Seeded random configurations, whole buffers against the oracle: replica
    count, layer count, pages, guard bytes after each page (page strides above
    the page size), input row strides wider than the rows, the layer stored, a
    token count spanning both store mappings, and slots mixing distinct random
    slots, page-aligned runs, pads and invalid slots, with rows drawn per token
    from normal, heavy-tailed, zero, subnormal and one-outlier distributions."""
    import torch
    rng = np.random.default_rng(9000 + seed)
    R = int(rng.integers(1, 9))
    L = int(rng.integers(1, 4))
    pages = int(rng.integers(4, 80))
    guard = int(rng.choice([0, 16, 64, 128]))
    layout = CacheLayout(replicas=R, layers=L, num_pages=pages, guard=guard)
    T = int(rng.integers(1, min(layout.capacity, 4000) + 1))
    LS, RS, IS = (512 + 8 * int(rng.integers(0, 4)), 64 + 8 * int(rng.integers(0, 4)),
                  128 + 8 * int(rng.integers(0, 4)))
    layer = int(rng.integers(0, L))
    # slots: runs of consecutive slots from page starts, then random distinct slots
    slots = np.empty(0, np.int64)
    free_pages = list(rng.permutation(pages))
    while slots.size < T // 2 and free_pages:
        p = free_pages.pop()
        n = int(rng.integers(1, 65))
        slots = np.concatenate([slots, p * 64 + np.arange(n)])
    used = set(slots.tolist())
    rest = np.array([s for s in rng.permutation(layout.capacity) if s not in used][:T - slots.size], np.int64)
    slots = np.concatenate([slots, rest])[:T]
    if T > 3:
        slots[rng.choice(T, T // 7, replace=False)] = -1
        bad = rng.choice(T, max(1, T // 50), replace=False)
        slots[bad] = np.where(rng.random(bad.size) < 0.5, layout.capacity + rng.integers(0, 99, bad.size),
                              -2 - rng.integers(0, 99, bad.size))
    wide_l, wide_r, wide_i = _random_rows(rng, T, LS), rng.integers(0, 65536, (T, RS), dtype=np.uint16), \
        _random_rows(rng, T, IS)
    x = LayerInputs(np.ascontiguousarray(wide_l[:, :512]), np.ascontiguousarray(wide_r[:, :64]),
                    np.ascontiguousarray(wide_i[:, :128]), slots)
    G.log(f"random config {seed}: R={R} L={L} pages={pages} guard={guard} T={T} strides {LS}/{RS}/{IS} layer={layer}")
    dev = G.DeviceCache(layout)
    try:
        dl, dr, di = G.to_dev_u16(wide_l), G.to_dev_u16(wide_r), G.to_dev_u16(wide_i)
        ds = G.to_dev_i64(slots)
        kvpub.check(kvpub.kvpub_store(dev.ctx, layer, T, dl.data_ptr(), LS, dr.data_ptr(), RS, di.data_ptr(),
                                      IS, ds.data_ptr(), torch.cuda.current_stream().cuda_stream), "kvpub_store")
        st, invalid, flags = dev.errors()
        kvpub.check(st, "kvpub_error_read")
        mains, idxs, want_invalid = G.oracle_replicas(orc, layout, [(layer, x)])
        assert invalid == want_invalid and flags == 0
        G.assert_full_parity(dev, mains, idxs)
    finally:
        dev.free()


@pytest.mark.parametrize("T", [500, 3000, 11000])
def test_fused_fanout_equals_per_replica_stores(orc, T):
    """The pages' A/B, checked for equal output: one store launch writing all four
    replicas, and four single-replica contexts over other buffers each storing the
    same rows (an insert per replica), leave byte-identical replicas equal to the
    oracle's.  At T=11000 the fused launch writes 34.7 MB (write-through path)
    while each single-replica launch writes 8.7 MB (streamed path)."""
    import torch
    rng = np.random.default_rng(606 + T)
    R = 4
    layout = CacheLayout(replicas=R, layers=1, num_pages=(T + 63) // 64 + 8)
    slots = rng.permutation(layout.capacity)[:T].astype(np.int64)
    slots[::53] = -1
    x = LayerInputs(*W._normal_rows(rng, T), slots)
    G.log(f"fan-out A/B parity: T={T}, R={R} fused vs {R} single-replica stores")
    fused = G.DeviceCache(layout)
    single_layout = CacheLayout(replicas=1, layers=1, num_pages=layout.num_pages)
    singles = [G.DeviceCache(single_layout) for _ in range(R)]
    try:
        d = G.DeviceInputs(x)
        kvpub.check(fused.store(0, d), "fused store")
        for sc in singles:
            kvpub.check(sc.store(0, d), "single-replica store")
        torch.cuda.synchronize()
        mains, idxs, _ = G.oracle_replicas(orc, layout, [(0, x)])
        G.assert_full_parity(fused, mains, idxs)
        for r, sc in enumerate(singles):
            gm, gi = sc.host()
            assert np.array_equal(gm[0], mains[r]) and np.array_equal(gi[0], idxs[r]), f"single-replica store {r}"
    finally:
        fused.free()
        for sc in singles:
            sc.free()


@pytest.mark.parametrize("R,guard", [(4, 0), (3, 0), (4, 64)])
def test_block_runs_of_large_launches(orc, R, guard):
    """Launches writing more than 32 MB store a block's 32 rows as one run when the
    block's eight groups are consecutive in the Main-KV array.  Dense pages (no guard:
    a run continues across a page boundary) and guarded pages (it cannot); block runs
    aligned and misaligned to the 32-token blocks; runs broken by a padded or an invalid
    slot, by a jump, by a page boundary; scattered groups; a ragged tail.  Whole buffers
    against the oracle, the invalid count."""
    rng = np.random.default_rng(71 + R + guard)
    T = (32 << 20) // (R * 788) + 4 * 32 + 13
    num_pages = 3 * ((T + 63) // 64) + 8
    layout = CacheLayout(replicas=R, layers=1, num_pages=num_pages, guard=guard)
    cap = layout.capacity
    slots = np.empty(T, np.int64)
    upper = rng.permutation(np.arange(cap // 2, cap))   # scattered slots, drawn without repeats
    pos, nxt, k, u = 0, 0, 0, 0
    while pos < T:
        kind = k % 6
        k += 1
        n = min(T - pos, [96, 64, 40, 33, 20, 128][kind])
        if kind == 4:                               # scattered: slots from the top half of the cache
            slots[pos:pos + n] = upper[u:u + n]
            u += n
        else:                                       # a run starting where the previous one ended (+ a skip)
            start = nxt + [0, 5, 64 - 7, 3, 0, 16][kind]
            slots[pos:pos + n] = start + np.arange(n)
            nxt = start + n
        pos += n
    assert nxt < cap // 2, "runs overran the lower half"
    # distinct slots (scattered picks are from the upper half), then breaks inside runs
    slots[np.arange(300, T, 997)] = -1
    slots[[45, 2000, T - 40]] = [cap + 1, 3 * cap, -5]
    assert np.unique(slots[slots >= 0]).size == np.count_nonzero(slots >= 0)
    lat, rope, ind = W._normal_rows(rng, T)
    x = LayerInputs(lat, rope, ind, slots)
    G.log(f"block runs: R={R} guard={guard} T={T} pages={num_pages}")
    dev = G.DeviceCache(layout)
    try:
        kvpub.check(dev.store(0, G.DeviceInputs(x)), "kvpub_store")
        st, invalid, flags = dev.errors()
        kvpub.check(st, "kvpub_error_read")
        assert invalid == 3 and flags == 0
        mains, idxs, inv = G.oracle_replicas(orc, layout, [(0, x)])
        assert inv == 3
        G.assert_full_parity(dev, mains, idxs)
    finally:
        dev.free()
