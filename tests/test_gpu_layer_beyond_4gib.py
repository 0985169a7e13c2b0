"""A layer whose span exceeds 2^32 bytes: the store's write-through path (32-bit
buffer offsets) and the gather's 32-bit page offsets do not apply there, so
both take their 64-bit forms.  One replica of 102,400 Main-KV pages (4.30 GB)
and its Indexer-K pages (0.87 GB) on the device; tokens go to pages above the
2^32-byte offset and to the first pages.  The expected bytes come from the
oracle on a compact host mirror that holds only the touched pages: the bytes a
slot receives do not depend on where its page sits, so device page p maps to
mirror page p (bottom pages) or p - TOP0 + BOTTOM (top pages)."""
import numpy as np
import pytest

from replicated_fp8_sparse_amd import kvpub, workloads as W
import gpu_util as G

pytestmark = pytest.mark.gpu

MAIN_PAGE, IDX_PAGE = 64 * 656, 64 * 132
P = 102_400                      # pages: 102,400 x 41,984 B = 4.30e9 B > 2^32
BOTTOM = 64                      # device pages [0, 64)
TOP0 = P - 1100                  # device pages [TOP0, P): offsets from 4.25e9 B up
FIRST_BEYOND = (1 << 32) // MAIN_PAGE + 1


def _to_mirror(slots):
    """Device slots -> mirror slots (pads stay -1, invalid slots stay invalid)."""
    cap_dev, cap_mir = P * 64, (BOTTOM + P - TOP0) * 64
    page = slots // 64
    out = slots.copy()
    top = (slots >= TOP0 * 64) & (slots < cap_dev)
    out[top] = (page[top] - TOP0 + BOTTOM) * 64 + slots[top] % 64
    bad = (slots != -1) & ((slots < 0) | (slots >= cap_dev))
    out[bad] = cap_mir + np.arange(int(bad.sum()))
    assert not np.any((slots >= BOTTOM * 64) & (slots < TOP0 * 64)), "slot outside the mirrored pages"
    return out


def test_layer_beyond_4gib_store_and_gather(orc):
    G.log("layer beyond 4 GiB: R=1, 102,400 pages; store T=3000 (streamed) and T=45,000 (write-back), gather")
    t = G.torch()
    assert TOP0 < FIRST_BEYOND < P and P * MAIN_PAGE > 1 << 32
    main = t.empty(P * MAIN_PAGE, dtype=t.uint8, device="cuda")
    idx = t.empty(P * IDX_PAGE, dtype=t.uint8, device="cuda")
    main.fill_(W.FILL)
    idx.fill_(W.FILL)
    cfg = kvpub.kvpub_config_init(1, 1, P)
    st, ctx = kvpub.kvpub_create(cfg, [main.data_ptr()], [idx.data_ptr()])
    kvpub.check(st, "kvpub_create")
    try:
        nm = BOTTOM + P - TOP0
        mirror_main = [np.full(nm * MAIN_PAGE, W.FILL, np.uint8)]
        mirror_idx = [np.full(nm * IDX_PAGE, W.FILL, np.uint8)]
        rng = np.random.default_rng(303)
        s = t.cuda.current_stream().cuda_stream
        top_slots = rng.permutation(np.arange(TOP0 * 64, P * 64))
        bottom_slots = rng.permutation(BOTTOM * 64)
        used = 0

        def store(T, n_bottom, what):
            nonlocal used
            sl = np.concatenate([top_slots[used:used + T - n_bottom - 4], bottom_slots[:n_bottom]]).astype(np.int64)
            used += T - n_bottom - 4
            sl = np.concatenate([sl, [-1, P * 64, -3, -1]]).astype(np.int64)
            rng.shuffle(sl)
            x = W.LayerInputs(*W._normal_rows(rng, T), sl)
            d = G.DeviceInputs(x)
            kvpub.check(kvpub.kvpub_store(ctx, 0, T, d.latent.data_ptr(), 512, d.rope.data_ptr(), 64,
                                          d.indexer.data_ptr(), 128, d.slots.data_ptr(), s), what)
            t.cuda.synchronize()
            xm = W.LayerInputs(x.latent, x.rope, x.indexer, _to_mirror(sl))
            inv = orc.store(mirror_main, mirror_idx, num_pages=nm, main_page_stride=MAIN_PAGE,
                            main_layer_stride=nm * MAIN_PAGE, idx_page_stride=IDX_PAGE,
                            idx_layer_stride=nm * IDX_PAGE, layer=0, latent=xm.latent, rope=xm.rope,
                            indexer=xm.indexer, slot_mapping=xm.slots)
            assert inv == 2
            return sl

        s1 = store(3000, 100, "store T=3000")            # 2.4 MB written: streamed stores
        s2 = store(45000, 200, "store T=45000")          # 35 MB written: write-back (layer too large for 32-bit offsets)
        assert 45000 * 788 > 32 << 20
        st, invalid, flags = kvpub.kvpub_error_read(ctx, True)
        kvpub.check(st)
        assert invalid == 4 and flags == 0

        # every byte of the mirrored pages (bottom and top ranges) against the mirror
        main_h = main.view(-1)
        for lo, hi, mlo in ((0, BOTTOM, 0), (TOP0, P, BOTTOM)):
            got = main_h[lo * MAIN_PAGE:hi * MAIN_PAGE].cpu().numpy()
            want = mirror_main[0][mlo * MAIN_PAGE:(mlo + hi - lo) * MAIN_PAGE]
            bad = np.flatnonzero(got != want)
            assert bad.size == 0, f"Main-KV pages {lo}..{hi}: {bad.size} bytes differ, first at {bad[0]}"
            got = idx[lo * IDX_PAGE:hi * IDX_PAGE].cpu().numpy()
            want = mirror_idx[0][mlo * IDX_PAGE:(mlo + hi - lo) * IDX_PAGE]
            bad = np.flatnonzero(got != want)
            assert bad.size == 0, f"Indexer-K pages {lo}..{hi}: {bad.size} bytes differ, first at {bad[0]}"
        # the pages in between were never written
        mid = main_h[BOTTOM * MAIN_PAGE:TOP0 * MAIN_PAGE]
        assert bool((mid == W.FILL).all()), "a page outside the stored slots changed"

        # the reader side over the same rows, pads and invalid slots included
        want_slots = np.concatenate([s1, s2[:4000]]).astype(np.int64)
        T = want_slots.size
        outs = [t.zeros((T, w), dtype=t.int16, device="cuda") for w in (512, 64, 128)]
        sd = G.to_dev_i64(want_slots)
        kvpub.check(kvpub.kvpub_gather(ctx, 0, 0, T, sd.data_ptr(), outs[0].data_ptr(), 512,
                                       outs[1].data_ptr(), 64, outs[2].data_ptr(), 128, s), "kvpub_gather")
        t.cuda.synchronize()
        want = orc.gather(mirror_main[0], mirror_idx[0], num_pages=nm, main_page_stride=MAIN_PAGE,
                          main_layer_stride=nm * MAIN_PAGE, idx_page_stride=IDX_PAGE,
                          idx_layer_stride=nm * IDX_PAGE, layer=0, slot_mapping=_to_mirror(want_slots))
        for got, w, name in zip(outs, want[:3], ("latent", "rope", "indexer")):
            assert np.array_equal(got.cpu().numpy().view(np.uint16), w), f"gathered {name}"
        st, invalid, _ = kvpub.kvpub_error_read(ctx, True)
        kvpub.check(st)
        assert invalid == int(((want_slots != -1) & ((want_slots < 0) | (want_slots >= P * 64))).sum())
        kvpub.check(kvpub.kvpub_destroy(ctx))
        ctx = None
    finally:
        if ctx is not None:
            kvpub.kvpub_destroy(ctx)
        del main, idx
        t.cuda.empty_cache()
