"""Pins for the CPU oracle: checks against what the format and the mathematics fix.

Each ``pin_*`` function takes an ``oracle.Oracle`` handle and raises
``AssertionError`` if the oracle disagrees with something that does not come
from the oracle itself:

* hand-computed OCP FP8 E4M3 codes (``golden/e4m3_hand_codes.txt``);
* an independent encoder by bit manipulation of the binary32 pattern (a
  different algorithm from the oracle's nearest-value search), exhaustively
  over every bf16 pattern and the binary32 patterns around every tie;
* torch's CPU cast to ``float8_e4m3fn`` (a library routine) below 464,
  where saturation plays no part;
* tile invariants: the element of largest magnitude maps to +-448 (0x7E),
  dequantized values lie within half an e4m3 step (at the tile scale) of
  the input, the chosen code is the nearest one, exact tiles round-trip;
* exact binary32 arithmetic of the tile: the scale bits equal RN32(amax/448)
  from exact rational rounding (all 128 bf16 mantissas, binary32-subnormal
  scales included), and each code is the encoding of the exactly rounded
  quotient RN32(x/scale) over every bf16 magnitude up to several amax values;
* layout invariants of the store: replicas identical, RoPE bits verbatim,
  each row dequantizes to its token's input at the documented offsets,
  every byte outside the written rows unchanged, invalid slots counted,
  token order irrelevant, R replicas == R single-replica inserts.

* the reader side (dequantizing gather): hand-derived products and their
  bf16 rounding (``golden/gather_hand_values.txt``), every finite code times a
  few hundred scales against integer round-to-nearest-even arithmetic, a
  bit-exact round trip of tiles whose values and scales are exact, the
  half-step error bound on random rows, zero rows for padded and out-of-range
  slots.

``tests/test_oracle_plants.py`` builds copies of the oracle with planted
mistakes and checks that at least one pin fails for each.
"""
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


# ---------------------------------------------------------------------------
# independent helpers written from the OCP FP8 E4M3 definition
# ---------------------------------------------------------------------------

def e4m3_decode(codes):
    """Decode e4m3fn codes to float64 (0x7F/0xFF -> nan)."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    val = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e.astype(np.float64) - 10))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


def e4m3_step(codes):
    """Spacing of the e4m3 grid at each code's binade: 2^(max(E,1) - 10)."""
    e = (np.asarray(codes, dtype=np.int64) >> 3) & 0xF
    return np.exp2(np.maximum(e, 1).astype(np.float64) - 10)


def e4m3_encode_bits(v):
    """Round-to-nearest-even saturating binary32 -> e4m3fn by bit manipulation."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    u = v.view(np.uint32).astype(np.int64)
    sign = (u >> 24) & 0x80
    mag = u & 0x7FFFFFFF
    f = np.abs(v.astype(np.float64))
    # below 2^-6 the grid is uniform with spacing 2^-9: scale exactly, round half to even
    q_sub = np.rint(np.minimum(f, 1.0) * 512.0).astype(np.int64)
    # normal range: keep 3 mantissa bits, round on the 20 dropped bits
    e = (mag >> 23) - 127
    mant = mag & 0x7FFFFF
    q = mant >> 20
    rem = mant & 0xFFFFF
    up = (rem > 0x80000) | ((rem == 0x80000) & ((q & 1) == 1))
    q = q + up
    e = np.where(q == 8, e + 1, e)
    q = np.where(q == 8, 0, q)
    over = (e > 8) | ((e == 8) & (q == 7))
    normal = ((e + 7) << 3) | q
    code = np.where(f < 2.0 ** -6, q_sub, np.where(over, 0x7E, normal))
    code = np.where(f >= 448.0, 0x7E, code)
    return (code | sign).astype(np.uint8)


def bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_rne(x):
    """binary32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def load_hand_codes():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_hand_codes.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split(None, 2)
            rows.append((float.fromhex(parts[0]), int(parts[1], 16), parts[2] if len(parts) > 2 else ""))
    return rows


def _all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (b >> 7) & 0xFF
    return b[exp != 0xFF]


# ---------------------------------------------------------------------------
# encoder pins
# ---------------------------------------------------------------------------

def pin_hand_codes(orc):
    rows = load_hand_codes()
    vals = np.array([r[0] for r in rows], dtype=np.float32)
    want = np.array([r[1] for r in rows], dtype=np.uint8)
    got = orc.e4m3_encode(vals)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "hand codes: " + "; ".join(
        f"{rows[i][0]!r} -> {got[i]:#04x}, want {want[i]:#04x} ({rows[i][2]})" for i in bad[:8])


def encoder_sweep_inputs():
    """Every finite bf16 pattern, each with several low-16-bit completions
    (0: ties live here; 1 / 0xFFFF: just off a tie; 0x8000: middle), plus the
    pattern divided by a few tile scales."""
    hi = _all_finite_bf16().astype(np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0xFFFF], dtype=np.uint32)
    u = (hi[:, None] | lows[None, :]).reshape(-1)
    base = u.view(np.float32)
    base = base[np.isfinite(base)]
    with np.errstate(over="ignore"):
        extra = [base.astype(np.float32) / np.float32(s) for s in (448.0, 3.7, 2.0 ** -20, 1e-30)]
    return np.concatenate([base] + [e[np.isfinite(e)] for e in extra]).astype(np.float32)


def pin_encoder_bruteforce(orc):
    v = encoder_sweep_inputs()
    got = orc.e4m3_encode(v)
    want = e4m3_encode_bits(v)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} encoder mismatches vs bit-level RNE, e.g. " + ", ".join(
        f"{float(v[i]).hex()} -> {got[i]:#04x} want {want[i]:#04x}" for i in bad[:6])


def pin_encoder_torch(orc):
    import torch
    v = encoder_sweep_inputs()
    v = v[np.abs(v) < 464.0]
    got = orc.e4m3_encode(v)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches vs torch float8_e4m3fn cast, e.g. " + ", ".join(
        f"{float(v[i]).hex()} -> {got[i]:#04x} want {want[i]:#04x}" for i in bad[:6])


def pin_encoder_nearest(orc):
    """The code is a nearest grid point of v (ties: even) for |v| < 448 -- checked
    against the decoded neighbours, a closed-form property."""
    v = encoder_sweep_inputs()
    v = v[np.abs(v) < 448.0]
    c = orc.e4m3_encode(v).astype(np.int64)
    d = e4m3_decode(c)
    x = v.astype(np.float64)
    assert np.all(np.signbit(d) == np.signbit(x)), "sign not preserved"
    mag = c & 0x7F
    err = np.abs(x - d)
    for nb in (mag - 1, mag + 1):
        ok = (nb >= 0) & (nb <= 0x7E)
        dn = e4m3_decode(np.where(ok, nb, 0)) * np.where(np.signbit(x), -1.0, 1.0)
        en = np.abs(x - dn)
        worse = ok & (err > en)
        assert not np.any(worse), f"not nearest at {x[np.argmax(worse)]!r}"
        tie = ok & (err == en)
        assert not np.any(tie & (mag & 1 == 1)), "tie not resolved to even"


# ---------------------------------------------------------------------------
# tile pins
# ---------------------------------------------------------------------------

def _random_tiles(rng, n):
    kinds = []
    t = rng.standard_normal((n, 128))
    kinds.append(t)
    heavy = rng.standard_t(3, size=(n, 128)) * np.exp(2 * rng.standard_normal((n, 1)))
    kinds.append(heavy)
    small = rng.standard_normal((n, 128)) * 1e-30
    kinds.append(small)
    big = rng.standard_normal((n, 128)) * 1e30
    kinds.append(big)
    out = np.concatenate(kinds).astype(np.float32)
    return f32_to_bf16_rne(out)


def pin_tile_exact(orc):
    """Tiles built from e4m3 values with amax = 448 * 2^k: scale is exactly 2^k and
    the codes are the ones the values came from (a closed form)."""
    rng = np.random.default_rng(11)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.int64)
    for k in (0, -7, 5, -60, 60):
        codes = rng.choice(finite, size=(64, 128))
        codes[np.arange(64), rng.integers(0, 128, 64)] = rng.choice([0x7E, 0xFE], 64)
        vals = e4m3_decode(codes) * 2.0 ** k
        bits = f32_to_bf16_rne(vals.astype(np.float32))
        assert np.all(bf16_to_f32(bits).astype(np.float64) == vals)
        got_c, got_s = orc.quant_tiles(bits)
        assert np.all(got_s == np.float32(2.0 ** k)), f"scale != 2^{k}: {got_s[:4]}"
        assert np.array_equal(got_c.astype(np.int64), codes), f"exact tile codes differ (k={k})"


def pin_tile_invariants(orc):
    rng = np.random.default_rng(12)
    bits = _random_tiles(rng, 2000)
    codes, scales = orc.quant_tiles(bits)
    x = bf16_to_f32(bits).astype(np.float64)
    amax = np.abs(x).max(axis=1)
    nz = amax > 0
    # the largest-magnitude elements map to +-448
    top = (np.abs(x) == amax[:, None]) & nz[:, None]
    assert np.all((codes[top] & 0x7F) == 0x7E), "amax element not at 0x7E"
    assert np.all((codes[nz] & 0x7F).max(axis=1) == 0x7E)
    # scale lies within an ulp of amax/448 (tolerance wide enough for any rounding)
    s = scales.astype(np.float64)
    rel = np.abs(s[nz] * 448.0 - amax[nz]) / amax[nz]
    assert np.all(rel <= 2.0 ** -23), f"scale off amax/448 by {rel.max()}"
    # dequantization within half an e4m3 step at the tile scale (+ binary32 quotient rounding)
    d = e4m3_decode(codes) * s[:, None]
    bound = 0.5 * e4m3_step(codes) * s[:, None] + np.abs(x) * 2.0 ** -24
    err = np.abs(d - x)
    assert np.all(err[nz] <= bound[nz] * (1 + 1e-12)), f"dequant error {np.max(err - bound)} above bound"
    # signs: nonzero inputs keep their sign; codes of zero tiles are zero
    neg = (x < 0) & nz[:, None]
    assert np.all(codes[neg] & 0x80), "negative input lost its sign"
    assert np.all(codes[~nz] == 0) and np.all(scales[~nz] == 0)


def pin_tile_nearest(orc):
    """Each code is the nearest grid point to x / scale, up to the binary32 rounding
    of the quotient (2^-24 relative)."""
    rng = np.random.default_rng(13)
    bits = _random_tiles(rng, 500)
    codes, scales = orc.quant_tiles(bits)
    x = bf16_to_f32(bits).astype(np.float64)
    s = scales.astype(np.float64)
    nz = s > 0
    q = np.where(nz[:, None], x / np.where(nz, s, 1.0)[:, None], 0.0)
    c = codes.astype(np.int64)
    mag = c & 0x7F
    sgn = np.where(np.signbit(q), -1.0, 1.0)
    err = np.abs(q - e4m3_decode(c))
    slack = np.abs(q) * 2.0 ** -23
    for nb in (mag - 1, mag + 1):
        ok = (nb >= 0) & (nb <= 0x7E) & nz[:, None]
        en = np.abs(q - sgn * e4m3_decode(np.where(ok, nb, 0)))
        assert not np.any(ok & (err > en + slack)), "code not nearest to x/scale"


# Exponent fields of the amax values the exact pins sweep (bf16 biased exponents):
# 0 is a bf16 subnormal amax; up to 9 the scale amax/448 is a binary32 subnormal;
# 71/72 straddle the smallest scale (2^-64) of the kernels' division-free path;
# 254 is the largest finite binade.
EXACT_AMAX_EXPONENTS = (0, 1, 2, 8, 9, 10, 11, 40, 71, 72, 73, 100, 126, 127, 128, 134, 135, 200, 253, 254)


def _tiles_with_amax(rng, amax_bits, n_per):
    """n_per tiles for each positive bf16 amax pattern: element 0 is +-amax, the
    other 127 are random bf16 values of magnitude <= amax (uniform over the bit
    patterns, which order like the magnitudes), random signs."""
    ab = np.repeat(np.asarray(amax_bits, dtype=np.int64), n_per)
    mags = (rng.random((ab.size, 128)) * (ab[:, None] + 1)).astype(np.int64)
    mags[:, 0] = ab
    signs = rng.integers(0, 2, size=mags.shape).astype(np.int64) << 15
    return (mags | signs).astype(np.uint16)


def pin_tile_scale_exact(orc):
    """The stored tile scale is RN32(amax / 448) bit for bit (reading: binary32
    division, round to nearest even, subnormals kept), against an exact rational
    rounding, for all 128 bf16 mantissas at exponents from a bf16 subnormal amax
    (binary32-subnormal scales) to the largest binade; and every code is the e4m3
    encoding of RN32(x / scale), the quotient rounded exactly."""
    from fractions import Fraction
    from exact_fp import rn32, rn32_div, f32_bits
    rng = np.random.default_rng(21)
    amax_bits = [(e << 7) | m for e in EXACT_AMAX_EXPONENTS for m in range(128) if (e << 7) | m]
    bits = _tiles_with_amax(rng, amax_bits, 1)
    codes, scales = orc.quant_tiles(bits)
    want = np.array([rn32(Fraction(float(bf16_to_f32(np.uint16(a)))) / 448) for a in amax_bits], np.float32)
    bad = np.nonzero(scales.view(np.uint32) != want.view(np.uint32))[0]
    assert bad.size == 0, f"{bad.size} scales differ from RN32(amax/448), e.g. " + ", ".join(
        f"amax {amax_bits[i]:#06x}: {float(scales[i]).hex()} want {float(want[i]).hex()}" for i in bad[:4])
    assert np.any((want > 0) & (want < np.finfo(np.float32).tiny)), "no binary32-subnormal scale swept"
    # the quotient, rounded exactly, then the independent bit-level encoder
    x = bf16_to_f32(bits)
    q = rn32_div(x, want[:, None])
    want_codes = e4m3_encode_bits(q)
    bad = np.argwhere(codes != want_codes)
    assert bad.size == 0, f"{len(bad)} codes differ from e4m3(RN32(x/scale)), e.g. " + ", ".join(
        f"x {float(x[i, j]).hex()} / {float(want[i]).hex()}: {codes[i, j]:#04x} want {want_codes[i, j]:#04x}"
        for i, j in bad[:4])
    # the integer divider itself agrees with exact rational rounding on a sample
    # (magnitudes: a Fraction has no signed zero)
    for i, j in zip(rng.integers(0, len(amax_bits), 300), rng.integers(0, 128, 300)):
        exact = rn32(abs(Fraction(float(x[i, j]))) / Fraction(float(want[i])))
        assert f32_bits(abs(float(q[i, j]))) == f32_bits(exact), (float(x[i, j]), float(want[i]))


# amax values whose tiles cover every bf16 magnitude up to them (both signs):
# scale 1 (448), a scale with a long binary expansion (1.0 -> RN32(1/448)), the
# next pattern above 448, a mid exponent, the smallest fast-path amax, a
# binary32-subnormal scale, the smallest bf16 subnormal and the largest bf16;
# and three mantissas (0x0A, 0x44, 0x18) for which a multiply by RN32(1/scale)
# lands on the other side of an e4m3 rounding boundary than RN32(x/scale) does
# for some x (15, 30 and 15 values; found by exhaustive search over all 128).
SWEEP_AMAX_BITS = (0x43E0, 0x3F80, 0x43E1, 0x4049, 0x2400, 0x0480, 0x0001, 0x7F7F, 0x3B9D, 0x5F11,
                   0x3F8A, 0x3FC4, 0x4A98)


def pin_tile_quotient_sweep(orc):
    """Over every bf16 magnitude up to each of several amax values (both signs),
    the tile's codes are e4m3(RN32(x / RN32(amax / 448))) with both roundings
    exact: catches a reciprocal multiply, a contracted or reordered quotient."""
    from fractions import Fraction
    from exact_fp import rn32, rn32_div
    rng = np.random.default_rng(22)
    failures = []
    for ab in SWEEP_AMAX_BITS:
        mags = np.arange(ab + 1, dtype=np.int64)
        vals = np.concatenate([mags, mags | 0x8000])
        vals = vals[rng.permutation(vals.size)]
        n_tiles = -(-vals.size // 127)
        body = np.resize(vals, n_tiles * 127).reshape(n_tiles, 127)     # wraps: every value at least once
        bits = np.concatenate([np.full((n_tiles, 1), ab), body], axis=1).astype(np.uint16)
        codes, scales = orc.quant_tiles(bits)
        scale = np.float32(rn32(Fraction(float(bf16_to_f32(np.uint16(ab)))) / 448))
        assert np.all(scales.view(np.uint32) == np.uint32(scale.view(np.uint32))), f"amax {ab:#06x}: scale"
        x = bf16_to_f32(bits)
        want = e4m3_encode_bits(rn32_div(x, scale))
        bad = np.argwhere(codes != want)
        if bad.size:
            failures.append(f"amax {ab:#06x}: {len(bad)} codes differ from e4m3(RN32(x/scale)), e.g. " + ", ".join(
                f"{float(x[i, j]).hex()}: {codes[i, j]:#04x} want {want[i, j]:#04x}" for i, j in bad[:2]))
    assert not failures, "; ".join(failures)


def pin_tile_special(orc):
    # all-zero tile, including -0.0 elements: 128 zero bytes, scale +0
    z = np.zeros((2, 128), dtype=np.uint16)
    z[1, ::3] = 0x8000
    c, s = orc.quant_tiles(z)
    assert np.all(c == 0) and np.all(s == 0) and not np.any(np.signbit(s))
    # -0.0 in a non-zero tile keeps its sign
    t = np.zeros((1, 128), dtype=np.uint16)
    t[0, 0] = 0x3F80          # 1.0
    t[0, 1] = 0x8000          # -0.0
    t[0, 2] = 0xBF80          # -1.0
    c, s = orc.quant_tiles(t)
    assert s[0] == np.float32(1.0) / np.float32(448.0)
    assert c[0, 0] == 0x7E and c[0, 1] == 0x80 and c[0, 2] == 0xFE and c[0, 3] == 0x00
    # subnormal amax: smallest bf16 subnormal 2^-133; the scale is a binary32
    # subnormal and must not flush to zero
    t = np.zeros((1, 128), dtype=np.uint16)
    t[0, 5] = 0x0001
    t[0, 6] = 0x8001
    c, s = orc.quant_tiles(t)
    assert 0 < s[0] < np.finfo(np.float32).tiny, s[0]
    assert c[0, 5] == 0x7E and c[0, 6] == 0xFE and c[0, 0] == 0x00
    # large amax near the bf16 maximum
    t = np.full((1, 128), 0x7F7F, dtype=np.uint16)       # max finite bf16
    t[0, 1] = 0xFF7F
    c, s = orc.quant_tiles(t)
    assert c[0, 0] == 0x7E and c[0, 1] == 0xFE and np.isfinite(s[0])


# ---------------------------------------------------------------------------
# layout pins
# ---------------------------------------------------------------------------

class SmallCache:
    """Host replicas with a per-page guard: pages of 64 slots followed by 64 guard bytes."""

    def __init__(self, R, pages, layers=2, guard=64):
        self.R, self.pages, self.layers = R, pages, layers
        self.mps = 64 * 656 + guard
        self.ips = 64 * 132 + guard
        self.mls = pages * self.mps
        self.ils = pages * self.ips
        # the end canary is generous so that a planted out-of-range write stays in the buffer
        self.main = [np.full(layers * self.mls + 4096, 0x5A, np.uint8) for _ in range(R)]
        self.idx = [np.full(layers * self.ils + 4096, 0x5A, np.uint8) for _ in range(R)]
        self.main_guard = np.zeros(layers * self.mls + 4096, bool)
        self.idx_guard = np.zeros(layers * self.ils + 4096, bool)
        for l in range(layers):
            for p in range(pages):
                b = l * self.mls + p * self.mps + 64 * 656
                self.main_guard[b:b + guard] = True
                b = l * self.ils + p * self.ips + 64 * 132
                self.idx_guard[b:b + guard] = True
        self.main_guard[layers * self.mls:] = True
        self.idx_guard[layers * self.ils:] = True
        for r in range(R):
            self.main[r][self.main_guard] = 0xA5
            self.idx[r][self.idx_guard] = 0xA5

    def store(self, orc, layer, latent, rope, indexer, slots, replicas=None):
        reps = range(self.R) if replicas is None else replicas
        return orc.store([self.main[r] for r in reps], [self.idx[r] for r in reps],
                         num_pages=self.pages, main_page_stride=self.mps,
                         main_layer_stride=self.mls, idx_page_stride=self.ips,
                         idx_layer_stride=self.ils, layer=layer, latent=latent,
                         rope=rope, indexer=indexer, slot_mapping=slots)


def small_inputs(rng, T, capacity, n_pad, n_invalid):
    latent = f32_to_bf16_rne(rng.standard_normal((T, 512)).astype(np.float32))
    rope = f32_to_bf16_rne(rng.standard_normal((T, 64)).astype(np.float32))
    indexer = f32_to_bf16_rne(rng.standard_normal((T, 128)).astype(np.float32))
    slots = rng.permutation(capacity)[:T].astype(np.int64)
    pos = rng.permutation(T)
    slots[pos[:n_pad]] = -1
    inv = pos[n_pad:n_pad + n_invalid]
    slots[inv] = capacity + np.arange(len(inv))
    if len(inv):
        slots[inv[0]] = -2
    # padded / invalid tokens carry NaN rows: they must never be read into the cache
    bad = slots < 0
    bad |= slots >= capacity
    latent[bad] = 0x7FC1
    indexer[bad] = 0xFFC1
    latent[pos[n_pad + n_invalid]] = 0           # one all-zero row
    indexer[pos[n_pad + n_invalid]] = 0
    return latent, rope, indexer, slots


def check_rows_in_cache(cache, layer, latent, rope, indexer, slots, r=0):
    """Read each valid token's bytes at the documented offsets and check they
    encode the token's rows; returns the mask of bytes that were expected to be
    written."""
    capacity = cache.pages * 64
    mw = np.zeros(cache.main[0].size, bool)
    iw = np.zeros(cache.idx[0].size, bool)
    M, I = cache.main[r], cache.idx[r]
    for t, s in enumerate(slots):
        if s < 0 or s >= capacity:
            continue
        p, o = divmod(int(s), 64)
        mb = layer * cache.mls + p * cache.mps + o * 656
        ib = layer * cache.ils + p * cache.ips + o * 128
        sb = layer * cache.ils + p * cache.ips + 64 * 128 + o * 4
        mw[mb:mb + 656] = True
        iw[ib:ib + 128] = True
        iw[sb:sb + 4] = True
        row = M[mb:mb + 656]
        assert np.array_equal(row[528:656].view(np.uint16), rope[t]), f"rope bits differ, token {t}"
        scales = row[512:528].view(np.float32).astype(np.float64)
        x = bf16_to_f32(latent[t]).astype(np.float64).reshape(4, 128)
        c = row[:512].reshape(4, 128)
        _check_tile_bytes(x, c, scales, f"main token {t}")
        xi = bf16_to_f32(indexer[t]).astype(np.float64).reshape(1, 128)
        ci = I[ib:ib + 128].reshape(1, 128)
        si = I[sb:sb + 4].view(np.float32).astype(np.float64)
        _check_tile_bytes(xi, ci, si, f"indexer token {t}")
    return mw, iw


def _check_tile_bytes(x, c, s, what):
    amax = np.abs(x).max(axis=1)
    for j in range(x.shape[0]):
        if amax[j] == 0:
            assert s[j] == 0 and np.all(c[j] == 0), f"{what} tile {j}: zero tile not zero bytes"
            continue
        assert abs(s[j] * 448.0 - amax[j]) <= amax[j] * 2.0 ** -23, f"{what} tile {j}: scale {s[j]}"
        d = e4m3_decode(c[j]) * s[j]
        bound = 0.5 * e4m3_step(c[j]) * s[j] + np.abs(x[j]) * 2.0 ** -24
        assert np.all(np.abs(d - x[j]) <= bound * (1 + 1e-12)), f"{what} tile {j}: dequant error"
        assert (c[j] & 0x7F).max() == 0x7E, f"{what} tile {j}: no 0x7E code"


def pin_layout(orc):
    rng = np.random.default_rng(14)
    cache = SmallCache(R=2, pages=16)
    T = 256
    latent, rope, indexer, slots = small_inputs(rng, T, 16 * 64, n_pad=25, n_invalid=4)
    before_m = cache.main[0].copy()
    before_i = cache.idx[0].copy()
    n_inv = cache.store(orc, 1, latent, rope, indexer, slots)
    assert n_inv == 4, f"invalid count {n_inv} != 4"
    for r in range(1, cache.R):
        assert np.array_equal(cache.main[r], cache.main[0]), "main replicas differ"
        assert np.array_equal(cache.idx[r], cache.idx[0]), "indexer replicas differ"
    mw, iw = check_rows_in_cache(cache, 1, latent, rope, indexer, slots)
    assert np.array_equal(cache.main[0][~mw], before_m[~mw]), "main bytes outside written rows changed"
    assert np.array_equal(cache.idx[0][~iw], before_i[~iw]), "indexer bytes outside written rows changed"
    assert np.all(cache.main[0][cache.main_guard] == 0xA5) and np.all(cache.idx[0][cache.idx_guard] == 0xA5)
    # written byte count: 656 + 132 per valid token per replica
    n_valid = int(np.sum((slots >= 0) & (slots < 16 * 64)))
    assert mw.sum() == 656 * n_valid and iw.sum() == 132 * n_valid


def pin_layout_order_and_fanout(orc):
    rng = np.random.default_rng(15)
    T = 200
    latent, rope, indexer, slots = small_inputs(rng, T, 8 * 64, n_pad=20, n_invalid=2)
    a = SmallCache(R=3, pages=8)
    a.store(orc, 0, latent, rope, indexer, slots)
    # token order is irrelevant when valid slots are distinct
    perm = rng.permutation(T)
    b = SmallCache(R=3, pages=8)
    b.store(orc, 0, latent[perm], rope[perm], indexer[perm], slots[perm])
    for r in range(3):
        assert np.array_equal(a.main[r], b.main[r]) and np.array_equal(a.idx[r], b.idx[r]), "order matters"
    # R-way fan-out == inserting into each replica on its own (gather-then-insert)
    c = SmallCache(R=3, pages=8)
    for r in range(3):
        c.store(orc, 0, latent, rope, indexer, slots, replicas=[r])
    for r in range(3):
        assert np.array_equal(a.main[r], c.main[r]) and np.array_equal(a.idx[r], c.idx[r]), "fan-out != insert"


def pin_store_empty(orc):
    cache = SmallCache(R=1, pages=2)
    before = cache.main[0].copy()
    e = np.zeros((0, 512), np.uint16)
    n = cache.store(orc, 0, e, np.zeros((0, 64), np.uint16), np.zeros((0, 128), np.uint16),
                    np.zeros(0, np.int64))
    assert n == 0 and np.array_equal(before, cache.main[0])


# ---------------------------------------------------------------------------
# reader-side pins (dequantizing gather)
# ---------------------------------------------------------------------------

def load_gather_hand_values():
    rows = []
    with open(os.path.join(GOLDEN, "gather_hand_values.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, s, b = line.split()[:3]
            rows.append((int(c, 16), np.array([int(s, 16)], np.uint32).view(np.float32)[0], int(b, 16)))
    return rows


def pin_gather_hand_values(orc):
    for code, scale, want in load_gather_hand_values():
        got = int(orc.dequant_tile(np.array([code], np.uint8), scale)[0])
        assert got == want, f"dequant {code:#04x} * {float(scale)!r}: {got:#06x} != {want:#06x}"


def _gather(orc, cache, layer, slots, r=0):
    return orc.gather(cache.main[r], cache.idx[r], num_pages=cache.pages, main_page_stride=cache.mps,
                      main_layer_stride=cache.mls, idx_page_stride=cache.ips, idx_layer_stride=cache.ils,
                      layer=layer, slot_mapping=slots)


def pin_gather_roundtrip_exact(orc):
    """Tiles of e4m3 values with amax 448 * 2^k: the scale is exactly 2^k, every
    quotient is exactly representable, and value * 2^k is exact in bf16 (4
    significant bits), so store followed by gather must give back the input bits."""
    rng = np.random.default_rng(21)
    T = 64
    grid = np.array([c for c in range(0x7F) if c != 0], np.uint8)
    vals = e4m3_decode(grid)
    lat = np.empty((T, 512), np.float64)
    idx = np.empty((T, 128), np.float64)
    for t in range(T):
        for j in range(4):
            k = int(rng.integers(-20, 21))
            v = rng.choice(vals, 128) * rng.choice([-1.0, 1.0], 128)
            v[int(rng.integers(0, 128))] = 448.0 * (1 if rng.random() < 0.5 else -1)
            lat[t, 128 * j:128 * (j + 1)] = v * 2.0 ** k
        k = int(rng.integers(-20, 21))
        v = rng.choice(vals, 128)
        v[0] = 448.0
        idx[t] = v * 2.0 ** k
    latent = f32_to_bf16_rne(lat.astype(np.float32))
    indexer = f32_to_bf16_rne(idx.astype(np.float32))
    assert np.array_equal(bf16_to_f32(latent).astype(np.float64), lat)        # exact in bf16
    rope = f32_to_bf16_rne(rng.standard_normal((T, 64)).astype(np.float32))
    cache = SmallCache(R=1, pages=4)
    slots = rng.permutation(4 * 64)[:T].astype(np.int64)
    cache.store(orc, 0, latent, rope, indexer, slots)
    g_lat, g_rope, g_idx, bad = _gather(orc, cache, 0, slots)
    assert bad == 0
    assert np.array_equal(g_lat, latent), "exact tiles do not round-trip (latent)"
    assert np.array_equal(g_idx, indexer), "exact tiles do not round-trip (indexer)"
    assert np.array_equal(g_rope, rope), "RoPE bits not returned verbatim"


def _rne_int(M, E, p, emin):
    """M * 2^E (M a positive Python int, the value exact) rounded to p significant
    bits, to nearest with ties to even, with the quantum at least 2^emin (the
    subnormal range): returns (M2, E2), the rounded value being M2 * 2^E2."""
    shift = max(M.bit_length() - p, emin - E)
    if shift <= 0:
        return M, E
    q, r = M >> shift, M & ((1 << shift) - 1)
    half = 1 << (shift - 1)
    if r > half or (r == half and q & 1):
        q += 1
    return q, E + shift


def _bf16_bits_of(neg, M, E):
    """bf16 bit pattern of (-1)^neg * M * 2^E, M * 2^E already a bf16 value."""
    sign = 0x8000 if neg else 0
    if M == 0:
        return sign
    n = M.bit_length()
    e = E + n - 1                                   # exponent of the leading bit
    if e >= -126:
        frac = (M << (8 - n)) & 0x7F if n <= 8 else (M >> (n - 8)) & 0x7F
        return sign | ((e + 127) << 7) | frac
    return sign | (M << (E + 133))                  # subnormal: M * 2^E = m * 2^-133


def _dequant_want(code, scale):
    """bf16 bits of RN_bf16(RN32(value(code) * scale)) with integer arithmetic only:
    value(code) from the OCP E4M3 definition (exponent field E, mantissa M: E = 0 gives
    M * 2^-9, else (8 + M) * 2^(E - 10)), scale from its binary32 fields."""
    neg_c = bool(code & 0x80)
    ef, mf = (code >> 3) & 15, code & 7
    Mv, Ev = (mf, -9) if ef == 0 else (8 + mf, ef - 10)
    u = int(np.float32(scale).view(np.uint32))
    es, ms = (u >> 23) & 0xFF, u & 0x7FFFFF
    Ms, Es = (ms, -149) if es == 0 else (ms | 0x800000, es - 150)
    neg = neg_c != bool(u >> 31)
    M, E = Mv * Ms, Ev + Es
    if M == 0:
        return 0x8000 if neg else 0
    M, E = _rne_int(M, E, 24, -149)                 # the binary32 product
    if M == 0:
        return 0x8000 if neg else 0
    M, E = _rne_int(M, E, 8, -133)                  # then bf16
    return _bf16_bits_of(neg, M, E)


def pin_gather_dequant_exhaustive(orc):
    """Every finite e4m3 code (254 patterns, both signs, subnormal codes included)
    times each of about 330 scales -- powers of two from 2^-140 to 2^110, random
    binary32 values over the same range, binary32 subnormals, and RN32(amax / 448)
    of random bf16 amax (the scales a store writes) -- dequantizes to
    RN_bf16(RN32(value * scale)) bit for bit, against integer round-to-nearest-even
    arithmetic written from the definitions (products whose binary32 or bf16
    result is subnormal included)."""
    from fractions import Fraction
    from exact_fp import rn32
    rng = np.random.default_rng(23)
    scales = [2.0 ** k for k in range(-140, 111, 5)]
    ex = rng.integers(-130, 100, 200)
    scales += [float(np.float32(rng.uniform(1.0, 2.0) * 2.0 ** int(k))) for k in ex]
    scales += [float(np.array([int(v)], np.uint32).view(np.float32)[0]) for v in rng.integers(1, 1 << 23, 20)]
    amax = rng.integers(1, 0x7F80, 60).astype(np.uint16)
    scales += [rn32(Fraction(float(bf16_to_f32(a))) / 448) for a in amax]
    scales = [s for s in scales if s > 0]
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    subnormal_out = 0
    for s in scales:
        got = orc.dequant_tile(codes, np.float32(s))
        want = np.array([_dequant_want(int(c), s) for c in codes], np.uint16)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"{bad.size} codes at scale {float(np.float32(s)).hex()} differ, e.g. " + ", ".join(
            f"{codes[i]:#04x}: {got[i]:#06x} want {want[i]:#06x}" for i in bad[:4])
        subnormal_out += int(np.count_nonzero(((want & 0x7F80) == 0) & ((want & 0x7F) != 0)))
    assert subnormal_out > 0, "no product with a bf16-subnormal result swept"


def pin_gather_bound_and_pads(orc):
    """Random rows: the gathered value is within half an e4m3 step (at the tile
    scale) of the input, plus the binary32 and bf16 roundings; padded and
    out-of-range slots give zero rows, out-of-range ones are counted."""
    rng = np.random.default_rng(22)
    T = 160
    latent, rope, indexer, slots = small_inputs(rng, T, 8 * 64, n_pad=10, n_invalid=3)
    cache = SmallCache(R=2, pages=8)
    cache.store(orc, 0, latent, rope, indexer, slots)
    g_lat, g_rope, g_idx, bad = _gather(orc, cache, 0, slots, r=1)
    assert bad == 3, f"out-of-range count {bad} != 3"
    valid = (slots >= 0) & (slots < 8 * 64)
    assert np.all(g_lat[~valid] == 0) and np.all(g_rope[~valid] == 0) and np.all(g_idx[~valid] == 0), \
        "padded / out-of-range rows not zero"
    assert np.array_equal(g_rope[valid], rope[valid]), "RoPE bits not returned verbatim"
    for x_bits, g_bits, ntile in ((latent, g_lat, 4), (indexer, g_idx, 1)):
        x = bf16_to_f32(x_bits[valid]).astype(np.float64).reshape(-1, ntile, 128)
        g = bf16_to_f32(g_bits[valid]).astype(np.float64).reshape(-1, ntile, 128)
        amax = np.abs(x).max(axis=2, keepdims=True)
        scale = amax / 448.0
        # e4m3 half step at the dequantized magnitude, in units of the scale
        q = np.abs(x) / np.where(scale > 0, scale, 1.0)
        step = np.exp2(np.maximum(np.floor(np.log2(np.maximum(q, 2.0 ** -6))), -6) - 3)
        bound = 0.5 * step * scale * (1 + 2.0 ** -20) + np.abs(x) * 2.0 ** -22 + np.abs(g) * 2.0 ** -8
        assert np.all(np.abs(g - x) <= bound), "gathered value outside the dequantization bound"


def pin_epoch(orc):
    assert orc.epoch_after(0, 61 * 100) == 6100
    assert orc.epoch_after(5, 0) == 5


ALL_PINS = [pin_hand_codes, pin_encoder_bruteforce, pin_encoder_torch, pin_encoder_nearest,
            pin_tile_exact, pin_tile_invariants, pin_tile_nearest, pin_tile_special,
            pin_tile_scale_exact, pin_tile_quotient_sweep,
            pin_layout, pin_layout_order_and_fanout, pin_store_empty, pin_epoch,
            pin_gather_hand_values, pin_gather_roundtrip_exact, pin_gather_dequant_exhaustive,
            pin_gather_bound_and_pads]
