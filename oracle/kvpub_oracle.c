/*
 * kvpub_oracle.c -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.
 *
 * A plain, slow, obviously-correct CPU definition of the replicated FP8
 * KV cache-store.  Only the test suite, the package's smoke check and the
 * benchmark's CPU-baseline leg may load the library built from this file;
 * the GPU library never calls it and shares no code, header, table or
 * constant generator with it.
 *
 * What it computes (vLLM PR #52863, "[Kernel][PCP] Publish replicated KV
 * updates through PyTorch symmetric memory"):
 *   - Summary / Design: each producer quantizes its final Main-KV and
 *     Indexer-K rows to FP8 once and writes those bytes into every replica
 *     of the paged KV cache;
 *   - "AS-IS: gather then insert" diagram: the fallback path inserts the same
 *     rows into each rank's local cache; the direct path must leave every
 *     replica byte-identical to that result (Correctness section), including
 *     padded and invalid slots and untouched guard bytes.
 * The result therefore has a plain definition: every replica equals the
 * cache before the call with each valid token's slot row replaced by the
 * encoding of its rows, and no other byte changed.  This file writes that
 * definition out: encode each token once ("gather"), then copy the bytes
 * into each replica in turn ("insert").
 *
 * The pages name the FP8 Main-KV format (fp8_ds_mla) without printing its
 * bytes or its scaling rule.  The readings taken here:
 *   - tile = 128 consecutive elements; scale = amax / 448 in binary32;
 *     code = e4m3(x / scale) with x / scale a binary32 division;
 *     an all-zero tile has scale +0 and all codes 0x00;
 *   - e4m3 = OCP 8-bit floating point E4M3 ("fn": no infinities, max 448),
 *     round to nearest, ties to even, magnitudes >= 448 saturate to 0x7E;
 *   - Main-KV row (656 B) = 512 latent codes | 4 fp32 tile scales (LE) |
 *     64 RoPE bf16 values copied bit for bit (LE);
 *   - Indexer-K page = 64 x 128 codes followed by 64 fp32 scales; one tile
 *     per token (the whole 128-element row);
 *   - slot s -> page s / 64, offset s % 64; s == -1 is a padded token and is
 *     skipped; any other s outside [0, pages*64) is skipped and counted.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math (no FMA contraction, IEEE
 * binary32 division with subnormals; on x86-64 float arithmetic is SSE).
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define KVO_SLOTS_PER_PAGE 64
#define KVO_LATENT 512
#define KVO_ROPE 64
#define KVO_INDEXER 128
#define KVO_TILE 128
#define KVO_MAIN_ROW_BYTES 656
#define KVO_IDX_CODES_BYTES 128

/* ------------------------------------------------------------------ */
/* bit helpers                                                         */
/* ------------------------------------------------------------------ */

/* bf16 -> binary32: a bf16 value is the upper 16 bits of a binary32 value. */
static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t float_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

static void put_le32(uint8_t *dst, uint32_t v)
{
    dst[0] = (uint8_t)(v & 0xFFu);
    dst[1] = (uint8_t)((v >> 8) & 0xFFu);
    dst[2] = (uint8_t)((v >> 16) & 0xFFu);
    dst[3] = (uint8_t)((v >> 24) & 0xFFu);
}

/* ------------------------------------------------------------------ */
/* OCP FP8 E4M3 ("fn" variant)                                          */
/* ------------------------------------------------------------------ */

/*
 * Magnitude of the non-negative e4m3 code c in 0x00..0x7E, from the format
 * definition: exponent field E = c >> 3 (bias 7), mantissa M = c & 7.
 *   E == 0: subnormal, value = M/8 * 2^-6 = M * 2^-9
 *   E >= 1: normal,    value = (1 + M/8) * 2^(E-7) = (8 + M) * 2^(E-10)
 * 0x7F (E=15, M=7) is NaN and is never produced by the encoder.
 * Every such value is exact in binary64.
 */
static double e4m3_magnitude(unsigned c)
{
    unsigned e = c >> 3, m = c & 7u;
    double v;
    int k;
    if (e == 0) {
        v = (double)m;
#if defined(KVO_PLANT) && KVO_PLANT == 12
        for (k = 0; k < 10; ++k) v *= 0.5;          /* planted: subnormal step halved */
#else
        for (k = 0; k < 9; ++k) v *= 0.5;           /* M * 2^-9 */
#endif
        return v;
    }
    v = (double)(8u + m);
    if ((int)e >= 10) {
        for (k = 10; k < (int)e; ++k) v *= 2.0;     /* (8+M) * 2^(E-10) */
    } else {
        for (k = (int)e; k < 10; ++k) v *= 0.5;
    }
    return v;
}

#define KVO_E4M3_MAX_CODE 0x7Eu   /* 448 */

/*
 * Round-to-nearest-even, saturating binary32 -> e4m3fn.
 * Definition: the e4m3 value nearest to v; on an exact tie the code whose
 * mantissa LSB is 0; magnitudes >= 448 give +-448 (0x7E / 0xFE), never NaN;
 * the sign bit is v's sign bit (so -0.0 and negatives that round to zero
 * give 0x80).
 * Distances are computed in binary64 and are exact: both operands are
 * within a factor of two of each other (Sterbenz), or one of them is zero.
 */
#if defined(KVO_PLANT) && KVO_PLANT == 3
#define KVO_SIGN_OF(u) 0u                        /* planted: sign dropped */
#else
#define KVO_SIGN_OF(u) (((u) >> 24) & 0x80u)
#endif
uint8_t kvo_e4m3_encode(float v)
{
    uint32_t u = float_bits(v);
    uint8_t sign = (uint8_t)KVO_SIGN_OF(u);
    double mag = (double)v;
    unsigned lo, hi;
    double below, above;

    if ((u & 0x7FFFFFFFu) > 0x7F800000u)          /* NaN: outside the contract */
        return (uint8_t)(sign | 0x7Fu);
    if (mag < 0.0) mag = -mag;
#if defined(KVO_PLANT) && KVO_PLANT == 2
    if (mag >= 464.0) return (uint8_t)(sign | 0x7Fu);   /* planted: overflow to NaN */
#endif
    if (mag >= e4m3_magnitude(KVO_E4M3_MAX_CODE))
        return (uint8_t)(sign | KVO_E4M3_MAX_CODE);

    /* bisection: lo = largest code with magnitude <= mag (code 0 is 0.0) */
    lo = 0u;
    hi = KVO_E4M3_MAX_CODE;                        /* magnitude(hi) > mag */
    while (hi - lo > 1u) {
        unsigned mid = (lo + hi) / 2u;
        if (e4m3_magnitude(mid) <= mag) lo = mid; else hi = mid;
    }
    below = mag - e4m3_magnitude(lo);
    above = e4m3_magnitude(hi) - mag;
#if defined(KVO_PLANT) && KVO_PLANT == 13
    (void)above;
    return (uint8_t)(sign | lo);                   /* planted: truncation */
#endif
    if (below < above) return (uint8_t)(sign | lo);
    if (above < below) return (uint8_t)(sign | hi);
#if defined(KVO_PLANT) && KVO_PLANT == 1
    return (uint8_t)(sign | hi);                   /* planted: ties away from zero */
#endif
    return (uint8_t)(sign | ((lo & 1u) ? hi : lo)); /* tie: even mantissa */
}

void kvo_e4m3_encode_array(const float *v, size_t n, uint8_t *out)
{
    size_t i;
    for (i = 0; i < n; ++i) out[i] = kvo_e4m3_encode(v[i]);
}

/* ------------------------------------------------------------------ */
/* one 128-element tile                                                 */
/* ------------------------------------------------------------------ */

#if defined(KVO_PLANT) && KVO_PLANT == 4
#define KVO_E4M3_MAX_VALUE 447.0f                  /* planted: wrong range */
#else
#define KVO_E4M3_MAX_VALUE 448.0f
#endif

/*
 * Per-tile absmax scaling onto the e4m3 range:
 *   amax  = max_k |x_k|           (exact)
 *   scale = amax / 448            (binary32 division, RNE, subnormals kept)
 *   code_k = e4m3(x_k / scale)    (binary32 division, then the encoder)
 * amax == 0: scale = +0.0 and every code is 0x00.
 * Dequantization is code_k * scale.
 */
void kvo_quant_tile(const uint16_t *x, uint8_t *codes, float *scale_out)
{
    float amax = 0.0f, scale;
    int k, n = KVO_TILE;
#if defined(KVO_PLANT) && KVO_PLANT == 5
    n = KVO_TILE - 1;                              /* planted: last element ignored by amax */
#endif
    for (k = 0; k < n; ++k) {
        float a = bf16_to_float(x[k]);
        if (a < 0.0f) a = -a;
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        memset(codes, 0, KVO_TILE);
        *scale_out = 0.0f;
        return;
    }
#if defined(KVO_PLANT) && KVO_PLANT == 17
    scale = amax * (1.0f / KVO_E4M3_MAX_VALUE);    /* planted: multiply by RN(1/448) */
#else
    scale = amax / KVO_E4M3_MAX_VALUE;
#endif
#if defined(KVO_PLANT) && KVO_PLANT == 18
    {
        const float inv = 1.0f / scale;            /* planted: quotient by reciprocal multiply */
        for (k = 0; k < KVO_TILE; ++k)
            codes[k] = kvo_e4m3_encode(bf16_to_float(x[k]) * inv);
    }
#else
    for (k = 0; k < KVO_TILE; ++k)
        codes[k] = kvo_e4m3_encode(bf16_to_float(x[k]) / scale);
#endif
    *scale_out = scale;
}

void kvo_quant_tiles(const uint16_t *x, size_t n_tiles, uint8_t *codes, float *scales)
{
    size_t i;
    for (i = 0; i < n_tiles; ++i)
        kvo_quant_tile(x + i * KVO_TILE, codes + i * KVO_TILE, scales + i);
}

/* ------------------------------------------------------------------ */
/* rows                                                                 */
/* ------------------------------------------------------------------ */

/*
 * Main-KV row, 656 bytes:
 *   [0, 512)    e4m3 codes of latent[0..511], tile-major, element order
 *   [512, 528)  fp32 scales of latent tiles 0..3, little-endian
 *   [528, 656)  rope[0..63] bf16 bit patterns, little-endian, unchanged
 */
void kvo_main_row(const uint16_t *latent, const uint16_t *rope, uint8_t *row)
{
    float scales[4];
    int j, k;
    for (j = 0; j < 4; ++j)
        kvo_quant_tile(latent + KVO_TILE * j, row + KVO_TILE * j, &scales[j]);
    for (j = 0; j < 4; ++j) {
#if defined(KVO_PLANT) && KVO_PLANT == 6
        put_le32(row + KVO_LATENT + 4 * j, float_bits(scales[3 - j]));  /* planted */
#else
        put_le32(row + KVO_LATENT + 4 * j, float_bits(scales[j]));
#endif
    }
    for (k = 0; k < KVO_ROPE; ++k) {
#if defined(KVO_PLANT) && KVO_PLANT == 7
        row[528 + 2 * k] = (uint8_t)(rope[k] >> 8);        /* planted: big-endian */
        row[528 + 2 * k + 1] = (uint8_t)(rope[k] & 0xFFu);
#else
        row[528 + 2 * k] = (uint8_t)(rope[k] & 0xFFu);
        row[528 + 2 * k + 1] = (uint8_t)(rope[k] >> 8);
#endif
    }
}

/* Indexer-K row: 128 codes of the single 128-element tile + its fp32 scale (LE). */
void kvo_indexer_row(const uint16_t *indexer, uint8_t *codes, uint8_t *scale_le)
{
    float scale;
    kvo_quant_tile(indexer, codes, &scale);
    put_le32(scale_le, float_bits(scale));
}

/* Encode T tokens' rows without placing them (used to check gathered rows). */
void kvo_encode_rows(int64_t T,
                     const uint16_t *latent, int64_t latent_stride,
                     const uint16_t *rope, int64_t rope_stride,
                     const uint16_t *indexer, int64_t indexer_stride,
                     uint8_t *main_rows, uint8_t *idx_codes, uint8_t *idx_scales)
{
    int64_t t;
    for (t = 0; t < T; ++t) {
        kvo_main_row(latent + t * latent_stride, rope + t * rope_stride,
                     main_rows + t * KVO_MAIN_ROW_BYTES);
        kvo_indexer_row(indexer + t * indexer_stride,
                        idx_codes + t * KVO_IDX_CODES_BYTES, idx_scales + t * 4);
    }
}

/* ------------------------------------------------------------------ */
/* the store: gather (encode once), then insert into every replica      */
/* ------------------------------------------------------------------ */

/*
 * Replica r's Main-KV bytes for (layer l, page p, offset o) start at
 *   main_bases[r] + l*main_layer_stride + p*main_page_stride + o*656,
 * its Indexer-K codes at
 *   idx_bases[r] + l*idx_layer_stride + p*idx_page_stride + o*128,
 * and its Indexer-K scale at
 *   idx_bases[r] + l*idx_layer_stride + p*idx_page_stride + 64*128 + o*4.
 * Strides are in bytes; row strides of the inputs are in elements.
 * Returns the number of invalid slots (not -1 and outside [0, pages*64)).
 */
int64_t kvo_store(uint32_t num_replicas,
                  uint8_t *const *main_bases, uint8_t *const *idx_bases,
                  uint64_t num_pages,
                  uint64_t main_page_stride, uint64_t main_layer_stride,
                  uint64_t idx_page_stride, uint64_t idx_layer_stride,
                  uint32_t layer, int64_t num_tokens,
                  const uint16_t *latent, int64_t latent_stride,
                  const uint16_t *rope, int64_t rope_stride,
                  const uint16_t *indexer, int64_t indexer_stride,
                  const int64_t *slot_mapping)
{
    const int64_t capacity = (int64_t)(num_pages * KVO_SLOTS_PER_PAGE);
    int64_t invalid = 0, t;
    uint32_t r;
    uint8_t row[KVO_MAIN_ROW_BYTES], icodes[KVO_IDX_CODES_BYTES], iscale[4];

    for (t = 0; t < num_tokens; ++t) {
        int64_t s = slot_mapping[t];
        uint64_t page, off;
#if defined(KVO_PLANT) && KVO_PLANT == 10
        if (s < 0) { ++invalid; continue; }          /* planted: pads counted as invalid */
#endif
        if (s == -1) continue;                       /* padded token */
        if (s < 0 || s >= capacity) { ++invalid; continue; }
#if defined(KVO_PLANT) && KVO_PLANT == 9
        page = (uint64_t)s % KVO_SLOTS_PER_PAGE;     /* planted: page/offset swapped */
        off = (uint64_t)s / KVO_SLOTS_PER_PAGE;
        if (page >= num_pages || off >= KVO_SLOTS_PER_PAGE) { ++invalid; continue; }
#else
        page = (uint64_t)s / KVO_SLOTS_PER_PAGE;
        off = (uint64_t)s % KVO_SLOTS_PER_PAGE;
#endif

        /* gather: encode this token's rows once */
        kvo_main_row(latent + t * latent_stride, rope + t * rope_stride, row);
        kvo_indexer_row(indexer + t * indexer_stride, icodes, iscale);

        /* insert into every replica */
        for (r = 0; r < num_replicas; ++r) {
            uint8_t *mpage = main_bases[r] + (uint64_t)layer * main_layer_stride
                             + page * main_page_stride;
            uint8_t *ipage = idx_bases[r] + (uint64_t)layer * idx_layer_stride
                             + page * idx_page_stride;
#if defined(KVO_PLANT) && KVO_PLANT == 11
            if (r > 0) break;                        /* planted: one replica only */
#endif
            memcpy(mpage + off * KVO_MAIN_ROW_BYTES, row, KVO_MAIN_ROW_BYTES);
            memcpy(ipage + off * KVO_IDX_CODES_BYTES, icodes, KVO_IDX_CODES_BYTES);
#if defined(KVO_PLANT) && KVO_PLANT == 8
            memcpy(ipage + KVO_SLOTS_PER_PAGE * KVO_IDX_CODES_BYTES + off * 8, iscale, 4);
#else
            memcpy(ipage + KVO_SLOTS_PER_PAGE * KVO_IDX_CODES_BYTES + off * 4, iscale, 4);
#endif
        }
    }
    return invalid;
}

/* ------------------------------------------------------------------ */
/* the reader: dequantizing gather from one replica                     */
/* ------------------------------------------------------------------ */

/*
 * What the attention side reads back from a replica (vLLM PR #52863,
 * Summary and Design: the existing attention kernels keep reading the local
 * replica, in the fp8_ds_mla layout this path writes).  Readings taken here:
 *   - element k of a tile = bf16(RN32(value(code_k) * scale)): the e4m3 value
 *     (exact in binary32) times the tile's fp32 scale, rounded once to
 *     binary32, then rounded to bf16 (nearest, ties to even);
 *   - RoPE: the 64 stored bf16 values, bit for bit;
 *   - a padded (-1) or out-of-range slot gives an all-zero output row; the
 *     out-of-range ones are counted, as in the store.
 */
static uint32_t get_le32(const uint8_t *src)
{
    return (uint32_t)src[0] | ((uint32_t)src[1] << 8) | ((uint32_t)src[2] << 16)
           | ((uint32_t)src[3] << 24);
}

static float float_from_bits(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Signed value of the e4m3 code c (0x7F / 0xFF, NaN, are never stored). */
static double e4m3_value(uint8_t c)
{
#if defined(KVO_PLANT) && KVO_PLANT == 14
    return e4m3_magnitude(c & 0x7Fu);               /* planted: sign dropped on decode */
#else
    double m = e4m3_magnitude(c & 0x7Fu);
    return (c & 0x80u) ? -m : m;
#endif
}

/*
 * binary32 -> bf16, round to nearest, ties to even: of the two bf16 values
 * around v (t = v with its low 16 bits cleared, and the next bf16 away from
 * zero) take the nearer; on a tie the one with an even bit pattern.  The
 * distances are exact in binary64.  Finite input only.
 */
static uint16_t float_to_bf16(float v)
{
    uint16_t t = (uint16_t)(float_bits(v) >> 16);
#if defined(KVO_PLANT) && KVO_PLANT == 20
    if ((t & 0x7F80u) == 0) return (uint16_t)(t & 0x8000u);   /* planted: bf16 subnormals flushed */
#endif
    double lo = (double)bf16_to_float(t), hi = (double)bf16_to_float((uint16_t)(t + 1u));
    double dl = (double)v - lo, dh = hi - (double)v;
    if (dl < 0) dl = -dl;
    if (dh < 0) dh = -dh;
#if defined(KVO_PLANT) && KVO_PLANT == 15
    return t;                                        /* planted: truncation */
#endif
    if (dl < dh) return t;
    if (dh < dl) return (uint16_t)(t + 1u);
    return (t & 1u) ? (uint16_t)(t + 1u) : t;
}

/* n codes sharing one scale -> n bf16 values. */
void kvo_dequant_tile(const uint8_t *codes, float scale, size_t n, uint16_t *out)
{
    size_t k;
    for (k = 0; k < n; ++k) {
        float v = (float)e4m3_value(codes[k]);       /* exact */
        float p = v * scale;                          /* one binary32 rounding */
#if defined(KVO_PLANT) && KVO_PLANT == 19
        if (p != 0.0f && p < 1.17549435e-38f && p > -1.17549435e-38f)
            p = p < 0.0f ? -0.0f : 0.0f;              /* planted: subnormal products flushed */
#endif
        out[k] = float_to_bf16(p);
    }
}

/*
 * Gather tokens t = 0..T-1 from one replica (bases already at the replica;
 * same strides as kvo_store): latent_out[t][0..511], rope_out[t][0..63] and
 * indexer_out[t][0..127] (bf16 bit patterns, row strides in elements).
 * Returns the number of out-of-range slots (not -1).
 */
int64_t kvo_gather(const uint8_t *main_base, const uint8_t *idx_base, uint64_t num_pages,
                   uint64_t main_page_stride, uint64_t main_layer_stride,
                   uint64_t idx_page_stride, uint64_t idx_layer_stride,
                   uint32_t layer, int64_t num_tokens, const int64_t *slot_mapping,
                   uint16_t *latent_out, int64_t latent_stride,
                   uint16_t *rope_out, int64_t rope_stride,
                   uint16_t *indexer_out, int64_t indexer_stride)
{
    const int64_t capacity = (int64_t)(num_pages * KVO_SLOTS_PER_PAGE);
    int64_t invalid = 0, t;
    int j, k;

    for (t = 0; t < num_tokens; ++t) {
        int64_t s = slot_mapping[t];
        uint16_t *lo = latent_out + t * latent_stride;
        uint16_t *ro = rope_out + t * rope_stride;
        uint16_t *io = indexer_out + t * indexer_stride;
        const uint8_t *row, *ipage;
        uint64_t page, off;
        if (s != -1 && (s < 0 || s >= capacity)) ++invalid;
        if (s < 0 || s >= capacity) {                /* padded or out of range: zeros */
            memset(lo, 0, KVO_LATENT * sizeof *lo);
            memset(ro, 0, KVO_ROPE * sizeof *ro);
            memset(io, 0, KVO_INDEXER * sizeof *io);
            continue;
        }
        page = (uint64_t)s / KVO_SLOTS_PER_PAGE;
        off = (uint64_t)s % KVO_SLOTS_PER_PAGE;
        row = main_base + (uint64_t)layer * main_layer_stride + page * main_page_stride
              + off * KVO_MAIN_ROW_BYTES;
        ipage = idx_base + (uint64_t)layer * idx_layer_stride + page * idx_page_stride;
        for (j = 0; j < KVO_LATENT / KVO_TILE; ++j) {
#if defined(KVO_PLANT) && KVO_PLANT == 16
            float scale = float_from_bits(get_le32(row + KVO_LATENT + 4 * ((j + 1) % 4)));  /* planted */
#else
            float scale = float_from_bits(get_le32(row + KVO_LATENT + 4 * j));
#endif
            kvo_dequant_tile(row + j * KVO_TILE, scale, KVO_TILE, lo + j * KVO_TILE);
        }
        for (k = 0; k < KVO_ROPE; ++k) {
            const uint8_t *b = row + KVO_LATENT + 16 + 2 * k;
            ro[k] = (uint16_t)(b[0] | (b[1] << 8));
        }
        kvo_dequant_tile(ipage + off * KVO_IDX_CODES_BYTES,
                         float_from_bits(get_le32(ipage + KVO_SLOTS_PER_PAGE * KVO_IDX_CODES_BYTES
                                                  + off * 4)),
                         KVO_INDEXER, io);
    }
    return invalid;
}

/* Epoch after n fence executions starting from e0: each advances it by one. */
uint64_t kvo_epoch_after(uint64_t e0, uint64_t n_fences)
{
    return e0 + n_fences;
}

/* Build-variant tag, so tests can tell a planted-mistake build from the real one. */
int kvo_plant_id(void)
{
#if defined(KVO_PLANT)
    return KVO_PLANT;
#else
    return 0;
#endif
}
