/* Drives the CPU oracle on heap buffers of exactly the sizes its layout
 * needs, so that a build with AddressSanitizer and UndefinedBehaviorSanitizer
 * reports any byte it touches outside them and any undefined operation
 * (shifts, overflow, misaligned access) on the way.  Covers the store into
 * several replicas and layers with tight page and layer strides (the last
 * slot of the last page ends exactly at the end of the buffer), input rows
 * with strides wider than the row, padded and invalid slots of every kind,
 * all-zero, subnormal and largest-bf16 rows, an empty call, the gather with
 * tight outputs, and the encoder on special binary32 values.  Prints "ok" and
 * exits 0, else names the failed check. */
#include <float.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's entry points (oracle/kvpub_oracle.c) */
int64_t kvo_store(uint32_t num_replicas, uint8_t *const *main_bases, uint8_t *const *idx_bases,
                  uint64_t num_pages, uint64_t main_page_stride, uint64_t main_layer_stride,
                  uint64_t idx_page_stride, uint64_t idx_layer_stride, uint32_t layer, int64_t num_tokens,
                  const uint16_t *latent, int64_t latent_stride, const uint16_t *rope, int64_t rope_stride,
                  const uint16_t *indexer, int64_t indexer_stride, const int64_t *slot_mapping);
int64_t kvo_gather(const uint8_t *main_base, const uint8_t *idx_base, uint64_t num_pages,
                   uint64_t main_page_stride, uint64_t main_layer_stride, uint64_t idx_page_stride,
                   uint64_t idx_layer_stride, uint32_t layer, int64_t num_tokens, const int64_t *slot_mapping,
                   uint16_t *latent_out, int64_t latent_stride, uint16_t *rope_out, int64_t rope_stride,
                   uint16_t *indexer_out, int64_t indexer_stride);
void kvo_encode_rows(int64_t T, const uint16_t *latent, int64_t latent_stride, const uint16_t *rope,
                     int64_t rope_stride, const uint16_t *indexer, int64_t indexer_stride, uint8_t *main_rows,
                     uint8_t *idx_codes, uint8_t *idx_scales);
void kvo_e4m3_encode_array(const float *v, size_t n, uint8_t *out);
void kvo_quant_tiles(const uint16_t *x, size_t n_tiles, uint8_t *codes, float *scales);
void kvo_dequant_tile(const uint8_t *codes, float scale, size_t n, uint16_t *out);

#define CHECK(c)                                                   \
    do {                                                           \
        if (!(c)) {                                                \
            printf("failed: %s (line %d)\n", #c, __LINE__);         \
            return 1;                                              \
        }                                                          \
    } while (0)

enum { R = 3, L = 2, P = 3, T = 200, LS = 520, RS = 72, IS = 136 };
#define MAIN_PAGE (64u * 656u)
#define IDX_PAGE (64u * 128u + 64u * 4u)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint16_t next_bf16(void) {           /* xorshift64*, finite bf16 patterns only */
    uint16_t b;
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    b = (uint16_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 48);
    if ((b & 0x7F80u) == 0x7F80u) b &= 0xBFFFu;   /* exponent all ones: clear one bit */
    return b;
}

static uint16_t *rows(size_t width, size_t stride) {   /* T rows, the last one ending the buffer */
    uint16_t *p = malloc(((size_t)(T - 1) * stride + width) * sizeof *p);
    size_t t, k;
    if (!p) return NULL;
    for (t = 0; t < T; ++t)
        for (k = 0; k < width; ++k) {
            uint16_t v = next_bf16();
            if (t == 0) v = (k & 1) ? 0x8000u : 0x0000u;          /* all zero, both signs */
            if (t == 1) v = (uint16_t)(v & 0x807Fu);               /* subnormal or zero */
            if (t == 2) v = (k & 2) ? 0xFF7Fu : 0x7F7Fu;           /* largest finite bf16 */
            p[t * stride + k] = v;
        }
    return p;
}

int main(void) {
    const size_t main_bytes = (size_t)L * P * MAIN_PAGE, idx_bytes = (size_t)L * P * IDX_PAGE;
    uint8_t *mains[R], *idxs[R];
    uint16_t *lat = rows(512, LS), *rope = rows(64, RS), *ind = rows(128, IS);
    int64_t *slots = malloc(T * sizeof *slots);
    uint16_t *glat = malloc(((size_t)(T - 1) * LS + 512) * 2), *grope = malloc(((size_t)(T - 1) * RS + 64) * 2),
             *gind = malloc(((size_t)(T - 1) * IS + 128) * 2);
    uint8_t *enc_rows = malloc((size_t)T * 656), *enc_codes = malloc((size_t)T * 128), *enc_scales = malloc((size_t)T * 4);
    const int64_t extra[8] = {-1, -1, 192, -2, INT64_MIN, INT64_MAX, 1000000, -1};
    const float special[] = {0.0f, -0.0f, FLT_TRUE_MIN, -FLT_TRUE_MIN, FLT_MIN, 0.0009765625f, 0.001953125f,
                             0.0029296875f, 1.0f, 1.0625f, 1.1875f, 447.0f, 448.0f, 463.99f, 464.0f, 1e30f,
                             FLT_MAX, -FLT_MAX, -448.0f, -1e-30f};
    const size_t n_special = sizeof special / sizeof special[0];
    uint8_t special_codes[sizeof special / sizeof special[0]];
    uint8_t tile_codes[128];
    float tile_scale;
    uint16_t back[128];
    int64_t t;
    int r;

    CHECK(lat && rope && ind && slots && glat && grope && gind && enc_rows && enc_codes && enc_scales);
    for (r = 0; r < R; ++r) {
        mains[r] = malloc(main_bytes);
        idxs[r] = malloc(idx_bytes);
        CHECK(mains[r] && idxs[r]);
        memset(mains[r], 0x5A, main_bytes);
        memset(idxs[r], 0x5A, idx_bytes);
    }
    /* every slot of the 3 pages once (a fixed permutation), then pads and invalid slots */
    for (t = 0; t < 192; ++t) slots[t] = (t * 77 + 5) % 192;
    for (t = 192; t < T; ++t) slots[t] = extra[t - 192];

    CHECK(kvo_store(R, mains, idxs, P, MAIN_PAGE, P * MAIN_PAGE, IDX_PAGE, P * IDX_PAGE, 1, T, lat, LS, rope, RS,
                    ind, IS, slots) == 5);
    CHECK(kvo_store(R, mains, idxs, P, MAIN_PAGE, P * MAIN_PAGE, IDX_PAGE, P * IDX_PAGE, 0, 0, lat, LS, rope, RS,
                    ind, IS, slots) == 0);
    for (r = 1; r < R; ++r) {
        CHECK(memcmp(mains[0], mains[r], main_bytes) == 0);
        CHECK(memcmp(idxs[0], idxs[r], idx_bytes) == 0);
    }
    for (t = 0; t < (int64_t)(P * MAIN_PAGE); ++t) CHECK(mains[0][t] == 0x5A);   /* layer 0 untouched */
    for (t = 0; t < (int64_t)(P * IDX_PAGE); ++t) CHECK(idxs[0][t] == 0x5A);

    CHECK(kvo_gather(mains[2], idxs[2], P, MAIN_PAGE, P * MAIN_PAGE, IDX_PAGE, P * IDX_PAGE, 1, T, slots, glat, LS,
                     grope, RS, gind, IS) == 5);
    for (t = 192; t < T; ++t) CHECK(glat[t * LS] == 0 && glat[t * LS + 511] == 0 && gind[t * IS + 127] == 0);
    for (t = 3; t < 192; ++t) CHECK(memcmp(&grope[t * RS], &rope[t * RS], 64 * 2) == 0);
    for (t = 0; t < 512; ++t) CHECK(glat[t] == 0);                               /* the all-zero row */

    kvo_encode_rows(T, lat, LS, rope, RS, ind, IS, enc_rows, enc_codes, enc_scales);
    kvo_e4m3_encode_array(special, n_special, special_codes);
    CHECK(special_codes[0] == 0x00 && special_codes[1] == 0x80 && special_codes[8] == 0x38);
    CHECK(special_codes[12] == 0x7E && special_codes[16] == 0x7E && special_codes[17] == 0xFE);
    kvo_quant_tiles(ind + 5 * IS, 1, tile_codes, &tile_scale);
    kvo_dequant_tile(tile_codes, tile_scale, 128, back);

    for (r = 0; r < R; ++r) {
        free(mains[r]);
        free(idxs[r]);
    }
    free(lat); free(rope); free(ind); free(slots); free(glat); free(grope); free(gind);
    free(enc_rows); free(enc_codes); free(enc_scales);
    printf("ok\n");
    return 0;
}
