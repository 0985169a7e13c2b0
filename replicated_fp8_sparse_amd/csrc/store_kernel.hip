// Fused FP8 cache-store for gfx950: one read of each token's final rows,
// quantized once, fanned out to R replica caches.
//
// vLLM PR #52863 "[Kernel][PCP] Publish replicated KV updates through PyTorch
// symmetric memory": the Design section has fused cache-store kernels write the
// final FP8 Main-KV and Indexer-K bytes to every replica; the "THIS PR"
// diagram replaces the gather + receive-side insert with stores to each cache.
// Here the R replicas are R buffers in this GPU's HBM.
//
// Work mapping (wave64).  A wave owns a group of 4 consecutive tokens.  A
// token has five 128-element tiles (4 latent + 1 indexer); a DPP row of 16
// lanes x 8 bf16 (one 16-byte load per lane) is exactly one tile, so one wave
// instruction covers 4 tiles and the 20 tiles of a group take 5 rounds with
// every lane busy:
//   round k = 0..3: token k's latent, lanes 16j..16j+15 = tile j;
//   round 4:        the indexer rows, lanes 16g..16g+15 = token g.
// Lanes 0..31 also carry the 4 tokens' RoPE rows (8 lanes x 16 B each), which
// are copied through unchanged.  Every input byte is loaded once, up front,
// with token indices clamped to the last token so no load waits on a branch
// or on the slot values.
//
// Per tile: amax from the bf16 magnitude bits (packed u16 max in-lane, then a
// 4-step DPP max within the row), scale = amax / 448 (IEEE binary32
// division), and per element code = e4m3fn(RN32(x / scale)).  RN32(x/scale)
// is computed as q = |x|*y, r = fma(-q, scale, |x|), q' = fma(r, y, q) with
// y = RN32(1/scale), sign restored from x.  For every scale >= 2^-64 this
// gives the same e4m3 code as a correctly rounded division for every bf16 x
// with |x| <= amax (the domain is finite and was checked exhaustively on the
// CPU); tiles with a smaller scale (and all-zero tiles) take the plain IEEE
// division path.  The conversion uses the gfx950 OCP e4m3 convert
// (round-to-nearest-even); |x/scale| < 450 for finite input, below the
// saturation boundary at 464, and quotients are clamped to 448 first.
//
// Every piece is stored straight to its slot in each replica (ordinary
// write-back stores, so neighbouring pieces of a 128-byte line merge in L2);
// the inputs are read with non-temporal loads (read once, never reused).
#include "kvpub_internal.h"

namespace kvpub {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

constexpr float kE4m3Max = 448.0f;
constexpr int kNumXcds = 8;

// Block b runs on XCD b % 8.  Give each XCD a contiguous range of token chunks
// so that neighbouring rows (which share cache lines at row boundaries and in
// the Indexer-K scale run) are written through the same L2.
__device__ __forceinline__ uint32_t xcd_chunk(uint32_t b, uint32_t n) {
    const uint32_t per = n / kNumXcds, rem = n % kNumXcds;
    const uint32_t x = b % kNumXcds, i = b / kNumXcds;
    return x * per + (x < rem ? x : rem) + i;
}

// Max over the 16 lanes of a DPP row.
__device__ __forceinline__ uint32_t row_max16(uint32_t v) {
    uint32_t t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
    v = v > t ? v : t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
    v = v > t ? v : t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    v = v > t ? v : t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);  // row_mirror
    v = v > t ? v : t;
    return v;
}

__device__ __forceinline__ u16x2 as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }

// Largest magnitude bit pattern among the lane's 8 bf16 values (sign cleared).
// Non-negative finite floats order like their bit patterns.
__device__ __forceinline__ uint32_t lane_amax_bits(u32x4 d) {
    const uint32_t m = 0x7FFF7FFFu;
    u16x2 a = __builtin_elementwise_max(as_u16x2(d.x & m), as_u16x2(d.y & m));
    u16x2 b = __builtin_elementwise_max(as_u16x2(d.z & m), as_u16x2(d.w & m));
    a = __builtin_elementwise_max(a, b);
    return (uint32_t)(a.x > a.y ? a.x : a.y);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Exact tile scale and reciprocal from a 128-entry table.
//
// A tile's amax is a bf16 value (128 + m) * 2^(E-134), E its biased exponent
// and m its 7 mantissa bits, so amax / 448 = ((128 + m) / 448) * 2^(E-134)
// exactly.  Rounding to binary32 commutes with scaling by a power of two as
// long as the result stays normal, hence
//   RN(amax / 448)         = RN((128 + m) / 448) * 2^(E-134)
//   RN(1 / RN(amax / 448)) = RN(1 / RN((128 + m) / 448)) * 2^(134-E).
// Each wave fills its own table once (IEEE divisions, two entries per lane,
// while its first loads are in flight) and applies the power of two with
// ldexp.  Used only on the fast path (E >= 72: the scale is >= 2^-64 and
// normal); other tiles divide.
struct ScaleEntry {
    float s;  // RN((128 + m) / 448)
    float y;  // RN(1 / s)
};
__device__ __forceinline__ ScaleEntry scale_entry(uint32_t m) {
    const float s = (float)(128u + m) / kE4m3Max;
    return ScaleEntry{s, 1.0f / s};
}
constexpr uint32_t kFastMinExponent = 72;   // amax >= 2^-55  <=>  scale >= 2^-64

// RN32(x / scale) from the correctly rounded reciprocal y (see the header):
// q = |x|*y, r = |x| - q*scale (exact, fused), q' = q + r*y, sign of x.
__device__ __forceinline__ float quotient_fast(float x, float scale, float y) {
    const float a = __builtin_fabsf(x);
    const float q = a * y;
    const float r = __builtin_fmaf(-q, scale, a);
    return __builtin_copysignf(__builtin_fmaf(r, y, q), x);
}

// IEEE division for tiles off the fast path; an all-zero tile gives +0
// (codes 0x00 whatever the signs of its zeros).
__device__ __forceinline__ float quotient_exact(float x, float scale) {
    return scale == 0.0f ? 0.0f : x / scale;
}

__device__ __forceinline__ u32x2 cvt8(const float (&q)[8]) {
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], w1, true);
    return u32x2{(uint32_t)w0, (uint32_t)w1};
}

__device__ __forceinline__ void unpack8(u32x4 d, float (&x)[8]) {
    x[0] = bf16_lo(d.x); x[1] = bf16_hi(d.x); x[2] = bf16_lo(d.y); x[3] = bf16_hi(d.y);
    x[4] = bf16_lo(d.z); x[5] = bf16_hi(d.z); x[6] = bf16_lo(d.w); x[7] = bf16_hi(d.w);
}

#ifndef KVPUB_WPC
#define KVPUB_WPC 16   // target waves per CU before a block takes several block-groups
#endif

// One group = 4 consecutive tokens: their rows (loaded once) and slots.
struct Group {
    u32x4 lat[4];    // latent of token k: lane l holds elements 8l..8l+7
    u32x4 ix;        // indexer of token g = l/16: elements 8(l%16)..+7
    u32x4 rp;        // RoPE of token (l/8)%4: elements 8(l%8)..+7 (lanes 32..63 repeat 0..31)
    int64_t s[4];    // wave-uniform slots of the 4 tokens, -1 past the last token
    int64_t sg;      // slot of this lane's indexer token
    int64_t sr;      // slot of this lane's RoPE token
};

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// What the loads need; these arrive as separate kernel arguments so that the
// hardware preloads them into SGPRs at wave launch (kernarg preloading), and
// the loads can be issued without first waiting for a kernel-argument fetch.
struct RowArgs {
    const uint16_t* latent;
    const uint16_t* rope;
    const uint16_t* indexer;
    const int64_t* slots;
    int64_t num_tokens;
    int32_t latent_stride, rope_stride, indexer_stride;   // elements
};

// Issue every load of a group.  Token indices past the end are clamped to the
// last token (always in bounds) and their slots forced to -1.
__device__ __forceinline__ void load_group(const RowArgs& a, int64_t t0, uint32_t lane, Group& G) {
    const int64_t last = a.num_tokens - 1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t t = t0 + k < last ? t0 + k : last;
        G.lat[k] = ld16(a.latent + t * a.latent_stride + lane * 8);
    }
    const int64_t ug = t0 + (lane >> 4), ur = t0 + ((lane >> 3) & 3u);
    const int64_t tg = ug < last ? ug : last, tr = ur < last ? ur : last;
    G.ix = ld16(a.indexer + tg * a.indexer_stride + (lane & 15u) * 8);
    G.rp = ld16(a.rope + tr * a.rope_stride + (lane & 7u) * 8);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t t = t0 + k < last ? t0 + k : last;
        const int64_t v = a.slots[t];
        G.s[k] = t0 + k <= last ? v : -1;
    }
    const int64_t vg = a.slots[tg], vr = a.slots[tr];
    G.sg = ug <= last ? vg : -1;
    G.sr = ur <= last ? vr : -1;
}

__device__ __forceinline__ bool slot_ok(int64_t s, int64_t capacity) {
    return (uint64_t)s < (uint64_t)capacity;   // negative slots wrap to huge values
}

// Quantize a group and hand every output piece to `out`:
//   out.codes(k, c)     Main-KV row bytes [8*lane, +8) of token k
//   out.scale(k, v)     row bytes [512 + 4*(lane/16), +4) of token k: the scale of
//                       tile lane/16 (lanes 0, 16, 32, 48)
//   out.rope(v)         row bytes [528 + 16*(lane%8), +16) of token lane/8 (lanes 0..31)
//   out.icodes(c)       Indexer-K codes [8*(lane%16), +8) of token lane/16
//   out.iscale(v)       Indexer-K scale of token lane/16 (lanes 16g only)
// tok[k] (wave-uniform), ok_r and ok_g (per lane) select what is stored; tab is
// the wave's copy of the scale table.  The five rounds are independent and are
// computed as one straight-line block (their reductions, table reads and
// divisions interleave); only the stores are conditional.
template <class Out>
__device__ __forceinline__ void quantize_group(const Group& G, uint32_t lane, const ScaleEntry* tab,
                                               const bool (&tok)[4], bool ok_r, bool ok_g, Out& out) {
    const u32x4 rows[5] = {G.lat[0], G.lat[1], G.lat[2], G.lat[3], G.ix};
    uint32_t ab[5];  // bf16 magnitude bits of each tile's amax (row-uniform)
#pragma unroll
    for (int i = 0; i < 5; ++i) ab[i] = row_max16(lane_amax_bits(rows[i]));
    ScaleEntry se[5];
    bool fast = true;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        se[i] = tab[ab[i] & 127u];
        const uint32_t E = ab[i] >> 7;
        fast = fast && E >= kFastMinExponent && E < 255u;
    }
    u32x2 codes[5];
    float scale[5];
    if (__all(fast)) {
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int E = (int)(ab[i] >> 7);
            const float s = __builtin_ldexpf(se[i].s, E - 134);
            const float y = __builtin_ldexpf(se[i].y, 134 - E);
            float x[8], q[8];
            unpack8(rows[i], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) q[e] = quotient_fast(x[e], s, y);
            codes[i] = cvt8(q);
            scale[i] = s;
        }
    } else {
        // some tile of the wave has a tiny (possibly subnormal) scale or is all
        // zeros: those tiles divide, the others take the fast path
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const uint32_t E = ab[i] >> 7;
            const bool f = E >= kFastMinExponent && E < 255u;
            const float s_fast = __builtin_ldexpf(se[i].s, (int)E - 134);
            const float y = __builtin_ldexpf(se[i].y, 134 - (int)E);
            const float s_exact = __uint_as_float(ab[i] << 16) / kE4m3Max;
            float x[8], q[8];
            unpack8(rows[i], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) q[e] = f ? quotient_fast(x[e], s_fast, y) : quotient_exact(x[e], s_exact);
            codes[i] = cvt8(q);
            scale[i] = f ? s_fast : s_exact;
        }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (!tok[k]) continue;
        out.codes(k, codes[k]);
        if ((lane & 15u) == 0) out.scale(k, __float_as_uint(scale[k]));
    }
    if (lane < 32 && ok_r) out.rope(G.rp);
    if (ok_g) {
        out.icodes(codes[4]);
        if ((lane & 15u) == 0) out.iscale(__float_as_uint(scale[4]));
    }
}

// Stores each piece at its slot in every replica.
template <int R>
struct ScatterOut {
    const StoreParams& p;
    const Group& G;
    uint32_t lane;
    __device__ uint64_t row_off(int64_t s) const {
        return (uint64_t)(s >> 6) * p.main_page_stride + (uint64_t)(s & 63) * 656u;
    }
    __device__ void codes(int k, u32x2 c) {
        const uint64_t o = row_off(G.s[k]);  // wave-uniform
#pragma unroll
        for (int r = 0; r < R; ++r) *reinterpret_cast<u32x2*>((p.main_base[r] + o) + (uint32_t)(lane * 8u)) = c;
    }
    __device__ void scale(int k, uint32_t v) {
        const uint64_t o = row_off(G.s[k]) + 512u;  // wave-uniform
#pragma unroll
        for (int r = 0; r < R; ++r)
            *reinterpret_cast<uint32_t*>((p.main_base[r] + o) + (uint32_t)((lane >> 4) * 4u)) = v;
    }
    __device__ void rope(u32x4 v) {
        const uint64_t o = row_off(G.sr) + 528u + (lane & 7u) * 16u;
#pragma unroll
        for (int r = 0; r < R; ++r) *reinterpret_cast<u32x4*>(p.main_base[r] + o) = v;
    }
    __device__ void icodes(u32x2 c) {
        const uint64_t o = (uint64_t)(G.sg >> 6) * p.idx_page_stride + (uint64_t)(G.sg & 63) * 128u +
                           (lane & 15u) * 8u;
#pragma unroll
        for (int r = 0; r < R; ++r) *reinterpret_cast<u32x2*>(p.idx_base[r] + o) = c;
    }
    __device__ void iscale(uint32_t v) {
        const uint64_t o = (uint64_t)(G.sg >> 6) * p.idx_page_stride + 8192u + (uint64_t)(G.sg & 63) * 4u;
#pragma unroll
        for (int r = 0; r < R; ++r) *reinterpret_cast<uint32_t*>(p.idx_base[r] + o) = v;
    }
};

// Each wave owns a contiguous run of p.groups_per_wave groups (4 tokens each);
// blocks are mapped XCD-aware so that neighbouring groups share an L2.
template <int R>
__global__ __launch_bounds__(kWavesPerBlock * 64) void store_kernel(
    const uint16_t* latent, const uint16_t* rope, const uint16_t* indexer, const int64_t* slots,
    int32_t num_tokens, uint32_t num_blocks, int32_t latent_stride, int32_t rope_stride,
    int32_t indexer_stride, int32_t groups_per_wave, const StoreParams p) {
    const RowArgs a{latent, rope, indexer, slots, num_tokens, latent_stride, rope_stride, indexer_stride};
    __shared__ ScaleEntry tab_lds[kWavesPerBlock][128];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t chunk = xcd_chunk(blockIdx.x, num_blocks);   // num_blocks == gridDim.x
    const int64_t ngroups = ((int64_t)num_tokens + kTokensPerWave - 1) / kTokensPerWave;
    const int64_t g0 = ((int64_t)chunk * kWavesPerBlock + wave) * groups_per_wave;
    const int64_t g1 = g0 + groups_per_wave < ngroups ? g0 + groups_per_wave : ngroups;
    ScaleEntry* tab = tab_lds[wave];  // the wave's own copy: no barrier needed
    for (int64_t g = g0; g < g1; ++g) {
        Group G;
        load_group(a, g * kTokensPerWave, lane, G);
        // Issued after the row loads, consumed only through the store masks below.
        const bool poisoned = (*p.status & kStatusPoisoned) != 0;  // a fence timed out: fail closed
        if (g == g0) {  // fill the wave's scale table while the loads are in flight
            uint32_t m = lane;
            asm volatile("" : "+v"(m));  // keeps the divisions below the row loads
            tab[m] = scale_entry(m);
            tab[64 + m] = scale_entry(64 + m);
        }
        // Invalid (neither -1 nor a slot of the cache) slots are skipped and counted.
        uint32_t nbad = 0;
        bool tok[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            tok[k] = !poisoned && slot_ok(G.s[k], p.capacity);
            nbad += (G.s[k] != -1 && !slot_ok(G.s[k], p.capacity)) ? 1u : 0u;
        }
        if (nbad != 0 && !poisoned && lane == 0) atomicAdd(p.invalid_count, (unsigned long long)nbad);
        ScatterOut<R> out{p, G, lane};
        quantize_group(G, lane, tab, tok, !poisoned && slot_ok(G.sr, p.capacity),
                       !poisoned && slot_ok(G.sg, p.capacity), out);
    }
}

}  // namespace

hipError_t launch_store(const StoreParams& p_in, uint32_t num_replicas, hipStream_t stream) {
    StoreParams p = p_in;
    const int64_t ngroups = (p.num_tokens + kTokensPerWave - 1) / kTokensPerWave;
    const int64_t max_waves = (int64_t)p.num_cus * KVPUB_WPC;
    p.groups_per_wave = ngroups <= max_waves ? 1 : (ngroups + max_waves - 1) / max_waves;
    const int64_t waves = (ngroups + p.groups_per_wave - 1) / p.groups_per_wave;
    const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    const dim3 grid((uint32_t)blocks), block(kWavesPerBlock * 64);
#define KVPUB_ROW_ARGS p.latent, p.rope, p.indexer, p.slots, (int32_t)p.num_tokens, (uint32_t)blocks, \
    (int32_t)p.latent_stride, (int32_t)p.rope_stride, (int32_t)p.indexer_stride, (int32_t)p.groups_per_wave
    (void)hipGetLastError();
    switch (num_replicas) {
        case 1: store_kernel<1><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS, p); break;
        case 2: store_kernel<2><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS, p); break;
        case 3: store_kernel<3><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS, p); break;
        case 4: store_kernel<4><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS, p); break;
        case 5: store_kernel<5><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS, p); break;
        case 6: store_kernel<6><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS, p); break;
        case 7: store_kernel<7><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS, p); break;
        case 8: store_kernel<8><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvpub
