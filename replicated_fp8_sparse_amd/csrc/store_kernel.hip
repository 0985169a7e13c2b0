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
// or on the slot values; the slots arrive through scalar loads and every
// store address is worked out while the rows are in flight.
//
// Per tile: amax = the largest magnitude (packed 16-bit maxima in-lane, then
// a 4-step DPP max within the row), scale = RN32(amax / 448), and per element
// code = e4m3fn(RN32(x / scale)).  The scale and its reciprocal y =
// RN32(1/scale) come from a short exact sequence (tile_scale), run once for a
// group's 20 tiles: each lane of a DPP row takes one of the row's five tiles,
// and row_newbcast hands each round's values back to the row.  In place of
// the division the quotient is
// q = x*y, t = fma(q, scale, -x), q' = fma(-t, y, q), which is the magnitude
// form fma(fma(-|x|y, scale, |x|), y, |x|y) with the sign of x put back.
// q' is not always RN32(x/scale) (it can differ in the last bit), but for
// every scale >= 2^-64 and every bf16 x with |x| <= amax it has the same e4m3
// code as the correctly rounded division: the domain is finite (9.8e8 signed
// pairs) and a CPU test walks all of it; tiles with a smaller scale (and
// all-zero tiles) take the plain IEEE division path.  The conversion uses the
// gfx950 OCP e4m3 convert (round-to-nearest-even, saturating only above 464):
// |x/scale| <= 448 (1 + 2^-23) for finite input, so no clamp is needed.
//
// Every piece is stored straight to its slot in each replica; the inputs are
// read with non-temporal loads (read once, never reused).  How the stores
// treat the L2 depends on the launch size (see put_at).  Batches of up to
// about a thousand tokens take small_store_kernel instead, which spreads a
// group's five rounds over five waves with the same per-tile arithmetic.
#include <type_traits>

#include "kvpub_internal.h"

namespace kvpub {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) uint8_t gbyte;   // a byte in global memory
typedef __attribute__((address_space(3))) uint8_t lbyte;   // a byte in LDS
template <class T> using gptr = __attribute__((address_space(1))) T*;
template <class T> using lptr = __attribute__((address_space(3))) T*;

constexpr uint32_t kRunBytes = 4 * 656;   // 2624 = 164 x 16 B
constexpr int64_t kCacheBytesPerToken = 656 + 128 + 4;              // per replica
constexpr int64_t kStreamingStoreBytes = int64_t(16) << 20;         // launches writing at most this stream
constexpr int64_t kWriteThroughBytes = int64_t(32) << 20;           // more than the 8 L2s hold: write through
constexpr int64_t kMaxStride32 = int64_t(1) << 28;                  // input row stride (elements): 32-bit loads
constexpr int kBlockRunWaves = 8;   // waves per block of those launches (block runs of 32 rows, 20,992 bytes)
// Batches up to this many tokens take small_store_kernel (up to twice as many
// with one or two replicas): measured crossover against the main kernel.
constexpr int64_t kSmallBatchTokens = 1024;

// Store policy by launch size:
//   NT (a launch writing at most kStreamingStoreBytes): the whole-line kind of
//     pieces (row runs, which cover whole 128-byte lines apart from the lines at
//     their two ends, and Indexer-K codes) are stored non-temporally, the
//     partial pieces (scales, the per-row path) with ordinary write-back
//     stores.  The whole lines are then not left dirty in L2 for the
//     end-of-kernel write-back, which a latency-bound launch would otherwise
//     wait for, while the partial lines still merge in L2.
//   WT (a launch writing more than kWriteThroughBytes, more than the eight
//     4 MB L2s can hold): the whole-line pieces are buffer stores with the
//     device-coherence bit, written through this XCD's L2 instead of held
//     dirty in it, so the writes stream out while the kernel runs instead of
//     being evicted later; the partial pieces (the per-row path, and the
//     16-byte Indexer-K scale runs, eight waves to a 128-byte line) stay
//     write-back, so they merge in L2 instead of reaching memory as partial
//     writes.  Buffer offsets are
//     32-bit, so WT needs each replica's layer to span less than 2^32 bytes;
//     the buffer's range check (num_records = the layer's span) drops any
//     whole-line store outside the layer.
//   otherwise (launches in between, or layers too large for WT): ordinary
//     write-back stores, which the L2s absorb.
template <bool NT, class T>
__device__ __forceinline__ void put(gptr<T> p, T v) {
    if (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer resource, 32-bit data format (gfx950)
constexpr int kDeviceCoherent = 16;      // buffer cache-policy bits: sc1

// Store v at base + off: `whole` marks a piece of the whole-line kind (see above).
// With a 32-bit offset the address is a uniform base plus a 32-bit lane offset,
// which the store instruction takes as is (no 64-bit address arithmetic).
template <bool NT, bool WT, bool whole, class T, class O>
__device__ __forceinline__ void put_at(gbyte* base, uint32_t region, O off, T v) {
    if constexpr (WT && whole) {
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)region, kRsrcWord3);
        const int o = (int)(uint32_t)off;
        if constexpr (sizeof(T) == 16) __builtin_amdgcn_raw_buffer_store_b128(v, r, o, 0, kDeviceCoherent);
        else if constexpr (sizeof(T) == 8) __builtin_amdgcn_raw_buffer_store_b64(v, r, o, 0, kDeviceCoherent);
        else __builtin_amdgcn_raw_buffer_store_b32(v, r, o, 0, kDeviceCoherent);
    } else {
        put<NT && whole>((gptr<T>)(base + off), v);
    }
}

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

// bf16 magnitude bits of the largest magnitude among the lane's 8 values,
// from the packed data (sign cleared: non-negative finite values order like
// their bit patterns; two 16-bit maxima per instruction).  Working on the
// packed rows keeps the unpacked values out of the registers until each
// round's quotients need them.
__device__ __forceinline__ u16x2 as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }
__device__ __forceinline__ uint32_t lane_amax_bits(u32x4 d) {
    const uint32_t m = 0x7FFF7FFFu;
    u16x2 a = __builtin_elementwise_max(as_u16x2(d.x & m), as_u16x2(d.y & m));
    u16x2 b = __builtin_elementwise_max(as_u16x2(d.z & m), as_u16x2(d.w & m));
    a = __builtin_elementwise_max(a, b);
    return (uint32_t)(a.x > a.y ? a.x : a.y);
}

// Lane 0 of every DPP row (lanes 0, 16, 32, 48).
constexpr uint64_t kLaneInRowMask = 0x0001000100010001ull;

// a in the lanes of `mask`, b elsewhere (the mask is a constant, so it sits in
// an SGPR pair and the select is one instruction).
__device__ __forceinline__ uint32_t select_lane_in_row(uint64_t mask, uint32_t a, uint32_t b) {
    uint32_t r;
    asm("v_cndmask_b32 %0, %1, %2, %3" : "=v"(r) : "v"(b), "v"(a), "s"(mask));
    return r;
}

// Lane I of each DPP row, broadcast to the whole row (row_newbcast:I).
template <int I>
__device__ __forceinline__ float bcast_lane(float v) {
    // every lane reads a valid source lane: a plain DPP move (no old value to keep)
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + I, 0xF, 0xF, false));
}
__device__ __forceinline__ float bcast_in_row(float v, int i) {   // i: a constant after unrolling
    switch (i) {
        case 0: return bcast_lane<0>(v);
        case 1: return bcast_lane<1>(v);
        case 2: return bcast_lane<2>(v);
        case 3: return bcast_lane<3>(v);
        default: return bcast_lane<4>(v);
    }
}

// Largest magnitude of 8 finite values (exact: a maximum rounds nothing).
// max3 with absolute-value source modifiers; written out so that no NaN
// quieting is added around it (the inputs are finite bf16 values).
__device__ __forceinline__ float max3_abs(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float lane_amax_f32(const float (&x)[8]) {
    float m = max3_abs(x[0], x[1], x[2]);
    m = max3_abs(m, x[3], x[4]);
    m = max3_abs(m, x[5], x[6]);
    return max3_abs(m, x[7], x[7]);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Exact tile scale and reciprocal without a division.
//
// A tile's amax is a bf16 value (128 + m) * 2^(E-134), E its biased exponent
// and m its 7 mantissa bits, so amax / 448 = ((128 + m) / 448) * 2^(E-134)
// exactly.  Rounding to binary32 commutes with scaling by a power of two as
// long as the result stays normal, hence
//   RN(amax / 448)         = RN((128 + m) / 448) * 2^(E-134)
//   RN(1 / RN(amax / 448)) = RN(1 / RN((128 + m) / 448)) * 2^(134-E).
// For n = 128 + m, S = RN(n / 448) comes from q0 = n * RN(1/448) and one
// remainder correction; Y = RN(1 / S) from the hardware reciprocal and one
// Newton step with fused multiply-adds.  Both sequences reproduce the
// correctly rounded values for all 128 mantissas (Y even when the reciprocal
// estimate is off by up to 3 ulp); the check is part of the CPU tests.  Used
// only on the fast path (E >= 72: the scale is >= 2^-64 and normal).
struct TileScale {
    float s;  // RN(amax / 448)
    float y;  // RN(1 / s)
};
__device__ __forceinline__ TileScale tile_scale(uint32_t ab) {
    const float n = (float)((ab & 127u) | 128u);
    const float c = 1.0f / kE4m3Max;   // RN(1/448), folded at compile time
    const float q0 = n * c;
    const float S = __builtin_fmaf(__builtin_fmaf(-q0, kE4m3Max, n), c, q0);
    const float y0 = __builtin_amdgcn_rcpf(S);
    const float Y = __builtin_fmaf(__builtin_fmaf(-S, y0, 1.0f), y0, y0);
    const int E = (int)(ab >> 7);
    return TileScale{__builtin_ldexpf(S, E - 134), __builtin_ldexpf(Y, 134 - E)};
}
constexpr uint32_t kFastMinExponent = 72;   // amax >= 2^-55  <=>  scale >= 2^-64

// A quotient with the e4m3 code of RN32(x / scale), from the correctly rounded
// reciprocal y (see the header): q = x*y, t = q*scale - x (exact, fused),
// q' = q - t*y.  Round-to-nearest is symmetric, so this is the magnitude
// computation with the sign of x put back, signed zeros included (x = -0
// gives t = +0 and q' = -0).
__device__ __forceinline__ float quotient_fast(float x, float scale, float y) {
    const float q = x * y;
    const float t = __builtin_fmaf(q, scale, -x);
    return __builtin_fmaf(-t, y, q);
}

// IEEE division for tiles off the fast path; an all-zero tile gives +0
// (codes 0x00 whatever the signs of its zeros).
__device__ __forceinline__ float quotient_exact(float x, float scale) {
    return scale == 0.0f ? 0.0f : x / scale;
}

__device__ __forceinline__ u32x2 cvt8(const float (&q)[8]) {
    // The convert writes one 16-bit half and keeps the other from its old
    // operand; the second convert of each word overwrites the half the first
    // one kept, so the first one's old operand is any value: its first input,
    // which dies there, so the result can take its register.
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], __float_as_int(q[0]), false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], __float_as_int(q[4]), false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], w1, true);
    return u32x2{(uint32_t)w0, (uint32_t)w1};
}

__device__ __forceinline__ void unpack8(u32x4 d, float (&x)[8]) {
    x[0] = bf16_lo(d.x); x[1] = bf16_hi(d.x); x[2] = bf16_lo(d.y); x[3] = bf16_hi(d.y);
    x[4] = bf16_lo(d.z); x[5] = bf16_hi(d.z); x[6] = bf16_lo(d.w); x[7] = bf16_hi(d.w);
}

// The rows of one group = 4 consecutive tokens, loaded once.
struct Group {
    u32x4 lat[4];    // latent of token k: lane l holds elements 8l..8l+7
    u32x4 ix;        // indexer of token g = l/16: elements 8(l%16)..+7
    u32x4 rp;        // RoPE of token (l/8)%4: elements 8(l%8)..+7 (lanes 32..63 repeat 0..31)
};

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Replica layer bases, held in SGPRs for the whole wave.
template <int R>
struct Bases {
    gbyte* main[R];
    gbyte* idx[R];
};

// Offsets within a replica's layer: 32-bit when every layer spans less than
// 4 GiB (O32), else 64-bit.
template <bool O32> using Off = typename std::conditional<O32, uint32_t, uint64_t>::type;

// Where a group's pieces go, worked out from the slots while its rows are in
// flight.  Offsets are bytes from a replica's layer base.
template <bool O32>
struct Dest {
    Off<O32> row[4];   // Main-KV row of token k (wave-uniform)
    uint32_t tok;      // bit k: token k is stored (wave-uniform)
    Off<O32> rope;     // this lane's RoPE piece (lanes 0..31)
    Off<O32> icode;    // this lane's Indexer-K code piece
    Off<O32> iscale;   // this lane's Indexer-K scale (all 16 lanes of a row)
    uint32_t ok_r, ok_g;   // this lane's RoPE / Indexer-K token is stored
    uint32_t run;      // the 4 rows are consecutive slots of one page (wave-uniform)
};

// s is a slot of the cache: 0 <= s < capacity.  With 32-bit offsets the
// capacity is below 2^32 (a layer spans less than 4 GiB and a page holds 64
// slots in at least 41984 bytes), so the test splits into two 32-bit ones on
// the slot's halves: scalar instructions (there is no 64-bit scalar less-than).
template <bool O32>
__device__ __forceinline__ bool slot_ok(int64_t s, int64_t capacity) {
    if constexpr (O32) {
        // the halves pass through registers so that the two tests are not
        // folded back into one 64-bit comparison (a vector instruction)
        uint32_t hi = (uint32_t)((uint64_t)s >> 32), lo = (uint32_t)s;
        asm volatile("" : "+s"(hi), "+s"(lo));
        return (hi == 0u) & (lo < (uint32_t)capacity);
    } else {
        return (uint64_t)s < (uint64_t)capacity;   // negative slots wrap to huge values
    }
}

// v_i for a per-lane index i in 0..3; v0..v3 wave-uniform.
template <class O>
__device__ __forceinline__ O pick4(O v0, O v1, O v2, O v3, uint32_t i) {
    const O a = (i & 1u) ? v1 : v0;
    const O b = (i & 1u) ? v3 : v2;
    return (i & 2u) ? b : a;
}

// The value is materialized in a register at this point, so later code
// cannot pull its computation below (past the wait for the row data).
template <class O> __device__ __forceinline__ O pin_s(O v) { asm volatile("" : "+s"(v)); return v; }
template <class O> __device__ __forceinline__ O pin_v(O v) { asm volatile("" : "+v"(v)); return v; }
__device__ __forceinline__ uint32_t pin_v32(uint32_t v) { asm volatile("" : "+v"(v)); return v; }
__device__ __forceinline__ gbyte* pin_ptr(uint8_t* v) {
    gbyte* g = (gbyte*)v;
    asm volatile("" : "+s"(g));
    return g;
}

template <int R>
__device__ __forceinline__ Bases<R> pin_bases(const StoreParams& p) {
    Bases<R> b;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        b.main[i] = pin_ptr(p.main_base[i]);
        b.idx[i] = pin_ptr(p.idx_base[i]);
    }
    return b;
}

// tok: bit k set if token k is stored (its slot is a slot of the cache and the
// context is not poisoned; wave-uniform).
template <bool O32>
__device__ __forceinline__ Dest<O32> destinations(int64_t s0, int64_t s1, int64_t s2, int64_t s3, uint32_t tok,
                                                  uint32_t lane, const StoreParams& p) {
    using O = Off<O32>;
    const int64_t sl[4] = {s0, s1, s2, s3};
    O row[4], irow[4], iscl[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if constexpr (O32) {
            // every offset of a slot that is stored fits in 32 bits; the
            // offsets of skipped slots are never used
            const uint32_t lo = (uint32_t)sl[k], page = lo >> 6, in = lo & 63u;
            row[k] = pin_s(page * (uint32_t)p.main_page_stride + in * 656u);
            const uint32_t ib = page * (uint32_t)p.idx_page_stride;
            irow[k] = ib + in * 128u;
            iscl[k] = ib + 8192u + in * 4u;
        } else {
            const uint64_t page = (uint64_t)sl[k] >> 6, in = (uint64_t)sl[k] & 63u;
            row[k] = pin_s(page * p.main_page_stride + in * 656u);
            irow[k] = page * p.idx_page_stride + in * 128u;
            iscl[k] = page * p.idx_page_stride + 8192u + in * 4u;
        }
    }
    const uint32_t g = lane >> 4, r = (lane >> 3) & 3u;
    Dest<O32> d;
#pragma unroll
    for (int k = 0; k < 4; ++k) d.row[k] = row[k];
    tok = __builtin_amdgcn_readfirstlane(tok);   // uniform; computed once, before the wait
    asm volatile("" : "+s"(tok));
    // the 4 rows are one contiguous run: all stored, consecutive slots of one page
    // (all four stored: with 32-bit offsets their high halves are zero)
    bool consecutive;
    if constexpr (O32) {
        const uint32_t l0 = (uint32_t)s0;
        consecutive = (uint32_t)s1 == l0 + 1u && (uint32_t)s2 == l0 + 2u && (uint32_t)s3 == l0 + 3u &&
                      (l0 & 63u) <= 60u;
    } else {
        consecutive = s1 == s0 + 1 && s2 == s0 + 2 && s3 == s0 + 3 && (s0 & 63) <= 60;
    }
    uint32_t run = (tok == 0xFu && consecutive) ? 1u : 0u;
    run = __builtin_amdgcn_readfirstlane(run);
    asm volatile("" : "+s"(run));
    d.tok = tok;
    d.run = run;
    d.rope = pin_v(pick4(row[0], row[1], row[2], row[3], r) + 528u + (lane & 7u) * 16u);
    d.icode = pin_v(pick4(irow[0], irow[1], irow[2], irow[3], g) + (lane & 15u) * 8u);
    d.iscale = pin_v(pick4(iscl[0], iscl[1], iscl[2], iscl[3], g));
    d.ok_r = pin_v32(lane < 32u ? (tok >> r) & 1u : 0u);
    d.ok_g = pin_v32((tok >> g) & 1u);
    return d;
}

// Rounds B..B+N-1 of a group: codes and scales of their tiles.  Each lane of
// DPP row j ends with the amax of the row's N tiles, so lane 16j + i takes tile
// (round B + i, row j) and one scale sequence covers the N rounds' tiles (lanes
// 16j + N.. repeat round B's tile).  UNPACKED: the in-lane maximum from the
// unpacked values, which may then stay live until the quotients (launches of
// few waves per SIMD: four max3 of magnitudes instead of the packed steps);
// else from the packed bf16 bits.
template <int B, int N, bool UNPACKED>
__device__ __forceinline__ void quantize_rounds(const u32x4 (&rows)[5], u32x2 (&codes)[5], float (&scale)[5]) {
    uint32_t ab[N];  // bf16 magnitude bits of each tile's amax (row-uniform)
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if constexpr (UNPACKED) {
            float x[8];
            unpack8(rows[B + i], x);
            // the shift (an ordinary instruction) also stands between the asm
            // result and the DPP reads, whose wait states are the compiler's
            ab[i] = row_max16(__float_as_uint(lane_amax_f32(x)) >> 16);
        } else {
            ab[i] = row_max16(lane_amax_bits(rows[B + i]));
        }
    }
    uint32_t mine = ab[0];
#pragma unroll
    for (int i = 1; i < N; ++i) mine = select_lane_in_row(kLaneInRowMask << i, ab[i], mine);
    const uint32_t E = mine >> 7;
    if (__all(E >= kFastMinExponent && E < 255u)) {
        const TileScale t = tile_scale(mine);
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const float si = bcast_in_row(t.s, i), yi = bcast_in_row(t.y, i);
            float x[8], q[8];
            unpack8(rows[B + i], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) q[e] = quotient_fast(x[e], si, yi);
            codes[B + i] = cvt8(q);
            scale[B + i] = si;
        }
    } else {
        // some tile of these rounds has a tiny (possibly subnormal) scale or is
        // all zeros: those tiles divide, the others take the fast path
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const uint32_t Ei = ab[i] >> 7;
            const bool f = Ei >= kFastMinExponent && Ei < 255u;
            const TileScale t = tile_scale(ab[i]);
            const float s_exact = __uint_as_float(ab[i] << 16) / kE4m3Max;
            float x[8], q[8];
            unpack8(rows[B + i], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) q[e] = f ? quotient_fast(x[e], t.s, t.y) : quotient_exact(x[e], s_exact);
            codes[B + i] = cvt8(q);
            scale[B + i] = f ? t.s : s_exact;
        }
    }
}

// Quantize a group and store every piece to each of the R replicas:
//   codes of token k  -> row bytes [8*lane, +8)
//   scale of tile j   -> row bytes [512 + 4j, +4)       (lane 16j)
//   RoPE              -> row bytes [528 + 16*(lane%8), +16) of token lane/8 (lanes 0..31)
//   Indexer-K codes   -> page bytes [128*(slot%64) + 8*(lane%16), +8) of token lane/16
//   Indexer-K scale   -> page bytes [8192 + 4*(slot%64), +4) (lane 16g)
// Streamed launches (one wave per SIMD at the graph-layer size) quantize in
// two phases: rounds 0-2 once their rows are in, while the last two rows are
// still on their way (a wave's six rows come back over about 0.3 us), then
// rounds 3-4; each phase's reductions and scale sequence interleave.  The
// other launches, several waves per SIMD, take all five rounds in one block.
// Only the stores are conditional.
// WPB (waves per block) above 4 turns on block runs (see below); img is the
// wave's run image, run_first the block's per-wave run words (block runs only).
template <int R, bool NT, bool WT, bool O32, int WPB>
__device__ __forceinline__ void quantize_store(const Group& G, const Dest<O32>& d, const Bases<R>& b, uint32_t lane,
                                               uint32_t wave, lbyte* img, lptr<uint32_t> run_first,
                                               uint32_t main_region, uint32_t idx_region) {
    const u32x4 rows[5] = {G.lat[0], G.lat[1], G.lat[2], G.lat[3], G.ix};
    u32x2 codes[5];
    float scale[5];
    if constexpr (NT) {
        quantize_rounds<0, 3, true>(rows, codes, scale);
        if (d.run) {   // rows 0-2 of the run image (below) while rows 3 and 4 are on their way
#pragma unroll
            for (int k = 0; k < 3; ++k) *(lptr<u32x2>)(img + k * 656u + lane * 8u) = codes[k];
        }
        __builtin_amdgcn_sched_barrier(0);
        quantize_rounds<3, 2, true>(rows, codes, scale);
    } else {
        quantize_rounds<0, 5, false>(rows, codes, scale);
    }
    // The four rows are one contiguous 2624-byte run (656 = 41 x 16): build it
    // in the wave's LDS image and store it as 16-byte pieces, three wave-wide
    // stores per replica instead of nine partial-line ones.
    if (d.run) {
#pragma unroll
        for (int k = NT ? 3 : 0; k < 4; ++k) *(lptr<u32x2>)(img + k * 656u + lane * 8u) = codes[k];
        if ((lane & 15u) == 0) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                *(lptr<uint32_t>)(img + k * 656u + 512u + (lane >> 4) * 4u) = __float_as_uint(scale[k]);
        }
        if (lane < 32u) *(lptr<u32x4>)(img + ((lane >> 3) & 3u) * 656u + 528u + (lane & 7u) * 16u) = G.rp;
    }
    bool block_run = false;
    if constexpr (WPB > 4) {
        // Block runs (launches of more than the L2s hold): when the block's WPB
        // waves all hold runs and the runs follow each other in the Main-KV
        // array (offsets base + w * 2624: consecutive slots, across a page
        // boundary too when pages are dense), the block stores its WPB * 2624
        // bytes as one run, every lane taking 16-byte pieces: longer bursts per
        // replica than four 2624-byte runs written by different waves.  Every
        // wave of the block reaches both barriers (no wave of a block returns
        // early), and every wave reads the same WPB words, so the decision is
        // the same in all of them.  Row offsets are multiples of 16, so the
        // all-ones word (not a run) never matches an expected offset.
        static_assert(O32, "block runs compare 32-bit offsets");
        if (lane == 0) run_first[wave] = d.run ? (uint32_t)d.row[0] : ~0u;
        __syncthreads();
        const uint32_t r0 = run_first[0];
        block_run = r0 != ~0u;
#pragma unroll
        for (uint32_t w = 1; w < (uint32_t)WPB; ++w) block_run = block_run && run_first[w] == r0 + w * kRunBytes;
        if (block_run) {
            const lbyte* bimg = img - wave * kRunBytes;   // the waves' images are contiguous
            for (uint32_t pc = threadIdx.x; pc < (uint32_t)WPB * (kRunBytes / 16u); pc += (uint32_t)WPB * 64u) {
                const u32x4 v = *(lptr<u32x4>)(bimg + pc * 16u);
#pragma unroll
                for (int r = 0; r < R; ++r) put_at<NT, WT, true>(b.main[r], main_region, r0 + pc * 16u, v);
            }
        }
    }
    if (block_run) {
        // stored above, by the whole block
    } else if (d.run) {
        // Only this wave touches its image, and LDS accesses of one wave
        // complete in order, so no barrier is needed.
        __builtin_amdgcn_wave_barrier();
        const u32x4 c0 = *(lptr<u32x4>)(img + lane * 16u);
        const u32x4 c1 = *(lptr<u32x4>)(img + 1024u + lane * 16u);
        const u32x4 c2 = lane < 36u ? *(lptr<u32x4>)(img + 2048u + lane * 16u) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const Off<O32> o = d.row[0] + lane * 16u;
            put_at<NT, WT, true>(b.main[r], main_region, o, c0);
            put_at<NT, WT, true>(b.main[r], main_region, o + 1024u, c1);
            if (lane < 36u) put_at<NT, WT, true>(b.main[r], main_region, o + 2048u, c2);
        }
    } else {
        // A tile's scale is the same in all 16 lanes of its row; the 16 lanes
        // store it to the same word, which the memory pipeline merges.
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (!((d.tok >> k) & 1u)) continue;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                put_at<NT, WT, false>(b.main[r], main_region, d.row[k] + lane * 8u, codes[k]);
                put_at<NT, WT, false>(b.main[r], main_region, d.row[k] + 512u + (lane >> 4) * 4u,
                                      __float_as_uint(scale[k]));
            }
        }
        if (d.ok_r) {
#pragma unroll
            for (int r = 0; r < R; ++r) put_at<NT, WT, false>(b.main[r], main_region, d.rope, G.rp);
        }
    }
    if (d.ok_g) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            put_at<NT, WT, true>(b.idx[r], idx_region, d.icode, codes[4]);
            put_at<NT, WT, false>(b.idx[r], idx_region, d.iscale, __float_as_uint(scale[4]));
        }
    }
}

// Row loads with 32-bit lane offsets, for the streamed launches (one wave per
// SIMD at the graph-layer size, where a wave's time to its first load is on
// the launch's critical path): each load is a uniform base in SGPRs plus a
// 32-bit offset per lane, the form the load instruction takes as is, so the
// six loads leave after a few 32-bit operations instead of 64-bit address
// arithmetic per lane (graph layer 3.99 -> 3.89 us; the write-back launches,
// with two waves per SIMD, lose 3 % with it and keep fetch_rows).  The four
// latent rows share one base (the group's first token, clamped to the batch)
// and add the row's distance in bytes; the RoPE and Indexer-K pieces take
// their lane's token the same way.  Needs every row stride at most
// kMaxStride32 elements (checked on the host): the largest offset,
// 3 rows x 2 B x stride + 1008, then stays below 2^32.
typedef __attribute__((address_space(1))) const uint8_t cgbyte;   // a byte of a global input

__device__ __forceinline__ u32x4 ld16_at(cgbyte* base, uint32_t off) {
    return __builtin_nontemporal_load((__attribute__((address_space(1))) const u32x4*)(base + off));
}

// Keep a uniform 64-bit input address in SGPRs: without the pin the compiler
// folds the lane offset into a 64-bit per-lane address.
__device__ __forceinline__ cgbyte* uniform_base(const uint16_t* p) {
    cgbyte* q = (cgbyte*)p;
    asm volatile("" : "+s"(q));
    return q;
}

__device__ __forceinline__ void fetch_rows32(const uint16_t* latent, const uint16_t* rope, const uint16_t* indexer,
                                             uint32_t latent_stride, uint32_t rope_stride, uint32_t indexer_stride,
                                             uint32_t t0, uint32_t last, uint32_t lane, Group& G) {
    const uint32_t tb = t0 < last ? t0 : last;
    const uint32_t ur = t0 + ((lane >> 3) & 3u), ug = t0 + (lane >> 4);
    const uint32_t kr = (ur < last ? ur : last) - tb, kg = (ug < last ? ug : last) - tb;
    // in order of first use by the two quantization phases: latent rows 0-2,
    // then row 3, the RoPE piece (first needed when the run image is built)
    // and the Indexer-K row
    cgbyte* lb = uniform_base(latent + (uint64_t)tb * latent_stride);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t t = t0 + k < last ? t0 + k : last;
        G.lat[k] = ld16_at(lb, (t - tb) * (latent_stride * 2u) + lane * 16u);
    }
    G.rp = ld16_at(uniform_base(rope + (uint64_t)tb * rope_stride), kr * (rope_stride * 2u) + (lane & 7u) * 16u);
    G.ix = ld16_at(uniform_base(indexer + (uint64_t)tb * indexer_stride),
                   kg * (indexer_stride * 2u) + (lane & 15u) * 16u);
}

// Slots of the group starting at token t0 (scalar loads).  Token indices
// past the end are clamped to the last token (always in bounds).
__device__ __forceinline__ void fetch_slots(const int64_t* __restrict__ slots, uint32_t t0, uint32_t last,
                                            int64_t (&sl)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) sl[k] = slots[t0 + k < last ? t0 + k : last];
}

// Row loads of the group starting at token t0, in order of first use: the
// RoPE piece (stored unchanged) first, so that no wait for it lands among the
// stores, where it would also wait for every store issued before it.
__device__ __forceinline__ void fetch_rows(const uint16_t* latent, const uint16_t* rope, const uint16_t* indexer,
                                           uint32_t latent_stride, uint32_t rope_stride, uint32_t indexer_stride,
                                           uint32_t t0, uint32_t last, uint32_t lane, Group& G) {
    const uint32_t ug = t0 + (lane >> 4), ur = t0 + ((lane >> 3) & 3u);
    const uint32_t tg = ug < last ? ug : last, tr = ur < last ? ur : last;
    G.rp = ld16(rope + (uint64_t)tr * rope_stride + (lane & 7u) * 8u);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t t = t0 + k < last ? t0 + k : last;
        G.lat[k] = ld16(latent + (uint64_t)t * latent_stride + lane * 8u);
    }
    G.ix = ld16(indexer + (uint64_t)tg * indexer_stride + (lane & 15u) * 8u);
}

// One group per wave; blocks are mapped XCD-aware so that neighbouring
// groups share an L2.  The arguments before p are what the first
// instructions need: they arrive preloaded in SGPRs (kernel-argument
// preloading); p is fetched while the row loads are in flight.  Token
// indices are 32-bit (a launch holds at most kMaxTokensPerLaunch tokens).
template <int R, bool NT, bool WT, bool O32, int WPB>
__global__ __launch_bounds__(WPB * 64) void store_kernel(
    const uint16_t* latent, const uint16_t* rope, const uint16_t* indexer,
    const int64_t* __restrict__ slots, uint32_t num_tokens, uint32_t latent_stride, uint32_t rope_stride,
    uint32_t indexer_stride, const CtxHead* __restrict__ head, const StoreParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t run_img[WPB][kRunBytes];
    __shared__ uint32_t run_first[WPB];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    constexpr uint32_t kBlockTokens = kTokensPerWave * WPB;
    const uint32_t num_blocks = (num_tokens + kBlockTokens - 1) / kBlockTokens;   // == gridDim.x
    const uint32_t tb = xcd_chunk(blockIdx.x, num_blocks) * kBlockTokens;       // the block's first token
    const uint32_t t0 = tb + wave * kTokensPerWave;
    // With block runs every wave takes part in the block's barriers: a wave past
    // the end of the batch carries on with no slot to store (its tokens are
    // clamped to the last one and marked padded); only without them may it leave.
    if ((WPB > 4 ? tb : t0) >= num_tokens) return;
    const uint32_t last = num_tokens - 1;
    // Scalar loads (slots, the status word and capacity) do not share a counter
    // with the row loads, so the destinations are worked out before the rows
    // arrive.  In streamed launches with 32-bit offsets the row loads leave
    // first: they have the longer way to go, and their addresses need no
    // scalar load.
    int64_t sl[4];
    Group G;
    CtxHead h;
    if constexpr (O32 && NT) {
        fetch_rows32(latent, rope, indexer, latent_stride, rope_stride, indexer_stride, t0, last, lane, G);
        __builtin_amdgcn_sched_barrier(0);
        fetch_slots(slots, t0, last, sl);
        h = *head;
    } else {
        fetch_slots(slots, t0, last, sl);
        h = *head;
        fetch_rows(latent, rope, indexer, latent_stride, rope_stride, indexer_stride, t0, last, lane, G);
    }
    __builtin_amdgcn_sched_barrier(0);
    const bool poisoned = (h.status & kStatusPoisoned) != 0;  // a fence timed out: fail closed
    // Slots of tokens past the end become -1; invalid slots (neither -1 nor a
    // slot of the cache) are skipped and counted.
    uint32_t ok = 0, pad = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        sl[k] = t0 + k <= last ? sl[k] : -1;
        ok |= slot_ok<O32>(sl[k], h.capacity) ? (1u << k) : 0u;
        pad |= sl[k] == -1 ? (1u << k) : 0u;
    }
    const uint32_t nbad = (uint32_t)__builtin_popcount(~(ok | pad) & 0xFu);
    if (nbad != 0 && !poisoned && lane == 0) atomicAdd(p.invalid_count, (unsigned long long)nbad);
    const Bases<R> b = pin_bases<R>(p);
    const Dest<O32> d = destinations<O32>(sl[0], sl[1], sl[2], sl[3], poisoned ? 0u : ok, lane, p);
    __builtin_amdgcn_sched_barrier(0);
    quantize_store<R, NT, WT, O32, WPB>(G, d, b, lane, wave, (lbyte*)&run_img[wave][0],
                                        (lptr<uint32_t>)&run_first[0], p.main_region, p.idx_region);
}

// Small batches (a decode step: tens of tokens; up to about a thousand).
// The launch is latency-bound there, and a wave's five rounds of arithmetic
// sit on its critical path, so the rounds of a group are spread over five
// waves instead: one block per group of 4 tokens, wave k < 4 takes token k's
// latent row (its four tiles) and, in lanes 0..7, its RoPE; wave 4 takes the
// four tokens' Indexer-K rows.  Same per-tile arithmetic as the main kernel;
// ordinary write-back stores, one row at a time (no row-run image: at larger
// batches the main kernel's merged run stores win).
constexpr int kSmallWaves = 5;

// L32: the rows are loaded from SGPR bases with 32-bit lane offsets (as in
// fetch_rows32; needs the Indexer-K row stride at most kMaxStride32
// elements), after the slot loads: with so few blocks the slots and the
// offsets that depend on them are the longer chain, so they leave first.
template <int R, bool L32>
__global__ __launch_bounds__(kSmallWaves * 64) void small_store_kernel(
    const uint16_t* latent, const uint16_t* rope, const uint16_t* indexer,
    const int64_t* __restrict__ slots, uint32_t num_tokens, uint32_t latent_stride, uint32_t rope_stride,
    uint32_t indexer_stride, const CtxHead* __restrict__ head, const StoreParams p) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t round = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // 0..4
    const uint32_t t0 = blockIdx.x * kTokensPerWave;
    const uint32_t last = num_tokens - 1;
    int64_t sl[4];
    fetch_slots(slots, t0, last, sl);
    const CtxHead h = *head;
    u32x4 row, rp = u32x4{0u, 0u, 0u, 0u};
    if constexpr (L32) {
        if (round < 4) {
            const uint32_t t = t0 + round < last ? t0 + round : last;
            rp = ld16_at(uniform_base(rope + (uint64_t)t * rope_stride), (lane & 7u) * 16u);
            row = ld16_at(uniform_base(latent + (uint64_t)t * latent_stride), lane * 16u);
        } else {
            const uint32_t tb = t0 < last ? t0 : last, ug = t0 + (lane >> 4);
            const uint32_t kg = (ug < last ? ug : last) - tb;
            row = ld16_at(uniform_base(indexer + (uint64_t)tb * indexer_stride),
                          kg * (indexer_stride * 2u) + (lane & 15u) * 16u);
        }
    } else {
        if (round < 4) {
            const uint32_t t = t0 + round < last ? t0 + round : last;
            rp = ld16(rope + (uint64_t)t * rope_stride + (lane & 7u) * 8u);
            row = ld16(latent + (uint64_t)t * latent_stride + lane * 8u);
        } else {
            const uint32_t ug = t0 + (lane >> 4), tg = ug < last ? ug : last;
            row = ld16(indexer + (uint64_t)tg * indexer_stride + (lane & 15u) * 8u);
        }
    }
    const bool poisoned = (h.status & kStatusPoisoned) != 0;
    uint32_t nbad = 0, tok = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        sl[k] = t0 + k <= last ? sl[k] : -1;
        const bool good = slot_ok<false>(sl[k], h.capacity);
        nbad += (sl[k] != -1 && !good) ? 1u : 0u;
        tok |= (!poisoned && good) ? (1u << k) : 0u;
    }
    if (round == 0 && nbad != 0 && !poisoned && lane == 0) atomicAdd(p.invalid_count, (unsigned long long)nbad);
    // Store offsets and replica bases (kernel arguments), worked out while the
    // rows are in flight: fetched after the data they would add a round trip.
    // Waves 0..3: the token's Main-KV row (uniform); wave 4: this lane's
    // token's Indexer-K codes and scale.  Offsets of skipped slots are unused.
    const Bases<R> b = pin_bases<R>(p);
    uint64_t off0, off1 = 0;
    if (round < 4) {
        const uint64_t s = (uint64_t)(round == 0 ? sl[0] : round == 1 ? sl[1] : round == 2 ? sl[2] : sl[3]);
        off0 = (s >> 6) * p.main_page_stride + (s & 63u) * 656u;
    } else {
        const uint32_t g = lane >> 4;
        const uint64_t s = (uint64_t)(g == 0 ? sl[0] : g == 1 ? sl[1] : g == 2 ? sl[2] : sl[3]);
        const uint64_t page = (s >> 6) * p.idx_page_stride, in = s & 63u;
        off0 = page + in * 128u;
        off1 = page + 8192u + in * 4u;
    }
    off0 = pin_v(off0);
    off1 = pin_v(off1);
    __builtin_amdgcn_sched_barrier(0);

    const uint32_t ab = row_max16(lane_amax_bits(row));
    const uint32_t E = ab >> 7;
    const bool f = E >= kFastMinExponent && E < 255u;
    const TileScale t = tile_scale(ab);
    float x[8], q[8];
    unpack8(row, x);
    float scale;
    if (__all(f)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = quotient_fast(x[e], t.s, t.y);
        scale = t.s;
    } else {
        const float s_exact = __uint_as_float(ab << 16) / kE4m3Max;
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = f ? quotient_fast(x[e], t.s, t.y) : quotient_exact(x[e], s_exact);
        scale = f ? t.s : s_exact;
    }
    const u32x2 codes = cvt8(q);

    if (round < 4) {
        if (!((tok >> round) & 1u)) return;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            gbyte* rw = b.main[r] + off0;
            *(gptr<u32x2>)(rw + lane * 8u) = codes;
            *(gptr<uint32_t>)(rw + 512u + (lane >> 4) * 4u) = __float_as_uint(scale);
            if (lane < 8u) *(gptr<u32x4>)(rw + 528u + lane * 16u) = rp;
        }
    } else {
        if (!((tok >> (lane >> 4)) & 1u)) return;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            *(gptr<u32x2>)(b.idx[r] + off0 + (lane & 15u) * 8u) = codes;
            *(gptr<uint32_t>)(b.idx[r] + off1) = __float_as_uint(scale);
        }
    }
}

}  // namespace

template <bool NT, bool WT, bool O32, int WPB>
static void launch_r(uint32_t num_replicas, hipStream_t stream, const uint16_t* lat,
                     const uint16_t* rp, const uint16_t* ix, const int64_t* sl, uint32_t n, const StoreParams& p) {
    const dim3 grid((n + kTokensPerWave * WPB - 1) / (kTokensPerWave * WPB)), block(WPB * 64);
#define KVPUB_ROW_ARGS lat, rp, ix, sl, n, (uint32_t)p.latent_stride, (uint32_t)p.rope_stride, \
    (uint32_t)p.indexer_stride, p.head, p
    switch (num_replicas) {
        case 1: store_kernel<1, NT, WT, O32, WPB><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS); break;
        case 2: store_kernel<2, NT, WT, O32, WPB><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS); break;
        case 3: store_kernel<3, NT, WT, O32, WPB><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS); break;
        case 4: store_kernel<4, NT, WT, O32, WPB><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS); break;
        case 5: store_kernel<5, NT, WT, O32, WPB><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS); break;
        case 6: store_kernel<6, NT, WT, O32, WPB><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS); break;
        case 7: store_kernel<7, NT, WT, O32, WPB><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS); break;
        default: store_kernel<8, NT, WT, O32, WPB><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS); break;
    }
#undef KVPUB_ROW_ARGS
}

template <bool L32>
static void launch_small_l(uint32_t num_replicas, uint32_t n, hipStream_t stream, const StoreParams& p) {
    const dim3 grid((n + kTokensPerWave - 1) / kTokensPerWave), block(kSmallWaves * 64);
#define KVPUB_ROW_ARGS p.latent, p.rope, p.indexer, p.slots, n, (uint32_t)p.latent_stride, \
    (uint32_t)p.rope_stride, (uint32_t)p.indexer_stride, p.head, p
    switch (num_replicas) {
        case 1: small_store_kernel<1, L32><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS); break;
        case 2: small_store_kernel<2, L32><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS); break;
        case 3: small_store_kernel<3, L32><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS); break;
        case 4: small_store_kernel<4, L32><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS); break;
        case 5: small_store_kernel<5, L32><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS); break;
        case 6: small_store_kernel<6, L32><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS); break;
        case 7: small_store_kernel<7, L32><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS); break;
        default: small_store_kernel<8, L32><<<grid, block, 0, stream>>>(KVPUB_ROW_ARGS); break;
    }
#undef KVPUB_ROW_ARGS
}

static void launch_small(uint32_t num_replicas, uint32_t n, hipStream_t stream, const StoreParams& p) {
    if (p.indexer_stride <= kMaxStride32) launch_small_l<true>(num_replicas, n, stream, p);
    else launch_small_l<false>(num_replicas, n, stream, p);
}

hipError_t launch_store(const StoreParams& p, uint32_t num_replicas, hipStream_t stream) {
    if (num_replicas < 1 || num_replicas > (uint32_t)kMaxReplicas) return hipErrorInvalidValue;
    // Small batches: five waves per group of 4 tokens.  Otherwise one wave per
    // group, with batches beyond kMaxTokensPerLaunch split so that the grid
    // stays far inside its limits, and the store policy chosen per launch.
    (void)hipGetLastError();
    if (p.num_tokens <= (num_replicas <= 2 ? 2 * kSmallBatchTokens : kSmallBatchTokens)) {
        launch_small(num_replicas, (uint32_t)p.num_tokens, stream, p);
        return hipGetLastError();
    }
    for (int64_t t = 0; t < p.num_tokens; t += kMaxTokensPerLaunch) {
        const int64_t n = p.num_tokens - t < kMaxTokensPerLaunch ? p.num_tokens - t : kMaxTokensPerLaunch;
        const uint16_t* lat = p.latent + t * p.latent_stride;
        const uint16_t* rp = p.rope + t * p.rope_stride;
        const uint16_t* ix = p.indexer + t * p.indexer_stride;
        const int64_t* sl = p.slots + t;
        const int64_t written = n * (int64_t)num_replicas * kCacheBytesPerToken;
        // every layer spans less than 4 GiB: 32-bit offsets (the write-through
        // path's buffer stores need them); streamed launches also load with
        // 32-bit offsets, which needs input rows at most kMaxStride32 elements apart
        const bool offsets32 = p.main_region != 0 && p.idx_region != 0;
        const bool loads32 = p.latent_stride <= kMaxStride32 && p.rope_stride <= kMaxStride32 &&
                             p.indexer_stride <= kMaxStride32;
        const uint32_t un = (uint32_t)n;
        // (launches over 32 MB: blocks of kBlockRunWaves waves with block runs)
        if (written <= kStreamingStoreBytes) {
            if (offsets32 && loads32)
                launch_r<true, false, true, kWavesPerBlock>(num_replicas, stream, lat, rp, ix, sl, un, p);
            else launch_r<true, false, false, kWavesPerBlock>(num_replicas, stream, lat, rp, ix, sl, un, p);
        } else if (written > kWriteThroughBytes && offsets32) {
            launch_r<false, true, true, kBlockRunWaves>(num_replicas, stream, lat, rp, ix, sl, un, p);
        } else {
            if (offsets32) launch_r<false, false, true, kWavesPerBlock>(num_replicas, stream, lat, rp, ix, sl, un, p);
            else launch_r<false, false, false, kWavesPerBlock>(num_replicas, stream, lat, rp, ix, sl, un, p);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kvpub
