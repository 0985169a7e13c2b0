// Dequantizing gather for gfx950: the reader side of the replicated cache.
//
// vLLM PR #52863 "[Kernel][PCP] Publish replicated KV updates through PyTorch
// symmetric memory", Summary and Design: the existing attention kernels keep
// reading the local replica, in the fp8_ds_mla layout the store writes.  This
// kernel reads the rows of given slots from one replica and turns them back
// into bf16: element = bf16(RN32(value(code) * scale)), RoPE bits copied.
//
// Work mapping (wave64), the store's mirror image.  A wave owns 4 consecutive
// output tokens; a DPP row of 16 lanes x 8 codes (8 bytes per lane) is one
// 128-element tile:
//   round k = 0..3: token k's latent, lanes 16j..16j+15 = tile j;
//   round 4:        the indexer rows, lanes 16g..16g+15 = token g;
// lanes 0..31 also carry the 4 tokens' RoPE rows (8 lanes x 16 B each).
// The slots and the capacity (from the context's device words, so a captured
// gather sees a grown storage) arrive together through scalar loads.  A padded or
// out-of-range slot reads slot 0's bytes (always in bounds, so no load sits
// behind a branch) and its output row is written as zeros; with no backed
// page at all nothing is read.  Decode: the gfx950 OCP e4m3 -> f32 convert
// (exact), one binary32 multiply by the tile scale, a round-to-nearest-even
// f32 -> bf16 convert; each lane stores 8 bf16 = 16 bytes.  Every output line
// is written whole, so the stores stream past L2 (non-temporal): nothing is
// left dirty for the end-of-kernel write-back.
#include "kvpub_internal.h"

namespace kvpub {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <class T> using gptr = __attribute__((address_space(1))) T*;
template <class T> using cgptr = const __attribute__((address_space(1))) T*;

constexpr int kGatherWaves = 4;                       // waves per block
constexpr int kGatherTokensPerBlock = 4 * kGatherWaves;
constexpr int kNumXcds = 8;

// Block b runs on XCD b % 8: give each XCD a contiguous range of token chunks.
__device__ __forceinline__ uint32_t xcd_chunk(uint32_t b, uint32_t n) {
    const uint32_t per = n / kNumXcds, rem = n % kNumXcds;
    const uint32_t x = b % kNumXcds, i = b / kNumXcds;
    return x * per + (x < rem ? x : rem) + i;
}

// Two bf16 bit patterns (low half first) from two binary32 values, nearest-even.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const bf16x2 h = __builtin_convertvector(f32x2{a, b}, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

// 8 codes (little-endian in c) times one scale -> 8 bf16 in 16 bytes.
__device__ __forceinline__ u32x4 dequant8(u32x2 c, float scale) {
    u32x4 r;
    // the convert's word select picks bytes 0,1 (false) or 2,3 (true) of its source
    const f32x2 a0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, false);
    const f32x2 a1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, true);
    const f32x2 b0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, false);
    const f32x2 b1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, true);
    r.x = pack_bf16(a0.x * scale, a0.y * scale);
    r.y = pack_bf16(a1.x * scale, a1.y * scale);
    r.z = pack_bf16(b0.x * scale, b0.y * scale);
    r.w = pack_bf16(b1.x * scale, b1.y * scale);
    return r;
}

__device__ __forceinline__ bool slot_ok(int64_t s, int64_t capacity) {
    return (uint64_t)s < (uint64_t)capacity;   // negative slots wrap to huge values
}

// v_i for a per-lane index i in 0..3; v0..v3 wave-uniform.
__device__ __forceinline__ uint64_t pick4(uint64_t v0, uint64_t v1, uint64_t v2, uint64_t v3, uint32_t i) {
    const uint64_t a = (i & 1u) ? v1 : v0;
    const uint64_t b = (i & 1u) ? v3 : v2;
    return (i & 2u) ? b : a;
}

template <class T>
__device__ __forceinline__ void st_nt(uint16_t* p, T v) {
    __builtin_nontemporal_store(v, (gptr<T>)p);
}

template <class T>
__device__ __forceinline__ T ld_nt(const uint8_t* p) {
    return __builtin_nontemporal_load((cgptr<T>)p);
}

// The arguments the first instructions need are plain scalars, preloaded in
// SGPRs (kernel-argument preloading): the slot loads issue at once.
// Off32: the layer spans less than 2^32 bytes, so the page offsets are 32-bit
// products (one scalar multiply each instead of a 64-bit sequence): the row
// loads wait on these, so they sit on the critical path.
template <bool Off32>
__global__ __launch_bounds__(kGatherWaves * 64) void gather_kernel(
    const int64_t* __restrict__ slots, uint32_t num_tokens, const uint8_t* main_base, const uint8_t* idx_base,
    uint64_t main_page_stride, uint64_t idx_page_stride, const CtxHead* __restrict__ head, const GatherParams p) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t num_blocks = (num_tokens + kGatherTokensPerBlock - 1) / kGatherTokensPerBlock;   // == gridDim.x
    const uint32_t t0 = (xcd_chunk(blockIdx.x, num_blocks) * kGatherWaves + wave) * 4u;
    if (t0 >= num_tokens) return;
    const uint32_t last = num_tokens - 1;
    // The four slots (token indices clamped to the last token: always in
    // bounds) and the capacity are fetched together, so a single scalar round
    // trip precedes the row loads; nothing waits on one before issuing another.
    int64_t sl[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) sl[k] = slots[t0 + k < last ? t0 + k : last];
    const int64_t capacity = head->capacity;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    if (capacity == 0) {
        // no page is backed (a VMM storage that lost a layer): read nothing,
        // every output row is zero and every non-padded slot is counted
        uint32_t n = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (t0 + k > last) break;
            n += sl[k] != -1 ? 1u : 0u;
            st_nt<u32x4>(p.latent + (uint64_t)(t0 + k) * p.latent_stride + lane * 8u, zero);
        }
        const uint32_t g = lane >> 4, r = (lane >> 3) & 3u;
        if (t0 + g <= last) st_nt<u32x4>(p.indexer + (uint64_t)(t0 + g) * p.indexer_stride + (lane & 15u) * 8u, zero);
        if (lane < 32u && t0 + r <= last) st_nt<u32x4>(p.rope + (uint64_t)(t0 + r) * p.rope_stride + (lane & 7u) * 8u, zero);
        if (n != 0 && lane == 0) atomicAdd(p.invalid_count, (unsigned long long)n);
        return;
    }
    uint64_t row[4], irow[4], iscl[4];
    uint32_t ok = 0, nbad = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t v = t0 + k <= last ? sl[k] : -1;
        const bool good = slot_ok(v, capacity);
        nbad += (v != -1 && !good) ? 1u : 0u;
        ok |= good ? (1u << k) : 0u;
        const uint64_t s = good ? (uint64_t)v : 0u;   // bad slots read slot 0 (in bounds) and emit zeros
        const uint64_t page = s >> 6, in = s & 63u;
        if constexpr (Off32) {
            const uint32_t pg = (uint32_t)page, o = (uint32_t)in;
            const uint32_t ib = pg * (uint32_t)idx_page_stride;
            row[k] = pg * (uint32_t)main_page_stride + o * 656u;
            irow[k] = ib + o * 128u;
            iscl[k] = ib + 8192u + o * 4u;
        } else {
            row[k] = page * main_page_stride + in * 656u;
            irow[k] = page * idx_page_stride + in * 128u;
            iscl[k] = page * idx_page_stride + 8192u + in * 4u;
        }
    }
    ok = __builtin_amdgcn_readfirstlane(ok);

    // loads (read once: non-temporal): four latent tiles (codes + the row's
    // scale), the indexer tile, RoPE
    const uint32_t j = lane >> 4, g = lane >> 4, r = (lane >> 3) & 3u;
    u32x2 code[5];
    float scale[5];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint8_t* rw = main_base + row[k];
        code[k] = ld_nt<u32x2>(rw + lane * 8u);
        scale[k] = ld_nt<float>(rw + 512u + j * 4u);
    }
    const uint64_t my_irow = pick4(irow[0], irow[1], irow[2], irow[3], g);
    const uint64_t my_iscl = pick4(iscl[0], iscl[1], iscl[2], iscl[3], g);
    code[4] = ld_nt<u32x2>(idx_base + my_irow + (lane & 15u) * 8u);
    scale[4] = ld_nt<float>(idx_base + my_iscl);
    const uint64_t my_rope = pick4(row[0], row[1], row[2], row[3], r) + 528u + (lane & 7u) * 16u;
    const u32x4 rp = ld_nt<u32x4>(main_base + my_rope);
    if (nbad != 0 && lane == 0) atomicAdd(p.invalid_count, (unsigned long long)nbad);

    // dequantize and store
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (t0 + k > last) break;                // uniform: the tail of the last group
        const u32x4 v = ((ok >> k) & 1u) ? dequant8(code[k], scale[k]) : zero;
        st_nt<u32x4>(p.latent + (uint64_t)(t0 + k) * p.latent_stride + lane * 8u, v);
    }
    if (t0 + g <= last) {
        const u32x4 v = ((ok >> g) & 1u) ? dequant8(code[4], scale[4]) : zero;
        st_nt<u32x4>(p.indexer + (uint64_t)(t0 + g) * p.indexer_stride + (lane & 15u) * 8u, v);
    }
    if (lane < 32u && t0 + r <= last) {
        const u32x4 v = ((ok >> r) & 1u) ? rp : zero;
        st_nt<u32x4>(p.rope + (uint64_t)(t0 + r) * p.rope_stride + (lane & 7u) * 8u, v);
    }
}

}  // namespace

hipError_t launch_gather(const GatherParams& p, hipStream_t stream) {
    (void)hipGetLastError();
    for (int64_t t = 0; t < p.num_tokens; t += kMaxTokensPerLaunch) {
        GatherParams q = p;
        q.num_tokens = p.num_tokens - t < kMaxTokensPerLaunch ? p.num_tokens - t : kMaxTokensPerLaunch;
        q.slots = p.slots + t;
        q.latent = p.latent + t * p.latent_stride;
        q.rope = p.rope + t * p.rope_stride;
        q.indexer = p.indexer + t * p.indexer_stride;
        const uint32_t blocks = (uint32_t)((q.num_tokens + kGatherTokensPerBlock - 1) / kGatherTokensPerBlock);
        if (q.offsets32)
            gather_kernel<true><<<dim3(blocks), dim3(kGatherWaves * 64), 0, stream>>>(
                q.slots, (uint32_t)q.num_tokens, q.main_base, q.idx_base, q.main_page_stride, q.idx_page_stride,
                q.head, q);
        else
            gather_kernel<false><<<dim3(blocks), dim3(kGatherWaves * 64), 0, stream>>>(
                q.slots, (uint32_t)q.num_tokens, q.main_base, q.idx_base, q.main_page_stride, q.idx_page_stride,
                q.head, q);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kvpub
