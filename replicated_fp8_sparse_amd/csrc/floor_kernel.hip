// Plain-stream floor kernel and an empty kernel (measurement only; see
// include/kvpub_floor.h).
//
// One 16-byte piece per lane: lane i loads input piece i (non-temporal) and
// stores it to output piece i of every output buffer.  Lanes past the output
// keep their loaded value alive with an empty asm use, so every input byte is
// read; lanes past the input store their index.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvpub_floor.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kMaxOuts = 8;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer resource, 32-bit data format (gfx950)
constexpr int kDeviceCoherent = 16;      // buffer cache-policy bits: sc1

struct Outs {
    u32x4* p[kMaxOuts];
};

template <int N, uint32_t POLICY>
__global__ __launch_bounds__(256) void floor_kernel(const u32x4* __restrict__ in, uint64_t in_pieces, Outs outs,
                                                   uint64_t out_pieces) {
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    u32x4 v;
    if (i < in_pieces) {
        v = __builtin_nontemporal_load(in + i);
    } else {
        const uint32_t k = (uint32_t)i;
        v = u32x4{k, k, k, k};
    }
    if (i >= out_pieces) {
        asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w));
        return;
    }
#pragma unroll
    for (int r = 0; r < N; ++r) {
        if constexpr (POLICY == KVPUB_FLOOR_WRITE_THROUGH) {
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)outs.p[r], 0, (int)(uint32_t)(out_pieces * 16u), kRsrcWord3);
            __builtin_amdgcn_raw_buffer_store_b128(v, rs, (int)(uint32_t)(i * 16u), 0, kDeviceCoherent);
        } else if constexpr (POLICY == KVPUB_FLOOR_NON_TEMPORAL) {
            __builtin_nontemporal_store(v, outs.p[r] + i);
        } else {
            outs.p[r][i] = v;
        }
    }
}

template <uint32_t POLICY>
void launch_n(uint32_t n, dim3 grid, hipStream_t s, const u32x4* in, uint64_t pin, const Outs& o, uint64_t pout) {
    switch (n) {
        case 1: floor_kernel<1, POLICY><<<grid, 256, 0, s>>>(in, pin, o, pout); break;
        case 2: floor_kernel<2, POLICY><<<grid, 256, 0, s>>>(in, pin, o, pout); break;
        case 3: floor_kernel<3, POLICY><<<grid, 256, 0, s>>>(in, pin, o, pout); break;
        case 4: floor_kernel<4, POLICY><<<grid, 256, 0, s>>>(in, pin, o, pout); break;
        case 5: floor_kernel<5, POLICY><<<grid, 256, 0, s>>>(in, pin, o, pout); break;
        case 6: floor_kernel<6, POLICY><<<grid, 256, 0, s>>>(in, pin, o, pout); break;
        case 7: floor_kernel<7, POLICY><<<grid, 256, 0, s>>>(in, pin, o, pout); break;
        default: floor_kernel<8, POLICY><<<grid, 256, 0, s>>>(in, pin, o, pout); break;
    }
}

// Nothing but the end of the program: the cost of a launch as such.
__global__ void empty_kernel() {}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" KVPUB_FLOOR_API int kvpub_floor_stream(const void* in, uint64_t in_bytes, void* const* outs,
                                                  uint32_t n_outs, uint64_t out_bytes, uint32_t policy,
                                                  void* stream) {
    if (!in || !outs || n_outs < 1 || n_outs > kMaxOuts || !aligned16(in)) return 1;
    if (in_bytes == 0 || out_bytes == 0 || in_bytes % 16 || out_bytes % 16) return 1;
    if (policy > KVPUB_FLOOR_WRITE_THROUGH) return 1;
    if (policy == KVPUB_FLOOR_WRITE_THROUGH && out_bytes > UINT32_MAX) return 1;
    Outs o = {};
    for (uint32_t r = 0; r < n_outs; ++r) {
        if (!outs[r] || !aligned16(outs[r])) return 1;
        o.p[r] = static_cast<u32x4*>(outs[r]);
    }
    const uint64_t pin = in_bytes / 16, pout = out_bytes / 16;
    const uint64_t n = pin > pout ? pin : pout;
    const uint64_t blocks = (n + 255) / 256;
    if (blocks > 0x7FFFFFFFull) return 1;
    const dim3 grid((uint32_t)blocks);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4* src = static_cast<const u32x4*>(in);
    (void)hipGetLastError();
    if (policy == KVPUB_FLOOR_WRITE_BACK) launch_n<KVPUB_FLOOR_WRITE_BACK>(n_outs, grid, s, src, pin, o, pout);
    else if (policy == KVPUB_FLOOR_NON_TEMPORAL) launch_n<KVPUB_FLOOR_NON_TEMPORAL>(n_outs, grid, s, src, pin, o, pout);
    else launch_n<KVPUB_FLOOR_WRITE_THROUGH>(n_outs, grid, s, src, pin, o, pout);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" KVPUB_FLOOR_API int kvpub_floor_empty(uint32_t blocks, uint32_t threads, void* stream) {
    if (blocks < 1 || blocks > 0x7FFFFFFFu || threads < 64 || threads > 1024 || threads % 64) return 1;
    (void)hipGetLastError();
    empty_kernel<<<dim3(blocks), dim3(threads), 0, static_cast<hipStream_t>(stream)>>>();
    return hipGetLastError() == hipSuccess ? 0 : 4;
}
