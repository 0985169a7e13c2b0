// Single-launch device-epoch fence for gfx950.
//
// vLLM PR #54030 "[Perf][PCP] Fuse direct-KV publication fence": the epoch
// moves onto the device and one kernel both publishes at system scope and
// waits for the peers, so a fence is one launch instead of two (Motivation:
// one fence per sparse layer makes launch overhead visible) and a captured
// graph advances the epoch on every replay (a host-held epoch cannot).  The
// second commit makes a timed-out fence fail closed.  PR #52863 Design: the
// barrier is a system-scope release/acquire and has separate lanes for
// overlapped micro-batches.
//
// Protocol per lane, run by lane 0 of one wavefront:
//   e = epoch[lane] + 1, written back with a system-scope release RMW;
//   signal[self] = e (system-scope release store);
//   for every participant q: acquire-load signal[q] until it is >= e.
// The expected value e is read from device memory, never passed as a kernel
// argument, so replaying a captured launch keeps advancing the epoch.  On one
// GPU there is one participant (this GPU) and the wait ends at once; with
// host-driven peers the other signals live in host-coherent memory.
// The wait is bounded by the wall clock (s_memrealtime).  On timeout the
// kernel sets the timeout and poisoned flags and returns normally; stores and
// fences of a poisoned context write nothing.
#include "kvpub_internal.h"

namespace kvpub {
namespace {

__global__ __launch_bounds__(64) void fence_kernel(const FenceParams p) {
    if (threadIdx.x != 0) return;
    if (__hip_atomic_load(p.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kStatusPoisoned)
        return;
    const uint64_t e =
        __hip_atomic_fetch_add(p.epoch, (uint64_t)1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM) + 1;
    __hip_atomic_store(p.signals + (size_t)p.self * kSignalStride, e, __ATOMIC_RELEASE,
                       __HIP_MEMORY_SCOPE_SYSTEM);
    const uint64_t start = wall_clock64();
    for (uint32_t q = 0; q < p.num_participants; ++q) {
        const uint64_t* sig = p.signals + (size_t)q * kSignalStride;
        while (__hip_atomic_load(sig, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM) < e) {
            if (wall_clock64() - start > p.timeout_ticks) {
                __hip_atomic_fetch_or(p.status, kStatusFenceTimeout | kStatusPoisoned,
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                return;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
}

}  // namespace

hipError_t launch_fence(const FenceParams& p, hipStream_t stream) {
    (void)hipGetLastError();
    fence_kernel<<<dim3(1), dim3(64), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace kvpub
