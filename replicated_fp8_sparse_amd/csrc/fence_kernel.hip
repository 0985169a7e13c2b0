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
//   e = epoch[lane] + 1, by an RMW at system scope with release semantics:
//       every write this GPU made before the fence is visible before the
//       epoch moves (with peers also acquire: what was published before it is
//       visible after);
//   with peers only: signal[self] = e (a release store), then for every
//       other participant q: acquire-load signal[q] until it is >= e.
// Alone (one participant) the release RMW is followed by acquire loads of the
// epoch itself until it is >= e (with one participant the epoch is the only
// signal): the release/acquire pair of PR #52863's Design section.  A context
// created with the release-only option skips the acquire half, which has
// nothing to act on alone (see fence_kernel).
// This GPU's own signal is never awaited: it was written just before, in
// program order, by the same wave.  The expected value e is read from device
// memory, never passed as a kernel argument, so replaying a captured launch
// keeps advancing the epoch.  With host-driven peers the other signals live
// in host-coherent memory.
// The wait is bounded by the wall clock (s_memrealtime).  On timeout the
// kernel sets the timeout and poisoned flags and returns normally; stores and
// fences of a poisoned context write nothing.
#include "kvpub_internal.h"

namespace kvpub {
namespace {

// Bounded acquire wait until *w >= e; on timeout the context's sticky timeout
// and poisoned flags are set.  Returns false on timeout.
__device__ __forceinline__ bool wait_at_least(const uint64_t* w, uint64_t e, uint32_t* status,
                                              uint64_t start, uint64_t timeout_ticks) {
    while (__hip_atomic_load(w, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM) < e) {
        if (wall_clock64() - start > timeout_ticks) {
            __hip_atomic_fetch_or(status, kStatusFenceTimeout | kStatusPoisoned, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_SYSTEM);
            return false;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    return true;
}

// Plain scalar arguments, so that they arrive preloaded in SGPRs.
__global__ __launch_bounds__(64) void fence_kernel(uint64_t* epoch, uint64_t* signals, uint32_t* status,
                                                   uint32_t num_participants, uint32_t self,
                                                   uint64_t timeout_ticks, uint32_t acquire_wait) {
    if (threadIdx.x != 0) return;
    if (num_participants == 1 && acquire_wait) {
        // Release RMW, then acquire loads of the epoch until it has reached the
        // value this fence moved it to.  The RMW's result already shows that
        // value, so the first load passes unless the epoch was moved back (by a
        // host-epoch fence on the same lane); the wait is bounded all the same.
        // No status check first: only a wait can poison, and one that follows
        // this wave's own RMW does not time out in normal use.
        const uint64_t e =
            __hip_atomic_fetch_add(epoch, (uint64_t)1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM) + 1;
        (void)wait_at_least(epoch, e, status, wall_clock64(), timeout_ticks);
        return;
    }
    if (num_participants == 1) {
        // The release-only option: a release RMW at system scope publishes
        // every write this GPU made before the fence, then the epoch moves, and
        // nothing more.  The acquire half has nothing to act on alone: no other
        // agent publishes into this GPU's memory, and this wave ends right after
        // the RMW, so work after the fence runs in later kernels, which are
        // ordered by their own acquire at dispatch (an acquire here would only
        // invalidate the L2 for them).
        __hip_atomic_fetch_add(epoch, (uint64_t)1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
        return;
    }
    if (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kStatusPoisoned) return;
    const uint64_t e =
        __hip_atomic_fetch_add(epoch, (uint64_t)1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_SYSTEM) + 1;
    uint64_t* own = signals + (size_t)self * kSignalStride;
    __hip_atomic_store(own, e, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    const uint64_t start = wall_clock64();
    for (uint32_t q = 0; q < num_participants; ++q) {
        if (q == self) continue;
        if (!wait_at_least(signals + (size_t)q * kSignalStride, e, status, start, timeout_ticks)) return;
    }
}

// The two-launch fence with a host-held epoch (PR #54030 Motivation: the
// design that the single-launch fence replaces, kept to reproduce the pages'
// comparison).  The host counts the epoch and passes the value e to both
// kernels as an argument: the first publishes it with a system-scope release
// store, the second acquire-waits until the word holds at least e.  A captured
// pair therefore carries the value of its capture: replays publish the same e
// again and the epoch does not advance.  With one participant only; like the
// one-participant single-launch fence, the publication does not read the
// status word.
__global__ __launch_bounds__(64) void host_epoch_publish_kernel(uint64_t* epoch, uint64_t e) {
    if (threadIdx.x != 0) return;
    __hip_atomic_store(epoch, e, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

__global__ __launch_bounds__(64) void host_epoch_wait_kernel(const uint64_t* epoch, uint32_t* status, uint64_t e,
                                                             uint64_t timeout_ticks) {
    if (threadIdx.x != 0) return;
    (void)wait_at_least(epoch, e, status, wall_clock64(), timeout_ticks);
}

}  // namespace

hipError_t launch_fence(const FenceParams& p, hipStream_t stream) {
    (void)hipGetLastError();
    fence_kernel<<<dim3(1), dim3(64), 0, stream>>>(p.epoch, p.signals, p.status, p.num_participants, p.self,
                                                   p.timeout_ticks, p.acquire_wait);
    return hipGetLastError();
}

hipError_t launch_host_epoch_fence(const FenceParams& p, uint64_t e, hipStream_t stream) {
    (void)hipGetLastError();
    host_epoch_publish_kernel<<<dim3(1), dim3(64), 0, stream>>>(p.epoch, e);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    host_epoch_wait_kernel<<<dim3(1), dim3(64), 0, stream>>>(p.epoch, p.status, e, p.timeout_ticks);
    return hipGetLastError();
}

}  // namespace kvpub
