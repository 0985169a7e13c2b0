/*
 * kvpub_floor.h -- a plain-stream floor kernel for measurement (MI355X, gfx950).
 *
 * C ABI of libkvpub_floor.so, a companion of libkvpub.so used by the
 * benchmark only.  It moves the same number of bytes as a cache-store launch
 * with none of its work: it reads `in_bytes` contiguous bytes once
 * (non-temporal 16-byte loads) and writes `out_bytes` contiguous bytes to each
 * of `n_outs` buffers as whole, aligned 16-byte pieces, so a launch's duration
 * is what the memory system needs for that traffic on this GPU.  The store's
 * algorithmic bytes per launch are valid tokens x (1408 read + R x 788
 * written) (vLLM PR #52863, Design: one read of the final rows, stores to
 * every replica); timing this kernel with in_bytes = T x 1408 and R outputs of
 * T x 788 bytes gives the achievable time for the store's bytes.  Each output
 * piece holds the input piece of the same index (pieces past the input's end
 * hold their own index in every word).  A second entry point launches an
 * empty kernel, the fixed per-launch cost.
 */
#ifndef KVPUB_FLOOR_H
#define KVPUB_FLOOR_H

#include <stdint.h>

#if defined(KVPUB_BUILD_SHARED)
#define KVPUB_FLOOR_API __attribute__((visibility("default")))
#else
#define KVPUB_FLOOR_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* How the output stores treat the L2. */
#define KVPUB_FLOOR_WRITE_BACK 0u     /* ordinary stores */
#define KVPUB_FLOOR_NON_TEMPORAL 1u   /* streamed past the L2 */
#define KVPUB_FLOOR_WRITE_THROUGH 2u  /* device-coherent buffer stores (sc1): written through the L2 */

/* Enqueue one launch on `stream` (a hipStream_t; NULL = the null stream).
 *   in:   device pointer, 16-byte aligned, in_bytes (a multiple of 16, > 0)
 *   outs: n_outs (1..8) device pointers, 16-byte aligned, out_bytes each
 *         (a multiple of 16, > 0; below 2^32 for KVPUB_FLOOR_WRITE_THROUGH)
 * Returns 0 when launched, 1 for an invalid argument (nothing launched), 4 if
 * the launch failed.  No allocation, no synchronization. */
KVPUB_FLOOR_API int kvpub_floor_stream(const void *in, uint64_t in_bytes, void *const *outs, uint32_t n_outs,
                                       uint64_t out_bytes, uint32_t policy, void *stream);

/* Enqueue one launch of an empty kernel (no instruction but the end) with
 * `blocks` (1..2^31-1) blocks of `threads` (64..1024, a multiple of 64)
 * threads on `stream`: the fixed cost of a launch of that shape, which a
 * replayed graph of such launches measures per node.  Returns 0 when
 * launched, 1 for an invalid argument (nothing launched), 4 if the launch
 * failed. */
KVPUB_FLOOR_API int kvpub_floor_empty(uint32_t blocks, uint32_t threads, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVPUB_FLOOR_H */
