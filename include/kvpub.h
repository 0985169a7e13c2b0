/*
 * kvpub.h -- replicated FP8 KV cache-store and device-epoch fence (MI355X, gfx950).
 *
 * C ABI of libkvpub.so.  Plain pointers and sizes only: device pointers are
 * HIP device addresses (for example torch tensors' data_ptr()), streams are
 * hipStream_t values passed as void*.
 *
 * What the library does, and where the pages define it:
 *   - kvpub_store: quantize each new token's final Main-KV row (bf16 latent
 *     [512] + bf16 RoPE [64]) and Indexer-K row (bf16 [128]) to FP8 once and
 *     write the bytes straight into every replica of a paged KV cache, with
 *     no gather and no receive-side insert (vLLM PR #52863 "[Kernel][PCP]
 *     Publish replicated KV updates through PyTorch symmetric memory",
 *     Summary, the "THIS PR: publish final rows directly" diagram, and the
 *     Design bullet on fused cache-store kernels writing to every peer).
 *     The replicas must end byte-identical to what gather-then-insert would
 *     give, padded and invalid slots and guard bytes included (same page,
 *     "Correctness and current-head validation").
 *   - kvpub_fence: one launch that advances a device-resident epoch with a
 *     system-scope release and then acquire-waits for every participant, so
 *     that a captured graph advances the epoch on every replay (vLLM PR
 *     #54030 "[Perf][PCP] Fuse direct-KV publication fence", its commit list
 *     and Motivation; PR #52863 Design bullet on the device-epoch barrier and
 *     separate DBO lanes).
 *   - kvpub_graph_create / kvpub_graph_replay: the store + fence sequence of
 *     several layers captured once in a hipGraph and replayed (PR #54030
 *     commit list: a two-GPU replay test checks that every replay advances the
 *     epoch; PR #52863 Design: graph replay is supported).
 *   - kvpub_gather: the reader side -- the rows of given slots read back from
 *     one replica and dequantized to bf16, which is what the attention kernels
 *     that keep reading the local replica consume (PR #52863 Summary and
 *     Design: the existing attention kernels read the local replica in the
 *     fp8_ds_mla layout this path writes).
 *   - kvpub_vmm_*: replica storage at stable virtual addresses that can grow
 *     without moving (PR #52863 Relationship to existing work: the path builds
 *     on a KV cache kept at a stable VA with its own rendezvous, so that the
 *     cache can expand without re-exchanging views).
 *   - all-or-nothing creation and fail-closed fences (PR #54030 commit list:
 *     opt-in allocation is all-or-nothing at startup; a fence timeout must not
 *     let work continue).
 *
 * Byte layout (the pages name the FP8 Main-KV format, fp8_ds_mla, without
 * printing its bytes; this is the library's reading):
 *   Main-KV row, 656 B, at replica + layer*main_layer_stride
 *                          + page*main_page_stride + offset*656:
 *     [0,512)   e4m3fn codes of latent[0..511]
 *     [512,528) fp32 scales of latent tiles [0,128) [128,256) [256,384) [384,512)
 *     [528,656) RoPE bf16 bit patterns, copied unchanged
 *   Indexer-K, at replica + layer*idx_layer_stride + page*idx_page_stride:
 *     [offset*128, +128)     e4m3fn codes of indexer[0..127]
 *     [8192 + offset*4, +4)  fp32 scale of the indexer row
 *   Scaling: per 128-element tile, scale = amax / 448 (binary32), code =
 *   e4m3fn(x / scale) with x / scale rounded to binary32, then rounded to
 *   nearest-even e4m3fn saturating at +-448; an all-zero tile stores scale
 *   +0 and codes 0x00.  All multi-byte fields are little-endian.
 *   Slots: slot s lives in page s / 64 at offset s % 64.  s == -1 marks a
 *   padded token: it is neither read nor written.  Any other slot outside
 *   [0, num_pages*64) is skipped and counted (kvpub_error_read).
 *
 * Errors: functions never abort and no C++ exception crosses this ABI.
 * Argument problems are reported before anything is launched, so nothing is
 * written.  Device-side problems (invalid slots, a fence that timed out) are
 * recorded in the context's device words and reported by kvpub_error_read.
 *
 * Logging: with the environment variable KVPUB_LOG=1 (read once), every
 * kvpub_create, kvpub_create_static and kvpub_destroy of a context prints one
 * line to stderr with its configuration and status; no other call logs.
 */
#ifndef KVPUB_H
#define KVPUB_H

#include <stdint.h>

#if defined(KVPUB_BUILD_SHARED)
#define KVPUB_API __attribute__((visibility("default")))
#else
#define KVPUB_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define KVPUB_ABI_VERSION 1u

#define KVPUB_SLOTS_PER_PAGE 64u
#define KVPUB_LATENT_DIM 512u
#define KVPUB_ROPE_DIM 64u
#define KVPUB_INDEXER_DIM 128u
#define KVPUB_MAIN_ROW_BYTES 656u
#define KVPUB_MAIN_PAGE_BYTES (64u * 656u)            /* 41984 */
#define KVPUB_IDX_PAGE_BYTES (64u * 128u + 64u * 4u)  /* 8448 */
#define KVPUB_IDX_SCALES_OFFSET (64u * 128u)          /* 8192 */
#define KVPUB_MAX_REPLICAS 8u
#define KVPUB_MAX_LANES 64u
#define KVPUB_MAX_PARTICIPANTS 8u
#define KVPUB_MAX_TOKENS (1ll << 30)

typedef struct kvpub_ctx kvpub_ctx;
typedef struct kvpub_graph kvpub_graph;
typedef struct kvpub_vmm kvpub_vmm;
typedef void *kvpub_stream_t; /* hipStream_t; NULL = the null stream */

typedef enum {
    KVPUB_OK = 0,
    KVPUB_ERR_INVALID_ARG = 1,   /* bad argument; nothing was launched */
    KVPUB_ERR_OUT_OF_MEMORY = 2, /* an allocation failed; nothing is left allocated */
    KVPUB_ERR_UNSUPPORTED = 3,   /* device is not gfx950, or the call does not support this
                                    configuration (documented per call) */
    KVPUB_ERR_HIP = 4,           /* a HIP runtime call failed */
    KVPUB_ERR_CAPTURING = 5,     /* a synchronizing call while a stream capture is active */
    KVPUB_ERR_FENCE_TIMEOUT = 6, /* a fence timed out: the context is poisoned */
    KVPUB_ERR_IN_USE = 7,        /* the device's static context (kvpub_create_static) is in use */
    KVPUB_STATUS_MAX_ENUM = 0x7FFFFFFF /* not a status: makes every non-negative int32 a valid
                                          kvpub_status value, so a C caller may pass any code */
} kvpub_status;

/* Sticky device flags reported by kvpub_error_read. */
#define KVPUB_FLAG_FENCE_TIMEOUT 0x1u /* a fence gave up waiting */
#define KVPUB_FLAG_POISONED 0x2u      /* later stores and fences do nothing */

typedef struct {
    uint32_t struct_size;       /* sizeof(kvpub_config) */
    uint32_t num_replicas;      /* R, 1..8 */
    uint32_t num_layers;        /* L >= 1 */
    uint32_t block_size;        /* slots per page; must be 64 */
    uint64_t num_pages;         /* pages per replica per layer, >= 1 */
    uint64_t main_page_stride;  /* bytes, >= 41984, multiple of 16 */
    uint64_t main_layer_stride; /* bytes, >= num_pages*main_page_stride, multiple of 16 (L == 1: see below) */
    uint64_t idx_page_stride;   /* bytes, >= 8448, multiple of 16 */
    uint64_t idx_layer_stride;  /* bytes, >= num_pages*idx_page_stride, multiple of 16 (L == 1: see below) */
    uint32_t num_lanes;         /* fence lanes (one per overlapped micro-batch), 1..64 */
    uint32_t num_participants;  /* fence participants, 1..8; > 1 only with host-driven peers (tests) */
    uint64_t fence_timeout_ns;  /* 0 = 5 s */
    int32_t device;             /* HIP device ordinal */
    uint32_t flags;             /* 0 or KVPUB_CONFIG_FENCE_RELEASE_ONLY; other bits must be 0 */
} kvpub_config;

/* With L == 1 the layer strides address nothing and are not checked; a value
 * above num_pages * page stride states the span the layer may grow into
 * (kvpub_vmm_create sets it to the reserved range), which large stores use as
 * the bound of their write-through buffer range.  Any value is safe: no store
 * goes beyond the context's capacity. */

/* kvpub_config.flags: with one participant, kvpub_fence is by default the
 * system-scope release RMW of the lane's epoch followed by acquire loads of the
 * epoch until it holds the value the RMW produced (with one participant the
 * epoch is the only signal) -- the release/acquire pair of vLLM PR #52863,
 * Design (device-epoch barrier).  With this flag it is the release RMW alone:
 * no other agent publishes into this GPU's memory, and work after the fence
 * runs in later kernels, which the queue orders with its own acquire at
 * dispatch, so the acquire half has nothing to act on; it saves the system-
 * scope cache invalidation of the acquire.  No effect with peers: their fence
 * always acquire-waits. */
#define KVPUB_CONFIG_FENCE_RELEASE_ONLY 0x1u

/* Fill *cfg with defaults for R replicas of L layers of num_pages dense pages:
 * page strides 41984 / 8448, layer strides num_pages * page stride, one lane,
 * one participant, device 0. */
KVPUB_API void kvpub_config_init(kvpub_config *cfg, uint32_t num_replicas, uint32_t num_layers,
                       uint64_t num_pages);

/* Create a context over R caller-owned replica buffers.
 * main_bases[r] / idx_bases[r]: device pointers, 16-byte aligned, each at least
 * (L-1)*layer_stride + num_pages*page_stride bytes.  The caller keeps ownership
 * and must keep them alive until kvpub_destroy.  The context owns only its
 * device words (status flags and slot capacity, invalid-slot counter, epochs,
 * participant signals) on `device`.
 * All-or-nothing: on any failure every resource it made is released and *out
 * is set to NULL.  Returns KVPUB_ERR_UNSUPPORTED unless the device is gfx950. */
KVPUB_API kvpub_status kvpub_create(const kvpub_config *cfg, void *const *main_bases,
                          void *const *idx_bases, kvpub_ctx **out);

/* kvpub_create for callers that cannot allocate: code that must not call
 * hipMalloc or any other allocator (tight serving loops, harnesses that forbid
 * allocation).  Same configuration rules, bases and behaviour as kvpub_create,
 * and the context is used and destroyed the same way (kvpub_destroy), but this
 * call allocates nothing, host or device: the context's device words (status
 * and capacity, invalid-slot counter, one epoch per lane) live in a fixed
 * 8448-byte array of the library's, one per GPU, held until the process ends,
 * and its host part in static storage.  The words are cleared and the capacity
 * written by a kernel enqueued on `stream` (a hipStream_t; NULL = the null
 * stream): work on the context must follow it on that stream or after it.
 * Limits: one participant (peers' signals need host memory:
 * KVPUB_ERR_UNSUPPORTED), device ordinal < 64, and one static context per GPU
 * at a time -- a second call while one is alive returns KVPUB_ERR_IN_USE.
 * Every static context on a GPU uses that GPU's one array, so calls on it that
 * overlap (another thread creating a static context the moment this one is
 * destroyed, while kernels of the old one still run on another stream) race;
 * kvpub_destroy synchronizes the device first.  Not during stream capture of
 * `stream` (KVPUB_ERR_CAPTURING).  kvpub_graph_create on such a context
 * captures on a temporary stream (creating the graph allocates, as always). */
KVPUB_API kvpub_status kvpub_create_static(const kvpub_config *cfg, void *const *main_bases,
                                           void *const *idx_bases, kvpub_stream_t stream, kvpub_ctx **out);

/* Quantize num_tokens tokens' final rows and write them into every replica's
 * layer `layer`, asynchronously on `stream`.
 *   latent:  bf16 [T, 512], row stride latent_row_stride elements
 *   rope:    bf16 [T, 64],  row stride rope_row_stride elements
 *   indexer: bf16 [T, 128], row stride indexer_row_stride elements
 *   slot_mapping: int64 [T] device array (-1 = padded token)
 * Inputs are device pointers, 16-byte aligned, with row strides that are
 * multiples of 8 elements, at least the row width and at most 2^31 - 1
 * elements; slot_mapping is 8-byte aligned.  Valid slots within one call must be distinct and inputs finite.
 * num_tokens == 0 returns KVPUB_OK and launches nothing.  No allocation and no
 * synchronization: safe under stream capture.  Inputs must stay alive until
 * the stream work completes. */
KVPUB_API kvpub_status kvpub_store(kvpub_ctx *ctx, uint32_t layer, int64_t num_tokens,
                         const void *latent, int64_t latent_row_stride,
                         const void *rope, int64_t rope_row_stride,
                         const void *indexer, int64_t indexer_row_stride,
                         const int64_t *slot_mapping, kvpub_stream_t stream);

/* Dequantizing gather from replica `replica`, layer `layer`, asynchronously on
 * `stream` (the reader side of the cache this library writes).  For token t
 * with slot s = slot_mapping[t]:
 *   latent_out[t][k]  = bf16(RN32(value(code_k) * scale_(k/128))) for k < 512,
 *   rope_out[t][k]    = the stored RoPE bits, k < 64,
 *   indexer_out[t][k] = bf16(RN32(value(icode_k) * iscale)), k < 128,
 * where value() is the OCP E4M3 value of a stored code, the product is rounded
 * once to binary32 and then to bf16 (nearest, ties to even).  s == -1 or s
 * outside [0, num_pages*64) gives all-zero output rows; the out-of-range ones
 * are added to the context's invalid-slot counter (kvpub_error_read).
 *   latent_out:  bf16 [T, 512], row stride latent_row_stride elements
 *   rope_out:    bf16 [T, 64],  row stride rope_row_stride elements
 *   indexer_out: bf16 [T, 128], row stride indexer_row_stride elements
 *   slot_mapping: int64 [T] device array
 * Outputs are caller-owned device buffers, 16-byte aligned, row strides
 * multiples of 8 elements, at least the row width and at most 2^31 - 1
 * elements; slot_mapping is 8-byte aligned.  Only the output rows are written; the cache is only read.  A
 * context poisoned by a fence timeout still gathers (reading publishes
 * nothing).  num_tokens == 0 returns KVPUB_OK and launches nothing.  No
 * allocation and no synchronization: safe under stream capture.  Argument
 * problems (replica >= R, layer >= L, bad pointers or strides, or a context
 * with no backed pages -- see kvpub_vmm_grow) return KVPUB_ERR_INVALID_ARG
 * before anything is launched. */
KVPUB_API kvpub_status kvpub_gather(kvpub_ctx *ctx, uint32_t replica, uint32_t layer, int64_t num_tokens,
                                    const int64_t *slot_mapping, void *latent_out, int64_t latent_row_stride,
                                    void *rope_out, int64_t rope_row_stride, void *indexer_out,
                                    int64_t indexer_row_stride, kvpub_stream_t stream);

/* Replica storage at stable virtual addresses, on cfg->device (vLLM PR
 * #52863, Relationship to existing work: the replicated cache builds on a
 * cache kept at a stable virtual address so that it can grow in place).
 * Reserves address space for cfg->num_replicas replicas of cfg->num_layers
 * layers of up to max_pages pages each (one Main-KV and one Indexer-K range
 * per replica) and backs the first cfg->num_pages pages of every layer with
 * device memory (contents undefined until written).  On success the layer
 * strides in *cfg are set to the reserved per-layer spans (max_pages * page
 * stride rounded up to the allocation granularity, plus one granule; every
 * layer is a reservation of its own), main_bases[r] /
 * idx_bases[r] receive the replicas' base addresses, and *cfg is ready for
 * kvpub_create.  The bases never change for the object's lifetime.
 * All-or-nothing: on failure nothing stays reserved or mapped and *out is
 * NULL.  Only backed pages may be accessed: a context over this storage must
 * not claim more pages than are backed (kvpub_vmm_grow keeps them equal). */
KVPUB_API kvpub_status kvpub_vmm_create(kvpub_config *cfg, uint64_t max_pages, void **main_bases,
                                        void **idx_bases, kvpub_vmm **out);

/* Back every layer of every replica up to num_pages pages (num_pages <=
 * max_pages; never shrinks).  Bytes already written and all addresses are
 * unchanged.  If ctx is not NULL it must be a context over exactly this
 * storage (same bases and strides, else KVPUB_ERR_INVALID_ARG); its capacity
 * becomes the backed page count, for launches made after the call and for
 * graphs captured before it alike (the kernels read the capacity from the
 * context's device words when they run).  Host-side, not
 * for use during stream capture or concurrently with launches on ctx from
 * another thread.  On failure the page count stays as it was, except in the
 * unlikely case that a layer's old backing could not be restored either:
 * then the storage reports 0 pages, ctx (if given) accepts no slot any more
 * (stores count every slot as invalid, new gathers are refused and gathers
 * captured earlier write zero rows), and
 * KVPUB_ERR_HIP is returned.  Growing copies each layer's backed bytes
 * once (the addresses stay, the physical memory behind them is replaced). */
KVPUB_API kvpub_status kvpub_vmm_grow(kvpub_vmm *vmm, uint64_t num_pages, kvpub_ctx *ctx);

/* Pages per layer currently backed. */
KVPUB_API kvpub_status kvpub_vmm_pages(kvpub_vmm *vmm, uint64_t *num_pages);

/* Synchronize the device, then unmap and release everything.  Contexts over
 * this storage must be destroyed first. */
KVPUB_API kvpub_status kvpub_vmm_destroy(kvpub_vmm *vmm);

/* One fence on `lane`, asynchronously on `stream`: a single one-wavefront
 * kernel that adds 1 to the lane's device epoch with a system-scope
 * read-modify-write that releases every write made on this GPU before the
 * fence.  With one participant it then acquire-loads the epoch until it holds
 * the new value (KVPUB_CONFIG_FENCE_RELEASE_ONLY: the release RMW alone).
 * With peers the RMW also acquires, then the kernel publishes the new value as
 * this participant's signal and acquire-waits until every other participant's
 * signal has reached it.  The expected value is never a kernel argument, so a captured
 * fence advances the epoch on every replay.  If the wait exceeds
 * fence_timeout_ns the kernel records KVPUB_FLAG_FENCE_TIMEOUT |
 * KVPUB_FLAG_POISONED and returns; from then on stores and fences of this
 * context write nothing (fail-closed; with one participant the wait can only
 * time out if the epoch was moved back, by kvpub_fence_host_epoch on the same
 * lane).
 * No allocation and no synchronization: safe under stream capture. */
KVPUB_API kvpub_status kvpub_fence(kvpub_ctx *ctx, uint32_t lane, kvpub_stream_t stream);

/* The pages' earlier fence, kept for comparison: two launches per fence and an
 * epoch held on the host (vLLM PR #54030 "[Perf][PCP] Fuse direct-KV
 * publication fence", Motivation and commit list: the fence used to be a
 * signal launch and a wait launch, and because the epoch lived on the host a
 * captured graph could not advance it on replay).  The context keeps a host
 * counter per lane; each call takes e = counter + 1 and enqueues on `stream` a
 * kernel that release-stores e into the lane's device epoch at system scope,
 * then a kernel that acquire-loads it until it is >= e (bounded by
 * fence_timeout_ns; a timeout sets KVPUB_FLAG_FENCE_TIMEOUT |
 * KVPUB_FLAG_POISONED), and the counter becomes e.  Under stream capture the
 * counter moves once, at capture: every replay publishes the captured values
 * again, so the device epoch stops advancing -- the failure the single-launch
 * kvpub_fence removes.  kvpub_epoch_read shows the published value.  Do not
 * mix it with kvpub_fence on one lane (the two count independently).  One
 * participant only (KVPUB_ERR_UNSUPPORTED otherwise).  No allocation and no
 * synchronization; the counter is not thread-safe. */
KVPUB_API kvpub_status kvpub_fence_host_epoch(kvpub_ctx *ctx, uint32_t lane, kvpub_stream_t stream);

/* One layer of a captured sequence. */
typedef struct {
    const void *latent;
    const void *rope;
    const void *indexer;
    int64_t latent_row_stride;
    int64_t rope_row_stride;
    int64_t indexer_row_stride;
    const int64_t *slot_mapping;
    int64_t num_tokens;
    uint32_t layer;
    uint32_t reserved; /* must be 0 */
} kvpub_layer_io;

/* Capture n x (kvpub_store(io[i]), kvpub_fence(lane)) once into a hipGraph
 * (on a private stream) and instantiate it.  The graph binds the pointers in
 * io: to publish new data, rewrite those buffers before a replay.  They must
 * outlive the graph.  Argument checks as for kvpub_store, done for every layer
 * before capture begins.  Captures on the context's private stream: create
 * graphs of one context from one thread at a time. */
KVPUB_API kvpub_status kvpub_graph_create(kvpub_ctx *ctx, const kvpub_layer_io *io, uint32_t n,
                                uint32_t lane, kvpub_graph **out);

/* Launch the instantiated graph once on `stream` (asynchronous). */
KVPUB_API kvpub_status kvpub_graph_replay(kvpub_graph *graph, kvpub_stream_t stream);

/* Release a graph (waits for nothing; do not destroy while a replay may run). */
KVPUB_API kvpub_status kvpub_graph_destroy(kvpub_graph *graph);

/* Synchronize the device, then read the lane's epoch (number of fences that
 * ran on it).  KVPUB_ERR_CAPTURING if a capture is active on the calling thread. */
KVPUB_API kvpub_status kvpub_epoch_read(kvpub_ctx *ctx, uint32_t lane, uint64_t *out);

/* Synchronize the device, then read the invalid-slot count and the sticky
 * flags (either output may be NULL).  clear != 0 resets the invalid-slot
 * count; the flags stay set for the context's lifetime.  Returns
 * KVPUB_ERR_FENCE_TIMEOUT if KVPUB_FLAG_FENCE_TIMEOUT is set, else KVPUB_OK. */
KVPUB_API kvpub_status kvpub_error_read(kvpub_ctx *ctx, uint64_t *invalid_slots, uint32_t *flags,
                              int clear);

/* Host address of participant p's signal word on `lane` (1 <= p <
 * num_participants).  It lives in host-coherent memory that the fence kernel
 * reads with system-scope acquire loads; a host thread stands in for peer p by
 * storing the epoch values it publishes.  Only meaningful with
 * num_participants > 1 (one GPU has no real peers). */
KVPUB_API kvpub_status kvpub_participant_signal(kvpub_ctx *ctx, uint32_t lane, uint32_t p,
                                      volatile uint64_t **out);

/* Synchronize the device and release the context's resources.  NULL is OK.
 * The replica buffers are the caller's and are left untouched. */
KVPUB_API kvpub_status kvpub_destroy(kvpub_ctx *ctx);

/* Static description of a status code. */
KVPUB_API const char *kvpub_strerror(kvpub_status status);

/* KVPUB_ABI_VERSION of the loaded library. */
KVPUB_API uint32_t kvpub_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVPUB_H */
