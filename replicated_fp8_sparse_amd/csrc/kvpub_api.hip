// C-ABI host side of libkvpub: argument checks, context lifetime, launches,
// graph capture.  Nothing here allocates or synchronizes on the store / fence
// path; creation is all-or-nothing (vLLM PR #54030 "[Perf][PCP] Fuse
// direct-KV publication fence", commit list: opt-in allocation either fully
// succeeds at startup or leaves nothing behind; teardown drops every view).
#include <algorithm>
#include <cstddef>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "kvpub.h"
#include "kvpub_internal.h"

using kvpub::FenceParams;
using kvpub::StoreParams;

struct kvpub_ctx {
    kvpub_config cfg;
    uint8_t* main_base[KVPUB_MAX_REPLICAS];
    uint8_t* idx_base[KVPUB_MAX_REPLICAS];
    uint8_t* words;            // device: status, invalid count, epochs
    uint64_t* host_signals;    // P > 1: host-coherent signals [lanes][P] (kSignalStride apart)
    uint64_t* host_signals_dev;
    uint64_t timeout_ticks;
    hipStream_t capture_stream;
    uint64_t host_epoch[KVPUB_MAX_LANES];   // kvpub_fence_host_epoch: the epoch each lane last published
    bool is_static;            // kvpub_create_static: words in the static array, this struct in static storage
};

struct kvpub_graph {
    kvpub_ctx* ctx;
    hipGraph_t graph;
    hipGraphExec_t exec;
};

namespace {

constexpr uint64_t kDefaultTimeoutNs = 5000000000ull;

size_t words_bytes(const kvpub_config& c) {
    return kvpub::kEpochOffset + (size_t)c.num_lanes * kvpub::kLine;
}

uint64_t* epoch_ptr(kvpub_ctx* c, uint32_t lane) {
    return reinterpret_cast<uint64_t*>(c->words + kvpub::kEpochOffset + (size_t)lane * kvpub::kLine);
}

// Participant signals exist only with peers; alone, the epoch is the barrier.
uint64_t* signals_dev_ptr(kvpub_ctx* c, uint32_t lane) {
    const uint32_t P = c->cfg.num_participants;
    if (P == 1) return nullptr;
    return c->host_signals_dev + (size_t)lane * P * kvpub::kSignalStride;
}

// Sets the context's device current for the lifetime of the guard.
struct DeviceGuard {
    int prev = -1;
    bool ok = true;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) { ok = false; prev = -1; return; }
        if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

// Test hook: KVPUB_TEST_FAIL_ALLOC_AT=k makes the k-th allocation of a
// kvpub_create call fail (k >= 1), to exercise the all-or-nothing cleanup.
struct AllocCounter {
    int fail_at = 0;
    int n = 0;
    AllocCounter() {
        const char* s = std::getenv("KVPUB_TEST_FAIL_ALLOC_AT");
        fail_at = s ? std::atoi(s) : 0;
    }
    bool next_fails() { return ++n == fail_at; }
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

kvpub_status map_hip(hipError_t e) {
    switch (e) {
        case hipSuccess: return KVPUB_OK;
        case hipErrorOutOfMemory: return KVPUB_ERR_OUT_OF_MEMORY;
        case hipErrorStreamCaptureUnsupported:
        case hipErrorStreamCaptureInvalidated:
        case hipErrorStreamCaptureImplicit:
        case hipErrorCapturedEvent:
        case hipErrorStreamCaptureWrongThread:
            return KVPUB_ERR_CAPTURING;
        default: return KVPUB_ERR_HIP;
    }
}

kvpub_status check_config(const kvpub_config* c) {
    if (!c || c->struct_size != sizeof(kvpub_config)) return KVPUB_ERR_INVALID_ARG;
    if (c->num_replicas < 1 || c->num_replicas > KVPUB_MAX_REPLICAS) return KVPUB_ERR_INVALID_ARG;
    if (c->num_layers < 1 || c->block_size != KVPUB_SLOTS_PER_PAGE) return KVPUB_ERR_INVALID_ARG;
    if (c->num_pages < 1 || c->num_pages > (1ull << 40)) return KVPUB_ERR_INVALID_ARG;
    if (c->main_page_stride < KVPUB_MAIN_PAGE_BYTES || c->main_page_stride % 16) return KVPUB_ERR_INVALID_ARG;
    if (c->idx_page_stride < KVPUB_IDX_PAGE_BYTES || c->idx_page_stride % 16) return KVPUB_ERR_INVALID_ARG;
    if (c->num_layers > 1) {
        if (c->main_layer_stride % 16 || c->idx_layer_stride % 16) return KVPUB_ERR_INVALID_ARG;
        if (c->main_layer_stride / c->main_page_stride < c->num_pages) return KVPUB_ERR_INVALID_ARG;
        if (c->idx_layer_stride / c->idx_page_stride < c->num_pages) return KVPUB_ERR_INVALID_ARG;
    }
    if (c->num_lanes < 1 || c->num_lanes > KVPUB_MAX_LANES) return KVPUB_ERR_INVALID_ARG;
    if (c->num_participants < 1 || c->num_participants > KVPUB_MAX_PARTICIPANTS) return KVPUB_ERR_INVALID_ARG;
    if (c->device < 0 || (c->flags & ~KVPUB_CONFIG_FENCE_RELEASE_ONLY) != 0) return KVPUB_ERR_INVALID_ARG;
    return KVPUB_OK;
}

kvpub_status check_store(const kvpub_ctx* ctx, uint32_t layer, int64_t T, const void* latent,
                         int64_t ls, const void* rope, int64_t rs, const void* indexer,
                         int64_t is, const int64_t* slots) {
    if (!ctx) return KVPUB_ERR_INVALID_ARG;
    if (layer >= ctx->cfg.num_layers) return KVPUB_ERR_INVALID_ARG;
    if (T < 0 || T > KVPUB_MAX_TOKENS) return KVPUB_ERR_INVALID_ARG;
    if (T == 0) return KVPUB_OK;
    if (!latent || !rope || !indexer || !slots) return KVPUB_ERR_INVALID_ARG;
    if (!aligned(latent, 16) || !aligned(rope, 16) || !aligned(indexer, 16) || !aligned(slots, 8))
        return KVPUB_ERR_INVALID_ARG;
    if (ls < (int64_t)KVPUB_LATENT_DIM || ls % 8 || ls > INT32_MAX) return KVPUB_ERR_INVALID_ARG;
    if (rs < (int64_t)KVPUB_ROPE_DIM || rs % 8 || rs > INT32_MAX) return KVPUB_ERR_INVALID_ARG;
    if (is < (int64_t)KVPUB_INDEXER_DIM || is % 8 || is > INT32_MAX) return KVPUB_ERR_INVALID_ARG;
    return KVPUB_OK;
}

StoreParams store_params(kvpub_ctx* ctx, uint32_t layer, int64_t T, const void* latent, int64_t ls,
                         const void* rope, int64_t rs, const void* indexer, int64_t is,
                         const int64_t* slots) {
    StoreParams p;
    std::memset(&p, 0, sizeof p);
    p.latent = static_cast<const uint16_t*>(latent);
    p.rope = static_cast<const uint16_t*>(rope);
    p.indexer = static_cast<const uint16_t*>(indexer);
    p.latent_stride = ls;
    p.rope_stride = rs;
    p.indexer_stride = is;
    p.slots = slots;
    p.num_tokens = T;
    p.main_page_stride = ctx->cfg.main_page_stride;
    p.idx_page_stride = ctx->cfg.idx_page_stride;
    for (uint32_t r = 0; r < ctx->cfg.num_replicas; ++r) {
        p.main_base[r] = ctx->main_base[r] + (uint64_t)layer * ctx->cfg.main_layer_stride;
        p.idx_base[r] = ctx->idx_base[r] + (uint64_t)layer * ctx->cfg.idx_layer_stride;
    }
    p.invalid_count = reinterpret_cast<unsigned long long*>(ctx->words + kvpub::kInvalidOffset);
    p.head = reinterpret_cast<const kvpub::CtxHead*>(ctx->words + kvpub::kStatusOffset);
    // The write-through store path takes 32-bit offsets within a replica's
    // layer span: every page the layer may ever hold (a VMM storage's capacity
    // can grow under a captured graph, so the span, not the current page count).
    // The layer stride is that span for one layer too: kvpub_vmm_create sets it
    // to the reserved range whatever the layer count.  Stores never go beyond
    // the capacity in the context's device words, so a span larger than the
    // caller's buffer only loosens this second range check.
    const uint64_t main_region = std::max(ctx->cfg.num_pages * ctx->cfg.main_page_stride, ctx->cfg.main_layer_stride);
    const uint64_t idx_region = std::max(ctx->cfg.num_pages * ctx->cfg.idx_page_stride, ctx->cfg.idx_layer_stride);
    if (main_region <= UINT32_MAX && idx_region <= UINT32_MAX) {
        p.main_region = (uint32_t)main_region;
        p.idx_region = (uint32_t)idx_region;
    }
    return p;
}

FenceParams fence_params(kvpub_ctx* ctx, uint32_t lane) {
    FenceParams f;
    f.epoch = epoch_ptr(ctx, lane);
    f.signals = signals_dev_ptr(ctx, lane);
    f.num_participants = ctx->cfg.num_participants;
    f.self = 0;
    f.status = reinterpret_cast<uint32_t*>(ctx->words + kvpub::kStatusOffset);
    f.timeout_ticks = ctx->timeout_ticks;
    f.acquire_wait = (ctx->cfg.flags & KVPUB_CONFIG_FENCE_RELEASE_ONLY) ? 0u : 1u;
    return f;
}

void release_static(kvpub_ctx* c);

void release(kvpub_ctx* c) {
    if (!c) return;
    if (c->is_static) { release_static(c); return; }
    if (c->capture_stream) (void)hipStreamDestroy(c->capture_stream);
    if (c->host_signals) (void)hipHostFree(c->host_signals);
    if (c->words) (void)hipFree(c->words);
    delete c;
}

// KVPUB_LOG=1: one line on stderr for each context created or destroyed (never
// on the store / fence / gather path).
bool log_enabled() {
    static const bool on = [] {
        const char* s = std::getenv("KVPUB_LOG");
        return s != nullptr && s[0] == '1';
    }();
    return on;
}

void log_create(const char* what, const kvpub_config* cfg, kvpub_status st, const kvpub_ctx* c) {
    if (!log_enabled()) return;
    if (cfg && cfg->struct_size == sizeof(kvpub_config))
        std::fprintf(stderr, "kvpub: %s R=%u L=%u pages=%llu lanes=%u participants=%u device=%d flags=%u -> %s (ctx %p)\n",
                     what, cfg->num_replicas, cfg->num_layers, (unsigned long long)cfg->num_pages, cfg->num_lanes,
                     cfg->num_participants, cfg->device, cfg->flags, kvpub_strerror(st), (const void*)c);
    else
        std::fprintf(stderr, "kvpub: %s (no valid config) -> %s\n", what, kvpub_strerror(st));
}

kvpub_status sync_device() {
    return map_hip(hipDeviceSynchronize());
}

// Timeout in wall-clock (s_memrealtime) ticks for a context on `device`.
hipError_t timeout_ticks_for(const kvpub_config* cfg, uint64_t* out) {
    int khz = 0;
    const hipError_t e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, cfg->device);
    if (e != hipSuccess) return e;
    if (khz <= 0) return hipErrorInvalidValue;
    const uint64_t ns = cfg->fence_timeout_ns ? cfg->fence_timeout_ns : kDefaultTimeoutNs;
    *out = (uint64_t)((double)ns * (double)khz / 1.0e6);
    if (*out == 0) *out = 1;
    return hipSuccess;
}

// ---- contexts that allocate nothing (kvpub_create_static) -------------------
//
// Their device words live in `scratch`, a file-scope device array of fixed
// size: the status line, the invalid-slot counter and the epochs of the
// largest lane count.  Each GPU holds its own copy for the life of the
// process.  In host code `scratch` names a host-side stand-in, not the device
// memory: the device address comes from hipGetSymbolAddress, resolved once per
// device with that device current, and only that address is used.  The host
// part of the context is one static struct per device.  One static context
// per device at a time: its words are that device's array.
constexpr size_t kStaticWordsBytes = kvpub::kEpochOffset + (size_t)KVPUB_MAX_LANES * kvpub::kLine;  // 8448
constexpr int kMaxStaticDevices = 64;

struct StaticSlot {
    uint8_t* words;   // device address of this device's `scratch`
    bool in_use;
    kvpub_ctx ctx;
};
StaticSlot g_static[kMaxStaticDevices];
std::mutex g_static_mu;

void release_static(kvpub_ctx* c) {
    std::lock_guard<std::mutex> lock(g_static_mu);
    g_static[c->cfg.device].in_use = false;
}

}  // namespace

static __device__ __align__(256) uint8_t scratch[kStaticWordsBytes];

namespace {

// Clears a static context's words (status, counter, every lane's epoch) and
// writes the capacity: one block, 16-byte vector stores.
__global__ __launch_bounds__(256) void init_words_kernel(uint8_t* words, uint32_t bytes, int64_t capacity) {
    for (uint32_t i = threadIdx.x * 16u; i < bytes; i += blockDim.x * 16u) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (i == 0) {   // the CtxHead line starts with {status, reserved, capacity}
            v.z = (uint32_t)((uint64_t)capacity & 0xFFFFFFFFu);
            v.w = (uint32_t)((uint64_t)capacity >> 32);
        }
        *reinterpret_cast<uint4*>(words + i) = v;
    }
}

// The device address of this device's `scratch` (the device must be current).
hipError_t static_words(int device, uint8_t** out) {
    StaticSlot& slot = g_static[device];
    if (!slot.words) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        slot.words = static_cast<uint8_t*>(ptr);
    }
    *out = slot.words;
    return hipSuccess;
}

}  // namespace

namespace kvpub {

bool ctx_uses_storage(const kvpub_ctx* ctx, uint32_t replicas, uint8_t* const* main_bases,
                      uint8_t* const* idx_bases, uint64_t main_layer_stride, uint64_t idx_layer_stride,
                      uint64_t main_page_stride, uint64_t idx_page_stride) {
    if (ctx->cfg.num_replicas != replicas) return false;
    if (ctx->cfg.main_layer_stride != main_layer_stride || ctx->cfg.idx_layer_stride != idx_layer_stride)
        return false;
    if (ctx->cfg.main_page_stride != main_page_stride || ctx->cfg.idx_page_stride != idx_page_stride)
        return false;
    for (uint32_t r = 0; r < replicas; ++r)
        if (ctx->main_base[r] != main_bases[r] || ctx->idx_base[r] != idx_bases[r]) return false;
    return true;
}

hipError_t ctx_set_pages(kvpub_ctx* ctx, uint64_t num_pages) {
    ctx->cfg.num_pages = num_pages;
    const int64_t capacity = (int64_t)(num_pages * KVPUB_SLOTS_PER_PAGE);
    DeviceGuard guard(ctx->cfg.device);
    if (!guard.ok) return hipErrorInvalidDevice;
    return hipMemcpy(ctx->words + kvpub::kStatusOffset + offsetof(CtxHead, capacity), &capacity, sizeof capacity,
                     hipMemcpyHostToDevice);
}

}  // namespace kvpub

extern "C" {

KVPUB_API void kvpub_config_init(kvpub_config* cfg, uint32_t num_replicas, uint32_t num_layers,
                                 uint64_t num_pages) {
    if (!cfg) return;
    std::memset(cfg, 0, sizeof *cfg);
    cfg->struct_size = sizeof(kvpub_config);
    cfg->num_replicas = num_replicas;
    cfg->num_layers = num_layers;
    cfg->block_size = KVPUB_SLOTS_PER_PAGE;
    cfg->num_pages = num_pages;
    cfg->main_page_stride = KVPUB_MAIN_PAGE_BYTES;
    cfg->main_layer_stride = num_pages * KVPUB_MAIN_PAGE_BYTES;
    cfg->idx_page_stride = KVPUB_IDX_PAGE_BYTES;
    cfg->idx_layer_stride = num_pages * KVPUB_IDX_PAGE_BYTES;
    cfg->num_lanes = 1;
    cfg->num_participants = 1;
    cfg->fence_timeout_ns = 0;
    cfg->device = 0;
    cfg->flags = 0;
}

static kvpub_status create_ctx(const kvpub_config* cfg, void* const* main_bases, void* const* idx_bases,
                               kvpub_ctx** out) {
    if (!out) return KVPUB_ERR_INVALID_ARG;
    *out = nullptr;
    kvpub_status st = check_config(cfg);
    if (st != KVPUB_OK) return st;
    if (!main_bases || !idx_bases) return KVPUB_ERR_INVALID_ARG;
    for (uint32_t r = 0; r < cfg->num_replicas; ++r) {
        if (!main_bases[r] || !idx_bases[r]) return KVPUB_ERR_INVALID_ARG;
        if (!aligned(main_bases[r], 16) || !aligned(idx_bases[r], 16)) return KVPUB_ERR_INVALID_ARG;
    }

    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) return KVPUB_ERR_HIP;
    if (cfg->device >= ndev) return KVPUB_ERR_INVALID_ARG;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, cfg->device) != hipSuccess) return KVPUB_ERR_HIP;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return KVPUB_ERR_UNSUPPORTED;

    DeviceGuard guard(cfg->device);
    if (!guard.ok) return KVPUB_ERR_HIP;

    kvpub_ctx* c = new (std::nothrow) kvpub_ctx;
    if (!c) return KVPUB_ERR_OUT_OF_MEMORY;
    std::memset(c, 0, sizeof *c);
    c->cfg = *cfg;
    for (uint32_t r = 0; r < cfg->num_replicas; ++r) {
        c->main_base[r] = static_cast<uint8_t*>(main_bases[r]);
        c->idx_base[r] = static_cast<uint8_t*>(idx_bases[r]);
    }

    AllocCounter alloc;
    const size_t wb = words_bytes(*cfg);
    hipError_t e = alloc.next_fails() ? hipErrorOutOfMemory : hipMalloc(&c->words, wb);
    if (e != hipSuccess) { c->words = nullptr; release(c); return map_hip(e); }
    e = hipMemset(c->words, 0, wb);
    if (e != hipSuccess) { release(c); return map_hip(e); }
    const int64_t capacity = (int64_t)(cfg->num_pages * KVPUB_SLOTS_PER_PAGE);
    e = hipMemcpy(c->words + kvpub::kStatusOffset + offsetof(kvpub::CtxHead, capacity), &capacity,
                  sizeof capacity, hipMemcpyHostToDevice);
    if (e != hipSuccess) { release(c); return map_hip(e); }

    if (cfg->num_participants > 1) {
        const size_t hb = (size_t)cfg->num_lanes * cfg->num_participants * kvpub::kLine;
        e = alloc.next_fails() ? hipErrorOutOfMemory
                               : hipHostMalloc(reinterpret_cast<void**>(&c->host_signals), hb,
                                               hipHostMallocCoherent | hipHostMallocMapped);
        if (e != hipSuccess) { c->host_signals = nullptr; release(c); return map_hip(e); }
        std::memset(c->host_signals, 0, hb);
        e = hipHostGetDevicePointer(reinterpret_cast<void**>(&c->host_signals_dev), c->host_signals, 0);
        if (e != hipSuccess) { release(c); return map_hip(e); }
    }

    e = alloc.next_fails() ? hipErrorOutOfMemory
                           : hipStreamCreateWithFlags(&c->capture_stream, hipStreamNonBlocking);
    if (e != hipSuccess) { c->capture_stream = nullptr; release(c); return map_hip(e); }

    if (timeout_ticks_for(cfg, &c->timeout_ticks) != hipSuccess) { release(c); return KVPUB_ERR_HIP; }

    *out = c;
    return KVPUB_OK;
}

KVPUB_API kvpub_status kvpub_create(const kvpub_config* cfg, void* const* main_bases,
                                   void* const* idx_bases, kvpub_ctx** out) {
    const kvpub_status st = create_ctx(cfg, main_bases, idx_bases, out);
    log_create("create", cfg, st, out ? *out : nullptr);
    return st;
}

static kvpub_status create_static_ctx(const kvpub_config* cfg, void* const* main_bases, void* const* idx_bases,
                                      kvpub_stream_t stream, kvpub_ctx** out) {
    if (!out) return KVPUB_ERR_INVALID_ARG;
    *out = nullptr;
    kvpub_status st = check_config(cfg);
    if (st != KVPUB_OK) return st;
    if (!main_bases || !idx_bases) return KVPUB_ERR_INVALID_ARG;
    for (uint32_t r = 0; r < cfg->num_replicas; ++r) {
        if (!main_bases[r] || !idx_bases[r]) return KVPUB_ERR_INVALID_ARG;
        if (!aligned(main_bases[r], 16) || !aligned(idx_bases[r], 16)) return KVPUB_ERR_INVALID_ARG;
    }
    // host-driven peers' signals would need host memory of their own
    if (cfg->num_participants != 1) return KVPUB_ERR_UNSUPPORTED;
    if (kvpub::kEpochOffset + (size_t)cfg->num_lanes * kvpub::kLine > kStaticWordsBytes) return KVPUB_ERR_INVALID_ARG;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) return KVPUB_ERR_HIP;
    if (cfg->device >= ndev) return KVPUB_ERR_INVALID_ARG;
    if (cfg->device >= kMaxStaticDevices) return KVPUB_ERR_UNSUPPORTED;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, cfg->device) != hipSuccess) return KVPUB_ERR_HIP;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return KVPUB_ERR_UNSUPPORTED;

    DeviceGuard guard(cfg->device);
    if (!guard.ok) return KVPUB_ERR_HIP;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cap) != hipSuccess) return KVPUB_ERR_HIP;
    if (cap != hipStreamCaptureStatusNone) return KVPUB_ERR_CAPTURING;
    uint64_t ticks = 0;
    if (timeout_ticks_for(cfg, &ticks) != hipSuccess) return KVPUB_ERR_HIP;

    std::lock_guard<std::mutex> lock(g_static_mu);
    StaticSlot& slot = g_static[cfg->device];
    if (slot.in_use) return KVPUB_ERR_IN_USE;
    uint8_t* words = nullptr;
    hipError_t e = static_words(cfg->device, &words);
    if (e != hipSuccess) return map_hip(e);

    (void)hipGetLastError();
    init_words_kernel<<<dim3(1), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
        words, (uint32_t)kStaticWordsBytes, (int64_t)(cfg->num_pages * KVPUB_SLOTS_PER_PAGE));
    e = hipGetLastError();
    if (e != hipSuccess) return map_hip(e);

    kvpub_ctx* c = &slot.ctx;
    std::memset(c, 0, sizeof *c);
    c->cfg = *cfg;
    for (uint32_t r = 0; r < cfg->num_replicas; ++r) {
        c->main_base[r] = static_cast<uint8_t*>(main_bases[r]);
        c->idx_base[r] = static_cast<uint8_t*>(idx_bases[r]);
    }
    c->words = words;
    c->timeout_ticks = ticks;
    c->is_static = true;
    slot.in_use = true;
    *out = c;
    return KVPUB_OK;
}

KVPUB_API kvpub_status kvpub_create_static(const kvpub_config* cfg, void* const* main_bases,
                                          void* const* idx_bases, kvpub_stream_t stream, kvpub_ctx** out) {
    const kvpub_status st = create_static_ctx(cfg, main_bases, idx_bases, stream, out);
    log_create("create_static", cfg, st, out ? *out : nullptr);
    return st;
}

KVPUB_API kvpub_status kvpub_store(kvpub_ctx* ctx, uint32_t layer, int64_t num_tokens,
                                  const void* latent, int64_t latent_row_stride, const void* rope,
                                  int64_t rope_row_stride, const void* indexer,
                                  int64_t indexer_row_stride, const int64_t* slot_mapping,
                                  kvpub_stream_t stream) {
    kvpub_status st = check_store(ctx, layer, num_tokens, latent, latent_row_stride, rope,
                                  rope_row_stride, indexer, indexer_row_stride, slot_mapping);
    if (st != KVPUB_OK || num_tokens == 0) return st;
    DeviceGuard guard(ctx->cfg.device);
    if (!guard.ok) return KVPUB_ERR_HIP;
    const StoreParams p = store_params(ctx, layer, num_tokens, latent, latent_row_stride, rope,
                                       rope_row_stride, indexer, indexer_row_stride, slot_mapping);
    return map_hip(kvpub::launch_store(p, ctx->cfg.num_replicas, static_cast<hipStream_t>(stream)));
}

KVPUB_API kvpub_status kvpub_gather(kvpub_ctx* ctx, uint32_t replica, uint32_t layer, int64_t num_tokens,
                                    const int64_t* slot_mapping, void* latent_out, int64_t latent_row_stride,
                                    void* rope_out, int64_t rope_row_stride, void* indexer_out,
                                    int64_t indexer_row_stride, kvpub_stream_t stream) {
    if (!ctx || replica >= ctx->cfg.num_replicas) return KVPUB_ERR_INVALID_ARG;
    // the kernel reads slot 0's bytes for every padded or out-of-range slot, so
    // at least one page must be backed (a VMM storage that lost a layer has none)
    if (ctx->cfg.num_pages == 0) return KVPUB_ERR_INVALID_ARG;
    // the outputs obey the same pointer, alignment and stride rules as the store's inputs
    kvpub_status st = check_store(ctx, layer, num_tokens, latent_out, latent_row_stride, rope_out,
                                  rope_row_stride, indexer_out, indexer_row_stride, slot_mapping);
    if (st != KVPUB_OK || num_tokens == 0) return st;
    DeviceGuard guard(ctx->cfg.device);
    if (!guard.ok) return KVPUB_ERR_HIP;
    kvpub::GatherParams g;
    std::memset(&g, 0, sizeof g);
    g.main_base = ctx->main_base[replica] + (uint64_t)layer * ctx->cfg.main_layer_stride;
    g.idx_base = ctx->idx_base[replica] + (uint64_t)layer * ctx->cfg.idx_layer_stride;
    g.main_page_stride = ctx->cfg.main_page_stride;
    g.idx_page_stride = ctx->cfg.idx_page_stride;
    g.head = reinterpret_cast<const kvpub::CtxHead*>(ctx->words + kvpub::kStatusOffset);
    g.slots = slot_mapping;
    g.num_tokens = num_tokens;
    g.latent = static_cast<uint16_t*>(latent_out);
    g.rope = static_cast<uint16_t*>(rope_out);
    g.indexer = static_cast<uint16_t*>(indexer_out);
    g.latent_stride = latent_row_stride;
    g.rope_stride = rope_row_stride;
    g.indexer_stride = indexer_row_stride;
    g.invalid_count = reinterpret_cast<unsigned long long*>(ctx->words + kvpub::kInvalidOffset);
    // every page the layer may ever hold (as for the store's buffer range):
    // 32-bit offsets if that span stays below 2^32 bytes
    const uint64_t main_span = std::max(ctx->cfg.num_pages * ctx->cfg.main_page_stride, ctx->cfg.main_layer_stride);
    const uint64_t idx_span = std::max(ctx->cfg.num_pages * ctx->cfg.idx_page_stride, ctx->cfg.idx_layer_stride);
    g.offsets32 = main_span <= UINT32_MAX && idx_span <= UINT32_MAX ? 1u : 0u;
    return map_hip(kvpub::launch_gather(g, static_cast<hipStream_t>(stream)));
}

KVPUB_API kvpub_status kvpub_fence(kvpub_ctx* ctx, uint32_t lane, kvpub_stream_t stream) {
    if (!ctx || lane >= ctx->cfg.num_lanes) return KVPUB_ERR_INVALID_ARG;
    DeviceGuard guard(ctx->cfg.device);
    if (!guard.ok) return KVPUB_ERR_HIP;
    return map_hip(kvpub::launch_fence(fence_params(ctx, lane), static_cast<hipStream_t>(stream)));
}

KVPUB_API kvpub_status kvpub_fence_host_epoch(kvpub_ctx* ctx, uint32_t lane, kvpub_stream_t stream) {
    if (!ctx || lane >= ctx->cfg.num_lanes) return KVPUB_ERR_INVALID_ARG;
    if (ctx->cfg.num_participants != 1) return KVPUB_ERR_UNSUPPORTED;
    DeviceGuard guard(ctx->cfg.device);
    if (!guard.ok) return KVPUB_ERR_HIP;
    const uint64_t e = ctx->host_epoch[lane] + 1;
    const hipError_t err = kvpub::launch_host_epoch_fence(fence_params(ctx, lane), e,
                                                          static_cast<hipStream_t>(stream));
    if (err == hipSuccess) ctx->host_epoch[lane] = e;
    return map_hip(err);
}

KVPUB_API kvpub_status kvpub_graph_create(kvpub_ctx* ctx, const kvpub_layer_io* io, uint32_t n,
                                         uint32_t lane, kvpub_graph** out) {
    if (!out) return KVPUB_ERR_INVALID_ARG;
    *out = nullptr;
    if (!ctx || !io || n == 0 || lane >= ctx->cfg.num_lanes) return KVPUB_ERR_INVALID_ARG;
    for (uint32_t i = 0; i < n; ++i) {
        if (io[i].reserved != 0) return KVPUB_ERR_INVALID_ARG;
        kvpub_status st = check_store(ctx, io[i].layer, io[i].num_tokens, io[i].latent,
                                      io[i].latent_row_stride, io[i].rope, io[i].rope_row_stride,
                                      io[i].indexer, io[i].indexer_row_stride, io[i].slot_mapping);
        if (st != KVPUB_OK) return st;
    }
    DeviceGuard guard(ctx->cfg.device);
    if (!guard.ok) return KVPUB_ERR_HIP;

    kvpub_graph* g = new (std::nothrow) kvpub_graph;
    if (!g) return KVPUB_ERR_OUT_OF_MEMORY;
    g->ctx = ctx;
    g->graph = nullptr;
    g->exec = nullptr;

    // A context from kvpub_create_static has no stream of its own: capture on
    // a temporary one.
    hipStream_t s = ctx->capture_stream;
    hipStream_t temp = nullptr;
    if (!s) {
        const hipError_t ce = hipStreamCreateWithFlags(&temp, hipStreamNonBlocking);
        if (ce != hipSuccess) { delete g; return map_hip(ce); }
        s = temp;
    }
    struct TempStream {
        hipStream_t s;
        ~TempStream() { if (s) (void)hipStreamDestroy(s); }
    } temp_guard{temp};
    hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) { delete g; return map_hip(e); }
    hipError_t launch_err = hipSuccess;
    for (uint32_t i = 0; i < n && launch_err == hipSuccess; ++i) {
        if (io[i].num_tokens > 0) {
            const StoreParams p = store_params(ctx, io[i].layer, io[i].num_tokens, io[i].latent,
                                               io[i].latent_row_stride, io[i].rope,
                                               io[i].rope_row_stride, io[i].indexer,
                                               io[i].indexer_row_stride, io[i].slot_mapping);
            launch_err = kvpub::launch_store(p, ctx->cfg.num_replicas, s);
        }
        if (launch_err == hipSuccess) launch_err = kvpub::launch_fence(fence_params(ctx, lane), s);
    }
    e = hipStreamEndCapture(s, &g->graph);
    if (launch_err != hipSuccess || e != hipSuccess) {
        if (g->graph) (void)hipGraphDestroy(g->graph);
        delete g;
        return map_hip(launch_err != hipSuccess ? launch_err : e);
    }
    e = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        (void)hipGraphDestroy(g->graph);
        delete g;
        return map_hip(e);
    }
    *out = g;
    return KVPUB_OK;
}

KVPUB_API kvpub_status kvpub_graph_replay(kvpub_graph* g, kvpub_stream_t stream) {
    if (!g || !g->exec) return KVPUB_ERR_INVALID_ARG;
    DeviceGuard guard(g->ctx->cfg.device);
    if (!guard.ok) return KVPUB_ERR_HIP;
    return map_hip(hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)));
}

KVPUB_API kvpub_status kvpub_graph_destroy(kvpub_graph* g) {
    if (!g) return KVPUB_OK;
    kvpub_status st = KVPUB_OK;
    {
        DeviceGuard guard(g->ctx->cfg.device);
        if (g->exec && hipGraphExecDestroy(g->exec) != hipSuccess) st = KVPUB_ERR_HIP;
        if (g->graph && hipGraphDestroy(g->graph) != hipSuccess) st = KVPUB_ERR_HIP;
    }
    delete g;
    return st;
}

KVPUB_API kvpub_status kvpub_epoch_read(kvpub_ctx* ctx, uint32_t lane, uint64_t* out) {
    if (!ctx || !out || lane >= ctx->cfg.num_lanes) return KVPUB_ERR_INVALID_ARG;
    DeviceGuard guard(ctx->cfg.device);
    if (!guard.ok) return KVPUB_ERR_HIP;
    kvpub_status st = sync_device();
    if (st != KVPUB_OK) return st;
    return map_hip(hipMemcpy(out, epoch_ptr(ctx, lane), sizeof(uint64_t), hipMemcpyDeviceToHost));
}

KVPUB_API kvpub_status kvpub_error_read(kvpub_ctx* ctx, uint64_t* invalid_slots, uint32_t* flags,
                                       int clear) {
    if (!ctx) return KVPUB_ERR_INVALID_ARG;
    DeviceGuard guard(ctx->cfg.device);
    if (!guard.ok) return KVPUB_ERR_HIP;
    kvpub_status st = sync_device();
    if (st != KVPUB_OK) return st;
    uint32_t status = 0;
    uint64_t invalid = 0;
    hipError_t e = hipMemcpy(&status, ctx->words + kvpub::kStatusOffset, sizeof status,
                             hipMemcpyDeviceToHost);
    if (e == hipSuccess)
        e = hipMemcpy(&invalid, ctx->words + kvpub::kInvalidOffset, sizeof invalid,
                      hipMemcpyDeviceToHost);
    if (e == hipSuccess && clear) e = hipMemset(ctx->words + kvpub::kInvalidOffset, 0, sizeof invalid);
    if (e == hipSuccess && clear) e = hipDeviceSynchronize();
    if (e != hipSuccess) return map_hip(e);
    if (invalid_slots) *invalid_slots = invalid;
    if (flags) *flags = status;
    return (status & kvpub::kStatusFenceTimeout) ? KVPUB_ERR_FENCE_TIMEOUT : KVPUB_OK;
}

KVPUB_API kvpub_status kvpub_participant_signal(kvpub_ctx* ctx, uint32_t lane, uint32_t p,
                                               volatile uint64_t** out) {
    if (!ctx || !out || lane >= ctx->cfg.num_lanes) return KVPUB_ERR_INVALID_ARG;
    if (ctx->cfg.num_participants < 2 || p < 1 || p >= ctx->cfg.num_participants)
        return KVPUB_ERR_INVALID_ARG;
    *out = ctx->host_signals + ((size_t)lane * ctx->cfg.num_participants + p) * kvpub::kSignalStride;
    return KVPUB_OK;
}

KVPUB_API kvpub_status kvpub_destroy(kvpub_ctx* ctx) {
    if (!ctx) return KVPUB_OK;
    const void* id = ctx;
    kvpub_status st;
    {
        DeviceGuard guard(ctx->cfg.device);
        st = sync_device();
        release(ctx);
    }
    if (log_enabled()) std::fprintf(stderr, "kvpub: destroy ctx %p -> %s\n", id, kvpub_strerror(st));
    return st;
}

KVPUB_API const char* kvpub_strerror(kvpub_status s) {
    switch (s) {
        case KVPUB_OK: return "ok";
        case KVPUB_ERR_INVALID_ARG: return "invalid argument";
        case KVPUB_ERR_OUT_OF_MEMORY: return "out of memory";
        case KVPUB_ERR_UNSUPPORTED: return "not supported (device not gfx950, or a configuration this call does not take)";
        case KVPUB_ERR_HIP: return "HIP runtime error";
        case KVPUB_ERR_CAPTURING: return "synchronizing call during stream capture";
        case KVPUB_ERR_FENCE_TIMEOUT: return "fence timed out; context poisoned";
        case KVPUB_ERR_IN_USE: return "the device's static context is in use";
        case KVPUB_STATUS_MAX_ENUM: break;
    }
    return "unknown status";
}

KVPUB_API uint32_t kvpub_abi_version(void) { return KVPUB_ABI_VERSION; }

}  // extern "C"
