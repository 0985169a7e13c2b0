// Internal interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct kvpub_ctx;

namespace kvpub {

constexpr int kMaxReplicas = 8;
constexpr int kTokensPerWave = 4;     // 4 tokens x 5 tiles = 5 rounds of 4 tiles per wave
constexpr int kWavesPerBlock = 4;     // 256 threads, 16 tokens per block (1, 2 and 8 measured: no better)
constexpr int kTokensPerBlock = kTokensPerWave * kWavesPerBlock;
constexpr int64_t kMaxTokensPerLaunch = int64_t(1) << 24;   // larger batches take several launches

constexpr uint32_t kStatusFenceTimeout = 0x1u;
constexpr uint32_t kStatusPoisoned = 0x2u;

// Words of a context that live in device memory, each on its own 128-byte line.
constexpr size_t kLine = 128;
constexpr size_t kStatusOffset = 0;          // the CtxHead line
constexpr size_t kInvalidOffset = kLine;
constexpr size_t kEpochOffset = 2 * kLine;          // + lane * kLine
constexpr size_t kSignalStride = kLine / 8;         // uint64 words between participant signals

// The first line of a context's device words: the status flags (set by a
// fence that timed out) and the number of slots per layer that may be written
// (set by the host at creation and when a VMM storage grows).  Kernels read
// both with one scalar load at launch time, so a captured graph sees a
// capacity raised after its capture.
struct CtxHead {
    uint32_t status;
    uint32_t reserved;
    int64_t capacity;            // num_pages * 64
};
static_assert(sizeof(CtxHead) == 16, "one 16-byte scalar load");

struct StoreParams {
    const uint16_t* latent;      // bf16 bit patterns
    const uint16_t* rope;
    const uint16_t* indexer;
    int64_t latent_stride;       // elements
    int64_t rope_stride;
    int64_t indexer_stride;
    const int64_t* slots;
    int64_t num_tokens;
    uint64_t main_page_stride;   // bytes
    uint64_t idx_page_stride;
    uint8_t* main_base[kMaxReplicas];  // replica r, already offset to the layer
    uint8_t* idx_base[kMaxReplicas];
    unsigned long long* invalid_count;
    const CtxHead* head;         // status and capacity
    uint32_t main_region;        // bytes of one replica's layer span (all the pages it may ever hold)
    uint32_t idx_region;         // if below 2^32, else 0: the write-through path needs 32-bit offsets
};

struct FenceParams {
    uint64_t* epoch;             // this lane's epoch word
    uint64_t* signals;           // this lane's participant signals, kSignalStride apart (null alone)
    uint32_t num_participants;
    uint32_t self;               // this GPU's participant index (0)
    uint32_t* status;
    uint64_t timeout_ticks;      // in wall-clock (s_memrealtime) ticks
    uint32_t acquire_wait;       // alone: acquire-wait on the epoch after the release RMW (else release only)
};

// Enqueue one store kernel on `stream`; returns the launch status.
hipError_t launch_store(const StoreParams& p, uint32_t num_replicas, hipStream_t stream);
struct GatherParams {
    const uint8_t* main_base;    // the replica, already offset to the layer
    const uint8_t* idx_base;
    uint64_t main_page_stride;   // bytes
    uint64_t idx_page_stride;
    const CtxHead* head;         // capacity (num_pages * 64)
    const int64_t* slots;
    int64_t num_tokens;
    uint16_t* latent;            // bf16 outputs
    uint16_t* rope;
    uint16_t* indexer;
    int64_t latent_stride;       // elements
    int64_t rope_stride;
    int64_t indexer_stride;
    unsigned long long* invalid_count;
    uint32_t offsets32;          // every offset within a layer fits in 32 bits (layer span < 2^32)
};

// Enqueue the dequantizing gather on `stream`; returns the launch status.
hipError_t launch_gather(const GatherParams& p, hipStream_t stream);
// True if ctx's replicas are exactly these bases with these layer and page strides.
bool ctx_uses_storage(const kvpub_ctx* ctx, uint32_t replicas, uint8_t* const* main_bases,
                      uint8_t* const* idx_bases, uint64_t main_layer_stride, uint64_t idx_layer_stride,
                      uint64_t main_page_stride, uint64_t idx_page_stride);
// Set the number of pages per layer that ctx's launches may write, on the host
// and in the device capacity word (synchronous copy; no launch on ctx may run).
hipError_t ctx_set_pages(kvpub_ctx* ctx, uint64_t num_pages);
// Enqueue one fence kernel on `stream`.
hipError_t launch_fence(const FenceParams& p, hipStream_t stream);
// Enqueue the two-launch host-epoch fence (publish e, then wait for e) on `stream`.
hipError_t launch_host_epoch_fence(const FenceParams& p, uint64_t e, hipStream_t stream);

}  // namespace kvpub
