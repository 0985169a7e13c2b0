// VMM-backed replica storage with stable addresses (host code).
//
// vLLM PR #52863, Relationship to existing work: the replicated cache builds
// on PRs that keep the KV cache at a stable virtual address with its own
// rendezvous, so that it can grow without moving (and without re-exchanging
// peer views).  Here one context's replicas live in address ranges reserved
// for the largest page count; the first num_pages pages of every layer are
// backed with device memory, and growing backs more pages behind the same
// addresses.  Bases never move, so contexts and captured graphs stay valid.
//
// Every layer of every replica and array (Main-KV, Indexer-K) has a
// reservation of its own, max_pages * page_stride rounded up to the
// allocation granularity plus one spare granule; the span is the layer
// stride.  The L reservations of one replica and array sit back to back: a
// range of L spans is reserved to find free addresses, released, and reserved
// again layer by layer at those addresses (each returned address is checked).
// A reservation holds exactly one chunk, mapped at its start.  On this
// runtime, granting access to a chunk fails when another, smaller chunk is
// already mapped lower in the same reservation, so chunks never share one.
// Growing a layer maps a bigger chunk at a scratch reservation, copies the
// backed bytes into it, and swaps it in behind the layer's address; the old
// chunk is released only once the new one is in place and accessible (on any
// failure the old one is put back).  Every chunk's access flags are read back
// before it is handed out.
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "kvpub.h"
#include "kvpub_internal.h"

namespace {

struct Chunk {
    size_t bytes;
    hipMemGenericAllocationHandle_t handle;
};

uint64_t round_up(uint64_t x, uint64_t g) { return (x + g - 1) / g * g; }

}  // namespace

struct kvpub_vmm {
    int device;
    uint32_t replicas, layers;
    uint64_t page_stride[2];            // Main-KV, Indexer-K
    uint64_t span[2];                   // reserved bytes per layer (the layer strides)
    uint64_t backed[2];                 // backed bytes per layer
    uint64_t max_pages, pages;
    size_t gran;
    bool broken;                        // a layer lost its backing: nothing may be accessed
    uint8_t* base[2][KVPUB_MAX_REPLICAS];
    std::vector<Chunk> chunk;           // [array][replica][layer]
    std::vector<uint8_t> reserved;      // [array][replica][layer]: the layer's reservation is held
    size_t index(int a, uint32_t r, uint32_t l) const { return ((size_t)a * replicas + r) * layers + l; }
    Chunk& at(int a, uint32_t r, uint32_t l) { return chunk[index(a, r, l)]; }
    uint8_t* layer_ptr(int a, uint32_t r, uint32_t l) { return base[a][r] + l * span[a]; }
};

namespace {

hipMemAllocationProp device_prop(int device) {
    hipMemAllocationProp prop;
    std::memset(&prop, 0, sizeof prop);
    prop.type = hipMemAllocationTypePinned;
    prop.location.type = hipMemLocationTypeDevice;
    prop.location.id = device;
    return prop;
}

// Map `h` (bytes long) at ptr and make it read-write for the device; the access
// flags are read back, and on any failure nothing stays mapped.
hipError_t map_rw(int device, uint8_t* ptr, size_t bytes, hipMemGenericAllocationHandle_t h) {
    hipError_t e = hipMemMap(ptr, bytes, 0, h, 0);
    if (e != hipSuccess) return e;
    hipMemAccessDesc acc;
    std::memset(&acc, 0, sizeof acc);
    acc.location = device_prop(device).location;
    acc.flags = hipMemAccessFlagsProtReadWrite;
    e = hipMemSetAccess(ptr, bytes, &acc, 1);
    unsigned long long f0 = 0, f1 = 0;
    hipMemLocation loc = acc.location;
    if (e == hipSuccess) e = hipMemGetAccess(&f0, &loc, ptr);
    if (e == hipSuccess) e = hipMemGetAccess(&f1, &loc, ptr + bytes - 1);
    if (e == hipSuccess && (f0 != hipMemAccessFlagsProtReadWrite || f1 != hipMemAccessFlagsProtReadWrite))
        e = hipErrorInvalidValue;
    if (e != hipSuccess) (void)hipMemUnmap(ptr, bytes);
    return e;
}

// Test hook for the failure paths of growing: KVPUB_TEST_VMM_GROW_FAIL=swap
// makes mapping the bigger chunk at the layer's address fail (the old chunk is
// put back); =restore makes putting the old chunk back fail as well (the
// storage becomes broken).  Read at every grow, host side only.
struct GrowFailHook {
    bool swap = false, restore = false;
    GrowFailHook() {
        const char* s = std::getenv("KVPUB_TEST_VMM_GROW_FAIL");
        if (!s) return;
        restore = std::strcmp(s, "restore") == 0;
        swap = restore || std::strcmp(s, "swap") == 0;
    }
};

// Back layer (a, r, l) with `bytes` (> what it has), keeping its contents.
hipError_t grow_layer(kvpub_vmm* v, int a, uint32_t r, uint32_t l, size_t bytes, uint8_t* scratch) {
    const GrowFailHook hook;
    Chunk& old = v->at(a, r, l);
    uint8_t* ptr = v->layer_ptr(a, r, l);
    const hipMemAllocationProp prop = device_prop(v->device);
    hipMemGenericAllocationHandle_t h{};
    hipError_t e = hipMemCreate(&h, bytes, &prop, 0);
    if (e != hipSuccess) return e;
    if (old.bytes) {   // copy the backed bytes through the scratch address
        e = map_rw(v->device, scratch, bytes, h);
        if (e == hipSuccess) {
            e = hipMemcpy(scratch, ptr, old.bytes, hipMemcpyDeviceToDevice);
            if (e == hipSuccess) e = hipDeviceSynchronize();   // the copy is done before either side is unmapped
            (void)hipMemUnmap(scratch, bytes);
        }
        if (e == hipSuccess) e = hipMemUnmap(ptr, old.bytes);
        if (e != hipSuccess) { (void)hipMemRelease(h); return e; }
    }
    e = hook.swap ? hipErrorInvalidValue : map_rw(v->device, ptr, bytes, h);
    if (e != hipSuccess) {
        (void)hipMemRelease(h);
        // put the old chunk back; if even that fails the layer is unbacked
        if (old.bytes && (hook.restore || map_rw(v->device, ptr, old.bytes, old.handle) != hipSuccess)) {
            (void)hipMemRelease(old.handle);
            old = Chunk{0, hipMemGenericAllocationHandle_t{}};
            v->broken = true;
        }
        return e;
    }
    if (old.bytes) (void)hipMemRelease(old.handle);
    old = Chunk{bytes, h};
    return hipSuccess;
}

// Back every layer of every replica up to `pages` pages.
hipError_t back_to(kvpub_vmm* v, uint64_t pages) {
    uint64_t want[2];
    for (int a = 0; a < 2; ++a) want[a] = round_up(pages * v->page_stride[a], v->gran);
    if (want[0] <= v->backed[0] && want[1] <= v->backed[1]) return hipSuccess;
    void* scratch = nullptr;
    const size_t sb = want[0] > want[1] ? want[0] : want[1];
    hipError_t e = hipMemAddressReserve(&scratch, sb, v->gran, nullptr, 0);
    if (e != hipSuccess) return e;
    for (int a = 0; a < 2 && e == hipSuccess; ++a) {
        if (want[a] <= v->backed[a]) continue;
        for (uint32_t r = 0; r < v->replicas && e == hipSuccess; ++r)
            for (uint32_t l = 0; l < v->layers && e == hipSuccess; ++l)
                if (v->at(a, r, l).bytes < want[a]) e = grow_layer(v, a, r, l, want[a], static_cast<uint8_t*>(scratch));
    }
    (void)hipMemAddressFree(scratch, sb);
    if (e != hipSuccess) return e;   // layers already grown stay grown; the page count is unchanged
    for (int a = 0; a < 2; ++a) v->backed[a] = want[a];
    v->pages = pages;
    return hipSuccess;
}

// Reserve the L layer spans of (array a, replica r) back to back, one
// reservation per layer.  A range of L spans is reserved and released to find
// free addresses; the layers are then reserved at those exact addresses.  Some
// other reservation may take part of the range in between: then everything is
// given back and the search is repeated a few times.
hipError_t reserve_layers(kvpub_vmm* v, int a, uint32_t r) {
    const uint64_t span = v->span[a], total = span * v->layers;
    for (int attempt = 0; attempt < 4; ++attempt) {
        void* range = nullptr;
        hipError_t e = hipMemAddressReserve(&range, total, v->gran, nullptr, 0);
        if (e != hipSuccess) return e;
        e = hipMemAddressFree(range, total);
        if (e != hipSuccess) return e;
        uint8_t* base = static_cast<uint8_t*>(range);
        uint32_t got = 0;
        for (; got < v->layers; ++got) {
            void* want = base + got * span;
            void* p = nullptr;
            if (hipMemAddressReserve(&p, span, v->gran, want, 0) != hipSuccess) break;
            if (p != want) { (void)hipMemAddressFree(p, span); break; }
        }
        if (got == v->layers) {
            v->base[a][r] = base;
            for (uint32_t l = 0; l < v->layers; ++l) v->reserved[v->index(a, r, l)] = 1;
            return hipSuccess;
        }
        for (uint32_t l = 0; l < got; ++l) (void)hipMemAddressFree(base + l * span, span);
    }
    return hipErrorOutOfMemory;
}

void release_vmm(kvpub_vmm* v) {
    for (int a = 0; a < 2; ++a)
        for (uint32_t r = 0; r < v->replicas; ++r) {
            for (uint32_t l = 0; l < v->layers && !v->chunk.empty(); ++l) {
                Chunk& c = v->at(a, r, l);
                if (c.bytes) {
                    (void)hipMemUnmap(v->layer_ptr(a, r, l), c.bytes);
                    (void)hipMemRelease(c.handle);
                }
                if (v->reserved[v->index(a, r, l)]) (void)hipMemAddressFree(v->layer_ptr(a, r, l), v->span[a]);
            }
        }
    delete v;
}

kvpub_status status_of(hipError_t e) {
    return e == hipSuccess ? KVPUB_OK : e == hipErrorOutOfMemory ? KVPUB_ERR_OUT_OF_MEMORY : KVPUB_ERR_HIP;
}

}  // namespace

extern "C" {

KVPUB_API kvpub_status kvpub_vmm_create(kvpub_config* cfg, uint64_t max_pages, void** main_bases,
                                        void** idx_bases, kvpub_vmm** out) {
    if (!out) return KVPUB_ERR_INVALID_ARG;
    *out = nullptr;
    if (!cfg || cfg->struct_size != sizeof(kvpub_config) || !main_bases || !idx_bases) return KVPUB_ERR_INVALID_ARG;
    if (cfg->num_replicas < 1 || cfg->num_replicas > KVPUB_MAX_REPLICAS || cfg->num_layers < 1)
        return KVPUB_ERR_INVALID_ARG;
    if (cfg->num_pages < 1 || max_pages < cfg->num_pages || max_pages > (1ull << 32)) return KVPUB_ERR_INVALID_ARG;
    if (cfg->main_page_stride < KVPUB_MAIN_PAGE_BYTES || cfg->main_page_stride % 16) return KVPUB_ERR_INVALID_ARG;
    if (cfg->idx_page_stride < KVPUB_IDX_PAGE_BYTES || cfg->idx_page_stride % 16) return KVPUB_ERR_INVALID_ARG;
    if (cfg->device < 0) return KVPUB_ERR_INVALID_ARG;

    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(cfg->device) != hipSuccess) return KVPUB_ERR_HIP;
    kvpub_vmm* v = new (std::nothrow) kvpub_vmm();
    if (!v) { (void)hipSetDevice(prev); return KVPUB_ERR_OUT_OF_MEMORY; }
    v->device = cfg->device;
    v->replicas = cfg->num_replicas;
    v->layers = cfg->num_layers;
    v->page_stride[0] = cfg->main_page_stride;
    v->page_stride[1] = cfg->idx_page_stride;
    v->max_pages = max_pages;
    v->chunk.assign((size_t)2 * v->replicas * v->layers, Chunk{0, hipMemGenericAllocationHandle_t{}});
    v->reserved.assign((size_t)2 * v->replicas * v->layers, 0);
    const hipMemAllocationProp prop = device_prop(cfg->device);
    hipError_t e = hipMemGetAllocationGranularity(&v->gran, &prop, hipMemAllocationGranularityRecommended);
    if (e == hipSuccess && v->gran == 0) e = hipErrorInvalidValue;
    for (int a = 0; a < 2 && e == hipSuccess; ++a) {
        v->span[a] = round_up(max_pages * v->page_stride[a], v->gran) + v->gran;   // + the spare granule
        for (uint32_t r = 0; r < v->replicas && e == hipSuccess; ++r) e = reserve_layers(v, a, r);
    }
    if (e == hipSuccess) e = back_to(v, cfg->num_pages);
    if (e != hipSuccess) {
        release_vmm(v);
        (void)hipSetDevice(prev);
        return status_of(e);
    }
    cfg->main_layer_stride = v->span[0];
    cfg->idx_layer_stride = v->span[1];
    for (uint32_t r = 0; r < v->replicas; ++r) {
        main_bases[r] = v->base[0][r];
        idx_bases[r] = v->base[1][r];
    }
    (void)hipSetDevice(prev);
    *out = v;
    return KVPUB_OK;
}

KVPUB_API kvpub_status kvpub_vmm_grow(kvpub_vmm* v, uint64_t num_pages, kvpub_ctx* ctx) {
    if (!v || num_pages > v->max_pages) return KVPUB_ERR_INVALID_ARG;
    if (ctx && !kvpub::ctx_uses_storage(ctx, v->replicas, v->base[0], v->base[1], v->span[0], v->span[1],
                                        v->page_stride[0], v->page_stride[1]))
        return KVPUB_ERR_INVALID_ARG;
    if (num_pages > v->pages) {
        int prev = -1;
        if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(v->device) != hipSuccess) return KVPUB_ERR_HIP;
        // no kernel may use the storage while chunks are swapped
        hipError_t e = v->broken ? hipErrorInvalidValue : hipDeviceSynchronize();
        if (e == hipSuccess) e = back_to(v, num_pages);
        (void)hipSetDevice(prev);
        if (v->broken) {
            v->pages = 0;
            if (ctx) (void)kvpub::ctx_set_pages(ctx, 0);   // every slot is out of range from now on
            return KVPUB_ERR_HIP;
        }
        if (e != hipSuccess) return status_of(e);
    }
    // the context's capacity, on the host and in its device words (which the
    // kernels of graphs captured earlier read as well)
    if (ctx && kvpub::ctx_set_pages(ctx, v->pages) != hipSuccess) return KVPUB_ERR_HIP;
    return KVPUB_OK;
}

KVPUB_API kvpub_status kvpub_vmm_pages(kvpub_vmm* v, uint64_t* num_pages) {
    if (!v || !num_pages) return KVPUB_ERR_INVALID_ARG;
    *num_pages = v->pages;
    return KVPUB_OK;
}

KVPUB_API kvpub_status kvpub_vmm_destroy(kvpub_vmm* v) {
    if (!v) return KVPUB_OK;
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(v->device) != hipSuccess) return KVPUB_ERR_HIP;
    const hipError_t e = hipDeviceSynchronize();
    release_vmm(v);
    (void)hipSetDevice(prev);
    return status_of(e);
}

}  // extern "C"
