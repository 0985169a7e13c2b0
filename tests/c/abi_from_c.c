/* Uses libkvpub.so from plain C (C99) through include/kvpub.h only, without a
 * GPU: the header compiles as C, the library links and loads, and the host-side
 * checks answer as documented.  Prints "ok" and exits 0, else names the check. */
#include <stdio.h>
#include <string.h>

#include "kvpub.h"

#define CHECK(c)                                                   \
    do {                                                           \
        if (!(c)) {                                                \
            printf("failed: %s (line %d)\n", #c, __LINE__);         \
            return 1;                                              \
        }                                                          \
    } while (0)

int main(void) {
    kvpub_config cfg;
    void *bases[2] = {(void *)16, (void *)32};
    kvpub_ctx *ctx = (kvpub_ctx *)1;
    kvpub_vmm *vmm = (kvpub_vmm *)1;
    uint64_t pages = 0;

    CHECK(kvpub_abi_version() == KVPUB_ABI_VERSION);
    kvpub_config_init(&cfg, 2, 3, 10);
    CHECK(cfg.struct_size == sizeof(kvpub_config));
    CHECK(cfg.block_size == KVPUB_SLOTS_PER_PAGE);
    CHECK(cfg.main_page_stride == KVPUB_MAIN_PAGE_BYTES && cfg.idx_page_stride == KVPUB_IDX_PAGE_BYTES);
    CHECK(cfg.main_layer_stride == 10ull * KVPUB_MAIN_PAGE_BYTES);

    cfg.num_replicas = KVPUB_MAX_REPLICAS + 1;                       /* rejected before any HIP call */
    CHECK(kvpub_create(&cfg, bases, bases, &ctx) == KVPUB_ERR_INVALID_ARG && ctx == NULL);
    kvpub_config_init(&cfg, 2, 3, 10);
    bases[1] = (void *)40;                                           /* misaligned base */
    CHECK(kvpub_create(&cfg, bases, bases, &ctx) == KVPUB_ERR_INVALID_ARG && ctx == NULL);
    CHECK(kvpub_create(&cfg, bases, bases, NULL) == KVPUB_ERR_INVALID_ARG);

    CHECK(kvpub_store(NULL, 0, 4, bases[0], 512, bases[0], 64, bases[0], 128, NULL, NULL) == KVPUB_ERR_INVALID_ARG);
    CHECK(kvpub_gather(NULL, 0, 0, 4, NULL, NULL, 512, NULL, 64, NULL, 128, NULL) == KVPUB_ERR_INVALID_ARG);
    CHECK(kvpub_fence(NULL, 0, NULL) == KVPUB_ERR_INVALID_ARG);
    CHECK(kvpub_fence_host_epoch(NULL, 0, NULL) == KVPUB_ERR_INVALID_ARG);
    CHECK(kvpub_graph_replay(NULL, NULL) == KVPUB_ERR_INVALID_ARG);
    CHECK(kvpub_graph_destroy(NULL) == KVPUB_OK);
    CHECK(kvpub_destroy(NULL) == KVPUB_OK);

    CHECK(kvpub_vmm_create(&cfg, 5, bases, bases, &vmm) == KVPUB_ERR_INVALID_ARG && vmm == NULL);
    CHECK(kvpub_vmm_grow(NULL, 8, NULL) == KVPUB_ERR_INVALID_ARG);
    CHECK(kvpub_vmm_pages(NULL, &pages) == KVPUB_ERR_INVALID_ARG);
    CHECK(kvpub_vmm_destroy(NULL) == KVPUB_OK);

    CHECK(strcmp(kvpub_strerror(KVPUB_OK), "ok") == 0);
    CHECK(strlen(kvpub_strerror(KVPUB_ERR_FENCE_TIMEOUT)) > 0);
    CHECK(strcmp(kvpub_strerror((kvpub_status)99), "unknown status") == 0);
    printf("ok\n");
    return 0;
}
