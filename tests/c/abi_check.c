/*
 * abi_check.c - a plain C99 consumer of include/peg.h: the header compiles
 * as C, the library links and loads from C, and its host-side checks answer
 * with the documented status codes. No call here passes its checks, so no
 * GPU work is enqueued and no GPU is needed.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "peg.h"

static int failures = 0;

static void expect(int cond, const char* what) {
    if (!cond) {
        fprintf(stderr, "FAIL: %s\n", what);
        ++failures;
    }
}

int main(void) {
    /* never dereferenced: every call below fails its host checks first */
    void* fake = (void*)(uintptr_t)0x10000;
    int32_t* ifake = (int32_t*)fake;
    float* ffake = (float*)fake;

    expect((peg_abi_version() >> 16) == 1, "ABI major version 1");
    expect(strcmp(peg_status_string(PEG_OK), peg_status_string(PEG_ERR_NULL_ARG)) != 0, "status strings differ");
    expect(peg_workspace_bytes(-1, 2, 8) == 0, "workspace of a bad shape is 0");
    expect(peg_workspace_bytes(4096, 2, 8) >= (size_t)4096 * 2 * 4, "workspace holds a rebuilt slot map");

    expect(peg_route_prep(ifake, 4, 2, 0, PEG_BINNED, 2, 0, ifake, ifake, NULL, ifake, NULL, NULL, fake,
                          1 << 20, NULL) == PEG_ERR_BAD_SHAPE, "route_prep E = 0");
    expect(peg_route_prep(NULL, 4, 2, 4, PEG_BINNED, 2, 0, ifake, ifake, NULL, ifake, NULL, NULL, fake, 1 << 20,
                          NULL) == PEG_ERR_NULL_ARG, "route_prep NULL top_experts");
    expect(peg_route_prep_noalloc(ifake, 131073, 1, 1024, PEG_BINNED, 200, 0, ifake, ifake, NULL, ifake, NULL, NULL,
                                  NULL) == PEG_ERR_SCRATCH_LIMIT, "route_prep_noalloc past its scratch");
    expect(PEG_NOALLOC_SCRATCH_BYTES == (1u << 20), "static scratch size");
    expect(peg_gather_binned(fake, 9, 4, 8, 2, 4, 2, ifake, ifake, ifake, ifake, fake, fake, 1 << 20, NULL) ==
               PEG_ERR_BAD_DTYPE, "gather_binned bad dtype");
    expect(peg_scatter_combine(fake, PEG_BF16, PEG_BINNED, 4, 8, 2, 4, 2, ifake, ifake, ifake, NULL, ifake, NULL,
                               NULL, fake, 1 << 20, NULL) == PEG_ERR_NULL_ARG, "scatter_combine NULL out");
    expect(peg_wgrad(fake, fake, PEG_BF16, PEG_BINNED, 4, 0, 2, 4, 2, ifake, ifake, ifake, NULL, ifake, ffake, fake,
                     1 << 20, NULL) == PEG_ERR_BAD_SHAPE, "wgrad H = 0");
    expect(peg_router_topk(fake, PEG_F32, 4, 8, 9, PEG_GATING_SOFTMAX, 1, ifake, ffake, NULL) == PEG_ERR_BAD_SHAPE,
           "router_topk K > E");
    expect(peg_routing_map_compact(fake, PEG_F32, (const uint8_t*)fake, 4, 8, 0, ffake, ifake, NULL) ==
               PEG_ERR_BAD_SHAPE, "compaction topk = 0");

    if (failures) return 1;
    printf("abi_check ok\n");
    return 0;
}
