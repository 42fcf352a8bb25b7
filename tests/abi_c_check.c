/*
 * abi_c_check.c -- a plain C11 user of include/moe_route.h: it compiles the header as C, links
 * libmoe_route.so and calls the entry points on arguments that fail validation, so no GPU is
 * needed (validation happens before any HIP call and returns a status). tests/test_abi_c.py builds
 * and runs it.
 */
#include <stdio.h>
#include <string.h>

#include "moe_route.h"

#define EXPECT(cond)                                                                              \
    do {                                                                                          \
        if (!(cond)) {                                                                            \
            fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__);                           \
            return 1;                                                                             \
        }                                                                                         \
    } while (0)

int main(void)
{
    EXPECT(strcmp(moe_status_str(MOE_OK), "MOE_OK") == 0);
    EXPECT(strstr(moe_status_str(MOE_ERR_WORKSPACE), "workspace") != NULL);
    /* k > E is invalid; E beyond the maximum is unsupported */
    EXPECT(moe_route_topk(NULL, 4, 8, 9, NULL, NULL, NULL) == MOE_ERR_INVALID);
    EXPECT(moe_route_topk(NULL, 4, MOE_MAX_EXPERTS + 1, 2, NULL, NULL, NULL) ==
           MOE_ERR_UNSUPPORTED);
    /* the workspace grows with the batch and is zero for invalid sizes */
    EXPECT(moe_dispatch_workspace_bytes(4096, 384, 8) > moe_dispatch_workspace_bytes(128, 384, 8));
    EXPECT(moe_dispatch_workspace_bytes(-1, 8, 2) == 0);
    /* E % n_ranks != 0 */
    moe_dispatch_out_t out;
    memset(&out, 0, sizeof out);
    EXPECT(moe_dispatch_layout(NULL, 4, 2, 9, 2, &out, NULL, 0, NULL) == MOE_ERR_INVALID);
    /* fp8 needs H % 128 == 0 */
    char dummy[64] __attribute__((aligned(16)));
    EXPECT(moe_dispatch_pack(dummy, MOE_BF16, 4, 96, 2, (const int32_t*)dummy, MOE_FP8_E4M3, dummy,
                             (float*)dummy, NULL) == MOE_ERR_UNSUPPORTED);
    EXPECT(moe_combine(dummy, MOE_BF16, 4, 256, 0, NULL, NULL, dummy, MOE_BF16, NULL) ==
           MOE_ERR_INVALID);
    EXPECT(moe_check_topk(NULL, 4, 2, 8, NULL, NULL) == MOE_ERR_INVALID);
    EXPECT(moe_ep_capacity(512, 384, 8, 8) == 512 * 8);
    printf("C ABI check: ok\n");
    return 0;
}
