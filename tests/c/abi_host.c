/* A C11 caller of the tile_gemm C ABI that needs no GPU: version, status
 * strings, plan and workspace queries, packed-B sizes and argument errors
 * (all answered on the host before any device work).  Prints one line per
 * check as "name value"; the test compares them with the binding's view. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tile_gemm.h"

int main(void) {
    printf("abi_version %d\n", tile_gemm_abi_version());
    printf("status_invalid %s\n", strncmp(tile_gemm_status_string(TG_ERR_INVALID_ARG), "TG_ERR_INVALID_ARG", 18) == 0
                                      ? "ok" : "bad");

    tg_options o;
    memset(&o, 0, sizeof o);
    o.struct_size = (int)sizeof o;
    tg_plan_info info;
    tg_status st = tile_gemm_plan(1, 8192, 8192, 8192, TG_BF16, &o, &info);
    printf("plan_status %d\n", (int)st);
    printf("plan_c2 %d %d %d %lld\n", info.config, info.block_m, info.block_n, (long long)info.grid);

    o.bias_mode = 1;
    o.activation = 2;
    st = tile_gemm_plan(1, 8191, 8193, 8190, TG_BF16, &o, &info);
    printf("plan_c3_tail %d %d %lld\n", (int)st, info.config, (long long)info.strip_blocks);

    int64_t bytes = -1;
    memset(&o, 0, sizeof o);
    o.struct_size = (int)sizeof o;
    o.split_k = 4;
    st = tile_gemm_workspace_size(1, 512, 512, 131072, TG_BF16, &o, &bytes);
    printf("workspace_split4 %d %lld\n", (int)st, (long long)bytes);

    printf("packed_ld %lld %lld\n", (long long)tile_gemm_packed_b_ld(8193, TG_BF16),
           (long long)tile_gemm_packed_b_ld(45, TG_F32));
    st = tile_gemm_packed_b_size(3, 100, 129, TG_F16, &bytes);
    printf("packed_size %d %lld\n", (int)st, (long long)bytes);

    /* argument errors: negative extent, NULL operands, ld too small */
    float c[4];
    printf("err_negative %d\n", (int)tile_gemm(-1, 2, 2, TG_F32, c, 2, c, 2, c, 2, 1.0f, 0.0f, NULL));
    printf("err_null %d\n", (int)tile_gemm(2, 2, 2, TG_F32, NULL, 2, c, 2, c, 2, 1.0f, 0.0f, NULL));
    printf("err_lda %d\n", (int)tile_gemm(2, 2, 4, TG_F32, c, 3, c, 2, c, 2, 1.0f, 0.0f, NULL));
    printf("err_pack_align %d\n", (int)tile_gemm_pack_b(1, 4, 4, TG_BF16, (const void *)0x10000, 4, 0, 0,
                                                        (void *)0x20010, 4096, NULL));
    return 0;
}
