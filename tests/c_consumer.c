/* A plain C99 program built against include/pipegemm.h and include/pipeattn.h
 * and linked with the library: the headers are valid C, and the pure-host
 * entry points answer a C caller without a device.  Prints "c consumer: OK"
 * and returns 0, or names the first failed check and returns 1. */
#include <stdio.h>
#include <string.h>

#include "pipeattn.h"
#include "pipegemm.h"

#define CHECK(cond, what)                                  \
    do {                                                   \
        if (!(cond)) {                                     \
            printf("c consumer: FAILED %s\n", what);       \
            return 1;                                      \
        }                                                  \
    } while (0)

int main(void)
{
    const int64_t budget = 160 * 1024;
    gemm_config cfg[512];
    gemm_config d;
    int n, i, found = 0;

    /* the LDS rule: S x (bM + bN) x bK x 2 bytes */
    CHECK(gemm_lds_bytes(128, 128, 32, 3, 0, GEMM_F16) == 3 * (128 + 128) * 32 * 2, "gemm_lds_bytes");
    /* 256 x 256 x 64 with 4 stages is over 160 KiB: a budget error, not "unsupported" */
    CHECK(gemm_check(GEMM_NN, 4096, 4096, 4096, GEMM_BF16, 256, 256, 64, 4, 0, 512, budget) == GEMM_ERR_LDS_BUDGET,
          "over-budget status");
    CHECK(strlen(gemm_last_error()) > 0, "message after a failed check");
    CHECK(gemm_check(GEMM_NT, 4096, 4096, 4096, GEMM_F16, 128, 128, 32, 3, 0, 256, budget) == GEMM_OK,
          "a built configuration");
    CHECK(strcmp(gemm_last_error(), "") == 0, "message cleared by GEMM_OK");
    /* the configuration space, counted then fetched */
    n = gemm_configs(GEMM_NT, GEMM_F16, NULL, 0);
    CHECK(n > 0 && n <= 512, "gemm_configs count");
    CHECK(gemm_configs(GEMM_NT, GEMM_F16, cfg, n) == n, "gemm_configs fetch");
    /* the gfx950 default for 4096^3 is one of the built configurations */
    CHECK(gemm_default_config(GEMM_NT, 4096, 4096, 4096, GEMM_F16, &d) == GEMM_OK, "gemm_default_config");
    for (i = 0; i < n; ++i)
        if (memcmp(&cfg[i], &d, sizeof d) == 0)
            found = 1;
    CHECK(found, "default is in the built space");
    CHECK(gemm_check(GEMM_NT, 4096, 4096, 4096, GEMM_F16, d.block_M, d.block_N, d.block_K, d.num_stages, d.a_lead,
                     d.threads, budget) == GEMM_OK,
          "default passes validation");
    /* attention: two tiles (K and V) per slot */
    CHECK(attn_lds_bytes(128, 128, 2) == 2 * 2 * 128 * 128 * 2, "attn_lds_bytes");
    CHECK(attn_check(4, 32, 32, 4096, 4096, 128, GEMM_F16, 0, 256, 128, 2, 512, budget) == GEMM_OK,
          "attention configuration");
    CHECK(attn_check(4, 32, 32, 4096, 4096, 128, GEMM_F16, 0, 256, 128, 3, 512, budget) == GEMM_ERR_LDS_BUDGET,
          "attention over budget");
    {
        int bm = 0, bn = 0, st = 0, th = 0;
        CHECK(attn_default_config(4, 32, 4096, 128, 1, &bm, &bn, &st, &th) == GEMM_OK && bm == 256 && bn == 128 &&
                  st == 2 && th == 512,
              "attn_default_config");
        CHECK(attn_check(4, 32, 32, 4096, 4096, 128, GEMM_F16, 1, bm, bn, st, th, budget) == GEMM_OK,
              "attn_check of the default configuration");
        CHECK(attn_default_config(1, 1, 1, 96, 0, &bm, &bn, &st, &th) == GEMM_ERR_UNSUPPORTED,
              "attn_default_config rejects dim 96");
    }
    printf("c consumer: OK (%d configurations; default %dx%dx%d S=%d lead=%d threads=%d)\n", n, d.block_M,
           d.block_N, d.block_K, d.num_stages, d.a_lead, d.threads);
    return 0;
}
