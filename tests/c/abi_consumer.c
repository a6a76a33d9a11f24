/*
 * A plain C99 consumer of the library's C ABI, using only its host-side
 * behaviour (no device is touched): the header compiles as C with strict
 * warnings, the library links, workspace sizing follows the documented
 * layout, and invalid arguments are rejected with the documented status
 * before anything is enqueued.  Built and run by tests/test_abi_c.py.
 */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "pdr_splat.h"

#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond); \
            return 1;                                                      \
        }                                                                  \
    } while (0)

static long long round256(long long v) { return (v + 255) / 256 * 256; }

int main(void) {
    /* an aligned, never dereferenced address: validation fails first */
    void *fake = (void *)(size_t)0x10000;
    float *ffake = (float *)fake;
    const int t = pdr_splat_tile_size();
    CHECK(t == 16 || t == 32);

    /* fixed part: header, 32-byte records, 32-byte thin-Gaussian records,
     * 8-byte boxes, per-tile counts, per-tile group totals, tile offsets, the
     * tile order, the 256 KiB order histogram; then 4 bytes per pair */
    {
        const int B = 2, N = 100, H = 40, W = 72, C = 3;
        const long long nTx = (W + t - 1) / t, nTy = (H + t - 1) / t, nT = B * nTx * nTy;
        const long long fixed = round256(256) + round256((long long)B * N * 32) +
                                round256((long long)B * N * 32) +
                                round256((long long)B * N * 8) + round256(nT * 4) +
                                round256(nT * 4) + round256((nT + 1) * 4) + round256(nT * 4) +
                                262144;
        CHECK(pdr_splat_workspace_bytes(B, N, H, W, C, 0) == fixed);
        CHECK(pdr_splat_workspace_bytes(B, N, H, W, C, 1000) == fixed + round256(4000));
    }
    CHECK(pdr_splat_workspace_bytes(0, 100, 40, 72, 3, 0) == PDR_ERR_INVALID_ARG);
    CHECK(pdr_splat_workspace_bytes(1, 100, 40, 72, 0, 0) == PDR_ERR_INVALID_ARG);
    CHECK(pdr_splat_workspace_bytes(1, 100, 40, 72, 3, -1) == PDR_ERR_INVALID_ARG);

    CHECK(pdr_splat_forward(NULL, ffake, 1, 4, 16, 16, 1, 3.0f, fake, 1 << 20, NULL) ==
          PDR_ERR_INVALID_ARG);
    CHECK(pdr_splat_forward(ffake, ffake, 1, 4, 16, 16, 1, (float)NAN, fake, 1 << 20, NULL) ==
          PDR_ERR_INVALID_ARG);
    CHECK(pdr_splat_forward(ffake, ffake, 1, 4, 16, 16, 1, 3.0f, (char *)fake + 4, 1 << 20,
                            NULL) == PDR_ERR_WORKSPACE);
    CHECK(pdr_splat_forward(ffake, ffake, 1, 4, 16, 16, 1, 3.0f, fake, 64, NULL) ==
          PDR_ERR_WORKSPACE);
    CHECK(pdr_splat_backward(ffake, NULL, ffake, 1, 4, 16, 16, 1, 3.0f, fake, 1 << 20, 1, NULL) ==
          PDR_ERR_INVALID_ARG);
    CHECK(pdr_splat_check(NULL, NULL, NULL) == PDR_ERR_INVALID_ARG);

    CHECK(pdr_loss_workspace_bytes(2, 40, 33, 3) > 0);
    CHECK(pdr_loss_workspace_bytes(0, 40, 33, 3) < 0);

    CHECK(pdr_splat_status_string(PDR_OK) != NULL);
    CHECK(strcmp(pdr_splat_status_string(PDR_OK), pdr_splat_status_string(PDR_ERR_OVERFLOW)));
    for (int k = 0; k < PDR_KERNEL_COUNT; k++) CHECK(pdr_splat_kernel_name(k) != NULL);

    printf("abi consumer ok\n");
    return 0;
}
