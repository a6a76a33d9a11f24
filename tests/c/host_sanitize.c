/*
 * The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
 * (built by tests/test_sanitizers.py with the sanitizers on the host pass
 * only, this driver compiled by clang against the same runtime).  Every call
 * below must be rejected by the host-side checks -- with a pdr_status other
 * than PDR_ERR_HIP, before anything is enqueued -- so no device is touched:
 * null pointers, non-finite radii and scales, misaligned or short
 * workspaces, unknown formats and algorithms, and sizes at and past every
 * documented limit, where the size arithmetic would overflow 32 bits.  The
 * size queries (workspace bytes, binning variant, loss workspace) are walked
 * over a grid of extreme sizes and must return a size or a status.
 * The sanitizers turn any out-of-bounds access or signed overflow on these
 * paths into a failure.
 */
#include <limits.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "pdr_splat.h"

static int failures = 0;

#define REJECTED(call)                                                                  \
    do {                                                                                \
        int rc_ = (call);                                                               \
        if (!(rc_ < 0 && rc_ != PDR_ERR_HIP)) {                                         \
            fprintf(stderr, "NOT REJECTED (%d) %s:%d: %s\n", rc_, __FILE__, __LINE__, #call); \
            failures++;                                                                 \
        }                                                                               \
    } while (0)

#define EXPECT(cond)                                                                    \
    do {                                                                                \
        if (!(cond)) {                                                                  \
            fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);             \
            failures++;                                                                 \
        }                                                                               \
    } while (0)

/* sizes each of which breaks at least one documented limit */
static const int bad_sizes[][5] = {
    {0, 16, 16, 16, 1},          {16, 0, 16, 16, 1},         {16, 16, 0, 16, 1},
    {16, 16, 16, 0, 1},          {16, 16, 16, 16, 0},        {-1, 16, 16, 16, 1},
    {16, -5, 16, 16, 1},         {16, 16, -16, 16, 1},       {16, 16, 16, -16, 1},
    {16, 16, 16, 16, -3},        {INT_MIN, 16, 16, 16, 1},   {16, INT_MIN, 16, 16, 1},
    {INT_MAX, INT_MAX, 16, 16, 1}, {1, INT_MAX, 16, 16, 1},  {1, 16, INT_MAX, 16, 1},
    {1, 16, 16, INT_MAX, 1},     {1, 16, 16, 16, INT_MAX},   {1, 16, 16, 16, INT_MAX - 4},
    {INT_MAX, 1, 16, 16, INT_MAX}, {65536, 65536, 16, 16, 1}, {1, (1 << 22) + 1, 16, 16, 1},
    {1, 16, 32768, 16, 1},       {1, 16, 16, 16385, 1},      {1 << 20, 1, 8192, 8192, 2},
    {1 << 21, 1, 16384, 16384, 1}, {INT_MAX, 1, 32767, 16384, 1},
    {4096, 4096, 16, 16, 200},   {1 << 30, 2, 16, 16, 1},
};

static void sized_entry_points(const int *s, float *f, void *ws) {
    const int B = s[0], N = s[1], H = s[2], W = s[3], C = s[4];
    const size_t big = (size_t)1 << 40;
    unsigned long long *cnt = (unsigned long long *)ws;
    REJECTED(pdr_splat_forward(f, f, B, N, H, W, C, 3.0f, ws, big, NULL));
    REJECTED(pdr_splat_forward_fmt(f, f, PDR_FMT_F16, B, N, H, W, C, 3.0f, ws, big, NULL));
    REJECTED(pdr_splat_backward(f, f, f, B, N, H, W, C, 3.0f, ws, big, 1, NULL));
    REJECTED(pdr_splat_backward_fmt(f, f, PDR_FMT_BF16, f, B, N, H, W, C, 3.0f, ws, big, 0, NULL));
    for (int algo = PDR_BWD_AUTO; algo <= PDR_BWD_SPAN; algo++)
        REJECTED(pdr_splat_backward_algo(f, f, PDR_FMT_F32, f, B, N, H, W, C, 3.0f, ws, big, 1,
                                         algo, NULL));
    REJECTED(pdr_splat_bin(f, B, N, H, W, C, 3.0f, (int *)ws, (int *)ws, 1000, ws, big, NULL));
    REJECTED(pdr_splat_count_support(f, B, N, H, W, C, 3.0f, cnt, ws, big, NULL));
    REJECTED(pdr_splat_forward_concat(f, f, 2, f, B, N, H, W, C, 3.0f, ws, big, NULL));
    REJECTED(pdr_splat_backward_concat(f, f, 2, f, f, B, N, H, W, C, 3.0f, ws, big, 1, NULL));
    REJECTED(pdr_splat_forward_noalloc(f, f, B, N, H, W, C, 3.0f, (int *)ws, NULL));
    long long wb = pdr_splat_workspace_bytes(B, N, H, W, C, 1000);
    EXPECT(wb == PDR_ERR_INVALID_ARG);
    EXPECT(pdr_splat_bin_variant(B, N, H, W) <= 7);
}

int main(void) {
    void *ws = (void *)(size_t)0x100000;   /* 256-aligned, never dereferenced */
    float *f = (float *)ws;
    const size_t big = (size_t)1 << 40;

    for (size_t i = 0; i < sizeof bad_sizes / sizeof bad_sizes[0]; i++)
        sized_entry_points(bad_sizes[i], f, ws);

    /* valid sizes, every other argument wrong in turn */
    {
        const int B = 2, N = 64, H = 40, W = 72, C = 3;
        const float radii[] = {0.0f, -1.0f, NAN, INFINITY, -INFINITY, -0.0f, 1e-45f * -1.0f};
        for (size_t r = 0; r < sizeof radii / sizeof radii[0]; r++) {
            REJECTED(pdr_splat_forward(f, f, B, N, H, W, C, radii[r], ws, big, NULL));
            REJECTED(pdr_splat_backward(f, f, f, B, N, H, W, C, radii[r], ws, big, 0, NULL));
            REJECTED(pdr_splat_bin(f, B, N, H, W, C, radii[r], (int *)ws, (int *)ws, 10, ws, big,
                                   NULL));
            REJECTED(pdr_splat_count_support(f, B, N, H, W, C, radii[r],
                                             (unsigned long long *)ws, ws, big, NULL));
            REJECTED(pdr_splat_forward_noalloc(f, f, B, N, H, W, C, radii[r], (int *)ws, NULL));
        }
        REJECTED(pdr_splat_forward(NULL, f, B, N, H, W, C, 3.0f, ws, big, NULL));
        REJECTED(pdr_splat_forward(f, NULL, B, N, H, W, C, 3.0f, ws, big, NULL));
        REJECTED(pdr_splat_forward(f, f, B, N, H, W, C, 3.0f, NULL, big, NULL));
        for (int mis = 1; mis < 256; mis *= 2)
            REJECTED(pdr_splat_forward(f, f, B, N, H, W, C, 3.0f, (char *)ws + mis, big, NULL));
        REJECTED(pdr_splat_forward(f, f, B, N, H, W, C, 3.0f, ws, 0, NULL));
        REJECTED(pdr_splat_forward(f, f, B, N, H, W, C, 3.0f, ws,
                                   (size_t)pdr_splat_workspace_bytes(B, N, H, W, C, 0) - 1, NULL));
        const int fmts[] = {-1, 3, 7, INT_MAX, INT_MIN};
        for (size_t k = 0; k < sizeof fmts / sizeof fmts[0]; k++) {
            REJECTED(pdr_splat_forward_fmt(f, f, fmts[k], B, N, H, W, C, 3.0f, ws, big, NULL));
            REJECTED(pdr_splat_backward_fmt(f, f, fmts[k], f, B, N, H, W, C, 3.0f, ws, big, 0,
                                            NULL));
            REJECTED(pdr_splat_backward_algo(f, f, PDR_FMT_F32, f, B, N, H, W, C, 3.0f, ws, big,
                                             0, fmts[k], NULL));
        }
        REJECTED(pdr_splat_backward(f, NULL, f, B, N, H, W, C, 3.0f, ws, big, 0, NULL));
        REJECTED(pdr_splat_backward(f, f, NULL, B, N, H, W, C, 3.0f, ws, big, 0, NULL));
        REJECTED(pdr_splat_bin(f, B, N, H, W, C, 3.0f, NULL, (int *)ws, 10, ws, big, NULL));
        REJECTED(pdr_splat_bin(f, B, N, H, W, C, 3.0f, (int *)ws, (int *)ws, -1, ws, big, NULL));
        REJECTED(pdr_splat_count_support(f, B, N, H, W, C, 3.0f, NULL, ws, big, NULL));
        /* concat: pixel-branch channel counts that are negative or overflow */
        const int cps[] = {-1, INT_MIN, INT_MAX, INT_MAX - 2};
        for (size_t k = 0; k < sizeof cps / sizeof cps[0]; k++) {
            REJECTED(pdr_splat_forward_concat(f, f, cps[k], f, B, N, H, W, C, 3.0f, ws, big, NULL));
            REJECTED(pdr_splat_backward_concat(f, f, cps[k], f, f, B, N, H, W, C, 3.0f, ws, big,
                                               1, NULL));
        }
        REJECTED(pdr_splat_forward_concat(f, NULL, 2, f, B, N, H, W, C, 3.0f, ws, big, NULL));
        REJECTED(pdr_splat_forward_noalloc(NULL, f, B, N, H, W, C, 3.0f, (int *)ws, NULL));
        REJECTED(pdr_splat_forward_noalloc(f, f, B, N, H, W, C, 3.0f, NULL, NULL));
        /* a problem whose fixed workspace part exceeds the static scratch */
        REJECTED(pdr_splat_forward_noalloc(f, f, 384, 4096, 128, 128, 3, 3.0f, (int *)ws, NULL));
        REJECTED(pdr_splat_check(NULL, NULL, NULL));
        long long out2[2];
        REJECTED(pdr_splat_status_async(NULL, (long long *)ws, NULL));
        REJECTED(pdr_splat_status_async(ws, NULL, NULL));
        REJECTED(pdr_splat_status_async(ws, (long long *)((char *)ws + 4), NULL));
        REJECTED(pdr_splat_status_async((char *)ws + 8, (long long *)ws, NULL));
        (void)out2;
    }

    /* size queries over extreme grids: a size or a status, never UB */
    {
        const int vals[] = {INT_MIN, -1, 0, 1, 15, 16, 17, 4095, 16384, 16385, 32767, 32768,
                            (1 << 22), (1 << 22) + 1, 1 << 30, INT_MAX};
        const long long pairs[] = {LLONG_MIN, -1, 0, 1, 0x7fffffffLL, 0x80000000LL, LLONG_MAX};
        const int nv = (int)(sizeof vals / sizeof vals[0]);
        for (int a = 0; a < nv; a++)
            for (int b = 0; b < nv; b++)
                for (int c = 0; c < nv; c += 3)
                    for (int d = 0; d < nv; d += 3) {
                        const int B = vals[a], N = vals[b], H = vals[c], W = vals[d];
                        for (int Cc = 0; Cc < 4; Cc++) {
                            const int C = Cc == 3 ? INT_MAX : Cc * 7 + 1 - (Cc == 0);
                            for (size_t p = 0; p < sizeof pairs / sizeof pairs[0]; p++) {
                                long long r = pdr_splat_workspace_bytes(B, N, H, W, C, pairs[p]);
                                EXPECT(r > 0 || r == PDR_ERR_INVALID_ARG);
                            }
                            long long l = pdr_loss_workspace_bytes(B, H, W, C);
                            EXPECT(l > 0 || l == PDR_ERR_INVALID_ARG);
                        }
                        int v = pdr_splat_bin_variant(B, N, H, W);
                        EXPECT((v >= 0 && v <= 7) || v == PDR_ERR_INVALID_ARG);
                        int sp = pdr_splat_backward_splits(B, N, H, W);
                        EXPECT(sp == 1 || sp == 2 || sp == 4 || sp == 8 || sp == PDR_ERR_INVALID_ARG);
                    }
    }

    /* loss */
    {
        const int B = 2, H = 40, W = 33, C = 3;
        double *loss = (double *)ws;
        REJECTED(pdr_loss_l1_ssim(NULL, f, B, H, W, C, 0.2f, 1e-4f, 9e-4f, f, loss, ws, big, NULL));
        REJECTED(pdr_loss_l1_ssim(f, f, B, H, W, C, 0.2f, 1e-4f, 9e-4f, f, NULL, ws, big, NULL));
        const float lams[] = {-0.1f, 1.5f, NAN, INFINITY};
        for (size_t k = 0; k < sizeof lams / sizeof lams[0]; k++)
            REJECTED(pdr_loss_l1_ssim(f, f, B, H, W, C, lams[k], 1e-4f, 9e-4f, f, loss, ws, big,
                                      NULL));
        const float cs[] = {0.0f, -1e-4f, NAN, INFINITY};
        for (size_t k = 0; k < sizeof cs / sizeof cs[0]; k++) {
            REJECTED(pdr_loss_l1_ssim(f, f, B, H, W, C, 0.2f, cs[k], 9e-4f, f, loss, ws, big, NULL));
            REJECTED(pdr_loss_l1_ssim(f, f, B, H, W, C, 0.2f, 1e-4f, cs[k], f, loss, ws, big, NULL));
        }
        REJECTED(pdr_loss_l1_ssim(f, f, B, H, W, C, 0.2f, 1e-4f, 9e-4f, f, loss, ws, 16, NULL));
        REJECTED(pdr_loss_l1_ssim(f, f, B, H, W, C, 0.2f, 1e-4f, 9e-4f, f, loss, (char *)ws + 4,
                                  big, NULL));
        for (size_t i = 0; i < sizeof bad_sizes / sizeof bad_sizes[0]; i++) {
            const int *s = bad_sizes[i];
            if (pdr_loss_workspace_bytes(s[0], s[2], s[3], s[4]) > 0) continue;   /* N-only limit */
            REJECTED(pdr_loss_l1_ssim(f, f, s[0], s[2], s[3], s[4], 0.2f, 1e-4f, 9e-4f, f, loss,
                                      ws, big, NULL));
        }
    }

    /* grid initialisation and activations */
    {
        const int grids[][7] = {
            {0, 8, 8, 64, 64, 3, 0},     {2, 0, 8, 64, 64, 3, 0},   {2, 8, 0, 64, 64, 3, 0},
            {2, 8, 8, 0, 64, 3, 0},      {2, 8, 8, 64, 0, 3, 0},    {2, 8, 8, 64, 64, 0, 0},
            {2, 65536, 65536, 64, 64, 3, 0}, {2, INT_MAX, 2, 64, 64, 3, 0},
            {INT_MAX, 8, 8, 64, 64, INT_MAX, 0}, {-2, 8, 8, 64, 64, 3, 0},
        };
        for (size_t k = 0; k < sizeof grids / sizeof grids[0]; k++) {
            const int *g = grids[k];
            REJECTED(pdr_grid_init(f, g[0], g[1], g[2], g[3], g[4], g[5], 0.5f, NULL, NULL));
            REJECTED(pdr_params_activate(f, f, g[0], g[1], g[2], g[3], g[4], g[5], NULL));
            REJECTED(pdr_params_activate_backward(f, f, f, g[0], g[1], g[2], g[3], g[4], g[5],
                                                  NULL));
        }
        const float scales[] = {0.0f, -0.5f, NAN, INFINITY};
        for (size_t k = 0; k < sizeof scales / sizeof scales[0]; k++)
            REJECTED(pdr_grid_init(f, 2, 8, 8, 64, 64, 3, scales[k], NULL, NULL));
        REJECTED(pdr_grid_init(NULL, 2, 8, 8, 64, 64, 3, 0.5f, NULL, NULL));
        REJECTED(pdr_params_activate(NULL, f, 2, 8, 8, 64, 64, 3, NULL));
        REJECTED(pdr_params_activate(f, NULL, 2, 8, 8, 64, 64, 3, NULL));
        REJECTED(pdr_params_activate_backward(f, NULL, f, 2, 8, 8, 64, 64, 3, NULL));
    }

    /* strings and timing tables, indexed with every out-of-range value */
    {
        const int ids[] = {INT_MIN, -1, PDR_KERNEL_COUNT, PDR_KERNEL_COUNT + 1, INT_MAX};
        for (size_t k = 0; k < sizeof ids / sizeof ids[0]; k++) {
            const char *s = pdr_splat_kernel_name(ids[k]);
            EXPECT(s == NULL || strlen(s) < 64);
        }
        for (int k = 0; k < PDR_KERNEL_COUNT; k++) EXPECT(strlen(pdr_splat_kernel_name(k)) > 0);
        const int codes[] = {INT_MIN, -6, -5, -4, -3, -2, -1, 0, 1, INT_MAX};
        for (size_t k = 0; k < sizeof codes / sizeof codes[0]; k++)
            EXPECT(strlen(pdr_splat_status_string(codes[k])) > 0);
        double ms[PDR_KERNEL_COUNT];
        long long n[PDR_KERNEL_COUNT];
        int was = pdr_splat_timing(1);
        EXPECT(pdr_splat_timing_read(ms, n, 1) >= 0);
        EXPECT(pdr_splat_timing_read(NULL, NULL, 0) >= 0);
        pdr_splat_timing(was);
        for (int k = 0; k < PDR_KERNEL_COUNT; k++) EXPECT(n[k] == 0 && ms[k] == 0.0);
    }

    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("host sanitize ok\n");
    return 0;
}
