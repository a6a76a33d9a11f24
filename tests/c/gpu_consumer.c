/*
 * A plain C99 program that renders through the library's C ABI on the GPU,
 * with nothing but the HIP runtime for device memory and a stream: reads a
 * problem from a file, runs pdr_splat_forward, checks the workspace status
 * (growing the workspace to the reported pair count on overflow), runs
 * pdr_splat_backward reusing the forward's binning, and writes the image
 * and the parameter gradients back.  Built and run by tests/test_abi_c.py,
 * which compares the results with the oracle.
 *
 * input:  int32 B, N, H, W, C; float32 radius; float32 params[B][N][5+C];
 *         float32 grad_image[B][H][W][C]
 * output: float32 image[B][H][W][C]; float32 grad_params[B][N][5+C];
 *         int64 pairs
 */
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "pdr_splat.h"

#define HIPCHECK(x)                                                              \
    do {                                                                         \
        hipError_t e_ = (x);                                                     \
        if (e_ != hipSuccess) {                                                  \
            fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_),   \
                    __FILE__, __LINE__);                                         \
            return 1;                                                            \
        }                                                                        \
    } while (0)

#define PDRCHECK(x)                                                              \
    do {                                                                         \
        int r_ = (x);                                                            \
        if (r_ != PDR_OK) {                                                      \
            fprintf(stderr, "pdr error %s at %s:%d\n", pdr_splat_status_string(r_), \
                    __FILE__, __LINE__);                                         \
            return 1;                                                            \
        }                                                                        \
    } while (0)

static int read_all(FILE *f, void *p, size_t bytes) { return fread(p, 1, bytes, f) == bytes; }

int main(int argc, char **argv) {
    int dims[5];
    float radius;
    FILE *f;
    size_t np, ni;
    float *params, *gimg, *image, *gparams;
    void *d_params, *d_gimg, *d_image, *d_gparams, *ws = NULL;
    hipStream_t st;
    long long pairs, need = 0;
    int attempt, rc = PDR_ERR_OVERFLOW;
    if (argc != 3) {
        fprintf(stderr, "usage: %s input output\n", argv[0]);
        return 2;
    }
    f = fopen(argv[1], "rb");
    if (!f || !read_all(f, dims, sizeof dims) || !read_all(f, &radius, sizeof radius)) return 2;
    np = (size_t)dims[0] * dims[1] * (5 + dims[4]);
    ni = (size_t)dims[0] * dims[2] * dims[3] * dims[4];
    params = (float *)malloc(np * 4);
    gparams = (float *)malloc(np * 4);
    gimg = (float *)malloc(ni * 4);
    image = (float *)malloc(ni * 4);
    if (!params || !gparams || !gimg || !image) return 2;
    if (!read_all(f, params, np * 4) || !read_all(f, gimg, ni * 4)) return 2;
    fclose(f);

    HIPCHECK(hipStreamCreate(&st));
    HIPCHECK(hipMalloc(&d_params, np * 4));
    HIPCHECK(hipMalloc(&d_gparams, np * 4));
    HIPCHECK(hipMalloc(&d_gimg, ni * 4));
    HIPCHECK(hipMalloc(&d_image, ni * 4));
    HIPCHECK(hipMemcpy(d_params, params, np * 4, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(d_gimg, gimg, ni * 4, hipMemcpyHostToDevice));

    /* deliberately small first guess: exercises the overflow protocol */
    pairs = (long long)dims[0] * dims[1];
    for (attempt = 0; attempt < 3 && rc == PDR_ERR_OVERFLOW; ++attempt) {
        long long bytes = pdr_splat_workspace_bytes(dims[0], dims[1], dims[2], dims[3], dims[4], pairs);
        if (bytes < 0) return 1;
        if (ws) HIPCHECK(hipFree(ws));
        HIPCHECK(hipMalloc(&ws, (size_t)bytes));
        PDRCHECK(pdr_splat_forward((const float *)d_params, (float *)d_image, dims[0], dims[1],
                                   dims[2], dims[3], dims[4], radius, ws, (size_t)bytes, st));
        rc = pdr_splat_check(ws, st, &need);
        if (rc == PDR_ERR_OVERFLOW) pairs = need;
        if (rc == PDR_OK)
            rc = pdr_splat_backward((const float *)d_params, (const float *)d_gimg,
                                    (float *)d_gparams, dims[0], dims[1], dims[2], dims[3],
                                    dims[4], radius, ws, (size_t)bytes, 1, st);
    }
    PDRCHECK(rc);
    PDRCHECK(pdr_splat_check(ws, st, &need));
    HIPCHECK(hipMemcpy(image, d_image, ni * 4, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(gparams, d_gparams, np * 4, hipMemcpyDeviceToHost));

    f = fopen(argv[2], "wb");
    if (!f) return 2;
    if (fwrite(image, 4, ni, f) != ni || fwrite(gparams, 4, np, f) != np ||
        fwrite(&need, sizeof need, 1, f) != 1)
        return 2;
    fclose(f);
    HIPCHECK(hipFree(ws));
    HIPCHECK(hipFree(d_params));
    HIPCHECK(hipFree(d_gparams));
    HIPCHECK(hipFree(d_gimg));
    HIPCHECK(hipFree(d_image));
    HIPCHECK(hipStreamDestroy(st));
    free(params);
    free(gparams);
    free(gimg);
    free(image);
    printf("gpu consumer ok (%d attempts, %lld pairs)\n", attempt, need);
    return 0;
}
