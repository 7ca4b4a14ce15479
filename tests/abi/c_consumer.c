/*
 * c_consumer.c -- a plain C99 program using libgq.so through include/gq.h only (no Python,
 * no torch): the boundary is an ordinary C ABI.  Built by the repository's build step with gcc
 * against the HIP runtime; run by tests/test_gpu_c_consumer.py.
 *
 * usage: c_consumer SCALE_IN OUT
 *   SCALE_IN  3 float32: the shared scale of each segment to quantise with
 *   OUT       written: 3 float32 (this program's own gq_global_norm), n float32 (gq_fused_mean
 *             with SCALE_IN), then 3 int32: gq_read_status, the status of a call with an
 *             invalid level count, and 1 if that call left a message in gq_last_error
 * Inputs: K = 3 workers of n = 10007 fp32 elements, x_k[i] = ((i*2654435761 + k*40503) mod
 * 2001 - 1000) / 1000 computed in uint32 arithmetic; segments [0, 4096), [4096, 4104),
 * [4104, n); uniform grid s = 31, 8-bit codes, int16 sums, seed 99, counter base 5.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "gq.h"

#define K 3
#define N 10007
#define NSEG 3

static int fail(const char *what, int code)
{
    fprintf(stderr, "c_consumer: %s failed (%d)\n", what, code);
    return 1;
}

int main(int argc, char **argv)
{
    static float host_x[K][N];
    static float host_out[N];
    const int64_t offsets[NSEG + 1] = {0, 4096, 4104, N};
    float scale_in[NSEG], scale_gpu[NSEG];
    void *dx[K];
    const void *ptrs[K];
    float *dscale_in = NULL, *dscale_gpu = NULL, *dout = NULL;
    gq_ctx *ctx = NULL;
    int32_t status[3];
    FILE *f;
    int k;
    int64_t i;
    if (argc != 3)
        return fail("usage: c_consumer SCALE_IN OUT", 2);
    f = fopen(argv[1], "rb");
    if (!f || fread(scale_in, sizeof(float), NSEG, f) != NSEG)
        return fail("reading SCALE_IN", 2);
    fclose(f);
    for (k = 0; k < K; ++k)
        for (i = 0; i < N; ++i) {
            uint32_t h = (uint32_t)i * 2654435761u + (uint32_t)k * 40503u;
            host_x[k][i] = ((float)(h % 2001u) - 1000.0f) / 1000.0f;
        }
    for (k = 0; k < K; ++k) {
        if (hipMalloc(&dx[k], sizeof host_x[k]) != hipSuccess)
            return fail("hipMalloc", 0);
        if (hipMemcpy(dx[k], host_x[k], sizeof host_x[k], hipMemcpyHostToDevice) != hipSuccess)
            return fail("hipMemcpy", 0);
        ptrs[k] = dx[k];
    }
    if (hipMalloc((void **)&dscale_in, 256) != hipSuccess ||
        hipMalloc((void **)&dscale_gpu, 256) != hipSuccess ||
        hipMalloc((void **)&dout, sizeof host_out) != hipSuccess)
        return fail("hipMalloc", 0);
    if (hipMemcpy(dscale_in, scale_in, sizeof scale_in, hipMemcpyHostToDevice) != hipSuccess)
        return fail("hipMemcpy", 0);
    if (gq_create(&ctx) != GQ_OK)
        return fail("gq_create", 0);
    k = gq_global_norm(ctx, ptrs, K, GQ_F32, N, offsets, NSEG, dscale_gpu, NULL, NULL);
    if (k != GQ_OK)
        return fail(gq_last_error(ctx), k);
    k = gq_fused_mean(ctx, ptrs, K, GQ_F32, N, offsets, NSEG, dscale_in, GQ_UNIFORM, 31, 8, 99u,
                      5u, 16, NULL, NULL, GQ_F32, dout, NULL);
    if (k != GQ_OK)
        return fail(gq_last_error(ctx), k);
    status[0] = gq_read_status(ctx, NULL);
    status[1] = gq_fused_mean(ctx, ptrs, K, GQ_F32, N, offsets, NSEG, dscale_in, GQ_UNIFORM, 200,
                              8, 99u, 5u, 16, NULL, NULL, GQ_F32, dout, NULL);
    status[2] = gq_last_error(ctx)[0] != '\0';
    if (hipMemcpy(scale_gpu, dscale_gpu, sizeof scale_gpu, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(host_out, dout, sizeof host_out, hipMemcpyDeviceToHost) != hipSuccess)
        return fail("hipMemcpy", 0);
    gq_destroy(ctx);
    for (k = 0; k < K; ++k)
        hipFree(dx[k]);
    hipFree(dscale_in);
    hipFree(dscale_gpu);
    hipFree(dout);
    f = fopen(argv[2], "wb");
    if (!f || fwrite(scale_gpu, sizeof(float), NSEG, f) != NSEG ||
        fwrite(host_out, sizeof(float), N, f) != N || fwrite(status, sizeof(int32_t), 3, f) != 3)
        return fail("writing OUT", 2);
    fclose(f);
    printf("c_consumer ok\n");
    return 0;
}
