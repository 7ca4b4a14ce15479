/*
 * c_consumer.c -- a plain C99 program using libgq.so through include/gq.h only (no Python,
 * no torch): the boundary is an ordinary C ABI.  Built by the repository's build step with gcc
 * against the HIP runtime; run by tests/test_gpu_c_consumer.py.
 *
 * usage: c_consumer SCALE_IN OUT
 *   SCALE_IN  3 float32: the shared scale of each segment to quantise with
 *   OUT       written: 3 float32 (this program's own gq_global_norm), n float32 (gq_fused_mean
 *             with SCALE_IN), then 3 int32: gq_read_status, the status of a call with an
 *             invalid level count, and 1 if that call left a message in gq_last_error; then
 *             n float32: the same mean step by step (gq_quantize_pack for every worker,
 *             gq_accumulate_codes, gq_dequantize); then one gq_powersgd_logquant step:
 *             p_codes (LN x LR int8), p_colmax (LR float32), q_codes (LM x LR int8),
 *             q_colmax (LR float32), E after the step (LN x LM float32), Q after (LM x LR).
 * Inputs: K = 3 workers of n = 10007 fp32 elements, x_k[i] = ((i*2654435761 + k*40503) mod
 * 2001 - 1000) / 1000 computed in uint32 arithmetic; segments [0, 4096), [4096, 4104),
 * [4104, n); uniform grid s = 31, 8-bit codes, int16 sums, seed 99, counter base 5.
 * LQ-SGD: G[i][j] = ((t*2654435761 + 12345) mod 2001 - 1000) / 1000 * 0.001 with t = i*LM + j,
 * E = 0, Q[j][c] = ((u*40503 + 777) mod 2001 - 1000) / 1000 with u = j*LR + c; alpha = 10,
 * 8-bit codes for P and 6-bit codes for Q'.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "gq.h"

#define K 3
#define N 10007
#define NSEG 3
#define LN 96
#define LM 72
#define LR 3

static int fail(const char *what, int code)
{
    fprintf(stderr, "c_consumer: %s failed (%d)\n", what, code);
    return 1;
}

int main(int argc, char **argv)
{
    static float host_x[K][N];
    static float host_out[N], host_out2[N];
    static float host_g[LN * LM], host_e[LN * LM], host_q[LM * LR];
    static int8_t host_pc[LN * LR], host_qc[LM * LR];
    float host_pm[LR], host_qm[LR];
    void *dcodes[K];
    const uint8_t *cptrs[K];
    void *dsums = NULL, *dout2 = NULL;
    float *dg = NULL, *de = NULL, *dq = NULL, *dpm = NULL, *dqm = NULL;
    int8_t *dpc = NULL, *dqc = NULL;
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
    /* the same mean step by step: every worker's codes, their integer sum, the decode */
    for (k = 0; k < K; ++k) {
        if (hipMalloc(&dcodes[k], N) != hipSuccess)
            return fail("hipMalloc", 0);
        cptrs[k] = (const uint8_t *)dcodes[k];
    }
    if (hipMalloc(&dsums, N * sizeof(int16_t)) != hipSuccess ||
        hipMalloc(&dout2, sizeof host_out2) != hipSuccess)
        return fail("hipMalloc", 0);
    for (k = 0; k < K; ++k) {
        int st = gq_quantize_pack(ctx, ptrs[k], GQ_F32, N, offsets, NSEG, dscale_in, GQ_UNIFORM,
                                  31, 8, 99u, (uint32_t)k, 5u, (uint8_t *)dcodes[k], NULL);
        if (st != GQ_OK)
            return fail(gq_last_error(ctx), st);
    }
    k = gq_accumulate_codes(ctx, cptrs, K, N, GQ_UNIFORM, 31, 8, 16, dsums, NULL);
    if (k != GQ_OK)
        return fail(gq_last_error(ctx), k);
    k = gq_dequantize(ctx, dsums, 16, N, offsets, NSEG, dscale_in, GQ_UNIFORM, 31, K, GQ_F32,
                      dout2, NULL);
    if (k != GQ_OK)
        return fail(gq_last_error(ctx), k);
    /* one LQ-SGD compressor step */
    for (i = 0; i < LN * LM; ++i) {
        uint32_t h = (uint32_t)i * 2654435761u + 12345u;
        host_g[i] = ((float)(h % 2001u) - 1000.0f) / 1000.0f * 0.001f;
        host_e[i] = 0.0f;
    }
    for (i = 0; i < LM * LR; ++i) {
        uint32_t h = (uint32_t)i * 40503u + 777u;
        host_q[i] = ((float)(h % 2001u) - 1000.0f) / 1000.0f;
    }
    if (hipMalloc((void **)&dg, sizeof host_g) != hipSuccess ||
        hipMalloc((void **)&de, sizeof host_e) != hipSuccess ||
        hipMalloc((void **)&dq, sizeof host_q) != hipSuccess ||
        hipMalloc((void **)&dpc, sizeof host_pc) != hipSuccess ||
        hipMalloc((void **)&dqc, sizeof host_qc) != hipSuccess ||
        hipMalloc((void **)&dpm, 256) != hipSuccess || hipMalloc((void **)&dqm, 256) != hipSuccess)
        return fail("hipMalloc", 0);
    if (hipMemcpy(dg, host_g, sizeof host_g, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(de, host_e, sizeof host_e, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(dq, host_q, sizeof host_q, hipMemcpyHostToDevice) != hipSuccess)
        return fail("hipMemcpy", 0);
    k = gq_powersgd_logquant(ctx, dg, de, dq, LN, LM, LR, 10.0, 8, 6, dpc, dpm, dqc, dqm, NULL,
                             NULL, NULL, NULL);
    if (k != GQ_OK)
        return fail(gq_last_error(ctx), k);
    if (hipMemcpy(host_out2, dout2, sizeof host_out2, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(host_pc, dpc, sizeof host_pc, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(host_qc, dqc, sizeof host_qc, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(host_pm, dpm, sizeof host_pm, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(host_qm, dqm, sizeof host_qm, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(host_e, de, sizeof host_e, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(host_q, dq, sizeof host_q, hipMemcpyDeviceToHost) != hipSuccess)
        return fail("hipMemcpy", 0);
    if (hipMemcpy(scale_gpu, dscale_gpu, sizeof scale_gpu, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(host_out, dout, sizeof host_out, hipMemcpyDeviceToHost) != hipSuccess)
        return fail("hipMemcpy", 0);
    gq_destroy(ctx);
    for (k = 0; k < K; ++k) {
        hipFree(dx[k]);
        hipFree(dcodes[k]);
    }
    hipFree(dscale_in);
    hipFree(dscale_gpu);
    hipFree(dout);
    hipFree(dsums);
    hipFree(dout2);
    hipFree(dg);
    hipFree(de);
    hipFree(dq);
    hipFree(dpc);
    hipFree(dqc);
    hipFree(dpm);
    hipFree(dqm);
    f = fopen(argv[2], "wb");
    if (!f || fwrite(scale_gpu, sizeof(float), NSEG, f) != NSEG ||
        fwrite(host_out, sizeof(float), N, f) != N || fwrite(status, sizeof(int32_t), 3, f) != 3 ||
        fwrite(host_out2, sizeof(float), N, f) != N ||
        fwrite(host_pc, 1, sizeof host_pc, f) != sizeof host_pc ||
        fwrite(host_pm, sizeof(float), LR, f) != LR ||
        fwrite(host_qc, 1, sizeof host_qc, f) != sizeof host_qc ||
        fwrite(host_qm, sizeof(float), LR, f) != LR ||
        fwrite(host_e, sizeof(float), LN * LM, f) != LN * LM ||
        fwrite(host_q, sizeof(float), LM * LR, f) != LM * LR)
        return fail("writing OUT", 2);
    fclose(f);
    printf("c_consumer ok\n");
    return 0;
}
