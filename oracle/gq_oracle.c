/*
 * gq_oracle.c -- plain, slow, obviously-correct CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the CPU-baseline leg of
 * the benchmark; never by the product library, with which it shares no code.
 *
 * Built with gcc -O2 -ffp-contract=off (no fast-math): every fp32 operation below is one
 * IEEE operation with round-to-nearest-even, fp64 where the comment says so.  Loops are in
 * index order; nothing is blocked, fused or reordered.  The page citations of each step are
 * in gq_oracle.h beside its declaration and repeated here where a reading was needed.
 */
#include "gq_oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ======================= random numbers ======================= */

/* SplitMix64 as published by Steele, Lea & Flood (OOPSLA 2014): the state advances by the
 * golden-ratio increment and the output is the mixed state. */
uint64_t orc_splitmix64_next(uint64_t *state)
{
    uint64_t z;
    *state += 0x9E3779B97F4A7C15ULL;
    z = *state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* MurmurHash3's 32-bit finaliser (Appleby, public domain). */
uint32_t orc_fmix32(uint32_t h)
{
    h ^= h >> 16;
    h *= 0x85EBCA6BU;
    h ^= h >> 13;
    h *= 0xC2B2AE35U;
    h ^= h >> 16;
    return h;
}

/* Worker k draws from its own stream: its key is output k+1 of SplitMix64 seeded with the
 * step seed, truncated to 32 bits. */
uint32_t orc_worker_key(uint64_t seed, uint32_t worker)
{
    uint64_t state = seed, z = 0;
    uint32_t j;
    for (j = 0; j <= worker; ++j)
        z = orc_splitmix64_next(&state);
    return (uint32_t)z;
}

/* The draw as an fp32 program makes it: the 32-bit hash rounded to the nearest fp32 (ties to
 * even: C's conversion under the default rounding mode), then scaled by 2^-32 (exact), so that
 * it has the precision of the fp32 probability p it is compared with.  Values within 128 of
 * 2^32 round to 1.0, which no p < 1 exceeds. */
double orc_uniform(uint32_t key, uint32_t counter)
{
    const float h = (float)orc_fmix32(counter ^ key);
    return (double)h * 0x1p-32;
}

void orc_hash_fill(uint32_t key, uint32_t counter0, int64_t cnt, uint32_t *out)
{
    int64_t t;
    for (t = 0; t < cnt; ++t)
        out[t] = orc_fmix32((counter0 + (uint32_t)t) ^ key);
}

/* ======================= global norm ======================= */

static float bf16_bits_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

double orc_load(const void *x, int32_t dtype, int64_t i)
{
    if (dtype == ORC_BF16)
        return (double)bf16_bits_to_f32(((const uint16_t *)x)[i]);
    return (double)((const float *)x)[i];
}

double orc_sumsq(const void *x, int32_t dtype, int64_t n, double acc)
{
    int64_t i;
    for (i = 0; i < n; ++i) {
        double v = orc_load(x, dtype, i);
        acc += v * v; /* v*v is exact in fp64: a 24-bit mantissa squared fits in 53 bits */
    }
    return acc;
}

/* [GQ] abstract: one global norm scales all workers.  Reading: the shared scale of segment g
 * is the largest per-worker L2 norm, so that |x_{k,i}| <= S_g for every worker k.
 * sumsq[k*nseg + g] holds worker k's sum of squares over segment g. */
int32_t orc_norm_finish(const double *sumsq, int32_t K, int32_t nseg, float *scale_out,
                        double *norms_out)
{
    int32_t g, k, bad = 0;
    for (g = 0; g < nseg; ++g) {
        double best = 0.0;
        int nonfinite = 0;
        for (k = 0; k < K; ++k) {
            double nrm = sqrt(sumsq[(int64_t)k * nseg + g]);
            if (norms_out)
                norms_out[(int64_t)k * nseg + g] = nrm;
            if (!isfinite(nrm))
                nonfinite = 1;
            else if (nrm > best)
                best = nrm;
        }
        {
            float S = (float)best;
            if (nonfinite || !isfinite(S)) {
                S = 0.0f;
                bad = 1;
            }
            scale_out[g] = S;
        }
    }
    return bad;
}

int32_t orc_global_norm(const void *const *xs, int32_t K, int32_t dtype, int64_t n,
                        const int64_t *offsets, int32_t nseg, float *scale_out,
                        double *norms_out)
{
    int32_t g, k, bad;
    size_t esz = dtype == ORC_BF16 ? 2 : 4;
    double *ss = (double *)malloc(sizeof(double) * (size_t)K * (size_t)(nseg > 0 ? nseg : 1));
    (void)n;
    for (g = 0; g < nseg; ++g) {
        int64_t lo = offsets[g], hi = offsets[g + 1];
        for (k = 0; k < K; ++k) {
            const char *base = (const char *)xs[k] + (size_t)lo * esz;
            ss[(int64_t)k * nseg + g] = orc_sumsq(base, dtype, hi - lo, 0.0);
        }
    }
    bad = orc_norm_finish(ss, K, nseg, scale_out, norms_out);
    free(ss);
    return bad;
}

/* ======================= quantisation ======================= */

/* A scale is usable when it is a positive finite fp32 whose reciprocal scale factor is
 * finite too; otherwise the whole segment maps to zero ("zero maps to zero"). */

/* Uniform grid (QSGD family, [USM] title and [NUQ] abstract: unbiased stochastic rounding
 * between the two neighbouring of s+1 equally spaced levels of |x|/S). */
static int32_t quant_uniform(int32_t s, float x, float S, uint32_t key, uint32_t counter)
{
    float inv, u;
    double l, p, r;
    int32_t m;
    if (!(S > 0.0f) || !(S <= FLT_MAX))
        return 0;
    inv = (float)s / S; /* fp32 division, correctly rounded */
    if (!(inv <= FLT_MAX))
        return 0;
    u = fabsf(x) * inv;          /* one fp32 multiply */
    if (!(u < (float)s))         /* u >= s (rounding at |x| = S) and NaN go to the top level */
        u = (float)s;
    l = floor((double)u);
    p = (double)u - l;           /* exact */
    r = orc_uniform(key, counter);
    m = (int32_t)l + (r < p ? 1 : 0);
    return signbit(x) ? -m : m; /* a NaN keeps the sign its sign bit gives it */
}

/* Exponential grid ([NUQ] abstract: nonuniform levels).  Levels of |x|/S are 0 and 2^(j-E)
 * for j = 1..E; stochastic rounding between the two neighbours keeps E[level] = |x|/S. */
static int32_t quant_exp(int32_t E, float x, float S, uint32_t key, uint32_t counter)
{
    float inv, u;
    double lo, hi, p, r;
    int32_t j, t;
    if (!(S > 0.0f) || !(S <= FLT_MAX))
        return 0;
    inv = 1.0f / S;
    if (!(inv <= FLT_MAX))
        return 0;
    u = fabsf(x) * inv;
    if (!(u < 1.0f))
        u = 1.0f;
    /* the largest level not above u */
    j = 0;
    for (t = 1; t <= E; ++t)
        if (ldexp(1.0, t - E) <= (double)u)
            j = t;
    if (j == E) {
        p = 0.0;
    } else {
        lo = j == 0 ? 0.0 : ldexp(1.0, j - E);
        hi = ldexp(1.0, j + 1 - E);
        p = ((double)u - lo) / (hi - lo); /* exact: the gap is a power of two */
    }
    r = orc_uniform(key, counter);
    if (r < p)
        j += 1;
    return (signbit(x) && j > 0) ? -j : j; /* the sign bit, as on the uniform grid */
}

int32_t orc_quant_one(int32_t grid, int32_t levels, float x, float S, uint32_t key,
                      uint32_t counter)
{
    if (grid == ORC_EXP)
        return quant_exp(levels, x, S, key, counter);
    return quant_uniform(levels, x, S, key, counter);
}

void orc_quantize(const void *x, int32_t dtype, int64_t n, const int64_t *offsets,
                  int32_t nseg, const float *scale, int32_t grid, int32_t levels,
                  uint64_t seed, uint32_t worker, uint32_t index_base, int32_t *levels_out)
{
    uint32_t key = orc_worker_key(seed, worker);
    int32_t g;
    int64_t i;
    (void)n;
    for (g = 0; g < nseg; ++g)
        for (i = offsets[g]; i < offsets[g + 1]; ++i)
            levels_out[i] = orc_quant_one(grid, levels, (float)orc_load(x, dtype, i),
                                          scale[g], key, index_base + (uint32_t)i);
}

void orc_quantize_list(const float *x, const float *S, const uint32_t *counter, int64_t cnt,
                       int32_t grid, int32_t levels, uint32_t key, int32_t *levels_out)
{
    int64_t t;
    for (t = 0; t < cnt; ++t)
        levels_out[t] = orc_quant_one(grid, levels, x[t], S[t], key, counter[t]);
}

/* ======================= codes ======================= */

/* [LQ] "Core claim": the message carries each value as its bin number in b bits.  Uniform
 * levels are stored in two's complement; exponential levels as a sign bit above the index j. */
static uint32_t encode_level(int32_t grid, int32_t bits, int32_t q)
{
    uint32_t mask = (1u << bits) - 1u;
    if (grid == ORC_EXP) {
        uint32_t j = (uint32_t)(q < 0 ? -q : q);
        uint32_t sign = q < 0 ? 1u : 0u;
        return (sign << (bits - 1)) | j;
    }
    return (uint32_t)q & mask;
}

void orc_pack(const int32_t *q, int64_t n, int32_t grid, int32_t bits, uint8_t *out)
{
    int64_t i;
    if (bits == 8) {
        for (i = 0; i < n; ++i)
            out[i] = (uint8_t)encode_level(grid, 8, q[i]);
        return;
    }
    memset(out, 0, (size_t)((n + 1) / 2));
    for (i = 0; i < n; ++i) {
        uint32_t c = encode_level(grid, 4, q[i]);
        if (i % 2 == 0)
            out[i / 2] = (uint8_t)(out[i / 2] | c);
        else
            out[i / 2] = (uint8_t)(out[i / 2] | (c << 4));
    }
}

int32_t orc_unpack_one(const uint8_t *codes, int64_t i, int32_t grid, int32_t bits)
{
    uint32_t c;
    if (bits == 8)
        c = codes[i];
    else
        c = (i % 2 == 0) ? (codes[i / 2] & 0xFu) : (codes[i / 2] >> 4);
    if (grid == ORC_EXP) {
        int32_t j = (int32_t)(c & ((1u << (bits - 1)) - 1u));
        return (c >> (bits - 1)) ? -j : j;
    }
    /* sign-extend a bits-wide two's-complement value */
    if (c & (1u << (bits - 1)))
        return (int32_t)c - (int32_t)(1u << bits);
    return (int32_t)c;
}

/* [GQ] abstract: Allreduce-compatibility.  Exponential levels become integers on the grid of
 * the smallest level 2^(1-E): level j -> 2^(j-1); then the sum is exact in integers. */
int64_t orc_lin(int32_t grid, int32_t q)
{
    if (grid == ORC_EXP) {
        int32_t j = q < 0 ? -q : q;
        int64_t v = j == 0 ? 0 : ((int64_t)1 << (j - 1));
        return q < 0 ? -v : v;
    }
    return q;
}

int64_t orc_accumulate(const uint8_t *const *codes, int32_t K, int64_t n, int32_t grid,
                       int32_t bits, int32_t acc_bits, void *sums)
{
    int64_t i, over = 0;
    int64_t lim = acc_bits == 16 ? 32767 : 2147483647LL;
    for (i = 0; i < n; ++i) {
        int64_t acc = 0;
        int32_t k;
        for (k = 0; k < K; ++k)
            acc += orc_lin(grid, orc_unpack_one(codes[k], i, grid, bits));
        if (acc > lim || acc < -lim - 1)
            ++over;
        if (acc_bits == 16)
            ((int16_t *)sums)[i] = (int16_t)acc;
        else
            ((int32_t *)sums)[i] = (int32_t)acc;
    }
    return over;
}

/* ======================= summable wire payload ======================= */

static int64_t wire_offset(int32_t grid, int32_t levels)
{
    return grid == ORC_EXP ? ((int64_t)1 << (levels - 1)) : (int64_t)levels;
}

int32_t orc_wire_lane_bytes(int32_t grid, int32_t levels, int32_t world)
{
    int64_t top = (int64_t)world * 2 * wire_offset(grid, levels);
    int32_t w;
    for (w = 1; w <= 4; w *= 2)
        if (top <= (int64_t)(((uint64_t)1 << (8 * w)) - 1))
            return w;
    return 0;
}

void orc_wire_encode(const int32_t *q, int64_t n, int32_t grid, int32_t levels, int32_t world,
                     uint8_t *payload)
{
    int32_t w = orc_wire_lane_bytes(grid, levels, world), b;
    int64_t o = wire_offset(grid, levels), i, nbytes = (n * w + 3) / 4 * 4;
    memset(payload, 0, (size_t)nbytes);
    for (i = 0; i < n; ++i) {
        uint64_t lane = (uint64_t)(orc_lin(grid, q[i]) + o);
        for (b = 0; b < w; ++b)
            payload[i * w + b] = (uint8_t)(lane >> (8 * b));
    }
}

void orc_wire_sum(const uint8_t *const *payloads, int32_t K, int64_t nbytes, uint8_t *out)
{
    int64_t t;
    int32_t k, b;
    for (t = 0; t < nbytes / 4; ++t) {
        uint32_t acc = 0;
        for (k = 0; k < K; ++k) {
            uint32_t word = 0;
            for (b = 0; b < 4; ++b)
                word |= (uint32_t)payloads[k][4 * t + b] << (8 * b);
            acc += word; /* wraps mod 2^32, as an unsigned 32-bit sum does */
        }
        for (b = 0; b < 4; ++b)
            out[4 * t + b] = (uint8_t)(acc >> (8 * b));
    }
}

void orc_wire_decode(const uint8_t *payload, int64_t n, int32_t grid, int32_t levels,
                     int32_t world, int32_t *sums)
{
    int32_t w = orc_wire_lane_bytes(grid, levels, world), b;
    int64_t o = wire_offset(grid, levels), i;
    for (i = 0; i < n; ++i) {
        uint64_t lane = 0;
        for (b = 0; b < w; ++b)
            lane |= (uint64_t)payload[i * w + b] << (8 * b);
        sums[i] = (int32_t)((int64_t)lane - (int64_t)world * o);
    }
}

/* ======================= decode ======================= */

float orc_decode_factor(int32_t grid, int32_t levels, int32_t K, float S)
{
    double D;
    if (!(S > 0.0f) || !(S <= FLT_MAX))
        return 0.0f;
    if (grid == ORC_EXP)
        D = (double)K * ldexp(1.0, levels - 1);
    else
        D = (double)levels * (double)K;
    return (float)((double)S / D);
}

static double bf16_value(uint32_t bits16)
{
    if ((bits16 & 0x7FFFu) == 0x7F80u) /* the step above the largest finite bf16 */
        return (bits16 & 0x8000u) ? -0x1p128 : 0x1p128;
    return (double)bf16_bits_to_f32((uint16_t)bits16);
}

uint16_t orc_f32_to_bf16(float v)
{
    uint32_t u, lo, hi;
    double dl, dh, dv;
    memcpy(&u, &v, sizeof u);
    if (isnan(v))
        return (uint16_t)((u >> 16) | 0x40u);
    lo = u >> 16;                     /* truncation toward zero */
    if ((u & 0xFFFFu) == 0)
        return (uint16_t)lo;          /* exactly representable */
    hi = lo + 1;                      /* next bf16 away from zero */
    dv = fabs((double)v);
    dl = fabs(bf16_value(lo));
    dh = fabs(bf16_value(hi));
    if (dv - dl < dh - dv)
        return (uint16_t)lo;
    if (dv - dl > dh - dv)
        return (uint16_t)hi;
    return (uint16_t)((lo & 1u) ? hi : lo); /* tie: even mantissa */
}

void orc_dequantize(const void *sums, int32_t acc_bits, int64_t n, const int64_t *offsets,
                    int32_t nseg, const float *scale, int32_t grid, int32_t levels, int32_t K,
                    int32_t out_dtype, void *out)
{
    int32_t g;
    int64_t i;
    (void)n;
    for (g = 0; g < nseg; ++g) {
        float f = orc_decode_factor(grid, levels, K, scale[g]);
        for (i = offsets[g]; i < offsets[g + 1]; ++i) {
            int64_t s = acc_bits == 16 ? ((const int16_t *)sums)[i] : ((const int32_t *)sums)[i];
            float mean = (float)s * f;
            if (out_dtype == ORC_BF16)
                ((uint16_t *)out)[i] = orc_f32_to_bf16(mean);
            else
                ((float *)out)[i] = mean;
        }
    }
}

/* ======================= baselines: per-worker scales ======================= */

/* [NUQ] abstract: QSGD normalises each worker's vector by its own L2 norm; QSGDinf (named
 * there, not defined) is read as normalisation by the largest magnitude. */
int32_t orc_worker_scales(const void *const *xs, int32_t K, int32_t dtype, int64_t n,
                          const int64_t *offsets, int32_t nseg, int32_t norm,
                          float *scales_out)
{
    int32_t g, k, bad = 0;
    int64_t i;
    (void)n;
    for (k = 0; k < K; ++k)
        for (g = 0; g < nseg; ++g) {
            double v = 0.0;
            float S;
            if (norm == ORC_NORM_MAX) {
                for (i = offsets[g]; i < offsets[g + 1]; ++i) {
                    double a = fabs(orc_load(xs[k], dtype, i));
                    if (isnan(a) || isnan(v))
                        v = NAN; /* a NaN anywhere makes the scale non-finite */
                    else if (a > v)
                        v = a;
                }
            } else {
                for (i = offsets[g]; i < offsets[g + 1]; ++i) {
                    double x = orc_load(xs[k], dtype, i);
                    v += x * x; /* exact square, index order */
                }
                v = sqrt(v);
            }
            S = (float)v;
            if (!isfinite(v) || !isfinite(S)) {
                S = 0.0f;
                bad = 1;
            }
            scales_out[(int64_t)k * nseg + g] = S;
        }
    return bad;
}

void orc_worker_mean(const void *const *xs, int32_t K, int32_t dtype, int64_t n,
                     const int64_t *offsets, int32_t nseg, const float *scales, int32_t grid,
                     int32_t levels, uint64_t seed, uint32_t index_base, int32_t out_dtype,
                     void *out)
{
    int32_t g, k;
    int64_t i;
    uint32_t *keys = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(K > 0 ? K : 1));
    (void)n;
    for (k = 0; k < K; ++k)
        keys[k] = orc_worker_key(seed, (uint32_t)k);
    for (g = 0; g < nseg; ++g)
        for (i = offsets[g]; i < offsets[g + 1]; ++i) {
            float acc = 0.0f;
            for (k = 0; k < K; ++k) {
                float S = scales[(int64_t)k * nseg + g];
                float f = orc_decode_factor(grid, levels, K, S);
                int32_t q = orc_quant_one(grid, levels, (float)orc_load(xs[k], dtype, i), S,
                                          keys[k], index_base + (uint32_t)i);
                acc = fmaf((float)orc_lin(grid, q), f, acc);
            }
            if (out_dtype == ORC_BF16)
                ((uint16_t *)out)[i] = orc_f32_to_bf16(acc);
            else
                ((float *)out)[i] = acc;
        }
    free(keys);
}

void orc_decode_workers(const uint8_t *const *codes, int32_t K, int64_t n,
                        const int64_t *offsets, int32_t nseg, const float *scales, int32_t grid,
                        int32_t levels, int32_t bits, int32_t out_dtype, void *out)
{
    int32_t g, k;
    int64_t i;
    (void)n;
    for (g = 0; g < nseg; ++g)
        for (i = offsets[g]; i < offsets[g + 1]; ++i) {
            float acc = 0.0f;
            for (k = 0; k < K; ++k) {
                float f = orc_decode_factor(grid, levels, K, scales[(int64_t)k * nseg + g]);
                int32_t q = orc_unpack_one(codes[k], i, grid, bits);
                acc = fmaf((float)orc_lin(grid, q), f, acc);
            }
            if (out_dtype == ORC_BF16)
                ((uint16_t *)out)[i] = orc_f32_to_bf16(acc);
            else
                ((float *)out)[i] = acc;
        }
}

/* ======================= LQ-SGD ======================= */

/* [LQ] "Core claim" Eq. (5) q(y) = log(1 + alpha y) / log(1 + alpha) on y = |F| / max|column|
 * (the normalisation asked for in referee major comment 1), then the nearest of the 2L+1
 * equally spaced values k/L of q, ties up.  Evaluated in fp64 straight from the formula. */
int32_t orc_logq_index(float y, double alpha, int32_t L)
{
    double z = log1p(alpha * (double)y) / log1p(alpha);
    double k = floor(z * (double)L + 0.5);
    if (k < 0.0)
        k = 0.0;
    if (k > (double)L)
        k = (double)L;
    return (int32_t)k;
}

/* [LQ] referee major comment 1, Eq. (6): the inverse map |y| = ((1 + alpha)^z - 1) / alpha. */
float orc_logq_level(int32_t k, double alpha, int32_t L)
{
    return (float)((pow(1.0 + alpha, (double)k / (double)L) - 1.0) / alpha);
}

void orc_logquant(const float *F, int64_t rows, int32_t r, double alpha, int32_t bits,
                  int8_t *codes, float *colmax, float *Fhat)
{
    int32_t L = (1 << (bits - 1)) - 1;
    int32_t c;
    int64_t i;
    for (c = 0; c < r; ++c) {
        float mx = 0.0f;
        for (i = 0; i < rows; ++i) {
            float a = fabsf(F[i * r + c]);
            if (a > mx)
                mx = a;
        }
        colmax[c] = mx;
        for (i = 0; i < rows; ++i) {
            float x = F[i * r + c];
            int32_t k = 0;
            if (mx > 0.0f) {
                float y = fabsf(x) / mx; /* fp32 division, in [0, 1] */
                k = orc_logq_index(y, alpha, L);
            }
            codes[i * r + c] = (int8_t)(x < 0.0f ? -k : k);
            if (Fhat) {
                float v = orc_logq_level(k, alpha, L) * mx; /* one fp32 multiply */
                Fhat[i * r + c] = x < 0.0f ? -v : v;
            }
        }
    }
}

/* [LQ] referee major comment 1: Q is computed from P after P is orthonormalised.  Modified
 * Gram-Schmidt over columns 0..r-1 in order, all arithmetic in fp64.
 *
 * The pages give no rule for a column that depends on the earlier ones.  Reading, from fp32
 * arithmetic alone: column c keeps, after the projections, the part p_c - sum_j a_j p_j with
 * a the coefficients of its projection on the earlier columns (a = R^-1 times column c of
 * R, over the live earlier columns).  If every column were moved by a relative amount rho
 * through rounding, that part would move by at most rho (|p_c| + sum_j |a_j| |p_j|) (triangle
 * inequality), so a column exactly dependent in exact arithmetic can keep that much.  Each
 * entry of P = M Q_prev is a sum of m products of fp32 values, whose rounding is of relative
 * size sqrt(m) u for mixed signs (u = 2^-24, fp32's unit roundoff); so rho = sqrt(m) u, and a
 * column whose remaining norm is at most rho (|p_c| + sum_j |a_j| |p_j|) has no direction of
 * its own that fp32 resolves: it is set to zero like a column with no norm at all. */
double orc_mgs_rho(int64_t m)
{
    return sqrt((double)m) * 0x1p-24;
}

void orc_mgs(float *P, int64_t n, int32_t r, int64_t m)
{
    double *V = (double *)malloc((size_t)(n * r) * sizeof(double));
    double R[8][8], nrm0[8], a[8];
    const double rho = orc_mgs_rho(m);
    int32_t c, j, k;
    int64_t i;
    for (i = 0; i < n * r; ++i)
        V[i] = (double)P[i];
    for (c = 0; c < r; ++c) {
        double nrm = 0.0, bound;
        for (j = 0; j < r; ++j)
            R[j][c] = 0.0;
        nrm0[c] = 0.0;
        for (i = 0; i < n; ++i)
            nrm0[c] += V[i * r + c] * V[i * r + c];
        nrm0[c] = sqrt(nrm0[c]);
        for (j = 0; j < c; ++j) {
            double d = 0.0;
            for (i = 0; i < n; ++i)
                d += V[i * r + j] * V[i * r + c];
            for (i = 0; i < n; ++i)
                V[i * r + c] -= d * V[i * r + j];
            R[j][c] = d;
        }
        for (i = 0; i < n; ++i)
            nrm += V[i * r + c] * V[i * r + c];
        nrm = sqrt(nrm);
        /* a = R[<c][<c]^-1 R[<c][c] by back substitution; a dead column (R[j][j] = 0) has
         * a zero row in R and takes no part */
        bound = nrm0[c];
        for (j = c - 1; j >= 0; --j) {
            a[j] = 0.0;
            if (R[j][j] > 0.0) {
                double t = R[j][c];
                for (k = j + 1; k < c; ++k)
                    t -= R[j][k] * a[k];
                a[j] = t / R[j][j];
            }
            bound += fabs(a[j]) * nrm0[j];
        }
        if (!(nrm > rho * bound))
            nrm = 0.0;
        R[c][c] = nrm;
        for (i = 0; i < n; ++i)
            V[i * r + c] = nrm > 0.0 ? V[i * r + c] / nrm : 0.0;
    }
    for (i = 0; i < n * r; ++i)
        P[i] = (float)V[i];
    free(V);
}

/* [LQ] "Core claim": one worker's compressor.  M = G + E is left in E; P = M Q_prev is
 * orthonormalised; Q' = M^T P; both factors are log-quantised (codes and maxima are the
 * worker's message, Ph and Qh their decoded values); Q <- Qh, the decoded Q, starts the next
 * step's power iteration (the warm start of the "Core claim"). */
static void lq_compress(const float *G, float *E, float *Q, int64_t n, int64_t m, int32_t r,
                        double alpha, int32_t bits_p, int32_t bits_q, int8_t *p_codes,
                        float *p_colmax, int8_t *q_codes, float *q_colmax, float *Ph, float *Qh,
                        float *P_pre, float *Q_pre)
{
    float *P = (float *)malloc((size_t)(n * r) * sizeof(float));
    float *Qn = (float *)malloc((size_t)(m * r) * sizeof(float));
    double *Qacc = (double *)malloc((size_t)(m * r) * sizeof(double));
    int64_t i, j;
    int32_t c;

    /* G' = G + E, the gradient with the previous error fed back (fp32, stored in E) */
    for (i = 0; i < n * m; ++i)
        E[i] = G[i] + E[i];

    /* P = M Q_prev (fp64 accumulation, one rounding to fp32) */
    for (i = 0; i < n; ++i)
        for (c = 0; c < r; ++c) {
            double acc = 0.0;
            for (j = 0; j < m; ++j)
                acc += (double)E[i * m + j] * (double)Q[j * r + c];
            P[i * r + c] = (float)acc;
        }
    orc_mgs(P, n, r, m);

    /* Q = M^T P: every Q[j][c] sums over i = 0..n-1 in order (rows outermost so that M is
     * read along its rows) */
    for (j = 0; j < m * r; ++j)
        Qacc[j] = 0.0;
    for (i = 0; i < n; ++i)
        for (j = 0; j < m; ++j)
            for (c = 0; c < r; ++c)
                Qacc[j * r + c] += (double)E[i * m + j] * (double)P[i * r + c];
    for (j = 0; j < m * r; ++j)
        Qn[j] = (float)Qacc[j];
    if (P_pre)
        memcpy(P_pre, P, (size_t)(n * r) * sizeof(float));
    if (Q_pre)
        memcpy(Q_pre, Qn, (size_t)(m * r) * sizeof(float));

    orc_logquant(P, n, r, alpha, bits_p, p_codes, p_colmax, Ph);
    orc_logquant(Qn, m, r, alpha, bits_q, q_codes, q_colmax, Qh);
    memcpy(Q, Qh, (size_t)(m * r) * sizeof(float));
    free(P);
    free(Qn);
    free(Qacc);
}

/* [LQ] "What carries the argument": G ~ P Q^T with error feedback E_t = G'_t - Ghat_t.
 * One worker, one power step: the compressor above, then E = M - Phat Qhat^T. */
void orc_powersgd_logquant(const float *G, float *E, float *Q, int64_t n, int64_t m,
                           int32_t r, double alpha, int32_t bits_p, int32_t bits_q,
                           int8_t *p_codes,
                           float *p_colmax, int8_t *q_codes, float *q_colmax, float *p_hat,
                           float *P_pre, float *Q_pre)
{
    float *Ph = (float *)malloc((size_t)(n * r) * sizeof(float));
    float *Qh = (float *)malloc((size_t)(m * r) * sizeof(float));
    int64_t i, j;
    int32_t c;

    lq_compress(G, E, Q, n, m, r, alpha, bits_p, bits_q, p_codes, p_colmax, q_codes, q_colmax,
                Ph, Qh, P_pre, Q_pre);
    /* E = M - Phat Qhat^T (fp64 products, one rounding) */
    for (i = 0; i < n; ++i)
        for (j = 0; j < m; ++j) {
            double acc = 0.0;
            for (c = 0; c < r; ++c)
                acc += (double)Ph[i * r + c] * (double)Qh[j * r + c];
            E[i * m + j] = (float)((double)E[i * m + j] - acc);
        }
    if (p_hat)
        memcpy(p_hat, Ph, (size_t)(n * r) * sizeof(float));
    free(Ph);
    free(Qh);
}

/* [LQ] K workers, one step each.  Every worker runs the compressor above on its own
 * M_w = G_w + E_w from its own warm start Q_w; the messages (codes and column maxima) are
 * exchanged whole, since log codes cannot be summed.  Every worker then forms the same
 * approximate global gradient (referee minor comment on Section III-A: Ghat_t stands for the
 * global gradient) as the mean of the decoded messages,
 *   Ghat = (1/K) sum_w Phat_w Qhat_w^T     (fp64 sum over w, then c; one rounding to fp32),
 * and feeds back E_w = M_w - Ghat ("What carries the argument"), taken against the unrounded
 * mean and rounded once, so that K = 1 is the single-worker step exactly.
 * Codes and maxima are stacked by worker: p_codes K x n x r, p_colmax K x r, q_codes
 * K x m x r, q_colmax K x r.  G_hat n x m. */
void orc_lq_step_workers(const float *const *G, float *const *E, float *const *Q, int32_t K,
                         int64_t n, int64_t m, int32_t r, double alpha, int32_t bits_p,
                         int32_t bits_q, int8_t *p_codes, float *p_colmax, int8_t *q_codes,
                         float *q_colmax, float *G_hat)
{
    float *Ph = (float *)malloc((size_t)K * (size_t)(n * r) * sizeof(float));
    float *Qh = (float *)malloc((size_t)K * (size_t)(m * r) * sizeof(float));
    int64_t i, j;
    int32_t c, w;

    for (w = 0; w < K; ++w)
        lq_compress(G[w], E[w], Q[w], n, m, r, alpha, bits_p, bits_q, p_codes + w * n * r,
                    p_colmax + w * r, q_codes + w * m * r, q_colmax + w * r, Ph + w * n * r,
                    Qh + w * m * r, NULL, NULL);
    for (i = 0; i < n; ++i)
        for (j = 0; j < m; ++j) {
            double acc = 0.0, mean;
            for (w = 0; w < K; ++w) {
                const float *pw = Ph + w * n * r, *qw = Qh + w * m * r;
                for (c = 0; c < r; ++c)
                    acc += (double)pw[i * r + c] * (double)qw[j * r + c];
            }
            mean = acc / (double)K;
            G_hat[i * m + j] = (float)mean;
            for (w = 0; w < K; ++w)
                E[w][i * m + j] = (float)((double)E[w][i * m + j] - mean);
        }
    free(Ph);
    free(Qh);
}
