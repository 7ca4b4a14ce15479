/*
 * gq_oracle.h -- plain CPU oracle for allreduce-compatible gradient quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark load this code.  The product library never links, calls or
 * includes it, and this oracle includes nothing from the product library: the two are
 * independent implementations of the same written definitions.
 *
 * Sources (web pages on the subject):
 *   [GQ]   "Quantize Once, Train Fast: Allreduce-Compatible Compression with Provable
 *          Guarantees" / "Global-QSGD: Allreduce-Compatible Quantization for Distributed
 *          Learning with Theoretical Guarantees" (EuroMLSys '25), abstract: one global
 *          norm scales every worker so unbiased quantized codes can be summed by Allreduce.
 *   [USM]  "Unbiased Single-scale and Multi-scale Quantizers for Distributed
 *          Optimization", abstract: all-reduce compatible compression.
 *   [NUQ]  "NUQSGD: Provably Communication-efficient Data-parallel SGD via Nonuniform
 *          Quantization", abstract: nonuniform (exponential) level grid vs QSGD.
 *   [LQ]   review of "Trustworthy Efficient Communication for Distributed Learning using
 *          LQ-SGD Algorithm": "Core claim" (Eq. 5 log quantizer, 2^b bins, warm start),
 *          "What carries the argument" (G ~ P Q^T, error feedback E_t = G'_t - Ghat_t),
 *          referee major comment 1 (normalise by the maximum magnitude; Eq. 6 inverse;
 *          Q_t computed from the orthonormalised P_t); referee minor comment on
 *          Section III-A (Ghat_t is the approximate global gradient).
 *
 * Every function below is pinned to something other than itself by the CPU tests; none
 * is parity unpinned.  Where each is pinned:
 *   splitmix64_next, fmix32, worker_key: published known answers (tests/golden/rng_kat.json);
 *   uniform, hash_fill: the zero draw at counter = key, the fp32 rounding of hashes built
 *     through the inverse finaliser, uniformity and independence statistics (test_oracle_rng);
 *   load, sumsq, norm_finish, global_norm: closed forms and exact math.fsum sums;
 *   quant_one, quantize, quantize_list, lin: exact levels, unbiasedness, the two-point
 *     variance, QSGD's variance bound, brute force over small inputs (test_oracle_quant);
 *   pack, unpack_one: hand-worked byte layouts (tests/golden/pack_layout.json);
 *   accumulate, decode_factor, dequantize, f32_to_bf16: the allreduce-compatibility identity,
 *     exact rationals, bf16 rounding against torch;
 *   wire_*: hand-worked lane layouts (tests/golden/wire_layout.json), no carry between lanes;
 *   worker_scales, worker_mean, decode_workers: numpy norms and maxima, Fraction sums
 *     (test_oracle_baselines);
 *   logq_index, logq_level, logquant: every bin boundary against 60-digit decimal arithmetic
 *     (test_oracle_lq);
 *   mgs_rho, mgs, powersgd_logquant, lq_step_workers: LAPACK QR, the exact rank-one case,
 *     error-feedback identities and telescoping (test_oracle_lq, test_oracle_lq_workers).
 * The test_oracle_mutations suite plants one-line mistakes in a copy of this oracle and
 * checks that these pins catch every one.
 */
#ifndef GQ_ORACLE_H
#define GQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };     /* element types of gradients and outputs */
enum { ORC_UNIFORM = 0, ORC_EXP = 1 };  /* level grids */

/* ---------------- counter-based random numbers ---------------- */
/* SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): advance the state, return one output. */
uint64_t orc_splitmix64_next(uint64_t *state);
/* MurmurHash3 32-bit finaliser fmix32 (Appleby, public domain). */
uint32_t orc_fmix32(uint32_t h);
/* Key of worker k: low 32 bits of SplitMix64 output number k+1 from state `seed`. */
uint32_t orc_worker_key(uint64_t seed, uint32_t worker);
/* Uniform draw in [0,1]: fp32(fmix32(counter XOR key)) * 2^-32, the hash rounded to the
 * nearest fp32 (ties to even), then scaled (exact in double). */
double orc_uniform(uint32_t key, uint32_t counter);
/* out[t] = fmix32((counter0 + t) XOR key) for t < cnt (raw 32-bit hashes). */
void orc_hash_fill(uint32_t key, uint32_t counter0, int64_t cnt, uint32_t *out);

/* ---------------- global norm (one shared scale) ---------------- */
/* Element i of a buffer as a double (bf16 and fp32 convert exactly). */
double orc_load(const void *x, int32_t dtype, int64_t i);
/* acc + sum_{i<n} x_i^2 in fp64, strictly in index order (chunks can be chained). */
double orc_sumsq(const void *x, int32_t dtype, int64_t n, double acc);
/* S_g = fp32(max_k sqrt(sumsq[k*nseg + g])) from per-worker, per-segment sums of squares.
 * A non-finite S_g is replaced by 0 and makes the return value 1 (else 0).  norms_out
 * (K*nseg doubles, k-major) may be NULL. */
int32_t orc_norm_finish(const double *sumsq, int32_t K, int32_t nseg, float *scale_out,
                        double *norms_out);
/* orc_sumsq of every (worker, segment) from 0, then orc_norm_finish. */
int32_t orc_global_norm(const void *const *xs, int32_t K, int32_t dtype, int64_t n,
                        const int64_t *offsets, int32_t nseg, float *scale_out,
                        double *norms_out);

/* ---------------- stochastic quantisation ---------------- */
/* Signed level of one element.  Uniform: value in [-s, s] (levels = s).
 * Exponential: sign * j with j in [0, E] (levels = E), level j>0 meaning 2^(j-E).
 * A NaN element (possible only under a caller-given finite scale) goes to the top level, with
 * the sign of its sign bit (both grids). */
int32_t orc_quant_one(int32_t grid, int32_t levels, float x, float S, uint32_t key,
                      uint32_t counter);
/* Quantise a segmented buffer of one worker; counter of element i is index_base + i. */
void orc_quantize(const void *x, int32_t dtype, int64_t n, const int64_t *offsets,
                  int32_t nseg, const float *scale, int32_t grid, int32_t levels,
                  uint64_t seed, uint32_t worker, uint32_t index_base, int32_t *levels_out);
/* Same element rule on a list: x[t] with scale S[t] and counter[t], all with one key. */
void orc_quantize_list(const float *x, const float *S, const uint32_t *counter, int64_t cnt,
                       int32_t grid, int32_t levels, uint32_t key, int32_t *levels_out);

/* ---------------- codes ---------------- */
/* Pack signed levels into b-bit codes (b = 4 or 8); element 2t in the low nibble of byte t. */
void orc_pack(const int32_t *q, int64_t n, int32_t grid, int32_t bits, uint8_t *out);
/* Signed level stored at element i of a packed buffer. */
int32_t orc_unpack_one(const uint8_t *codes, int64_t i, int32_t grid, int32_t bits);
/* Integer value of a signed level on the common fixed-point grid of its level set:
 * uniform -> the level itself; exponential sign*j -> sign * 2^(j-1) (0 for j = 0). */
int64_t orc_lin(int32_t grid, int32_t signed_level);
/* sums_i = sum_k lin(code_{k,i}) stored as int16 or int32.  Returns the number of
 * elements whose sum does not fit the accumulator (those are stored truncated). */
int64_t orc_accumulate(const uint8_t *const *codes, int32_t K, int64_t n, int32_t grid,
                       int32_t bits, int32_t acc_bits, void *sums);

/* ---------------- summable wire payload ---------------- */
/* Reading of "the codes can be summed by Allreduce" for a collective whose sum is on
 * unsigned 32-bit words: element i is stored as the unsigned lane lin_i + o (o = s, or
 * 2^(E-1) on the exponential grid) of W bytes, little-endian, element i at byte i*W.  W is
 * the smallest of 1, 2, 4 whose range holds world * 2o, so adding `world` payloads word by
 * word never carries from one lane into the next.  Returns 0 when no width fits. */
int32_t orc_wire_lane_bytes(int32_t grid, int32_t levels, int32_t world);
/* Payload of signed levels q[0..n): round_up(n*W, 4) bytes, the padding zero. */
void orc_wire_encode(const int32_t *q, int64_t n, int32_t grid, int32_t levels, int32_t world,
                     uint8_t *payload);
/* out = word-wise sum (mod 2^32) of K payloads of nbytes bytes (a multiple of 4). */
void orc_wire_sum(const uint8_t *const *payloads, int32_t K, int64_t nbytes, uint8_t *out);
/* sums_i = lane_i - world * o: the integer sum of the world workers' linear values. */
void orc_wire_decode(const uint8_t *payload, int64_t n, int32_t grid, int32_t levels,
                     int32_t world, int32_t *sums);

/* ---------------- decode of the mean ---------------- */
/* f = fp32(S / D) with the division in fp64, D = s*K (uniform) or K*2^(E-1) (exponential);
 * 0 when S is not a positive finite number. */
float orc_decode_factor(int32_t grid, int32_t levels, int32_t K, float S);
/* fp32 -> bf16 by round-to-nearest-even, found by comparing the two neighbours. */
uint16_t orc_f32_to_bf16(float v);
/* mean_i = fp32(sum_i) * f_g (one fp32 multiply), stored as fp32 or bf16. */
void orc_dequantize(const void *sums, int32_t acc_bits, int64_t n, const int64_t *offsets,
                    int32_t nseg, const float *scale, int32_t grid, int32_t levels, int32_t K,
                    int32_t out_dtype, void *out);

/* ---------------- baselines with per-worker scales (not summable) ---------------- */
/* [NUQ] abstract: QSGD, in which every worker normalises by its own L2 norm, and its
 * heuristic variant QSGDinf, read here as the same quantiser normalised by the largest
 * magnitude (the L-infinity norm); NUQSGD proper is the exponential grid with per-worker L2
 * norms.  Codes scaled this way are not summable: the receiver decodes every worker's codes
 * with that worker's own scale and adds the decoded values. */
enum { ORC_NORM_L2 = 0, ORC_NORM_MAX = 1 };
/* scales_out[k*nseg + g] for every worker k and segment g: L2 -> fp32(sqrt(sum of squares in
 * fp64)); MAX -> the largest |x| (exact).  A non-finite value is replaced by 0 and makes the
 * return value 1 (else 0). */
int32_t orc_worker_scales(const void *const *xs, int32_t K, int32_t dtype, int64_t n,
                          const int64_t *offsets, int32_t nseg, int32_t norm,
                          float *scales_out);
/* mean_i for i in segment g: acc = +0, then for k = 0..K-1 in order
 * acc = fmaf((float)lin(q_{k,i}), f_{k,g}, acc) (one rounding per worker), where q_{k,i} is the
 * level of x_{k,i} under worker k's own scale S_{k,g} (orc_quant_one with worker k's key and
 * counter index_base + i) and f_{k,g} = orc_decode_factor(grid, levels, K, S_{k,g}); stored as
 * fp32 or bf16. */
void orc_worker_mean(const void *const *xs, int32_t K, int32_t dtype, int64_t n,
                     const int64_t *offsets, int32_t nseg, const float *scales, int32_t grid,
                     int32_t levels, uint64_t seed, uint32_t index_base, int32_t out_dtype,
                     void *out);

/* The receiver's side after an allgather of such codes: mean_i = the same fma chain as
 * orc_worker_mean with q_{k,i} read from worker k's packed codes (orc_unpack_one). */
void orc_decode_workers(const uint8_t *const *codes, int32_t K, int64_t n,
                        const int64_t *offsets, int32_t nseg, const float *scales, int32_t grid,
                        int32_t levels, int32_t bits, int32_t out_dtype, void *out);

/* ---------------- LQ-SGD: log quantiser and one PowerSGD step ---------------- */
/* Magnitude index in [0, L] of y in [0, 1]: the level k/L nearest to
 * q(y) = log(1 + alpha*y) / log(1 + alpha), ties going up.  L = 2^(bits-1) - 1. */
int32_t orc_logq_index(float y, double alpha, int32_t L);
/* Decode level k: fp32(((1 + alpha)^(k/L) - 1) / alpha). */
float orc_logq_level(int32_t k, double alpha, int32_t L);
/* Quantise each column of F (rows x r, row-major) after dividing by its max magnitude.
 * codes rows x r int8; colmax r fp32; Fhat rows x r (may be NULL). */
void orc_logquant(const float *F, int64_t rows, int32_t r, double alpha, int32_t bits,
                  int8_t *codes, float *colmax, float *Fhat);
/* Relative rounding rho = sqrt(m) 2^-24 of an entry of P = M Q_prev that sums m products of
 * fp32 values (the reading in gq_oracle.c). */
double orc_mgs_rho(int64_t m);
/* Modified Gram-Schmidt on the columns of P (n x r, r <= 8, row-major, fp32 in and out), fp64
 * math; m is the number of products summed in each entry of P.  Column c is numerically
 * dependent on the earlier ones, and set to zero like a column that is exactly zero, when the
 * norm it keeps after the projections is at most rho (|p_c| + sum_j |a_j| |p_j|), rho =
 * orc_mgs_rho(m), a the coefficients of its projection on the earlier columns. */
void orc_mgs(float *P, int64_t n, int32_t r, int64_t m);
/* One compressor step: M = G + E; P = M Qprev; P <- MGS(P); Q = M^T P; quantise P with
 * bits_p and Q with bits_q (the review's referee comment on Section V names b_p and b_q as
 * separate settings); E <- M - Phat Qhat^T; Qprev <- Qhat.  E and Q are updated in place.
 * P_pre and Q_pre (may be NULL) receive the unquantised factors. */
void orc_powersgd_logquant(const float *G, float *E, float *Q, int64_t n, int64_t m,
                           int32_t r, double alpha, int32_t bits_p, int32_t bits_q,
                           int8_t *p_codes,
                           float *p_colmax, int8_t *q_codes, float *q_colmax, float *p_hat,
                           float *P_pre, float *Q_pre);
/* K workers (1 <= K): each compresses its own M_w = G_w + E_w from its own warm start Q_w as
 * above; Ghat = fp32((1/K) sum_w Phat_w Qhat_w^T) (fp64 sums); E_w <- fp32(M_w - that mean);
 * Q_w <- Qhat_w.  Messages stacked by worker: p_codes K x n x r, p_colmax K x r,
 * q_codes K x m x r, q_colmax K x r.  G_hat n x m. */
void orc_lq_step_workers(const float *const *G, float *const *E, float *const *Q, int32_t K,
                         int64_t n, int64_t m, int32_t r, double alpha, int32_t bits_p,
                         int32_t bits_q, int8_t *p_codes, float *p_colmax, int8_t *q_codes,
                         float *q_colmax, float *G_hat);

#ifdef __cplusplus
}
#endif

#endif
