// gq_lq.hip -- gfx950 kernels of one LQ-SGD compressor step, for one worker or for K workers.
//
// Method (review of "Trustworthy Efficient Communication for Distributed Learning using LQ-SGD
// Algorithm"): PowerSGD's factorisation G ~ P Q^T with error feedback E_t = G'_t - Ghat_t
// ("What carries the argument"), Q warm-started from the previous step and both factors
// log-quantised by Eq. 5 onto 2^b bins ("Core claim"), after normalising each column by its
// largest magnitude and orthonormalising P first (referee major comment 1; Eq. 6 decodes).
//
// Design for CDNA4.  The step is HBM-bound: at rank r <= 8 the products do at most 2r flops
// per 4-byte element, far below the MFMA ridge, so they stay on the vector ALUs with fp32 FMA
// and the work is organised around the three passes over the n x m matrix:
//   pass 1  E <- G + E and P = E Q              (read G, E; write E)   k_lq_ef_mq
//   pass 2  Q' = E^T Pt                         (read E)               k_lq_mtp + k_lq_qsum
//   pass 3  E <- E - Phat Q'hat^T               (read E; write E)      k_lq_ef_update_q (one
//                                                                      worker, r <= 4: quantises
//                                                                      P and Q' itself), or
//                                                                      k_lq_quant_elems, then
//                                                                      k_lq_ef_update (one
//                                                                      worker) or the K
//                                                                      workers' k_lq_mean_ef
// With K workers (each its own G, E and warm start Q; the review's "Core claim" compresses each
// worker's factors before the exchange) every per-worker kernel runs all K in one launch, the
// worker taken from a grid dimension, and the last pass becomes k_lq_mean_ef: the mean of the
// K decoded messages, Ghat = (1/K) sum_w Phat_w Qhat_w^T (the approximate global gradient of
// the referee's comment on Section III-A), written once, and E_w <- M_w - Ghat for each worker
// (read K E's; write K E's and Ghat).
// Cache use: G and the incoming E are streamed once (non-temporal loads); the passes over M
// read it with ordinary loads, so what the column pass brings in can still be cached when the
// last pass reads it again.
// Row passes give each block 4 rows so every Q value fetched (from L2: Q is at most
// m x 8 fp32) is used 4 times, and issue all of a column group's row loads before the first
// store; Q is read in its own row-major layout (a thread's 4 columns are 4r consecutive
// floats), so no transposed copy is made.  The column pass gives each
// 512-thread block 128 rows x (64*VEC) columns (64 rows when that leaves too few blocks to
// fill the GPU) and reduces its 8 waves in LDS, so the per-chunk partials stay a few percent
// of the pass.
// Orthonormalisation: pass 1 also emits each block's r x r Gram contribution (products of the
// fp32 P values, exact in fp64); k_lq_solve sums them in a fixed order and runs Cholesky-QR
// twice in r x r space -- T1 from G, then T2 from T1^T G T1, which measures and removes the
// error of the first factorisation -- and the column pass forms Pt = P T1 T2 tile by tile.  In exact
// arithmetic P T is the Gram-Schmidt Q factor of P (columns in order; a column with no
// remaining norm is zero).  The kernels that produce Pt and Q' also take their column maxima
// (integer atomicMax on the bit patterns of |v|: exact and order-independent), so the log
// quantiser runs element by element: it encodes with a table of the L bin boundaries rounded
// up to fp32 (so "y >= boundary" is decided exactly) and decodes with a table of the L+1
// Eq. 6 levels.
#include <float.h>
#include <math.h>

#include <cmath>
#include <cstring>

#include "gq_lq.h"

namespace gq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowsA = 4;      // rows per block in the row passes
constexpr int kBlockA = 256;
constexpr int kWavesC = 8;     // waves per column-pass block
// Rows per block of the one-worker last pass (k_lq_ef_update_q): 64, or 32 at rank 1, where
// requantising a block's Q' values costs least and more, shorter blocks fill the GPU better
// (4096 x 4096 step: 0.087 -> 0.083 ms; 16 rows, or 32 at rank 4, ran slower).
template <int RANK>
constexpr int rows_q() { return RANK == 1 ? 32 : 64; }
// Highest rank whose one-worker last pass quantises the factors itself (k_lq_ef_update_q):
// each of its blocks quantises its columns' r values of Q' again, which at r = 7 cost more than
// the separate quantiser it saves (measured at 4096 x 4096: 29.7 us against 23.2 + 4.7 us;
// at r = 1, 24.0 against 22.5 + 4.7).
constexpr int kFoldRankMax = 4;
// Rows per column-pass chunk: 128, or 64 when 128-row chunks would give fewer than
// kColBlocksMin blocks (the pass is then latency-bound and wants more of them).
constexpr int kColBlocksMin = 1024;
// MI355X's Infinity Cache (the last level before HBM)
constexpr double kMallBytes = 256.0 * 1024 * 1024;
// threads of the one-block solve: 16 waves, 8 at rank 8 (so that its r x r work fits in
// registers)
template <int RANK>
constexpr int solve_block() { return RANK > 7 ? 512 : 1024; }

template <int VEC>
__device__ __forceinline__ void ldv_nt(const float *p, float (&v)[VEC]) {
  if constexpr (VEC == 4) {
    const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  } else {
    v[0] = __builtin_nontemporal_load(p);
  }
}

template <int VEC>
__device__ __forceinline__ void ldv(const float *p, float (&v)[VEC]) {
  if constexpr (VEC == 4) {
    const f32x4 t = *reinterpret_cast<const f32x4 *>(p);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  } else {
    v[0] = *p;
  }
}

template <int VEC>
__device__ __forceinline__ void stv(float *p, const float (&v)[VEC]) {
  if constexpr (VEC == 4) {
    f32x4 t = {v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4 *>(p) = t;
  } else {
    *p = v[0];
  }
}

template <int VEC>
__device__ __forceinline__ void stv_nt(float *p, const float (&v)[VEC]) {
  if constexpr (VEC == 4) {
    f32x4 t = {v[0], v[1], v[2], v[3]};
    __builtin_nontemporal_store(t, reinterpret_cast<f32x4 *>(p));
  } else {
    __builtin_nontemporal_store(v[0], p);
  }
}

// q[c][v] = Q[(j + v) * RANK + c]: the VEC rows of the row-major m x RANK factor that this
// thread's VEC columns need (4*RANK consecutive floats when VEC = 4; j is a multiple of 4).
template <int RANK, int VEC>
__device__ __forceinline__ void load_q_rows(const float *Q, int64_t j, float (&q)[RANK][VEC]) {
  if constexpr (VEC == 4) {
    float f[4 * RANK];
    const f32x4 *p = reinterpret_cast<const f32x4 *>(Q + j * RANK);
#pragma unroll
    for (int i = 0; i < RANK; ++i) {
      const f32x4 t = p[i];
      f[4 * i] = t.x; f[4 * i + 1] = t.y; f[4 * i + 2] = t.z; f[4 * i + 3] = t.w;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int c = 0; c < RANK; ++c) q[c][v] = f[v * RANK + c];
  } else {
#pragma unroll
    for (int c = 0; c < RANK; ++c) q[c][0] = Q[j * RANK + c];
  }
}

// v of another lane by a DPP row operation (CTRL) in the rows ROW_MASK enables; 0 elsewhere.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF,
                                                    false));
}

// Sum over the wave with DPP row operations only (no LDS traffic, fixed order); the total is
// in lane 63.  Pairs and quads (quad_perm), half-rows (row_half_mirror), rows (row_mirror),
// then row 0 into row 1 and row 2 into row 3 (row_bcast:15), then rows 0-1 into 2-3
// (row_bcast:31).
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
  v += dpp_f<0xB1, 0xF>(v);
  v += dpp_f<0x4E, 0xF>(v);
  v += dpp_f<0x141, 0xF>(v);
  v += dpp_f<0x140, 0xF>(v);
  v += dpp_f<0x142, 0xA>(v);
  v += dpp_f<0x143, 0xC>(v);
  return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Index (a, b), a <= b, of packed upper-triangle entry t of a RANK x RANK matrix.
template <int RANK>
__device__ __forceinline__ void tri_index(int t, int &a, int &b) {
  a = 0;
  while (t >= RANK - a) {
    t -= RANK - a;
    ++a;
  }
  b = a + t;
}

// Pass 1: E <- G + E (the gradient with the previous error fed back), P = E Q, and the block's
// share of the Gram matrix P^T P (packed upper triangle, fp64, stored entry-major so that the
// solve reads each entry's partials contiguously).
// Worker blockIdx.y of the step: its own G, E and Q; its slices of the stacked P and partials.
// NT_M stores M non-temporally: when the step's M matrices together exceed the Infinity Cache,
// dirty lines left there by this pass would be written back while the column pass reads M and
// slow it (measured: 141 -> 96 us for 8 x 4096 x 4096 at r = 1); when they fit, the cached M
// is what makes the next two passes fast, so ordinary stores are kept.
template <int RANK, int VEC, bool NT_M>
__global__ __launch_bounds__(kBlockA) void k_lq_ef_mq(const LqWorkerPtrs W,
                                                      float *__restrict__ P_all,
                                                      double *__restrict__ gpart_all, int64_t n,
                                                      int64_t m) {
  constexpr int NG = RANK * (RANK + 1) / 2;
  const int wk = blockIdx.y;
  const float *__restrict__ G = W.G[wk];
  float *__restrict__ E = W.E[wk];
  const float *__restrict__ Q = W.Q[wk];
  float *__restrict__ P = P_all + (int64_t)wk * n * RANK;
  double *__restrict__ gpart = gpart_all + (int64_t)wk * NG * gridDim.x;
  __shared__ float red[kBlockA / 64][kRowsA * RANK];
  __shared__ float pv[kRowsA * RANK];
  const int64_t row0 = (int64_t)blockIdx.x * kRowsA;
  float acc[kRowsA][RANK];
#pragma unroll
  for (int rr = 0; rr < kRowsA; ++rr)
#pragma unroll
    for (int c = 0; c < RANK; ++c) acc[rr][c] = 0.0f;
  const int nr = n - row0 < kRowsA ? (int)(n - row0) : kRowsA;
  for (int64_t j = (int64_t)threadIdx.x * VEC; j < m; j += (int64_t)kBlockA * VEC) {
    // every load of this column group is issued before the first store
    float g[kRowsA][VEC], e[kRowsA][VEC];
#pragma unroll
    for (int rr = 0; rr < kRowsA; ++rr)
      if (rr < nr) {
        ldv_nt<VEC>(G + (row0 + rr) * m + j, g[rr]);
        ldv_nt<VEC>(E + (row0 + rr) * m + j, e[rr]);
      }
    float q[RANK][VEC];
    load_q_rows<RANK, VEC>(Q, j, q);
#pragma unroll
    for (int rr = 0; rr < kRowsA; ++rr) {
      if (rr < nr) {
        float mv[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) mv[v] = g[rr][v] + e[rr][v];
        if constexpr (NT_M)
          stv_nt<VEC>(E + (row0 + rr) * m + j, mv);
        else
          stv<VEC>(E + (row0 + rr) * m + j, mv);
#pragma unroll
        for (int c = 0; c < RANK; ++c)
#pragma unroll
          for (int v = 0; v < VEC; ++v) acc[rr][c] = fmaf(mv[v], q[c][v], acc[rr][c]);
      }
    }
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int rr = 0; rr < kRowsA; ++rr)
#pragma unroll
    for (int c = 0; c < RANK; ++c) {
      const float s = wave_sum_to_lane63(acc[rr][c]);
      if (lane == 63) red[w][rr * RANK + c] = s;
    }
  __syncthreads();
  if (threadIdx.x < kRowsA * RANK) {
    const int t = threadIdx.x;
    const int64_t row = row0 + t / RANK;
    float s = 0.0f;
    for (int i = 0; i < kBlockA / 64; ++i) s += red[i][t];
    if (row >= n) s = 0.0f;
    pv[t] = s;
    if (row < n) P[row * RANK + t % RANK] = s;
  }
  __syncthreads();
  if (threadIdx.x < NG) {
    int a, b;
    tri_index<RANK>(threadIdx.x, a, b);
    double g = 0.0;
#pragma unroll
    for (int rr = 0; rr < kRowsA; ++rr) g += (double)pv[rr * RANK + a] * (double)pv[rr * RANK + b];
    gpart[(int64_t)threadIdx.x * gridDim.x + blockIdx.x] = g;  // entry-major: [NG][nblocks]
  }
}

// v from lane l (l a compile-time or wave-uniform index): two v_readlane_b32.
__device__ __forceinline__ double readlane_d(double v, int l) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = __builtin_amdgcn_readlane((unsigned)b, l);
  const unsigned hi = __builtin_amdgcn_readlane((unsigned)(b >> 32), l);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// 1/sqrt(d) for a positive normal d (a pivot of a Gram matrix of fp32 vectors always is): the
// hardware estimate refined by two Newton steps y <- y (3/2 - (d/2) y^2), each of which
// squares the relative error, so the result is good to fp64 rounding.
__device__ __forceinline__ double rsqrt_refined(double d) {
  const double h = 0.5 * d;
  double y = __builtin_amdgcn_rsq(d);
#pragma unroll
  for (int it = 0; it < 2; ++it) y = fma(y, fma(-h * y, y, 0.5), y);
  return y;
}

// Upper-triangular T with (P T)^T (P T) = I given G = P^T P, column by column as Gram-Schmidt
// does it, through the Cholesky factor G = R^T R (R upper triangular), and T = R^-1 from
// T R = I: T[a][c] = (delta_ac - sum_{k<c} T[a][k] R[k][c]) / R[c][c].
// Dependent columns: R[c][c] is the norm column c keeps after the projections, and
// a_j = sum_{k<c} T[j][k] R[k][c] are its coefficients on the earlier columns.  If rounding
// moved every column by a relative amount rho, that remainder would move by at most
// rho (|p_c| + sum_j |a_j| |p_j|); with rho = sqrt(m) 2^-24, the rounding of an fp32 sum of
// m products (the entries of P = M Q), a column whose R[c][c] is within that bound has no
// direction of its own that fp32 resolves, and its row of R and column of T are zero.
// rho2 = rho^2 is compared with the squares (R[c][c]^2 against rho2 * bound^2).
// Spread over the lanes of one wave: lane j (< RANK) holds column j of G (g[k] = G[k][j]) and
// of R, and row j of T.  Step c reads column c of R from lane c with v_readlane (uniform
// values); with it every lane forms its own entries of row c of R and of column c of T, so T
// needs no exchange at all; the c terms |a_j| |p_j| of the bound are read from lanes 0..c-1.
// Products accumulate by fused multiply-add in fp64.
template <int RANK>
__device__ __forceinline__ void lane_cholqr_T(const double (&g)[RANK], int j, double rho2,
                                              double (&trow)[RANK]) {
  double rcol[RANK];  // R[k][j]
  double gjj = 0.0;   // G[j][j]
#pragma unroll
  for (int k = 0; k < RANK; ++k) {
    rcol[k] = 0.0;
    trow[k] = 0.0;
    if (k == j) gjj = g[k];
  }
  const double pj = sqrt(gjj);  // |p_j|
#pragma unroll
  for (int c = 0; c < RANK; ++c) {
    double rkc[RANK > 1 ? RANK - 1 : 1];  // R[k][c], k < c
#pragma unroll
    for (int k = 0; k < c; ++k) rkc[k] = readlane_d(rcol[k], c);
    const double gcc = readlane_d(g[c], c);  // G[c][c]: the column's squared norm
    double d = gcc;
#pragma unroll
    for (int k = 0; k < c; ++k) d = fma(-rkc[k], rkc[k], d);
    double v = g[c];  // G[c][j]
    double u = j == c ? 1.0 : 0.0;
#pragma unroll
    for (int k = 0; k < c; ++k) {
      v = fma(-rkc[k], rcol[k], v);
      u = fma(-trow[k], rkc[k], u);  // T[j][k] R[k][c]; T[j][k] = 0 for k < j
    }
    // lane j < c: u = -a_j; the bound |p_c| + sum_{j<c} |a_j| |p_j| in lane order
    const double term = fabs(u) * pj;
    double bound = sqrt(gcc);
#pragma unroll
    for (int k = 0; k < c; ++k) bound += readlane_d(term, k);
    if (d > rho2 * bound * bound) {  // the same value in every lane
      const double inv = rsqrt_refined(d), rc = d * inv;
      if (j > c) rcol[c] = v * inv;
      if (j == c) rcol[c] = rc;
      trow[c] = u * inv;
    }
  }
}

// Orthonormalise P (r x r part): fixed-order sum of the block Gram partials, then two
// Cholesky-QR rounds in r x r space (lane-parallel in one wave) giving T = T1 T2.
// One block per worker (blockIdx.x).
template <int RANK>
__global__ __launch_bounds__(solve_block<RANK>()) void k_lq_solve(const double *__restrict__ gpart_all,
                                                          int64_t nblocks,
                                                          double *__restrict__ T_all,
                                                          unsigned *__restrict__ cmax_all,
                                                          double rho2) {
  constexpr int NG = RANK * (RANK + 1) / 2;
  const int wk = blockIdx.x;
  const double *__restrict__ gpart = gpart_all + (int64_t)wk * NG * nblocks;
  double *__restrict__ Tout = T_all + wk * RANK * RANK;
  unsigned *__restrict__ cmax_bits = cmax_all + wk * 2 * RANK;
  __shared__ double Gs[RANK][RANK];
  __shared__ double T1s[RANK][RANK], T2s[RANK][RANK];  // rows of T1 and of T2
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid < 2 * RANK) cmax_bits[tid] = 0u;  // column maxima of Pt and Q' start at +0
  // wave w sums entries t = w, w + NW, ...: lane l adds blocks l, l + 64, ... in order, UB
  // loads per entry issued together, then the lanes are combined in a fixed butterfly
  constexpr int NW = solve_block<RANK>() / 64, TE = (NG + NW - 1) / NW, UB = TE > 2 ? 8 : 16;
  double acc[TE];
#pragma unroll
  for (int e = 0; e < TE; ++e) acc[e] = 0.0;
  for (int64_t b0 = lane; b0 < nblocks; b0 += UB * 64) {
    double v[TE][UB];
#pragma unroll
    for (int e = 0; e < TE; ++e) {
      const int t = w + e * NW;
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int64_t b = b0 + (int64_t)u * 64;
        v[e][u] = (t < NG && b < nblocks) ? gpart[(int64_t)t * nblocks + b] : 0.0;
      }
    }
#pragma unroll
    for (int e = 0; e < TE; ++e)
#pragma unroll
      for (int u = 0; u < UB; ++u) acc[e] += v[e][u];
  }
#pragma unroll
  for (int e = 0; e < TE; ++e) {
    const int t = w + e * NW;
    const double sum = wave_sum_d(acc[e]);
    if (t < NG && lane == 0) {
      int a, b;
      tri_index<RANK>(t, a, b);
      Gs[a][b] = sum;
      Gs[b][a] = sum;
    }
  }
  __syncthreads();
  // r x r part in wave 0 (lane j < RANK owns column j of G and row j of T; lanes beyond
  // compute lane 0's values); the other waves only take part in the barriers
  const int jc = lane < RANK ? lane : 0;
  if (w == 0) {
    double g[RANK], t1[RANK];
#pragma unroll
    for (int k = 0; k < RANK; ++k) g[k] = Gs[k][jc];
    lane_cholqr_T<RANK>(g, jc, rho2, t1);
    if (lane < RANK)
#pragma unroll
      for (int k = 0; k < RANK; ++k) T1s[lane][k] = t1[k];
  }
  __syncthreads();
  if (w == 0) {
    // column jc of W = G T1 (T1[x][jc] = 0 for x > jc), then column jc of T1^T W, the Gram
    // matrix of P T1; the entries of G and T1 are broadcast from LDS
    double wcol[RANK];
#pragma unroll
    for (int b = 0; b < RANK; ++b) wcol[b] = 0.0;
#pragma unroll 1
    for (int x = 0; x < RANK; ++x) {
      const double tx = T1s[x][jc];
#pragma unroll
      for (int b = 0; b < RANK; ++b) wcol[b] = fma(Gs[b][x], tx, wcol[b]);
    }
    double g[RANK];
#pragma unroll
    for (int c = 0; c < RANK; ++c) {
      double sum = 0.0;
#pragma unroll
      for (int b = 0; b <= c; ++b) sum = fma(T1s[b][c], wcol[b], sum);
      g[c] = sum;
    }
    double t2[RANK];
    lane_cholqr_T<RANK>(g, jc, rho2, t2);
    if (lane < RANK)
#pragma unroll
      for (int k = 0; k < RANK; ++k) T2s[lane][k] = t2[k];
  }
  __syncthreads();
  // row jc of T = T1 T2: T[jc][c] sums T1[jc][k] T2[k][c] over k (T1[jc][k] = 0 for k < jc)
  if (w == 0 && lane < RANK) {
    double trow[RANK];
#pragma unroll
    for (int c = 0; c < RANK; ++c) trow[c] = 0.0;
#pragma unroll 1
    for (int k = 0; k < RANK; ++k) {
      const double t1k = T1s[jc][k];
#pragma unroll
      for (int c = 0; c < RANK; ++c) trow[c] = fma(t1k, T2s[k][c], trow[c]);
    }
#pragma unroll
    for (int c = 0; c < RANK; ++c) Tout[jc * RANK + c] = trow[c];
  }
}

// Pass 2 (partials): part[chunk][j][c] = sum over the chunk's rows of E[row][j] * Pt[row][c].
// Each block first forms its chunk's rows of Pt = fp32(P T) (fp64 products) in LDS; the blocks
// of the first column tile also store them (Pt for the quantiser, the optional p_pre copy)
// and take the column maxima of Pt: the bit patterns of non-negative floats order like
// unsigned integers, so integer atomicMax (in LDS per block, then once per column in memory)
// is the exact, order-independent maximum.  Wave w takes rows w, w + 8, ... of the chunk, in
// batches of loads issued together; waves 4..7 hand their sums to waves 0..3 through LDS, and
// the four pair sums are added in wave order and written as contiguous (j, c) runs.
// Worker blockIdx.z: M is its E; P, T, Pt, p_pre (if any), the maxima and the partials are
// its slices of the stacked buffers.
template <int RANK, int VEC, int ROWSC>
__global__ __launch_bounds__(kWavesC * 64) void k_lq_mtp(const LqWorkerPtrs W,
                                                         const float *__restrict__ P_all,
                                                         const double *__restrict__ T_all,
                                                         float *__restrict__ Pt_all,
                                                         float *__restrict__ p_pre_all,
                                                         unsigned *__restrict__ cmax_all,
                                                         float *__restrict__ part_all, int64_t n,
                                                         int64_t m) {
  const int wk = blockIdx.z;
  const float *__restrict__ M = W.E[wk];
  const float *__restrict__ P = P_all + (int64_t)wk * n * RANK;
  const double *__restrict__ T = T_all + wk * RANK * RANK;
  float *__restrict__ Pt = Pt_all + (int64_t)wk * n * RANK;
  float *__restrict__ p_pre = p_pre_all ? p_pre_all + (int64_t)wk * n * RANK : nullptr;
  unsigned *__restrict__ cmax_bits = cmax_all + wk * 2 * RANK;
  float *__restrict__ part = part_all + (int64_t)wk * gridDim.y * m * RANK;
  constexpr int RW = ROWSC / kWavesC;   // rows per wave
  // rows per load batch: all of them at low rank; 4 above, which with the half-size LDS
  // reduction below lets a CU hold more blocks at once
  constexpr int RB = RANK <= 4 ? RW : 4;
  static_assert(RW % RB == 0, "row batches must tile the wave's rows");
  constexpr int COLS = 64 * VEC;        // columns per block
  __shared__ float red[kWavesC / 2][COLS * RANK];
  __shared__ float ptile[ROWSC * RANK];
  __shared__ unsigned smax[RANK];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t j0 = (int64_t)blockIdx.x * COLS;
  const int64_t j = j0 + (int64_t)lane * VEC;
  const int64_t r0 = (int64_t)blockIdx.y * ROWSC;
  const int64_t r1 = r0 + ROWSC < n ? r0 + ROWSC : n;
  const bool first_tile = blockIdx.x == 0;
  float mv[RB][VEC];
  // the first batch of rows is in flight while the Pt tile is formed
#pragma unroll
  for (int u = 0; u < RB; ++u) {
    const int64_t row = r0 + w + (int64_t)u * kWavesC;
    if (j < m && row < r1) {
      ldv<VEC>(M + row * m + j, mv[u]);
    } else {
#pragma unroll
      for (int v = 0; v < VEC; ++v) mv[u][v] = 0.0f;
    }
  }
  if (first_tile && threadIdx.x < RANK) smax[threadIdx.x] = 0u;
  __syncthreads();
  for (int e = threadIdx.x; e < ROWSC * RANK; e += kWavesC * 64) {
    const int64_t row = r0 + e / RANK;
    const int c = e % RANK;
    float o = 0.0f;
    if (row < r1) {
      double sum = 0.0;
      for (int a = 0; a <= c; ++a) sum += (double)P[row * RANK + a] * T[a * RANK + c];
      o = (float)sum;
      if (first_tile) {
        Pt[row * RANK + c] = o;
        if (p_pre) p_pre[row * RANK + c] = o;
        atomicMax(&smax[c], __float_as_uint(fabsf(o)));
      }
    }
    ptile[e] = o;
  }
  __syncthreads();
  if (first_tile && threadIdx.x < RANK) atomicMax(&cmax_bits[threadIdx.x], smax[threadIdx.x]);
  float acc[VEC][RANK];
#pragma unroll
  for (int v = 0; v < VEC; ++v)
#pragma unroll
    for (int c = 0; c < RANK; ++c) acc[v][c] = 0.0f;
  if (j < m) {
#pragma unroll 1
    for (int u0 = 0; u0 < RW; u0 += RB) {
      if (u0 > 0) {
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          const int64_t row = r0 + w + (int64_t)(u0 + u) * kWavesC;
          if (row < r1) {
            ldv<VEC>(M + row * m + j, mv[u]);
          } else {
#pragma unroll
            for (int v = 0; v < VEC; ++v) mv[u][v] = 0.0f;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const int64_t row = r0 + w + (int64_t)(u0 + u) * kWavesC;
        if (row < r1) {
          const int lr = w + (u0 + u) * kWavesC;
          float p[RANK];
#pragma unroll
          for (int c = 0; c < RANK; ++c) p[c] = ptile[lr * RANK + c];
#pragma unroll
          for (int v = 0; v < VEC; ++v)
#pragma unroll
            for (int c = 0; c < RANK; ++c) acc[v][c] = fmaf(mv[u][v], p[c], acc[v][c]);
        }
      }
    }
  }
  // waves 4..7 hand their sums to waves 0..3, which add them and leave the four sums in LDS
  if (w >= kWavesC / 2) {
#pragma unroll
    for (int v = 0; v < VEC; ++v)
#pragma unroll
      for (int c = 0; c < RANK; ++c) red[w - kWavesC / 2][(lane * VEC + v) * RANK + c] = acc[v][c];
  }
  __syncthreads();
  if (w < kWavesC / 2) {
#pragma unroll
    for (int v = 0; v < VEC; ++v)
#pragma unroll
      for (int c = 0; c < RANK; ++c) {
        float *slot = &red[w][(lane * VEC + v) * RANK + c];
        *slot = acc[v][c] + *slot;
      }
  }
  __syncthreads();
  const int64_t ncols = m - j0 < COLS ? m - j0 : COLS;
  float *dst = part + ((int64_t)blockIdx.y * m + j0) * RANK;
  for (int o = threadIdx.x; o < ncols * RANK; o += kWavesC * 64) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kWavesC / 2; ++i) s += red[i][o];
    dst[o] = s;
  }
}

// Pass 2 (final): Q'[j][c] = sum over the chunks' partials and the column maxima of Q' (as for
// Pt in k_lq_mtp).  Each output is summed by G threads -- group g takes chunks g, g + G, ...
// in order, with a batch of loads in flight -- and the group sums are added in group order.
// G = 1 normally; a short factor (at most kQsumShort outputs, e.g. rank 1 or 2 of 4096 rows)
// takes G = 8 so that it still spreads over 128+ blocks.  Every block publishes its column
// maxima once (r global atomics per block).
constexpr int kQsumShort = 8192;

// Worker blockIdx.y: its slices of the partials, of Q', of q_pre (if any) and of the maxima
// (cmax_all holds 2 RANK words per worker; Q' takes the second RANK).
template <int RANK, int G>
__global__ __launch_bounds__(256) void k_lq_qsum(const float *__restrict__ part_all,
                                                 float *__restrict__ Qn_all,
                                                 float *__restrict__ q_pre_all,
                                                 unsigned *__restrict__ cmax_all, int64_t count,
                                                 int nchunks) {
  constexpr int OUT = 256 / G, NB = 32 / G > 8 ? 32 / G : 8;  // outputs per block, loads per batch
  const int wk = blockIdx.y;
  const float *__restrict__ part = part_all + (int64_t)wk * nchunks * count;
  float *__restrict__ Qn = Qn_all + (int64_t)wk * count;
  float *__restrict__ q_pre = q_pre_all ? q_pre_all + (int64_t)wk * count : nullptr;
  unsigned *__restrict__ cmax_bits = cmax_all + wk * 2 * RANK + RANK;
  __shared__ float ps[G][OUT];
  __shared__ unsigned smax[RANK];
  const int il = threadIdx.x % OUT, g = threadIdx.x / OUT;
  const int64_t i = (int64_t)blockIdx.x * OUT + il;
  if (threadIdx.x < RANK) smax[threadIdx.x] = 0u;
  float s = 0.0f;
  if (i < count) {
    for (int ch0 = g; ch0 < nchunks; ch0 += NB * G) {
      float v[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int ch = ch0 + u * G;
        v[u] = ch < nchunks ? part[(int64_t)ch * count + i] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < NB; ++u)
        if (ch0 + u * G < nchunks) s += v[u];
    }
  }
  if constexpr (G > 1) {
    ps[g][il] = s;
    __syncthreads();
    if (g == 0) {
      float t = 0.0f;
#pragma unroll
      for (int k = 0; k < G; ++k) t += ps[k][il];
      s = t;
    }
  } else {
    __syncthreads();  // smax is initialised
  }
  if (g == 0 && i < count) {
    Qn[i] = s;
    if (q_pre) q_pre[i] = s;
    atomicMax(&smax[i % RANK], __float_as_uint(fabsf(s)));
  }
  __syncthreads();
  if (threadIdx.x < RANK) atomicMax(&cmax_bits[threadIdx.x], smax[threadIdx.x]);
}

// Log-quantise one factor value x of a column with maximum mx: the code and the decoded value
// (Eq. 5 encode: k = the number of boundaries thr[0..L-1] at or below y = |x| / mx; Eq. 6
// decode by the level table lvl[0..L]).  Boundary k lies at y where L log(1 + alpha y) /
// log(1 + alpha) = k + 1/2, so with tl = L / log2(1 + alpha) the count is about
// floor(tl log2(1 + alpha y) + 1/2); the estimate is then moved, one boundary at a time, until
// thr[k - 1] <= y < thr[k] holds, which fixes k exactly as a search of the table would (a NaN
// y counts no boundary).  The estimate is rarely off by more than one step.
__device__ __forceinline__ void logq_one(float x, float mx, const float *thr, const float *lvl,
                                         int L, float alpha, float tl, int8_t &code, float &fh) {
  int k = 0;
  if (mx > 0.0f) {
    const float y = fabsf(x) / mx;  // IEEE division, in [0, 1]
    const float t = tl * __log2f(fmaf(alpha, y, 1.0f)) + 0.5f;
    k = t >= (float)L ? L : (t >= 1.0f ? (int)t : 0);
    while (k < L && thr[k] <= y) ++k;
    while (k > 0 && !(thr[k - 1] <= y)) --k;
  }
  code = (int8_t)(x < 0.0f ? -k : k);
  const float v = lvl[k] * mx;
  fh = x < 0.0f ? -v : v;
}

struct ColJob {
  const float *F;        // rows x r
  int64_t rows;
  int r;
  int8_t *codes;         // rows x r
  float *colmax;         // r
  float *Fhat;           // rows x r or nullptr
  float *Fhat2;          // rows x r or nullptr (second copy)
};

// One block per column: max magnitude, then the Eq. 5 encode and Eq. 6 decode of logq_one.
__global__ __launch_bounds__(1024) void k_lq_quant_cols(ColJob j0, ColJob j1, int ncols0,
                                                        const float *tab, int L, float alpha,
                                                        float tl) {
  __shared__ float thr[128];
  __shared__ float lvl[128];
  __shared__ float wmax[16];
  const int tid = threadIdx.x;
  if (tid < L) thr[tid] = tab[tid];
  if (tid <= L) lvl[tid] = tab[L + tid];
  const bool first = (int)blockIdx.x < ncols0;
  const ColJob &J = first ? j0 : j1;
  const int c = first ? (int)blockIdx.x : (int)blockIdx.x - ncols0;
  float mx = 0.0f;
  for (int64_t i = tid; i < J.rows; i += blockDim.x) mx = fmaxf(mx, fabsf(J.F[i * J.r + c]));
  mx = wave_max_f(mx);
  if ((tid & 63) == 0) wmax[tid >> 6] = mx;
  __syncthreads();
  mx = 0.0f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) mx = fmaxf(mx, wmax[i]);
  if (tid == 0) J.colmax[c] = mx;
  for (int64_t i = tid; i < J.rows; i += blockDim.x) {
    int8_t code;
    float fh;
    logq_one(J.F[i * J.r + c], mx, thr, lvl, L, alpha, tl, code, fh);
    J.codes[i * J.r + c] = code;
    if (J.Fhat) J.Fhat[i * J.r + c] = fh;
    if (J.Fhat2) J.Fhat2[i * J.r + c] = fh;
  }
}

// Log-quantise both factors element by element, the column maxima already known (cmax_bits:
// RANK words for Pt, then RANK for Q'), each with its own tables (code widths b_p and b_q),
// by logq_one.
struct ElemJob {
  const float *Pt;       // n x r
  const float *Qn;       // m x r
  int64_t n, m;
  int r;
  const unsigned *cmax_bits;
  int8_t *p_codes, *q_codes;
  float *p_colmax, *q_colmax;
  float *Ph, *p_hat;     // decoded P (scratch) and the optional output copy
  float *Qh;             // decoded Q (written into the worker's Q)
};

// Worker blockIdx.y: every pointer of J0 is the base of a buffer stacked by worker (p_hat may
// be null); the decoded Q goes into the worker's own Q.
__global__ __launch_bounds__(256) void k_lq_quant_elems(const ElemJob J0, const LqWorkerPtrs W,
                                                        const float *tab_p, int Lp, float tlp,
                                                        const float *tab_q, int Lq, float tlq,
                                                        float alpha) {
  __shared__ float thr[2][128];
  __shared__ float lvl[2][128];
  const int tid = threadIdx.x;
  const int wk = blockIdx.y;
  ElemJob J = J0;
  {
    const int64_t pn = J0.n * J0.r, qm = J0.m * J0.r;
    J.Pt += wk * pn;
    J.Qn += wk * qm;
    J.cmax_bits += wk * 2 * J0.r;
    J.p_codes += wk * pn;
    J.q_codes += wk * qm;
    J.p_colmax += wk * J0.r;
    J.q_colmax += wk * J0.r;
    J.Ph += wk * pn;
    if (J0.p_hat) J.p_hat += wk * pn;
    J.Qh = W.Q[wk];
  }
  const int64_t np = J.n * J.r, nq = J.m * J.r;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + tid;
  // the element and its column maximum are fetched while the tables are staged
  const bool live = e < np + nq;
  const bool isp = e < np;
  const int64_t i = isp ? e : e - np;
  const int c = live ? (int)(i % J.r) : 0;
  const float x = live ? (isp ? J.Pt[i] : J.Qn[i]) : 0.0f;
  const float mx = live ? __uint_as_float(J.cmax_bits[isp ? c : J.r + c]) : 0.0f;
  if (tid < Lp) thr[0][tid] = tab_p[tid];
  if (tid <= Lp) lvl[0][tid] = tab_p[Lp + tid];
  if (tid < Lq) thr[1][tid] = tab_q[tid];
  if (tid <= Lq) lvl[1][tid] = tab_q[Lq + tid];
  __syncthreads();
  if (blockIdx.x == 0 && tid < 2 * J.r) {
    const float mxv = __uint_as_float(J.cmax_bits[tid]);
    if (tid < J.r) J.p_colmax[tid] = mxv; else J.q_colmax[tid - J.r] = mxv;
  }
  if (!live) return;
  const int t = isp ? 0 : 1;
  int8_t code;
  float fh;
  logq_one(x, mx, thr[t], lvl[t], isp ? Lp : Lq, alpha, isp ? tlp : tlq, code, fh);
  if (isp) {
    J.p_codes[i] = code;
    J.Ph[i] = fh;
    if (J.p_hat) J.p_hat[i] = fh;
  } else {
    J.q_codes[i] = code;
    J.Qh[i] = fh;
  }
}

// Pass 3 of one worker with the log quantiser folded in: block (x, y) owns columns
// [x * 64 VEC, (x + 1) * 64 VEC) and rows [y * RC, (y + 1) * RC).  Once the column pass has
// left Pt, Q' and their column maxima, the block quantises its columns' rows of Q' and its
// rows of Pt into LDS (the first row chunk also stores the Q codes and the decoded Q as the
// warm start, the first column tile the P codes and the decoded P), then updates its tile of
// E <- E - Phat Qhat^T, each entry's products summed by fused multiply-adds over the columns of
// the factors in order.  Each value of Q'
// is quantised by every row chunk and each value of Pt by every column tile (a few thousand
// values per block, against the block's 64 VEC x RC elements of E).
template <int RANK, int VEC, int RC>
__global__ __launch_bounds__(256) void k_lq_ef_update_q(const ElemJob J, const LqWorkerPtrs W,
                                                        const float *tab_p, int Lp, float tlp,
                                                        const float *tab_q, int Lq, float tlq,
                                                        float alpha) {
  constexpr int COLS = 64 * VEC;
  __shared__ float thr[2][128];
  __shared__ float lvl[2][128];
  __shared__ float qh[COLS * RANK];
  __shared__ float ph[RC * RANK];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t n = J.n, m = J.m;
  const int64_t j0 = (int64_t)blockIdx.x * COLS, r0 = (int64_t)blockIdx.y * RC;
  float *__restrict__ E = W.E[0];
  float *__restrict__ Qh = W.Q[0];
  // the wave's first RB rows of its columns are loaded before the factors are quantised, so
  // that the quantisation runs while they are in flight
  constexpr int RB = 4;  // rows loaded together per wave
  const int64_t j = j0 + (int64_t)lane * VEC;
  const int64_t r1 = r0 + RC < n ? r0 + RC : n;
  int64_t rb = r0 + w * RB;
  float mv[RB][VEC];
  if (j < m)
#pragma unroll
    for (int u = 0; u < RB; ++u)
      if (rb + u < r1) ldv<VEC>(E + (rb + u) * m + j, mv[u]);
  if (tid < Lp) thr[0][tid] = tab_p[tid];
  if (tid <= Lp) lvl[0][tid] = tab_p[Lp + tid];
  if (tid < Lq) thr[1][tid] = tab_q[tid];
  if (tid <= Lq) lvl[1][tid] = tab_q[Lq + tid];
  __syncthreads();
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid < 2 * RANK) {
    const float mxv = __uint_as_float(J.cmax_bits[tid]);
    if (tid < RANK) J.p_colmax[tid] = mxv; else J.q_colmax[tid - RANK] = mxv;
  }
  for (int e = tid; e < COLS * RANK; e += 256) {
    const int64_t i = j0 * RANK + e;  // element (j0 + e / RANK, e % RANK) of Q'
    float fh = 0.0f;
    if (i < m * RANK) {
      int8_t code;
      logq_one(J.Qn[i], __uint_as_float(J.cmax_bits[RANK + e % RANK]), thr[1], lvl[1], Lq,
               alpha, tlq, code, fh);
      if (blockIdx.y == 0) {
        J.q_codes[i] = code;
        Qh[i] = fh;
      }
    }
    qh[e] = fh;
  }
  for (int e = tid; e < RC * RANK; e += 256) {
    const int64_t i = r0 * RANK + e;  // element (r0 + e / RANK, e % RANK) of Pt
    float fh = 0.0f;
    if (i < n * RANK) {
      int8_t code;
      logq_one(J.Pt[i], __uint_as_float(J.cmax_bits[e % RANK]), thr[0], lvl[0], Lp, alpha, tlp,
               code, fh);
      if (blockIdx.x == 0) {
        J.p_codes[i] = code;
        if (J.p_hat) J.p_hat[i] = fh;
      }
    }
    ph[e] = fh;
  }
  __syncthreads();
  if (j >= m) return;
  float q[RANK][VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v)
#pragma unroll
    for (int c = 0; c < RANK; ++c) q[c][v] = qh[(lane * VEC + v) * RANK + c];
  for (; rb < r1; rb += 4 * RB) {
    // the wave's next RB rows are loaded before this batch is updated and stored
    const int64_t rn = rb + 4 * RB;
    float nx[RB][VEC];
#pragma unroll
    for (int u = 0; u < RB; ++u)
      if (rn + u < r1) ldv<VEC>(E + (rn + u) * m + j, nx[u]);
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      if (rb + u < r1) {
        const int lr = (int)(rb + u - r0);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          float s = 0.0f;
#pragma unroll
          for (int c = 0; c < RANK; ++c) s = fmaf(ph[lr * RANK + c], q[c][v], s);
          mv[u][v] -= s;
        }
        stv<VEC>(E + (rb + u) * m + j, mv[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < RB; ++u)
#pragma unroll
      for (int v = 0; v < VEC; ++v) mv[u][v] = nx[u][v];
  }
}

// Pass 3 of one worker at ranks above kFoldRankMax, the factors already quantised by
// k_lq_quant_elems: E <- E - Phat Qhat^T (Qhat row-major m x RANK), 4 rows per block, each
// entry's products summed by fused multiply-adds over the columns in order (the same
// arithmetic as k_lq_ef_update_q).
template <int RANK, int VEC>
__global__ __launch_bounds__(kBlockA) void k_lq_ef_update(float *__restrict__ E,
                                                          const float *__restrict__ Ph,
                                                          const float *__restrict__ Qh,
                                                          int64_t n, int64_t m) {
  const int64_t row0 = (int64_t)blockIdx.x * kRowsA;
  float p[kRowsA][RANK];
#pragma unroll
  for (int rr = 0; rr < kRowsA; ++rr)
#pragma unroll
    for (int c = 0; c < RANK; ++c) p[rr][c] = row0 + rr < n ? Ph[(row0 + rr) * RANK + c] : 0.0f;
  const int nr = n - row0 < kRowsA ? (int)(n - row0) : kRowsA;
  for (int64_t j = (int64_t)threadIdx.x * VEC; j < m; j += (int64_t)kBlockA * VEC) {
    float q[RANK][VEC];
    float mv[kRowsA][VEC];
#pragma unroll
    for (int rr = 0; rr < kRowsA; ++rr)
      if (rr < nr) ldv<VEC>(E + (row0 + rr) * m + j, mv[rr]);
    load_q_rows<RANK, VEC>(Qh, j, q);
#pragma unroll
    for (int rr = 0; rr < kRowsA; ++rr) {
      if (rr < nr) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          float s = 0.0f;
#pragma unroll
          for (int c = 0; c < RANK; ++c) s = fmaf(p[rr][c], q[c][v], s);
          mv[rr][v] -= s;
        }
        stv<VEC>(E + (row0 + rr) * m + j, mv[rr]);
      }
    }
  }
}

// Last pass of a step of K workers: the approximate global gradient
// Ghat = (1/K) sum_w Phat_w Qhat_w^T for 4 rows at a time (sums over workers, then columns of
// the factors, by fused multiply-add), stored once, and E_w <- M_w - Ghat for every worker
// (E_w holds M_w).  The 4 rows' decoded P entries of every worker are staged in LDS (at most
// 16 x 4 x 8 floats); each worker's decoded Q rows are read from its own Q (m x r, L2-resident).
// Two workers' rows are loaded before either is stored.  At K = 1 this is the one-worker update with
// Ghat also stored.
template <int RANK, int VEC>
__global__ __launch_bounds__(kBlockA) void k_lq_mean_ef(const LqWorkerPtrs W, int K,
                                                        const float *__restrict__ Ph_all,
                                                        float *__restrict__ Ghat, float invK,
                                                        int64_t n, int64_t m) {
  __shared__ float ps[kLqMaxWorkers * kRowsA * RANK];
  const int64_t row0 = (int64_t)blockIdx.x * kRowsA;
  const int nr = n - row0 < kRowsA ? (int)(n - row0) : kRowsA;
  for (int t = threadIdx.x; t < K * kRowsA * RANK; t += kBlockA) {
    const int wk = t / (kRowsA * RANK), rr = (t / RANK) % kRowsA, c = t % RANK;
    ps[t] = rr < nr ? Ph_all[((int64_t)wk * n + row0 + rr) * RANK + c] : 0.0f;
  }
  __syncthreads();
  for (int64_t j = (int64_t)threadIdx.x * VEC; j < m; j += (int64_t)kBlockA * VEC) {
    float g[kRowsA][VEC];
#pragma unroll
    for (int rr = 0; rr < kRowsA; ++rr)
#pragma unroll
      for (int v = 0; v < VEC; ++v) g[rr][v] = 0.0f;
#pragma unroll 1
    for (int wk = 0; wk < K; ++wk) {
      float q[RANK][VEC];
      load_q_rows<RANK, VEC>(W.Q[wk], j, q);
#pragma unroll
      for (int rr = 0; rr < kRowsA; ++rr) {
        float p[RANK];
#pragma unroll
        for (int c = 0; c < RANK; ++c) p[c] = ps[(wk * kRowsA + rr) * RANK + c];
#pragma unroll
        for (int v = 0; v < VEC; ++v)
#pragma unroll
          for (int c = 0; c < RANK; ++c) g[rr][v] = fmaf(p[c], q[c][v], g[rr][v]);
      }
    }
#pragma unroll
    for (int rr = 0; rr < kRowsA; ++rr)
      if (rr < nr) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) g[rr][v] *= invK;
        stv<VEC>(Ghat + (row0 + rr) * m + j, g[rr]);
      }
#pragma unroll 1
    for (int wk = 0; wk < K; wk += 2) {
      const bool two = wk + 1 < K;
      float *E0 = W.E[wk];
      float *E1 = two ? W.E[wk + 1] : E0;
      float a[kRowsA][VEC], b[kRowsA][VEC];
#pragma unroll
      for (int rr = 0; rr < kRowsA; ++rr) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) b[rr][v] = 0.0f;
        if (rr < nr) {
          ldv<VEC>(E0 + (row0 + rr) * m + j, a[rr]);
          if (two) ldv<VEC>(E1 + (row0 + rr) * m + j, b[rr]);
        }
      }
#pragma unroll
      for (int rr = 0; rr < kRowsA; ++rr)
        if (rr < nr) {
#pragma unroll
          for (int v = 0; v < VEC; ++v) {
            a[rr][v] -= g[rr][v];
            b[rr][v] -= g[rr][v];
          }
          stv<VEC>(E0 + (row0 + rr) * m + j, a[rr]);
          if (two) stv<VEC>(E1 + (row0 + rr) * m + j, b[rr]);
        }
    }
  }
}

// ---------------------------------------------------------------- host helpers
size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Grow the scratch.  The buffer it replaces is retired, not freed: work already enqueued, or
// a captured graph, may still use it (it is freed by lq_trim or lq_release).
hipError_t ensure(LqState &st, size_t bytes, hipStream_t) {
  if (bytes <= st.bytes) return hipSuccess;
  const size_t want = bytes + bytes / 4;
  void *fresh = nullptr;
  if (hipMalloc(&fresh, want) != hipSuccess) return hipErrorOutOfMemory;
  if (st.scratch) st.retired.push_back(st.scratch);
  st.scratch = fresh;
  st.bytes = want;
  return hipSuccess;
}

// Boundaries b_k = ((1+alpha)^((k+1/2)/L) - 1)/alpha rounded up to fp32 (so y >= thr[k] holds
// exactly when y >= b_k), and levels d_k = fp32(((1+alpha)^(k/L) - 1)/alpha).
hipError_t tables(LqState &st, double alpha, int bits, hipStream_t s, const LqTables **out) {
  auto key = std::make_pair(alpha, bits);
  auto it = st.tables.find(key);
  if (it == st.tables.end()) {
    LqTables t;
    t.L = (1 << (bits - 1)) - 1;
    const int L = t.L;
    t.host.assign(2 * L + 1, 0.0f);
    const double lg = std::log1p(alpha);
    for (int k = 0; k < L; ++k) {
      const double b = std::expm1(lg * (2.0 * k + 1.0) / (2.0 * L)) / alpha;
      float f = (float)b;
      if ((double)f < b) f = std::nextafter(f, INFINITY);
      t.host[k] = f;
    }
    for (int k = 0; k <= L; ++k) t.host[L + k] = (float)(std::expm1(lg * k / L) / alpha);
    t.alpha = (float)alpha;
    t.tl = (float)(L / std::log2(1.0 + alpha));
    hipError_t e = hipMalloc(&t.dev, t.host.size() * sizeof(float));
    if (e != hipSuccess) return hipErrorOutOfMemory;
    e = hipMemcpyAsync(t.dev, t.host.data(), t.host.size() * sizeof(float), hipMemcpyHostToDevice, s);
    if (e != hipSuccess) {
      (void)hipFree(t.dev);
      return e;
    }
    it = st.tables.emplace(key, std::move(t)).first;
  }
  *out = &it->second;
  return hipSuccess;
}

// Scratch of a step, every buffer stacked by worker.
struct StepBufs {
  float *P, *Pt, *part, *Qn, *Ph;
  double *gpart, *T;
  unsigned *cmax_bits;  // 2 RANK words per worker: Pt's column maxima, then Q''s
  int nchunks, rows_chunk;
  int64_t nblocks;
};

// One step of K workers (K = 1: the single-worker step).  Every per-worker kernel runs all
// workers in one launch, the worker taken from a grid dimension.
struct StepIO {
  LqWorkerPtrs W;
  int K;
  int64_t n, m;
  int8_t *p_codes, *q_codes;     // stacked by worker
  float *p_colmax, *q_colmax;    // stacked by worker
  float *p_hat, *p_pre, *q_pre;  // stacked by worker, or null
  float *G_hat;                  // null: one worker, E <- M - Phat Qhat^T
};

template <int RANK, int VEC>
void launch_step(const StepIO &io, const StepBufs &b, const LqTables &tp, const LqTables &tq,
                 hipStream_t s) {
  const int64_t n = io.n, m = io.m;
  const unsigned K = (unsigned)io.K;
  if ((double)K * (double)n * (double)m * 4.0 > kMallBytes)
    hipLaunchKernelGGL((k_lq_ef_mq<RANK, VEC, true>), dim3((unsigned)b.nblocks, K), dim3(kBlockA),
                       0, s, io.W, b.P, b.gpart, n, m);
  else
    hipLaunchKernelGGL((k_lq_ef_mq<RANK, VEC, false>), dim3((unsigned)b.nblocks, K),
                       dim3(kBlockA), 0, s, io.W, b.P, b.gpart, n, m);
  hipLaunchKernelGGL((k_lq_solve<RANK>), dim3(K), dim3(solve_block<RANK>()), 0, s, b.gpart,
                     b.nblocks, b.T, b.cmax_bits, (double)m * 0x1p-48);
  const dim3 gcol((unsigned)((m + 64 * VEC - 1) / (64 * VEC)), (unsigned)b.nchunks, K);
  if (b.rows_chunk == 64)
    hipLaunchKernelGGL((k_lq_mtp<RANK, VEC, 64>), gcol, dim3(kWavesC * 64), 0, s, io.W, b.P,
                       b.T, b.Pt, io.p_pre, b.cmax_bits, b.part, n, m);
  else
    hipLaunchKernelGGL((k_lq_mtp<RANK, VEC, 128>), gcol, dim3(kWavesC * 64), 0, s, io.W, b.P,
                       b.T, b.Pt, io.p_pre, b.cmax_bits, b.part, n, m);
  if (m * RANK <= kQsumShort)
    hipLaunchKernelGGL((k_lq_qsum<RANK, 8>), dim3((unsigned)((m * RANK + 31) / 32), K),
                       dim3(256), 0, s, b.part, b.Qn, io.q_pre, b.cmax_bits, m * RANK,
                       b.nchunks);
  else
    hipLaunchKernelGGL((k_lq_qsum<RANK, 1>), dim3((unsigned)((m * RANK + 255) / 256), K),
                       dim3(256), 0, s, b.part, b.Qn, io.q_pre, b.cmax_bits, m * RANK,
                       b.nchunks);
  ElemJob je{b.Pt, b.Qn, n, m, RANK, b.cmax_bits, io.p_codes, io.q_codes, io.p_colmax,
             io.q_colmax, b.Ph, io.p_hat, nullptr};
  if (io.G_hat) {
    hipLaunchKernelGGL(k_lq_quant_elems, dim3((unsigned)(((n + m) * RANK + 255) / 256), K),
                       dim3(256), 0, s, je, io.W, tp.dev, tp.L, tp.tl, tq.dev, tq.L, tq.tl,
                       tp.alpha);
    hipLaunchKernelGGL((k_lq_mean_ef<RANK, VEC>), dim3((unsigned)b.nblocks), dim3(kBlockA), 0,
                       s, io.W, io.K, b.Ph, io.G_hat, 1.0f / (float)io.K, n, m);
  } else if (RANK > kFoldRankMax) {
    // one worker at a higher rank: the quantiser, then the plain last pass
    hipLaunchKernelGGL(k_lq_quant_elems, dim3((unsigned)(((n + m) * RANK + 255) / 256), K),
                       dim3(256), 0, s, je, io.W, tp.dev, tp.L, tp.tl, tq.dev, tq.L, tq.tl,
                       tp.alpha);
    hipLaunchKernelGGL((k_lq_ef_update<RANK, VEC>), dim3((unsigned)b.nblocks), dim3(kBlockA),
                       0, s, io.W.E[0], b.Ph, io.W.Q[0], n, m);
  } else {
    // one worker: the quantiser runs inside the last pass
    constexpr int RQ = rows_q<RANK>();
    const dim3 g3((unsigned)((m + 64 * VEC - 1) / (64 * VEC)), (unsigned)((n + RQ - 1) / RQ));
    hipLaunchKernelGGL((k_lq_ef_update_q<RANK, VEC, RQ>), g3, dim3(256), 0, s, je, io.W,
                       tp.dev, tp.L, tp.tl, tq.dev, tq.L, tq.tl, tp.alpha);
  }
}

template <int RANK>
void launch_step_v(const StepIO &io, bool vec4, const StepBufs &b, const LqTables &tp,
                   const LqTables &tq, hipStream_t s) {
  if (vec4)
    launch_step<RANK, 4>(io, b, tp, tq, s);
  else
    launch_step<RANK, 1>(io, b, tp, tq, s);
}

}  // namespace

hipError_t lq_logquant(LqState &st, const float *F, int64_t rows, int r, double alpha, int bits,
                       int8_t *codes, float *colmax, float *Fhat, hipStream_t s) {
  const LqTables *tab = nullptr;
  hipError_t e = tables(st, alpha, bits, s, &tab);
  if (e != hipSuccess) return e;
  ColJob j{F, rows, r, codes, colmax, Fhat, nullptr};
  hipLaunchKernelGGL(k_lq_quant_cols, dim3(r), dim3(1024), 0, s, j, j, r, tab->dev, tab->L,
                     tab->alpha, tab->tl);
  return hipGetLastError();
}

namespace {

// Scratch for K workers, the launch shapes, and the launches.
hipError_t run_step(LqState &st, const StepIO &io, int r, double alpha, int bits_p, int bits_q,
                    hipStream_t s) {
  const LqTables *tp = nullptr, *tq = nullptr;
  hipError_t e = tables(st, alpha, bits_p, s, &tp);
  if (e != hipSuccess) return e;
  e = tables(st, alpha, bits_q, s, &tq);  // map insertion keeps tp valid
  if (e != hipSuccess) return e;
  const int64_t n = io.n, m = io.m;
  const size_t K = (size_t)io.K;
  StepBufs b;
  const bool vec4 = (m % 4) == 0;
  const int64_t col_tiles = vec4 ? (m + 255) / 256 : (m + 63) / 64;
  b.rows_chunk = col_tiles * ((n + 127) / 128) * (int64_t)K < kColBlocksMin ? 64 : 128;
  b.nchunks = (int)((n + b.rows_chunk - 1) / b.rows_chunk);
  b.nblocks = (n + kRowsA - 1) / kRowsA;
  if (b.nchunks > 65535) return hipErrorInvalidValue;  // chunks are a grid dimension
  const int64_t ng = r * (r + 1) / 2;
  size_t off = 0;
  const size_t oP = off; off += align256(K * sizeof(float) * n * r);
  const size_t oG = off; off += align256(K * sizeof(double) * b.nblocks * ng);
  const size_t oPt = off; off += align256(K * sizeof(float) * n * r);
  const size_t oPart = off; off += align256(K * sizeof(float) * (size_t)b.nchunks * m * r);
  const size_t oQn = off; off += align256(K * sizeof(float) * m * r);
  const size_t oPh = off; off += align256(K * sizeof(float) * n * r);
  const size_t oT = off; off += align256(K * sizeof(double) * r * r);
  const size_t oC = off; off += align256(K * sizeof(unsigned) * 2 * r);
  e = ensure(st, off, s);
  if (e != hipSuccess) return e;
  char *base = static_cast<char *>(st.scratch);
  b.P = reinterpret_cast<float *>(base + oP);
  b.gpart = reinterpret_cast<double *>(base + oG);
  b.Pt = reinterpret_cast<float *>(base + oPt);
  b.part = reinterpret_cast<float *>(base + oPart);
  b.Qn = reinterpret_cast<float *>(base + oQn);
  b.Ph = reinterpret_cast<float *>(base + oPh);
  b.T = reinterpret_cast<double *>(base + oT);
  b.cmax_bits = reinterpret_cast<unsigned *>(base + oC);
  switch (r) {
    case 1: launch_step_v<1>(io, vec4, b, *tp, *tq, s); break;
    case 2: launch_step_v<2>(io, vec4, b, *tp, *tq, s); break;
    case 3: launch_step_v<3>(io, vec4, b, *tp, *tq, s); break;
    case 4: launch_step_v<4>(io, vec4, b, *tp, *tq, s); break;
    case 5: launch_step_v<5>(io, vec4, b, *tp, *tq, s); break;
    case 6: launch_step_v<6>(io, vec4, b, *tp, *tq, s); break;
    case 7: launch_step_v<7>(io, vec4, b, *tp, *tq, s); break;
    case 8: launch_step_v<8>(io, vec4, b, *tp, *tq, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t lq_step(LqState &st, const LqStepArgs &a, hipStream_t s) {
  StepIO io;
  std::memset(&io, 0, sizeof io);
  io.W.G[0] = a.G;
  io.W.E[0] = a.E;
  io.W.Q[0] = a.Q;
  io.K = 1;
  io.n = a.n;
  io.m = a.m;
  io.p_codes = a.p_codes;
  io.q_codes = a.q_codes;
  io.p_colmax = a.p_colmax;
  io.q_colmax = a.q_colmax;
  io.p_hat = a.p_hat;
  io.p_pre = a.p_pre;
  io.q_pre = a.q_pre;
  io.G_hat = nullptr;
  return run_step(st, io, a.r, a.alpha, a.bits_p, a.bits_q, s);
}

hipError_t lq_step_workers(LqState &st, const LqWorkersStepArgs &a, hipStream_t s) {
  if (a.K < 1 || a.K > kLqMaxWorkers) return hipErrorInvalidValue;
  StepIO io;
  std::memset(&io, 0, sizeof io);
  io.W = a.W;
  io.K = a.K;
  io.n = a.n;
  io.m = a.m;
  io.p_codes = a.p_codes;
  io.q_codes = a.q_codes;
  io.p_colmax = a.p_colmax;
  io.q_colmax = a.q_colmax;
  io.G_hat = a.G_hat;
  io.p_pre = a.p_pre;
  io.q_pre = a.q_pre;
  return run_step(st, io, a.r, a.alpha, a.bits_p, a.bits_q, s);
}

void lq_trim(LqState &st) {
  for (void *p : st.retired) (void)hipFree(p);
  st.retired.clear();
}

void lq_release(LqState &st) {
  lq_trim(st);
  if (st.scratch) (void)hipFree(st.scratch);
  st.scratch = nullptr;
  st.bytes = 0;
  for (auto &kv : st.tables) (void)hipFree(kv.second.dev);
  st.tables.clear();
}

}  // namespace gq
