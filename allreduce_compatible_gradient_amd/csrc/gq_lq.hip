// gq_lq.hip -- gfx950 kernels of one LQ-SGD compressor step (one worker).
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
//   pass 3  E <- E - Phat Q'hat^T               (read E; write E)      k_lq_ef_update
// Row passes give each block 4 rows so every Q value fetched (from L2: Q is at most
// m x 8 fp32) is used 4 times; Q is read in its own row-major layout (a thread's 4 columns
// are 4r consecutive floats), so no transposed copy is made.  The column pass gives each
// 512-thread block 128 rows x (64*VEC) columns and reduces its 8 waves in LDS, so the
// per-chunk partials stay a few percent of the pass.
// Orthonormalisation: pass 1 also emits each block's r x r Gram contribution (products of the
// fp32 P values, exact in fp64); k_lq_solve sums them in a fixed order and runs Cholesky-QR
// twice in r x r space -- T1 from G, then T2 from T1^T G T1, which measures and removes the
// error of the first factorisation -- and applies T = T1 T2 to P.  In exact arithmetic P T is
// the Gram-Schmidt Q factor of P (columns in order; a column with no remaining norm is zero).
// The log quantiser encodes with a table of the L bin boundaries rounded up to fp32 (so
// "y >= boundary" is decided exactly) and decodes with a table of the L+1 Eq. 6 levels.
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
constexpr int kRowsC = 128;    // rows per chunk in the column pass
constexpr int kWavesC = 8;
constexpr int kBlockSolve = 256;

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
__device__ __forceinline__ void stv(float *p, const float (&v)[VEC]) {
  if constexpr (VEC == 4) {
    f32x4 t = {v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4 *>(p) = t;
  } else {
    *p = v[0];
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

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
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
// share of the Gram matrix P^T P (packed upper triangle, fp64).
template <int RANK, int VEC>
__global__ __launch_bounds__(kBlockA) void k_lq_ef_mq(const float *__restrict__ G,
                                                      float *__restrict__ E,
                                                      const float *__restrict__ Q,
                                                      float *__restrict__ P,
                                                      double *__restrict__ gpart, int64_t n,
                                                      int64_t m) {
  constexpr int NG = RANK * (RANK + 1) / 2;
  __shared__ float red[kBlockA / 64][kRowsA * RANK];
  __shared__ float pv[kRowsA * RANK];
  const int64_t row0 = (int64_t)blockIdx.x * kRowsA;
  float acc[kRowsA][RANK];
#pragma unroll
  for (int rr = 0; rr < kRowsA; ++rr)
#pragma unroll
    for (int c = 0; c < RANK; ++c) acc[rr][c] = 0.0f;
  for (int64_t j = (int64_t)threadIdx.x * VEC; j < m; j += (int64_t)kBlockA * VEC) {
    float q[RANK][VEC];
    load_q_rows<RANK, VEC>(Q, j, q);
#pragma unroll
    for (int rr = 0; rr < kRowsA; ++rr) {
      const int64_t row = row0 + rr;
      if (row < n) {
        float g[VEC], e[VEC], mv[VEC];
        ldv_nt<VEC>(G + row * m + j, g);
        ldv_nt<VEC>(E + row * m + j, e);
#pragma unroll
        for (int v = 0; v < VEC; ++v) mv[v] = g[v] + e[v];
        stv<VEC>(E + row * m + j, mv);
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
      const float s = wave_sum_f(acc[rr][c]);
      if (lane == 0) red[w][rr * RANK + c] = s;
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
    gpart[(int64_t)blockIdx.x * NG + threadIdx.x] = g;
  }
}

// Upper-triangular T with (P T)^T (P T) = I given G = P^T P: Gram-Schmidt carried out on G
// (column c: remove its components along the previous orthonormal columns, then normalise;
// a column with no remaining norm becomes zero).  RANK x RANK, in registers.
template <int RANK>
__device__ __forceinline__ void gram_schmidt_T(const double (&G)[RANK][RANK],
                                               double (&T)[RANK][RANK]) {
#pragma unroll
  for (int a = 0; a < RANK; ++a)
#pragma unroll
    for (int b = 0; b < RANK; ++b) T[a][b] = 0.0;
#pragma unroll
  for (int c = 0; c < RANK; ++c) {
    double wv[RANK];
#pragma unroll
    for (int a = 0; a < RANK; ++a) wv[a] = a == c ? 1.0 : 0.0;
#pragma unroll
    for (int j = 0; j < c; ++j) {
      double d = 0.0;  // (P T_j)^T (P wv) = T_j^T G wv
#pragma unroll
      for (int a = 0; a <= j; ++a) {
        double gw = 0.0;
#pragma unroll
        for (int b = 0; b <= c; ++b) gw += G[a][b] * wv[b];
        d += T[a][j] * gw;
      }
#pragma unroll
      for (int a = 0; a <= j; ++a) wv[a] -= d * T[a][j];
    }
    double nrm2 = 0.0;
#pragma unroll
    for (int a = 0; a <= c; ++a) {
      double gw = 0.0;
#pragma unroll
      for (int b = 0; b <= c; ++b) gw += G[a][b] * wv[b];
      nrm2 += wv[a] * gw;
    }
    const double inv = nrm2 > 0.0 ? 1.0 / sqrt(nrm2) : 0.0;
#pragma unroll
    for (int a = 0; a <= c; ++a) T[a][c] = wv[a] * inv;
  }
}

// Orthonormalise P: fixed-order sum of the block Gram partials, two Cholesky-QR rounds in
// r x r space (one thread), then Pt = fp32(P T) with fp64 products.
template <int RANK>
__global__ __launch_bounds__(kBlockSolve) void k_lq_solve(const float *__restrict__ P,
                                                          const double *__restrict__ gpart,
                                                          int64_t nblocks, float *__restrict__ Pt,
                                                          float *__restrict__ p_pre, int64_t n) {
  constexpr int NG = RANK * (RANK + 1) / 2;
  __shared__ double red[kBlockSolve / 64][NG];
  __shared__ double Gs[RANK][RANK];
  __shared__ double Ts[RANK][RANK];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  double g[NG];
#pragma unroll
  for (int t = 0; t < NG; ++t) g[t] = 0.0;
  for (int64_t b = tid; b < nblocks; b += kBlockSolve)
#pragma unroll
    for (int t = 0; t < NG; ++t) g[t] += gpart[b * NG + t];
#pragma unroll
  for (int t = 0; t < NG; ++t) {
    const double s = wave_sum_d(g[t]);
    if (lane == 0) red[w][t] = s;
  }
  __syncthreads();
  if (tid < NG) {
    double s = 0.0;
    for (int i = 0; i < kBlockSolve / 64; ++i) s += red[i][tid];
    int a, b;
    tri_index<RANK>(tid, a, b);
    Gs[a][b] = s;
    Gs[b][a] = s;
  }
  __syncthreads();
  if (tid == 0) {
    double G[RANK][RANK], T1[RANK][RANK], T2[RANK][RANK];
#pragma unroll
    for (int a = 0; a < RANK; ++a)
#pragma unroll
      for (int b = 0; b < RANK; ++b) G[a][b] = Gs[a][b];
    gram_schmidt_T<RANK>(G, T1);
    // G <- T1^T G T1 (the Gram matrix of P T1), with T2 as scratch for G T1
#pragma unroll
    for (int a = 0; a < RANK; ++a)
#pragma unroll
      for (int c = 0; c < RANK; ++c) {
        double s = 0.0;
#pragma unroll
        for (int b = 0; b <= c; ++b) s += G[a][b] * T1[b][c];
        T2[a][c] = s;
      }
#pragma unroll
    for (int a = 0; a < RANK; ++a)
#pragma unroll
      for (int c = 0; c < RANK; ++c) {
        double s = 0.0;
#pragma unroll
        for (int b = 0; b <= a; ++b) s += T1[b][a] * T2[b][c];
        G[a][c] = s;
      }
    gram_schmidt_T<RANK>(G, T2);
#pragma unroll
    for (int a = 0; a < RANK; ++a)
#pragma unroll
      for (int c = 0; c < RANK; ++c) {
        double s = 0.0;
#pragma unroll
        for (int k = a; k <= c; ++k) s += T1[a][k] * T2[k][c];
        Ts[a][c] = s;
      }
  }
  __syncthreads();
  for (int64_t i = tid; i < n; i += kBlockSolve) {
    double v[RANK];
#pragma unroll
    for (int c = 0; c < RANK; ++c) v[c] = (double)P[i * RANK + c];
#pragma unroll
    for (int c = 0; c < RANK; ++c) {
      double s = 0.0;
#pragma unroll
      for (int a = 0; a <= c; ++a) s += v[a] * Ts[a][c];
      const float o = (float)s;
      Pt[i * RANK + c] = o;
      if (p_pre) p_pre[i * RANK + c] = o;
    }
  }
}

// Pass 2 (partials): part[chunk][j][c] = sum over the chunk's rows of E[row][j] * Pt[row][c].
template <int RANK, int VEC>
__global__ __launch_bounds__(kWavesC * 64) void k_lq_mtp(const float *__restrict__ M,
                                                         const float *__restrict__ Pt,
                                                         float *__restrict__ part, int64_t n,
                                                         int64_t m) {
  __shared__ float red[kWavesC][64 * VEC];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t j = (int64_t)blockIdx.x * 64 * VEC + (int64_t)lane * VEC;
  const int64_t r0 = (int64_t)blockIdx.y * kRowsC;
  const int64_t r1 = r0 + kRowsC < n ? r0 + kRowsC : n;
  const bool active = j < m;
  float acc[VEC][RANK];
#pragma unroll
  for (int v = 0; v < VEC; ++v)
#pragma unroll
    for (int c = 0; c < RANK; ++c) acc[v][c] = 0.0f;
  if (active) {
    for (int64_t row = r0 + w; row < r1; row += kWavesC) {
      float p[RANK], mv[VEC];
#pragma unroll
      for (int c = 0; c < RANK; ++c) p[c] = Pt[row * RANK + c];
      ldv_nt<VEC>(M + row * m + j, mv);
#pragma unroll
      for (int v = 0; v < VEC; ++v)
#pragma unroll
        for (int c = 0; c < RANK; ++c) acc[v][c] = fmaf(mv[v], p[c], acc[v][c]);
    }
  }
#pragma unroll
  for (int c = 0; c < RANK; ++c) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) red[w][lane * VEC + v] = acc[v][c];
    __syncthreads();
    if (w == 0 && active) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        float s = 0.0f;
        for (int i = 0; i < kWavesC; ++i) s += red[i][lane * VEC + v];
        part[((int64_t)blockIdx.y * m + j + v) * RANK + c] = s;
      }
    }
    __syncthreads();
  }
}

// Pass 2 (final): Q'[j][c] = sum over chunks, in chunk order.
__global__ void k_lq_qsum(const float *part, float *Qn, float *q_pre, int64_t count,
                          int nchunks) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) {
    float s = 0.0f;
    for (int ch = 0; ch < nchunks; ++ch) s += part[(int64_t)ch * count + i];
    Qn[i] = s;
    if (q_pre) q_pre[i] = s;
  }
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

// One block per column: max magnitude, then Eq. 5 encode by the boundary table and Eq. 6
// decode by the level table.
__global__ __launch_bounds__(1024) void k_lq_quant_cols(ColJob j0, ColJob j1, int ncols0,
                                                        const float *tab, int L) {
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
    const float x = J.F[i * J.r + c];
    int k = 0;
    if (mx > 0.0f) {
      const float y = fabsf(x) / mx;  // IEEE division, in [0, 1]
      int lo = 0, hi = L;             // k = #{boundaries <= y}
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (thr[mid] <= y)
          lo = mid + 1;
        else
          hi = mid;
      }
      k = lo;
    }
    J.codes[i * J.r + c] = (int8_t)(x < 0.0f ? -k : k);
    const float v = lvl[k] * mx;
    const float fh = x < 0.0f ? -v : v;
    if (J.Fhat) J.Fhat[i * J.r + c] = fh;
    if (J.Fhat2) J.Fhat2[i * J.r + c] = fh;
  }
}

// Pass 3: E <- E - Phat Qhat^T (Qhat row-major m x RANK).
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
  for (int64_t j = (int64_t)threadIdx.x * VEC; j < m; j += (int64_t)kBlockA * VEC) {
    float q[RANK][VEC];
    load_q_rows<RANK, VEC>(Qh, j, q);
#pragma unroll
    for (int rr = 0; rr < kRowsA; ++rr) {
      const int64_t row = row0 + rr;
      if (row < n) {
        float mv[VEC];
        ldv_nt<VEC>(E + row * m + j, mv);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          float s = 0.0f;
#pragma unroll
          for (int c = 0; c < RANK; ++c) s = fmaf(p[rr][c], q[c][v], s);
          mv[v] -= s;
        }
        stv<VEC>(E + row * m + j, mv);
      }
    }
  }
}

// ---------------------------------------------------------------- host helpers
size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

hipError_t ensure(LqState &st, size_t bytes, hipStream_t s) {
  if (bytes <= st.bytes) return hipSuccess;
  if (st.scratch) {
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return e;
    (void)hipFree(st.scratch);
    st.scratch = nullptr;
    st.bytes = 0;
  }
  const size_t want = bytes + bytes / 4;
  hipError_t e = hipMalloc(&st.scratch, want);
  if (e != hipSuccess) {
    st.scratch = nullptr;
    return hipErrorOutOfMemory;
  }
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

struct StepBufs {
  float *P, *Pt, *part, *Qn, *Ph;
  double *gpart;
  int nchunks;
  int64_t nblocks;
};

template <int RANK, int VEC>
void launch_step(const LqStepArgs &a, const StepBufs &b, const LqTables &tab, hipStream_t s) {
  const int64_t n = a.n, m = a.m;
  hipLaunchKernelGGL((k_lq_ef_mq<RANK, VEC>), dim3((unsigned)b.nblocks), dim3(kBlockA), 0, s,
                     a.G, a.E, a.Q, b.P, b.gpart, n, m);
  hipLaunchKernelGGL((k_lq_solve<RANK>), dim3(1), dim3(kBlockSolve), 0, s, b.P, b.gpart,
                     b.nblocks, b.Pt, a.p_pre, n);
  hipLaunchKernelGGL((k_lq_mtp<RANK, VEC>),
                     dim3((unsigned)((m + 64 * VEC - 1) / (64 * VEC)), (unsigned)b.nchunks),
                     dim3(kWavesC * 64), 0, s, a.E, b.Pt, b.part, n, m);
  hipLaunchKernelGGL(k_lq_qsum, dim3((unsigned)((m * RANK + 255) / 256)), dim3(256), 0, s,
                     b.part, b.Qn, a.q_pre, m * RANK, b.nchunks);
  ColJob jp{b.Pt, n, RANK, a.p_codes, a.p_colmax, b.Ph, a.p_hat};
  ColJob jq{b.Qn, m, RANK, a.q_codes, a.q_colmax, a.Q, nullptr};
  hipLaunchKernelGGL(k_lq_quant_cols, dim3(2 * RANK), dim3(1024), 0, s, jp, jq, RANK, tab.dev,
                     tab.L);
  hipLaunchKernelGGL((k_lq_ef_update<RANK, VEC>), dim3((unsigned)b.nblocks), dim3(kBlockA), 0,
                     s, a.E, b.Ph, a.Q, n, m);
}

template <int RANK>
void launch_step_v(const LqStepArgs &a, bool vec4, const StepBufs &b, const LqTables &tab,
                   hipStream_t s) {
  if (vec4)
    launch_step<RANK, 4>(a, b, tab, s);
  else
    launch_step<RANK, 1>(a, b, tab, s);
}

}  // namespace

hipError_t lq_logquant(LqState &st, const float *F, int64_t rows, int r, double alpha, int bits,
                       int8_t *codes, float *colmax, float *Fhat, hipStream_t s) {
  const LqTables *tab = nullptr;
  hipError_t e = tables(st, alpha, bits, s, &tab);
  if (e != hipSuccess) return e;
  ColJob j{F, rows, r, codes, colmax, Fhat, nullptr};
  hipLaunchKernelGGL(k_lq_quant_cols, dim3(r), dim3(1024), 0, s, j, j, r, tab->dev, tab->L);
  return hipGetLastError();
}

hipError_t lq_step(LqState &st, const LqStepArgs &a, hipStream_t s) {
  const LqTables *tab = nullptr;
  hipError_t e = tables(st, a.alpha, a.bits, s, &tab);
  if (e != hipSuccess) return e;
  const int64_t n = a.n, m = a.m, r = a.r;
  StepBufs b;
  b.nchunks = (int)((n + kRowsC - 1) / kRowsC);
  b.nblocks = (n + kRowsA - 1) / kRowsA;
  const int64_t ng = r * (r + 1) / 2;
  size_t off = 0;
  const size_t oP = off; off += align256(sizeof(float) * n * r);
  const size_t oG = off; off += align256(sizeof(double) * b.nblocks * ng);
  const size_t oPt = off; off += align256(sizeof(float) * n * r);
  const size_t oPart = off; off += align256(sizeof(float) * (size_t)b.nchunks * m * r);
  const size_t oQn = off; off += align256(sizeof(float) * m * r);
  const size_t oPh = off; off += align256(sizeof(float) * n * r);
  e = ensure(st, off, s);
  if (e != hipSuccess) return e;
  char *base = static_cast<char *>(st.scratch);
  b.P = reinterpret_cast<float *>(base + oP);
  b.gpart = reinterpret_cast<double *>(base + oG);
  b.Pt = reinterpret_cast<float *>(base + oPt);
  b.part = reinterpret_cast<float *>(base + oPart);
  b.Qn = reinterpret_cast<float *>(base + oQn);
  b.Ph = reinterpret_cast<float *>(base + oPh);
  const bool vec4 = (m % 4) == 0;
  switch (a.r) {
    case 1: launch_step_v<1>(a, vec4, b, *tab, s); break;
    case 2: launch_step_v<2>(a, vec4, b, *tab, s); break;
    case 3: launch_step_v<3>(a, vec4, b, *tab, s); break;
    case 4: launch_step_v<4>(a, vec4, b, *tab, s); break;
    case 5: launch_step_v<5>(a, vec4, b, *tab, s); break;
    case 6: launch_step_v<6>(a, vec4, b, *tab, s); break;
    case 7: launch_step_v<7>(a, vec4, b, *tab, s); break;
    case 8: launch_step_v<8>(a, vec4, b, *tab, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

void lq_release(LqState &st) {
  if (st.scratch) (void)hipFree(st.scratch);
  st.scratch = nullptr;
  st.bytes = 0;
  for (auto &kv : st.tables) (void)hipFree(kv.second.dev);
  st.tables.clear();
}

}  // namespace gq
