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
// and the work is organised around the passes over the n x m matrix:
//   pass 1  E <- G + E and P = E Q          (read G, E; write E)      k_lq_ef_mq
//   pass 2  Q' = E^T P                      (read E)                  k_lq_mtp (+ k_lq_qsum)
//   pass 3  E <- E - Phat Q'hat^T           (read E; write E)         k_lq_ef_update
// Row passes give each block 4 rows so every Q value loaded from L2 is used 4 times; the
// column pass gives each 512-thread block 256 rows x (64*VEC) columns and reduces its 8 waves
// in LDS, so the per-chunk partials stay a few percent of the pass.  The orthonormalisation
// (a single workgroup) is two rounds of Cholesky-QR in fp64 (the r x r Gram matrix in one
// reduction, Gram-Schmidt on it by one thread, then P <- P T): in exact arithmetic this is
// the Gram-Schmidt Q factor, and the second round restores orthogonality to fp64 accuracy.
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

constexpr int kRowsA = 4;     // rows per block in the row passes
constexpr int kBlockA = 256;
constexpr int kRowsC = 256;   // rows per chunk in the column pass
constexpr int kWavesC = 8;
constexpr int kBlockOrth = 1024;

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

// Qt (r x m) <- Q (m x r).
__global__ void k_lq_transpose(const float *Q, float *Qt, int64_t m, int r) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < m * r) {
    const int64_t j = i / r;
    const int c = (int)(i % r);
    Qt[(int64_t)c * m + j] = Q[i];
  }
}

// Pass 1: E <- G + E (the gradient with the previous error fed back) and P = E Q.
template <int RANK, int VEC>
__global__ __launch_bounds__(kBlockA) void k_lq_ef_mq(const float *__restrict__ G,
                                                      float *__restrict__ E,
                                                      const float *__restrict__ Qt,
                                                      float *__restrict__ P, int64_t n,
                                                      int64_t m) {
  __shared__ float red[kBlockA / 64][kRowsA * RANK];
  const int64_t row0 = (int64_t)blockIdx.x * kRowsA;
  float acc[kRowsA][RANK];
#pragma unroll
  for (int rr = 0; rr < kRowsA; ++rr)
#pragma unroll
    for (int c = 0; c < RANK; ++c) acc[rr][c] = 0.0f;
  for (int64_t j = (int64_t)threadIdx.x * VEC; j < m; j += (int64_t)kBlockA * VEC) {
    float q[RANK][VEC];
#pragma unroll
    for (int c = 0; c < RANK; ++c) ldv<VEC>(Qt + (int64_t)c * m + j, q[c]);
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
    if (row < n) {
      float s = 0.0f;
      for (int i = 0; i < kBlockA / 64; ++i) s += red[i][t];
      P[row * RANK + t % RANK] = s;
    }
  }
}

// Orthonormalise the columns of P (n x RANK): two rounds of Cholesky-QR in fp64 on one
// workgroup.  Each round forms the Gram matrix, runs modified Gram-Schmidt on it (one thread,
// RANK x RANK) to get the upper-triangular T with P T orthonormal, and applies T.  A column
// whose remaining norm is not positive becomes zero.
template <int RANK>
__global__ __launch_bounds__(kBlockOrth) void k_lq_orth(const float *P, double *W, float *Pt,
                                                        float *p_pre, int64_t n) {
  constexpr int NG = RANK * (RANK + 1) / 2;
  __shared__ double red[kBlockOrth / 64][NG];
  __shared__ double Gm[RANK][RANK];
  __shared__ double T[RANK][RANK];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int64_t i = tid; i < n * RANK; i += kBlockOrth) W[i] = (double)P[i];
  __syncthreads();
  for (int round = 0; round < 2; ++round) {
    double g[NG];
#pragma unroll
    for (int t = 0; t < NG; ++t) g[t] = 0.0;
    for (int64_t i = tid; i < n; i += kBlockOrth) {
      double v[RANK];
#pragma unroll
      for (int c = 0; c < RANK; ++c) v[c] = W[i * RANK + c];
      int t = 0;
#pragma unroll
      for (int a = 0; a < RANK; ++a)
#pragma unroll
        for (int b = a; b < RANK; ++b) g[t++] += v[a] * v[b];
    }
#pragma unroll
    for (int t = 0; t < NG; ++t) {
      const double s = wave_sum_d(g[t]);
      if (lane == 0) red[w][t] = s;
    }
    __syncthreads();
    if (tid < NG) {
      double s = 0.0;
      for (int i = 0; i < kBlockOrth / 64; ++i) s += red[i][tid];
      int a = 0, t = tid;
      while (t >= RANK - a) {
        t -= RANK - a;
        ++a;
      }
      const int b = a + t;
      Gm[a][b] = s;
      Gm[b][a] = s;
    }
    __syncthreads();
    if (tid == 0) {
      for (int c = 0; c < RANK; ++c)
        for (int a = 0; a < RANK; ++a) T[a][c] = 0.0;
      for (int c = 0; c < RANK; ++c) {
        double wv[RANK];
        for (int a = 0; a < RANK; ++a) wv[a] = a == c ? 1.0 : 0.0;
        for (int j = 0; j < c; ++j) {
          // d = (P T_j)^T (P wv) = T_j^T G wv
          double d = 0.0;
          for (int a = 0; a <= j; ++a) {
            double gw = 0.0;
            for (int b = 0; b < RANK; ++b) gw += Gm[a][b] * wv[b];
            d += T[a][j] * gw;
          }
          for (int a = 0; a <= j; ++a) wv[a] -= d * T[a][j];
        }
        double nrm2 = 0.0;
        for (int a = 0; a < RANK; ++a) {
          double gw = 0.0;
          for (int b = 0; b < RANK; ++b) gw += Gm[a][b] * wv[b];
          nrm2 += wv[a] * gw;
        }
        const double inv = nrm2 > 0.0 ? 1.0 / sqrt(nrm2) : 0.0;
        for (int a = 0; a < RANK; ++a) T[a][c] = wv[a] * inv;
      }
    }
    __syncthreads();
    for (int64_t i = tid; i < n; i += kBlockOrth) {
      double v[RANK], o[RANK];
#pragma unroll
      for (int c = 0; c < RANK; ++c) v[c] = W[i * RANK + c];
#pragma unroll
      for (int c = 0; c < RANK; ++c) {
        double s = 0.0;
#pragma unroll
        for (int a = 0; a <= c; ++a) s += v[a] * T[a][c];
        o[c] = s;
      }
#pragma unroll
      for (int c = 0; c < RANK; ++c) W[i * RANK + c] = o[c];
    }
    __syncthreads();
  }
  for (int64_t i = tid; i < n * RANK; i += kBlockOrth) {
    const float v = (float)W[i];
    Pt[i] = v;
    if (p_pre) p_pre[i] = v;
  }
}

// Pass 2 (partials): part[chunk][j][c] = sum over the chunk's rows of E[row][j] * P[row][c].
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
  float *Fhat_t;         // r x rows or nullptr (transposed copy)
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
    if (J.Fhat_t) J.Fhat_t[(int64_t)c * J.rows + i] = fh;
  }
}

// Pass 3: E <- E - Phat Qhat^T.
template <int RANK, int VEC>
__global__ __launch_bounds__(kBlockA) void k_lq_ef_update(float *__restrict__ E,
                                                          const float *__restrict__ Ph,
                                                          const float *__restrict__ Qht,
                                                          int64_t n, int64_t m) {
  const int64_t row0 = (int64_t)blockIdx.x * kRowsA;
  float p[kRowsA][RANK];
#pragma unroll
  for (int rr = 0; rr < kRowsA; ++rr)
#pragma unroll
    for (int c = 0; c < RANK; ++c) p[rr][c] = row0 + rr < n ? Ph[(row0 + rr) * RANK + c] : 0.0f;
  for (int64_t j = (int64_t)threadIdx.x * VEC; j < m; j += (int64_t)kBlockA * VEC) {
    float q[RANK][VEC];
#pragma unroll
    for (int c = 0; c < RANK; ++c) ldv<VEC>(Qht + (int64_t)c * m + j, q[c]);
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

template <int RANK, int VEC>
void launch_step(const LqStepArgs &a, float *Qt, float *P, double *W, float *Pt, float *part,
                 int nchunks, float *Qn, float *Ph, float *Qht, const LqTables &tab,
                 hipStream_t s) {
  const int64_t n = a.n, m = a.m;
  hipLaunchKernelGGL(k_lq_transpose, dim3((unsigned)((m * RANK + 255) / 256)), dim3(256), 0, s,
                     a.Q, Qt, m, RANK);
  hipLaunchKernelGGL((k_lq_ef_mq<RANK, VEC>), dim3((unsigned)((n + kRowsA - 1) / kRowsA)),
                     dim3(kBlockA), 0, s, a.G, a.E, Qt, P, n, m);
  hipLaunchKernelGGL((k_lq_orth<RANK>), dim3(1), dim3(kBlockOrth), 0, s, P, W, Pt, a.p_pre, n);
  hipLaunchKernelGGL((k_lq_mtp<RANK, VEC>),
                     dim3((unsigned)((m + 64 * VEC - 1) / (64 * VEC)), (unsigned)nchunks),
                     dim3(kWavesC * 64), 0, s, a.E, Pt, part, n, m);
  hipLaunchKernelGGL(k_lq_qsum, dim3((unsigned)((m * RANK + 255) / 256)), dim3(256), 0, s, part,
                     Qn, a.q_pre, m * RANK, nchunks);
  ColJob jp{Pt, n, RANK, a.p_codes, a.p_colmax, Ph, a.p_hat, nullptr};
  ColJob jq{Qn, m, RANK, a.q_codes, a.q_colmax, a.Q, nullptr, Qht};
  hipLaunchKernelGGL(k_lq_quant_cols, dim3(2 * RANK), dim3(1024), 0, s, jp, jq, RANK, tab.dev,
                     tab.L);
  hipLaunchKernelGGL((k_lq_ef_update<RANK, VEC>), dim3((unsigned)((n + kRowsA - 1) / kRowsA)),
                     dim3(kBlockA), 0, s, a.E, Ph, Qht, n, m);
}

template <int RANK>
void launch_step_v(const LqStepArgs &a, bool vec4, float *Qt, float *P, double *W, float *Pt,
                   float *part, int nchunks, float *Qn, float *Ph, float *Qht,
                   const LqTables &tab, hipStream_t s) {
  if (vec4)
    launch_step<RANK, 4>(a, Qt, P, W, Pt, part, nchunks, Qn, Ph, Qht, tab, s);
  else
    launch_step<RANK, 1>(a, Qt, P, W, Pt, part, nchunks, Qn, Ph, Qht, tab, s);
}

}  // namespace

hipError_t lq_logquant(LqState &st, const float *F, int64_t rows, int r, double alpha, int bits,
                       int8_t *codes, float *colmax, float *Fhat, hipStream_t s) {
  const LqTables *tab = nullptr;
  hipError_t e = tables(st, alpha, bits, s, &tab);
  if (e != hipSuccess) return e;
  ColJob j{F, rows, r, codes, colmax, Fhat, nullptr, nullptr};
  hipLaunchKernelGGL(k_lq_quant_cols, dim3(r), dim3(1024), 0, s, j, j, r, tab->dev, tab->L);
  return hipGetLastError();
}

hipError_t lq_step(LqState &st, const LqStepArgs &a, hipStream_t s) {
  const LqTables *tab = nullptr;
  hipError_t e = tables(st, a.alpha, a.bits, s, &tab);
  if (e != hipSuccess) return e;
  const int64_t n = a.n, m = a.m, r = a.r;
  const int nchunks = (int)((n + kRowsC - 1) / kRowsC);
  size_t off = 0;
  const size_t oQt = off; off += align256(sizeof(float) * r * m);
  const size_t oP = off; off += align256(sizeof(float) * n * r);
  const size_t oW = off; off += align256(sizeof(double) * n * r);
  const size_t oPt = off; off += align256(sizeof(float) * n * r);
  const size_t oPart = off; off += align256(sizeof(float) * (size_t)nchunks * m * r);
  const size_t oQn = off; off += align256(sizeof(float) * m * r);
  const size_t oPh = off; off += align256(sizeof(float) * n * r);
  const size_t oQht = off; off += align256(sizeof(float) * r * m);
  e = ensure(st, off, s);
  if (e != hipSuccess) return e;
  char *base = static_cast<char *>(st.scratch);
  float *Qt = reinterpret_cast<float *>(base + oQt);
  float *P = reinterpret_cast<float *>(base + oP);
  double *W = reinterpret_cast<double *>(base + oW);
  float *Pt = reinterpret_cast<float *>(base + oPt);
  float *part = reinterpret_cast<float *>(base + oPart);
  float *Qn = reinterpret_cast<float *>(base + oQn);
  float *Ph = reinterpret_cast<float *>(base + oPh);
  float *Qht = reinterpret_cast<float *>(base + oQht);
  const bool vec4 = (m % 4) == 0;
  switch (a.r) {
    case 1: launch_step_v<1>(a, vec4, Qt, P, W, Pt, part, nchunks, Qn, Ph, Qht, *tab, s); break;
    case 2: launch_step_v<2>(a, vec4, Qt, P, W, Pt, part, nchunks, Qn, Ph, Qht, *tab, s); break;
    case 3: launch_step_v<3>(a, vec4, Qt, P, W, Pt, part, nchunks, Qn, Ph, Qht, *tab, s); break;
    case 4: launch_step_v<4>(a, vec4, Qt, P, W, Pt, part, nchunks, Qn, Ph, Qht, *tab, s); break;
    case 5: launch_step_v<5>(a, vec4, Qt, P, W, Pt, part, nchunks, Qn, Ph, Qht, *tab, s); break;
    case 6: launch_step_v<6>(a, vec4, Qt, P, W, Pt, part, nchunks, Qn, Ph, Qht, *tab, s); break;
    case 7: launch_step_v<7>(a, vec4, Qt, P, W, Pt, part, nchunks, Qn, Ph, Qht, *tab, s); break;
    case 8: launch_step_v<8>(a, vec4, Qt, P, W, Pt, part, nchunks, Qn, Ph, Qht, *tab, s); break;
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
