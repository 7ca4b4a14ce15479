// gq_stream.hip -- gfx950 kernels of the Global-QSGD path: global norm, stochastic
// quantisation + packing, integer sum of codes, decode of the mean, and the fused single pass.
//
// Method (Global-QSGD / "Quantize Once, Train Fast", abstract): one global norm scales every
// worker; unbiased stochastic rounding onto a grid all workers share; the integer codes are
// summed (Allreduce); the mean is decoded once.  Uniform grid: QSGD family ("Unbiased
// Single-scale and Multi-scale Quantizers", abstract).  Exponential grid: "NUQSGD", abstract.
//
// Design for CDNA4: every kernel is an HBM stream.  A thread owns groups of 8 consecutive
// elements (one 32 B fp32 or 16 B bf16 load, issued non-temporal so the 256 MB Infinity Cache
// is not polluted by data that is never re-read); a 256-thread block walks 8192-element tiles
// with a grid-stride loop, so 2048 resident blocks cover all 256 CUs whatever the size.  Tiles
// never cross segments, so the per-segment scale is one scalar load per tile.  Codes are
// packed in registers (8 int8 -> one 8 B store, 8 nibbles -> one 4 B store).  No MFMA: there
// is no contraction on this path.  Reductions are fixed-order (no float atomics), so results
// are bit-stable from run to run.
//
// Arithmetic contract (each step is one IEEE operation, so any conforming implementation of
// the same definition gets the same bits; compiled with -ffp-contract=off and IEEE fp32
// denormals): u = |x| * inv is one fp32 multiply; floor, fraction and the scaling of
// the fraction by 2^32 are exact; the draw r = h * 2^-32 satisfies r < p exactly when
// h < ceil(p * 2^32), which is the integer comparison used here.
#include <float.h>
#include <math.h>

#include "gq_internal.h"

namespace gq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxGrid = 2048;

// MurmurHash3's 32-bit finaliser (Appleby, public domain).
__device__ __forceinline__ uint32_t fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}

__device__ __forceinline__ void tile_of(const TileView &tv, int64_t t, int64_t &begin,
                                        int &len, int &seg) {
  if (tv.tiles == nullptr) {
    begin = t * kTile;
    const int64_t rest = tv.n - begin;
    len = rest < kTile ? (int)rest : kTile;
    seg = 0;
  } else {
    const Tile tl = tv.tiles[t];
    begin = tl.begin;
    len = tl.len;
    seg = tl.seg;
  }
}

__device__ __forceinline__ int64_t seg_first_tile(const TileView &tv, int g) {
  if (tv.seg_tile_start == nullptr) return g == 0 ? 0 : tv.ntiles;
  return tv.seg_tile_start[g];
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float v) {
  const uint32_t u = __float_as_uint(v);
  if (v != v) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Eight consecutive elements starting at e0 (a multiple of 8).
template <int DT>
__device__ __forceinline__ void load8(const void *base, int64_t e0, float (&x)[8]) {
  if constexpr (DT == 0) {
    const f32x4 *p = reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + e0);
    const f32x4 a = __builtin_nontemporal_load(p);
    const f32x4 b = __builtin_nontemporal_load(p + 1);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + e0);
    const u32x4 v = __builtin_nontemporal_load(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
}

// The last group of a buffer whose length is not a multiple of 8: cnt < 8 elements, rest 0.
template <int DT>
__device__ __forceinline__ void load_tail(const void *base, int64_t e0, int cnt, float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (e < cnt) {
      if constexpr (DT == 0)
        x[e] = static_cast<const float *>(base)[e0 + e];
      else
        x[e] = bf16_to_f32(static_cast<const uint16_t *>(base)[e0 + e]);
    } else {
      x[e] = 0.0f;
    }
  }
}

template <int DT>
__device__ __forceinline__ void load_group(const void *base, int64_t e0, int cnt, float (&x)[8]) {
  if (cnt == 8)
    load8<DT>(base, e0, x);
  else
    load_tail<DT>(base, e0, cnt, x);
}

// ---------------------------------------------------------------- per-segment constants
struct SegQ {
  float inv;      // s / S (uniform) or 1 / S (exponential)
  bool valid;     // S is a positive finite number and inv is finite
};

template <int GRID>
__device__ __forceinline__ SegQ seg_quant(float S, int levels) {
  SegQ q;
  q.valid = (S > 0.0f) && (S <= FLT_MAX);
  const float num = GRID == 0 ? (float)levels : 1.0f;
  q.inv = q.valid ? num / S : 0.0f;  // IEEE division (correctly rounded)
  if (!(q.inv <= FLT_MAX)) {
    q.valid = false;
    q.inv = 0.0f;
  }
  return q;
}

__device__ __forceinline__ float seg_decode(float S, double denom) {
  if (!((S > 0.0f) && (S <= FLT_MAX))) return 0.0f;
  return (float)((double)S / denom);
}

// ---------------------------------------------------------------- element quantisers
// Uniform grid: signed level in [-s, s].
__device__ __forceinline__ int32_t quant_uniform(float x, float inv, float sf, uint32_t h) {
  const float u = fminf(fabsf(x) * inv, sf);  // NaN -> s
  const float fl = floorf(u);
  const float p = u - fl;                     // exact
  const uint32_t c = (uint32_t)ceilf(p * 4294967296.0f);
  const int32_t m = (int32_t)fl + (h < c ? 1 : 0);
  return x < 0.0f ? -m : m;
}

// Exponential grid: signed index sign*j, j in [0, E]; level j > 0 is 2^(j-E).
__device__ __forceinline__ int32_t quant_exp(float x, float inv, int E, float two_em1,
                                             uint32_t h) {
  const float u = fminf(fabsf(x) * inv, 1.0f);
  const uint32_t b = __float_as_uint(u);
  const int e = (int)(b >> 23) - 127;  // binade of u (u normal when e >= 1 - E)
  int j;
  float p;
  if (e < 1 - E) {
    j = 0;
    p = u * two_em1;                   // (u - 0) / 2^(1-E), exact
  } else {
    j = E + e;
    p = __uint_as_float((b & 0x7FFFFFu) | 0x3F800000u) - 1.0f;  // u / 2^e - 1, exact
  }
  const uint32_t c = (uint32_t)ceilf(p * 4294967296.0f);
  j += (h < c) ? 1 : 0;
  return (x < 0.0f && j > 0) ? -j : j;
}

template <int GRID>
__device__ __forceinline__ int32_t quant_one(float x, const SegQ &q, int levels, float sf,
                                             float two_em1, uint32_t h) {
  if constexpr (GRID == 0)
    return quant_uniform(x, q.inv, sf, h);
  else
    return quant_exp(x, q.inv, levels, two_em1, h);
}

// Integer value on the common grid: the level (uniform) or sign * 2^(j-1) (exponential).
template <int GRID>
__device__ __forceinline__ int32_t lin_of(int32_t q) {
  if constexpr (GRID == 0) {
    return q;
  } else {
    const uint32_t j = (uint32_t)(q < 0 ? -q : q);
    const int32_t v = (int32_t)((1u << j) >> 1);
    return q < 0 ? -v : v;
  }
}

// Code bits of a signed level (bits wide, not yet positioned).
template <int GRID>
__device__ __forceinline__ uint32_t code_bits(int32_t q, int bits) {
  if constexpr (GRID == 0) {
    return (uint32_t)q & ((1u << bits) - 1u);
  } else {
    const uint32_t j = (uint32_t)(q < 0 ? -q : q);
    return (q < 0 ? (1u << (bits - 1)) : 0u) | j;
  }
}

// Signed level from code bits.
template <int GRID>
__device__ __forceinline__ int32_t level_of_code(uint32_t c, int bits) {
  if constexpr (GRID == 0) {
    return ((int32_t)(c << (32 - bits))) >> (32 - bits);
  } else {
    const int32_t j = (int32_t)(c & ((1u << (bits - 1)) - 1u));
    return (c >> (bits - 1)) & 1u ? -j : j;
  }
}

// Store 8 codes of bits width for elements e0..e0+cnt-1.
__device__ __forceinline__ void store_codes(uint8_t *codes, int64_t e0, int cnt, int bits,
                                            const uint32_t (&c)[8]) {
  if (bits == 8) {
    const uint32_t lo = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    const uint32_t hi = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    if (cnt == 8) {
      u32x2 v = {lo, hi};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(codes + e0));
    } else {
      for (int e = 0; e < cnt; ++e) codes[e0 + e] = (uint8_t)c[e];
    }
  } else {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) w |= c[e] << (4 * e);
    if (cnt == 8) {
      __builtin_nontemporal_store(w, reinterpret_cast<uint32_t *>(codes + e0 / 2));
    } else {
      for (int b = 0; b < (cnt + 1) / 2; ++b) codes[e0 / 2 + b] = (uint8_t)(w >> (8 * b));
    }
  }
}

// Load the 8 code fields of elements e0..e0+7 (missing tail fields read as 0).
__device__ __forceinline__ void load_codes(const uint8_t *codes, int64_t e0, int cnt, int bits,
                                           uint32_t (&c)[8]) {
  if (bits == 8) {
    uint32_t lo = 0, hi = 0;
    if (cnt == 8) {
      const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(codes + e0));
      lo = v.x;
      hi = v.y;
    } else {
      for (int e = 0; e < cnt; ++e) {
        const uint32_t b = codes[e0 + e];
        if (e < 4) lo |= b << (8 * e); else hi |= b << (8 * (e - 4));
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c[e] = (lo >> (8 * e)) & 0xFFu;
      c[e + 4] = (hi >> (8 * e)) & 0xFFu;
    }
  } else {
    uint32_t w = 0;
    if (cnt == 8) {
      w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(codes + e0 / 2));
    } else {
      for (int b = 0; b < (cnt + 1) / 2; ++b) w |= (uint32_t)codes[e0 / 2 + b] << (8 * b);
      w &= cnt >= 8 ? 0xFFFFFFFFu : ((1u << (4 * cnt)) - 1u);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = (w >> (4 * e)) & 0xFu;
  }
}

__device__ __forceinline__ void store_sums(void *sums, int acc_bits, int64_t e0, int cnt,
                                           const int32_t (&acc)[8]) {
  if (acc_bits == 16) {
    int16_t *s = static_cast<int16_t *>(sums) + e0;
    if (cnt == 8) {
      u32x4 v;
      v.x = ((uint32_t)acc[0] & 0xFFFFu) | ((uint32_t)acc[1] << 16);
      v.y = ((uint32_t)acc[2] & 0xFFFFu) | ((uint32_t)acc[3] << 16);
      v.z = ((uint32_t)acc[4] & 0xFFFFu) | ((uint32_t)acc[5] << 16);
      v.w = ((uint32_t)acc[6] & 0xFFFFu) | ((uint32_t)acc[7] << 16);
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(s));
    } else {
      for (int e = 0; e < cnt; ++e) s[e] = (int16_t)acc[e];
    }
  } else {
    int32_t *s = static_cast<int32_t *>(sums) + e0;
    if (cnt == 8) {
      u32x4 a = {(uint32_t)acc[0], (uint32_t)acc[1], (uint32_t)acc[2], (uint32_t)acc[3]};
      u32x4 b = {(uint32_t)acc[4], (uint32_t)acc[5], (uint32_t)acc[6], (uint32_t)acc[7]};
      __builtin_nontemporal_store(a, reinterpret_cast<u32x4 *>(s));
      __builtin_nontemporal_store(b, reinterpret_cast<u32x4 *>(s) + 1);
    } else {
      for (int e = 0; e < cnt; ++e) s[e] = acc[e];
    }
  }
}

__device__ __forceinline__ void load_sums(const void *sums, int acc_bits, int64_t e0, int cnt,
                                          int32_t (&acc)[8]) {
  if (acc_bits == 16) {
    const int16_t *s = static_cast<const int16_t *>(sums) + e0;
    if (cnt == 8) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(s));
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = ((int32_t)(w[i] << 16)) >> 16;
        acc[2 * i + 1] = ((int32_t)w[i]) >> 16;
      }
    } else {
      for (int e = 0; e < 8; ++e) acc[e] = e < cnt ? s[e] : 0;
    }
  } else {
    const int32_t *s = static_cast<const int32_t *>(sums) + e0;
    if (cnt == 8) {
      const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(s));
      const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(s) + 1);
      acc[0] = (int32_t)a.x; acc[1] = (int32_t)a.y; acc[2] = (int32_t)a.z; acc[3] = (int32_t)a.w;
      acc[4] = (int32_t)b.x; acc[5] = (int32_t)b.y; acc[6] = (int32_t)b.z; acc[7] = (int32_t)b.w;
    } else {
      for (int e = 0; e < 8; ++e) acc[e] = e < cnt ? s[e] : 0;
    }
  }
}

__device__ __forceinline__ void store_mean(void *out, int out_dtype, int64_t e0, int cnt,
                                           const float (&v)[8]) {
  if (out_dtype == 0) {
    float *o = static_cast<float *>(out) + e0;
    if (cnt == 8) {
      f32x4 a = {v[0], v[1], v[2], v[3]};
      f32x4 b = {v[4], v[5], v[6], v[7]};
      __builtin_nontemporal_store(a, reinterpret_cast<f32x4 *>(o));
      __builtin_nontemporal_store(b, reinterpret_cast<f32x4 *>(o) + 1);
    } else {
      for (int e = 0; e < cnt; ++e) o[e] = v[e];
    }
  } else {
    uint16_t *o = static_cast<uint16_t *>(out) + e0;
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = f32_to_bf16(v[e]);
    if (cnt == 8) {
      u32x4 w = {b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16),
                 b[6] | (b[7] << 16)};
      __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(o));
    } else {
      for (int e = 0; e < cnt; ++e) o[e] = (uint16_t)b[e];
    }
  }
}

// ---------------------------------------------------------------- block reductions (fp64)
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sum over the block in a fixed order; every thread receives the result.
__device__ __forceinline__ double block_sum(double v, double *lds) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds[w] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += lds[i];
  return t;
}

// ================================================================ kernels
// Per (worker, tile) fp64 sum of squares.  Grid: (tiles, K).
template <int DT>
__global__ __launch_bounds__(kBlock) void k_norm_partial(NormArgs a) {
  __shared__ double lds[kBlock / 64];
  const int k = blockIdx.y;
  const void *src = a.grads[k];
  for (int64_t t = blockIdx.x; t < a.tv.ntiles; t += gridDim.x) {
    int64_t begin;
    int len, seg;
    tile_of(a.tv, t, begin, len, seg);
    const int ng = (len + 7) >> 3;
    double acc = 0.0;
    for (int gi = threadIdx.x; gi < ng; gi += kBlock) {
      float x[8];
      load_group<DT>(src, begin + 8 * (int64_t)gi, min(8, len - 8 * gi), x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double v = (double)x[e];
        acc = __fma_rn(v, v, acc);  // v*v is exact in fp64, so this is the plain sum
      }
    }
    const double tot = block_sum(acc, lds);
    if (threadIdx.x == 0) a.partial[(int64_t)k * a.tv.ntiles + t] = tot;
  }
}

// One block per segment: fixed-order sum of the tile partials, sqrt, max over workers.
__global__ __launch_bounds__(kBlock) void k_norm_finalize(NormArgs a) {
  __shared__ double lds[kBlock / 64];
  const int g = blockIdx.x;
  const int64_t t0 = seg_first_tile(a.tv, g), t1 = seg_first_tile(a.tv, g + 1);
  double best = 0.0;
  bool bad = false;
  for (int k = 0; k < a.K; ++k) {
    double acc = 0.0;
    const double *part = a.partial + (int64_t)k * a.tv.ntiles;
    for (int64_t t = t0 + threadIdx.x; t < t1; t += kBlock) acc += part[t];
    const double nrm = sqrt(block_sum(acc, lds));
    if (a.norms_out && threadIdx.x == 0) a.norms_out[(int64_t)k * a.tv.nseg + g] = nrm;
    if (!isfinite(nrm))
      bad = true;
    else if (nrm > best)
      best = nrm;
  }
  if (threadIdx.x == 0) {
    float S = (float)best;
    if (bad || !isfinite(S)) {
      S = 0.0f;
      atomicOr(a.status, 1u);
    }
    a.scale_out[g] = S;
  }
}

// Quantise one worker's buffer and pack the codes.
template <int DT, int GRID>
__global__ __launch_bounds__(kBlock) void k_quantize_pack(QuantArgs a) {
  const float sf = (float)a.levels;
  const float two_em1 = ldexpf(1.0f, a.levels - 1);
  for (int64_t t = blockIdx.x; t < a.tv.ntiles; t += gridDim.x) {
    int64_t begin;
    int len, seg;
    tile_of(a.tv, t, begin, len, seg);
    const SegQ q = seg_quant<GRID>(a.scale[seg], a.levels);
    const int ng = (len + 7) >> 3;
    for (int gi = threadIdx.x; gi < ng; gi += kBlock) {
      const int64_t e0 = begin + 8 * (int64_t)gi;
      const int cnt = min(8, len - 8 * gi);
      uint32_t c[8];
      if (q.valid) {
        float x[8];
        load_group<DT>(a.grad, e0, cnt, x);
        const uint32_t ctr = a.index_base + (uint32_t)e0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t h = fmix32((ctr + e) ^ a.key);
          c[e] = code_bits<GRID>(quant_one<GRID>(x[e], q, a.levels, sf, two_em1, h), a.bits);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) c[e] = 0;
      }
      store_codes(a.codes, e0, cnt, a.bits, c);
    }
  }
}

// sums_i = sum_k lin(code_{k,i}).
template <int GRID>
__global__ __launch_bounds__(kBlock) void k_accumulate(AccArgs a) {
  const int64_t ng = (a.n + 7) >> 3;
  for (int64_t gi = (int64_t)blockIdx.x * kBlock + threadIdx.x; gi < ng;
       gi += (int64_t)gridDim.x * kBlock) {
    const int64_t e0 = 8 * gi;
    const int cnt = (int)min((int64_t)8, a.n - e0);
    int32_t acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k = 0; k < a.K; ++k) {
      uint32_t c[8];
      load_codes(a.codes[k], e0, cnt, a.bits, c);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += lin_of<GRID>(level_of_code<GRID>(c[e], a.bits));
    }
    store_sums(a.sums, a.acc_bits, e0, cnt, acc);
  }
}

// mean_i = fp32(sums_i) * f_g.
__global__ __launch_bounds__(kBlock) void k_dequantize(DequantArgs a) {
  for (int64_t t = blockIdx.x; t < a.tv.ntiles; t += gridDim.x) {
    int64_t begin;
    int len, seg;
    tile_of(a.tv, t, begin, len, seg);
    const float f = seg_decode(a.scale[seg], a.denom);
    const int ng = (len + 7) >> 3;
    for (int gi = threadIdx.x; gi < ng; gi += kBlock) {
      const int64_t e0 = begin + 8 * (int64_t)gi;
      const int cnt = min(8, len - 8 * gi);
      int32_t acc[8];
      load_sums(a.sums, a.acc_bits, e0, cnt, acc);
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (float)acc[e] * f;
      store_mean(a.out, a.out_dtype, e0, cnt, v);
    }
  }
}

// Fused pass: for each element, K quantisations in registers, integer sum, one decode.
// KT > 0 fixes K at compile time (loads of all workers are issued before any arithmetic);
// KT = 0 loops over a runtime K.
template <int KT, int DT, int GRID>
__global__ __launch_bounds__(kBlock) void k_fused(FusedArgs a) {
  const int K = KT > 0 ? KT : a.K;
  const float sf = (float)a.levels;
  const float two_em1 = ldexpf(1.0f, a.levels - 1);
  const bool store_codes_ = a.store_codes != 0;
  for (int64_t t = blockIdx.x; t < a.tv.ntiles; t += gridDim.x) {
    int64_t begin;
    int len, seg;
    tile_of(a.tv, t, begin, len, seg);
    const float S = a.scale[seg];
    const SegQ q = seg_quant<GRID>(S, a.levels);
    const float f = seg_decode(S, a.denom);
    const int ng = (len + 7) >> 3;
    for (int gi = threadIdx.x; gi < ng; gi += kBlock) {
      const int64_t e0 = begin + 8 * (int64_t)gi;
      const int cnt = min(8, len - 8 * gi);
      int32_t acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (q.valid) {
        const uint32_t ctr = a.index_base + (uint32_t)e0;
        if constexpr (KT > 0) {
          float x[KT][8];
#pragma unroll
          for (int k = 0; k < KT; ++k) load_group<DT>(a.grads[k], e0, cnt, x[k]);
#pragma unroll
          for (int k = 0; k < KT; ++k) {
            uint32_t c[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint32_t h = fmix32((ctr + e) ^ a.keys[k]);
              const int32_t lv = quant_one<GRID>(x[k][e], q, a.levels, sf, two_em1, h);
              acc[e] += lin_of<GRID>(lv);
              c[e] = code_bits<GRID>(lv, a.bits);
            }
            if (store_codes_) store_codes(a.codes[k], e0, cnt, a.bits, c);
          }
        } else {
          for (int k = 0; k < K; ++k) {
            float x[8];
            load_group<DT>(a.grads[k], e0, cnt, x);
            uint32_t c[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint32_t h = fmix32((ctr + e) ^ a.keys[k]);
              const int32_t lv = quant_one<GRID>(x[e], q, a.levels, sf, two_em1, h);
              acc[e] += lin_of<GRID>(lv);
              c[e] = code_bits<GRID>(lv, a.bits);
            }
            if (store_codes_) store_codes(a.codes[k], e0, cnt, a.bits, c);
          }
        }
      } else if (store_codes_) {
        const uint32_t z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int k = 0; k < K; ++k) store_codes(a.codes[k], e0, cnt, a.bits, z);
      }
      if (a.sums) store_sums(a.sums, a.acc_bits, e0, cnt, acc);
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (float)acc[e] * f;
      store_mean(a.out, a.out_dtype, e0, cnt, v);
    }
  }
}

__global__ void k_clear_u32(unsigned *p, int count) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0u;
}

int grid_for(int64_t work) {
  return (int)(work < kMaxGrid ? (work > 0 ? work : 1) : kMaxGrid);
}

}  // namespace

// ================================================================ launchers
hipError_t launch_global_norm(const NormArgs &a, int dtype, hipStream_t s) {
  if (a.tv.ntiles > 0) {
    dim3 grid(grid_for(a.tv.ntiles), a.K);
    if (dtype == 0)
      hipLaunchKernelGGL(k_norm_partial<0>, grid, dim3(kBlock), 0, s, a);
    else
      hipLaunchKernelGGL(k_norm_partial<1>, grid, dim3(kBlock), 0, s, a);
  }
  if (a.tv.nseg > 0)
    hipLaunchKernelGGL(k_norm_finalize, dim3(a.tv.nseg), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quantize_pack(const QuantArgs &a, int dtype, int grid, hipStream_t s) {
  if (a.tv.ntiles == 0) return hipSuccess;
  dim3 g(grid_for(a.tv.ntiles));
  if (dtype == 0 && grid == 0) hipLaunchKernelGGL((k_quantize_pack<0, 0>), g, dim3(kBlock), 0, s, a);
  if (dtype == 0 && grid == 1) hipLaunchKernelGGL((k_quantize_pack<0, 1>), g, dim3(kBlock), 0, s, a);
  if (dtype == 1 && grid == 0) hipLaunchKernelGGL((k_quantize_pack<1, 0>), g, dim3(kBlock), 0, s, a);
  if (dtype == 1 && grid == 1) hipLaunchKernelGGL((k_quantize_pack<1, 1>), g, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_accumulate(const AccArgs &a, int grid, hipStream_t s) {
  const int64_t ng = (a.n + 7) / 8;
  if (ng == 0) return hipSuccess;
  dim3 g(grid_for((ng + kBlock - 1) / kBlock));
  if (grid == 0)
    hipLaunchKernelGGL(k_accumulate<0>, g, dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL(k_accumulate<1>, g, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dequantize(const DequantArgs &a, hipStream_t s) {
  if (a.tv.ntiles == 0) return hipSuccess;
  hipLaunchKernelGGL(k_dequantize, dim3(grid_for(a.tv.ntiles)), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template <int DT, int GRID>
static void launch_fused_k(const FusedArgs &a, dim3 g, hipStream_t s) {
  switch (a.K) {
    case 1: hipLaunchKernelGGL((k_fused<1, DT, GRID>), g, dim3(kBlock), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_fused<2, DT, GRID>), g, dim3(kBlock), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_fused<4, DT, GRID>), g, dim3(kBlock), 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_fused<8, DT, GRID>), g, dim3(kBlock), 0, s, a); break;
    case 16: hipLaunchKernelGGL((k_fused<16, DT, GRID>), g, dim3(kBlock), 0, s, a); break;
    default: hipLaunchKernelGGL((k_fused<0, DT, GRID>), g, dim3(kBlock), 0, s, a); break;
  }
}

hipError_t launch_fused(const FusedArgs &a, int dtype, int grid, hipStream_t s) {
  if (a.tv.ntiles == 0) return hipSuccess;
  dim3 g(grid_for(a.tv.ntiles));
  if (dtype == 0 && grid == 0) launch_fused_k<0, 0>(a, g, s);
  if (dtype == 0 && grid == 1) launch_fused_k<0, 1>(a, g, s);
  if (dtype == 1 && grid == 0) launch_fused_k<1, 0>(a, g, s);
  if (dtype == 1 && grid == 1) launch_fused_k<1, 1>(a, g, s);
  return hipGetLastError();
}

hipError_t launch_clear_u32(unsigned *p, int count, hipStream_t s) {
  hipLaunchKernelGGL(k_clear_u32, dim3((count + 255) / 256), dim3(256), 0, s, p, count);
  return hipGetLastError();
}

}  // namespace gq
