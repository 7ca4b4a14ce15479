// gq_stream.hip -- gfx950 kernels of the Global-QSGD path: global norm, stochastic
// quantisation + packing, integer sum of codes, decode of the mean, the fused single pass,
// and the summable wire payload (offset-binary lanes that a uint32 Allreduce adds exactly);
// and of the per-worker-scale baselines the NUQSGD abstract compares against (QSGD, QSGDinf,
// NUQSGD): per-worker scales, their one-pass mean and the receiver's decode of their codes.
//
// Method (Global-QSGD / "Quantize Once, Train Fast", abstract): one global norm scales every
// worker; unbiased stochastic rounding onto a grid all workers share; the integer codes are
// summed (Allreduce); the mean is decoded once.  Uniform grid: QSGD family ("Unbiased
// Single-scale and Multi-scale Quantizers", abstract).  Exponential grid: "NUQSGD", abstract.
//
// Design for CDNA4.  Every kernel is an HBM stream, so the design is about how a wave touches
// memory.  A wave walks 512-element chunks; lane L owns NP "parts" of P consecutive elements,
// part j at chunk offset j*64*P + L*P, so every load and store instruction of the wave covers
// one contiguous block (1 KB of fp32, 256 B of int8 codes, ...): whole cache lines, never the
// half-line writes a 32-byte-per-lane layout produces.  Gradient loads are non-temporal (they
// are read once; keeping them out of the 256 MB Infinity Cache lets a pure read stream run at
// ~7 TB/s on MI355X).  The element-wise kernels launch one 256-thread block per tile, in the
// XCD order of xcd_tile (each XCD streams its own contiguous eighth of the buffers), with
// 2048-element tiles where several read streams mix with a write stream and 32 KB of input
// (8192 fp32 or 16384 bf16 elements) for one read and one write stream; tiles never cross
// segments, so the per-segment scale is one scalar load per tile.  The one-worker quantisers
// run a full tile through a copy of their loop whose part and chunk counts are constants.
// The norm pass (read only) keeps a fixed grid striding over 65536-element tiles, one fp64
// partial each.  Codes are packed in registers.  No MFMA: there is no contraction here.
// Reductions are fixed-order (no float atomics): results are bit-stable.
//
// Arithmetic contract (each step is one IEEE operation, so any conforming implementation of
// the same definition gets the same bits; compiled with -ffp-contract=off and IEEE fp32
// denormals): u = |x| * inv is one fp32 multiply; floor, fraction and the scaling of the
// fraction by 2^32 are exact; the draw is r = fp32(h) * 2^-32, the 32-bit hash h converted to
// fp32 (round to nearest even, one v_cvt_f32_u32) and scaled exactly, so r < p is the fp32
// comparison fp32(h) < p * 2^32.  Uniform sums are carried in fp32, which is exact because
// |sum| <= 64 * 127 < 2^24.
#include <float.h>
#include <math.h>

#include <type_traits>

#include "gq_internal.h"

namespace gq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kChunk = 512;  // elements per wave iteration

// ---------------------------------------------------------------- random numbers
// MurmurHash3's 32-bit finaliser (Appleby, public domain) applied to (counter XOR key).  Its
// first step h ^= h >> 16 distributes over XOR, so it is split: mix16(counter) once per element
// (shared by all workers) and mix16(key) once per worker, on the host.
__device__ __forceinline__ uint32_t mix16(uint32_t v) { return v ^ (v >> 16); }

__device__ __forceinline__ uint32_t fmix32_tail(uint32_t h) {
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}

// ---------------------------------------------------------------- tiles and lane map
__device__ __forceinline__ void tile_of(const TileView &tv, int64_t t, int tile_elems,
                                        int64_t &begin, int &len, int &seg) {
  if (tv.tiles == nullptr) {
    begin = t * tile_elems;
    const int64_t rest = tv.n - begin;
    len = rest < tile_elems ? (int)rest : tile_elems;
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

// Block -> tile order of the element-wise kernels, which launch one block per tile.  The
// hardware hands workgroups to the 8 XCDs in turn (block b to XCD b mod 8), so giving block b
// tile (b mod 8) * q + b / 8 (q = ntiles / 8; the last ntiles mod 8 tiles in order) makes every
// XCD stream its own contiguous eighth of each buffer, and blocks in dispatch order keep each
// of those regions' active window compact; with consecutive tiles spread over the XCDs, or a
// fixed grid striding over the whole buffer, the streams of reads mixed with a stream of
// writes ran 10-15% slower.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t ntiles) {
  const int64_t q = ntiles >> 3;
  return b < 8 * q ? (b & 7) * q + (b >> 3) : b;
}

// Offset within the tile of part j of this lane in chunk ci.
template <int P>
__device__ __forceinline__ int part_offset(int ci, int j, int lane) {
  return ci * kChunk + j * 64 * P + lane * P;
}

// ---------------------------------------------------------------- element loads / stores
// A part is P elements starting at element e0 (a multiple of P); cnt of them exist (cnt == P
// except in the last part of a buffer whose length is not a multiple of 8).
template <int DT, int P>
__device__ __forceinline__ void load_part(const void *base, int64_t e0, int cnt, float (&x)[P]) {
  if (cnt == P) {
    if constexpr (DT == 0) {
      const f32x4 *p = reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + e0);
#pragma unroll
      for (int q = 0; q < P / 4; ++q) {
        const f32x4 v = __builtin_nontemporal_load(p + q);
        x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
      }
    } else if constexpr (P == 8) {
      const u32x4 v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + e0));
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
      const u32x2 v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(base) + e0));
      const uint32_t w[2] = {v.x, v.y};
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < P; ++e) {
      if (e < cnt) {
        if constexpr (DT == 0)
          x[e] = static_cast<const float *>(base)[e0 + e];
        else
          x[e] = __uint_as_float((uint32_t)static_cast<const uint16_t *>(base)[e0 + e] << 16);
      } else {
        x[e] = 0.0f;
      }
    }
  }
}

// One part of one worker as held between its load and its use: fp32 values, or bf16 elements
// left in the words they were loaded in (element 2i in the low half of word i) and widened
// where they are used, so that a buffer of bf16 parts takes half the registers.
template <int DT, int P>
struct PartBuf;
template <int P>
struct PartBuf<0, P> {
  float v[P];
  __device__ __forceinline__ void load(const void *base, int64_t e0, int cnt) {
    load_part<0, P>(base, e0, cnt, v);
  }
  __device__ __forceinline__ float get(int e) const { return v[e]; }
};
template <int P>
struct PartBuf<1, P> {
  uint32_t w[P / 2];
  __device__ __forceinline__ void load(const void *base, int64_t e0, int cnt) {
    const uint16_t *b = static_cast<const uint16_t *>(base);
    if (cnt == P) {
      if constexpr (P == 8) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(b + e0));
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
      } else {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(b + e0));
        w[0] = v.x; w[1] = v.y;
      }
    } else {
#pragma unroll
      for (int i = 0; i < P / 2; ++i) w[i] = 0u;
#pragma unroll
      for (int e = 0; e < P; ++e)
        if (e < cnt) w[e >> 1] |= (uint32_t)b[e0 + e] << ((e & 1) * 16);
    }
  }
  __device__ __forceinline__ float get(int e) const {
    return __uint_as_float((e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
  }
};

// Store kind of the quantisers' code and lane stores (NT: non-temporal).  A non-temporal
// store goes to HBM without waiting for the rest of its 128-byte line; where a wave's store
// begins inside a line (segments that start off a line, as most of ResNet-50's tensors do for
// 4-bit codes), the neighbouring wave writes the rest of each line and the two parts reach HBM
// separately, 26% more write traffic than the codes' bytes.  Plain stores go through L2, which
// merges the parts.  The host picks the kind per launch (whole lines: non-temporal, which
// measured 3-5% faster there than plain stores); a run-time choice per tile inside one kernel
// changed the kernels' code enough to cost bf16 input 3-70%.
template <bool NT, typename T>
__device__ __forceinline__ void put(T v, T *p) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

// Codes: c[e] holds the code field (bits wide) of element e0 + e.
template <int P, bool NT>
__device__ __forceinline__ void store_codes(uint8_t *codes, int64_t e0, int cnt, int bits,
                                            const uint32_t (&c)[P]) {
  if (bits == 8) {
    uint32_t w[P / 4];
#pragma unroll
    for (int i = 0; i < P / 4; ++i)
      w[i] = c[4 * i] | (c[4 * i + 1] << 8) | (c[4 * i + 2] << 16) | (c[4 * i + 3] << 24);
    if (cnt == P) {
      if constexpr (P == 4) {
        put<NT>(w[0], reinterpret_cast<uint32_t *>(codes + e0));
      } else {
        u32x2 v = {w[0], w[1]};
        put<NT>(v, reinterpret_cast<u32x2 *>(codes + e0));
      }
    } else {
      for (int e = 0; e < cnt; ++e) codes[e0 + e] = (uint8_t)c[e];
    }
  } else {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < P; ++e) w |= c[e] << (4 * e);
    if (cnt == P) {
      if constexpr (P == 4)
        put<NT>((uint16_t)w, reinterpret_cast<uint16_t *>(codes + e0 / 2));
      else
        put<NT>(w, reinterpret_cast<uint32_t *>(codes + e0 / 2));
    } else {
      for (int b = 0; b < (cnt + 1) / 2; ++b) codes[e0 / 2 + b] = (uint8_t)(w >> (8 * b));
    }
  }
}

template <int P>
__device__ __forceinline__ void load_codes(const uint8_t *codes, int64_t e0, int cnt, int bits,
                                           uint32_t (&c)[P]) {
  if (bits == 8) {
    uint32_t w[P / 4];
    if (cnt == P) {
      if constexpr (P == 4) {
        w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(codes + e0));
      } else {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(codes + e0));
        w[0] = v.x;
        w[1] = v.y;
      }
    } else {
#pragma unroll
      for (int i = 0; i < P / 4; ++i) w[i] = 0;
      for (int e = 0; e < cnt; ++e) w[e / 4] |= (uint32_t)codes[e0 + e] << (8 * (e % 4));
    }
#pragma unroll
    for (int e = 0; e < P; ++e) c[e] = (w[e / 4] >> (8 * (e % 4))) & 0xFFu;
  } else {
    uint32_t w = 0;
    if (cnt == P) {
      if constexpr (P == 4)
        w = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(codes + e0 / 2));
      else
        w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(codes + e0 / 2));
    } else {
      for (int b = 0; b < (cnt + 1) / 2; ++b) w |= (uint32_t)codes[e0 / 2 + b] << (8 * b);
      w &= (1u << (4 * cnt)) - 1u;
    }
#pragma unroll
    for (int e = 0; e < P; ++e) c[e] = (w >> (4 * e)) & 0xFu;
  }
}

template <int P>
__device__ __forceinline__ void store_sums(void *sums, int acc_bits, int64_t e0, int cnt,
                                           const int32_t (&a)[P]) {
  if (acc_bits == 16) {
    int16_t *s = static_cast<int16_t *>(sums) + e0;
    if (cnt == P) {
      uint32_t w[P / 2];
#pragma unroll
      for (int i = 0; i < P / 2; ++i)
        w[i] = ((uint32_t)a[2 * i] & 0xFFFFu) | ((uint32_t)a[2 * i + 1] << 16);
      if constexpr (P == 4) {
        u32x2 v = {w[0], w[1]};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(s));
      } else {
        u32x4 v = {w[0], w[1], w[2], w[3]};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(s));
      }
    } else {
      for (int e = 0; e < cnt; ++e) s[e] = (int16_t)a[e];
    }
  } else {
    int32_t *s = static_cast<int32_t *>(sums) + e0;
    if (cnt == P) {
#pragma unroll
      for (int q = 0; q < P / 4; ++q) {
        u32x4 v = {(uint32_t)a[4 * q], (uint32_t)a[4 * q + 1], (uint32_t)a[4 * q + 2],
                   (uint32_t)a[4 * q + 3]};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(s) + q);
      }
    } else {
      for (int e = 0; e < cnt; ++e) s[e] = a[e];
    }
  }
}

template <int P>
__device__ __forceinline__ void load_sums(const void *sums, int acc_bits, int64_t e0, int cnt,
                                          int32_t (&a)[P]) {
  if (acc_bits == 16) {
    const int16_t *s = static_cast<const int16_t *>(sums) + e0;
    if (cnt == P) {
      uint32_t w[P / 2];
      if constexpr (P == 4) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(s));
        w[0] = v.x;
        w[1] = v.y;
      } else {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(s));
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
      }
#pragma unroll
      for (int i = 0; i < P / 2; ++i) {
        a[2 * i] = ((int32_t)(w[i] << 16)) >> 16;
        a[2 * i + 1] = ((int32_t)w[i]) >> 16;
      }
    } else {
      for (int e = 0; e < P; ++e) a[e] = e < cnt ? s[e] : 0;
    }
  } else {
    const int32_t *s = static_cast<const int32_t *>(sums) + e0;
    if (cnt == P) {
#pragma unroll
      for (int q = 0; q < P / 4; ++q) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(s) + q);
        a[4 * q] = (int32_t)v.x; a[4 * q + 1] = (int32_t)v.y;
        a[4 * q + 2] = (int32_t)v.z; a[4 * q + 3] = (int32_t)v.w;
      }
    } else {
      for (int e = 0; e < P; ++e) a[e] = e < cnt ? s[e] : 0;
    }
  }
}

// Round-to-nearest-even fp32 -> bf16 (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float v) {
  const uint32_t u = __float_as_uint(v);
  if (v != v) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int P>
__device__ __forceinline__ void store_mean(void *out, int out_dtype, int64_t e0, int cnt,
                                           const float (&v)[P]) {
  if (out_dtype == 0) {
    float *o = static_cast<float *>(out) + e0;
    if (cnt == P) {
#pragma unroll
      for (int q = 0; q < P / 4; ++q) {
        f32x4 w = {v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
        __builtin_nontemporal_store(w, reinterpret_cast<f32x4 *>(o) + q);
      }
    } else {
      for (int e = 0; e < cnt; ++e) o[e] = v[e];
    }
  } else {
    uint16_t *o = static_cast<uint16_t *>(out) + e0;
    uint32_t b[P];
#pragma unroll
    for (int e = 0; e < P; ++e) b[e] = f32_to_bf16(v[e]);
    if (cnt == P) {
      if constexpr (P == 4) {
        u32x2 w = {b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2 *>(o));
      } else {
        u32x4 w = {b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16),
                   b[6] | (b[7] << 16)};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(o));
      }
    } else {
      for (int e = 0; e < cnt; ++e) o[e] = (uint16_t)b[e];
    }
  }
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

// Smallest float a with fl(a * inv) >= bound (inv positive and finite): a product by a positive
// constant rounds monotonically, so every |x| below it has fl(|x| * inv) < bound.  Found from
// the quotient by at most three one-ulp steps each way and verified at a and at the float
// before it; 0 (which no |x| is below) if the verification fails.
// The larger of m and |x| by IEEE 754-2019 maximum, which returns a NaN operand: a lane's largest
// magnitude compared once against the threshold gives the same answer as comparing each
// element (a NaN fails both ways), in one v_maximum3_f32 per two elements.
__device__ __forceinline__ float max_abs(float m, float x) {
  return __builtin_elementwise_maximum(m, fabsf(x));
}

__device__ __forceinline__ float below_bound(float inv, float bound) {
  uint32_t b = __float_as_uint(bound / inv);  // IEEE division, not negative
#pragma unroll
  for (int i = 0; i < 3; ++i)
    if (b > 0u && __uint_as_float(b - 1u) * inv >= bound) --b;
#pragma unroll
  for (int i = 0; i < 3; ++i)
    if (!(__uint_as_float(b) * inv >= bound) && b < 0x7F800000u) ++b;
  const bool ok = (__uint_as_float(b) * inv >= bound) &&
                  (b == 0u || __uint_as_float(b - 1u) * inv < bound);
  return ok ? __uint_as_float(b) : 0.0f;
}

// ---------------------------------------------------------------- element quantisers
// The sign of a level is the sign bit of x on both grids (IEEE 754's signBit, the sign that
// copysign transfers): a NaN element under a caller-given finite scale, clamped to the top
// level, keeps the sign its bit gives it, and -0 has level 0, which carries no sign.
// Uniform grid.  Returns the level magnitude m in [0, s] as a float (exact small integer);
// the signed level is copysign(m, x).
__device__ __forceinline__ float quant_uniform_mag(float x, float inv, float sf, uint32_t h) {
  const float u = fminf(fabsf(x) * inv, sf);  // NaN -> s
  const float fl = floorf(u);
  const float p = u - fl;                     // exact
  return (float)h < p * 4294967296.0f ? ceilf(u) : fl;  // p > 0 then, so ceil(u) = fl + 1
}

// Exponential grid: index j in [0, E] of the level (level j > 0 is 2^(j-E)).  Above the
// lowest level u lies in the binade of level j = E + exponent(u), and the probability of
// rounding up is u / 2^exponent - 1, whose 23 mantissa bits times 2^32 are the integer
// mantissa << 9; below it, p = u / 2^(1-E), and p * 2^32 = u * 2^(E+31) is one exact
// power-of-two scaling (lo_scale = 2^(E+31); u <= 1 keeps it far from overflow).
__device__ __forceinline__ uint32_t quant_exp_index(float x, float inv, int E, float lo_scale,
                                                    uint32_t h) {
  const float u = fminf(fabsf(x) * inv, 1.0f);
  const uint32_t b = __float_as_uint(u);
  const int32_t jn = (int32_t)(b >> 23) - (127 - E);  // <= 0 below the lowest level
  const bool low = jn <= 0;
  const float c_hi = (float)((b & 0x7FFFFFu) << 9);  // exact: 23 significant bits
  const float c_lo = u * lo_scale;
  const float c = low ? c_lo : c_hi;
  return (low ? 0u : (uint32_t)jn) + ((float)h < c ? 1u : 0u);
}

// Code field of a uniform level (signed, two's complement in `bits`).
__device__ __forceinline__ uint32_t uniform_code(float m, float x, int bits) {
  return (uint32_t)(int32_t)copysignf(m, x) & ((1u << bits) - 1u);
}

// x's sign bit as a condition (an integer comparison of the bit pattern, so a NaN or -0 keeps
// the sign its bit gives it).
__device__ __forceinline__ bool sign_bit(float x) { return (int32_t)__float_as_uint(x) < 0; }

// Code field of an exponential index: x's sign bit above j (zero has no sign).
__device__ __forceinline__ uint32_t exp_code(uint32_t j, float x, int bits) {
  return ((sign_bit(x) && j > 0) ? (1u << (bits - 1)) : 0u) | j;
}

// Signed integer value on the common grid of an exponential index: sign * 2^(j-1), 0 for j = 0.
__device__ __forceinline__ int32_t exp_lin(uint32_t j, bool neg) {
  const int32_t v = (int32_t)((1u << j) >> 1);
  return neg ? -v : v;
}

// The same with the sign taken from x's sign bit.
__device__ __forceinline__ int32_t exp_lin_of(uint32_t j, float x) {
  return exp_lin(j, sign_bit(x));
}

template <int GRID>
__device__ __forceinline__ int32_t lin_of_code(uint32_t c, int bits) {
  if constexpr (GRID == 0) {
    return ((int32_t)(c << (32 - bits))) >> (32 - bits);
  } else {
    const uint32_t j = c & ((1u << (bits - 1)) - 1u);
    return exp_lin(j, ((c >> (bits - 1)) & 1u) != 0);
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

// ================================================================ global norm
// Per (worker, norm tile) fp64 sum of squares.  Grid: (tiles, K).
template <int DT>
__global__ __launch_bounds__(kBlock) void k_norm_partial(NormArgs a) {
  constexpr int P = DT == 0 ? 4 : 8;
  constexpr int NP = kChunk / (64 * P);
  __shared__ double lds[kBlock / 64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int k = blockIdx.y;
  const void *src = a.grads[k];
  for (int64_t t = blockIdx.x; t < a.tv.ntiles; t += gridDim.x) {
    int64_t begin;
    int len, seg;
    tile_of(a.tv, t, a.tile, begin, len, seg);
    const int nch = (len + kChunk - 1) / kChunk;
    double acc = 0.0;
    for (int ci = wv; ci < nch; ci += kBlock / 64) {
      float x[NP][P];
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int o = part_offset<P>(ci, j, lane);
        const int cnt = min(P, len - o);
        if (cnt > 0) {
          load_part<DT, P>(src, begin + o, cnt, x[j]);
        } else {
#pragma unroll
          for (int e = 0; e < P; ++e) x[j][e] = 0.0f;
        }
      }
#pragma unroll
      for (int j = 0; j < NP; ++j)
#pragma unroll
        for (int e = 0; e < P; ++e) {
          const double v = (double)x[j][e];
          acc = __fma_rn(v, v, acc);  // v*v is exact in fp64, so this is the plain sum
        }
    }
    const double tot = block_sum(acc, lds);
    if (threadIdx.x == 0) a.partial[(int64_t)k * a.tv.ntiles + t] = tot;
  }
}

// One block per (segment, worker): fixed-order sum of the tile partials, sqrt.
__global__ __launch_bounds__(kBlock) void k_norm_segments(NormArgs a) {
  __shared__ double lds[kBlock / 64];
  const int g = blockIdx.x, k = blockIdx.y;
  const int64_t t0 = seg_first_tile(a.tv, g), t1 = seg_first_tile(a.tv, g + 1);
  const double *part = a.partial + (int64_t)k * a.tv.ntiles;
  double acc = 0.0;
  for (int64_t t = t0 + threadIdx.x; t < t1; t += kBlock) acc += part[t];
  const double nrm = sqrt(block_sum(acc, lds));
  if (threadIdx.x == 0) a.norms[(int64_t)k * a.tv.nseg + g] = nrm;
}

// One thread per segment: S_g = fp32(max_k norm), 0 (and a status flag) if not finite.
__global__ void k_norm_scale(NormArgs a) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= a.tv.nseg) return;
  double best = 0.0;
  bool bad = false;
  for (int k = 0; k < a.K; ++k) {
    const double nrm = a.norms[(int64_t)k * a.tv.nseg + g];
    if (a.norms_out) a.norms_out[(int64_t)k * a.tv.nseg + g] = nrm;
    if (!isfinite(nrm))
      bad = true;
    else if (nrm > best)
      best = nrm;
  }
  float S = (float)best;
  if (bad || !isfinite(S)) {
    S = 0.0f;
    atomicOr(a.status, 1u);
  }
  a.scale_out[g] = S;
}

// The two kernels above in one, for inputs with few norm tiles (K x tiles <= kNormFinishMax):
// one block per segment; wave w sums the partials of workers w, w + 4, ... (lane l adds
// partials l, l + 64, ... in order, then the wave's fixed-order butterfly), and one thread takes
// the maximum over the workers in worker order as k_norm_scale does.  The summation order
// differs from k_norm_segments' (the path is chosen by size alone, so a given input always
// takes the same one).
__global__ __launch_bounds__(kBlock) void k_norm_finish(NormArgs a) {
  __shared__ double nrm_s[kMaxWorkers];
  const int g = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t t0 = seg_first_tile(a.tv, g), t1 = seg_first_tile(a.tv, g + 1);
  for (int k = w; k < a.K; k += kBlock / 64) {
    const double *part = a.partial + (int64_t)k * a.tv.ntiles;
    constexpr int UB = 8;  // loads in flight per lane
    double acc = 0.0;
    for (int64_t t = t0 + lane; t < t1; t += UB * 64) {
      double v[UB];
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int64_t tt = t + (int64_t)u * 64;
        v[u] = tt < t1 ? part[tt] : 0.0;
      }
#pragma unroll
      for (int u = 0; u < UB; ++u)
        if (t + (int64_t)u * 64 < t1) acc += v[u];
    }
    const double nrm = sqrt(wave_sum(acc));
    if (lane == 0) {
      nrm_s[k] = nrm;
      if (a.norms_out) a.norms_out[(int64_t)k * a.tv.nseg + g] = nrm;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double best = 0.0;
    bool bad = false;
    for (int k = 0; k < a.K; ++k) {
      const double nrm = nrm_s[k];
      if (!isfinite(nrm))
        bad = true;
      else if (nrm > best)
        best = nrm;
    }
    float S = (float)best;
    if (bad || !isfinite(S)) {
      S = 0.0f;
      atomicOr(a.status, 1u);
    }
    a.scale_out[g] = S;
  }
}

// ================================================================ quantise + pack (one worker)
// With the fused pass's fast path: a part whose elements, in every active lane, lie below the
// lowest nonzero level (the lane's largest magnitude, NaN-propagating, against the tile's
// threshold) has levels 0 and +-1 only, and it rounds up when fp32(h) < fl(|x| * inv) * 2^32
// (uniform) or fl(|x| * inv) * 2^(E+31) (exponential): bit for bit the general path's codes
// without its clamp, floor, fraction and exponent split.
template <int DT, int GRID, bool AL, bool NT>
__global__ __launch_bounds__(kBlock) void k_quantize_pack(QuantArgs a) {
  constexpr int P = DT == 0 ? 4 : 8;
  constexpr int NP = kChunk / (64 * P);
  constexpr int WAVES = kBlock / 64;
  constexpr int CPW = quant_tile(DT) / kChunk / WAVES;  // chunks per wave in a full tile
  // chunks whose loads a wave issues before it uses the first: all of its share of an fp32
  // tile (8 loads of 1 KB in flight per wave); one at a time for bf16, which measured faster
  constexpr int GR = DT == 0 ? CPW : 1;
  static_assert(CPW % GR == 0, "group size");
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const float sf = (float)a.levels;
  const float lo_scale = ldexpf(1.0f, a.levels + 31);
  const float up_scale = GRID == 0 ? 4294967296.0f : lo_scale;
  const float bound = GRID == 0 ? 1.0f : ldexpf(1.0f, 1 - a.levels);
  for (int64_t b = blockIdx.x; b < a.tv.ntiles; b += gridDim.x) {
    const int64_t t = xcd_tile(b, a.tv.ntiles);
    int64_t begin;
    int len, seg;
    tile_of(a.tv, t, quant_tile(DT), begin, len, seg);
    const SegQ q = seg_quant<GRID>(a.scale[seg], a.levels);
    const float fast_below = q.valid ? below_bound(q.inv, bound) : 0.0f;
    // codes of one part of cnt elements at e0, from its loaded values (zeros where missing)
    auto quant_part = [&](int64_t e0, int cnt, const float (&x)[P]) {
      uint32_t c[P];
      const uint32_t ctr = a.index_base + (uint32_t)e0;
      // AL (index_base a multiple of 8, e0 a multiple of P): ctr + e, e < P, only fills ctr's
      // zero low bits, so it is ctr ^ e with the same upper half: mix16(ctr + e) = mix16(ctr) ^ e
      const uint32_t m0 = mix16(ctr) ^ a.key_mix;
      float big = 0.0f;
#pragma unroll
      for (int e = 0; e < P; ++e) big = max_abs(big, x[e]);
      if (__all(big < fast_below)) {
#pragma unroll
        for (int e = 0; e < P; ++e) {
          const uint32_t h = fmix32_tail(AL ? m0 ^ (uint32_t)e : mix16(ctr + e) ^ a.key_mix);
          const uint32_t up = (float)h < fabsf(x[e]) * q.inv * up_scale ? 1u : 0u;
          if constexpr (GRID == 0)
            c[e] = (sign_bit(x[e]) ? (0u - up) : up) & ((1u << a.bits) - 1u);
          else
            c[e] = exp_code(up, x[e], a.bits);
        }
      } else {
#pragma unroll
        for (int e = 0; e < P; ++e) {
          const uint32_t h = fmix32_tail(AL ? m0 ^ (uint32_t)e : mix16(ctr + e) ^ a.key_mix);
          if constexpr (GRID == 0)
            c[e] = uniform_code(quant_uniform_mag(x[e], q.inv, sf, h), x[e], a.bits);
          else
            c[e] = exp_code(quant_exp_index(x[e], q.inv, a.levels, lo_scale, h), x[e], a.bits);
        }
      }
      store_codes<P, NT>(a.codes, e0, cnt, a.bits, c);
    };
    auto zero_part = [&](int64_t e0, int cnt) {
      uint32_t c[P];
#pragma unroll
      for (int e = 0; e < P; ++e) c[e] = 0;
      store_codes<P, NT>(a.codes, e0, cnt, a.bits, c);
    };
    if (len == quant_tile(DT)) {
      // a full tile: each wave issues the loads of GR chunks before it uses the first
      for (int i0 = 0; i0 < CPW; i0 += GR) {
        if (!q.valid) {
#pragma unroll
          for (int i = 0; i < GR; ++i)
#pragma unroll
            for (int j = 0; j < NP; ++j)
              zero_part(begin + part_offset<P>(wv + (i0 + i) * WAVES, j, lane), P);
          continue;
        }
        PartBuf<DT, P> buf[GR][NP];
#pragma unroll
        for (int i = 0; i < GR; ++i)
#pragma unroll
          for (int j = 0; j < NP; ++j)
            buf[i][j].load(a.grad, begin + part_offset<P>(wv + (i0 + i) * WAVES, j, lane), P);
#pragma unroll
        for (int i = 0; i < GR; ++i)
#pragma unroll
          for (int j = 0; j < NP; ++j) {
            float x[P];
#pragma unroll
            for (int e = 0; e < P; ++e) x[e] = buf[i][j].get(e);
            quant_part(begin + part_offset<P>(wv + (i0 + i) * WAVES, j, lane), P, x);
          }
      }
    } else {
      const int nch = (len + kChunk - 1) / kChunk;
      for (int ci = wv; ci < nch; ci += WAVES) {
#pragma unroll
        for (int j = 0; j < NP; ++j) {
          const int o = part_offset<P>(ci, j, lane);
          const int cnt = min(P, len - o);
          if (cnt <= 0) continue;
          if (q.valid) {
            float x[P];
            load_part<DT, P>(a.grad, begin + o, cnt, x);
            quant_part(begin + o, cnt, x);
          } else {
            zero_part(begin + o, cnt);
          }
        }
      }
    }
  }
}

// ================================================================ integer sum of codes
// sums_i = sum_k lin(code_{k,i}).  P = 8 for int16 sums (16 B stores), 4 for int32.  The code
// loads of KB workers are issued together (the sum is exact in any order).
template <int GRID, int P, int BITS>
__global__ __launch_bounds__(kBlock) void k_accumulate(AccArgs a) {
  constexpr int NP = kChunk / (64 * P);
  constexpr int KB = 4;  // workers whose code loads are issued together
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const TileView tv{nullptr, nullptr, (a.n + kTileMix - 1) / kTileMix, a.n, 1};
  for (int64_t b = blockIdx.x; b < tv.ntiles; b += gridDim.x) {
    const int64_t t = xcd_tile(b, tv.ntiles);
    int64_t begin;
    int len, seg;
    tile_of(tv, t, kTileMix, begin, len, seg);
    const int nch = (len + kChunk - 1) / kChunk;
    for (int ci = wv; ci < nch; ci += kBlock / 64) {
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int o = part_offset<P>(ci, j, lane);
        const int cnt = min(P, len - o);
        if (cnt <= 0) continue;
        const int64_t e0 = begin + o;
        int32_t acc[P];
#pragma unroll
        for (int e = 0; e < P; ++e) acc[e] = 0;
        for (int k0 = 0; k0 < a.K; k0 += KB) {
          // a batch past the last worker loads the last worker's codes again and adds nothing
          uint32_t c[KB][P];
#pragma unroll
          for (int u = 0; u < KB; ++u)
            load_codes<P>(a.codes[min(k0 + u, a.K - 1)], e0, cnt, BITS, c[u]);
#pragma unroll
          for (int u = 0; u < KB; ++u)
            if (k0 + u < a.K)
#pragma unroll
              for (int e = 0; e < P; ++e) acc[e] += lin_of_code<GRID>(c[u][e], BITS);
        }
        store_sums<P>(a.sums, a.acc_bits, e0, cnt, acc);
      }
    }
  }
}

// ================================================================ decode of the mean
template <int P, int ACC>
__global__ __launch_bounds__(kBlock) void k_dequantize(DequantArgs a) {
  constexpr int NP = kChunk / (64 * P);
  constexpr int CPW = kTileMix / kChunk / (kBlock / 64);  // chunks per wave in a full tile
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int64_t b = blockIdx.x; b < a.tv.ntiles; b += gridDim.x) {
    const int64_t t = xcd_tile(b, a.tv.ntiles);
    int64_t begin;
    int len, seg;
    tile_of(a.tv, t, kTileMix, begin, len, seg);
    const float f = seg_decode(a.scale[seg], a.denom);
    if (len == kTileMix) {
      // a full tile: the wave's loads are all issued before the first conversion
      int32_t sv[CPW][NP][P];
#pragma unroll
      for (int i = 0; i < CPW; ++i)
#pragma unroll
        for (int j = 0; j < NP; ++j)
          load_sums<P>(a.sums, ACC, begin + part_offset<P>(wv + i * (kBlock / 64), j, lane), P,
                       sv[i][j]);
#pragma unroll
      for (int i = 0; i < CPW; ++i)
#pragma unroll
        for (int j = 0; j < NP; ++j) {
          float v[P];
#pragma unroll
          for (int e = 0; e < P; ++e) v[e] = (float)sv[i][j][e] * f;
          store_mean<P>(a.out, a.out_dtype, begin + part_offset<P>(wv + i * (kBlock / 64), j, lane),
                        P, v);
        }
      continue;
    }
    const int nch = (len + kChunk - 1) / kChunk;
    for (int ci = wv; ci < nch; ci += kBlock / 64) {
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int o = part_offset<P>(ci, j, lane);
        const int cnt = min(P, len - o);
        if (cnt <= 0) continue;
        const int64_t e0 = begin + o;
        int32_t sv[P];
        load_sums<P>(a.sums, ACC, e0, cnt, sv);
        float v[P];
#pragma unroll
        for (int e = 0; e < P; ++e) v[e] = (float)sv[e] * f;
        store_mean<P>(a.out, a.out_dtype, e0, cnt, v);
      }
    }
  }
}

// ================================================================ summable wire payload
// Element e travels as the unsigned lane lin_e + o of WB bytes at byte e*WB (little-endian),
// o = s or 2^(E-1), WB wide enough that `world` payloads added as unsigned 32-bit words never
// carry between lanes.  A part is P lanes at byte e0*WB (aligned: e0 is a multiple of P).
template <int P, int WB, bool NT>
__device__ __forceinline__ void store_lanes(uint8_t *payload, int64_t e0, int cnt, int64_t n,
                                            const uint32_t (&v)[P]) {
  if (cnt == P) {
    if constexpr (WB == 1) {
      uint32_t w[P / 4];
#pragma unroll
      for (int i = 0; i < P / 4; ++i)
        w[i] = v[4 * i] | (v[4 * i + 1] << 8) | (v[4 * i + 2] << 16) | (v[4 * i + 3] << 24);
      if constexpr (P == 4)
        put<NT>(w[0], reinterpret_cast<uint32_t *>(payload + e0));
      else
        put<NT>((u32x2){w[0], w[1]}, reinterpret_cast<u32x2 *>(payload + e0));
    } else if constexpr (WB == 2) {
      uint32_t w[P / 2];
#pragma unroll
      for (int i = 0; i < P / 2; ++i) w[i] = v[2 * i] | (v[2 * i + 1] << 16);
      if constexpr (P == 4)
        put<NT>((u32x2){w[0], w[1]}, reinterpret_cast<u32x2 *>(payload + 2 * e0));
      else
        put<NT>((u32x4){w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4 *>(payload + 2 * e0));
    } else {
#pragma unroll
      for (int i = 0; i < P / 4; ++i)
        put<NT>((u32x4){v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]},
                reinterpret_cast<u32x4 *>(payload + 4 * (e0 + 4 * i)));
    }
  } else {
    // the buffer's last part: its lanes byte by byte, then the zero padding to 4 bytes
#pragma unroll
    for (int e = 0; e < P; ++e)
      if (e < cnt)
#pragma unroll
        for (int b = 0; b < WB; ++b) payload[(e0 + e) * WB + b] = (uint8_t)(v[e] >> (8 * b));
    const int64_t end = n * WB, padded = (end + 3) / 4 * 4;
    for (int64_t q = end; q < padded; ++q) payload[q] = 0;
  }
}

template <int P, int WB>
__device__ __forceinline__ void load_lanes(const uint8_t *payload, int64_t e0, int cnt,
                                           uint32_t (&v)[P]) {
  if (cnt == P) {
    if constexpr (WB == 1) {
      uint32_t w[P / 4];
      if constexpr (P == 4) {
        w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(payload + e0));
      } else {
        const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(payload + e0));
        w[0] = t.x;
        w[1] = t.y;
      }
#pragma unroll
      for (int i = 0; i < P; ++i) v[i] = (w[i / 4] >> (8 * (i % 4))) & 0xFFu;
    } else if constexpr (WB == 2) {
      uint32_t w[P / 2];
      if constexpr (P == 4) {
        const u32x2 t =
            __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(payload + 2 * e0));
        w[0] = t.x;
        w[1] = t.y;
      } else {
        const u32x4 t =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(payload + 2 * e0));
        w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
      }
#pragma unroll
      for (int i = 0; i < P; ++i) v[i] = (w[i / 2] >> (16 * (i % 2))) & 0xFFFFu;
    } else {
#pragma unroll
      for (int i = 0; i < P / 4; ++i) {
        const u32x4 t = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(payload + 4 * (e0 + 4 * i)));
        v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < P; ++e) {
      v[e] = 0;
      if (e < cnt)
#pragma unroll
        for (int b = 0; b < WB; ++b) v[e] |= (uint32_t)payload[(e0 + e) * WB + b] << (8 * b);
    }
  }
}

// One worker's quantisation (identical to k_quantize_pack) written as wire lanes.
template <int DT, int GRID, int WB, bool AL, bool NT>
__global__ __launch_bounds__(kBlock) void k_quantize_wire(WireQuantArgs a) {
  constexpr int P = DT == 0 ? 4 : 8;
  constexpr int NP = kChunk / (64 * P);
  constexpr int WAVES = kBlock / 64;
  constexpr int CPW = quant_tile(DT) / kChunk / WAVES;  // chunks per wave in a full tile
  // chunks whose loads a wave issues before it uses the first (as in k_quantize_pack)
  constexpr int GR = DT == 0 ? CPW : 1;
  static_assert(CPW % GR == 0, "group size");
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const float sf = (float)a.levels;
  const float lo_scale = ldexpf(1.0f, a.levels + 31);
  for (int64_t b = blockIdx.x; b < a.tv.ntiles; b += gridDim.x) {
    const int64_t t = xcd_tile(b, a.tv.ntiles);
    int64_t begin;
    int len, seg;
    tile_of(a.tv, t, quant_tile(DT), begin, len, seg);
    const SegQ q = seg_quant<GRID>(a.scale[seg], a.levels);
    // the fused pass's fast path: a part whose elements, in every active lane, lie below the
    // lowest nonzero level has levels 0 and +-1 only (bit for bit the general path's)
    const float bound = GRID == 0 ? 1.0f : ldexpf(1.0f, 1 - a.levels);
    const float up_scale = GRID == 0 ? 4294967296.0f : lo_scale;
    // bf16: |x| scaled by inv_up = inv * up_scale in one product, exact under the conditions
    // k_fused's double-buffered pass states (a tile outside them takes the general path)
    const float inv_up = q.inv * up_scale;
    const bool fold_ok =
        DT == 0 || (q.inv >= 0x1p-16f && inv_up < 0x1p127f && (GRID == 0 || a.levels <= 95));
    const float fast_below = q.valid && fold_ok ? below_bound(q.inv, bound) : 0.0f;
    // lanes of one part of cnt elements at e0, from its loaded values (zeros where missing)
    auto wire_part = [&](int64_t e0, int cnt, const float (&x)[P]) {
      uint32_t v[P];
      const uint32_t ctr = a.index_base + (uint32_t)e0;
      // AL (index_base a multiple of 8, e0 a multiple of P): ctr + e, e < P, only fills ctr's
      // zero low bits, so it is ctr ^ e with the same upper half: mix16(ctr + e) = mix16(ctr) ^ e
      const uint32_t m0 = mix16(ctr) ^ a.key_mix;
      float big = 0.0f;
#pragma unroll
      for (int e = 0; e < P; ++e) big = max_abs(big, x[e]);
      if (__all(big < fast_below)) {
#pragma unroll
        for (int e = 0; e < P; ++e) {
          const uint32_t h = fmix32_tail(AL ? m0 ^ (uint32_t)e : mix16(ctr + e) ^ a.key_mix);
          const float up = DT == 1 ? fabsf(x[e]) * inv_up : fabsf(x[e]) * q.inv * up_scale;
          const int32_t lin = (float)h < up ? (x[e] < 0.0f ? -1 : 1) : 0;
          v[e] = (uint32_t)(lin + a.offset);
        }
      } else {
#pragma unroll
        for (int e = 0; e < P; ++e) {
          const uint32_t h = fmix32_tail(AL ? m0 ^ (uint32_t)e : mix16(ctr + e) ^ a.key_mix);
          int32_t lin;
          if constexpr (GRID == 0)
            lin = (int32_t)copysignf(quant_uniform_mag(x[e], q.inv, sf, h), x[e]);
          else
            lin = exp_lin_of(quant_exp_index(x[e], q.inv, a.levels, lo_scale, h), x[e]);
          v[e] = (uint32_t)(lin + a.offset);
        }
      }
      store_lanes<P, WB, NT>(a.payload, e0, cnt, a.tv.n, v);
    };
    auto offset_part = [&](int64_t e0, int cnt) {
      uint32_t v[P];
#pragma unroll
      for (int e = 0; e < P; ++e) v[e] = (uint32_t)a.offset;
      store_lanes<P, WB, NT>(a.payload, e0, cnt, a.tv.n, v);
    };
    if (len == quant_tile(DT)) {
      // a full tile: each wave issues the loads of GR chunks before it uses the first
      for (int i0 = 0; i0 < CPW; i0 += GR) {
        if (!q.valid) {
#pragma unroll
          for (int i = 0; i < GR; ++i)
#pragma unroll
            for (int j = 0; j < NP; ++j)
              offset_part(begin + part_offset<P>(wv + (i0 + i) * WAVES, j, lane), P);
          continue;
        }
        PartBuf<DT, P> buf[GR][NP];
#pragma unroll
        for (int i = 0; i < GR; ++i)
#pragma unroll
          for (int j = 0; j < NP; ++j)
            buf[i][j].load(a.grad, begin + part_offset<P>(wv + (i0 + i) * WAVES, j, lane), P);
#pragma unroll
        for (int i = 0; i < GR; ++i)
#pragma unroll
          for (int j = 0; j < NP; ++j) {
            float x[P];
#pragma unroll
            for (int e = 0; e < P; ++e) x[e] = buf[i][j].get(e);
            wire_part(begin + part_offset<P>(wv + (i0 + i) * WAVES, j, lane), P, x);
          }
      }
    } else {
      const int nch = (len + kChunk - 1) / kChunk;
      for (int ci = wv; ci < nch; ci += WAVES) {
#pragma unroll
        for (int j = 0; j < NP; ++j) {
          const int o = part_offset<P>(ci, j, lane);
          const int cnt = min(P, len - o);
          if (cnt <= 0) continue;
          if (q.valid) {
            float x[P];
            load_part<DT, P>(a.grad, begin + o, cnt, x);
            wire_part(begin + o, cnt, x);
          } else {
            offset_part(begin + o, cnt);
          }
        }
      }
    }
  }
}

// A summed payload of `world` workers back to the mean: sum = lane - world*o, then the decode
// of k_dequantize.
template <int P, int WB>
__global__ __launch_bounds__(kBlock) void k_dequantize_wire(WireDequantArgs a) {
  constexpr int NP = kChunk / (64 * P);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int64_t b = blockIdx.x; b < a.tv.ntiles; b += gridDim.x) {
    const int64_t t = xcd_tile(b, a.tv.ntiles);
    int64_t begin;
    int len, seg;
    tile_of(a.tv, t, kTileMix, begin, len, seg);
    const float f = seg_decode(a.scale[seg], a.denom);
    if (len == kTileMix) {
      constexpr int CPW = kTileMix / kChunk / (kBlock / 64);
      uint32_t lv[CPW][NP][P];
#pragma unroll
      for (int i = 0; i < CPW; ++i)
#pragma unroll
        for (int j = 0; j < NP; ++j)
          load_lanes<P, WB>(a.payload, begin + part_offset<P>(wv + i * (kBlock / 64), j, lane), P,
                            lv[i][j]);
#pragma unroll
      for (int i = 0; i < CPW; ++i)
#pragma unroll
        for (int j = 0; j < NP; ++j) {
          float m[P];
#pragma unroll
          for (int e = 0; e < P; ++e)
            m[e] = (float)(int32_t)((int64_t)lv[i][j][e] - a.world_offset) * f;
          store_mean<P>(a.out, a.out_dtype, begin + part_offset<P>(wv + i * (kBlock / 64), j, lane),
                        P, m);
        }
      continue;
    }
    const int nch = (len + kChunk - 1) / kChunk;
    for (int ci = wv; ci < nch; ci += kBlock / 64) {
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int o = part_offset<P>(ci, j, lane);
        const int cnt = min(P, len - o);
        if (cnt <= 0) continue;
        const int64_t e0 = begin + o;
        uint32_t v[P];
        load_lanes<P, WB>(a.payload, e0, cnt, v);
        float m[P];
#pragma unroll
        for (int e = 0; e < P; ++e)
          m[e] = (float)(int32_t)((int64_t)v[e] - a.world_offset) * f;
        store_mean<P>(a.out, a.out_dtype, e0, cnt, m);
      }
    }
  }
}

// ================================================================ fused pass
// For each element: the K workers' quantisations in registers, their integer sum, one decode.
// Workers are processed in batches of KB whose loads are all issued before any arithmetic.
// KT > 0 fixes K at compile time; KT = 0 loops over a runtime K.
//
// Fast path (FAST, without code stores): when one worker's elements in every lane of the wave
// have |x| below fast_below -- so that fl(|x| * inv) is below the lowest nonzero level (1 on
// the uniform grid, 2^(1-E) on the exponential one), as for almost every element of a large
// tensor -- the level is 0 or 1 and the draw rounds up when fp32(h) < fl(|x| * inv) * 2^32
// (uniform) or fl(|x| * inv) * 2^(E+31) (exponential), so the clamp, floor, fraction,
// exponent split and level selection of the general path drop out.  The results are the
// general path's bit for bit (adding copysign(0, x) or +0 to a sum that starts at +0 gives the
// same sum).  Used on the exponential grid (ResNet-50's 161 tensors x 8 workers: 0.190 ->
// 0.184 ms) and in the double-buffered bf16 pass below; in the single-buffered bf16 pass the
// uniform grid's shortcut saved instructions but no time (the waits for each batch's loads were
// then exposed), so it is not used there.
// The per-segment constants of k_fused.  In the double-buffered pass (pipe) the fast path
// scales |x| by inv_up = inv * 2^32 (or inv * 2^(E+31)) in one product.  Below the threshold
// fl(|x| * inv) < 1, and scaling it by that power of two is exact, so the one product equals
// it whenever fl(|x| * inv) is a normal number; when it is subnormal both thresholds lie in
// (0, 1] (products below 2^-126 * 2^(E+31) <= 1, hence E <= 95), where fp32(h) < threshold
// holds for h = 0 alone, so the two round up alike; they differ only if
// fl(|x| * inv) underflows to zero for a nonzero x, which inv >= 2^-16 rules out for bf16
// (whose smallest magnitude is 2^-133).  A segment whose scale fails these conditions takes
// the general path throughout (fast_below = 0).  The fast path runs on the exponential grid,
// and on the uniform grid in the double-buffered pass.
template <int GRID>
__device__ __forceinline__ SegConst seg_const(float S, int levels, double denom, int pipe) {
  const SegQ q = seg_quant<GRID>(S, levels);
  const float lo_scale = ldexpf(1.0f, levels + 31);
  const float inv_up = q.inv * (GRID == 0 ? 4294967296.0f : lo_scale);
  const bool fold_ok = q.inv >= 0x1p-16f && inv_up < 0x1p127f && (GRID == 0 || levels <= 95);
  const float fast_below =
      q.valid && (GRID == 1 || pipe) && (!pipe || fold_ok)
          ? below_bound(q.inv, GRID == 1 ? ldexpf(1.0f, 1 - levels) : 1.0f)
          : 0.0f;
  return SegConst{q.valid ? q.inv : 0.0f, seg_decode(S, denom), fast_below, inv_up};
}

template <int DT, int P, int NP, int KB>
__device__ __forceinline__ void fused_load(const FusedArgs &a, int k0, int kn,
                                           const int64_t (&e0)[NP], const int (&cnt)[NP],
                                           PartBuf<DT, P> (&x)[KB][NP]) {
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    if (kb < kn)
#pragma unroll
      for (int j = 0; j < NP; ++j)
        if (cnt[j] > 0) x[kb][j].load(a.grads[k0 + kb], e0[j], cnt[j]);
}

// FOLD: the fast path scales |x| by inv_up = inv * 2^32 (uniform) or inv * lo_scale
// (exponential) in one product, which the caller has shown equal to scaling fl(|x| * inv).
template <int DT, int GRID, int P, int NP, int KB, bool STORE, bool FAST, bool FOLD>
__device__ __forceinline__ void fused_compute(const FusedArgs &a, int k0, int kn,
                                              const PartBuf<DT, P> (&x)[KB][NP],
                                              const int64_t (&e0)[NP], const int (&cnt)[NP],
                                              const uint32_t (&am)[NP][P], const SegQ &q,
                                              float sf, float lo_scale, float fast_below,
                                              float inv_up, float (&accf)[NP][P],
                                              int32_t (&acci)[NP][P]) {
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    if (kb >= kn) break;
    const uint32_t km = a.key_mix[k0 + kb];
    bool fast = false;
    if constexpr (!STORE && FAST) {
      // parts past the end hold no elements and are left out; a part's missing elements
      // are loaded as zeros
      float big = 0.0f;
#pragma unroll
      for (int j = 0; j < NP; ++j)
        if (cnt[j] > 0)
#pragma unroll
          for (int e = 0; e < P; ++e) big = max_abs(big, x[kb][j].get(e));
      fast = __all(big < fast_below);
    }
    if (fast) {
#pragma unroll
      for (int j = 0; j < NP; ++j)
#pragma unroll
        for (int e = 0; e < P; ++e) {
          const float xv = x[kb][j].get(e);
          const uint32_t h = fmix32_tail(am[j][e] ^ km);
          const float up = FOLD ? fabsf(xv) * inv_up
                                : fabsf(xv) * q.inv * (GRID == 0 ? 4294967296.0f : lo_scale);
          if constexpr (GRID == 0)
            accf[j][e] += (float)h < up ? copysignf(1.0f, xv) : 0.0f;
          else
            acci[j][e] += (float)h < up ? (xv < 0.0f ? -1 : 1) : 0;
        }
      continue;
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      uint32_t c[P];
#pragma unroll
      for (int e = 0; e < P; ++e) {
        const float xv = x[kb][j].get(e);
        const uint32_t h = fmix32_tail(am[j][e] ^ km);
        if constexpr (GRID == 0) {
          const float m = quant_uniform_mag(xv, q.inv, sf, h);
          accf[j][e] += copysignf(m, xv);
          if constexpr (STORE) c[e] = uniform_code(m, xv, a.bits);
        } else {
          const uint32_t jj = quant_exp_index(xv, q.inv, a.levels, lo_scale, h);
          acci[j][e] += exp_lin_of(jj, xv);
          if constexpr (STORE) c[e] = exp_code(jj, xv, a.bits);
        }
      }
      if constexpr (STORE)
        if (cnt[j] > 0) store_codes<P, true>(a.codes[k0 + kb], e0[j], cnt[j], a.bits, c);
    }
  }
}

template <int DT, int GRID, int P, int NP, int KB, bool STORE>
__device__ __forceinline__ void fused_batch(const FusedArgs &a, int k0, int kn,
                                            const int64_t (&e0)[NP], const int (&cnt)[NP],
                                            const uint32_t (&am)[NP][P], const SegQ &q,
                                            float sf, float lo_scale, float fast_below,
                                            float (&accf)[NP][P], int32_t (&acci)[NP][P]) {
  PartBuf<DT, P> x[KB][NP];
  fused_load<DT, P, NP, KB>(a, k0, kn, e0, cnt, x);
  fused_compute<DT, GRID, P, NP, KB, STORE, GRID == 1, false>(a, k0, kn, x, e0, cnt, am, q, sf,
                                                              lo_scale, fast_below, 0.0f, accf,
                                                              acci);
}

// Without the code stores both grids fit in 128 VGPRs (4 waves per SIMD, enough loads in
// flight per CU to cover HBM latency); the code-storing variants keep more values live and
// get 256 (2 waves per SIMD) rather than spilling.
template <int KT, int DT, int GRID, bool STORE>
__global__ __launch_bounds__(kBlock)
__attribute__((amdgpu_waves_per_eu(!STORE ? 4 : 2, 8)))
void k_fused(FusedArgs a) {
  constexpr int P = DT == 0 ? 4 : 8;
  constexpr int NP = kChunk / (64 * P);
  // workers per batch: all of a small compiled K, 8 of 16; 4 where the fast path's second
  // branch needs the registers (the exponential grid without code stores)
  constexpr bool FASTP = !STORE && GRID == 1;
  constexpr int KB = FASTP && (KT == 0 || KT > 4) ? 4 : (KT == 16 ? 8 : (KT > 0 ? KT : 4));
  // bf16, 16 workers, no code stores: four batches of 4 workers, double-buffered so that the
  // next batch's loads are in flight while the current one is quantised, with the fast path on
  // both grids (GPT-2's buckets: 1.158 -> 0.946 ms from the double buffering, -> 0.84 ms with
  // the uniform grid's fast path, its per-lane maximum vote and one-product scaling)
  constexpr bool PIPE = !STORE && DT == 1 && KT == 16;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int K = KT > 0 ? KT : a.K;
  const float sf = (float)a.levels;
  const float lo_scale = ldexpf(1.0f, a.levels + 31);
  for (int64_t b = blockIdx.x; b < a.tv.ntiles; b += gridDim.x) {
    const int64_t t = xcd_tile(b, a.tv.ntiles);
    int64_t begin;
    int len, seg;
    tile_of(a.tv, t, kTileMix, begin, len, seg);
    // from the table k_seg_consts filled, or (a small pass other than the double-buffered one,
    // which the table's launch would cost more than this) computed here
    SegConst sc;
    if constexpr (PIPE)
      sc = a.segc[seg];
    else
      sc = a.segc ? a.segc[seg] : seg_const<GRID>(a.scale[seg], a.levels, a.denom, 0);
    const SegQ q{sc.inv, sc.inv > 0.0f};
    const float f = sc.f;
    const float inv_up = sc.inv_up;
    const float fast_below = sc.fast_below;
    const int nch = (len + kChunk - 1) / kChunk;
    for (int ci = wv; ci < nch; ci += kBlock / 64) {
      int64_t e0[NP];
      int cnt[NP];
      uint32_t am[NP][P];
      float accf[NP][P];
      int32_t acci[NP][P];
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int o = part_offset<P>(ci, j, lane);
        cnt[j] = min(P, len - o);
        e0[j] = begin + o;
        const uint32_t ctr = a.index_base + (uint32_t)e0[j];
#pragma unroll
        for (int e = 0; e < P; ++e) {
          am[j][e] = mix16(ctr + e);
          accf[j][e] = 0.0f;
          acci[j][e] = 0;
        }
      }
      if (q.valid) {
        if constexpr (PIPE) {
          PartBuf<DT, P> xa[4][NP], xb[4][NP];
          fused_load<DT, P, NP, 4>(a, 0, 4, e0, cnt, xa);
          fused_load<DT, P, NP, 4>(a, 4, 4, e0, cnt, xb);
          fused_compute<DT, GRID, P, NP, 4, STORE, true, true>(a, 0, 4, xa, e0, cnt, am, q,
                                                                     sf, lo_scale, fast_below,
                                                                     inv_up, accf, acci);
          fused_load<DT, P, NP, 4>(a, 8, 4, e0, cnt, xa);
          fused_compute<DT, GRID, P, NP, 4, STORE, true, true>(a, 4, 4, xb, e0, cnt, am, q,
                                                                     sf, lo_scale, fast_below,
                                                                     inv_up, accf, acci);
          fused_load<DT, P, NP, 4>(a, 12, 4, e0, cnt, xb);
          fused_compute<DT, GRID, P, NP, 4, STORE, true, true>(a, 8, 4, xa, e0, cnt, am, q,
                                                                     sf, lo_scale, fast_below,
                                                                     inv_up, accf, acci);
          fused_compute<DT, GRID, P, NP, 4, STORE, true, true>(a, 12, 4, xb, e0, cnt, am, q,
                                                                     sf, lo_scale, fast_below,
                                                                     inv_up, accf, acci);
        } else if constexpr (KT > 0) {
#pragma unroll 1
          for (int k0 = 0; k0 < KT; k0 += KB)
            fused_batch<DT, GRID, P, NP, KB, STORE>(a, k0, KB, e0, cnt, am, q, sf, lo_scale,
                                                    fast_below, accf, acci);
        } else {
#pragma unroll 1
          for (int k0 = 0; k0 < K; k0 += KB)
            fused_batch<DT, GRID, P, NP, KB, STORE>(a, k0, min(KB, K - k0), e0, cnt, am, q,
                                                    sf, lo_scale, fast_below, accf, acci);
        }
      } else if (STORE) {
        const uint32_t z[P] = {};
        for (int k = 0; k < K; ++k)
#pragma unroll
          for (int j = 0; j < NP; ++j)
            if (cnt[j] > 0) store_codes<P, true>(a.codes[k], e0[j], cnt[j], a.bits, z);
      }
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        if (cnt[j] <= 0) continue;
        int32_t s[P];
        float v[P];
#pragma unroll
        for (int e = 0; e < P; ++e) {
          // uniform sums are carried exactly in fp32; exponential sums in int32
          const float sumf = GRID == 0 ? accf[j][e] : (float)acci[j][e];
          s[e] = GRID == 0 ? (int32_t)accf[j][e] : acci[j][e];
          v[e] = sumf * f;
        }
        if (a.sums) store_sums<P>(a.sums, a.acc_bits, e0[j], cnt[j], s);
        store_mean<P>(a.out, a.out_dtype, e0[j], cnt[j], v);
      }
    }
  }
}

// ================================================================ per-worker-scale baselines
// QSGD / QSGDinf / NUQSGD with each worker's own scale: codes that are not summable, decoded by
// the receiver worker by worker.

__device__ __forceinline__ unsigned block_max_u32(unsigned v, unsigned *lds) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (unsigned)__shfl_xor((int)v, off, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds[w] = v;
  __syncthreads();
  unsigned t = 0u;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t = max(t, lds[i]);
  return t;
}

// Largest magnitude per (worker, norm tile), kept as the bit pattern of |x|: non-negative
// floats order like their patterns and an infinity or NaN lies above every finite value, so
// the integer maximum is exact and independent of order.  Grid: (tiles, K).
template <int DT>
__global__ __launch_bounds__(kBlock) void k_absmax_partial(NormArgs a) {
  constexpr int P = DT == 0 ? 4 : 8;
  constexpr int NP = kChunk / (64 * P);
  __shared__ unsigned lds[kBlock / 64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int k = blockIdx.y;
  const void *src = a.grads[k];
  unsigned *part = reinterpret_cast<unsigned *>(a.partial);
  for (int64_t t = blockIdx.x; t < a.tv.ntiles; t += gridDim.x) {
    int64_t begin;
    int len, seg;
    tile_of(a.tv, t, a.tile, begin, len, seg);
    const int nch = (len + kChunk - 1) / kChunk;
    unsigned m = 0u;
    for (int ci = wv; ci < nch; ci += kBlock / 64) {
      float x[NP][P];
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int o = part_offset<P>(ci, j, lane);
        const int cnt = min(P, len - o);
        if (cnt > 0) {
          load_part<DT, P>(src, begin + o, cnt, x[j]);
        } else {
#pragma unroll
          for (int e = 0; e < P; ++e) x[j][e] = 0.0f;
        }
      }
#pragma unroll
      for (int j = 0; j < NP; ++j)
#pragma unroll
        for (int e = 0; e < P; ++e) m = max(m, __float_as_uint(x[j][e]) & 0x7FFFFFFFu);
    }
    m = block_max_u32(m, lds);
    if (threadIdx.x == 0) part[(int64_t)k * a.tv.ntiles + t] = m;
  }
}

// One block per (segment, worker): the segment's tile partials reduced in a fixed order, then
// S = fp32(sqrt(sum)) (L2) or the largest magnitude (MAX); a non-finite S is stored as 0 and
// raises the status flag.
template <int NORM>
__global__ __launch_bounds__(kBlock) void k_worker_scales(NormArgs a, float *scales_out) {
  __shared__ double lds[kBlock / 64];
  __shared__ unsigned ldu[kBlock / 64];
  const int g = blockIdx.x, k = blockIdx.y;
  const int64_t t0 = seg_first_tile(a.tv, g), t1 = seg_first_tile(a.tv, g + 1);
  float S;
  bool bad;
  if constexpr (NORM == 0) {
    const double *part = a.partial + (int64_t)k * a.tv.ntiles;
    double acc = 0.0;
    for (int64_t t = t0 + threadIdx.x; t < t1; t += kBlock) acc += part[t];
    const double nrm = sqrt(block_sum(acc, lds));
    S = (float)nrm;
    bad = !(nrm <= DBL_MAX) || !(S <= FLT_MAX);
  } else {
    const unsigned *part = reinterpret_cast<const unsigned *>(a.partial) + (int64_t)k * a.tv.ntiles;
    unsigned m = 0u;
    for (int64_t t = t0 + threadIdx.x; t < t1; t += kBlock) m = max(m, part[t]);
    m = block_max_u32(m, ldu);
    S = __uint_as_float(m);
    bad = m >= 0x7F800000u;
  }
  if (threadIdx.x == 0) {
    if (bad) {
      S = 0.0f;
      atomicOr(a.status, 1u);
    }
    scales_out[(int64_t)k * a.tv.nseg + g] = S;
  }
}

// Per (worker, segment): the quantiser's s/S or 1/S (0 when the scale is not usable: the
// worker then adds nothing) and the decode factor fp32(S / D).
template <int GRID>
__global__ void k_worker_factors(const float *scales, int64_t count, int levels, double denom,
                                 float2 *fac) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  const float S = scales[i];
  const SegQ q = seg_quant<GRID>(S, levels);
  fac[i] = make_float2(q.valid ? q.inv : 0.0f, seg_decode(S, denom));
}

template <int DT, int P, int NP, int KB>
__device__ __forceinline__ void worker_load(const WorkerMeanArgs &a, int k0, int kn,
                                            const int64_t (&e0)[NP], const int (&cnt)[NP],
                                            PartBuf<DT, P> (&x)[KB][NP]) {
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    if (kb < kn)
#pragma unroll
      for (int j = 0; j < NP; ++j)
        if (cnt[j] > 0) x[kb][j].load(a.grads[k0 + kb], e0[j], cnt[j]);
}

template <int DT, int GRID, int P, int NP, int KB>
__device__ __forceinline__ void worker_compute(const WorkerMeanArgs &a, int k0, int kn,
                                               const PartBuf<DT, P> (&x)[KB][NP], float2 fl,
                                               const uint32_t (&am)[NP][P], float sf,
                                               float lo_scale, float (&acc)[NP][P]) {
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    if (kb >= kn) break;
    // worker k's factors sit in lane k of fl: read them into scalar registers
    const float inv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fl.x), k0 + kb));
    const float fac = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fl.y), k0 + kb));
    if (!(inv > 0.0f)) continue;
    const uint32_t km = a.key_mix[k0 + kb];
#pragma unroll
    for (int j = 0; j < NP; ++j)
#pragma unroll
      for (int e = 0; e < P; ++e) {
        const float xv = x[kb][j].get(e);
        const uint32_t h = fmix32_tail(am[j][e] ^ km);
        float l;
        if constexpr (GRID == 0)
          l = copysignf(quant_uniform_mag(xv, inv, sf, h), xv);
        else
          l = (float)exp_lin_of(quant_exp_index(xv, inv, a.levels, lo_scale, h), xv);
        acc[j][e] = fmaf(l, fac, acc[j][e]);  // one rounding per worker, in worker order
      }
  }
}

template <int DT, int GRID, int P, int NP, int KB>
__device__ __forceinline__ void worker_batch(const WorkerMeanArgs &a, int k0, int kn,
                                             float2 fl, const int64_t (&e0)[NP],
                                             const int (&cnt)[NP], const uint32_t (&am)[NP][P],
                                             float sf, float lo_scale, float (&acc)[NP][P]) {
  PartBuf<DT, P> x[KB][NP];
  worker_load<DT, P, NP, KB>(a, k0, kn, e0, cnt, x);
  worker_compute<DT, GRID, P, NP, KB>(a, k0, kn, x, fl, am, sf, lo_scale, acc);
}

// For each element: every worker quantised with its own scale and decoded with its own factor,
// accumulated by fused multiply-add in worker order.
template <int KT, int DT, int GRID>
__global__ __launch_bounds__(kBlock)
__attribute__((amdgpu_waves_per_eu(4, 8)))
void k_worker_mean(WorkerMeanArgs a) {
  constexpr int P = DT == 0 ? 4 : 8;
  constexpr int NP = kChunk / (64 * P);
  constexpr int KB = KT == 16 ? 8 : (KT > 0 ? KT : 4);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int K = KT > 0 ? KT : a.K;
  const float sf = (float)a.levels;
  const float lo_scale = ldexpf(1.0f, a.levels + 31);
  for (int64_t b = blockIdx.x; b < a.tv.ntiles; b += gridDim.x) {
    const int64_t t = xcd_tile(b, a.tv.ntiles);
    int64_t begin;
    int len, seg;
    tile_of(a.tv, t, kTileMix, begin, len, seg);
    const int nch = (len + kChunk - 1) / kChunk;
    // lane k holds worker k's (s/S or 1/S, decode factor) for this tile's segment (K <= 64)
    const float2 fl = a.fac[(int64_t)(lane < K ? lane : 0) * a.tv.nseg + seg];
    // bf16, 16 workers: double-buffered batches of 4 as in k_fused (the fast path measured
    // slower in this kernel: 0.985 against 0.948 ms on GPT-2's buckets, and is not used)
    constexpr bool PIPE = KT == 16 && DT == 1;
    for (int ci = wv; ci < nch; ci += kBlock / 64) {
      int64_t e0[NP];
      int cnt[NP];
      uint32_t am[NP][P];
      float acc[NP][P];
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int o = part_offset<P>(ci, j, lane);
        cnt[j] = min(P, len - o);
        e0[j] = begin + o;
        const uint32_t ctr = a.index_base + (uint32_t)e0[j];
#pragma unroll
        for (int e = 0; e < P; ++e) {
          am[j][e] = mix16(ctr + e);
          acc[j][e] = 0.0f;
        }
      }
      if constexpr (PIPE) {
        PartBuf<DT, P> xa[4][NP], xb[4][NP];
        worker_load<DT, P, NP, 4>(a, 0, 4, e0, cnt, xa);
        worker_load<DT, P, NP, 4>(a, 4, 4, e0, cnt, xb);
        worker_compute<DT, GRID, P, NP, 4>(a, 0, 4, xa, fl, am, sf, lo_scale, acc);
        worker_load<DT, P, NP, 4>(a, 8, 4, e0, cnt, xa);
        worker_compute<DT, GRID, P, NP, 4>(a, 4, 4, xb, fl, am, sf, lo_scale, acc);
        worker_load<DT, P, NP, 4>(a, 12, 4, e0, cnt, xb);
        worker_compute<DT, GRID, P, NP, 4>(a, 8, 4, xa, fl, am, sf, lo_scale, acc);
        worker_compute<DT, GRID, P, NP, 4>(a, 12, 4, xb, fl, am, sf, lo_scale, acc);
      } else {
#pragma unroll 1
        for (int k0 = 0; k0 < K; k0 += KB)
          worker_batch<DT, GRID, P, NP, KB>(a, k0, min(KB, K - k0), fl, e0, cnt, am, sf,
                                            lo_scale, acc);
      }
#pragma unroll
      for (int j = 0; j < NP; ++j)
        if (cnt[j] > 0) store_mean<P>(a.out, a.out_dtype, e0[j], cnt[j], acc[j]);
    }
  }
}

// The receiver's side after an allgather of per-worker-scaled codes: each worker's packed
// codes decoded with its own factor (lane k of `fl`), accumulated by fused multiply-add in
// worker order.  P elements per part: 8 for bf16 output, 4 for fp32, so that every store
// instruction of a wave writes one contiguous 1 KB block (with 8 fp32 per lane, each 16-byte
// store would cover only every other 16 bytes of the wave's span, and the half-written lines
// reach memory as partial writes).
template <int GRID, int BITS, int P>
__global__ __launch_bounds__(kBlock) void k_decode_workers(DecodeWorkersArgs a) {
  constexpr int NP = kChunk / (64 * P);
  constexpr int KB = 4;  // workers whose code loads are issued together
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int64_t b = blockIdx.x; b < a.tv.ntiles; b += gridDim.x) {
    const int64_t t = xcd_tile(b, a.tv.ntiles);
    int64_t begin;
    int len, seg;
    tile_of(a.tv, t, kTileMix, begin, len, seg);
    const float fl = a.fac[(int64_t)(lane < a.K ? lane : 0) * a.tv.nseg + seg].y;
    const int nch = (len + kChunk - 1) / kChunk;
    for (int ci = wv; ci < nch; ci += kBlock / 64) {
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int o = part_offset<P>(ci, j, lane);
        const int cnt = min(P, len - o);
        if (cnt <= 0) continue;
        const int64_t e0 = begin + o;
        float acc[P];
#pragma unroll
        for (int e = 0; e < P; ++e) acc[e] = 0.0f;
        for (int k0 = 0; k0 < a.K; k0 += KB) {
          // the code loads of KB workers go out together (a batch past the last worker loads
          // the last worker's codes again and adds nothing); products are added in worker order
          uint32_t c[KB][P];
#pragma unroll
          for (int u = 0; u < KB; ++u)
            load_codes<P>(a.codes[min(k0 + u, a.K - 1)], e0, cnt, BITS, c[u]);
#pragma unroll
          for (int u = 0; u < KB; ++u) {
            if (k0 + u >= a.K) break;
            const float f =
                __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fl), k0 + u));
#pragma unroll
            for (int e = 0; e < P; ++e)
              acc[e] = fmaf((float)lin_of_code<GRID>(c[u][e], BITS), f, acc[e]);
          }
        }
        store_mean<P>(a.out, a.out_dtype, e0, cnt, acc);
      }
    }
  }
}

__global__ void k_clear_u32(unsigned *p, int count) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0u;
}

int grid_for(int64_t work, int cap) {
  return (int)(work < cap ? (work > 0 ? work : 1) : cap);
}

}  // namespace

// ================================================================ launchers
hipError_t launch_global_norm(const NormArgs &a, int dtype, hipStream_t s) {
  if (a.tv.ntiles > 0) {
    dim3 grid(grid_for(a.tv.ntiles, kNormGrid), a.K);
    if (dtype == 0)
      hipLaunchKernelGGL(k_norm_partial<0>, grid, dim3(kBlock), 0, s, a);
    else
      hipLaunchKernelGGL(k_norm_partial<1>, grid, dim3(kBlock), 0, s, a);
  }
  if (a.tv.nseg > 0 && (int64_t)a.K * a.tv.ntiles <= kNormFinishMax) {
    hipLaunchKernelGGL(k_norm_finish, dim3(a.tv.nseg), dim3(kBlock), 0, s, a);
  } else if (a.tv.nseg > 0) {
    hipLaunchKernelGGL(k_norm_segments, dim3(a.tv.nseg, a.K), dim3(kBlock), 0, s, a);
    hipLaunchKernelGGL(k_norm_scale, dim3((a.tv.nseg + 255) / 256), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <bool AL, bool NT>
static void launch_qp(const QuantArgs &a, int dtype, int grid, dim3 g, hipStream_t s) {
  if (dtype == 0 && grid == 0)
    hipLaunchKernelGGL((k_quantize_pack<0, 0, AL, NT>), g, dim3(kBlock), 0, s, a);
  if (dtype == 0 && grid == 1)
    hipLaunchKernelGGL((k_quantize_pack<0, 1, AL, NT>), g, dim3(kBlock), 0, s, a);
  if (dtype == 1 && grid == 0)
    hipLaunchKernelGGL((k_quantize_pack<1, 0, AL, NT>), g, dim3(kBlock), 0, s, a);
  if (dtype == 1 && grid == 1)
    hipLaunchKernelGGL((k_quantize_pack<1, 1, AL, NT>), g, dim3(kBlock), 0, s, a);
}

hipError_t launch_quantize_pack(const QuantArgs &a, int dtype, int grid, bool nt,
                                hipStream_t s) {
  if (a.tv.ntiles == 0) return hipSuccess;
  dim3 g(grid_for(a.tv.ntiles, kGridAll));
  // counters that start on a multiple of 8 are mixed once per part
  const bool al = (a.index_base & 7u) == 0;
  if (al && nt) launch_qp<true, true>(a, dtype, grid, g, s);
  if (al && !nt) launch_qp<true, false>(a, dtype, grid, g, s);
  if (!al && nt) launch_qp<false, true>(a, dtype, grid, g, s);
  if (!al && !nt) launch_qp<false, false>(a, dtype, grid, g, s);
  return hipGetLastError();
}

hipError_t launch_accumulate(const AccArgs &a, int grid, hipStream_t s) {
  const int64_t ntiles = (a.n + kTileMix - 1) / kTileMix;
  if (ntiles == 0) return hipSuccess;
  dim3 g(grid_for(ntiles, kGridAll));
  const bool b8 = a.bits == 8;
  if (a.acc_bits == 16) {
    if (grid == 0 && b8) hipLaunchKernelGGL((k_accumulate<0, 8, 8>), g, dim3(kBlock), 0, s, a);
    if (grid == 0 && !b8) hipLaunchKernelGGL((k_accumulate<0, 8, 4>), g, dim3(kBlock), 0, s, a);
    if (grid == 1 && b8) hipLaunchKernelGGL((k_accumulate<1, 8, 8>), g, dim3(kBlock), 0, s, a);
    if (grid == 1 && !b8) hipLaunchKernelGGL((k_accumulate<1, 8, 4>), g, dim3(kBlock), 0, s, a);
  } else {
    if (grid == 0 && b8) hipLaunchKernelGGL((k_accumulate<0, 4, 8>), g, dim3(kBlock), 0, s, a);
    if (grid == 0 && !b8) hipLaunchKernelGGL((k_accumulate<0, 4, 4>), g, dim3(kBlock), 0, s, a);
    if (grid == 1 && b8) hipLaunchKernelGGL((k_accumulate<1, 4, 8>), g, dim3(kBlock), 0, s, a);
    if (grid == 1 && !b8) hipLaunchKernelGGL((k_accumulate<1, 4, 4>), g, dim3(kBlock), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_dequantize(const DequantArgs &a, hipStream_t s) {
  if (a.tv.ntiles == 0) return hipSuccess;
  dim3 g(grid_for(a.tv.ntiles, kGridAll));
  // 16-byte accesses on both sides: int16 -> bf16 with 8 elements per part, else 4
  if (a.acc_bits == 16 && a.out_dtype == 1)
    hipLaunchKernelGGL((k_dequantize<8, 16>), g, dim3(kBlock), 0, s, a);
  else if (a.acc_bits == 16)
    hipLaunchKernelGGL((k_dequantize<4, 16>), g, dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL((k_dequantize<4, 32>), g, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template <int DT, int GRID, bool AL, bool NT>
static void launch_qw(const WireQuantArgs &a, int wb, dim3 g, hipStream_t s) {
  if (wb == 1)
    hipLaunchKernelGGL((k_quantize_wire<DT, GRID, 1, AL, NT>), g, dim3(kBlock), 0, s, a);
  if (wb == 2)
    hipLaunchKernelGGL((k_quantize_wire<DT, GRID, 2, AL, NT>), g, dim3(kBlock), 0, s, a);
  if (wb == 4)
    hipLaunchKernelGGL((k_quantize_wire<DT, GRID, 4, AL, NT>), g, dim3(kBlock), 0, s, a);
}

template <int DT, int GRID>
static void launch_qw(const WireQuantArgs &a, int wb, bool nt, dim3 g, hipStream_t s) {
  // counters that start on a multiple of 8 are mixed once per part
  const bool al = (a.index_base & 7u) == 0;
  if (al && nt) launch_qw<DT, GRID, true, true>(a, wb, g, s);
  if (al && !nt) launch_qw<DT, GRID, true, false>(a, wb, g, s);
  if (!al && nt) launch_qw<DT, GRID, false, true>(a, wb, g, s);
  if (!al && !nt) launch_qw<DT, GRID, false, false>(a, wb, g, s);
}

hipError_t launch_quantize_wire(const WireQuantArgs &a, int dtype, int grid, int wb, bool nt,
                                hipStream_t s) {
  if (a.tv.ntiles == 0) return hipSuccess;
  const dim3 g(grid_for(a.tv.ntiles, kGridAll));
  if (dtype == 0 && grid == 0) launch_qw<0, 0>(a, wb, nt, g, s);
  if (dtype == 0 && grid == 1) launch_qw<0, 1>(a, wb, nt, g, s);
  if (dtype == 1 && grid == 0) launch_qw<1, 0>(a, wb, nt, g, s);
  if (dtype == 1 && grid == 1) launch_qw<1, 1>(a, wb, nt, g, s);
  return hipGetLastError();
}

hipError_t launch_dequantize_wire(const WireDequantArgs &a, int wb, hipStream_t s) {
  if (a.tv.ntiles == 0) return hipSuccess;
  const dim3 g(grid_for(a.tv.ntiles, kGridAll));
  // 16-byte output stores: 8 elements per part for bf16 output, 4 for fp32
  if (a.out_dtype == 1) {
    if (wb == 1) hipLaunchKernelGGL((k_dequantize_wire<8, 1>), g, dim3(kBlock), 0, s, a);
    if (wb == 2) hipLaunchKernelGGL((k_dequantize_wire<8, 2>), g, dim3(kBlock), 0, s, a);
    if (wb == 4) hipLaunchKernelGGL((k_dequantize_wire<8, 4>), g, dim3(kBlock), 0, s, a);
  } else {
    if (wb == 1) hipLaunchKernelGGL((k_dequantize_wire<4, 1>), g, dim3(kBlock), 0, s, a);
    if (wb == 2) hipLaunchKernelGGL((k_dequantize_wire<4, 2>), g, dim3(kBlock), 0, s, a);
    if (wb == 4) hipLaunchKernelGGL((k_dequantize_wire<4, 4>), g, dim3(kBlock), 0, s, a);
  }
  return hipGetLastError();
}

template <int GRID>
__global__ void k_seg_consts(const float *scale, int nseg, int levels, double denom, int pipe,
                             SegConst *out) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= nseg) return;
  out[g] = seg_const<GRID>(scale[g], levels, denom, pipe);
}

template <int DT, int GRID, bool STORE>
static void launch_fused_k(const FusedArgs &a, dim3 g, hipStream_t s) {
  switch (a.K) {
    case 1: hipLaunchKernelGGL((k_fused<1, DT, GRID, STORE>), g, dim3(kBlock), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_fused<2, DT, GRID, STORE>), g, dim3(kBlock), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_fused<4, DT, GRID, STORE>), g, dim3(kBlock), 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_fused<8, DT, GRID, STORE>), g, dim3(kBlock), 0, s, a); break;
    case 16: hipLaunchKernelGGL((k_fused<16, DT, GRID, STORE>), g, dim3(kBlock), 0, s, a); break;
    default: hipLaunchKernelGGL((k_fused<0, DT, GRID, STORE>), g, dim3(kBlock), 0, s, a); break;
  }
}

template <bool STORE>
static void launch_fused_s(const FusedArgs &a, int dtype, int grid, dim3 g, hipStream_t s) {
  if (dtype == 0 && grid == 0) launch_fused_k<0, 0, STORE>(a, g, s);
  if (dtype == 0 && grid == 1) launch_fused_k<0, 1, STORE>(a, g, s);
  if (dtype == 1 && grid == 0) launch_fused_k<1, 0, STORE>(a, g, s);
  if (dtype == 1 && grid == 1) launch_fused_k<1, 1, STORE>(a, g, s);
}

hipError_t launch_fused(const FusedArgs &a, int dtype, int grid, hipStream_t s) {
  if (a.tv.ntiles == 0) return hipSuccess;
  // the double-buffered pass: bf16, 16 workers, no code stores
  const int pipe = dtype == 1 && a.K == 16 && !a.store_codes;
  if (!pipe && a.tv.ntiles <= kSegConstTilesMin) {
    FusedArgs b = a;
    b.segc = nullptr;  // constants computed per tile
    dim3 g(grid_for(a.tv.ntiles, kGridAll));
    if (a.store_codes)
      launch_fused_s<true>(b, dtype, grid, g, s);
    else
      launch_fused_s<false>(b, dtype, grid, g, s);
    return hipGetLastError();
  }
  const dim3 gs((unsigned)((a.tv.nseg + 255) / 256));
  if (grid == 0)
    hipLaunchKernelGGL(k_seg_consts<0>, gs, dim3(256), 0, s, a.scale, a.tv.nseg, a.levels,
                       a.denom, pipe, a.segc);
  else
    hipLaunchKernelGGL(k_seg_consts<1>, gs, dim3(256), 0, s, a.scale, a.tv.nseg, a.levels,
                       a.denom, pipe, a.segc);
  dim3 g(grid_for(a.tv.ntiles, kGridAll));
  if (a.store_codes)
    launch_fused_s<true>(a, dtype, grid, g, s);
  else
    launch_fused_s<false>(a, dtype, grid, g, s);
  return hipGetLastError();
}

hipError_t launch_worker_scales(const NormArgs &a, int dtype, int norm, float *scales_out,
                                hipStream_t s) {
  if (a.tv.ntiles > 0) {
    dim3 grid(grid_for(a.tv.ntiles, kNormGrid), a.K);
    if (norm == 0 && dtype == 0) hipLaunchKernelGGL(k_norm_partial<0>, grid, dim3(kBlock), 0, s, a);
    if (norm == 0 && dtype == 1) hipLaunchKernelGGL(k_norm_partial<1>, grid, dim3(kBlock), 0, s, a);
    if (norm == 1 && dtype == 0) hipLaunchKernelGGL(k_absmax_partial<0>, grid, dim3(kBlock), 0, s, a);
    if (norm == 1 && dtype == 1) hipLaunchKernelGGL(k_absmax_partial<1>, grid, dim3(kBlock), 0, s, a);
  }
  if (a.tv.nseg > 0) {
    if (norm == 0)
      hipLaunchKernelGGL(k_worker_scales<0>, dim3(a.tv.nseg, a.K), dim3(kBlock), 0, s, a, scales_out);
    else
      hipLaunchKernelGGL(k_worker_scales<1>, dim3(a.tv.nseg, a.K), dim3(kBlock), 0, s, a, scales_out);
  }
  return hipGetLastError();
}

template <int DT, int GRID>
static void launch_worker_mean_k(const WorkerMeanArgs &a, dim3 g, hipStream_t s) {
  switch (a.K) {
    case 8: hipLaunchKernelGGL((k_worker_mean<8, DT, GRID>), g, dim3(kBlock), 0, s, a); break;
    case 16: hipLaunchKernelGGL((k_worker_mean<16, DT, GRID>), g, dim3(kBlock), 0, s, a); break;
    default: hipLaunchKernelGGL((k_worker_mean<0, DT, GRID>), g, dim3(kBlock), 0, s, a); break;
  }
}

hipError_t launch_worker_mean(const WorkerMeanArgs &a, const float *scales, int dtype, int grid,
                              hipStream_t s) {
  const int64_t count = (int64_t)a.K * a.tv.nseg;
  float2 *fac = const_cast<float2 *>(a.fac);
  if (grid == 0)
    hipLaunchKernelGGL(k_worker_factors<0>, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s,
                       scales, count, a.levels, a.denom, fac);
  else
    hipLaunchKernelGGL(k_worker_factors<1>, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s,
                       scales, count, a.levels, a.denom, fac);
  if (a.tv.ntiles > 0) {
    dim3 g(grid_for(a.tv.ntiles, kGridAll));
    if (dtype == 0 && grid == 0) launch_worker_mean_k<0, 0>(a, g, s);
    if (dtype == 0 && grid == 1) launch_worker_mean_k<0, 1>(a, g, s);
    if (dtype == 1 && grid == 0) launch_worker_mean_k<1, 0>(a, g, s);
    if (dtype == 1 && grid == 1) launch_worker_mean_k<1, 1>(a, g, s);
  }
  return hipGetLastError();
}

template <int P>
static void launch_dw(const DecodeWorkersArgs &a, int grid, dim3 g, hipStream_t s) {
  const bool b8 = a.bits == 8;
  if (grid == 0 && b8) hipLaunchKernelGGL((k_decode_workers<0, 8, P>), g, dim3(kBlock), 0, s, a);
  if (grid == 0 && !b8) hipLaunchKernelGGL((k_decode_workers<0, 4, P>), g, dim3(kBlock), 0, s, a);
  if (grid == 1 && b8) hipLaunchKernelGGL((k_decode_workers<1, 8, P>), g, dim3(kBlock), 0, s, a);
  if (grid == 1 && !b8) hipLaunchKernelGGL((k_decode_workers<1, 4, P>), g, dim3(kBlock), 0, s, a);
}

hipError_t launch_decode_workers(const DecodeWorkersArgs &a, const float *scales, int grid,
                                 int levels, double denom, hipStream_t s) {
  const int64_t count = (int64_t)a.K * a.tv.nseg;
  float2 *fac = const_cast<float2 *>(a.fac);
  if (grid == 0)
    hipLaunchKernelGGL(k_worker_factors<0>, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s,
                       scales, count, levels, denom, fac);
  else
    hipLaunchKernelGGL(k_worker_factors<1>, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s,
                       scales, count, levels, denom, fac);
  if (a.tv.ntiles > 0) {
    dim3 g(grid_for(a.tv.ntiles, kGridAll));
    if (a.out_dtype == 1)
      launch_dw<8>(a, grid, g, s);
    else
      launch_dw<4>(a, grid, g, s);
  }
  return hipGetLastError();
}

hipError_t launch_clear_u32(unsigned *p, int count, hipStream_t s) {
  hipLaunchKernelGGL(k_clear_u32, dim3((count + 255) / 256), dim3(256), 0, s, p, count);
  return hipGetLastError();
}

}  // namespace gq
