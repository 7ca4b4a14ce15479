// gq_internal.h -- types shared by the host API (gq_api.cpp) and the gfx950 kernels (*.hip)
// of libgq.so.  Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gq {

constexpr int kMaxWorkers = 64;
constexpr int kGroup = 8;            // elements per thread step: one 32 B fp32 / 16 B bf16 load
// Elements per tile (a tile never crosses a segment): 8192 fp32 for the one-worker quantisers
// (one read and one write stream; see quant_tile), 2048 for the kernels that mix several
// streams with a write stream (fused pass, integer sum, decodes), whose grids of small tiles
// in the XCD order of gq_stream.hip stream fastest (measured on the 1.3e9 x 8 fused pass:
// 9.2 ms with 8192-element tiles on 4096 resident blocks, 8.0 ms like this).
constexpr int kTile = 8192;
constexpr int kTileMix = 2048;
// The one-worker quantisers' tile is 32 KB of input: kTile fp32 or 2 kTile bf16 elements
// (measured on GPT-2's bf16 buckets: 8192-element tiles ran 5-6% slower).
constexpr int quant_tile(int dtype) { return dtype == 1 ? 2 * kTile : kTile; }
constexpr int kNormTile = 65536;     // elements per tile of the norm pass (one fp64 partial each)
constexpr int kNormTileMin = 4096;   // ... halved down to this while K x tiles < kNormGrid

constexpr int kBlock = 256;          // threads per block of the streaming kernels
constexpr int kGridAll = 1 << 30;    // grid cap of the element-wise kernels: one block per tile
constexpr int kNormGrid = 2048;      // blocks per worker of the norm pass
// Up to this many partials (K x tiles) one kernel finishes the norm (a block per segment sums
// every worker's partials and takes the maximum); above it the per-worker sums get a block
// each and the maximum a kernel of its own.
constexpr int64_t kNormFinishMax = 65536;
// Fused passes of at most this many tiles (other than the double-buffered bf16 one) compute
// their segment constants per tile.
constexpr int64_t kSegConstTilesMin = 4096;

// Tile of the norm pass for K workers of n elements: 65536, halved while the K x tiles blocks
// would not fill the GPU (kNormGrid), down to 4096.  The tile fixes the fp64 summation order,
// so every norm entry point takes it from here.
inline int norm_tile(int K, int64_t n) {
  int tile = kNormTile;
  while (tile > kNormTileMin && (int64_t)K * ((n + tile - 1) / tile) < kNormGrid) tile >>= 1;
  return tile;
}

// One tile of a segmented buffer: elements [begin, begin + len) of segment `seg`.
struct Tile {
  int64_t begin;
  int32_t len;
  int32_t seg;
};

// How tiles map onto segments.  With tiles == nullptr there is one segment [0, n) cut into
// tiles of the kernel's own size (kTileMix, quant_tile or the norm's tile); otherwise tiles[t]
// describes tile t and seg_tile_start[g] is the first tile of segment g (nseg + 1 entries).
struct TileView {
  const Tile *tiles;
  const int64_t *seg_tile_start;
  int64_t ntiles;
  int64_t n;
  int32_t nseg;
};

struct NormArgs {
  const void *grads[kMaxWorkers];
  double *partial;        // K * ntiles
  double *norms;          // K * nseg (scratch)
  float *scale_out;       // nseg
  double *norms_out;      // K * nseg or nullptr
  unsigned *status;       // bit 0: a non-finite norm
  TileView tv;
  int32_t K;
  int32_t tile;           // elements per tile (norm_tile)
};

struct QuantArgs {
  const void *grad;
  const float *scale;
  uint8_t *codes;
  TileView tv;
  int32_t levels;
  int32_t bits;
  uint32_t key_mix;       // key ^ (key >> 16): the key's share of fmix32's first step
  uint32_t index_base;
};

struct AccArgs {
  const uint8_t *codes[kMaxWorkers];
  void *sums;
  int64_t n;
  int32_t K;
  int32_t bits;
  int32_t acc_bits;
};

struct DequantArgs {
  const void *sums;
  const float *scale;
  void *out;
  TileView tv;
  int32_t acc_bits;
  int32_t out_dtype;
  double denom;           // D: s*K (uniform) or K*2^(E-1) (exponential)
};

struct WireQuantArgs {
  const void *grad;
  const float *scale;
  uint8_t *payload;
  TileView tv;
  int32_t levels;
  int32_t offset;         // o: s (uniform) or 2^(E-1) (exponential)
  uint32_t key_mix;
  uint32_t index_base;
};

struct WireDequantArgs {
  const uint8_t *payload;
  const float *scale;
  void *out;
  TileView tv;
  int64_t world_offset;   // world * o
  int32_t out_dtype;
  double denom;
};

// Per-segment constants of the fused pass, computed once per segment before the pass (tiles
// are small, so computing them per tile cost the vector ALUs about one instruction per
// worker-element) -- except in a pass of at most kSegConstTilesMin tiles (not the
// double-buffered bf16 one), whose time the extra launch would stretch by more than that: inv = s/S or 1/S (0 when the scale is not
// usable), the decode factor f, the fast path's threshold fast_below (0: no fast path) and
// inv_up = inv * 2^32 (uniform) or inv * 2^(E+31) (exponential).
struct SegConst {
  float inv;
  float f;
  float fast_below;
  float inv_up;
};

struct FusedArgs {
  const void *grads[kMaxWorkers];
  uint8_t *codes[kMaxWorkers];   // all nullptr unless codes are materialised
  uint32_t key_mix[kMaxWorkers];  // key ^ (key >> 16) per worker
  const float *scale;
  SegConst *segc;                // nseg entries (scratch), filled by launch_fused
  void *sums;                    // nullptr unless sums are materialised
  void *out;
  TileView tv;
  double denom;
  int32_t K;
  int32_t levels;
  int32_t bits;
  int32_t acc_bits;
  int32_t out_dtype;
  int32_t store_codes;
  uint32_t index_base;
};

struct WorkerMeanArgs {
  const void *grads[kMaxWorkers];
  uint32_t key_mix[kMaxWorkers];  // key ^ (key >> 16) per worker
  const float2 *fac;             // K * nseg: (s/S or 1/S, 0 if unusable; decode factor)
  void *out;
  TileView tv;
  double denom;                  // D: s*K (uniform) or K*2^(E-1) (exponential)
  int32_t K;
  int32_t levels;
  int32_t out_dtype;
  uint32_t index_base;
};

struct DecodeWorkersArgs {
  const uint8_t *codes[kMaxWorkers];
  const float2 *fac;             // K * nseg, as in WorkerMeanArgs (only the factor is used)
  void *out;
  TileView tv;
  int32_t K;
  int32_t bits;
  int32_t out_dtype;
};

// Kernel launchers (gq_stream.hip).  Each returns the launch error, if any.
hipError_t launch_global_norm(const NormArgs &a, int dtype, hipStream_t s);
// nt: every wave store of the output lands on whole 128-byte lines (stores_on_lines), so the
// quantisers store non-temporally; otherwise they store through L2.
hipError_t launch_quantize_pack(const QuantArgs &a, int dtype, int grid, bool nt,
                                hipStream_t s);
hipError_t launch_accumulate(const AccArgs &a, int grid, hipStream_t s);
hipError_t launch_dequantize(const DequantArgs &a, hipStream_t s);
hipError_t launch_fused(const FusedArgs &a, int dtype, int grid, hipStream_t s);
hipError_t launch_quantize_wire(const WireQuantArgs &a, int dtype, int grid, int wb, bool nt,
                                hipStream_t s);
hipError_t launch_dequantize_wire(const WireDequantArgs &a, int wb, hipStream_t s);
// Per-worker scales: a.partial holds K * ntiles fp64 sums (norm 0) or uint32 maxima (norm 1).
hipError_t launch_worker_scales(const NormArgs &a, int dtype, int norm, float *scales_out,
                                hipStream_t s);
// Fills a.fac from `scales`, then the per-element pass.
hipError_t launch_worker_mean(const WorkerMeanArgs &a, const float *scales, int dtype, int grid,
                              hipStream_t s);
// Fills a.fac from `scales`, then decodes the K code streams.
hipError_t launch_decode_workers(const DecodeWorkersArgs &a, const float *scales, int grid,
                                 int levels, double denom, hipStream_t s);
hipError_t launch_clear_u32(unsigned *p, int count, hipStream_t s);

}  // namespace gq
