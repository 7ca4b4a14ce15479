// gq_api.cpp -- host side of libgq.so: the C ABI declared in include/gq.h.
//
// Every call validates its arguments on the host first (nothing is enqueued on failure),
// resolves the segment layout to a cached device tile table, derives the per-worker random
// keys, and enqueues the kernels on the caller's stream.  No call synchronises except
// gq_read_status, gq_trim and gq_destroy.  Device buffers a call has used (scratch, tables)
// are never freed while the context lives unless the caller asks (gq_trim): a buffer replaced
// by a larger one, or a table evicted from the cache, is retired, so that work still queued
// and graphs captured from earlier calls keep valid pointers.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "gq.h"
#include "gq_internal.h"
#include "gq_lq.h"

#define GQ_EXPORT extern "C" __attribute__((visibility("default")))

using gq::Tile;
using gq::TileView;

namespace {

struct SegTable {
  void *dev = nullptr;       // Tile[ntiles] followed by int64_t[nseg + 1]
  std::vector<char> host;    // kept alive: the source of the stream-ordered upload
  int64_t ntiles = 0;
  int32_t nseg = 0;
};

}  // namespace

struct gq_ctx {
  int device = 0;
  std::string err;
  void *scratch = nullptr;
  size_t scratch_bytes = 0;
  std::vector<SegTable> retired;    // replaced scratch (dev only) and evicted tables
  unsigned *status = nullptr;       // device word: bit 0 = non-finite norm
  unsigned *status_host = nullptr;  // pinned
  std::map<std::pair<std::vector<int64_t>, int>, SegTable> segcache;  // (offsets, tile size)
  gq::LqState lq;
};

namespace {

gq_status fail(gq_ctx *c, gq_status code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (c) c->err = buf;
  return code;
}

gq_status hip_fail(gq_ctx *c, hipError_t e, const char *what) {
  return fail(c, GQ_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
}

#define TRY(x)                     \
  do {                             \
    gq_status st_ = (x);           \
    if (st_ != GQ_OK) return st_;  \
  } while (0)

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): worker k's key is the low 32 bits of the
// generator's output number k+1 when started from state `seed`.
uint32_t worker_key(uint64_t seed, uint32_t worker) {
  uint64_t state = seed;
  uint64_t out = 0;
  for (uint32_t i = 0; i <= worker; ++i) {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    out = z ^ (z >> 31);
  }
  return static_cast<uint32_t>(out);
}

// The key's share of the first step of MurmurHash3's fmix32 (h ^= h >> 16 distributes over
// the XOR of counter and key), so the kernels mix the counter once for all workers.
uint32_t key_mix(uint32_t key) { return key ^ (key >> 16); }

gq_status ensure_scratch(gq_ctx *c, size_t bytes, hipStream_t) {
  if (bytes <= c->scratch_bytes) return GQ_OK;
  size_t want = bytes < (1u << 20) ? (1u << 20) : bytes + bytes / 4;
  void *fresh = nullptr;
  if (hipMalloc(&fresh, want) != hipSuccess)
    return fail(c, GQ_ENOMEM, "scratch allocation of %zu bytes failed", want);
  if (c->scratch) {
    SegTable old;
    old.dev = c->scratch;
    c->retired.push_back(std::move(old));
  }
  c->scratch = fresh;
  c->scratch_bytes = want;
  return GQ_OK;
}

// Validate the segment description (no table is built).
gq_status check_segments(gq_ctx *c, int64_t n, const int64_t *offsets, int32_t nseg) {
  if (n < 0) return fail(c, GQ_EINVAL, "n = %lld is negative", (long long)n);
  if (nseg < 1) return fail(c, GQ_EINVAL, "nseg = %d must be >= 1", nseg);
  if (offsets == nullptr) {
    if (nseg != 1) return fail(c, GQ_EINVAL, "offsets = NULL needs nseg = 1");
    return GQ_OK;
  }
  if (offsets[0] != 0) return fail(c, GQ_EINVAL, "offsets[0] = %lld, must be 0", (long long)offsets[0]);
  if (offsets[nseg] != n)
    return fail(c, GQ_EINVAL, "offsets[nseg] = %lld, must equal n = %lld",
                (long long)offsets[nseg], (long long)n);
  for (int32_t g = 0; g < nseg; ++g) {
    if (offsets[g + 1] < offsets[g]) return fail(c, GQ_EINVAL, "offsets decrease at segment %d", g);
    if (g > 0 && (offsets[g] % gq::kGroup) != 0)
      return fail(c, GQ_EALIGN, "interior offset %d = %lld is not a multiple of 8", g,
                  (long long)offsets[g]);
  }
  return GQ_OK;
}

// Whether every wave store of a quantiser's output lands on whole 128-byte lines: a wave
// stores 64 lanes' parts of P >= 4 elements (at least 128 bytes) at a multiple of its own size
// from a tile's start, and tiles start at segment starts plus multiples of the tile, so it does
// when the output's base and each segment's first byte (offsets[g] elements of bits_per_elem
// bits) sit on line boundaries.
static bool stores_on_lines(const void *out, const int64_t *offsets, int32_t nseg,
                            int bits_per_elem) {
  if ((reinterpret_cast<uintptr_t>(out) & 127) != 0) return false;
  if (offsets != nullptr)
    for (int32_t g = 0; g < nseg; ++g)
      if (((offsets[g] * bits_per_elem) & 1023) != 0) return false;
  return true;
}

// Validate the segment description and build the tile view (cached per layout).
gq_status resolve_segments(gq_ctx *c, int64_t n, const int64_t *offsets, int32_t nseg,
                           hipStream_t s, TileView *tv, int tile = gq::kTile) {
  TRY(check_segments(c, n, offsets, nseg));
  tv->n = n;
  tv->nseg = nseg;
  if (offsets == nullptr || nseg == 1) {
    tv->tiles = nullptr;
    tv->seg_tile_start = nullptr;
    tv->ntiles = (n + tile - 1) / tile;
    return GQ_OK;
  }
  auto key = std::make_pair(std::vector<int64_t>(offsets, offsets + nseg + 1), tile);
  auto it = c->segcache.find(key);
  if (it == c->segcache.end()) {
    if (c->segcache.size() >= 64) {
      for (auto &kv : c->segcache) c->retired.push_back(std::move(kv.second));
      c->segcache.clear();
    }
    SegTable t;
    std::vector<Tile> tiles;
    std::vector<int64_t> start(nseg + 1, 0);
    for (int32_t g = 0; g < nseg; ++g) {
      start[g] = (int64_t)tiles.size();
      for (int64_t b = offsets[g]; b < offsets[g + 1]; b += tile) {
        const int64_t rest = offsets[g + 1] - b;
        tiles.push_back(Tile{b, (int32_t)(rest < tile ? rest : tile), g});
      }
    }
    start[nseg] = (int64_t)tiles.size();
    t.ntiles = (int64_t)tiles.size();
    t.nseg = nseg;
    const size_t tb = tiles.size() * sizeof(Tile), sb = start.size() * sizeof(int64_t);
    t.host.resize(tb + sb);
    if (tb) std::memcpy(t.host.data(), tiles.data(), tb);
    std::memcpy(t.host.data() + tb, start.data(), sb);
    if (hipMalloc(&t.dev, tb + sb) != hipSuccess)
      return fail(c, GQ_ENOMEM, "segment table allocation failed");
    hipError_t e = hipMemcpyAsync(t.dev, t.host.data(), tb + sb, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) {
      (void)hipFree(t.dev);
      return hip_fail(c, e, "segment table upload");
    }
    it = c->segcache.emplace(std::move(key), std::move(t)).first;
  }
  const SegTable &t = it->second;
  tv->tiles = static_cast<const Tile *>(t.dev);
  tv->seg_tile_start = reinterpret_cast<const int64_t *>(static_cast<const char *>(t.dev) +
                                                         t.ntiles * sizeof(Tile));
  tv->ntiles = t.ntiles;
  return GQ_OK;
}

gq_status check_codec(gq_ctx *c, int32_t grid, int32_t levels, int32_t bits) {
  if (grid != GQ_UNIFORM && grid != GQ_EXP) return fail(c, GQ_EINVAL, "grid = %d", grid);
  if (bits != 4 && bits != 8) return fail(c, GQ_EINVAL, "bits = %d, must be 4 or 8", bits);
  const int32_t maxlv = (1 << (bits - 1)) - 1;
  if (levels < 1 || levels > maxlv)
    return fail(c, GQ_EINVAL, "levels = %d outside [1, %d] for %d-bit codes", levels, maxlv, bits);
  if (grid == GQ_EXP && levels > 30) return fail(c, GQ_EINVAL, "exponential levels = %d > 30", levels);
  return GQ_OK;
}

int64_t max_lin(int32_t grid, int32_t levels) {
  return grid == GQ_UNIFORM ? levels : (int64_t)1 << (levels - 1);
}

gq_status check_acc(gq_ctx *c, int32_t grid, int32_t levels, int32_t K, int32_t acc_bits) {
  if (acc_bits != 16 && acc_bits != 32) return fail(c, GQ_EINVAL, "acc_bits = %d", acc_bits);
  const int64_t lim = ((int64_t)1 << (acc_bits - 1)) - 1;
  if ((int64_t)K * max_lin(grid, levels) > lim)
    return fail(c, GQ_EOVERFLOW, "K * max level %lld = %lld does not fit int%d",
                (long long)max_lin(grid, levels), (long long)K * max_lin(grid, levels), acc_bits);
  return GQ_OK;
}

gq_status check_K(gq_ctx *c, int32_t K) {
  if (K < 1 || K > gq::kMaxWorkers) return fail(c, GQ_EINVAL, "K = %d outside [1, 64]", K);
  return GQ_OK;
}

gq_status check_dtype(gq_ctx *c, int32_t dt, const char *what) {
  if (dt != GQ_F32 && dt != GQ_BF16) return fail(c, GQ_EINVAL, "%s = %d", what, dt);
  return GQ_OK;
}

// Device buffers of an empty problem may be NULL (zero-size allocations have no address).
gq_status check_ptr(gq_ctx *c, const void *p, const char *what, bool may_be_null = false) {
  if (p == nullptr) return may_be_null ? GQ_OK : fail(c, GQ_EINVAL, "%s is NULL", what);
  if (!aligned16(p)) return fail(c, GQ_EALIGN, "%s is not 16-byte aligned", what);
  return GQ_OK;
}

gq_status check_counter(gq_ctx *c, int64_t n, uint32_t index_base) {
  if ((uint64_t)n + index_base > ((uint64_t)1 << 32))
    return fail(c, GQ_EINVAL, "n + index_base exceeds 2^32");
  return GQ_OK;
}

double decode_denominator(int32_t grid, int32_t levels, int32_t K) {
  return grid == GQ_UNIFORM ? (double)levels * (double)K : (double)K * std::ldexp(1.0, levels - 1);
}

}  // namespace

// ---------------------------------------------------------------- fixed scratch (no allocation)
// For callers that cannot allocate device memory (graph capture, tight serving loops): one
// fixed buffer per GPU, in the library's code object, that gq_global_norm_noalloc uses for its
// tile table, tile partials and per-worker norms.  In host code `scratch` names a host-side
// stand-in; its device address comes from hipGetSymbolAddress, resolved once per device (at
// gq_create, with that device current) and kept in g_fixed[device].
static __device__ __align__(256) unsigned char scratch[GQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_fixed_mu;
void *g_fixed[kMaxDevices] = {};

// The device address of `scratch` on the current device (resolved on the first call there).
hipError_t fixed_scratch(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_fixed_mu);
  if (!g_fixed[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_fixed[dev] = p;
  }
  *out = g_fixed[dev];
  return hipSuccess;
}

// The tile table of a segment layout given by value (at most kSegArgMax segments), built on
// the device so that no host buffer has to be uploaded: each block scans the segments' tile
// counts (one thread per segment) into every segment's first tile, block 0 stores those, and
// tile t finds its segment by binary search over them (an empty segment owns no tile).  The
// table is the one resolve_segments builds on the host.
constexpr int kSegArgMax = 256;
struct SegArg {
  int64_t offsets[kSegArgMax + 1];
  int64_t ntiles;
  int32_t nseg;
  int32_t tile;
};

__global__ __launch_bounds__(kSegArgMax) void k_build_tiles(const SegArg sa, Tile *tiles,
                                                            int64_t *start) {
  __shared__ int64_t st[kSegArgMax + 1];
  const int g = threadIdx.x;
  int64_t cnt = 0;
  if (g < sa.nseg) cnt = (sa.offsets[g + 1] - sa.offsets[g] + sa.tile - 1) / sa.tile;
  st[g + 1] = cnt;
  if (g == 0) st[0] = 0;
  __syncthreads();
  for (int d = 1; d < kSegArgMax; d <<= 1) {  // inclusive scan of st[1..kSegArgMax]
    const int64_t v = g >= d ? st[g + 1 - d] : 0;
    __syncthreads();
    st[g + 1] += v;
    __syncthreads();
  }
  if (blockIdx.x == 0)
    for (int i = g; i <= sa.nseg; i += kSegArgMax) start[i] = st[i];
  for (int64_t t = (int64_t)blockIdx.x * kSegArgMax + g; t < sa.ntiles;
       t += (int64_t)gridDim.x * kSegArgMax) {
    int lo = 0, hi = sa.nseg;  // the segment lo with st[lo] <= t < st[lo + 1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (st[mid] <= t)
        lo = mid;
      else
        hi = mid;
    }
    const int64_t b = sa.offsets[lo] + (t - st[lo]) * sa.tile;
    const int64_t rest = sa.offsets[lo + 1] - b;
    tiles[t] = Tile{b, (int32_t)(rest < sa.tile ? rest : sa.tile), lo};
  }
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

// ================================================================ ABI
GQ_EXPORT const char *gq_version(void) { return "gq 0.1 (gfx950)"; }

GQ_EXPORT gq_status gq_create(gq_ctx **out) {
  if (!out) return GQ_EINVAL;
  *out = nullptr;
  gq_ctx *c = new (std::nothrow) gq_ctx();
  if (!c) return GQ_ENOMEM;
  if (hipGetDevice(&c->device) != hipSuccess || hipMalloc(&c->status, sizeof(unsigned)) != hipSuccess ||
      hipHostMalloc(&c->status_host, sizeof(unsigned), hipHostMallocDefault) != hipSuccess ||
      hipMemset(c->status, 0, sizeof(unsigned)) != hipSuccess) {
    if (c->status) (void)hipFree(c->status);
    if (c->status_host) (void)hipHostFree(c->status_host);
    delete c;
    return GQ_ENOMEM;
  }
  void *fixed = nullptr;  // resolve the fixed scratch of this device now, while it is current
  if (fixed_scratch(&fixed) != hipSuccess) {
    (void)hipFree(c->status);
    (void)hipHostFree(c->status_host);
    delete c;
    return GQ_ELAUNCH;
  }
  *out = c;
  return GQ_OK;
}

GQ_EXPORT gq_status gq_trim(gq_ctx *c) {
  if (!c) return GQ_EINVAL;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(c, e, "hipDeviceSynchronize");
  for (auto &t : c->retired) (void)hipFree(t.dev);
  c->retired.clear();
  gq::lq_trim(c->lq);
  return GQ_OK;
}

GQ_EXPORT void gq_destroy(gq_ctx *c) {
  if (!c) return;
  (void)hipDeviceSynchronize();
  for (auto &t : c->retired) (void)hipFree(t.dev);
  if (c->scratch) (void)hipFree(c->scratch);
  if (c->status) (void)hipFree(c->status);
  if (c->status_host) (void)hipHostFree(c->status_host);
  for (auto &kv : c->segcache) (void)hipFree(kv.second.dev);
  gq::lq_release(c->lq);
  delete c;
}

GQ_EXPORT const char *gq_last_error(const gq_ctx *c) { return c ? c->err.c_str() : "no context"; }

GQ_EXPORT gq_status gq_read_status(gq_ctx *c, void *stream) {
  if (!c) return GQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(c->status_host, c->status, sizeof(unsigned), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(c, e, "reading the status word");
  const unsigned v = *c->status_host;
  e = gq::launch_clear_u32(c->status, 1, s);
  if (e != hipSuccess) return hip_fail(c, e, "clearing the status word");
  if (v & 1u) return fail(c, GQ_ENONFINITE, "a global norm was not finite; its segment scale was set to 0");
  return GQ_OK;
}

GQ_EXPORT gq_status gq_global_norm(gq_ctx *c, const void *const *grads, int32_t K, int32_t dtype,
                                   int64_t n, const int64_t *offsets, int32_t nseg,
                                   float *scale_out, double *norms_out, void *stream) {
  if (!c) return GQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TRY(check_K(c, K));
  TRY(check_dtype(c, dtype, "dtype"));
  if (!grads) return fail(c, GQ_EINVAL, "grads is NULL");
  for (int k = 0; k < K; ++k) TRY(check_ptr(c, grads[k], "grads[k]", n == 0));
  TRY(check_ptr(c, scale_out, "scale_out"));
  if (norms_out) TRY(check_ptr(c, norms_out, "norms_out"));
  TileView tv;
  const int tile = gq::norm_tile(K, n);
  TRY(resolve_segments(c, n, offsets, nseg, s, &tv, tile));
  const size_t npart = (size_t)K * (size_t)tv.ntiles;
  TRY(ensure_scratch(c, (npart + (size_t)K * nseg) * sizeof(double), s));
  gq::NormArgs a;
  std::memset(&a, 0, sizeof a);
  for (int k = 0; k < K; ++k) a.grads[k] = grads[k];
  a.partial = static_cast<double *>(c->scratch);
  a.norms = a.partial + npart;
  a.scale_out = scale_out;
  a.norms_out = norms_out;
  a.status = c->status;
  a.tv = tv;
  a.K = K;
  a.tile = tile;
  hipError_t e = gq::launch_global_norm(a, dtype, s);
  return e == hipSuccess ? GQ_OK : hip_fail(c, e, "global norm launch");
}

GQ_EXPORT gq_status gq_global_norm_noalloc(gq_ctx *c, const void *const *grads, int32_t K,
                                           int32_t dtype, int64_t n, const int64_t *offsets,
                                           int32_t nseg, float *scale_out, double *norms_out,
                                           void *stream) {
  if (!c) return GQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TRY(check_K(c, K));
  TRY(check_dtype(c, dtype, "dtype"));
  if (!grads) return fail(c, GQ_EINVAL, "grads is NULL");
  for (int k = 0; k < K; ++k) TRY(check_ptr(c, grads[k], "grads[k]", n == 0));
  TRY(check_ptr(c, scale_out, "scale_out"));
  if (norms_out) TRY(check_ptr(c, norms_out, "norms_out"));
  TRY(check_segments(c, n, offsets, nseg));
  const bool table = offsets != nullptr && nseg > 1;
  if (table && nseg > kSegArgMax)
    return fail(c, GQ_EINVAL, "nseg = %d: the allocation-free norm takes at most %d segments",
                nseg, kSegArgMax);
  const int64_t tile = gq::norm_tile(K, n);
  int64_t ntiles = 0;
  if (table)
    for (int32_t g = 0; g < nseg; ++g) ntiles += (offsets[g + 1] - offsets[g] + tile - 1) / tile;
  else
    ntiles = (n + tile - 1) / tile;
  // fixed scratch: [tile table | first tile of every segment | K x ntiles partials | K x nseg
  // norms], each part 256-byte aligned
  const size_t o_tiles = 0;
  const size_t o_start = o_tiles + (table ? align256((size_t)ntiles * sizeof(Tile)) : 0);
  const size_t o_part = o_start + (table ? align256((size_t)(nseg + 1) * sizeof(int64_t)) : 0);
  const size_t o_norms = o_part + align256((size_t)K * (size_t)ntiles * sizeof(double));
  const size_t need = o_norms + align256((size_t)K * (size_t)nseg * sizeof(double));
  if (need > (size_t)GQ_NOALLOC_SCRATCH_BYTES)
    return fail(c, GQ_EINVAL,
                "the allocation-free norm needs %zu bytes of scratch for K = %d, n = %lld, "
                "nseg = %d; its fixed buffer holds %zu",
                need, K, (long long)n, nseg, (size_t)GQ_NOALLOC_SCRATCH_BYTES);
  void *fixed = nullptr;
  hipError_t e = fixed_scratch(&fixed);
  if (e != hipSuccess) return hip_fail(c, e, "resolving the fixed scratch");
  char *base = static_cast<char *>(fixed);
  TileView tv;
  tv.n = n;
  tv.nseg = nseg;
  tv.ntiles = ntiles;
  tv.tiles = nullptr;
  tv.seg_tile_start = nullptr;
  if (table) {
    SegArg sa;
    std::memcpy(sa.offsets, offsets, (size_t)(nseg + 1) * sizeof(int64_t));
    sa.ntiles = ntiles;
    sa.nseg = nseg;
    sa.tile = (int32_t)tile;
    Tile *tiles = reinterpret_cast<Tile *>(base + o_tiles);
    int64_t *start = reinterpret_cast<int64_t *>(base + o_start);
    const int64_t blocks = (ntiles + kSegArgMax - 1) / kSegArgMax;
    hipLaunchKernelGGL(k_build_tiles, dim3((unsigned)(blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks))),
                       dim3(kSegArgMax), 0, s, sa, tiles, start);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(c, e, "tile table launch");
    tv.tiles = tiles;
    tv.seg_tile_start = start;
  }
  gq::NormArgs a;
  std::memset(&a, 0, sizeof a);
  for (int k = 0; k < K; ++k) a.grads[k] = grads[k];
  a.partial = reinterpret_cast<double *>(base + o_part);
  a.norms = reinterpret_cast<double *>(base + o_norms);
  a.scale_out = scale_out;
  a.norms_out = norms_out;
  a.status = c->status;
  a.tv = tv;
  a.K = K;
  a.tile = (int32_t)tile;
  e = gq::launch_global_norm(a, dtype, s);
  return e == hipSuccess ? GQ_OK : hip_fail(c, e, "global norm launch");
}

GQ_EXPORT gq_status gq_quantize_pack(gq_ctx *c, const void *grad, int32_t dtype, int64_t n,
                                     const int64_t *offsets, int32_t nseg, const float *scale,
                                     int32_t grid, int32_t levels, int32_t bits, uint64_t seed,
                                     uint32_t worker, uint32_t index_base, uint8_t *codes,
                                     void *stream) {
  if (!c) return GQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TRY(check_dtype(c, dtype, "dtype"));
  TRY(check_codec(c, grid, levels, bits));
  TRY(check_ptr(c, grad, "grad", n == 0));
  TRY(check_ptr(c, scale, "scale"));
  TRY(check_ptr(c, codes, "codes", n == 0));
  TRY(check_counter(c, n, index_base));
  TileView tv;
  TRY(resolve_segments(c, n, offsets, nseg, s, &tv, gq::quant_tile(dtype)));
  gq::QuantArgs a;
  a.grad = grad;
  a.scale = scale;
  a.codes = codes;
  a.tv = tv;
  a.levels = levels;
  a.bits = bits;
  a.key_mix = key_mix(worker_key(seed, worker));
  a.index_base = index_base;
  hipError_t e = gq::launch_quantize_pack(a, dtype, grid,
                                         stores_on_lines(codes, offsets, nseg, bits), s);
  return e == hipSuccess ? GQ_OK : hip_fail(c, e, "quantize launch");
}

GQ_EXPORT gq_status gq_accumulate_codes(gq_ctx *c, const uint8_t *const *codes, int32_t K, int64_t n,
                                        int32_t grid, int32_t levels, int32_t bits,
                                        int32_t acc_bits, void *sums, void *stream) {
  if (!c) return GQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TRY(check_K(c, K));
  TRY(check_codec(c, grid, levels, bits));
  TRY(check_acc(c, grid, levels, K, acc_bits));
  if (n < 0) return fail(c, GQ_EINVAL, "n is negative");
  if (!codes) return fail(c, GQ_EINVAL, "codes is NULL");
  for (int k = 0; k < K; ++k) TRY(check_ptr(c, codes[k], "codes[k]", n == 0));
  TRY(check_ptr(c, sums, "sums", n == 0));
  gq::AccArgs a;
  std::memset(&a, 0, sizeof a);
  for (int k = 0; k < K; ++k) a.codes[k] = codes[k];
  a.sums = sums;
  a.n = n;
  a.K = K;
  a.bits = bits;
  a.acc_bits = acc_bits;
  hipError_t e = gq::launch_accumulate(a, grid, s);
  return e == hipSuccess ? GQ_OK : hip_fail(c, e, "accumulate launch");
}

GQ_EXPORT gq_status gq_dequantize(gq_ctx *c, const void *sums, int32_t acc_bits, int64_t n,
                                  const int64_t *offsets, int32_t nseg, const float *scale,
                                  int32_t grid, int32_t levels, int32_t K, int32_t out_dtype,
                                  void *out, void *stream) {
  if (!c) return GQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TRY(check_K(c, K));
  if (grid != GQ_UNIFORM && grid != GQ_EXP) return fail(c, GQ_EINVAL, "grid = %d", grid);
  if (levels < 1 || levels > (grid == GQ_EXP ? 30 : 127))
    return fail(c, GQ_EINVAL, "levels = %d", levels);
  if (acc_bits != 16 && acc_bits != 32) return fail(c, GQ_EINVAL, "acc_bits = %d", acc_bits);
  TRY(check_dtype(c, out_dtype, "out_dtype"));
  TRY(check_ptr(c, sums, "sums", n == 0));
  TRY(check_ptr(c, scale, "scale"));
  TRY(check_ptr(c, out, "out", n == 0));
  TileView tv;
  TRY(resolve_segments(c, n, offsets, nseg, s, &tv, gq::kTileMix));
  gq::DequantArgs a;
  a.sums = sums;
  a.scale = scale;
  a.out = out;
  a.tv = tv;
  a.acc_bits = acc_bits;
  a.out_dtype = out_dtype;
  a.denom = decode_denominator(grid, levels, K);
  hipError_t e = gq::launch_dequantize(a, s);
  return e == hipSuccess ? GQ_OK : hip_fail(c, e, "dequantize launch");
}

// ---------------------------------------------------------------- summable wire payload
namespace {
int64_t wire_offset(int32_t grid, int32_t levels) {
  return grid == GQ_EXP ? ((int64_t)1 << (levels - 1)) : (int64_t)levels;
}

bool wire_codec_ok(int32_t grid, int32_t levels) {
  if (grid == GQ_UNIFORM) return levels >= 1 && levels <= 127;
  if (grid == GQ_EXP) return levels >= 1 && levels <= 30;
  return false;
}
}  // namespace

GQ_EXPORT int32_t gq_wire_lane_bytes(int32_t grid, int32_t levels, int32_t world) {
  if (!wire_codec_ok(grid, levels) || world < 1 || world > 65536) return 0;
  const int64_t top = (int64_t)world * 2 * wire_offset(grid, levels);
  for (int32_t w = 1; w <= 4; w *= 2)
    if (top <= (int64_t)((((uint64_t)1) << (8 * w)) - 1)) return w;
  return 0;
}

GQ_EXPORT gq_status gq_quantize_wire(gq_ctx *c, const void *grad, int32_t dtype, int64_t n,
                                     const int64_t *offsets, int32_t nseg, const float *scale,
                                     int32_t grid, int32_t levels, uint64_t seed,
                                     uint32_t worker, uint32_t index_base, int32_t world,
                                     void *payload, void *stream) {
  if (!c) return GQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TRY(check_dtype(c, dtype, "dtype"));
  const int32_t wb = gq_wire_lane_bytes(grid, levels, world);
  if (wb == 0)
    return fail(c, GQ_EINVAL, "no lane width holds %d workers at grid %d, levels %d", world,
                grid, levels);
  TRY(check_ptr(c, grad, "grad", n == 0));
  TRY(check_ptr(c, scale, "scale"));
  TRY(check_ptr(c, payload, "payload", n == 0));
  TRY(check_counter(c, n, index_base));
  TileView tv;
  TRY(resolve_segments(c, n, offsets, nseg, s, &tv, gq::quant_tile(dtype)));
  gq::WireQuantArgs a;
  a.grad = grad;
  a.scale = scale;
  a.payload = static_cast<uint8_t *>(payload);
  a.tv = tv;
  a.levels = levels;
  a.offset = (int32_t)wire_offset(grid, levels);
  a.key_mix = key_mix(worker_key(seed, worker));
  a.index_base = index_base;
  hipError_t e = gq::launch_quantize_wire(
      a, dtype, grid, wb, stores_on_lines(payload, offsets, nseg, 8 * wb), s);
  return e == hipSuccess ? GQ_OK : hip_fail(c, e, "quantize_wire launch");
}

GQ_EXPORT gq_status gq_dequantize_wire(gq_ctx *c, const void *payload, int64_t n,
                                       const int64_t *offsets, int32_t nseg,
                                       const float *scale, int32_t grid, int32_t levels,
                                       int32_t world, int32_t out_dtype, void *out,
                                       void *stream) {
  if (!c) return GQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t wb = gq_wire_lane_bytes(grid, levels, world);
  if (wb == 0)
    return fail(c, GQ_EINVAL, "no lane width holds %d workers at grid %d, levels %d", world,
                grid, levels);
  TRY(check_dtype(c, out_dtype, "out_dtype"));
  TRY(check_ptr(c, payload, "payload", n == 0));
  TRY(check_ptr(c, scale, "scale"));
  TRY(check_ptr(c, out, "out", n == 0));
  TileView tv;
  TRY(resolve_segments(c, n, offsets, nseg, s, &tv, gq::kTileMix));
  gq::WireDequantArgs a;
  a.payload = static_cast<const uint8_t *>(payload);
  a.scale = scale;
  a.out = out;
  a.tv = tv;
  a.world_offset = (int64_t)world * wire_offset(grid, levels);
  a.out_dtype = out_dtype;
  a.denom = decode_denominator(grid, levels, world);
  hipError_t e = gq::launch_dequantize_wire(a, wb, s);
  return e == hipSuccess ? GQ_OK : hip_fail(c, e, "dequantize_wire launch");
}

GQ_EXPORT gq_status gq_fused_mean(gq_ctx *c, const void *const *grads, int32_t K, int32_t dtype,
                                  int64_t n, const int64_t *offsets, int32_t nseg,
                                  const float *scale, int32_t grid, int32_t levels, int32_t bits,
                                  uint64_t seed, uint32_t index_base, int32_t acc_bits,
                                  uint8_t *const *codes_or_null, void *sums_or_null,
                                  int32_t out_dtype, void *out, void *stream) {
  if (!c) return GQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TRY(check_K(c, K));
  TRY(check_dtype(c, dtype, "dtype"));
  TRY(check_dtype(c, out_dtype, "out_dtype"));
  TRY(check_codec(c, grid, levels, bits));
  TRY(check_acc(c, grid, levels, K, acc_bits));
  TRY(check_counter(c, n, index_base));
  if (!grads) return fail(c, GQ_EINVAL, "grads is NULL");
  for (int k = 0; k < K; ++k) TRY(check_ptr(c, grads[k], "grads[k]", n == 0));
  if (codes_or_null)
    for (int k = 0; k < K; ++k) TRY(check_ptr(c, codes_or_null[k], "codes[k]", n == 0));
  if (sums_or_null) TRY(check_ptr(c, sums_or_null, "sums", n == 0));
  TRY(check_ptr(c, scale, "scale"));
  TRY(check_ptr(c, out, "out", n == 0));
  TileView tv;
  TRY(resolve_segments(c, n, offsets, nseg, s, &tv, gq::kTileMix));
  TRY(ensure_scratch(c, (size_t)nseg * sizeof(gq::SegConst), s));
  gq::FusedArgs a;
  std::memset(&a, 0, sizeof a);
  a.segc = static_cast<gq::SegConst *>(c->scratch);
  for (int k = 0; k < K; ++k) {
    a.grads[k] = grads[k];
    a.codes[k] = codes_or_null ? codes_or_null[k] : nullptr;
    a.key_mix[k] = key_mix(worker_key(seed, (uint32_t)k));
  }
  a.scale = scale;
  a.sums = sums_or_null;
  a.out = out;
  a.tv = tv;
  a.denom = decode_denominator(grid, levels, K);
  a.K = K;
  a.levels = levels;
  a.bits = bits;
  a.acc_bits = acc_bits;
  a.out_dtype = out_dtype;
  a.store_codes = codes_or_null ? 1 : 0;
  a.index_base = index_base;
  hipError_t e = gq::launch_fused(a, dtype, grid, s);
  return e == hipSuccess ? GQ_OK : hip_fail(c, e, "fused launch");
}

// ---------------------------------------------------------------- per-worker-scale baselines
GQ_EXPORT gq_status gq_worker_scales(gq_ctx *c, const void *const *grads, int32_t K, int32_t dtype,
                                     int64_t n, const int64_t *offsets, int32_t nseg, int32_t norm,
                                     float *scales_out, void *stream) {
  if (!c) return GQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TRY(check_K(c, K));
  TRY(check_dtype(c, dtype, "dtype"));
  if (norm != GQ_NORM_L2 && norm != GQ_NORM_MAX) return fail(c, GQ_EINVAL, "norm = %d", norm);
  if (!grads) return fail(c, GQ_EINVAL, "grads is NULL");
  for (int k = 0; k < K; ++k) TRY(check_ptr(c, grads[k], "grads[k]", n == 0));
  TRY(check_ptr(c, scales_out, "scales_out"));
  TileView tv;
  const int tile = gq::norm_tile(K, n);
  TRY(resolve_segments(c, n, offsets, nseg, s, &tv, tile));
  TRY(ensure_scratch(c, (size_t)K * (size_t)tv.ntiles * sizeof(double), s));
  gq::NormArgs a;
  std::memset(&a, 0, sizeof a);
  for (int k = 0; k < K; ++k) a.grads[k] = grads[k];
  a.partial = static_cast<double *>(c->scratch);
  a.status = c->status;
  a.tv = tv;
  a.K = K;
  a.tile = tile;
  hipError_t e = gq::launch_worker_scales(a, dtype, norm, scales_out, s);
  return e == hipSuccess ? GQ_OK : hip_fail(c, e, "worker scales launch");
}

GQ_EXPORT gq_status gq_worker_mean(gq_ctx *c, const void *const *grads, int32_t K, int32_t dtype,
                                   int64_t n, const int64_t *offsets, int32_t nseg,
                                   const float *scales, int32_t grid, int32_t levels,
                                   uint64_t seed, uint32_t index_base, int32_t out_dtype,
                                   void *out, void *stream) {
  if (!c) return GQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TRY(check_K(c, K));
  TRY(check_dtype(c, dtype, "dtype"));
  TRY(check_dtype(c, out_dtype, "out_dtype"));
  if (grid != GQ_UNIFORM && grid != GQ_EXP) return fail(c, GQ_EINVAL, "grid = %d", grid);
  if (levels < 1 || levels > (grid == GQ_EXP ? 30 : 127))
    return fail(c, GQ_EINVAL, "levels = %d outside [1, %d]", levels, grid == GQ_EXP ? 30 : 127);
  TRY(check_counter(c, n, index_base));
  if (!grads) return fail(c, GQ_EINVAL, "grads is NULL");
  for (int k = 0; k < K; ++k) TRY(check_ptr(c, grads[k], "grads[k]", n == 0));
  TRY(check_ptr(c, scales, "scales"));
  TRY(check_ptr(c, out, "out", n == 0));
  TileView tv;
  TRY(resolve_segments(c, n, offsets, nseg, s, &tv, gq::kTileMix));
  TRY(ensure_scratch(c, (size_t)K * (size_t)nseg * sizeof(float2), s));
  gq::WorkerMeanArgs a;
  std::memset(&a, 0, sizeof a);
  for (int k = 0; k < K; ++k) {
    a.grads[k] = grads[k];
    a.key_mix[k] = key_mix(worker_key(seed, (uint32_t)k));
  }
  a.fac = static_cast<const float2 *>(c->scratch);
  a.out = out;
  a.tv = tv;
  a.denom = decode_denominator(grid, levels, K);
  a.K = K;
  a.levels = levels;
  a.out_dtype = out_dtype;
  a.index_base = index_base;
  hipError_t e = gq::launch_worker_mean(a, scales, dtype, grid, s);
  return e == hipSuccess ? GQ_OK : hip_fail(c, e, "worker mean launch");
}

GQ_EXPORT gq_status gq_decode_workers(gq_ctx *c, const uint8_t *const *codes, int32_t K, int64_t n,
                                      const int64_t *offsets, int32_t nseg, const float *scales,
                                      int32_t grid, int32_t levels, int32_t bits,
                                      int32_t out_dtype, void *out, void *stream) {
  if (!c) return GQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TRY(check_K(c, K));
  TRY(check_codec(c, grid, levels, bits));
  TRY(check_dtype(c, out_dtype, "out_dtype"));
  if (!codes) return fail(c, GQ_EINVAL, "codes is NULL");
  for (int k = 0; k < K; ++k) TRY(check_ptr(c, codes[k], "codes[k]", n == 0));
  TRY(check_ptr(c, scales, "scales"));
  TRY(check_ptr(c, out, "out", n == 0));
  TileView tv;
  TRY(resolve_segments(c, n, offsets, nseg, s, &tv, gq::kTileMix));
  TRY(ensure_scratch(c, (size_t)K * (size_t)nseg * sizeof(float2), s));
  gq::DecodeWorkersArgs a;
  std::memset(&a, 0, sizeof a);
  for (int k = 0; k < K; ++k) a.codes[k] = codes[k];
  a.fac = static_cast<const float2 *>(c->scratch);
  a.out = out;
  a.tv = tv;
  a.K = K;
  a.bits = bits;
  a.out_dtype = out_dtype;
  hipError_t e = gq::launch_decode_workers(a, scales, grid, levels,
                                           decode_denominator(grid, levels, K), s);
  return e == hipSuccess ? GQ_OK : hip_fail(c, e, "decode workers launch");
}

GQ_EXPORT gq_status gq_logquant(gq_ctx *c, const float *F, int64_t rows, int32_t r, double alpha,
                                int32_t bits, int8_t *codes, float *colmax, float *F_hat_or_null,
                                void *stream) {
  if (!c) return GQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (rows < 0) return fail(c, GQ_EINVAL, "rows is negative");
  if (r < 1 || r > gq::kLqMaxRank) return fail(c, GQ_EINVAL, "r = %d outside [1, %d]", r, gq::kLqMaxRank);
  if (!(alpha > 0.0) || !std::isfinite(alpha)) return fail(c, GQ_EINVAL, "alpha must be positive and finite");
  if (bits < 2 || bits > 8) return fail(c, GQ_EINVAL, "bits = %d outside [2, 8]", bits);
  TRY(check_ptr(c, F, "F", rows == 0));
  TRY(check_ptr(c, codes, "codes", rows == 0));
  TRY(check_ptr(c, colmax, "colmax"));
  if (F_hat_or_null) TRY(check_ptr(c, F_hat_or_null, "F_hat", rows == 0));
  hipError_t e = gq::lq_logquant(c->lq, F, rows, r, alpha, bits, codes, colmax, F_hat_or_null, s);
  return e == hipSuccess ? GQ_OK : hip_fail(c, e, "logquant launch");
}

GQ_EXPORT gq_status gq_powersgd_logquant(gq_ctx *c, const float *G, float *E, float *Q, int64_t n,
                                         int64_t m, int32_t r, double alpha, int32_t bits_p,
                                         int32_t bits_q, int8_t *p_codes, float *p_colmax, int8_t *q_codes,
                                         float *q_colmax, float *p_hat_or_null,
                                         float *p_pre_or_null, float *q_pre_or_null, void *stream) {
  if (!c) return GQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (n < 1 || m < 1) return fail(c, GQ_EINVAL, "n = %lld, m = %lld must be >= 1", (long long)n, (long long)m);
  if (n > gq::kLqMaxRows) return fail(c, GQ_EINVAL, "n = %lld above %lld rows", (long long)n, (long long)gq::kLqMaxRows);
  if (m > (1ll << 30)) return fail(c, GQ_EINVAL, "m too large");
  if (r < 1 || r > gq::kLqMaxRank) return fail(c, GQ_EINVAL, "r = %d outside [1, %d]", r, gq::kLqMaxRank);
  if (!(alpha > 0.0) || !std::isfinite(alpha)) return fail(c, GQ_EINVAL, "alpha must be positive and finite");
  if (bits_p < 2 || bits_p > 8) return fail(c, GQ_EINVAL, "bits_p = %d outside [2, 8]", bits_p);
  if (bits_q < 2 || bits_q > 8) return fail(c, GQ_EINVAL, "bits_q = %d outside [2, 8]", bits_q);
  TRY(check_ptr(c, G, "G"));
  TRY(check_ptr(c, E, "E"));
  TRY(check_ptr(c, Q, "Q"));
  TRY(check_ptr(c, p_codes, "p_codes"));
  TRY(check_ptr(c, p_colmax, "p_colmax"));
  TRY(check_ptr(c, q_codes, "q_codes"));
  TRY(check_ptr(c, q_colmax, "q_colmax"));
  if (p_hat_or_null) TRY(check_ptr(c, p_hat_or_null, "p_hat"));
  if (p_pre_or_null) TRY(check_ptr(c, p_pre_or_null, "p_pre"));
  if (q_pre_or_null) TRY(check_ptr(c, q_pre_or_null, "q_pre"));
  gq::LqStepArgs a{G, E, Q, n, m, r, alpha, bits_p, bits_q, p_codes, p_colmax, q_codes, q_colmax,
                   p_hat_or_null, p_pre_or_null, q_pre_or_null};
  hipError_t e = gq::lq_step(c->lq, a, s);
  if (e == hipErrorOutOfMemory) return fail(c, GQ_ENOMEM, "LQ scratch allocation failed");
  return e == hipSuccess ? GQ_OK : hip_fail(c, e, "powersgd_logquant launch");
}

GQ_EXPORT gq_status gq_lq_step_workers(gq_ctx *c, const float *const *G, float *const *E,
                                       float *const *Q, int32_t K, int64_t n, int64_t m, int32_t r,
                                       double alpha, int32_t bits_p, int32_t bits_q,
                                       int8_t *p_codes, float *p_colmax, int8_t *q_codes,
                                       float *q_colmax, float *G_hat, float *p_pre_or_null,
                                       float *q_pre_or_null, void *stream) {
  if (!c) return GQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (K < 1 || K > gq::kLqMaxWorkers) return fail(c, GQ_EINVAL, "K = %d outside [1, %d]", K, gq::kLqMaxWorkers);
  if (!G || !E || !Q) return fail(c, GQ_EINVAL, "G, E and Q must be arrays of K pointers");
  if (n < 1 || m < 1) return fail(c, GQ_EINVAL, "n = %lld, m = %lld must be >= 1", (long long)n, (long long)m);
  if (n > gq::kLqMaxRows) return fail(c, GQ_EINVAL, "n = %lld above %lld rows", (long long)n, (long long)gq::kLqMaxRows);
  if (m > (1ll << 30)) return fail(c, GQ_EINVAL, "m too large");
  if (r < 1 || r > gq::kLqMaxRank) return fail(c, GQ_EINVAL, "r = %d outside [1, %d]", r, gq::kLqMaxRank);
  if (!(alpha > 0.0) || !std::isfinite(alpha)) return fail(c, GQ_EINVAL, "alpha must be positive and finite");
  if (bits_p < 2 || bits_p > 8) return fail(c, GQ_EINVAL, "bits_p = %d outside [2, 8]", bits_p);
  if (bits_q < 2 || bits_q > 8) return fail(c, GQ_EINVAL, "bits_q = %d outside [2, 8]", bits_q);
  for (int k = 0; k < K; ++k) {
    TRY(check_ptr(c, G[k], "G[k]"));
    TRY(check_ptr(c, E[k], "E[k]"));
    TRY(check_ptr(c, Q[k], "Q[k]"));
    if (E[k] == G_hat) return fail(c, GQ_EINVAL, "G_hat is E[%d]", k);
    for (int l = 0; l < k; ++l)
      if (E[l] == E[k] || Q[l] == Q[k])
        return fail(c, GQ_EINVAL, "workers %d and %d share an E or a Q buffer", l, k);
  }
  TRY(check_ptr(c, p_codes, "p_codes"));
  TRY(check_ptr(c, p_colmax, "p_colmax"));
  TRY(check_ptr(c, q_codes, "q_codes"));
  TRY(check_ptr(c, q_colmax, "q_colmax"));
  TRY(check_ptr(c, G_hat, "G_hat"));
  if (p_pre_or_null) TRY(check_ptr(c, p_pre_or_null, "p_pre"));
  if (q_pre_or_null) TRY(check_ptr(c, q_pre_or_null, "q_pre"));
  gq::LqWorkersStepArgs a;
  std::memset(&a, 0, sizeof a);
  for (int k = 0; k < K; ++k) {
    a.W.G[k] = G[k];
    a.W.E[k] = E[k];
    a.W.Q[k] = Q[k];
  }
  a.K = K;
  a.n = n;
  a.m = m;
  a.r = r;
  a.alpha = alpha;
  a.bits_p = bits_p;
  a.bits_q = bits_q;
  a.p_codes = p_codes;
  a.p_colmax = p_colmax;
  a.q_codes = q_codes;
  a.q_colmax = q_colmax;
  a.G_hat = G_hat;
  a.p_pre = p_pre_or_null;
  a.q_pre = q_pre_or_null;
  hipError_t e = gq::lq_step_workers(c->lq, a, s);
  if (e == hipErrorOutOfMemory) return fail(c, GQ_ENOMEM, "LQ scratch allocation failed");
  return e == hipSuccess ? GQ_OK : hip_fail(c, e, "lq_step_workers launch");
}
