// gq_ceiling.hip -- measurement probe for bench.py (libgq_ceiling.so, not part of libgq.so).
//
// A plain stream with the same memory pattern as the hot kernels and no arithmetic beyond a
// sum: K fp32 input streams read with the lane map of the streaming kernels (non-temporal
// 16-byte loads, each wave instruction one contiguous 1 KB block) and, optionally, one fp32
// output stream (their sum).  Its bandwidth is the empirical ceiling the quantisation kernels
// are compared with, beside the 8 TB/s HBM peak.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define GQC_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Srcs {
  const float *x[16];
};

// Lane L of a wave owns quads at chunk offsets 4L + 256j, j < Q: each instruction one
// contiguous 1 KB block, Q blocks per wave per stream and iteration.
template <int K, int Q, bool WRITE>
__global__ __launch_bounds__(256) void k_stream(Srcs s, int64_t nchunks, float *out,
                                                float *sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  f32x4 keep = {0.f, 0.f, 0.f, 0.f};
  for (int64_t c = wave; c < nchunks; c += nwaves) {
    f32x4 a[Q];
#pragma unroll
    for (int j = 0; j < Q; ++j) a[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
      for (int j = 0; j < Q; ++j)
        a[j] += __builtin_nontemporal_load(
            reinterpret_cast<const f32x4 *>(s.x[k] + c * 256 * Q + 256 * j + 4 * lane));
#pragma unroll
    for (int j = 0; j < Q; ++j) {
      if (WRITE)
        __builtin_nontemporal_store(a[j], reinterpret_cast<f32x4 *>(out + c * 256 * Q + 256 * j +
                                                                    4 * lane));
      else
        keep += a[j];
    }
  }
  if (!WRITE && keep.x == 1.25e-37f && keep.y == -3.0e33f) sink[0] = keep.z;
}

template <int K, bool WRITE>
hipError_t launch_q(Srcs s, int Q, int64_t n, float *out, float *sink, int grid, hipStream_t st) {
  const dim3 g(grid), b(256);
  const int64_t nchunks = n / (256 * Q);
  switch (Q) {
    case 1: hipLaunchKernelGGL((k_stream<K, 1, WRITE>), g, b, 0, st, s, nchunks, out, sink); break;
    case 2: hipLaunchKernelGGL((k_stream<K, 2, WRITE>), g, b, 0, st, s, nchunks, out, sink); break;
    case 4: hipLaunchKernelGGL((k_stream<K, 4, WRITE>), g, b, 0, st, s, nchunks, out, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool WRITE>
hipError_t launch(Srcs s, int K, int Q, int64_t n, float *out, float *sink, int grid,
                  hipStream_t st) {
  switch (K) {
    case 1: return launch_q<1, WRITE>(s, Q, n, out, sink, grid, st);
    case 2: return launch_q<2, WRITE>(s, Q, n, out, sink, grid, st);
    case 4: return launch_q<4, WRITE>(s, Q, n, out, sink, grid, st);
    case 8: return launch_q<8, WRITE>(s, Q, n, out, sink, grid, st);
    case 16: return launch_q<16, WRITE>(s, Q, n, out, sink, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Streams the first (n / 2048) * 2048 elements of K fp32 buffers (K in {1, 2, 4, 8, 16}) with
// `grid` 256-thread blocks and Q in {1, 2, 4} quads per lane per stream; with out != NULL
// also writes their sum there.  sink: one device float (written only to keep the read-only
// variant from being optimised away).  All pointers 16-byte aligned device memory.  Returns 0
// on success, 1 on a bad argument, 2 on a launch error.
GQC_EXPORT int gqc_stream(const float *const *srcs, int K, int64_t n, float *out, float *sink,
                          int grid, int Q, void *stream) {
  if (K < 1 || K > 16 || n < 0 || !srcs || !sink || grid < 1 || grid > 65536) return 1;
  if (Q != 1 && Q != 2 && Q != 4) return 1;
  Srcs s = {};
  for (int k = 0; k < K; ++k) {
    if (!srcs[k] || (reinterpret_cast<uintptr_t>(srcs[k]) & 15)) return 1;
    s.x[k] = srcs[k];
  }
  if (out && (reinterpret_cast<uintptr_t>(out) & 15)) return 1;
  const int64_t neff = n / 2048 * 2048;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = out ? launch<true>(s, K, Q, neff, out, sink, grid, st)
                           : launch<false>(s, K, Q, neff, nullptr, sink, grid, st);
  return e == hipSuccess ? 0 : 2;
}
