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

template <int K, bool WRITE>
__global__ __launch_bounds__(256) void k_stream(Srcs s, int64_t nchunks, float *out,
                                                float *sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  f32x4 keep = {0.f, 0.f, 0.f, 0.f};
  for (int64_t c = wave; c < nchunks; c += nwaves) {
    const int64_t o0 = c * 512 + 4 * lane, o1 = o0 + 256;
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < K; ++k) {
      a += __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(s.x[k] + o0));
      b += __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(s.x[k] + o1));
    }
    if (WRITE) {
      __builtin_nontemporal_store(a, reinterpret_cast<f32x4 *>(out + o0));
      __builtin_nontemporal_store(b, reinterpret_cast<f32x4 *>(out + o1));
    } else {
      keep += a + b;
    }
  }
  if (!WRITE && keep.x == 1.25e-37f && keep.y == -3.0e33f) sink[0] = keep.z;
}

template <bool WRITE>
hipError_t launch(Srcs s, int K, int64_t nchunks, float *out, float *sink, hipStream_t st) {
  const dim3 g(4096), b(256);
  switch (K) {
    case 1: hipLaunchKernelGGL((k_stream<1, WRITE>), g, b, 0, st, s, nchunks, out, sink); break;
    case 2: hipLaunchKernelGGL((k_stream<2, WRITE>), g, b, 0, st, s, nchunks, out, sink); break;
    case 4: hipLaunchKernelGGL((k_stream<4, WRITE>), g, b, 0, st, s, nchunks, out, sink); break;
    case 8: hipLaunchKernelGGL((k_stream<8, WRITE>), g, b, 0, st, s, nchunks, out, sink); break;
    case 16: hipLaunchKernelGGL((k_stream<16, WRITE>), g, b, 0, st, s, nchunks, out, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// Streams the first (n / 512) * 512 elements of K fp32 buffers (K in {1, 2, 4, 8, 16}); with
// out != NULL also writes their sum there.  sink: one device float (written only to keep the
// read-only variant from being optimised away).  All pointers 16-byte aligned device memory.
// Returns 0 on success, 1 on a bad argument, 2 on a launch error.
GQC_EXPORT int gqc_stream(const float *const *srcs, int K, int64_t n, float *out, float *sink,
                          void *stream) {
  if (K < 1 || K > 16 || n < 0 || !srcs || !sink) return 1;
  Srcs s = {};
  for (int k = 0; k < K; ++k) {
    if (!srcs[k] || (reinterpret_cast<uintptr_t>(srcs[k]) & 15)) return 1;
    s.x[k] = srcs[k];
  }
  if (out && (reinterpret_cast<uintptr_t>(out) & 15)) return 1;
  const int64_t nchunks = n / 512;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = out ? launch<true>(s, K, nchunks, out, sink, st)
                           : launch<false>(s, K, nchunks, nullptr, sink, st);
  return e == hipSuccess ? 0 : 2;
}
