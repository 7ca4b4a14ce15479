// gq_lq.h -- internal interface of the LQ-SGD kernels (gq_lq.hip) used by gq_api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <utility>
#include <vector>

namespace gq {

constexpr int kLqMaxRank = 8;

// Encode/decode tables of the log quantiser for one (alpha, bits), on the device.
struct LqTables {
  float *dev = nullptr;        // thr[L] then lvl[L + 1]
  std::vector<float> host;     // source of the stream-ordered upload, kept alive
  int L = 0;
};

struct LqState {
  void *scratch = nullptr;
  size_t bytes = 0;
  std::map<std::pair<double, int>, LqTables> tables;
};

struct LqStepArgs {
  const float *G;
  float *E;
  float *Q;
  int64_t n, m;
  int32_t r;
  double alpha;
  int32_t bits_p, bits_q;  // code widths of P and of Q'
  int8_t *p_codes;
  float *p_colmax;
  int8_t *q_codes;
  float *q_colmax;
  float *p_hat;
  float *p_pre;
  float *q_pre;
};

hipError_t lq_logquant(LqState &st, const float *F, int64_t rows, int r, double alpha, int bits,
                       int8_t *codes, float *colmax, float *Fhat, hipStream_t s);
hipError_t lq_step(LqState &st, const LqStepArgs &a, hipStream_t s);
void lq_release(LqState &st);

}  // namespace gq
