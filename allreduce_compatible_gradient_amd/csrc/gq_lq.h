// gq_lq.h -- internal interface of the LQ-SGD kernels (gq_lq.hip) used by gq_api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <utility>
#include <vector>

namespace gq {

constexpr int kLqMaxRank = 8;
constexpr int kLqMaxWorkers = 16;
// rows of the n x m matrices: the column pass's row chunks (64 rows or more) are a grid dimension
constexpr int64_t kLqMaxRows = 65535ll * 64;

// Per-worker matrices of a step of K workers (entries beyond K unused).
struct LqWorkerPtrs {
  const float *G[kLqMaxWorkers];  // n x m gradients
  float *E[kLqMaxWorkers];        // n x m errors (in/out; hold M = G + E between passes)
  float *Q[kLqMaxWorkers];        // m x r warm starts (in/out)
};

// Encode/decode tables of the log quantiser for one (alpha, bits), on the device.
struct LqTables {
  float *dev = nullptr;        // thr[L] then lvl[L + 1]
  std::vector<float> host;     // source of the stream-ordered upload, kept alive
  int L = 0;
  float alpha = 0.0f;          // the quantiser's alpha, as fp32
  float tl = 0.0f;             // L / log2(1 + alpha): the encode's first estimate
};

// Scratch of the steps.  A buffer replaced by a larger one is retired, not freed: a captured
// graph may still hold it; lq_trim frees the retired buffers.
struct LqState {
  void *scratch = nullptr;
  size_t bytes = 0;
  std::vector<void *> retired;
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

// K workers, each compressing its own M_w = G_w + E_w from its own warm start; messages stacked
// by worker; G_hat = (1/K) sum_w Phat_w Qhat_w^T; E_w <- M_w - G_hat; Q_w <- Qhat_w.
struct LqWorkersStepArgs {
  LqWorkerPtrs W;
  int32_t K;
  int64_t n, m;
  int32_t r;
  double alpha;
  int32_t bits_p, bits_q;
  int8_t *p_codes;   // K x n x r
  float *p_colmax;   // K x r
  int8_t *q_codes;   // K x m x r
  float *q_colmax;   // K x r
  float *G_hat;      // n x m
  float *p_pre;      // K x n x r, or null: the orthonormalised P of every worker
  float *q_pre;      // K x m x r, or null: every worker's Q' before quantisation
};

hipError_t lq_logquant(LqState &st, const float *F, int64_t rows, int r, double alpha, int bits,
                       int8_t *codes, float *colmax, float *Fhat, hipStream_t s);
hipError_t lq_step(LqState &st, const LqStepArgs &a, hipStream_t s);
hipError_t lq_step_workers(LqState &st, const LqWorkersStepArgs &a, hipStream_t s);
void lq_trim(LqState &st);
void lq_release(LqState &st);

}  // namespace gq
