// Parameter block shared by the qsa_index_logits_topk kernels (indexer logits on the vector
// units and on the matrix cores, block top-k with expansion) and their launchers.
#pragma once

#include "qsa_internal.h"

namespace qsa {

struct SelectParams {
  int T, R, Hi, c, budget, Pc, c_pages, cbt_stride, cbt_width, cols, col_stride, key_tiles;
  int c_log2;         // log2(c) (c is a power of two)
  int key_blocks;     // 128-key blocks per request in the kmax array
  int mfma_min_rows;  // requests with more rows than this are scored by the MFMA kernel
  int row_lo, row_hi;  // the rows of this launch (a window under a logits memory cap); the
                       // per-row workspace arrays are indexed by row - row_lo
  bool fp8;
  bool relu;          // ReLU-sum aggregation (every request on the ReLU matrix-core kernel)
  // Factors F of the fast scores' error bounds E = F * kappa * A (kappa = max |k| over the
  // request's keys, A = sum |q|): the head-folded float32 score of the vector-unit logits, and
  // the matrix-core score.  They depend on Hi and the aggregation only (set by the host).
  double e_fold, e_mfma;
  const int32_t* qsl;
  const int32_t* seq_lens;
  const void* q_idx;
  const void* ckv;
  const int32_t* cbt;
  int32_t* packed;
  int64_t p_rs;
  float* logits;
  float* kmax;  // [R, key_blocks]: an upper bound of max |k| over each block of 128 keys
  int32_t* band_idx;
  double* band_score;
  int* work;  // [8] work counters of the MFMA kernel's queues, zeroed by the VALU kernel
  // [window rows]: a matrix-core row's logits are stored as fp16 values h, the score being
  // h * 2^lexp[row] (lexp >= 0 keeps every score of the row inside the fp16 range).
  int32_t* lexp;
};

// The parameter block of a qsa_index_logits_topk call over workspace `ws` (no workspace
// pointers when ws is null: for plans made before a workspace exists).
SelectParams select_params(const qsa_topk_args& a, const TopkLayout& L, char* ws);

// Requests with more rows than this are scored by the matrix-core logits kernel.
constexpr int kMfmaMinRows = 16;
// ... and at most this many indexer heads (they are folded into one Q in registers).
constexpr int kMfmaMaxHeads = 16;

// Launchers (each next to its kernels); arguments are validated by the caller.
// mfma: the call has requests scored on the matrix cores (rows_per_chunk is then 16).
hipError_t launch_logits_valu(const SelectParams& P, int rows_per_chunk, bool mfma,
                              hipStream_t s);
// Whether launch_logits_valu runs the wide instance (one-row requests filling the chip with
// 2048-key workgroups), the layout the fused decode prepare + logits kernel shares.
bool logits_wide(const SelectParams& P, int rows_per_chunk, bool mfma);
// ReLU-sum logits on the matrix cores (logits_relu.hip): every head's product a column of one
// contraction; the top-k bounds these scores with u = 2^-23.
hipError_t launch_logits_relu_mfma(const SelectParams& P, hipStream_t s);
// The persistent variant (logits_list.hip): `grid` workgroups walk the call's work list of
// (request, 1024-key item) pairs; at most kLogitsListReqs requests.
constexpr int kLogitsListReqs = 1024;
hipError_t launch_logits_list(const SelectParams& P, int nr, bool relu, bool kmax, unsigned grid,
                              hipStream_t s);
hipError_t launch_logits_mfma(const SelectParams& P, int max_query_len, hipStream_t s);
hipError_t launch_topk_select(const SelectParams& P, hipStream_t s);
// The error-bound factors of SelectParams (topk.hip).
void topk_bound_factors(int Hi, bool relu, double& e_fold, double& e_mfma);

}  // namespace qsa
