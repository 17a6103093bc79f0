// qsa_index_logits_topk: workspace layout and launch order of the indexer logits kernels
// (logits.hip, logits_mfma.hip) and the block top-k (topk.hip).  Follows QSAIndexer.forward
// (page "vllm.models.qwen4_exp.nvidia.qsa").
#include "select.h"

namespace qsa {

TopkLayout topk_layout(const qsa_topk_args& a) {
  TopkLayout L{};
  const int64_t T = a.num_tokens, R = a.num_requests;
  L.cols = a.max_seq_len / a.compress_ratio;
  if (L.cols < 1) L.cols = 1;
  L.col_stride = (L.cols + 63) / 64 * 64;
  L.key_tiles = (L.cols + kLogitsTilesPerWG * kLogitsKeysPerWG - 1) /
                (kLogitsTilesPerWG * kLogitsKeysPerWG);
  // Rows per window: all of them, or as many as the logits cap allows (at least one).
  int64_t rows = T;
  if (a.max_logits_bytes > 0) {
    rows = a.max_logits_bytes / ((int64_t)L.col_stride * (int64_t)sizeof(float));
    rows = rows < 1 ? 1 : (rows > T ? T : rows);
  }
  L.rows = (int32_t)rows;
  auto align = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t off = 0;
  L.off_logits = off;     off = align(off + (size_t)rows * L.col_stride * sizeof(float));
  L.key_blocks = (L.cols + 127) / 128;
  L.off_kmax = off;       off = align(off + (size_t)R * L.key_blocks * sizeof(float));
  L.off_band_idx = off;   off = align(off + (size_t)rows * L.col_stride * sizeof(int32_t));
  L.off_band_score = off; off = align(off + (size_t)rows * L.col_stride * sizeof(double));
  L.off_work = off;       off = align(off + 8 * sizeof(int));
  L.off_lexp = off;       off = align(off + (size_t)rows * sizeof(int32_t));
  L.total = off;
  return L;
}

SelectParams select_params(const qsa_topk_args& a, const TopkLayout& L, char* ws) {
  SelectParams P{};
  P.T = a.num_tokens;
  P.R = a.num_requests;
  P.Hi = a.num_index_heads;
  P.c = a.compress_ratio;
  P.c_log2 = __builtin_ctz((unsigned)a.compress_ratio);
  P.budget = a.budget;
  P.Pc = a.c_page_size;
  P.c_pages = a.c_pages;
  P.cbt_stride = a.c_block_table_stride;
  P.cbt_width = a.c_block_table_width;
  P.cols = L.cols;
  P.col_stride = L.col_stride;
  P.key_tiles = L.key_tiles;
  P.key_blocks = L.key_blocks;
  P.fp8 = a.index_dtype == QSA_DTYPE_FP8_E4M3;
  P.relu = a.index_agg == QSA_AGG_RELU_SUM;
  topk_bound_factors(P.Hi, P.relu, P.e_fold, P.e_mfma);
  P.qsl = a.query_start_loc;
  P.seq_lens = a.seq_lens;
  P.q_idx = a.q_idx;
  P.ckv = a.ckv;
  P.cbt = a.c_block_table;
  P.packed = a.packed;
  P.p_rs = a.packed_row_stride;
  if (ws != nullptr) {
    P.logits = reinterpret_cast<float*>(ws + L.off_logits);
    P.kmax = reinterpret_cast<float*>(ws + L.off_kmax);
    P.band_idx = reinterpret_cast<int32_t*>(ws + L.off_band_idx);
    P.band_score = reinterpret_cast<double*>(ws + L.off_band_score);
    P.work = reinterpret_cast<int*>(ws + L.off_work);
    P.lexp = reinterpret_cast<int32_t*>(ws + L.off_lexp);
  }
  P.row_lo = 0;
  P.row_hi = P.T;
  const bool mfma_ok = !P.relu && P.Hi <= kMfmaMaxHeads;
  P.mfma_min_rows = mfma_ok ? kMfmaMinRows : INT32_MAX;
  return P;
}

hipError_t launch_topk(const qsa_topk_args& a, const TopkLayout& L, char* ws, hipStream_t s,
                       Phase phase) {
  SelectParams P = select_params(a, L, ws);
  // Plain sum: requests with more than kMfmaMinRows rows are scored by the per-head matrix-core
  // contraction (bf16 or e4m3 operands), the others by the VALU kernel; each kernel skips the
  // other's requests.  ReLU-sum: every request goes to logits_relu_mfma_kernel, which clamps
  // each head's product before the head sum (the per-head contraction keeps the heads summed
  // in its accumulator, so it cannot clamp them).
  const bool mfma = P.mfma_min_rows == kMfmaMinRows && a.max_query_len > kMfmaMinRows;
  if (phase == Phase::kSecond) return launch_topk_select(P, s);
  const int rows_per_chunk = mfma ? kMfmaMinRows : a.max_query_len;
  // Window by window (one window without a logits cap; the split calls take one only): the
  // logits of the window's rows, then their selection, reusing the workspace.
  for (int lo = 0; lo < P.T; lo += L.rows) {
    P.row_lo = lo;
    P.row_hi = lo + L.rows < P.T ? lo + L.rows : P.T;
    hipError_t e = P.relu ? launch_logits_relu_mfma(P, s)
                          : launch_logits_valu(P, rows_per_chunk, mfma, s);
    if (e != hipSuccess) return e;
    if (mfma && (e = launch_logits_mfma(P, a.max_query_len, s)) != hipSuccess) return e;
    if (phase == Phase::kFirst) return hipSuccess;
    if ((e = launch_topk_select(P, s)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qsa
