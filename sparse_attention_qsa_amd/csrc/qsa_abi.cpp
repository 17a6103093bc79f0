// Host side of libqsa: argument validation, workspace sizing and dispatch.  Every check runs
// before any HIP call, so an invalid call has no side effect (and needs no GPU).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "qsa_internal.h"

namespace {

using qsa::kHeadDim;
using qsa::kRotaryDim;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

#define QSA_REQUIRE(cond, code) \
  do {                          \
    if (!(cond)) return (code); \
  } while (0)

constexpr qsa_status kInval = QSA_ERR_INVALID_ARGUMENT;
constexpr qsa_status kNotSup = QSA_ERR_NOT_SUPPORTED;

qsa_status check_dtype(qsa_dtype d) {
  return (d == QSA_DTYPE_BF16 || d == QSA_DTYPE_FP8_E4M3) ? QSA_OK : kNotSup;
}

qsa_status validate_compress(const qsa_compress_args* a) {
  QSA_REQUIRE(a != nullptr, kInval);
  QSA_REQUIRE(a->num_tokens >= 0 && a->num_requests >= 1, kInval);
  QSA_REQUIRE(a->head_dim == kHeadDim && a->rotary_dim == kRotaryDim, kNotSup);
  QSA_REQUIRE(a->num_index_heads >= 1 && a->num_index_heads <= 16, kNotSup);
  QSA_REQUIRE(pow2(a->compress_ratio) && a->compress_ratio >= 2 && a->compress_ratio <= 64,
              kNotSup);
  if (qsa_status s = check_dtype(a->index_dtype)) return s;
  const bool mrope = a->mrope_section[0] || a->mrope_section[1] || a->mrope_section[2];
  if (mrope) {
    QSA_REQUIRE(a->mrope_section[0] >= 0 && a->mrope_section[1] >= 0 && a->mrope_section[2] >= 0,
                kInval);
    QSA_REQUIRE(a->mrope_section[0] + a->mrope_section[1] + a->mrope_section[2] == kRotaryDim / 2,
                kInval);
    QSA_REQUIRE(a->ring_pos != nullptr, kInval);
  }
  QSA_REQUIRE(a->query_start_loc && a->seq_lens && a->q_proj && a->k_proj && a->positions &&
                  a->cos_sin && a->q_norm_weight && a->k_norm_weight && a->ring &&
                  a->ring_page && a->ckv && a->c_block_table && a->q_idx,
              kInval);
  QSA_REQUIRE(a->max_query_len >= 1 && a->max_position >= 1, kInval);
  QSA_REQUIRE(a->q_proj_row_stride >= (int64_t)a->num_index_heads * kHeadDim &&
                  a->q_proj_row_stride % 2 == 0,
              kInval);
  QSA_REQUIRE(a->k_proj_row_stride >= kHeadDim && a->k_proj_row_stride % 2 == 0, kInval);
  QSA_REQUIRE(a->ring_size >= a->compress_ratio && a->ring_pages >= 1, kInval);
  QSA_REQUIRE(a->c_page_size >= 1 && a->c_pages >= 1 && a->c_block_table_width >= 1 &&
                  a->c_block_table_stride >= a->c_block_table_width,
              kInval);
  QSA_REQUIRE(aligned(a->q_proj, 4) && aligned(a->k_proj, 4) && aligned(a->ring, 4) &&
                  aligned(a->q_norm_weight, 4) && aligned(a->k_norm_weight, 4) &&
                  aligned(a->ckv, 4) && aligned(a->q_idx, 4),
              kInval);
  if (a->main_qkv) {  // main-attention prepare
    QSA_REQUIRE(a->num_q_heads >= 1 && a->num_q_heads <= 128 && a->num_kv_heads >= 1 &&
                    a->num_kv_heads <= 64,
                kNotSup);
    QSA_REQUIRE(a->main_kv_dtype == QSA_DTYPE_BF16 || a->main_kv_dtype == QSA_DTYPE_FP8_E4M3,
                kNotSup);
    QSA_REQUIRE(a->main_q_norm_weight && a->main_k_norm_weight && a->main_q &&
                    a->main_kv_cache && a->main_slot_mapping,
                kInval);
    QSA_REQUIRE(a->main_qkv_row_stride % 2 == 0 &&
                    a->main_qkv_row_stride >=
                        (int64_t)(2 * a->num_q_heads + 2 * a->num_kv_heads) * kHeadDim,
                kInval);
    QSA_REQUIRE(a->main_num_pages >= 1 && a->main_page_size >= 1, kInval);
    const int64_t elt = a->main_kv_dtype == QSA_DTYPE_FP8_E4M3 ? 1 : 2;
    QSA_REQUIRE((a->main_kv_page_stride * elt) % 16 == 0 &&
                    (a->main_kv_head_stride * elt) % 16 == 0 &&
                    (a->main_kv_token_stride * elt) % 16 == 0 &&
                    a->main_kv_token_stride >= 2 * kHeadDim && a->main_kv_head_stride >= 0 &&
                    a->main_kv_page_stride >= 0,
                kInval);
    if (a->main_kv_dtype == QSA_DTYPE_FP8_E4M3) {
      QSA_REQUIRE(a->main_k_scale > 0.0f && a->main_v_scale > 0.0f && a->main_k_scale < 3.0e38f &&
                      a->main_v_scale < 3.0e38f,
                  kInval);
    }
    QSA_REQUIRE(aligned(a->main_qkv, 4) && aligned(a->main_q_norm_weight, 4) &&
                    aligned(a->main_k_norm_weight, 4) && aligned(a->main_q, 4) &&
                    aligned(a->main_kv_cache, 16) && aligned(a->main_slot_mapping, 8),
                kInval);
  }
  return QSA_OK;
}

qsa_status validate_topk(const qsa_topk_args* a) {
  QSA_REQUIRE(a != nullptr, kInval);
  QSA_REQUIRE(a->num_tokens >= 0 && a->num_requests >= 1, kInval);
  QSA_REQUIRE(a->head_dim == kHeadDim, kNotSup);
  QSA_REQUIRE(a->num_index_heads >= 1 && a->num_index_heads <= 16, kNotSup);
  QSA_REQUIRE(pow2(a->compress_ratio) && a->compress_ratio >= 2 && a->compress_ratio <= 64,
              kNotSup);
  if (qsa_status s = check_dtype(a->index_dtype)) return s;
  QSA_REQUIRE(a->budget >= a->compress_ratio && a->budget % a->compress_ratio == 0, kInval);
  QSA_REQUIRE(a->num_decode_requests >= 0 && a->num_decode_requests <= a->num_requests &&
                  a->decode_query_len >= 0,
              kInval);
  QSA_REQUIRE(a->max_query_len >= 1 && a->max_seq_len >= 1, kInval);
  QSA_REQUIRE(a->query_start_loc && a->seq_lens && a->q_idx && a->ckv && a->c_block_table &&
                  a->packed,
              kInval);
  QSA_REQUIRE(a->packed_row_stride >= (int64_t)a->budget + a->compress_ratio, kInval);
  QSA_REQUIRE(a->c_page_size >= 1 && a->c_pages >= 1 && a->c_block_table_width >= 1 &&
                  a->c_block_table_stride >= a->c_block_table_width,
              kInval);
  QSA_REQUIRE(aligned(a->ckv, 16) && aligned(a->q_idx, 4) && aligned(a->packed, 4), kInval);
  // Compressed cache rows are numbered in 32 bits (2^31 rows would be 512 GiB of bf16 keys).
  QSA_REQUIRE((int64_t)a->c_pages * a->c_page_size <= INT32_MAX, kNotSup);
  // A row's fast scores are held in the registers of one workgroup.
  QSA_REQUIRE(a->max_seq_len / a->compress_ratio <= qsa::kTopkMaxCols, kNotSup);
  QSA_REQUIRE(a->index_agg == QSA_AGG_SUM || a->index_agg == QSA_AGG_RELU_SUM, kNotSup);
  QSA_REQUIRE(a->max_logits_bytes >= 0, kInval);
  return QSA_OK;
}

qsa_status validate_gqa(const qsa_gqa_args* a) {
  QSA_REQUIRE(a != nullptr, kInval);
  QSA_REQUIRE(a->num_tokens >= 0 && a->num_requests >= 1, kInval);
  QSA_REQUIRE(a->head_dim == kHeadDim, kNotSup);
  QSA_REQUIRE(a->num_kv_heads >= 1 && a->num_q_heads >= a->num_kv_heads &&
                  a->num_q_heads % a->num_kv_heads == 0,
              kInval);
  const int G = a->num_q_heads / a->num_kv_heads;
  QSA_REQUIRE(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, kNotSup);
  QSA_REQUIRE(a->page_size >= 16 && a->page_size % 16 == 0, kNotSup);
  QSA_REQUIRE(a->q && a->kv_cache && a->block_table && a->token_to_req && a->packed && a->out,
              kInval);
  QSA_REQUIRE(a->num_pages >= 1 && a->block_table_width >= 1 &&
                  a->block_table_stride >= a->block_table_width,
              kInval);
  QSA_REQUIRE(a->packed_width >= 1 && a->packed_row_stride >= (int64_t)a->packed_width + 1, kInval);
  QSA_REQUIRE(a->kv_dtype == QSA_DTYPE_BF16 || a->kv_dtype == QSA_DTYPE_FP8_E4M3, kNotSup);
  QSA_REQUIRE(a->k_scale >= 0.0f && a->v_scale >= 0.0f && a->k_scale < 3.0e38f &&
                  a->v_scale < 3.0e38f,
              kInval);
  // Rows are gathered as 16-byte pieces: every stride is a multiple of 16 bytes.
  const int64_t elt = a->kv_dtype == QSA_DTYPE_FP8_E4M3 ? 1 : 2;
  QSA_REQUIRE((a->kv_page_stride * elt) % 16 == 0 && (a->kv_head_stride * elt) % 16 == 0 &&
                  (a->kv_token_stride * elt) % 16 == 0 && a->kv_token_stride >= 2 * kHeadDim &&
                  a->kv_head_stride >= 0 && a->kv_page_stride >= 0,
              kInval);
  const int64_t last = ((int64_t)(a->num_pages - 1) * a->kv_page_stride +
                        (int64_t)(a->num_kv_heads - 1) * a->kv_head_stride +
                        (int64_t)(a->page_size - 1) * a->kv_token_stride + 2 * kHeadDim) * elt;
  QSA_REQUIRE(last < (int64_t(1) << 36), kNotSup);  // 16-byte offsets fit 32 bits
  QSA_REQUIRE(a->q_row_stride % 2 == 0 &&
                  a->q_row_stride >= (int64_t)a->num_q_heads * a->q_head_stride,
              kInval);
  // A KV head's query heads are one matrix-core operand, read with 16-byte loads.
  QSA_REQUIRE(a->q_head_stride == kHeadDim, kNotSup);
  QSA_REQUIRE(a->out_row_stride % 2 == 0 && a->out_head_stride % 2 == 0 &&
                  a->out_head_stride >= kHeadDim,
              kInval);
  if (a->gate) {
    QSA_REQUIRE(a->gate_row_stride % 2 == 0 && a->gate_head_stride % 2 == 0 &&
                    a->gate_head_stride >= kHeadDim && aligned(a->gate, 4),
                kInval);
  }
  QSA_REQUIRE(aligned(a->q, 4) && aligned(a->kv_cache, 16) && aligned(a->out, 4) &&
                  aligned(a->packed, 4),
              kInval);
  QSA_REQUIRE(a->num_kv_heads <= 65535 && a->scale >= 0.0f, kInval);
  QSA_REQUIRE(a->row_tiles == 0 || a->row_tiles == 1, kInval);
  return QSA_OK;
}

qsa_status from_hip(hipError_t e) { return e == hipSuccess ? QSA_OK : QSA_ERR_HIP; }

qsa_status run_topk(const qsa_topk_args* a, void* ws, size_t ws_bytes, void* stream,
                    qsa::Phase phase) {
  if (a == nullptr || a->num_tokens < 0) return kInval;
  if (a->num_tokens == 0) return QSA_OK;  // nothing else is examined
  if (qsa_status s = validate_topk(a)) return s;
  const qsa::TopkLayout L = qsa::topk_layout(*a);
  if (ws == nullptr || ws_bytes < L.total) return QSA_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned(ws, 256)) return kInval;
  // The split calls hand the workspace over between them: one window only.
  if (phase != qsa::Phase::kAll && L.rows < a->num_tokens) return kNotSup;
  return from_hip(qsa::launch_topk(*a, L, static_cast<char*>(ws),
                                   reinterpret_cast<hipStream_t>(stream), phase));
}

qsa_status run_gqa(const qsa_gqa_args* a, void* ws, size_t ws_bytes, void* stream,
                   qsa::Phase phase) {
  if (a == nullptr || a->num_tokens < 0) return kInval;
  if (a->num_tokens == 0) return QSA_OK;  // nothing else is examined
  if (qsa_status s = validate_gqa(a)) return s;
  const qsa::GqaPlan plan = qsa::gqa_plan(*a);
  if (plan.ws_bytes > 0) {
    if (ws == nullptr || ws_bytes < plan.ws_bytes) return QSA_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(ws, 256)) return kInval;
  }
  return from_hip(qsa::launch_gqa(*a, plan, static_cast<char*>(ws),
                                  reinterpret_cast<hipStream_t>(stream), phase));
}

}  // namespace

extern "C" {

int32_t qsa_abi_version(void) { return QSA_ABI_VERSION; }

const char* qsa_status_string(qsa_status s) {
  switch (s) {
    case QSA_OK: return "QSA_OK";
    case QSA_ERR_INVALID_ARGUMENT: return "QSA_ERR_INVALID_ARGUMENT";
    case QSA_ERR_NOT_SUPPORTED: return "QSA_ERR_NOT_SUPPORTED";
    case QSA_ERR_WORKSPACE_TOO_SMALL: return "QSA_ERR_WORKSPACE_TOO_SMALL";
    case QSA_ERR_HIP: return "QSA_ERR_HIP";
  }
  return "QSA_ERR_UNKNOWN";
}

qsa_status qsa_compress(const qsa_compress_args* a, void* stream) {
  if (a == nullptr || a->num_tokens < 0) return kInval;
  if (a->num_tokens == 0) return QSA_OK;  // nothing else is examined
  if (qsa_status s = validate_compress(a)) return s;
  return from_hip(qsa::launch_compress(*a, reinterpret_cast<hipStream_t>(stream)));
}

size_t qsa_index_logits_topk_workspace_size(const qsa_topk_args* a) {
  if (validate_topk(a) != QSA_OK) return 0;
  return qsa::topk_layout(*a).total;
}

qsa_status qsa_index_logits_topk(const qsa_topk_args* a, void* ws, size_t ws_bytes,
                                 void* stream) {
  return run_topk(a, ws, ws_bytes, stream, qsa::Phase::kAll);
}

qsa_status qsa_index_logits(const qsa_topk_args* a, void* ws, size_t ws_bytes, void* stream) {
  return run_topk(a, ws, ws_bytes, stream, qsa::Phase::kFirst);
}

qsa_status qsa_block_topk(const qsa_topk_args* a, void* ws, size_t ws_bytes, void* stream) {
  return run_topk(a, ws, ws_bytes, stream, qsa::Phase::kSecond);
}

}  // extern "C"

namespace {

// qsa_compress + qsa_index_logits_topk as one call: validated as the two calls are, fused when
// prep_logits_fusable says so, else the two calls back to back.
qsa_status run_prep_topk(const qsa_compress_args* c, const qsa_topk_args* t, void* ws,
                         size_t ws_bytes, void* stream, qsa::Phase phase) {
  if (c == nullptr || t == nullptr || c->num_tokens < 0 || t->num_tokens < 0) return kInval;
  if (c->num_tokens > 0) {
    if (qsa_status s = validate_compress(c)) return s;
  }
  if (t->num_tokens > 0) {
    if (qsa_status s = validate_topk(t)) return s;
    const qsa::TopkLayout L = qsa::topk_layout(*t);
    if (ws == nullptr || ws_bytes < L.total) return QSA_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(ws, 256)) return kInval;
    if (phase != qsa::Phase::kAll && L.rows < t->num_tokens) return kNotSup;
    if (c->num_tokens > 0 && qsa::prep_logits_fusable(*c, *t))
      return from_hip(qsa::launch_prep_logits_topk(*c, *t, L, static_cast<char*>(ws),
                                                   reinterpret_cast<hipStream_t>(stream),
                                                   phase));
  }
  if (qsa_status s = qsa_compress(c, stream)) return s;
  return run_topk(t, ws, ws_bytes, stream, phase);
}

}  // namespace

extern "C" {

qsa_status qsa_compress_index_logits_topk(const qsa_compress_args* c, const qsa_topk_args* t,
                                          void* ws, size_t ws_bytes, void* stream) {
  return run_prep_topk(c, t, ws, ws_bytes, stream, qsa::Phase::kAll);
}

qsa_status qsa_compress_index_logits(const qsa_compress_args* c, const qsa_topk_args* t,
                                     void* ws, size_t ws_bytes, void* stream) {
  return run_prep_topk(c, t, ws, ws_bytes, stream, qsa::Phase::kFirst);
}

int32_t qsa_compress_index_logits_topk_fused(const qsa_compress_args* c,
                                             const qsa_topk_args* t) {
  if (c == nullptr || t == nullptr || c->num_tokens < 0 || t->num_tokens < 0) return -1;
  if (c->num_tokens > 0 && validate_compress(c) != QSA_OK) return -1;
  if (t->num_tokens > 0 && validate_topk(t) != QSA_OK) return -1;
  return c->num_tokens > 0 && t->num_tokens > 0 && qsa::prep_logits_fusable(*c, *t) ? 1 : 0;
}

int32_t qsa_sparse_gqa_num_splits(const qsa_gqa_args* a) {
  if (validate_gqa(a) != QSA_OK) return 0;
  return qsa::gqa_plan(*a).splits;
}

int32_t qsa_sparse_gqa_merge_kernel(const qsa_gqa_args* a) {
  if (validate_gqa(a) != QSA_OK) return -1;
  const qsa::GqaPlan p = qsa::gqa_plan(*a);
  return p.splits > 1 && !p.merge_in_wg ? 1 : 0;
}

size_t qsa_sparse_gqa_workspace_size(const qsa_gqa_args* a) {
  if (validate_gqa(a) != QSA_OK) return 0;
  return qsa::gqa_plan(*a).ws_bytes;
}

qsa_status qsa_sparse_gqa(const qsa_gqa_args* a, void* ws, size_t ws_bytes, void* stream) {
  return run_gqa(a, ws, ws_bytes, stream, qsa::Phase::kAll);
}

qsa_status qsa_sparse_gqa_partial(const qsa_gqa_args* a, void* ws, size_t ws_bytes,
                                  void* stream) {
  return run_gqa(a, ws, ws_bytes, stream, qsa::Phase::kFirst);
}

qsa_status qsa_sparse_gqa_merge(const qsa_gqa_args* a, void* ws, size_t ws_bytes, void* stream) {
  return run_gqa(a, ws, ws_bytes, stream, qsa::Phase::kSecond);
}

qsa_status qsa_sparse_gqa_noalloc(const qsa_gqa_args* a, void* stream) {
  if (a == nullptr || a->num_tokens < 0) return kInval;
  if (a->num_tokens == 0) return QSA_OK;  // nothing else is examined
  if (qsa_status s = validate_gqa(a)) return s;
  const qsa::GqaPlan plan = qsa::gqa_plan(*a);
  if (plan.ws_bytes > qsa::kGqaScratchBytes) return QSA_ERR_WORKSPACE_TOO_SMALL;
  char* ws = nullptr;
  if (plan.ws_bytes > 0) {
    if (qsa_status s = from_hip(qsa::gqa_scratch(&ws))) return s;
  }
  return from_hip(qsa::launch_gqa(*a, plan, ws, reinterpret_cast<hipStream_t>(stream),
                                  qsa::Phase::kAll));
}

size_t qsa_sparse_gqa_noalloc_scratch_bytes(void) { return qsa::kGqaScratchBytes; }

qsa_status qsa_diag_e4m3_decode(float* out, void* stream) {
  if (out == nullptr || !aligned(out, 4)) return kInval;
  return from_hip(qsa::launch_diag_e4m3(out, reinterpret_cast<hipStream_t>(stream)));
}

qsa_status qsa_diag_read_bandwidth(const void* src, const int32_t* chunk_index, int64_t n_chunks,
                                   int32_t chunk_bytes, uint32_t* sink, void* stream) {
  if (src == nullptr || sink == nullptr || n_chunks < 0 || !aligned(src, 16) ||
      !aligned(sink, 4) || chunk_bytes < 1024 || chunk_bytes > 4096 || chunk_bytes % 1024 != 0)
    return kInval;
  if (n_chunks == 0) return QSA_OK;
  return from_hip(qsa::launch_diag_read(src, chunk_index, n_chunks, chunk_bytes, sink,
                                        reinterpret_cast<hipStream_t>(stream)));
}

qsa_status qsa_diag_fp64_sqrt_div(const double* in, double* out, int64_t n, void* stream) {
  if (in == nullptr || out == nullptr || n < 0 || !aligned(in, 8) || !aligned(out, 8))
    return kInval;
  if (n == 0) return QSA_OK;
  return from_hip(qsa::launch_diag_fp64(in, out, n, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
