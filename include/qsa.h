/*
 * qsa.h -- C ABI of libqsa.so, the MI355X (gfx950) implementation of the QSA sparse-attention
 * hot path:
 *
 *   qsa_compress           indexer Q prep, key pooling into the compressed-key cache, raw-key
 *                          ring update
 *   qsa_index_logits_topk  indexer logits, block top-k, expansion into the packed selection
 *                          buffer
 *   qsa_sparse_gqa         paged sparse GQA over the selected tokens, split across the
 *                          selection with a log-sum-exp merge, optional sigmoid output gate
 *
 * Pages the calls follow (cited by title and section):
 *   "vllm.models.qwen4_exp.nvidia.qsa" (newest revision): QSAIndexer.forward -- the indexer
 *       contract, its unfused reference path and the packed selection buffer;
 *       Qwen4ExpQSAImpl.forward -- the attention contract.
 *   "vllm.models.qwen4_exp.nvidia.qsa" (docs.vllm.ai): QSAIndexer.forward with the fused
 *       qsa_pre_indexer launch, the model for qsa_compress.
 *   "indexer_qsa.py": apply_qsa_rope, _supports_fused_pre_indexer.
 *   "vllm.models.qwen4_exp.nvidia.ops.qsa": qsa_compress_groups_with_ratio,
 *       qsa_store_cache_rows, qsa_sparse_paged_attention, _select_config.
 *   patch "qwen4_exp: FP8 E4M3 KV reader for QSA with a static scale sidecar": the body of
 *       _qsa_sparse_paged_gqa_splitk_kernel.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every data pointer is DEVICE memory owned by the caller; the library never allocates,
 *    frees, synchronises, or reads device data on the host.  Calls are asynchronous on the
 *    given stream (a hipStream_t; NULL = the default stream) and are safe to capture in a
 *    HIP graph (no memset nodes, no host reads).
 *  - bf16 tensors are passed as uint16_t bit patterns, fp8 tensors as uint8_t OCP e4m3fn
 *    codes.  Strides are in ELEMENTS; the innermost dimension is always contiguous.
 *  - Index tensors are int32, positions int64 (as on the pages).
 *  - Every argument is validated on the host before any launch: an error returns
 *    QSA_ERR_INVALID_ARGUMENT (shape / stride / metadata inconsistencies the host can see,
 *    the pages' ValueError), QSA_ERR_NOT_SUPPORTED (dtype, head_dim, rotary_dim or feature
 *    outside what is built, the pages' NotImplementedError), or QSA_ERR_WORKSPACE_TOO_SMALL,
 *    and leaves nothing launched.  QSA_ERR_HIP reports a failed launch.
 *  - Device metadata the host cannot see (request lengths, page tables, positions, packed
 *    indices) is bounds-checked in the kernels: an out-of-range page or index is masked
 *    exactly as documented per call, and no kernel ever reads or writes outside the buffers
 *    the sizes describe.  Faults inside a kernel surface at the caller's next stream sync.
 *  - num_tokens == 0 returns QSA_OK and launches nothing; no other argument is examined, so
 *    empty tensors may pass NULL pointers.
 *  - Calls that write overlapping buffers must not run concurrently on different streams.
 */
#ifndef QSA_H_
#define QSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_ABI_VERSION 9

typedef enum qsa_status {
  QSA_OK = 0,
  QSA_ERR_INVALID_ARGUMENT = 1,
  QSA_ERR_NOT_SUPPORTED = 2,
  QSA_ERR_WORKSPACE_TOO_SMALL = 3,
  QSA_ERR_HIP = 4
} qsa_status;

/* Indexer storage type: bf16, or OCP e4m3fn "without scales" (page
 * "vllm.models.qwen4_exp.nvidia.qsa", QSAIndexer.__init__, the indexer_kv_dtype branch). */
typedef enum qsa_dtype { QSA_DTYPE_BF16 = 0, QSA_DTYPE_FP8_E4M3 = 1 } qsa_dtype;

/* Head aggregation of the indexer score: the plain sum over heads (the reading of the pages'
 * weight-free selection), or the sum of max(0, .) of each head's product (an alternative kept
 * in case that reading is wrong). */
typedef enum qsa_agg { QSA_AGG_SUM = 0, QSA_AGG_RELU_SUM = 1 } qsa_agg;

/* ------------------------------------------------------------------------------------------
 * qsa_compress
 *
 * Follows QSAIndexer.forward's unfused reference path (page "vllm.models.qwen4_exp.nvidia.qsa")
 * and the fused qsa_pre_indexer launch it replaces (docs.vllm.ai revision):
 *   (1) indexer Q: per head, Gemma RMSNorm with q_norm_weight -> bf16 -> NeoX RoPE on dims
 *       0..63 at the row's rotary position (1-D, or interleaved MRoPE) -> bf16 -> [e4m3fn];
 *   (2) every group of compress_ratio raw keys that this step's rows complete (group g ends
 *       at token (g+1)*c - 1) is averaged -> bf16 -> RMSNorm with k_norm_weight -> bf16 ->
 *       RoPE at the position of token g*c (its logical position for 1-D RoPE, its position
 *       triple for MRoPE) -> bf16 -> [e4m3fn] and stored as compressed row g of the request
 *       (qsa_compress_groups_with_ratio + qsa_store_cache_rows, "vllm.models.qwen4_exp.
 *       nvidia.ops.qsa");
 *   (3) the raw-key ring then receives the step's last min(S, rows) keys (and their position
 *       triples for MRoPE) in slot token % S.  All ring reads of step (2) complete before any
 *       ring write.
 * Arithmetic is the canonical float64 chain of this project (halving sums over the 128 dims,
 * correctly rounded sqrt and divide, float64 -> float32 -> bf16 rounding, RNE e4m3fn cast that
 * maps overflow to NaN), so q_idx and the cache bytes are reproducible bit for bit.
 *
 * Main-attention prepare (optional, in the same launch; skipped when main_qkv is NULL).
 * Follows the fused qsa_prepare call of QSAIndexer.forward and Qwen4ExpQSAAttention (page
 * "vllm.models.qwen4_exp.nvidia.qsa": one launch does the indexer prepare, the main Q/K norm,
 * RoPE and gate split and the main K/V cache write):
 *   main_qkv row: for each of the Hq query heads its q (128 values) then its output gate (128
 *   values), then the Hkv K heads, then the Hkv V heads (bf16);
 *   (4) main Q: per head Gemma RMSNorm with main_q_norm_weight -> bf16 -> NeoX RoPE on dims
 *       0..63 with the same table and rotary position as the indexer Q -> bf16 -> main_q;
 *   (5) main K: the same with main_k_norm_weight; K and V (as given) are stored for every row
 *       whose main_slot_mapping entry s is >= 0 at page s / P, offset s % P of the main cache
 *       (rows whose page is >= main_num_pages are skipped too).  A bf16 cache receives the bf16
 *       values; an FP8_E4M3 cache receives e4m3fn(x / scale) with the quotient in float32,
 *       clamped to +-448 (the cache writer the FP8 KV reader patch page describes saturates).
 *   The gate is not copied: qsa_sparse_gqa reads it in place (gate = main_qkv + 128, gate
 *   head stride 256, gate row stride main_qkv_row_stride).
 * The main cache layout and strides are those of qsa_sparse_gqa's kv_cache.
 * ------------------------------------------------------------------------------------------ */
typedef struct qsa_compress_args {
  int32_t num_tokens;               /* T: rows of this step                                  */
  int32_t num_requests;             /* R                                                     */
  const int32_t* query_start_loc;   /* [R+1] row offsets, non-decreasing, [R] == T           */
  const int32_t* seq_lens;          /* [R] tokens of the request INCLUDING this step's rows;
                                       row i of request r sits at p = seq_lens[r]-n_r+i      */
  int32_t max_query_len;            /* host upper bound of n_r (selects the ring-write plan) */
  const uint16_t* q_proj;           /* [T, Hi*128] bf16 indexer Q (pre-projected)            */
  int64_t q_proj_row_stride;
  const uint16_t* k_proj;           /* [T, 128] bf16 raw indexer keys                        */
  int64_t k_proj_row_stride;
  const int64_t* positions;         /* [T] rotary positions, or [T,3] (T,H,W) for MRoPE      */
  int32_t mrope_section[3];         /* all zero: 1-D RoPE; else interleaved MRoPE sections,
                                       summing to rotary_dim/2                               */
  const float* cos_sin;             /* [max_position, 64]: cos in cols 0..31, sin in 32..63;
                                       positions are clamped into [0, max_position)          */
  int32_t max_position;
  const uint16_t* q_norm_weight;    /* [128] bf16 (Gemma convention: scale is 1 + w)        */
  const uint16_t* k_norm_weight;    /* [128] bf16                                            */
  float eps;                        /* RMSNorm epsilon (rms_norm_eps, 1e-6 by default)       */
  uint16_t* ring;                   /* [ring_pages, ring_size, 128] bf16 raw-key ring        */
  int64_t* ring_pos;                /* [ring_pages, ring_size, 3] int64, MRoPE only, else NULL */
  const int32_t* ring_page;         /* [R] ring page of each request; out of range: the
                                       request's ring is neither read (reads as 0) nor written */
  int32_t ring_pages;
  int32_t ring_size;                /* S >= compress_ratio (the pages require the ring to be
                                       wider than a group)                                   */
  void* ckv;                        /* [c_pages, c_page_size, 128] bf16 or e4m3fn            */
  const int32_t* c_block_table;     /* [R, c_block_table_stride] compressed-cache pages      */
  int32_t c_block_table_stride;
  int32_t c_block_table_width;      /* valid columns of c_block_table; a group whose page
                                       column or page is out of range is not stored          */
  int32_t c_page_size;              /* compressed rows per page                              */
  int32_t c_pages;
  int32_t num_index_heads;          /* Hi (1..16)                                            */
  int32_t head_dim;                 /* must be 128                                           */
  int32_t rotary_dim;               /* must be 64                                            */
  int32_t compress_ratio;           /* c: power of two, 2..64                                */
  qsa_dtype index_dtype;
  void* q_idx;                      /* OUT [T, Hi, 128] in index_dtype, contiguous           */
  /* main-attention prepare (all ignored when main_qkv is NULL)                              */
  const uint16_t* main_qkv;         /* [T, (2*Hq + 2*Hkv)*128] bf16, layout above            */
  int64_t main_qkv_row_stride;      /* in elements, even                                     */
  int32_t num_q_heads;              /* Hq (1..128)                                           */
  int32_t num_kv_heads;             /* Hkv (1..64)                                           */
  const uint16_t* main_q_norm_weight; /* [128] bf16                                          */
  const uint16_t* main_k_norm_weight; /* [128] bf16                                          */
  float main_eps;                   /* the main q_norm / k_norm epsilon                      */
  uint16_t* main_q;                 /* OUT [T, Hq, 128] bf16, contiguous                     */
  void* main_kv_cache;              /* [pages, Hkv, P, 256] bf16 or e4m3fn, strides below    */
  int64_t main_kv_page_stride;      /* strides in elements; multiples of 16 bytes            */
  int64_t main_kv_head_stride;
  int64_t main_kv_token_stride;     /* >= 256                                                */
  int32_t main_num_pages;
  int32_t main_page_size;           /* P >= 1                                                */
  const int64_t* main_slot_mapping; /* [T] page * P + offset; negative: the row is not stored */
  qsa_dtype main_kv_dtype;          /* BF16 or FP8_E4M3                                      */
  float main_k_scale;               /* FP8_E4M3: stored code = e4m3fn(K / k_scale); > 0      */
  float main_v_scale;               /* FP8_E4M3: stored code = e4m3fn(V / v_scale); > 0      */
} qsa_compress_args;

qsa_status qsa_compress(const qsa_compress_args* args, void* stream);

/* ------------------------------------------------------------------------------------------
 * qsa_index_logits_topk
 *
 * Follows QSAIndexer.forward's selection (qsa_select_paged_decode / qsa_select_paged_prefill /
 * expand_qsa_block_indices) and the packed-buffer contract of QSAIndexer.output_width and
 * packed_output_width (page "vllm.models.qwen4_exp.nvidia.qsa"):
 *   a row at position p sees vis = floor((p+1)/c) compressed blocks; its score for block j is
 *   the sum over the Hi indexer heads of q_idx[row,h,:] . ckv[j,:] (weight-free); it keeps
 *   every block if vis <= budget/c, else the budget/c best (higher score first, an exactly
 *   equal score to the lower block index).  The packed row (W = budget + c - 1 columns + 1):
 *   the kept blocks' tokens g*c..g*c+c-1 in ascending order, then the tail tokens
 *   vis*c..p, then -1 padding, and the number of valid entries in column W.
 * The selected set is EXACT with respect to the float64 score summed in the canonical order
 * (per head a halving sum over the 128 dims, heads added in order): the kernels rank fast
 * float32 scores, certify every block outside a proven error band, and re-score only the
 * band in float64.
 * Decode requests (the leading num_decode_requests, each with decode_query_len rows) and the
 * remaining prefill requests may be mixed in one call.
 * A visible block whose page is out of range scores as an all-zero key.
 * ------------------------------------------------------------------------------------------ */
typedef struct qsa_topk_args {
  int32_t num_tokens;               /* T                                                     */
  int32_t num_requests;             /* R                                                     */
  const int32_t* query_start_loc;   /* [R+1]                                                 */
  const int32_t* seq_lens;          /* [R] (as for qsa_compress)                             */
  int32_t num_decode_requests;      /* leading requests with decode_query_len rows each      */
  int32_t decode_query_len;
  int32_t max_query_len;            /* host upper bound of n_r over all requests             */
  int32_t max_seq_len;              /* host upper bound of seq_lens (sizes the workspace)    */
  const void* q_idx;                /* [T, Hi, 128] index_dtype (qsa_compress's output)      */
  const void* ckv;                  /* [c_pages, c_page_size, 128] index_dtype               */
  const int32_t* c_block_table;
  int32_t c_block_table_stride;
  int32_t c_block_table_width;
  int32_t c_page_size;
  int32_t c_pages;                  /* c_pages * c_page_size < 2^31 (else NOT_SUPPORTED)     */
  int32_t num_index_heads;          /* Hi (1..16)                                            */
  int32_t head_dim;                 /* must be 128                                           */
  int32_t compress_ratio;           /* c (power of two)                                      */
  int32_t budget;                   /* token budget B, a multiple of c                       */
  qsa_dtype index_dtype;
  int32_t* packed;                  /* OUT [T, B + c] int32 (W + 1 columns), row stride below */
  int64_t packed_row_stride;
  qsa_agg index_agg;                /* SUM (0), or RELU_SUM: score = sum_h max(0, q_h . k),
                                       heads in order; RELU_SUM scores every request on the
                                       matrix cores, one head per operand column            */
  int64_t max_logits_bytes;         /* 0: no cap.  Else the rows are scored and selected in
                                       windows of consecutive rows whose logits fit this many
                                       bytes (4 per compressed column, rounded to 64), each
                                       window reusing the workspace: see below              */
} qsa_topk_args;

size_t qsa_index_logits_topk_workspace_size(const qsa_topk_args* args);
qsa_status qsa_index_logits_topk(const qsa_topk_args* args, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Logits memory cap (the pages bound the prefill logits buffer by a size in MB): with
 * max_logits_bytes > 0 the call runs window by window over rows [w*n, (w+1)*n), n =
 * max(1, max_logits_bytes / (4 * ceil(max_seq_len / c / 64) * 64)), and the workspace query
 * sizes everything per-row (logits, band spill) for n rows instead of T.  The result is the
 * same packed buffer, bit for bit.  A row window is also the unit of the split calls below:
 * they return QSA_ERR_NOT_SUPPORTED when the cap makes more than one window. */

/* The two kernels of qsa_index_logits_topk as separate calls, for a caller that times them
 * one by one: qsa_index_logits runs the scoring (fast logits, float32 or, for matrix-core
 * rows, scaled fp16, and per-block key bounds
 * into the workspace), qsa_block_topk the selection and expansion from that workspace.  Run in
 * this order on one stream, with the same arguments and the same, otherwise untouched,
 * workspace, they have exactly the effect of qsa_index_logits_topk.  The workspace contents
 * in between are private to the library. */
qsa_status qsa_index_logits(const qsa_topk_args* args, void* workspace, size_t workspace_bytes,
                            void* stream);
qsa_status qsa_block_topk(const qsa_topk_args* args, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ------------------------------------------------------------------------------------------
 * qsa_compress_index_logits_topk
 *
 * qsa_compress(compress_args) followed by qsa_index_logits_topk(topk_args, workspace) on one
 * stream, as one call: the same outputs, bit for bit (q_idx, the compressed cache, the ring,
 * the packed rows; workspace: qsa_index_logits_topk_workspace_size(topk_args)).  Both argument
 * blocks are validated before anything runs; an invalid one leaves every buffer untouched.
 * Follows QSAIndexer.forward (page "vllm.models.qwen4_exp.nvidia.qsa"), whose decode path runs
 * the indexer prepare and then the paged selection on the same requests.
 *
 * When the step is a batch of one-row requests (num_tokens == num_requests, max_query_len 1
 * in both blocks, the rows' offsets starting at 0) large enough for the wide vector-unit
 * scoring layout, with no main-attention prepare, plain-sum aggregation, no logits window, and
 * both blocks naming the same requests, q_idx, compressed cache and block table, the scoring
 * kernel does the indexer prepare itself and the compress launch is saved
 * (qsa_compress_index_logits_topk_fused returns 1; 0 when the two calls run back to back, -1
 * for invalid arguments).  In that case no request's visible compressed rows may lie in a page
 * that another request's step writes (a group this step completes).
 * qsa_compress_index_logits runs the first part only (the prepare and the scoring), for a
 * caller that times qsa_block_topk separately: followed by qsa_block_topk(topk_args) with the
 * same workspace it has exactly the effect of qsa_compress_index_logits_topk.
 * ------------------------------------------------------------------------------------------ */
qsa_status qsa_compress_index_logits_topk(const qsa_compress_args* compress_args,
                                          const qsa_topk_args* topk_args, void* workspace,
                                          size_t workspace_bytes, void* stream);
qsa_status qsa_compress_index_logits(const qsa_compress_args* compress_args,
                                     const qsa_topk_args* topk_args, void* workspace,
                                     size_t workspace_bytes, void* stream);
int32_t qsa_compress_index_logits_topk_fused(const qsa_compress_args* compress_args,
                                             const qsa_topk_args* topk_args);

/* ------------------------------------------------------------------------------------------
 * qsa_sparse_gqa
 *
 * Follows qsa_sparse_paged_attention ("vllm.models.qwen4_exp.nvidia.ops.qsa") and the body of
 * _qsa_sparse_paged_gqa_splitk_kernel (FP8 KV reader patch page, bf16 branch): for every row
 * and Q head hq (KV head hq / (Hq/Hkv)), attend over entries 0..min(count, W)-1 of the row's
 * packed buffer, where count is its column W; entry t maps to page block_table[req, t / P],
 * slot t % P.  Negative entries, entries whose page column or page is out of range are
 * masked.  Softmax scale = `scale` (0: head_dim^-0.5); a row with no valid entry yields 0.
 * The selection is split into `num_splits` parts per (row, KV head) whose float32 partials are
 * merged by log-sum-exp; the sigmoid of `gate` (if not NULL) multiplies the merged output; the
 * result is written as bf16.  With bf16 K/V and 2..8 splits (forced, or chosen automatically
 * for 128..256 (row, KV head) pairs) the parts are the waves of one workgroup and are merged in
 * it; otherwise each part is a workgroup and a second kernel merges their partials, which then
 * take workspace.
 * KV cache layout: token row of KV head h on page pg starts at
 *     kv_cache + pg*kv_page_stride + h*kv_head_stride + slot*kv_token_stride
 * and holds K in its first head_dim values and V in the next head_dim (the pages' kv_cache
 * [pages, Hkv, P, 2*head_dim], split at head_size after transpose(1, 2)).
 * FP8 main KV (the FP8 KV reader patch page, e4m3 branch): with kv_dtype FP8_E4M3 the cache
 * holds OCP e4m3fn codes (one byte per value, strides in bytes) and static per-tensor scales:
 * K = code * k_scale and V = code * v_scale.  k_scale is applied to the scores and v_scale to
 * the output, never to the cached values.
 * ------------------------------------------------------------------------------------------ */
typedef struct qsa_gqa_args {
  int32_t num_tokens;               /* T                                                     */
  int32_t num_requests;             /* R (rows of block_table)                               */
  int32_t num_q_heads;              /* Hq                                                    */
  int32_t num_kv_heads;             /* Hkv; Hq / Hkv in {1, 2, 4, 8, 16}                     */
  int32_t head_dim;                 /* must be 128                                           */
  const uint16_t* q;                /* [T, Hq, 128] bf16                                     */
  int64_t q_row_stride;
  int64_t q_head_stride;            /* must be 128 (a row's heads contiguous)                */
  const void* kv_cache;             /* bf16 or e4m3fn (kv_dtype), layout above               */
  int64_t kv_page_stride;           /* strides in elements; multiples of 16 bytes            */
  int64_t kv_head_stride;
  int64_t kv_token_stride;
  int32_t num_pages;
  int32_t page_size;                /* P: a multiple of 16                                   */
  const int32_t* block_table;       /* [R, block_table_stride]                               */
  int32_t block_table_stride;
  int32_t block_table_width;        /* valid columns                                         */
  const int32_t* token_to_req;      /* [T]; a request outside [0, R) masks the whole row     */
  const int32_t* packed;            /* [T, W + 1] packed selection buffer                    */
  int64_t packed_row_stride;
  int32_t packed_width;             /* W (selection columns; the count is column W)          */
  const uint16_t* gate;             /* [T, Hq, 128] bf16 or NULL                             */
  int64_t gate_row_stride;
  int64_t gate_head_stride;
  float scale;                      /* 0 -> head_dim^-0.5                                    */
  int32_t num_splits;               /* 0: automatic; >= 1 forces (clamped to the tile count) */
  uint16_t* out;                    /* OUT [T, Hq, 128] bf16, fully overwritten              */
  int64_t out_row_stride;
  int64_t out_head_stride;
  qsa_dtype kv_dtype;               /* BF16 (0) or FP8_E4M3                                  */
  float k_scale;                    /* FP8_E4M3: K = code * k_scale; 0 -> 1; ignored for bf16 */
  float v_scale;                    /* FP8_E4M3: V = code * v_scale; 0 -> 1; ignored for bf16 */
  int32_t row_tiles;                /* 1: row-tiled prefill attention where it applies (bf16
                                       K/V, Hq = 8 Hkv, one split, T >= 2048): 32-row tiles of
                                       one request share each loaded K/V window, every
                                       (row, token) pair a row did not select masked; pays off
                                       when nearby rows select overlapping tokens.  0: off.
                                       Results equal the per-row path within rounding.      */
} qsa_gqa_args;

/* Splits the call will use (after the automatic choice and clamping). */
int32_t qsa_sparse_gqa_num_splits(const qsa_gqa_args* args);
/* 1 if the call runs the separate merge kernel (so that qsa_sparse_gqa_merge below has work), 0
 * if not (one split, or splits merged inside the attention workgroup), -1 for invalid
 * arguments. */
int32_t qsa_sparse_gqa_merge_kernel(const qsa_gqa_args* args);
size_t qsa_sparse_gqa_workspace_size(const qsa_gqa_args* args);
qsa_status qsa_sparse_gqa(const qsa_gqa_args* args, void* workspace, size_t workspace_bytes,
                          void* stream);

/* The two kernels of qsa_sparse_gqa as separate calls (for per-kernel timing):
 * qsa_sparse_gqa_partial computes the split partials (with one split, or splits merged in the
 * workgroup: the gated output itself), qsa_sparse_gqa_merge merges them into the output (a
 * no-op when qsa_sparse_gqa_merge_kernel is 0).  In this order on
 * one stream, with the same arguments and workspace, they have exactly the effect of
 * qsa_sparse_gqa. */
qsa_status qsa_sparse_gqa_partial(const qsa_gqa_args* args, void* workspace,
                                  size_t workspace_bytes, void* stream);
qsa_status qsa_sparse_gqa_merge(const qsa_gqa_args* args, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * qsa_sparse_gqa_noalloc: qsa_sparse_gqa for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, kernels and results as qsa_sparse_gqa with a workspace; the split partials go to a
 * static device array of qsa_sparse_gqa_noalloc_scratch_bytes() bytes (40 MiB) that the library
 * holds on every GPU it runs on until the process ends.  The call allocates and frees nothing.
 * Limits and behaviour:
 *   - a call whose partials need more than that (qsa_sparse_gqa_workspace_size of the same
 *     arguments) returns QSA_ERR_WORKSPACE_TOO_SMALL before any launch; every automatic split
 *     plan fits (its partials stay below 34 MB for any T, Hq, Hkv), a forced num_splits may not;
 *   - every call on one GPU shares that GPU's array: calls that overlap in time on one GPU (two
 *     streams, two threads) race and give undefined results.  Serialise them on one stream.
 *     Nothing needs clearing between calls: each call writes every partial it reads.
 *   - the first call on a device looks up the array's device address (hipGetSymbolAddress);
 *     a failure there returns QSA_ERR_HIP.
 * ------------------------------------------------------------------------------------------ */
qsa_status qsa_sparse_gqa_noalloc(const qsa_gqa_args* args, void* stream);
size_t qsa_sparse_gqa_noalloc_scratch_bytes(void);

/* ------------------------------------------------------------------------------------------
 * Diagnostics: the device arithmetic the bit-exact parts of the path rest on, exposed so a test
 * can compare it with the host's IEEE results.
 *
 * qsa_diag_e4m3_decode: out [512] float (device): out[c] is e4m3fn code c through the hardware
 *   converter of the logits kernels, out[256 + c] through the definitional decoder used by the
 *   float64 re-scoring (OCP e4m3fn, as torch.float8_e4m3fn decodes it).
 * qsa_diag_fp64_sqrt_div: for n doubles in[i] (device), writes out[3i] = sqrt(x),
 *   out[3i+1] = 1/x, out[3i+2] = 1/sqrt(x) (device) -- the operations of the RMSNorm chain,
 *   which must be correctly rounded.
 * ------------------------------------------------------------------------------------------ */
qsa_status qsa_diag_e4m3_decode(float* out, void* stream);
qsa_status qsa_diag_fp64_sqrt_div(const double* in, double* out, int64_t n, void* stream);

/* qsa_diag_read_bandwidth: a read-bandwidth probe with the access patterns of the path's HBM
 * kernels, for measuring practical ceilings.  Reads n_chunks chunks of chunk_bytes (1024, 2048,
 * 3072 or 4096) from src (device, 16-byte aligned): chunk i at i * chunk_bytes (a streaming read)
 * or, with chunk_index (device int32 [n_chunks]) not NULL, at chunk_index[i] * chunk_bytes (a
 * gather; the caller keeps every chunk inside its buffer).  16 bytes per lane, eight chunks per
 * wavefront in flight; the XOR of everything read is folded into *sink (device) so that no load
 * is dead.  Writes nothing else. */
qsa_status qsa_diag_read_bandwidth(const void* src, const int32_t* chunk_index, int64_t n_chunks,
                                   int32_t chunk_bytes, uint32_t* sink, void* stream);

/* ------------------------------------------------------------------------------------------ */
const char* qsa_status_string(qsa_status status);
int32_t qsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H_ */
