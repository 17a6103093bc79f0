// qsa_compress kernels: indexer Q prep, pooling of completed key groups into the compressed-key
// cache, and the raw-key ring update.
//
// Follows QSAIndexer.forward's unfused reference path (page "vllm.models.qwen4_exp.nvidia.qsa")
// and qsa_compress_groups_with_ratio / qsa_store_cache_rows (page
// "vllm.models.qwen4_exp.nvidia.ops.qsa"); optionally, in the same launch, the main-attention
// prepare of the fused qsa_prepare call (Qwen4ExpQSAAttention: main Q/K norm and RoPE, K/V
// written to the main cache).  Both vector layouts follow the canonical float64 chain the
// oracle defines (halving sums, rotation pairs), so every value is bit-identical to it: a
// pooled group owns a wavefront (lane l holds dims 2l and 2l+1; the halving sum folds the upper
// half of the lanes onto the lower half), and the Q and K vectors, which are many at prefill
// sizes, take a 16-lane row each (no cross-lane traffic beyond DPP shifts).
#include "prep_ops.h"

#pragma clang fp contract(off)

namespace qsa {
namespace {

// Waves [0, ceil(T*Hi/4)): indexer Q vectors, four per wave.  Waves [T*Hi, T*Hi + T): the group (if any) completed by
// row (wave - T*Hi), and -- when fuse_ring -- that row's ring write.  Each wave issues every
// load its result needs as early as its addresses are known: the rotation's cos / sin go out
// with (or right after) the positions and land while the norm is computed.
__global__ __launch_bounds__(256) void prep_compress_kernel(CompressParams P) {
  const int lane = threadIdx.x & 63, l = lane & 15;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nq = (int64_t)P.T * P.Hi, nqw = (nq + 3) / 4;
  if (wave < nqw) {
    const int64_t v = 4 * wave + (lane >> 4);
    float y[8];
    int row;
    norm_rope_row(P, v, nq, P.Hi, P.qw, P.eps, lane,
                  [&](int rw, int h) { return P.q_proj + (int64_t)rw * P.q_rs + h * 64; }, y,
                  row);
    if (v < nq) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (P.fp8) {
          reinterpret_cast<uint16_t*>(P.q_idx)[v * 64 + l + 16 * k] =
              (uint16_t)(f32_to_e4m3(y[2 * k]) | (f32_to_e4m3(y[2 * k + 1]) << 8));
        } else {
          reinterpret_cast<uint32_t*>(P.q_idx)[v * 64 + l + 16 * k] =
              bf16_pair(y[2 * k], y[2 * k + 1]);
        }
      }
    }
    return;
  }
  const int64_t row64 = wave - nqw;
  if (row64 >= P.T) {
    // ---- main-attention prepare: waves [0, ceil(T*Hq/4)) of this range normalise and rotate
    // the main Q heads, the next ceil(T*Hkv/4) the K heads, stored with their V heads; four
    // vectors per wave.
    if (!P.main) return;
    int64_t mw = row64 - P.T;
    const int64_t nmq = (int64_t)P.T * P.Hq, nmqw = (nmq + 3) / 4;
    const int64_t nkv = (int64_t)P.T * P.Hkv;
    float y[8];
    int row;
    if (mw < nmqw) {
      const int64_t v = 4 * mw + (lane >> 4);
      // q of head h: pairs 128h .. 128h+63 of the row (its gate follows).
      norm_rope_row(P, v, nmq, P.Hq, P.mqw, P.m_eps, lane,
                    [&](int rw, int h) { return P.mqkv + (int64_t)rw * P.m_rs + 128 * h; }, y,
                    row);
      if (v < nmq) {
#pragma unroll
        for (int k = 0; k < 4; ++k) P.mq[v * 64 + l + 16 * k] = bf16_pair(y[2 * k], y[2 * k + 1]);
      }
      return;
    }
    mw -= nmqw;
    if (mw >= (nkv + 3) / 4) return;
    const int64_t v = 4 * mw + (lane >> 4);
    const int64_t vc = v < nkv ? v : nkv - 1;
    const int hh = (int)(vc % P.Hkv);
    // K head hh: pairs 64 (2Hq + hh) ..; its V head: 64 (2Hq + Hkv + hh) ..
    uint32_t vu[4];
    {
      const uint32_t* vs = P.mqkv + (int64_t)(vc / P.Hkv) * P.m_rs + 64 * ((int64_t)P.Hq * 2 + P.Hkv + hh);
#pragma unroll
      for (int k = 0; k < 4; ++k) vu[k] = vs[l + 16 * k];
    }
    const int64_t slot = P.slots[vc / P.Hkv];
    norm_rope_row(P, v, nkv, P.Hkv, P.mkw, P.m_eps, lane,
                  [&](int rw, int h) {
                    return P.mqkv + (int64_t)rw * P.m_rs + 64 * ((int64_t)P.Hq * 2 + h);
                  },
                  y, row);
    if (v >= nkv || slot < 0 || slot / P.m_P >= P.m_pages) return;
    const int64_t base =
        (slot / P.m_P) * P.m_ps + (int64_t)hh * P.m_hs + (slot % P.m_P) * P.m_ts;  // elements
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t e = base + 2 * (l + 16 * k);  // element of dim pair l + 16k
      if (P.main_fp8) {
        uint16_t* c = reinterpret_cast<uint16_t*>(P.mcache);  // byte pairs
        c[e / 2] = (uint16_t)(scaled_e4m3_sat(y[2 * k], P.k_scale) |
                              (scaled_e4m3_sat(y[2 * k + 1], P.k_scale) << 8));
        c[(e + kHeadDim) / 2] = (uint16_t)(scaled_e4m3_sat(bf16lo(vu[k]), P.v_scale) |
                                           (scaled_e4m3_sat(bf16hi(vu[k]), P.v_scale) << 8));
      } else {
        uint32_t* c = reinterpret_cast<uint32_t*>(P.mcache);  // bf16 pairs
        c[e / 2] = bf16_pair(y[2 * k], y[2 * k + 1]);
        c[(e + kHeadDim) / 2] = vu[k];
      }
    }
    return;
  }
  const int row = (int)row64;
  const ReqInfo ri = wave_find_request(P, row, lane);
  if (ri.r < 0) return;
  const int r = ri.r, q0 = ri.q0, L = ri.L, rp = ri.rp;
  const int start = L - ri.n;
  if (start < 0) return;
  const int p = start + (row - q0);
  const bool ring_ok = rp >= 0 && rp < P.ring_pages;

  if ((p + 1) % P.c == 0) {
    const int g = (p + 1) / P.c - 1;
    float y0, y1;
    int page;
    compress_group(P, r, q0, start, rp, ring_ok, g, lane, y0, y1, page);
    if (page >= 0 && page < P.c_pages)
      store_index_pair(P, P.ckv, (int64_t)page * P.Pc + (g % P.Pc), lane, y0, y1);
  }
  if (P.fuse_ring) ring_store_row(P, row, r, p, L, lane);
}

// Separate ring update, launched after prep_compress_kernel when the step's writes could alias
// slots that its reads still need (long prefill chunks).
__global__ __launch_bounds__(256) void ring_store_kernel(CompressParams P) {
  __shared__ int32_t qsl_s[kQslCap];
  const int32_t* qsl = stage_qsl(P.qsl, P.R, qsl_s);
  const int lane = threadIdx.x & 63;
  const int64_t row64 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  if (row64 >= P.T) return;
  const int row = (int)row64;
  const int r = find_request(qsl, P.R, row);
  if (r < 0) return;
  const int q0 = qsl[r], n = qsl[r + 1] - q0, L = P.seq_lens[r];
  if (L - n < 0) return;
  ring_store_row(P, row, r, L - n + (row - q0), L, lane);
}

}  // namespace

CompressParams compress_params(const qsa_compress_args& a) {
  CompressParams P{};
  P.T = a.num_tokens;
  P.R = a.num_requests;
  P.Hi = a.num_index_heads;
  P.c = a.compress_ratio;
  P.S = a.ring_size;
  P.ring_pages = a.ring_pages;
  P.Pc = a.c_page_size;
  P.c_pages = a.c_pages;
  P.cbt_stride = a.c_block_table_stride;
  P.cbt_width = a.c_block_table_width;
  P.max_pos = a.max_position;
  P.mrope = a.mrope_section[0] || a.mrope_section[1] || a.mrope_section[2];
  P.sec_h = a.mrope_section[1];
  P.sec_w = a.mrope_section[2];
  P.fp8 = a.index_dtype == QSA_DTYPE_FP8_E4M3;
  // Reads of the ring reach back at most c-1 tokens before the step, writes cover its last
  // min(S, n) tokens: they cannot share a slot when n + c - 2 < S.
  P.fuse_ring = (int64_t)a.max_query_len + a.compress_ratio - 2 < a.ring_size;
  P.qsl = a.query_start_loc;
  P.seq_lens = a.seq_lens;
  P.q_proj = reinterpret_cast<const uint32_t*>(a.q_proj);
  P.q_rs = a.q_proj_row_stride / 2;
  P.k_proj = reinterpret_cast<const uint32_t*>(a.k_proj);
  P.k_rs = a.k_proj_row_stride / 2;
  P.pos = a.positions;
  P.cos_sin = a.cos_sin;
  P.qw = a.q_norm_weight;
  P.kw = a.k_norm_weight;
  P.eps = (double)a.eps;
  P.ring = reinterpret_cast<uint32_t*>(a.ring);
  P.ring_pos = a.ring_pos;
  P.ring_page = a.ring_page;
  P.ckv = a.ckv;
  P.cbt = a.c_block_table;
  P.q_idx = a.q_idx;
  P.main = a.main_qkv != nullptr;
  if (P.main) {
    P.main_fp8 = a.main_kv_dtype == QSA_DTYPE_FP8_E4M3;
    P.Hq = a.num_q_heads;
    P.Hkv = a.num_kv_heads;
    P.m_pages = a.main_num_pages;
    P.m_P = a.main_page_size;
    P.mqkv = reinterpret_cast<const uint32_t*>(a.main_qkv);
    P.m_rs = a.main_qkv_row_stride / 2;
    P.mqw = a.main_q_norm_weight;
    P.mkw = a.main_k_norm_weight;
    P.m_eps = (double)a.main_eps;
    P.mq = reinterpret_cast<uint32_t*>(a.main_q);
    P.mcache = a.main_kv_cache;
    P.m_ps = a.main_kv_page_stride;
    P.m_hs = a.main_kv_head_stride;
    P.m_ts = a.main_kv_token_stride;
    P.slots = a.main_slot_mapping;
    P.k_scale = a.main_k_scale;
    P.v_scale = a.main_v_scale;
  }
  return P;
}

hipError_t launch_compress(const qsa_compress_args& a, hipStream_t s) {
  const CompressParams P = compress_params(a);
  const int64_t waves = ((int64_t)P.T * P.Hi + 3) / 4 + P.T +
                        (P.main ? ((int64_t)P.T * P.Hq + 3) / 4 + ((int64_t)P.T * P.Hkv + 3) / 4
                                : 0);
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL(prep_compress_kernel, dim3((unsigned)blocks), dim3(256), 0, s, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || P.fuse_ring) return e;
  hipLaunchKernelGGL(ring_store_kernel, dim3((unsigned)((P.T + 3) / 4)), dim3(256), 0, s, P);
  return hipGetLastError();
}

}  // namespace qsa
