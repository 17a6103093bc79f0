// Block top-k over the indexer logits and expansion of the kept blocks into the packed
// selection buffer.  Follows QSAIndexer.forward's selection (qsa_select_paged_decode /
// qsa_select_paged_prefill / expand_qsa_block_indices) and the packed-buffer contract of
// QSAIndexer.output_width / packed_output_width (page "vllm.models.qwen4_exp.nvidia.qsa").
//
// Exactness.  The selection must equal the one defined on the float64 score summed in the
// canonical order.  The logits kernel computes a fast float32 score with the heads folded into Q
// (sum_h q[h] . k = (sum_h q[h]) . k).  With kappa = max |k| over the request's keys and
// A = sum_{h,d} |q[h,d]|, the fold and the float32 dot differ from the exact score by at most
// gamma_{Hi+128} * kappa * A (gamma_n = n u / (1 - n u), u = 2^-24), and the canonical float64
// score by a further ~1e-13 relative; E below is twice that.  If T is the kb-th largest fast
// score, a block with fast score > T + 2E is certainly kept, one below T - 2E certainly dropped,
// and only the band in between is re-scored in float64 in the canonical order and ranked by
// (score desc, block asc).
#include <type_traits>

#include "select.h"

namespace qsa {
namespace {
// Order-preserving map of float32 onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fval(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <int NT, typename T>
__device__ __forceinline__ T block_sum(T v, T* scratch) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  __syncthreads();
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  T s = 0;
  for (int i = 0; i < NT / 64; ++i) s += scratch[i];
  return s;
}

// Value of lane l + N of the same row of 16 lanes (DPP row_shl); lanes past the row's end get
// zero (bound_ctrl, so no old value has to be set up).  Only the lanes whose partner exists
// use the result.
template <int N>
__device__ __forceinline__ double row_down(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)u, 0x100 + N, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), 0x100 + N, 0xF, 0xF, true);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
template <int N>
__device__ __forceinline__ float row_down(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x100 + N, 0xF, 0xF, true));
}

// Key values of the 16-lane group's lane l: dim pairs i = l, l+16, l+32, l+48 (dims 2i, 2i+1),
// exact as floats; zero for an out-of-range row (j < 0, a column past cw, or its page outside
// the cache).  `cbt_row` is the request's block-table row (LDS copy or global), cw its width.
__device__ __forceinline__ void key_pairs16(const SelectParams& P, const int32_t* cbt_row,
                                           int cw, int j, int l, float (&k)[8]) {
  int64_t off = -1;
  if (j >= 0) {
    const int col = j / P.Pc;
    const int page = col < cw ? cbt_row[col] : -1;
    if (page >= 0 && page < P.c_pages) off = ((int64_t)page * P.Pc + (j - col * P.Pc)) * kHeadDim;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = l + 16 * q;
    float k0 = 0.0f, k1 = 0.0f;
    if (off >= 0) {
      if (P.fp8) {
        const uint32_t u = reinterpret_cast<const uint16_t*>(P.ckv)[off / 2 + i];
        // The hardware converter (OCP e4m3fn on gfx950) equals the definition on every code.
        const auto f = __builtin_amdgcn_cvt_pk_f32_fp8(u, false);
        k0 = f[0];
        k1 = f[1];
      } else {
        const uint32_t u = reinterpret_cast<const uint32_t*>(P.ckv)[off / 2 + i];
        k0 = bf16lo(u);
        k1 = bf16hi(u);
      }
    }
    k[2 * q] = k0;
    k[2 * q + 1] = k1;
  }
}

// Canonical float64 score of compressed row j against the row's Q, computed by a group of 16
// lanes (l = lane % 16).  Per head the 128 exact products are summed by halving: pairs
// (2i, 2i+1) give v_i; then v_i += v_{i+32} for i < 32, += v_{i+16} for i < 16, ..., += v_{i+1}
// for i < 1.  Lane l holds v_l, v_{l+16}, v_{l+32}, v_{l+48}, so the first two halvings are
// in-lane and the last four take the partner 8, 4, 2, 1 lanes up.  The heads are then added in
// order (RELU, the ReLU-sum: each head's sum clamped at 0 first).  Q is read from LDS as
// float64 (Q64: the row's heads fit) or as float32 converted here; both hold the same values.
// The result is valid in lane l = 0.
template <bool Q64, bool RELU>
__device__ double canonical_score16(const SelectParams& P, const float* qrow,
                                    const int32_t* cbt_row, int cw, int j, int l) {
  float k[8];
  key_pairs16(P, cbt_row, cw, j, l, k);
  double kd[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) kd[t] = (double)k[t];
  double s = 0.0;
  for (int h = 0; h < P.Hi; ++h) {
    double v[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = l + 16 * t;
      double q0, q1;
      if constexpr (Q64) {
        const double2 qq =
            *reinterpret_cast<const double2*>(reinterpret_cast<const double*>(qrow) +
                                              h * kHeadDim + 2 * i);
        q0 = qq.x;
        q1 = qq.y;
      } else {
        const float2 qq = *reinterpret_cast<const float2*>(qrow + h * kHeadDim + 2 * i);
        q0 = (double)qq.x;
        q1 = (double)qq.y;
      }
      v[t] = fma(q0, kd[2 * t], q1 * kd[2 * t + 1]);  // both products exact: p0 + p1 rounded
    }
    double x = (v[0] + v[2]) + (v[1] + v[3]);
    x = x + row_down<8>(x);
    x = x + row_down<4>(x);
    x = x + row_down<2>(x);
    x = x + row_down<1>(x);
    if constexpr (RELU) x = x > 0.0 ? x : 0.0;  // ReLU-sum: max(0, head product)
    s = (h == 0) ? x : s + x;
  }
  return s;
}

// Head-folded float32 scores (sum_h q_h) . k of band entries, by groups of 16 lanes: lane l
// takes dims 8l .. 8l+7 (one 16-byte bf16 or 8-byte fp8 load), a group handles entries b, b +
// groups, ... and the loads of kFoldBatch entries are in flight together.  The summation order
// is free: the error bound of the VALU logits holds for any order.  Writes out[b] (lane 0 of
// the group); rows out of range (column past cw, page outside the cache) score 0.
constexpr int kFoldBatch = 4;
__device__ __forceinline__ void folded_scores16(const SelectParams& P, const float* qfold,
                                                const int32_t* cbt_row, int cw,
                                                const int32_t* band, int nb, int groups,
                                                int grp, int l, double* out) {
  float qf[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) qf[d] = qfold[8 * l + d];
  for (int base = 0; base < nb; base += kFoldBatch * groups) {
    uint4 raw[kFoldBatch];
#pragma unroll
    for (int u = 0; u < kFoldBatch; ++u) {
      const int b = base + u * groups + grp;
      raw[u] = make_uint4(0u, 0u, 0u, 0u);
      if (b < nb) {
        const int j = band[b];
        const int col = j / P.Pc;
        const int page = col < cw ? cbt_row[col] : -1;
        if (page >= 0 && page < P.c_pages) {
          const int64_t row = (int64_t)page * P.Pc + (j - col * P.Pc);
          if (P.fp8) {
            const uint2 v = *reinterpret_cast<const uint2*>(
                reinterpret_cast<const uint8_t*>(P.ckv) + row * kHeadDim + 8 * l);
            raw[u].x = v.x;
            raw[u].y = v.y;
          } else {
            raw[u] = *reinterpret_cast<const uint4*>(
                reinterpret_cast<const uint16_t*>(P.ckv) + row * kHeadDim + 8 * l);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kFoldBatch; ++u) {
      float k[8];
      if (P.fp8) {
        const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(raw[u].x, false);
        const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(raw[u].x, true);
        const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(raw[u].y, false);
        const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(raw[u].y, true);
        k[0] = a[0]; k[1] = a[1]; k[2] = b[0]; k[3] = b[1];
        k[4] = c[0]; k[5] = c[1]; k[6] = d[0]; k[7] = d[1];
      } else {
        const uint32_t w4[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          k[2 * d] = bf16lo(w4[d]);
          k[2 * d + 1] = bf16hi(w4[d]);
        }
      }
      float x = 0.0f;
#pragma unroll
      for (int d = 0; d < 8; ++d) x += qf[d] * k[d];
      x = x + row_down<8>(x);
      x = x + row_down<4>(x);
      x = x + row_down<2>(x);
      x = x + row_down<1>(x);
      const int b = base + u * groups + grp;
      if (l == 0 && b < nb) out[b] = x;
    }
  }
}

// Top-k kernel configurations: NT threads holding E scores each; the threshold's radix select
// over a float32 row takes PASSES passes of RB-bit digits over the top RB*PASSES bits of the
// order-preserving key (the rest stay unresolved: the threshold lies in one bin's value
// interval, which the band absorbs; a matrix-core row, fp16, is resolved exactly in two 8-bit
// passes of its own); bands of up to BAND entries and block-table rows of up to CBT columns
// live in LDS; the first PF scores of a row are loaded
// before the request lookup (the rest once the visible range is known).  The decode
// configurations spend LDS on few, fast rows; the prefill one (many rows, eight sharing a CU)
// keeps its LDS small and loads after the lookup, when the row's width and type are known.
template <int NT_, int E_, int RB_, int PASSES_, int BAND_, int CBT_, int PF_, int WPE_ = 1>
struct TopkCfg {
  static constexpr int NT = NT_, E = E_, RB = RB_, PASSES = PASSES_, BAND = BAND_, CBT = CBT_;
  static constexpr int PF = PF_;
  static constexpr int WPE = WPE_;  // waves per SIMD the registers must allow (1: no bound)
};
using TopkDecode8 = TopkCfg<512, 8, 12, 2, 1024, 2048, 8192>;
using TopkDecode16 = TopkCfg<512, 16, 12, 2, 1024, 2048, 8192>;
using TopkDecode32 = TopkCfg<512, 32, 12, 2, 1024, 2048, 8192>;
using TopkDecode1k = TopkCfg<1024, 32, 12, 2, 1024, 2048, 8192>;
using TopkPrefill = TopkCfg<256, 16, 8, 3, 256, 512, 0, 8>;
constexpr int kTopkPrefillMinRows = 1024;  // rows in the call from which TopkPrefill is used

// Inclusive prefix sum over the 64 lanes of a wavefront: shifts within rows of 16, then the
// row totals broadcast to the later rows (DPP, no LDS round trips).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return v;
}


// float32 thresholds that are conservative for the float64 ones: x > up(t) implies x > t, and
// x < down(t) implies x < t.
__device__ __forceinline__ float next_up_f32(float f) {  // f finite
  if (f == 0.0f) return __uint_as_float(1u);
  const uint32_t u = __float_as_uint(f);
  return __uint_as_float(f > 0.0f ? u + 1u : u - 1u);
}
__device__ __forceinline__ float round_up_f32(double t) {
  const float f = (float)t;
  return (double)f >= t ? f : next_up_f32(f);
}
__device__ __forceinline__ float round_down_f32(double t) {
  const float f = (float)t;
  return (double)f <= t ? f : -next_up_f32(-f);
}

// One workgroup of NT threads per row; thread t holds the fast scores of blocks
// t*E .. t*E+E-1 in registers for the whole selection (blocks past the visible range as -inf,
// which no threshold below admits).
template <typename C>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::WPE)))
void topk_kernel(SelectParams P) {
  constexpr int NT = C::NT, E = C::E;
  constexpr int kRadixBits = C::RB, kRadixBins = 1 << C::RB, kBandCap = C::BAND;
  constexpr int kTopkCbtCap = C::CBT;
  constexpr uint32_t kLowMask = (1u << (32 - C::RB * C::PASSES)) - 1u;  // unresolved bits
  static_assert(32 % E == 0 || E == 32, "a thread's blocks share one word of the mask");
  static_assert(kRadixBins >= NT, "every thread scans at least one bin");
  constexpr int kWaves = NT / 64, kPB = kRadixBins / NT;  // bins per thread in the scans
  extern __shared__ uint32_t sel_mask[];  // [ceil(cols / 32)] band-selected blocks
  __shared__ __attribute__((aligned(16))) int hist[2][kRadixBins];
  __shared__ int s_int[8];
  __shared__ int s_wave[kWaves];
  __shared__ double s_dbl[kWaves];
  __shared__ float s_flt[kWaves];
  // The row's Q: as float64 when its heads fit (Hi <= 8), else as float32.
  __shared__ __attribute__((aligned(16))) float qrow[16 * kHeadDim];
  __shared__ float qfold[kHeadDim];
  __shared__ int32_t band_idx_s[kBandCap];
  __shared__ int32_t band2_idx_s[kBandCap];
  __shared__ double band_score_s[kBandCap];
  __shared__ int32_t cbt_s[kTopkCbtCap];

  // The call's rows run in windows (one without a logits cap); the per-row workspace arrays
  // hold the window's rows.
  const int row = P.row_lo + blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t wrow = blockIdx.x;  // row - row_lo
  const int W = P.budget + P.c - 1, kb = P.budget / P.c;
  int32_t* out = P.packed + (int64_t)row * P.p_rs;
  // Barriers: LDS-only ones wait for the wave's LDS operations and nothing else (the fence of
  // __syncthreads would also wait for every global load in flight, such as the prefetches
  // below); the full one publishes global writes (bands too large for LDS).
  auto lds_barrier = [] {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // ---- loads that need only the row, issued first: this thread's fast scores (the row is
  // padded to col_stride), its share of the Q row, and the request metadata for the lookup.
  // Scores past C::PF are loaded once the row's visible range is known (a short request of a
  // call with long ones would otherwise read a long row it does not use).
  const float* lg = P.logits + wrow * P.col_stride;
  const int jb = tid * E;
  const int pf_end = min(P.col_stride, C::PF);
  float sc[E];
#pragma unroll
  for (int i = 0; i < E; i += 4) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (jb + i < pf_end) v = *reinterpret_cast<const float4*>(lg + jb + i);
    sc[i] = v.x;
    sc[i + 1] = v.y;
    sc[i + 2] = v.z;
    sc[i + 3] = v.w;
  }
  constexpr int kQPer = (16 * kHeadDim + NT - 1) / NT;
  uint32_t qv[kQPer];  // raw bf16 / e4m3 codes
#pragma unroll
  for (int k = 0; k < kQPer; ++k) {
    const int i = min(tid + k * NT, P.Hi * kHeadDim - 1);
    const int64_t idx = (int64_t)row * P.Hi * kHeadDim + i;
    qv[k] = P.fp8 ? (uint32_t)reinterpret_cast<const uint8_t*>(P.q_idx)[idx]
                  : (uint32_t)reinterpret_cast<const uint16_t*>(P.q_idx)[idx];
  }
  // The row's request: the thread whose interval [qsl[i], qsl[i+1]) holds the row publishes
  // the request and its metadata (loaded with the interval, not after it).
  bool mine = false;
  for (int i = tid; i < P.R; i += NT) {
    const int a = P.qsl[i], b = P.qsl[i + 1], Li = P.seq_lens[i];
    if (a <= row && row < b) {
      s_int[0] = i;
      s_int[1] = a;
      s_int[2] = b - a;
      s_int[3] = Li;
      mine = true;
    }
  }
  {
    int4* h4 = reinterpret_cast<int4*>(&hist[0][0]);
    for (int i = tid; i < 2 * kRadixBins / 4; i += NT) h4[i] = make_int4(0, 0, 0, 0);
  }
  // The request's values are the same for every thread: read into scalar registers, so that
  // the arithmetic on them below runs on the scalar unit.
  const int any_mine = __builtin_amdgcn_readfirstlane(__syncthreads_or(mine));
  int p = -1, L = 0, n_req = 0, r = -1;
  if (any_mine) {
    r = __builtin_amdgcn_readfirstlane(s_int[0]);
    n_req = __builtin_amdgcn_readfirstlane(s_int[2]);
    L = __builtin_amdgcn_readfirstlane(s_int[3]);
    if (L - n_req >= 0) p = L - n_req + (row - __builtin_amdgcn_readfirstlane(s_int[1]));
  }
  if (p < 0) {  // inert row: no entries, count 0
    for (int col = tid; col <= W; col += NT) out[col] = col < W ? -1 : 0;
    return;
  }
  // seq_lens beyond the max_seq_len the workspace was sized for would overrun the logits
  // row: such rows are clamped (their selection is then undefined but stays in bounds).
  const int vis = min((p + 1) >> P.c_log2, P.cols);  // c is a power of two
  const int tail = min(p + 1 - vis * P.c, P.c - 1);
  if (vis <= kb) {  // every visible block: tokens 0..vis*c+tail-1
    const int cnt = vis * P.c + tail;
    for (int col = tid; col <= W; col += NT) out[col] = col < cnt ? col : (col < W ? -1 : cnt);
    return;
  }
  // Loads that need the request, in flight during the radix passes: max |k| of its 128-key
  // blocks (for the error bound) and its block-table row (for the band's key rows).
  float km = 0.0f;
  {
    const int nt = min(P.key_blocks, (min(L >> P.c_log2, P.cols) + 127) / 128);
    for (int t = tid; t < nt; t += NT) km = fmaxf(km, P.kmax[(int64_t)r * P.key_blocks + t]);
  }
  const int cw = min(P.cbt_width, (vis + P.Pc - 1) / P.Pc);
  const bool cbt_in_lds = cw <= kTopkCbtCap;
  constexpr int kCbtPer = (kTopkCbtCap + NT - 1) / NT;
  int cbt_v[kCbtPer];
#pragma unroll
  for (int k = 0; k < kCbtPer; ++k) {
    const int c = tid + k * NT;
    cbt_v[k] = (cbt_in_lds && c < cw) ? P.cbt[(int64_t)r * P.cbt_stride + c] : -1;
  }
  // Rows scored on the matrix cores hold fp16 logits scaled by 2^-lexp (in the row's
  // float32-sized stride).
  const bool f16_row = n_req > P.mfma_min_rows;  // block-uniform
  double qa = 0.0;
  const bool q64 = P.Hi <= 8;
#pragma unroll
  for (int k = 0; k < kQPer; ++k) {
    const int i = tid + k * NT;
    if (i < P.Hi * kHeadDim) {
      const float f = P.fp8 ? e4m3_to_f32_exact(qv[k]) : bf16_to_f32((uint16_t)qv[k]);
      if (q64) reinterpret_cast<double*>(qrow)[i] = (double)f;
      else qrow[i] = f;
      qa += fabs((double)f);
    }
  }
  const int mask_words = (vis + 31) >> 5;
  for (int i = tid; i < mask_words; i += NT) sel_mask[i] = 0u;

  // Shared steps of both row types.  The error-bound inputs are reduced per wave during the
  // last radix pass (published by that pass's barrier).
  auto publish_bound_inputs = [&] {
    const float kmw = wave_max(km);
    double qaw = qa;
#pragma unroll
    for (int mm = 32; mm >= 1; mm >>= 1) qaw += shfl_xor_f64(qaw, mm);
    if (lane == 0) {
      s_flt[w] = kmw;
      s_dbl[w] = qaw;
    }
  };
  double E_f = 0.0, Ebound = 0.0;
  auto bounds = [&] {
    if (cbt_in_lds) {
#pragma unroll
      for (int k = 0; k < kCbtPer; ++k) {
        const int c = tid + k * NT;
        if (c < cw) cbt_s[c] = cbt_v[k];
      }
    }
    double kappa = 0.0, A = 0.0;
    for (int i = 0; i < kWaves; ++i) {
      kappa = fmax(kappa, (double)s_flt[i]);
      A += s_dbl[i];
    }
    // Bounds of the head-folded float32 score (the VALU logits, and the second level below)
    // and of the matrix-core score (topk_bound_factors).
    E_f = P.e_fold * kappa * A + 1e-30;
    Ebound = f16_row ? P.e_mfma * kappa * A + 1e-30 : E_f;
  };
  // Certainly kept above hi, certainly dropped below lo; float32 forms widen the band only.
  // A score b stands for canonical scores in [b - d(b), b + d(b)] with d(b) = Ebound (float32
  // rows) or, in the scaled units of a matrix-core row, Ebound 2^-erow + 2^-14 + r |b|
  // (rounding to nearest fp16 moves a value by at most 2^-11 of the result; r adds a margin).
  // Both ends increase with b, so the kb-th largest canonical
  // score lies in [T_lo - d(T_lo), T_hi + d(T_hi)]; a block is certainly kept if b - d(b)
  // exceeds the upper end and certainly dropped if b + d(b) is below the lower end.  hi and lo
  // solve those two conditions for b.
  uint32_t keepbits = 0, bandbits = 0;
  if (f16_row) {
    // ---- matrix-core rows: the row's scores are fp16 values h (score h * 2^erow), worked on
    // in these scaled units.  The 16-bit order-preserving keys of a pair of scores share a word
    // (score 2m in the low half, 2m + 1 in the high half), and two passes of 8-bit digits
    // resolve the kb-th largest key exactly, so the threshold is one fp16 value T.
    static_assert(E % 8 == 0, "a thread's fp16 scores are whole 16-byte words");
    constexpr int E2 = E / 2;
    uint32_t rw[E2], kp[E2];
    const int erow = P.lexp[wrow];
    const uint16_t* lb = reinterpret_cast<const uint16_t*>(lg);
#pragma unroll
    for (int i = 0; i < E; i += 8) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (jb + i < vis) v = *reinterpret_cast<const uint4*>(lb + jb + i);
      rw[i / 2] = v.x;
      rw[i / 2 + 1] = v.y;
      rw[i / 2 + 2] = v.z;
      rw[i / 2 + 3] = v.w;
    }
    const int nv = min(max(vis - jb, 0), E);  // this thread's visible scores: i < nv
    // Per half: sign clear -> b | 0x8000, sign set -> ~b (as fkey on float32).
#pragma unroll
    for (int m = 0; m < E2; ++m) {
      const uint32_t sgn = (rw[m] >> 15) & 0x00010001u;
      kp[m] = rw[m] ^ 0x80008000u ^ (sgn * 0x7FFFu);
    }
    // One 256-bin pass: thread t < 256 owns bin 255 - t, a workgroup prefix sum gives the count
    // above each bin; returns the bin holding the krem-th largest and the rank within it.
    auto scan256 = [&](const int* h, int& kr) {
      const int S = tid < 256 ? h[255 - tid] : 0;
      const int incl = wave_incl_scan(S);
      if (lane == 63) s_wave[w] = incl;
      lds_barrier();
      int above = incl - S;
      for (int i = 0; i < w; ++i) above += s_wave[i];
      if (above < kr && kr <= above + S) {
        s_int[4] = 255 - tid;
        s_int[5] = kr - above;
      }
      lds_barrier();
      kr = __builtin_amdgcn_readfirstlane(s_int[5]);
      return __builtin_amdgcn_readfirstlane(s_int[4]);
    };
    int krem = kb;
#pragma unroll
    for (int m = 0; m < E2; ++m) {
      if (2 * m < nv) atomicAdd(&hist[0][(kp[m] >> 8) & 0xFFu], 1);
      if (2 * m + 1 < nv) atomicAdd(&hist[0][kp[m] >> 24], 1);
    }
    lds_barrier();
    const uint32_t d0 = (uint32_t)scan256(hist[0], krem);
#pragma unroll
    for (int m = 0; m < E2; ++m) {
      if (2 * m < nv && ((kp[m] >> 8) & 0xFFu) == d0) atomicAdd(&hist[1][kp[m] & 0xFFu], 1);
      if (2 * m + 1 < nv && (kp[m] >> 24) == d0) atomicAdd(&hist[1][(kp[m] >> 16) & 0xFFu], 1);
    }
    publish_bound_inputs();
    lds_barrier();
    const uint32_t key16 = (d0 << 8) | (uint32_t)scan256(hist[1], krem);
    const uint32_t tb = (key16 & 0x8000u) ? (key16 ^ 0x8000u) : (key16 ^ 0xFFFFu);
    auto f16f = [](uint32_t bits) {
      return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
    };
    const double T = (double)f16f(tb);  // the kb-th largest fast score, scaled
    bounds();
    // A stored value h stands for fast scores within 2^-11 |h| of it (rounding to nearest; a
    // subnormal one within 2^-14, however the conversions treat subnormals), and the fast
    // score for canonical scores within Ebound, which is 2^-erow of it in these units.
    constexpr double rr = 0x1p-11 * (1.0 + 0x1p-20);
    // x / (1 -+ rr) as products with the rounded reciprocals (within 2^-52 of the quotients,
    // far inside the 2^-40 widening below).
    constexpr double kInvLo = 1.0 / (1.0 - rr), kInvHi = 1.0 / (1.0 + rr);
    const double Es = __builtin_amdgcn_ldexp(Ebound, -erow) + 0x1p-14;
    const double x = T + rr * fabs(T) + 2.0 * Es;   // b - r|b| must exceed x
    const double y = T - rr * fabs(T) - 2.0 * Es;   // b + r|b| must reach y
    const double bh = x * (x >= 0.0 ? kInvLo : kInvHi);
    const double bl = y * (y >= 0.0 ? kInvHi : kInvLo);
    const float hi = round_up_f32(bh + fabs(bh) * 0x1p-40 + 1e-30);
    const float lo = round_down_f32(bl - fabs(bl) * 0x1p-40 - 1e-30);
    // ---- classify (invisible scores are neither kept nor in the band)
#pragma unroll
    for (int m = 0; m < E2; ++m) {
      const float f0 = f16f(rw[m] & 0xFFFFu), f1 = f16f(rw[m] >> 16);
      const bool v0 = 2 * m < nv, v1 = 2 * m + 1 < nv;
      keepbits |= (v0 && f0 > hi ? 1u : 0u) << (2 * m);
      keepbits |= (v1 && f1 > hi ? 1u : 0u) << (2 * m + 1);
      bandbits |= (v0 && f0 <= hi && f0 >= lo ? 1u : 0u) << (2 * m);
      bandbits |= (v1 && f1 <= hi && f1 >= lo ? 1u : 0u) << (2 * m + 1);
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; i += 4) {  // the rest of the visible scores
      if (jb + i >= pf_end && jb + i < vis) {
        const float4 v = *reinterpret_cast<const float4*>(lg + jb + i);
        sc[i] = v.x;
        sc[i + 1] = v.y;
        sc[i + 2] = v.z;
        sc[i + 3] = v.w;
      }
    }
    uint32_t key[E];  // order-preserving keys of the fast scores
#pragma unroll
    for (int i = 0; i < E; ++i) {
      sc[i] = jb + i < vis ? sc[i] : -__builtin_inff();
      key[i] = fkey(sc[i]);
    }

    // ---- radix select.  Thread t reads the counts of bins (bins-1) - t*kPB - i (i < kPB):
    // lower threads own higher bins, so a workgroup prefix sum gives the count above each bin.
    // Only visible blocks are counted (the -inf entries of a short row would all add to one
    // bin, and its LDS atomics would serialise).  Histograms alternate between two buffers; a
    // pass clears the one the next-but-one uses.
    uint32_t prefix = 0, pmask = 0;
    int krem = kb;
#pragma unroll
    for (int pass = 0; pass < C::PASSES; ++pass) {
      const int shift = 32 - kRadixBits * (pass + 1);
      int* h = hist[pass & 1];
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const uint32_t u = key[i];
        if (jb + i < vis && (u & pmask) == prefix)
          atomicAdd(&h[(u >> shift) & (kRadixBins - 1)], 1);
      }
      if (pass >= 1 && pass + 1 < C::PASSES) {  // the buffer of pass + 1 was read by pass - 1
        for (int i = tid; i < kRadixBins; i += NT) hist[(pass + 1) & 1][i] = 0;
      }
      if (pass == C::PASSES - 1) publish_bound_inputs();
      lds_barrier();
      int c[kPB], S = 0;
      const int b0 = kRadixBins - (tid + 1) * kPB;  // c[i] = count of bin b0 + kPB - 1 - i
#pragma unroll
      for (int i = 0; i < kPB; ++i) {
        c[i] = h[b0 + kPB - 1 - i];
        S += c[i];
      }
      const int incl = wave_incl_scan(S);
      if (lane == 63) s_wave[w] = incl;
      lds_barrier();
      int above = incl - S;
      for (int i = 0; i < w; ++i) above += s_wave[i];
      if (above < krem && krem <= above + S) {
#pragma unroll
        for (int i = 0; i < kPB; ++i) {
          if (above < krem && krem <= above + c[i]) {
            s_int[4] = b0 + kPB - 1 - i;
            s_int[5] = krem - above;
          }
          above += c[i];
        }
      }
      lds_barrier();
      prefix |= (uint32_t)__builtin_amdgcn_readfirstlane(s_int[4]) << shift;
      pmask |= (uint32_t)(kRadixBins - 1) << shift;
      krem = __builtin_amdgcn_readfirstlane(s_int[5]);
    }
    // The kb-th largest fast score lies in [T_lo, T_hi], the values of the keys with this
    // prefix.
    const double T_lo = (double)fval(prefix), T_hi = (double)fval(prefix | kLowMask);
    bounds();
    const float hi = round_up_f32(T_hi + 2.0 * Ebound);
    const float lo = round_down_f32(T_lo - 2.0 * Ebound);
    // ---- classify
#pragma unroll
    for (int i = 0; i < E; ++i) {
      keepbits |= (sc[i] > hi ? 1u : 0u) << i;
      bandbits |= (sc[i] <= hi && sc[i] >= lo ? 1u : 0u) << i;
    }
  }
  const bool mfma_row = f16_row;
  const int32_t* cbt_row = cbt_in_lds ? cbt_s : P.cbt + (int64_t)r * P.cbt_stride;

  // ---- collect the band in block order: one workgroup scan of the per-thread counts (band
  // entries in the low half, certain keeps in the high half of a packed int).
  const int my_cnt = __builtin_popcount(bandbits) | (__builtin_popcount(keepbits) << 16);
  const int cl_incl = wave_incl_scan(my_cnt);
  if (lane == 63) s_wave[w] = cl_incl;
  if (tid == 0) s_int[6] = 0;  // the second level's counter, read after later barriers
  lds_barrier();
  int cl_off = cl_incl - my_cnt, tot = 0;
  for (int i = 0; i < kWaves; ++i) {
    cl_off += i < w ? s_wave[i] : 0;
    tot += s_wave[i];
  }
  tot = __builtin_amdgcn_readfirstlane(tot);  // the same in every thread
  int need = kb - (tot >> 16);
  int nb = tot & 0xFFFF;
  const bool in_lds = nb <= kBandCap;
  int32_t* bidx = in_lds ? band_idx_s : P.band_idx + wrow * P.col_stride;
  {
    int o = cl_off & 0xFFFF;
    for (uint32_t bits = bandbits; bits; bits &= bits - 1) bidx[o++] = jb + __builtin_ctz(bits);
  }
  if (in_lds) lds_barrier(); else __syncthreads();
  double* bscore = in_lds ? band_score_s : P.band_score + wrow * P.col_stride;
  const int32_t* band = bidx;
  const int groups = NT / 16;  // 16-lane groups: one band entry each at a time
  const int grp = tid >> 4, l16 = tid & 15;

  // The second level narrows the band only where its bound is the tighter one.
  if (mfma_row && need > 0 && E_f < Ebound) {
    // ---- second level: the band's head-folded float32 scores (error <= E_f) select within
    // the band exactly as the first level selected within the row; the rest of the band goes
    // to the float64 re-scoring.
    for (int d = tid; d < kHeadDim; d += NT) {
      auto qat = [&](int i) {
        return q64 ? (float)reinterpret_cast<const double*>(qrow)[i] : qrow[i];
      };
      float f = qat(d);
      for (int hh = 1; hh < P.Hi; ++hh) f = f + qat(hh * kHeadDim + d);
      qfold[d] = f;
    }
    lds_barrier();
    folded_scores16(P, qfold, cbt_row, cw, bidx, nb, groups, grp, l16, bscore);
    if (in_lds) lds_barrier(); else __syncthreads();
    // The need-th largest folded score of the band (ranks made unique by position).
    for (int b = tid; b < nb; b += NT) {
      const double sb = bscore[b];
      int rank = 0;
      for (int b2 = 0; b2 < nb; ++b2) {
        const double s2 = bscore[b2];
        rank += (s2 > sb) || (s2 == sb && b2 < b);
      }
      if (rank == need - 1) s_dbl[0] = sb;
    }
    lds_barrier();
    const double hi2 = s_dbl[0] + 2.0 * E_f, lo2 = s_dbl[0] - 2.0 * E_f;
    // The band's new list: in LDS with the first, or in the row's logits (no longer needed).
    int32_t* band2 = in_lds ? band2_idx_s
                            : reinterpret_cast<int32_t*>(P.logits + wrow * P.col_stride);
    int n_in2_local = 0;
    for (int b = tid; b < nb; b += NT) {
      const double sb = bscore[b];
      const int j = bidx[b];
      if (sb > hi2) {
        atomicOr(&sel_mask[j >> 5], 1u << (j & 31));
        ++n_in2_local;
      } else if (sb >= lo2) {
        band2[atomicAdd(&s_int[6], 1)] = j;
      }
    }
    need -= block_sum<NT>(n_in2_local, s_wave);  // its barriers also publish band2
    nb = __builtin_amdgcn_readfirstlane(s_int[6]);
    band = band2;
  }

  // ---- re-score the band in float64, canonical order (16 lanes per entry; a wave whose four
  // groups hold no entry of the round skips it)
  auto rescore = [&](auto q64_tag, auto relu_tag) {
    constexpr bool kQ64 = decltype(q64_tag)::value, kRelu = decltype(relu_tag)::value;
    for (int b0 = 0; b0 < nb; b0 += groups) {
      if (b0 + 4 * w >= nb) break;  // wave-uniform: later rounds start further on
      const int b = b0 + grp;
      const double s = canonical_score16<kQ64, kRelu>(P, qrow, cbt_row, cw,
                                                      b < nb ? band[b] : -1, l16);
      if (l16 == 0 && b < nb) bscore[b] = s;
    }
  };
  if (q64) {
    if (P.relu) rescore(std::true_type{}, std::true_type{});
    else rescore(std::true_type{}, std::false_type{});
  } else {
    if (P.relu) rescore(std::false_type{}, std::true_type{});
    else rescore(std::false_type{}, std::false_type{});
  }
  if (in_lds) lds_barrier(); else __syncthreads();

  // ---- rank the band: keep its `need` best by (score desc, block asc).
  constexpr int kRankRadixMin = 256;
  if (need > 0 && nb > kRankRadixMin) {  // block-uniform
    // A large band (many exact ties, e.g. an all-zero cache): the need-th best entry by a radix
    // select over the 96-bit key (order-preserving float64 score, then the complemented block
    // index), eight bits per pass; then every entry at or above it is kept.  A score of -0 is
    // keyed as +0: equal scores tie whatever their sign.
    auto dkey = [](double x) {
      const uint64_t u = (uint64_t)__double_as_longlong(x == 0.0 ? 0.0 : x);
      return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
    };
    uint64_t pre_hi = 0, msk_hi = 0;
    uint32_t pre_lo = 0, msk_lo = 0;
    int kr = need;
    int* h = hist[0];
    for (int pass = 0; pass < 12; ++pass) {
      for (int i = tid; i < 256; i += NT) h[i] = 0;
      lds_barrier();
      const int sh = pass < 8 ? 56 - 8 * pass : 24 - 8 * (pass - 8);
      for (int b = tid; b < nb; b += NT) {
        const uint64_t kh = dkey(bscore[b]);
        const uint32_t kl = ~(uint32_t)band[b];
        if ((kh & msk_hi) == pre_hi && (kl & msk_lo) == pre_lo)
          atomicAdd(&h[pass < 8 ? (uint32_t)(kh >> sh) & 0xFFu : (kl >> sh) & 0xFFu], 1);
      }
      lds_barrier();
      const int S = tid < 256 ? h[255 - tid] : 0;  // thread t owns bin 255 - t
      const int incl = wave_incl_scan(S);
      if (lane == 63) s_wave[w] = incl;
      lds_barrier();
      int above = incl - S;
      for (int i = 0; i < w; ++i) above += s_wave[i];
      if (above < kr && kr <= above + S) {
        s_int[4] = 255 - tid;
        s_int[5] = kr - above;
      }
      lds_barrier();
      const uint32_t d = (uint32_t)__builtin_amdgcn_readfirstlane(s_int[4]);
      kr = __builtin_amdgcn_readfirstlane(s_int[5]);
      if (pass < 8) {
        pre_hi |= (uint64_t)d << sh;
        msk_hi |= 0xFFull << sh;
      } else {
        pre_lo |= d << sh;
        msk_lo |= 0xFFu << sh;
      }
    }
    for (int b = tid; b < nb; b += NT) {
      const uint64_t kh = dkey(bscore[b]);
      const int j = band[b];
      if (kh > pre_hi || (kh == pre_hi && ~(uint32_t)j >= pre_lo))
        atomicOr(&sel_mask[j >> 5], 1u << (j & 31));
    }
  } else {
  // A 16-lane group per entry, each lane comparing against every 16th entry, the counts
  // summed on DPP.
  for (int b0 = 0; b0 < nb; b0 += groups) {
    if (b0 + 4 * w >= nb) break;  // wave-uniform, as in the re-scoring
    const int b = b0 + grp;
    const bool live = b < nb;
    const double sb = live ? bscore[b] : 0.0;
    const int jbb = live ? band[b] : 0;
    int rank = 0;
    if (live) {
      for (int b2 = l16; b2 < nb; b2 += 16) {
        const double s2 = bscore[b2];
        rank += (s2 > sb) || (s2 == sb && band[b2] < jbb);
      }
    }
    rank += __builtin_amdgcn_update_dpp(0, rank, 0x108, 0xF, 0xF, false);  // row_shl:8
    rank += __builtin_amdgcn_update_dpp(0, rank, 0x104, 0xF, 0xF, false);  // row_shl:4
    rank += __builtin_amdgcn_update_dpp(0, rank, 0x102, 0xF, 0xF, false);  // row_shl:2
    rank += __builtin_amdgcn_update_dpp(0, rank, 0x101, 0xF, 0xF, false);  // row_shl:1
    if (live && l16 == 0 && rank < need) atomicOr(&sel_mask[jbb >> 5], 1u << (jbb & 31));
  }
  }
  lds_barrier();

  // ---- stable compaction in block order (one workgroup-wide scan) and expansion into tokens
  const uint32_t emask = E == 32 ? 0xFFFFFFFFu : ((1u << E) - 1u);
  const uint32_t selbits =
      keepbits | (jb < vis ? (sel_mask[jb >> 5] >> (jb & 31)) & emask : 0u);
  const int cnt = __builtin_popcount(selbits);
  const int incl = wave_incl_scan(cnt);
  if (lane == 63) s_wave[w] = incl;
  lds_barrier();
  int pos = incl - cnt, total = 0;
  for (int i = 0; i < kWaves; ++i) {
    pos += i < w ? s_wave[i] : 0;
    total += s_wave[i];
  }
  const int sel = min(__builtin_amdgcn_readfirstlane(total), kb), count = sel * P.c + tail;
  // The selected blocks in order go to LDS (the band's score array is free now), and the row
  // is written with coalesced stores; a list too long for it is expanded in place.
  constexpr int kListCap = kBandCap * 2;  // int32 entries in band_score_s
  int32_t* list = reinterpret_cast<int32_t*>(band_score_s);
  const bool list_in_lds = kb <= kListCap;
  for (uint32_t bits = selbits; bits; bits &= bits - 1, ++pos) {
    const int j = jb + __builtin_ctz(bits);
    if (pos < kb) {
      if (list_in_lds) {
        list[pos] = j;
      } else {
        for (int m = 0; m < P.c; ++m) out[pos * P.c + m] = j * P.c + m;
      }
    }
  }
  if (list_in_lds) {
    lds_barrier();
    // Block b's c tokens by thread b (mod NT), then the tail, the padding and the count.
    // With c a multiple of 4 on a 16-byte aligned row a block is c / 4 16-byte stores.
    if ((P.c & 3) == 0 && ((uintptr_t)out & 15u) == 0) {  // block-uniform
      for (int b = tid; b < sel; b += NT) {
        const int t0 = list[b] * P.c;
        int4* o = reinterpret_cast<int4*>(out + b * P.c);
        for (int q = 0; q < (P.c >> 2); ++q)
          o[q] = make_int4(t0 + 4 * q, t0 + 4 * q + 1, t0 + 4 * q + 2, t0 + 4 * q + 3);
      }
    } else {
      for (int b = tid; b < sel; b += NT) {
        const int t0 = list[b] * P.c;
        int32_t* o = out + b * P.c;
        for (int m = 0; m < P.c; ++m) o[m] = t0 + m;
      }
    }
    for (int col = sel * P.c + tid; col <= W; col += NT)
      out[col] = col < count ? vis * P.c + (col - sel * P.c) : (col < W ? -1 : count);
  } else {
    for (int col = sel * P.c + tid; col <= W; col += NT)
      out[col] = col < count ? vis * P.c + (col - sel * P.c) : (col < W ? -1 : count);
  }
}

template <typename C>
hipError_t launch_topk_kernel(const SelectParams& P, size_t mask_bytes, hipStream_t s) {
  hipLaunchKernelGGL((topk_kernel<C>), dim3(P.row_hi - P.row_lo), dim3(C::NT), mask_bytes, s,
                     P);
  return hipGetLastError();
}

}  // namespace

// Error-bound factors of the fast scores, E = F * kappa * A, with gamma_n = n u / (1 - n u):
//  * the head-folded float32 score (the VALU logits): Hi - 1 folding additions and a 128-term
//    dot product, u = 2^-24 (ReLU-sum scores come from the matrix cores: u = 2^-23), F twice
//    gamma_{Hi+130} / (1 - gamma_{Hi+130});
//  * the matrix-core score: Q folded in float32 (heads in order, gamma_{Hi-1}), split into bf16
//    terms hi + mid + lo (residual <= 2^-24 |f|; |hi| <= (1 + 2^-8) |f|, |mid| + |lo| <=
//    2^-7 |f|); per k-step the 32 exact hi products summed by the matrix cores, all mid and lo
//    products in one more sum (any order and rounding: u = 2^-23), and the five partial sums
//    added on the vector unit (u = 2^-24); F twice that, widened by 2^-20.
void topk_bound_factors(int Hi, bool relu, double& e_fold, double& e_mfma) {
  auto gam = [](double n, double u) { return n * u / (1.0 - n * u); };
  const double gam_f = (double)(Hi + 130) * (relu ? 0x1p-23 : 0x1p-24);
  e_fold = 2.0 * gam_f / (1.0 - gam_f);
  const double g_fold = gam(Hi - 1, 0x1p-24);
  const double gam_m = g_fold + (0x1p-24 + gam(34, 0x1p-23) * (1.0 + 0x1p-7) +
                                 gam(2 * kHeadDim + 2, 0x1p-23) * 0x1p-7 +
                                 gam(4, 0x1p-24) * (1.0 + 0x1p-6)) * (1.0 + g_fold);
  e_mfma = 2.0 * gam_m * (1.0 + 0x1p-20);
}

hipError_t launch_topk_select(const SelectParams& P, hipStream_t s) {
  const size_t mask_bytes = (size_t)(P.cols + 31) / 32 * sizeof(uint32_t);
  if (P.row_hi - P.row_lo >= kTopkPrefillMinRows && P.cols <= TopkPrefill::NT * TopkPrefill::E)
    return launch_topk_kernel<TopkPrefill>(P, mask_bytes, s);
  if (P.cols <= 512 * 8) return launch_topk_kernel<TopkDecode8>(P, mask_bytes, s);
  if (P.cols <= 512 * 16) return launch_topk_kernel<TopkDecode16>(P, mask_bytes, s);
  if (P.cols <= 512 * 32) return launch_topk_kernel<TopkDecode32>(P, mask_bytes, s);
  return launch_topk_kernel<TopkDecode1k>(P, mask_bytes, s);
}

}  // namespace qsa
