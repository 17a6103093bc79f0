// Indexer logits under the ReLU-sum aggregation on the matrix cores: for every row and compressed
// block, sum over the index heads of max(0, q_h . k), with each head's dot product a column of a
// v_mfma_f32_16x16x32 contraction (bf16, or e4m3 codes).  Follows the scoring step of
// QSAIndexer.forward (page "vllm.models.qwen4_exp.nvidia.qsa") with the aggregation switch in
// place of its head sum.
//
// Error bound: every product of two bf16 (or two e4m3) values is exact in float32; a head's 128
// products are accumulated in an order the matrix core does not specify, so with faithful
// rounding (u = 2^-23) the head's score is within gamma_130 of its exact value times
// sum_d |q_hd k_d|; max(0, .) does not increase the distance, and the head sum is a DPP tree
// over the 16 head lanes: any one head's value meets at most min(Hi - 1, 4) roundings (adding a
// zero column past Hi is exact), which adds at most gamma_{Hi-1}.  The top-k bounds the whole
// score by gamma_{Hi+130} (u = 2^-23) kappa A.
#include "logits_tile.h"

namespace qsa {
namespace {
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kReluKeys = 1024;  // keys per workgroup: 8 waves x 128 (one 128-key block each)

// Grid (key items, R), 512 threads.  Workgroup (k, r) scores keys 1024k .. 1024k+1023 of
// request r against each of its rows in [row_lo, row_hi).  Wave w holds keys 1024k + 128w +
// 16g + (lane % 16), g < 8, as the A operand: for k-step ks (dims 32ks .. 32ks+31) lane l holds
// dims 32ks + 8(l/16) .. +7 of its key, one 16-byte (bf16) or 8-byte (e4m3) load, so the
// wave's 128 keys are in registers once and serve every row.  The row's Q is the B operand:
// lane l holds head l % 16 (zero past Hi: its column adds nothing), the same 8 dims.  The
// product's lane l ends with keys 4(l/16) + e, e < 4, of head l % 16: max(0, .), a DPP sum over
// the 16 head lanes, and lane 4(l/16) + e' stores key 4(l/16) + e'.
template <bool F8>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void logits_relu_mfma_kernel(SelectParams P) {
  using frag_t = std::conditional_t<F8, long, bf16x8_t>;
  constexpr int kRowB = F8 ? 128 : 256;  // bytes of a key row
  constexpr int kT = 512;
  __shared__ int32_t rows_s[kReluKeys];
  const int r = blockIdx.y, k = blockIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, l4 = lane >> 4;
  const int jw = k * kReluKeys;
  // Block-table entries of this thread's keys (loaded with the request metadata).
  int col[kReluKeys / kT], page[kReluKeys / kT];
#pragma unroll
  for (int i = 0; i < kReluKeys / kT; ++i) {
    col[i] = (jw + (int)threadIdx.x + kT * i) / P.Pc;
    page[i] = P.cbt[(int64_t)r * P.cbt_stride + min(col[i], P.cbt_width - 1)];
  }
  // Row range of the request, clamped into [0, T) (device data the host never saw).
  const int q0 = max(0, min(P.qsl[r], P.T));
  const int n = max(0, min(P.qsl[r + 1], P.T) - q0), L = P.seq_lens[r];
  const int vis_max = (n > 0 && n <= L) ? min(L / P.c, P.cols) : 0;
  const int rb = min(max(P.row_lo - q0, 0), n), re = min(max(P.row_hi - q0, 0), n);
  if (rb >= re || jw >= vis_max) return;  // workgroup-uniform, before any barrier
#pragma unroll
  for (int i = 0; i < kReluKeys / kT; ++i) {
    const int j = jw + threadIdx.x + kT * i;
    const bool ok = j < vis_max && col[i] < P.cbt_width && page[i] >= 0 && page[i] < P.c_pages;
    rows_s[threadIdx.x + kT * i] = ok ? page[i] * P.Pc + (j - col[i] * P.Pc) : -1;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // ---- the wave's 128 keys as A fragments.  A key past the visible range reads the cache's
  // first row (its score is never stored); a visible key whose page is outside the cache is
  // zeroed below (it scores as an all-zero key).
  const char* ckv = reinterpret_cast<const char*>(P.ckv);
  frag_t kf[8][4];
  uint32_t okm = 0;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const int rw = rows_s[128 * w + 16 * g + l16];
    okm |= (uint32_t)(rw >= 0) << g;
    const char* src = ckv + (int64_t)max(rw, 0) * kRowB + (8 * l4) * (F8 ? 1 : 2);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      kf[g][ks] = *reinterpret_cast<const frag_t*>(src + 32 * ks * (F8 ? 1 : 2));
  }
  // Upper bound of max |k| over the wave's block of 128 keys (masked keys excluded).
  float km = 0.0f;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    float m = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if constexpr (F8) {
        const uint64_t u = (uint64_t)kf[g][ks];
        const uint32_t w0 = (uint32_t)u, w1 = (uint32_t)(u >> 32);
        const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false);
        const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
        const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false);
        const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
        const float ab = fmaxf(fmaxf(fabsf(a[0]), fabsf(a[1])), fmaxf(fabsf(b[0]), fabsf(b[1])));
        const float cd = fmaxf(fmaxf(fabsf(c[0]), fabsf(c[1])), fmaxf(fabsf(d[0]), fabsf(d[1])));
        m = fmaxf(m, fmaxf(ab, cd));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)kf[g][ks][e]));
      }
    }
    km = fmaxf(km, ((okm >> g) & 1u) ? m : 0.0f);  // masked keys dropped by a select
    if (!((okm >> g) & 1u)) {  // an all-zero key (selects: the row may hold NaN)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if constexpr (F8) kf[g][ks] = 0l;
        else kf[g][ks] = bf16x8_t{};
      }
    }
  }
  km = wave_max(km);
  const int blk = k * (kReluKeys / 128) + w;
  if (lane == 0 && blk < P.key_blocks) P.kmax[(int64_t)r * P.key_blocks + blk] = km;

  // ---- every row of the request in this window
  const char* qb = reinterpret_cast<const char*>(P.q_idx);
  for (int rr = rb; rr < re; ++rr) {
    const int row = q0 + rr;
    frag_t qf[4];
    const char* qsrc = qb +
                       ((int64_t)row * P.Hi + min(l16, P.Hi - 1)) * kHeadDim * (F8 ? 1 : 2) +
                       (8 * l4) * (F8 ? 1 : 2);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const frag_t v = *reinterpret_cast<const frag_t*>(qsrc + 32 * ks * (F8 ? 1 : 2));
      if constexpr (F8) qf[ks] = l16 < P.Hi ? v : 0l;
      else qf[ks] = l16 < P.Hi ? v : bf16x8_t{};
    }
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        P.logits + (int64_t)(row - P.row_lo) * P.col_stride, 0, vis_max * 4, 0x00020000);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if constexpr (F8)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(kf[g][ks], qf[ks], acc, 0, 0, 0);
        else
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[g][ks], qf[ks], acc, 0, 0, 0);
      }
      // Lane l: keys 4(l/16) + e of head l % 16.  ReLU, then the sum over the 16 head lanes.
      float s[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] = logits_tile::group_sum<16>(fmaxf(acc[e], 0.0f));
      const float v = l16 == 0 ? s[0] : (l16 == 1 ? s[1] : (l16 == 2 ? s[2] : s[3]));
      const int j = jw + 128 * w + 16 * g + 4 * l4 + l16;
      const uint32_t off = l16 < 4 ? (uint32_t)j * 4u : 0xFFFFFFF0u;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, off, 0, 0);
    }
  }
}

}  // namespace

hipError_t launch_logits_relu_mfma(const SelectParams& P, hipStream_t s) {
  const dim3 grid((P.cols + kReluKeys - 1) / kReluKeys, P.R), block(512);
  if (P.fp8)
    hipLaunchKernelGGL(logits_relu_mfma_kernel<true>, grid, block, 0, s, P);
  else
    hipLaunchKernelGGL(logits_relu_mfma_kernel<false>, grid, block, 0, s, P);
  return hipGetLastError();
}

}  // namespace qsa
