// qsa_sparse_gqa kernels: split-K paged sparse GQA over the packed selection, and the
// log-sum-exp merge of the splits with the optional sigmoid output gate.
//
// Follows qsa_sparse_paged_attention (page "vllm.models.qwen4_exp.nvidia.ops.qsa") and the
// bf16 branch of _qsa_sparse_paged_gqa_splitk_kernel (FP8 KV reader patch page): per (row, KV
// head, split), tiles of selected tokens are gathered through the block table, invalid entries
// are masked, an exp2 online softmax with scale head_dim^-0.5 * log2(e) accumulates P.V with P
// rounded to bf16, and each split emits float32 (o, lse) partials merged afterwards; with one
// split the kernel writes the gated bf16 output directly.
//
// MI355X layout (VALU only; the work is HBM-bound gather traffic):
//   * one wavefront per (row, KV head, split); a tile is 64 selected tokens;
//   * Q.K: lane <-> token.  Each lane pulls its token's 256-byte K row with 16-byte loads and
//     dots it with the G query heads; Q is wave-uniform and read through the scalar cache, so
//     v_dot2c_f32_bf16 takes it straight from SGPRs;
//   * P.V: lane <-> dims (2l, 2l+1).  Token t's V row is one coalesced 256-byte wave load
//     whose base comes from lane t by readlane; two tokens' values are packed per dot2.
#include "qsa_internal.h"

namespace qsa {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(4))) uint32_t* const_u32_ptr;

struct GqaParams {
  int T, R, Hq, Hkv, pages, P, bt_stride, bt_width, W, splits, tiles_per_split;
  const uint16_t* q;
  int64_t q_rs, q_hs;
  const uint16_t* kv;
  int64_t kv_ps, kv_hs, kv_ts;
  const int32_t* bt;
  const int32_t* t2r;
  const int32_t* packed;
  int64_t p_rs;
  const uint16_t* gate;
  int64_t g_rs, g_hs;
  float scale_log2;
  uint16_t* out;
  int64_t o_rs, o_hs;
  float* part_o;    // [splits, T, Hq, 128]
  float* part_lse;  // [splits, T, Hq]
};

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float sigmoidf(float x) { return 1.0f / (1.0f + expf(-x)); }

// V tile in LDS, transposed for P.V: token pair u, lane l holds (v[2u][l], v[2u+1][l]) as two
// adjacent dwords; pair rows are padded to 130 dwords so the writes of the 64 tokens of one dim
// pair hit 64 distinct banks.
constexpr int kVRow = 130;

template <int G>
__global__ __launch_bounds__(64) void gqa_partial_kernel(GqaParams P) {
  const int row = blockIdx.x, kvh = blockIdx.y, split = blockIdx.z;
  const int lane = threadIdx.x;
  __shared__ uint32_t pb[G][32];          // bf16 probabilities, packed as token pairs
  __shared__ uint32_t vt[32 * kVRow];     // the tile's V, transposed

  int count = P.packed[(int64_t)row * P.p_rs + P.W];
  count = count < 0 ? 0 : (count > P.W ? P.W : count);
  const int r = P.t2r[row];
  if (r < 0 || r >= P.R) count = 0;
  const int ntiles = (count + 63) >> 6;
  const int tile_lo = split * P.tiles_per_split;
  const int tile_hi = min(ntiles, tile_lo + P.tiles_per_split);

  // Q heads kvh*G .. kvh*G+G-1 of this row, read through the scalar cache.
  const const_u32_ptr qs = (const_u32_ptr)(P.q + (int64_t)row * P.q_rs + (int64_t)kvh * G * P.q_hs);
  constexpr int qhs = kHeadDim / 2;  // heads are contiguous: head stride in bf16 pairs

  float m[G], l[G], acc[G][2];
#pragma unroll
  for (int g = 0; g < G; ++g) { m[g] = -INFINITY; l[g] = 0.0f; acc[g][0] = acc[g][1] = 0.0f; }

  const int32_t* sel = P.packed + (int64_t)row * P.p_rs;
  const int32_t* btr = P.bt + (int64_t)(r < 0 ? 0 : r) * P.bt_stride;
  const char* kvb = reinterpret_cast<const char*>(P.kv);

  // Selected entry of this lane's token in tile tt (-1 past the count or the split).
  auto load_idx = [&](int tt) -> int {
    const int t = tt * 64 + lane;
    return (tt < tile_hi && t < count) ? sel[t] : -1;
  };
  // Cache row of an entry, as a 16-byte offset (strides are multiples of 8 elements); invalid
  // entries (negative, past the block table, page out of range) map to the first row.
  auto resolve = [&](int idx, uint32_t& off16, bool& valid) {
    valid = idx >= 0;
    const int col = valid ? idx / P.P : 0;
    valid = valid && col < P.bt_width;
    const int page = valid ? btr[col] : -1;
    valid = valid && page >= 0 && page < P.pages;
    const int slot = idx - col * P.P;
    const int64_t off = valid ? ((int64_t)page * P.kv_ps + (int64_t)kvh * P.kv_hs +
                                 (int64_t)slot * P.kv_ts) : 0;
    off16 = (uint32_t)(off >> 3);
  };
  // This lane's token row: K (first 256 bytes) or V (next 256 bytes), 16 x 16-byte loads.
  auto load_row = [&](uint32_t off16, int half, uint4 (&x)[16]) {
    const uint4* p = reinterpret_cast<const uint4*>(kvb + (size_t)off16 * 16 + half * 256);
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = p[i];
  };

  // The index of tile t+2 and the cache rows of tile t+1 are resolved while tile t is
  // computed, so a tile's gathers issue without waiting on the index -> block-table chain.
  uint32_t off_c = 0, off_n = 0;
  bool valid_c = false, valid_n = false;
  resolve(load_idx(tile_lo), off_c, valid_c);
  resolve(load_idx(tile_lo + 1), off_n, valid_n);
  int idx_nn = load_idx(tile_lo + 2);
  for (int tile = tile_lo; tile < tile_hi; ++tile) {
    // ---- gathers: K and V rows of this lane's token
    uint4 k4[16], v4[16];
    load_row(off_c, 0, k4);
    load_row(off_c, 1, v4);
    uint32_t off_nn = 0;
    bool valid_nn = false;
    resolve(idx_nn, off_nn, valid_nn);
    idx_nn = load_idx(tile + 3);

    // ---- V into the transposed LDS tile (masked tokens as zeros)
    {
      const int u = lane >> 1, h = lane & 1;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t w4[4] = {v4[i].x, v4[i].y, v4[i].z, v4[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) vt[u * kVRow + 2 * (4 * i + e) + h] = valid_c ? w4[e] : 0u;
      }
    }
    if (!valid_c) {
#pragma unroll
      for (int i = 0; i < 16; ++i) k4[i] = make_uint4(0, 0, 0, 0);
    }

    // ---- scores of this lane's token against the G heads.  The Q base is laundered per tile
    // so the compiler re-reads Q from the scalar cache chunk by chunk instead of hoisting all
    // G*64 dwords into (spilled) SGPRs.
    uint64_t qaddr = reinterpret_cast<uint64_t>(qs);
    asm volatile("" : "+s"(qaddr));
    const const_u32_ptr qt = reinterpret_cast<const_u32_ptr>(qaddr);
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t kk[4] = {k4[i].x, k4[i].y, k4[i].z, k4[i].w};
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s[g] = dot2_bf16(qt[g * qhs + 4 * i + e], kk[e], s[g]);
      }
    }

    // ---- online softmax (base 2); P rounded to bf16 as the reference does before P.V
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float z = valid_c ? s[g] * P.scale_log2 : -INFINITY;
      const float mn = fmaxf(m[g], wave_max(z));
      float alpha = 1.0f, pr = 0.0f;
      if (mn != -INFINITY) {
        alpha = exp2f(m[g] - mn);
        pr = exp2f(z - mn);
      }
      const uint32_t pbits = f32_to_bf16(pr);
      l[g] = l[g] * alpha + bf16_to_f32(pbits);
      acc[g][0] *= alpha;
      acc[g][1] *= alpha;
      m[g] = mn;
      reinterpret_cast<uint16_t*>(pb[g])[lane] = (uint16_t)pbits;
    }
    __syncthreads();

    // ---- P.V over token pairs: lane l owns dims 2l, 2l+1
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const uint2 ab = *reinterpret_cast<const uint2*>(&vt[u * kVRow + 2 * lane]);
      const uint32_t vd0 = __builtin_amdgcn_perm(ab.y, ab.x, 0x05040100u);  // lo halves
      const uint32_t vd1 = __builtin_amdgcn_perm(ab.y, ab.x, 0x07060302u);  // hi halves
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint32_t pp = pb[g][u];
        acc[g][0] = dot2_bf16(pp, vd0, acc[g][0]);
        acc[g][1] = dot2_bf16(pp, vd1, acc[g][1]);
      }
    }
    __syncthreads();
    off_c = off_n;
    valid_c = valid_n;
    off_n = off_nn;
    valid_n = valid_nn;
  }

  // ---- epilogue
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float lsum = wave_sum(l[g]);
    const int hq = kvh * G + g;
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
    float o0 = acc[g][0] * inv, o1 = acc[g][1] * inv;
    if (P.splits == 1) {
      if (P.gate) {
        const uint32_t gp = reinterpret_cast<const uint32_t*>(
            P.gate + (int64_t)row * P.g_rs + (int64_t)hq * P.g_hs)[lane];
        o0 *= sigmoidf(bf16lo(gp));
        o1 *= sigmoidf(bf16hi(gp));
      }
      reinterpret_cast<uint32_t*>(P.out + (int64_t)row * P.o_rs + (int64_t)hq * P.o_hs)[lane] =
          (f32_to_bf16(o0) & 0xFFFFu) | (f32_to_bf16(o1) << 16);
    } else {
      const int64_t pi = ((int64_t)split * P.T + row) * P.Hq + hq;
      reinterpret_cast<float2*>(P.part_o + pi * kHeadDim)[lane] = make_float2(o0, o1);
      if (lane == 0) P.part_lse[pi] = lsum > 0.0f ? m[g] + log2f(lsum) : -INFINITY;
    }
  }
}

// Grid (T, Hq), one wavefront.  Lane s reads split s's log-sum-exp (all splits at once), the
// weights are formed in-wave, then lane l merges dims 2l, 2l+1 of every split with independent
// loads.  splits <= 64.
__global__ __launch_bounds__(64) void gqa_merge_kernel(GqaParams P) {
  const int row = blockIdx.x, hq = blockIdx.y, lane = threadIdx.x;
  const int64_t stride = (int64_t)P.T * P.Hq;   // between splits
  const int64_t pi0 = (int64_t)row * P.Hq + hq;
  const float lse = lane < P.splits ? P.part_lse[lane * stride + pi0] : -INFINITY;
  const float M = wave_max(lse);
  float o0 = 0.0f, o1 = 0.0f;
  if (M != -INFINITY) {
    const float wgt = lse == -INFINITY ? 0.0f : exp2f(lse - M);
    const float inv = 1.0f / wave_sum(wgt);
#pragma unroll 8
    for (int s = 0; s < P.splits; ++s) {
      const float ws = __shfl(wgt, s, kWave);
      const float2 o = reinterpret_cast<const float2*>(P.part_o + (s * stride + pi0) * kHeadDim)[lane];
      o0 += ws * o.x;
      o1 += ws * o.y;
    }
    o0 *= inv;
    o1 *= inv;
    if (P.gate) {
      const uint32_t gp = reinterpret_cast<const uint32_t*>(
          P.gate + (int64_t)row * P.g_rs + (int64_t)hq * P.g_hs)[lane];
      o0 *= sigmoidf(bf16lo(gp));
      o1 *= sigmoidf(bf16hi(gp));
    }
  }
  reinterpret_cast<uint32_t*>(P.out + (int64_t)row * P.o_rs + (int64_t)hq * P.o_hs)[lane] =
      (f32_to_bf16(o0) & 0xFFFFu) | (f32_to_bf16(o1) << 16);
}

template <int G>
hipError_t launch_partial(const GqaParams& P, hipStream_t s) {
  hipLaunchKernelGGL(gqa_partial_kernel<G>, dim3(P.T, P.Hkv, P.splits), dim3(64), 0, s, P);
  return hipGetLastError();
}

}  // namespace

GqaPlan gqa_plan(const qsa_gqa_args& a) {
  GqaPlan p{};
  p.tiles = (a.packed_width + 63) / 64;
  if (p.tiles < 1) p.tiles = 1;
  int target = a.num_splits;
  if (target <= 0) {
    // Aim for about 2048 workgroups (8 per CU) so the gathers keep HBM busy.
    const int64_t base = (int64_t)a.num_tokens * a.num_kv_heads;
    target = base >= 2048 ? 1 : (int)((2048 + base - 1) / base);
  }
  if (target > p.tiles) target = p.tiles;
  if (target > 64) target = 64;  // the merge reads one split per lane
  p.tiles_per_split = (p.tiles + target - 1) / target;
  p.splits = (p.tiles + p.tiles_per_split - 1) / p.tiles_per_split;
  p.ws_bytes = 0;
  if (p.splits > 1) {
    const size_t n = (size_t)p.splits * a.num_tokens * a.num_q_heads;
    p.ws_bytes = (n * kHeadDim * sizeof(float) + 255) / 256 * 256 + n * sizeof(float);
  }
  return p;
}

hipError_t launch_gqa(const qsa_gqa_args& a, const GqaPlan& plan, char* ws, hipStream_t s) {
  GqaParams P{};
  P.T = a.num_tokens;
  P.R = a.num_requests;
  P.Hq = a.num_q_heads;
  P.Hkv = a.num_kv_heads;
  P.pages = a.num_pages;
  P.P = a.page_size;
  P.bt_stride = a.block_table_stride;
  P.bt_width = a.block_table_width;
  P.W = a.packed_width;
  P.splits = plan.splits;
  P.tiles_per_split = plan.tiles_per_split;
  P.q = a.q;
  P.q_rs = a.q_row_stride;
  P.q_hs = a.q_head_stride;
  P.kv = a.kv_cache;
  P.kv_ps = a.kv_page_stride;
  P.kv_hs = a.kv_head_stride;
  P.kv_ts = a.kv_token_stride;
  P.bt = a.block_table;
  P.t2r = a.token_to_req;
  P.packed = a.packed;
  P.p_rs = a.packed_row_stride;
  P.gate = a.gate;
  P.g_rs = a.gate_row_stride;
  P.g_hs = a.gate_head_stride;
  const float scale = a.scale > 0.0f ? a.scale : 1.0f / sqrtf((float)a.head_dim);
  P.scale_log2 = scale * 1.4426950408889634f;
  P.out = a.out;
  P.o_rs = a.out_row_stride;
  P.o_hs = a.out_head_stride;
  if (plan.splits > 1) {
    const size_t n = (size_t)plan.splits * a.num_tokens * a.num_q_heads;
    P.part_o = reinterpret_cast<float*>(ws);
    P.part_lse = reinterpret_cast<float*>(ws + (n * kHeadDim * sizeof(float) + 255) / 256 * 256);
  }
  hipError_t e;
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: e = launch_partial<1>(P, s); break;
    case 2: e = launch_partial<2>(P, s); break;
    case 4: e = launch_partial<4>(P, s); break;
    case 8: e = launch_partial<8>(P, s); break;
    case 16: e = launch_partial<16>(P, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || plan.splits == 1) return e;
  hipLaunchKernelGGL(gqa_merge_kernel, dim3(P.T, P.Hq), dim3(64), 0, s, P);
  return hipGetLastError();
}

}  // namespace qsa
