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
//   * one wavefront per (row, KV head, split); a tile is 64 selected tokens.  The split's
//     entries are resolved to cache rows up front (index and block-table loads all in flight
//     together) and kept in LDS;
//   * K and V are gathered with coalesced 16-byte loads, 16 lanes per 256-byte row.  K goes
//     straight to LDS (global_load_lds_dwordx4, no registers) one tile ahead; V goes to
//     registers at the start of its tile and lands while Q.K and the softmax run;
//   * Q.K: lane <-> token, reading its K row from LDS; Q is wave-uniform and read through the
//     scalar cache, so v_dot2c_f32_bf16 takes it straight from SGPRs;
//   * P.V: lane <-> (token quarter, 8 dims); the bf16 probabilities go through LDS packed per
//     token pair, two tokens' values per dot2; the quarters are summed at the end.
#include <type_traits>

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

// The partial kernel's workgroup is one wavefront, whose LDS operations complete in order:
// data written to LDS by some lanes is readable by the others once the writes are done, with
// no s_barrier and no memory fence (a fence would also wait for the loads in flight).
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// Per-head maximum over the wavefront of G values per lane (value g of lane t belongs to head
// g), returned wave-uniform.  The heads are reduced together: at each exchange across a lane
// bit a lane keeps one half of the heads it carries and receives the partner's copy of that
// half, so G = 2^k heads cost 2^k - 1 exchanges plus 6 - k ordinary steps instead of 6G.
// Afterwards head h is held by lane h * 64 / G.
template <int G>
__device__ __forceinline__ void tile_max(const float (&z)[G], float (&mt)[G]) {
  constexpr int K = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : G == 8 ? 3 : 4;
  const int lane = threadIdx.x & 63;
  float v[G];
#pragma unroll
  for (int g = 0; g < G; ++g) v[g] = z[g];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int bit = 32 >> j;
    const bool hi = (lane & bit) != 0;
    constexpr int kMaxN = G / 2;
#pragma unroll
    for (int i = 0; i < kMaxN; ++i) {
      const int n = G >> (j + 1);
      if (i >= n) break;
      const float keep = hi ? v[n + i] : v[i];
      const float send = hi ? v[i] : v[n + i];
      v[i] = fmaxf(keep, __shfl_xor(send, bit, kWave));
    }
  }
#pragma unroll
  for (int bit = 32 >> K; bit >= 1; bit >>= 1) v[0] = fmaxf(v[0], __shfl_xor(v[0], bit, kWave));
#pragma unroll
  for (int h = 0; h < G; ++h)
    mt[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[0]), h * (64 / G)));
}

// K tile in LDS: token t's 256-byte row at 256*t bytes, its 16-byte chunk c stored in slot
// c ^ (t & 15), so that 16 consecutive lanes reading chunk c of their own rows touch 16
// different slots (all 64 banks once).  The tile is filled by LDS-direct loads
// (global_load_lds_dwordx4): load i writes 1 KiB at 1024*i, lane L at 16*L, which is token
// 4i + L/16, slot L%16.
constexpr int kKTileDw = 64 * 64;
constexpr int kChunkTiles = 8;  // tiles whose cache rows are resolved together

template <int G>
__global__ __launch_bounds__(64) void gqa_partial_kernel(GqaParams P) {
  const int row = blockIdx.x, kvh = blockIdx.y, split = blockIdx.z;
  const int lane = threadIdx.x;
  const int qq = lane >> 4;   // quarter: the token of a coalesced load within its group of 4
  const int ch = lane & 15;   // 16-byte chunk of a 256-byte row
  __shared__ __attribute__((aligned(16))) uint32_t kt[kKTileDw];
  // bf16 probabilities, packed per P.V token pair: pr[(j*4 + quarter) * G + g] holds
  // (p[g][8j + quarter], p[g][8j + 4 + quarter]).
  __shared__ __attribute__((aligned(16))) uint32_t pr[32 * G];
  // Resolved cache rows (16-byte offsets) of the tiles of the current chunk, and their masks.
  __shared__ __attribute__((aligned(16))) uint32_t offs[kChunkTiles * 64];
  __shared__ uint64_t vms[kChunkTiles];

  // The split's tile range comes from the packed width, so that its first index loads need
  // not wait for the count: the count, the request and the first chunk's entries are read in
  // one round trip.
  int count = P.packed[(int64_t)row * P.p_rs + P.W];
  const int r = P.t2r[row];
  const int tile_lo = split * P.tiles_per_split;
  const int tile_end = min((P.W + 63) >> 6, tile_lo + P.tiles_per_split);

  // Q heads kvh*G .. kvh*G+G-1 of this row, read through the scalar cache.
  const const_u32_ptr qs = (const_u32_ptr)(P.q + (int64_t)row * P.q_rs + (int64_t)kvh * G * P.q_hs);
  constexpr int qhs = kHeadDim / 2;  // heads are contiguous: head stride in bf16 pairs

  // m, l: running max and (per-lane partial) normaliser per head; acc: this lane's 8 dims
  // (8*ch .. 8*ch+7) of every head, over the tokens of its quarter.
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[g][d] = 0.0f;
  }

  const int32_t* sel = P.packed + (int64_t)row * P.p_rs;
  const int32_t* btr = P.bt + (int64_t)(r < 0 || r >= P.R ? 0 : r) * P.bt_stride;
  const char* kvb = reinterpret_cast<const char*>(P.kv);

  // Cache rows (16-byte offsets) of the 16 tokens this lane loads in chunk tile k.
  auto row_offsets = [&](int k, uint32_t (&o)[16]) {
    const uint4* src = reinterpret_cast<const uint4*>(offs + k * 64 + qq * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 x = src[i];
      o[4 * i] = x.x;
      o[4 * i + 1] = x.y;
      o[4 * i + 2] = x.z;
      o[4 * i + 3] = x.w;
    }
  };
  // K rows of chunk tile k into LDS (no registers); coalesced: 16 lanes per 256-byte row.
  auto issue_k = [&](int k) {
    uint32_t o[16];
    row_offsets(k, o);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = 4 * i + qq;
      const char* src = kvb + (size_t)o[i] * 16 + 16 * (ch ^ (t & 15));
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)src,
          (__attribute__((address_space(3))) void*)(kt + 256 * i), 16, 0, 0);
    }
  };
  // V rows of chunk tile k into registers: v4[i] = chunk ch of token 4i + qq.
  auto issue_v = [&](int k, uint4 (&v4)[16]) {
    uint32_t o[16];
    row_offsets(k, o);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      v4[i] = (reinterpret_cast<const uint4*>(kvb + (size_t)o[i] * 16) + 16)[ch];
  };

  for (int c0 = tile_lo; c0 < tile_end; c0 += kChunkTiles) {
    // ---- resolve the chunk's entries to cache rows: all index loads, then all block-table
    // loads, in flight together.  The loads are unconditional, at clamped addresses (the
    // row's W entries and the block table's first column exist).  Invalid entries (negative,
    // past the block table, page out of range, past the count) read the first row and are
    // masked.
    int idx[kChunkTiles], page[kChunkTiles];
#pragma unroll
    for (int k = 0; k < kChunkTiles; ++k) idx[k] = sel[min((c0 + k) * 64 + lane, P.W - 1)];
    asm volatile("" : "+v"(idx[0]), "+v"(idx[1]), "+v"(idx[2]), "+v"(idx[3]), "+v"(idx[4]),
                 "+v"(idx[5]), "+v"(idx[6]), "+v"(idx[7]));
    if (c0 == tile_lo) {
      count = count < 0 ? 0 : (count > P.W ? P.W : count);
      if (r < 0 || r >= P.R) count = 0;
    }
    const int nt = min(kChunkTiles, min(tile_end, (count + 63) >> 6) - c0);
    if (nt <= 0) break;  // wave-uniform
#pragma unroll
    for (int k = 0; k < kChunkTiles; ++k) {
      const int t = (c0 + k) * 64 + lane;
      if (!(k < nt && t < count) || idx[k] < 0) idx[k] = -1;
      const int col = idx[k] >= 0 ? idx[k] / P.P : 0;
      page[k] = btr[min(col, P.bt_width - 1)];
    }
    asm volatile("" : "+v"(page[0]), "+v"(page[1]), "+v"(page[2]), "+v"(page[3]),
                 "+v"(page[4]), "+v"(page[5]), "+v"(page[6]), "+v"(page[7]));
#pragma unroll
    for (int k = 0; k < kChunkTiles; ++k) {
      const int col = idx[k] >= 0 ? idx[k] / P.P : P.bt_width;
      const bool valid = col < P.bt_width && page[k] >= 0 && page[k] < P.pages;
      const int slot = idx[k] - col * P.P;
      const int64_t off = valid ? ((int64_t)page[k] * P.kv_ps + (int64_t)kvh * P.kv_hs +
                                   (int64_t)slot * P.kv_ts) : 0;
      // Stored so that lane L's 16 rows (tokens 4i + L/16) are contiguous.
      offs[k * 64 + (lane & 3) * 16 + (lane >> 2)] = (uint32_t)(off >> 3);
      const uint64_t vm = __ballot(valid);
      if (lane == 0) vms[k] = vm;
    }
    wave_lds_sync();
    issue_k(0);

    // One tile: its V loads are issued first and overlap Q.K and the softmax; its K rows were
    // loaded into LDS during the previous tile.  With MORE it loads the next tile's K once
    // Q.K is done.  The last tile of a chunk is a separate instance, so that every path into
    // a tile has exactly the tile's K loads in flight before its V loads (which lets the wait
    // below be exact).
    auto tile = [&](int k, auto more_tag) {
      constexpr bool more = decltype(more_tag)::value;
      uint4 v4[16];
      asm volatile("" ::: "memory");  // V loads strictly after the K loads
      issue_v(k, v4);
      // The 16 V loads of this tile are the only memory loads issued after its K loads.
      __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16): this tile's K rows have landed
      wave_lds_sync();

      // ---- scores of this lane's token against the G heads, K read from LDS two chunks at a
      // time (the next pair in flight while a pair is used).
      float s[G];
#pragma unroll
      for (int g = 0; g < G; ++g) s[g] = 0.0f;
      uint32_t kbase = lane * 256, sw = lane & 15;
      asm volatile("" : "+v"(kbase), "+v"(sw));
      auto kread = [&](int i) {
        return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(kt) + kbase +
                                               16 * (i ^ sw));
      };
      // Q.K runs in steps of (K chunk i, group of GB heads).  The Q of the next step is
      // requested through the scalar cache while a step is computed; its base address is
      // laundered and tied to the running scores, so that only two steps' Q (2 x 4GB dwords)
      // are live in SGPRs, instead of all G*64 dwords being hoisted (and spilled).
      constexpr int GB = G < 4 ? G : 4;
      constexpr int kSteps = 16 * (G / GB);
      auto load_q = [&](int st, uint32_t (&q)[GB][4]) {
        const int i = st / (G / GB), g0 = (st % (G / GB)) * GB;
        uint64_t qaddr = reinterpret_cast<uint64_t>(qs);
        if constexpr (G == 1) asm volatile("" : "+s"(qaddr), "+v"(s[0]));
        else if constexpr (G == 2) asm volatile("" : "+s"(qaddr), "+v"(s[0]), "+v"(s[1]));
        else {
#pragma unroll
          for (int g = 0; g < G; g += 4)
            asm volatile("" : "+s"(qaddr), "+v"(s[g]), "+v"(s[g + 1]), "+v"(s[g + 2]),
                         "+v"(s[g + 3]));
        }
        const const_u32_ptr qt = reinterpret_cast<const_u32_ptr>(qaddr);
#pragma unroll
        for (int g = 0; g < GB; ++g) {
#pragma unroll
          for (int e = 0; e < 4; ++e) q[g][e] = qt[(g0 + g) * qhs + 4 * i + e];
        }
      };
      uint32_t qc[GB][4];
      load_q(0, qc);
      uint4 ka = kread(0), kb = kread(1);
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const uint4 k0 = ka, k1 = kb;
        if (i + 2 < 16) {
          ka = kread(i + 2);
          kb = kread(i + 3);
        }
#pragma unroll
        for (int st = i * (G / GB); st < (i + 2) * (G / GB); ++st) {
          uint32_t qn[GB][4];
          if (st + 1 < kSteps) load_q(st + 1, qn);
          const uint4 kc = (st / (G / GB)) == i ? k0 : k1;
          const uint32_t kk[4] = {kc.x, kc.y, kc.z, kc.w};
          const int g0 = (st % (G / GB)) * GB;
#pragma unroll
          for (int g = 0; g < GB; ++g) {
#pragma unroll
            for (int e = 0; e < 4; ++e) s[g0 + g] = dot2_bf16(qc[g][e], kk[e], s[g0 + g]);
          }
          if (st + 1 < kSteps) {
#pragma unroll
            for (int g = 0; g < GB; ++g) {
#pragma unroll
              for (int e = 0; e < 4; ++e) qc[g][e] = qn[g][e];
            }
          }
        }
      }
      const uint64_t vmask = vms[k];
      const bool valid = (vmask >> lane) & 1ull;
      // Every K read has returned before the next tile's rows overwrite the tile.  The
      // scheduling barriers keep the phases in order: nothing that needs this tile's V is
      // moved up into Q.K (which would wait for V early).
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (more) issue_k(k + 1);
      __builtin_amdgcn_sched_barrier(0);

      // ---- online softmax (base 2); P rounded to bf16 as the reference does before P.V.
      // A masked token's score is never used, so its (possibly poisoned) K needs no zeroing.
      const int pslot = ((lane >> 3) * 4 + (lane & 3)) * G;  // pair of token `lane`
      const int phalf = (lane >> 2) & 1;                      // its half of the pair
      float z[G], mt[G];
#pragma unroll
      for (int g = 0; g < G; ++g) z[g] = valid ? s[g] * P.scale_log2 : -INFINITY;
      tile_max<G>(z, mt);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mn = fmaxf(m[g], mt[g]);
        float alpha = 1.0f, pexp = 0.0f;
        if (mn != -INFINITY) {
          alpha = exp2f(m[g] - mn);
          pexp = exp2f(z[g] - mn);
        }
        const uint32_t pbits = f32_to_bf16(pexp);
        l[g] = l[g] * alpha + bf16_to_f32(pbits);
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[g][d] *= alpha;
        m[g] = mn;
        reinterpret_cast<uint16_t*>(pr)[2 * (pslot + g) + phalf] = (uint16_t)pbits;
      }
      // This tile's V has landed (only the next tile's K loads may still be in flight).
      if constexpr (more) __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16)
      else __builtin_amdgcn_s_waitcnt(0x0F70);                 // vmcnt(0)
      // A masked token's V may hold anything (NaN-poisoned slots included): zero it.
      if (vmask != ~0ull) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (!((vmask >> (4 * i + qq)) & 1ull)) v4[i] = make_uint4(0, 0, 0, 0);
      }
      wave_lds_sync();

      // ---- P.V: pair j = tokens 8j+qq and 8j+4+qq (loads 2j and 2j+1 of this lane)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t pp[G];
#pragma unroll
        for (int g = 0; g < G; ++g) pp[g] = pr[(j * 4 + qq) * G + g];
        const uint4 a = v4[2 * j], b = v4[2 * j + 1];
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t vlo = __builtin_amdgcn_perm(bw[e], aw[e], 0x05040100u);  // dim 2e
          const uint32_t vhi = __builtin_amdgcn_perm(bw[e], aw[e], 0x07060302u);  // dim 2e+1
#pragma unroll
          for (int g = 0; g < G; ++g) {
            acc[g][2 * e] = dot2_bf16(pp[g], vlo, acc[g][2 * e]);
            acc[g][2 * e + 1] = dot2_bf16(pp[g], vhi, acc[g][2 * e + 1]);
          }
        }
      }
      wave_lds_sync();
    };
    for (int k = 0; k + 1 < nt; ++k) tile(k, std::true_type{});
    tile(nt - 1, std::false_type{});
    // The chunk's last tile issued no loads; the next chunk overwrites offs after this.
    wave_lds_sync();
  }

  // ---- epilogue: sum the four quarters' accumulators, normalise, write dims 8ch..8ch+7
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      float v = acc[g][d];
      v += __shfl_xor(v, 16, kWave);
      v += __shfl_xor(v, 32, kWave);
      acc[g][d] = v;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float lsum = wave_sum(l[g]);
    const int hq = kvh * G + g;
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
    if (qq != 0) continue;
    float o[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] = acc[g][d] * inv;
    if (P.splits == 1) {
      // Gate and output rows are only 4-byte aligned: dword accesses.
      if (P.gate) {
        const uint32_t* gp = reinterpret_cast<const uint32_t*>(
            P.gate + (int64_t)row * P.g_rs + (int64_t)hq * P.g_hs) + 4 * ch;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t gw = gp[e];
          o[2 * e] *= sigmoidf(bf16lo(gw));
          o[2 * e + 1] *= sigmoidf(bf16hi(gw));
        }
      }
      uint32_t* op = reinterpret_cast<uint32_t*>(
          P.out + (int64_t)row * P.o_rs + (int64_t)hq * P.o_hs) + 4 * ch;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        op[e] = (f32_to_bf16(o[2 * e]) & 0xFFFFu) | (f32_to_bf16(o[2 * e + 1]) << 16);
    } else {
      const int64_t pi = ((int64_t)split * P.T + row) * P.Hq + hq;
      float4* dst = reinterpret_cast<float4*>(P.part_o + pi * kHeadDim) + 2 * ch;
      dst[0] = make_float4(o[0], o[1], o[2], o[3]);
      dst[1] = make_float4(o[4], o[5], o[6], o[7]);
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
