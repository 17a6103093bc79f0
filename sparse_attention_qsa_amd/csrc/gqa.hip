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
// MI355X layout: one wavefront per (row, KV head, split), tiles of 32 selected tokens; with
// bf16 K/V and at most 8 splits the splits of a (row, KV head) are the waves of one workgroup,
// which merges them in LDS (no partials in memory, no merge kernel).  The
// split's entries are resolved to cache rows up front (index and block-table loads all in
// flight together) and kept in LDS; K and V rows are gathered straight into LDS with
// coalesced 16-byte LDS-direct loads, a tile ahead; both contractions (Q.K over the G heads
// of a KV head, and P.V) run on the matrix cores, which leaves the wave's VALU time to the
// softmax (measured: the dot2 form of these contractions kept the SIMDs busy while the
// gathers waited on them).
#include <mutex>
#include <type_traits>

#include "qsa_internal.h"

namespace qsa {
namespace {


struct GqaParams {
  int T, R, Hq, Hkv, pages, P, bt_stride, bt_width, W, splits, tiles_per_split;
  const uint16_t* q;
  int64_t q_rs, q_hs;
  const uint8_t* kv;
  int64_t kv_ps, kv_hs, kv_ts;  // bytes
  float v_scale;                // output scale: 1 for bf16, the V dequantization scale for fp8
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
  // Row tiles (prefill): flags [Hkv, T / kRT], set to 1 for each (tile, KV head) whose outputs
  // the row-tiled kernel wrote (the per-row kernel then skips those rows); NULL: none.
  int32_t* rt_flags;
};


__device__ __forceinline__ float sigmoidf(float x) { return 1.0f / (1.0f + expf(-x)); }

// The partial kernel's workgroup is one wavefront, whose LDS operations complete in order:
// data written to LDS by some lanes is readable by the others once the writes are done, with
// no s_barrier and no memory fence (a fence would also wait for the loads in flight).
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 32;        // selected tokens per tile (one MFMA K step of P.V)
constexpr int kChunkTiles = 8;   // tiles whose cache rows are resolved together
constexpr int kMergeWaves = 8;   // splits merged inside one workgroup (bf16 K/V)
constexpr int kRT = 32;          // rows per tile of the row-tiled (prefill) kernel

__device__ __forceinline__ void lds_dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// K and V tiles in LDS: token t's row (256 bytes bf16, 128 bytes fp8) at t * row, its 16-byte
// chunk c in slot c ^ (t & 15) (bf16) or c ^ (t & 7) (fp8).  They are filled by LDS-direct
// loads of 1 KiB: bf16 load i writes tokens 4i .. 4i+3 (lane L: token 4i + L/16, slot L%16),
// fp8 load i tokens 8i .. 8i+7 (lane L: token 8i + L/8, slot L%8).
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// 8-byte LDS read the compiler does not see: it would otherwise guard it with a wait for every
// LDS-direct load in flight (it cannot tell which ones write the bytes read).  The caller
// waits (lgkmcnt) before using the result.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2_t lds_read_b64_async(uint32_t addr) {
  u32x2_t v;
  asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}

// The in-workgroup merge of gqa_partial_kernel<G, F8, NW > 1>.  Wave w leaves its split's
// normalised partial (G heads x 128 dims, float32, at po + w * po_stride) and its log-sum-exp in
// LDS; then wave w merges heads w, w + NW, ...: lane l takes dims 2l, 2l+1 of all NW partials,
// weights them by exp2(lse - max lse) (a split without tokens has lse -inf and weight 0), and
// writes the gated bf16 output -- the merge kernel's arithmetic, the weights summed in split
// order.  po must not be in use by any wave when this is called (every tile is done).
template <int G, int NW>
__device__ __forceinline__ void merge_in_workgroup(const GqaParams& P, int row, int kvh, int wv,
                                                   int lane, float m, float ltot,
                                                   const f32x4_t (&acc)[8], float* po,
                                                   int po_stride) {
  static_assert(G * kHeadDim * 4 <= 2 * kTile * 256, "a partial fits the wave's K/V buffers");
  __shared__ float lse_s[NW][16];
  const int l16 = lane & 15, g4 = lane >> 4;
  if (l16 < G) {
    const float inv = ltot > 0.0f ? P.v_scale / ltot : 0.0f;
    float* mine = po + wv * po_stride + l16 * kHeadDim;
#pragma unroll
    for (int db = 0; db < 8; ++db)
      *reinterpret_cast<float4*>(mine + 16 * db + 4 * g4) =
          make_float4(acc[db][0] * inv, acc[db][1] * inv, acc[db][2] * inv, acc[db][3] * inv);
    if (g4 == 0) lse_s[wv][l16] = ltot > 0.0f ? m + log2f(ltot) : -INFINITY;
  }
  __syncthreads();  // no global loads are in flight here
  for (int h = wv; h < G; h += NW) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, lse_s[w][h]);
    float o0 = 0.0f, o1 = 0.0f;
    const int hq = kvh * G + h;
    if (M != -INFINITY) {
      float wsum = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float ls = lse_s[w][h];
        const float wgt = ls == -INFINITY ? 0.0f : exp2f(ls - M);
        const float2 o =
            *reinterpret_cast<const float2*>(po + w * po_stride + h * kHeadDim + 2 * lane);
        wsum += wgt;
        o0 += wgt * o.x;
        o1 += wgt * o.y;
      }
      const float inv = 1.0f / wsum;
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
}

// One wavefront per (row, KV head, split), ordered by XCD (below).  Both contractions run on
// the matrix cores (v_mfma_f32_16x16x32_bf16), with the G query heads of the KV head padded
// to the 16 columns of the instruction:
//   * Q.K: S^T (tokens x heads) = K (tokens x dims) . Q^T; K fragments are read from the LDS
//     tile, Q^T fragments stay in registers.  Lane l ends up with tokens 16b + 4(l/16) + e,
//     e < 4, of head l % 16;
//   * softmax per head across the 64 lanes' 32 tokens (exp2, P rounded to bf16);
//   * P.V: O^T (dims x heads) += V^T (dims x tokens) . P^T.  P^T's fragment is exactly what
//     each lane holds after the softmax (token k-slot 8(l/16) + j is token 4(l/16) + j for
//     j < 4, else 16 + 4(l/16) + j - 4); V^T's fragments come from the V tile through the
//     transposing LDS read ds_read_b64_tr_b16, whose 16-lane groups return column l % 16 of
//     the 4 x 16 block their 16 eight-byte reads form.
// K and V are gathered with LDS-direct 16-byte loads, 16 lanes per 256-byte row; the next
// tile's K is in flight during the softmax and P.V, its V during Q.K and the softmax.
// With F8 the rows are e4m3 codes (128 bytes each): the fragments are read as bytes and
// converted to bf16 (exactly: every e4m3 value is a bf16 value), V's through the transposing
// byte read ds_read_b64_tr_b8, whose 16-lane groups give lane i byte i % 8 of the reads of
// lanes i / 8 + 2r, r < 8.  The dequantization scales act on the scores and on the output.
//
// NW > 1 (bf16 K/V): a workgroup of NW waves takes one (row, KV head), wave w its split w (the
// plan has at most NW splits); the waves' partials are merged in LDS by the workgroup, with the
// merge kernel's arithmetic, and no merge kernel runs.
template <int G, bool F8, int NW = 1>
__global__ __launch_bounds__(64 * NW) void gqa_partial_kernel(GqaParams P) {
  static_assert(G <= 16, "the MFMA columns hold at most 16 heads");
  static_assert(NW == 1 || !F8, "in-workgroup merging is built for bf16 K/V");
  constexpr int kRow = F8 ? 128 : 256;        // bytes of a token's K (or V) row
  constexpr int kLoads = kTile * kRow / 1024;  // LDS-direct loads per tile and part
  // Workgroup b runs on XCD b mod 8 (round-robin dispatch).  The work order (KV head, row,
  // split) -- (KV head, row) with NW > 1 -- is cut into 8 contiguous chunks, chunk x for XCD x,
  // so that the workgroups one XCD runs at a time share a request: rows of one request
  // (prefill) or the verify rows of one request find the K/V rows they have in common in that
  // XCD's L2.
  const uint32_t total = (uint32_t)P.T * (uint32_t)(P.Hkv * (NW > 1 ? 1 : P.splits));
  const uint32_t chunk = (total + 7u) >> 3;
  const uint32_t wi = (blockIdx.x & 7u) * chunk + (blockIdx.x >> 3);
  if (wi >= total) return;  // the grid is 8 * chunk >= total (workgroup-uniform)
  const int wv = NW > 1 ? (int)(threadIdx.x >> 6) : 0;  // this wave's buffers
  const int split = NW > 1 ? wv : (int)(wi % (uint32_t)P.splits);
  const uint32_t rk = NW > 1 ? wi : wi / (uint32_t)P.splits;
  const int row = (int)(rk % (uint32_t)P.T), kvh = (int)(rk / (uint32_t)P.T);
  if (P.rt_flags != nullptr) {  // rows the row-tiled kernel already wrote
    const int ntiles = P.T / kRT;
    if (row / kRT < ntiles && P.rt_flags[(int64_t)kvh * ntiles + row / kRT] != 0) return;
  }
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
  // Per wave: the K and V tiles (kt, vt: one buffer, so that the merge can reuse it for the
  // wave's partial), the resolved cache rows (16-byte offsets) of the chunk's tiles -- token
  // 4i + q of tile k at offs[k * 32 + 8q + i], so that lane group q's 8 rows are contiguous --
  // and the tiles' validity masks.
  __shared__ __attribute__((aligned(16))) uint8_t kv_s[NW][2 * kTile * kRow];
  __shared__ __attribute__((aligned(16))) uint32_t offs_s[NW][kChunkTiles * kTile];
  __shared__ uint32_t vms_s[NW][kChunkTiles];
  uint8_t* const kt = kv_s[wv];
  uint8_t* const vt = kv_s[wv] + kTile * kRow;
  uint32_t* const offs = offs_s[wv];
  uint32_t* const vms = vms_s[wv];

  // The split's tile range comes from the packed width, so that its first index loads need
  // not wait for the count: the count, the request and the first chunk's entries are read in
  // one round trip.
  int count = P.packed[(int64_t)row * P.p_rs + P.W];
  const int r = P.t2r[row];
  const int tile_lo = split * P.tiles_per_split;
  const int tile_end = min((P.W + kTile - 1) / kTile, tile_lo + P.tiles_per_split);

  const int32_t* sel = P.packed + (int64_t)row * P.p_rs;
  const int32_t* btr = P.bt + (int64_t)(r < 0 || r >= P.R ? 0 : r) * P.bt_stride;
  const char* kvb = reinterpret_cast<const char*>(P.kv);

  // Q^T fragments: head l16 (zero past G), dims 32ks + 8 g4 .. +7.
  bf16x8_t qfr[4];
  {
    const uint4* qrow = reinterpret_cast<const uint4*>(
        P.q + (int64_t)row * P.q_rs + (int64_t)(kvh * G + (l16 < G ? l16 : 0)) * P.q_hs);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 v = qrow[4 * ks + g4];
      if (l16 >= G) v = make_uint4(0, 0, 0, 0);
      qfr[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // Per head (this lane's l16): running max, this lane's share of the normaliser, and the
  // output dims 16 db + 4 g4 + e.
  float m = -INFINITY, lsum = 0.0f;
  f32x4_t acc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Rows of chunk tile k for this lane's loads: tokens 4i + g4, i < 8.
  auto row_offsets = [&](int k, uint32_t (&o)[8]) {
    const uint4* src = reinterpret_cast<const uint4*>(offs + k * kTile + 8 * g4);
    const uint4 x = src[0], y = src[1];
    o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
    o[4] = y.x; o[5] = y.y; o[6] = y.z; o[7] = y.w;
  };
  // One tile's K (part 0) or V (part 1) rows into LDS: kLoads coalesced LDS-direct loads.
  auto issue_rows = [&](int k, int part, uint8_t* dst) {
    if constexpr (F8) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int t = 8 * i + (lane >> 3);
        const uint32_t o = offs[k * kTile + 8 * (t & 3) + (t >> 2)];
        lds_dma16(kvb + (size_t)o * 16 + kRow * part + 16 * ((lane & 7) ^ (t & 7)),
                  dst + 1024 * i);
      }
    } else {
      uint32_t o[8];
      row_offsets(k, o);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = 4 * i + g4;
        lds_dma16(kvb + (size_t)o[i] * 16 + 256 * part + 16 * (l16 ^ (t & 15)),
                  dst + 1024 * i);
      }
    }
  };
  // Eight e4m3 codes (two words, code j in byte j % 4 of word j / 4) as bf16, exactly.
  auto e4m3x8_to_bf16 = [](uint32_t w0, uint32_t w1) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false);
    const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
    bf16x8_t r;
    r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)b[0]; r[3] = (__bf16)b[1];
    r[4] = (__bf16)c[0]; r[5] = (__bf16)c[1]; r[6] = (__bf16)d[0]; r[7] = (__bf16)d[1];
    return r;
  };

  for (int c0 = tile_lo; c0 < tile_end; c0 += kChunkTiles) {
    // ---- resolve the chunk's entries to cache rows: all index loads, then all block-table
    // loads, in flight together.  The loads are unconditional, at clamped addresses (the
    // row's W entries and the block table's first column exist).  Invalid entries (negative,
    // past the block table, page out of range, past the count) read the first row and are
    // masked.  Lane l resolves entries l, l+64, l+128, l+192 of the chunk.
    int idx[4], page[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) idx[j] = sel[min(c0 * kTile + lane + 64 * j, P.W - 1)];
    asm volatile("" : "+v"(idx[0]), "+v"(idx[1]), "+v"(idx[2]), "+v"(idx[3]));
    if (c0 == tile_lo) {
      count = count < 0 ? 0 : (count > P.W ? P.W : count);
      if (r < 0 || r >= P.R) count = 0;
    }
    const int nt = min(kChunkTiles, min(tile_end, (count + kTile - 1) / kTile) - c0);
    if (nt <= 0) break;  // wave-uniform
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = c0 * kTile + lane + 64 * j;
      if (e >= count || idx[j] < 0) idx[j] = -1;
      const int col = idx[j] >= 0 ? idx[j] / P.P : 0;
      page[j] = btr[min(col, P.bt_width - 1)];
    }
    asm volatile("" : "+v"(page[0]), "+v"(page[1]), "+v"(page[2]), "+v"(page[3]));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = idx[j] >= 0 ? idx[j] / P.P : P.bt_width;
      const bool valid = col < P.bt_width && page[j] >= 0 && page[j] < P.pages;
      const int slot = idx[j] - col * P.P;
      const int64_t off = valid ? ((int64_t)page[j] * P.kv_ps + (int64_t)kvh * P.kv_hs +
                                   (int64_t)slot * P.kv_ts) : 0;
      const int e = lane + 64 * j, k = e >> 5, t = e & 31;
      offs[k * kTile + 8 * (t & 3) + (t >> 2)] = (uint32_t)(off >> 4);
      const uint64_t vm = __ballot(valid);
      if (lane == 0) {
        vms[2 * j] = (uint32_t)vm;
        vms[2 * j + 1] = (uint32_t)(vm >> 32);
      }
    }
    wave_lds_sync();
    issue_rows(0, 0, kt);

    // One tile: its V loads are issued first and land during Q.K and the softmax; its K rows
    // were loaded during the previous tile.  With MORE it loads the next tile's K once Q.K is
    // done and its V once P.V is done.  The last tile of a chunk is a separate instance, so
    // that every path into a tile has exactly the tile's K loads in flight before its V loads
    // (which lets the waits below be exact).
    auto tile = [&](int k, auto more_tag) {
      constexpr bool more = decltype(more_tag)::value;
      if (k == 0) {
        asm volatile("" ::: "memory");  // V loads strictly after the K loads
        issue_rows(0, 1, vt);
      }
      // The kLoads V loads of this tile are the only memory loads issued after its K loads.
      if constexpr (F8) __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4): K rows have landed
      else __builtin_amdgcn_s_waitcnt(0x0F78);               // vmcnt(8)
      wave_lds_sync();

      // ---- Q.K on the matrix cores: token blocks b = 0, 1 of 16.
      f32x4_t sacc[2];
      u32x2_t kw[2][4];  // fp8: the K fragments' codes, all read before the first is used
      if constexpr (F8) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const int t = 16 * bb + l16;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)  // dims 32 ks + 8 g4 .. +7: chunk 2 ks + g4/2, half
            kw[bb][ks] = lds_read_b64_async(
                lds_u32(kt + t * 128 + 16 * ((2 * ks + (g4 >> 1)) ^ (t & 7)) + 8 * (g4 & 1)));
        }
        // The wait names every fragment, so nothing that reads them can move above it.
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(kw[0][0]), "+v"(kw[0][1]), "+v"(kw[0][2]), "+v"(kw[0][3]),
                       "+v"(kw[1][0]), "+v"(kw[1][1]), "+v"(kw[1][2]), "+v"(kw[1][3])
                     :
                     : "memory");
      }
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        sacc[bb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        const int t = 16 * bb + l16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          bf16x8_t kf;
          if constexpr (F8) {
            kf = e4m3x8_to_bf16(kw[bb][ks][0], kw[bb][ks][1]);
          } else {
            kf = *reinterpret_cast<const bf16x8_t*>(
                kt + t * 256 + 16 * ((4 * ks + g4) ^ (t & 15)));
          }
          sacc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qfr[ks], sacc[bb], 0, 0, 0);
        }
      }
      // Every K read has returned before the next tile's rows overwrite the tile.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if constexpr (more) issue_rows(k + 1, 0, kt);

      // ---- online softmax (base 2) for head l16; P rounded to bf16 as the reference does
      // before P.V.  A masked token's score is never used, so its (possibly poisoned) K needs
      // no zeroing.
      const uint32_t vmask = vms[k];
      float z[8];
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * bb + 4 * g4 + e;
          z[4 * bb + e] = ((vmask >> t) & 1u) ? sacc[bb][e] * P.scale_log2 : -INFINITY;
        }
      }
      float tmax = z[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, z[i]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
      const float mn = fmaxf(m, tmax);
      // exp2 of arguments <= 0 (hardware v_exp_f32; results below 2^-126 flush to zero, far
      // below the bf16 rounding of P), P rounded to bf16 by v_cvt_pk_bf16_f32 (RNE).
      float alpha = 1.0f;
      bf16x8_t pfr;
      float psum = 0.0f;
      if (mn != -INFINITY) {
        alpha = __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pfr[i] = (__bf16)__builtin_amdgcn_exp2f(z[i] - mn);
          psum += (float)pfr[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) pfr[i] = (__bf16)0.0f;
      }
      m = mn;
      lsum = lsum * alpha + psum;
      // Rescale the accumulators only when some head's max moved (wave-uniform test).
      if (__ballot(alpha != 1.0f) != 0ull) {
#pragma unroll
        for (int db = 0; db < 8; ++db) acc[db] *= alpha;
      }

      // This tile's V has landed (only the next tile's K loads may still be in flight).
      if constexpr (more) {
        if constexpr (F8) __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
        else __builtin_amdgcn_s_waitcnt(0x0F78);               // vmcnt(8)
      } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);                    // vmcnt(0)
      }
      // A masked token's V row may hold anything (NaN-poisoned slots included): zero it.
      if (vmask != 0xFFFFFFFFu) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
          const int t = F8 ? 8 * i + (lane >> 3) : 4 * i + g4;
          if (!((vmask >> t) & 1u))
            *reinterpret_cast<uint4*>(vt + t * kRow + 16 * (F8 ? (lane & 7) : l16)) =
                make_uint4(0, 0, 0, 0);
        }
      }
      wave_lds_sync();

      // ---- P.V on the matrix cores: dim blocks db of 16.  Transposing reads: lane (g4, l16)
      // supplies the 8 bytes of token 4 g4 + l16/4 (then 16 + that), dims 16 db + 4 (l16 % 4)
      // .. +3, and receives dim 16 db + l16 of the group's 4 tokens.
      if constexpr (F8) {
        // Lane (g4, l16) supplies the 8 bytes of token T(l16 / 2), dims 16 db + 8 (l16 & 1)
        // .. +7, where T(j) is the k-slot j token of group g4 (4 g4 + j, then 16 + 4 g4 + j-4);
        // it receives dim 16 db + l16 of the group's 8 tokens, in k-slot order.
        const int jj = l16 >> 1;
        const int tr = jj < 4 ? 4 * g4 + jj : 16 + 4 * g4 + (jj - 4);
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const uint32_t a = lds_u32(vt + tr * 128 + 16 * (db ^ (tr & 7)) + 8 * (l16 & 1));
          typedef int i32x2_t __attribute__((ext_vector_type(2)));
          const i32x2_t w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) i32x2_t*)(uintptr_t)a);
          const bf16x8_t vf = e4m3x8_to_bf16((uint32_t)w[0], (uint32_t)w[1]);
          acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pfr, acc[db], 0, 0, 0);
        }
      } else {
        const int tr_t0 = 4 * g4 + (l16 >> 2), tr_t1 = tr_t0 + 16, q4 = l16 & 3;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const int c = 2 * db + (q4 >> 1), h8 = 8 * (q4 & 1);
          const uint32_t a0 = lds_u32(vt + tr_t0 * 256 + 16 * (c ^ (tr_t0 & 15)) + h8);
          const uint32_t a1 = lds_u32(vt + tr_t1 * 256 + 16 * (c ^ (tr_t1 & 15)) + h8);
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(uintptr_t)a0);
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(uintptr_t)a1);
          const bf16x8_t vf = __builtin_bit_cast(
              bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pfr, acc[db], 0, 0, 0);
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // V reads done: the tile is free
      if constexpr (more) {
        asm volatile("" ::: "memory");  // next V loads strictly after the next K loads
        issue_rows(k + 1, 1, vt);
      }
    };
    for (int k = 0; k + 1 < nt; ++k) tile(k, std::true_type{});
    tile(nt - 1, std::false_type{});
    // The chunk's last tile issued no loads; the next chunk overwrites offs after this.
    wave_lds_sync();
  }

  // ---- epilogue: lanes with l16 < G hold head l16, dims 16 db + 4 g4 + e.
  const float ltot = lsum + __shfl_xor(lsum, 16, kWave) + __shfl_xor(lsum, 32, kWave) +
                     __shfl_xor(__shfl_xor(lsum, 16, kWave), 32, kWave);
  if constexpr (NW > 1) {
    merge_in_workgroup<G, NW>(P, row, kvh, wv, lane, m, ltot, acc,
                              reinterpret_cast<float*>(kv_s), 2 * kTile * kRow / 4);
    return;
  }
  if (l16 >= G) return;
  const int hq = kvh * G + l16;
  const float inv = ltot > 0.0f ? P.v_scale / ltot : 0.0f;
  if (P.splits == 1) {
    // Gate and output rows are only 4-byte aligned: dword accesses.
    const uint32_t* gp = P.gate ? reinterpret_cast<const uint32_t*>(
                                      P.gate + (int64_t)row * P.g_rs + (int64_t)hq * P.g_hs)
                                : nullptr;
    uint32_t* op = reinterpret_cast<uint32_t*>(P.out + (int64_t)row * P.o_rs +
                                               (int64_t)hq * P.o_hs);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = acc[db][e] * inv;
      const int d0 = 16 * db + 4 * g4;
      if (gp) {
        const uint32_t g01 = gp[d0 / 2], g23 = gp[d0 / 2 + 1];
        o[0] *= sigmoidf(bf16lo(g01));
        o[1] *= sigmoidf(bf16hi(g01));
        o[2] *= sigmoidf(bf16lo(g23));
        o[3] *= sigmoidf(bf16hi(g23));
      }
      op[d0 / 2] = (f32_to_bf16(o[0]) & 0xFFFFu) | (f32_to_bf16(o[1]) << 16);
      op[d0 / 2 + 1] = (f32_to_bf16(o[2]) & 0xFFFFu) | (f32_to_bf16(o[3]) << 16);
    }
  } else {
    const int64_t pi = ((int64_t)split * P.T + row) * P.Hq + hq;
    float4* dst = reinterpret_cast<float4*>(P.part_o + pi * kHeadDim);
#pragma unroll
    for (int db = 0; db < 8; ++db)
      dst[4 * db + g4] = make_float4(acc[db][0] * inv, acc[db][1] * inv, acc[db][2] * inv,
                                     acc[db][3] * inv);
    if (g4 == 0) P.part_lse[pi] = ltot > 0.0f ? m + log2f(ltot) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------------------------
// Row-tiled attention for long prefill chunks (bf16 K/V, G = 8; opt-in: row_tiles = 1).
// Workgroup (tile, KV head)
// takes the kRT = 32 rows tile * 32 .. +31 when they all belong to one request.  Every row's
// selection is a set of that request's tokens, and nearby rows together select most of them,
// so instead of gathering each row's tokens on its own the workgroup walks the request's
// 32-token windows that any of its rows selected, in ascending order, loads each window's K
// and V once into LDS, and scores it against all 32 x 8 queries, each (row, token) pair the row
// did not select masked out of the softmax.  A window is a contiguous run of tokens (whole
// 16-token pages), so its K/V rows come in 8 KiB contiguous blocks.
//   * Row masks: a bit per (row, token) over a span of kRTSpan tokens in LDS (64 KiB), built
//     from the rows' packed entries (negative entries, entries past the count or the block
//     table are left out, as in the per-row kernel); a row that lists a token twice would need
//     it counted twice, so such a tile is left to the per-row kernel (flag 0).
//   * Waves: wave w holds rows 4w .. 4w+3 as two MFMA column blocks (2 rows x 8 heads each),
//     their Q^T fragments in registers; K fragments and (transposed) V fragments of a window are
//     read once and serve both blocks.  Three window buffers keep two windows in flight.
//   * Softmax per query as in the per-row kernel (base 2, P rounded to bf16).  V elements of
//     tokens that no row selected (slots past the request, unwritten slots, pages outside the
//     cache) are zeroed in the fragments: P is 0 there, but 0 x NaN would not be.
// The flag [kvh][tile] says whether this kernel wrote the tile's outputs; the per-row kernel
// runs after it and takes the rows of every tile it did not.
constexpr int kRTSpan = 16384;               // tokens whose row masks are held at a time
constexpr int kRTWords = kRTSpan / 32;
constexpr int kRTBt = kRTSpan / 16 + 2;      // block-table entries of a span (pages >= 16)
constexpr int kRTMinRows = 2048;             // calls with at least this many rows use it

template <int G>
__global__ __launch_bounds__(512) void gqa_rowtile_kernel(GqaParams P) {
  static_assert(G == 8, "a column block is two rows of eight heads");
  __shared__ uint32_t bits[kRT][kRTWords];                                  // 64 KiB
  __shared__ __attribute__((aligned(16))) uint8_t kvt[3][2][kTile * 256];  // 48 KiB
  __shared__ int32_t bt_s[kRTBt];
  __shared__ __attribute__((aligned(4))) uint16_t wlist[kRTWords];  // active windows, ascending
  __shared__ uint32_t wany[kRTWords];     // per active window: tokens some row selected
  __shared__ int s_cnt[kRT];
  __shared__ int s_int[8];
  __shared__ int s_wsum[8];

  const int tile = blockIdx.x, kvh = blockIdx.y;
  const int ntiles = P.T / kRT;
  const int row0 = tile * kRT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, g4 = lane >> 4;
  int32_t* flag = P.rt_flags + (int64_t)kvh * ntiles + tile;

  // ---- the tile's request (all 32 rows must share it) and the rows' counts
  if (tid < kRT) {
    const int row = row0 + tid;
    s_cnt[tid] = min(max(P.packed[(int64_t)row * P.p_rs + P.W], 0), P.W);
    if (tid == 0) s_int[0] = P.t2r[row];
  }
  __syncthreads();
  {
    const int r0 = s_int[0];
    int bad = 0;
    if (tid < kRT) bad = (P.t2r[row0 + tid] != r0) || r0 < 0 || r0 >= P.R;
    if (__syncthreads_or(bad)) {
      if (tid == 0) *flag = 0;
      return;
    }
  }
  const int r = s_int[0];
  const int32_t* btr = P.bt + (int64_t)r * P.bt_stride;
  const int64_t tok_lim = (int64_t)P.bt_width * P.P;  // entries at or past this are masked
  const char* kvb = reinterpret_cast<const char*>(P.kv);

  // ---- Q^T fragments of the wave's two column blocks: column l16 is row 4w + 2i + l16/8,
  // head kvh * 8 + l16 % 8; dims 32 ks + 8 g4 .. +7.
  bf16x8_t qfr[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = row0 + 4 * w + 2 * i + (l16 >> 3);
    const uint4* qrow = reinterpret_cast<const uint4*>(
        P.q + (int64_t)row * P.q_rs + (int64_t)(kvh * G + (l16 & 7)) * P.q_hs);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qfr[i][ks] = __builtin_bit_cast(bf16x8_t, qrow[4 * ks + g4]);
  }
  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.0f, 0.0f};
  f32x4_t acc[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[i][db] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // The row of this thread's entry scan: 16 threads per row.
  const int srow = tid >> 4, ssub = tid & 15;
  const int32_t* sent = P.packed + (int64_t)(row0 + srow) * P.p_rs;
  const int scnt = s_cnt[srow];

  for (int64_t s0 = 0;; s0 += kRTSpan) {
    // ---- row masks of span [s0, s0 + kRTSpan): clear, then set a bit per entry
    for (int i = tid; i < kRT * kRTWords; i += 512) (&bits[0][0])[i] = 0u;
    if (tid == 0) { s_int[1] = 0; s_int[2] = 0; s_int[3] = 0; }
    __syncthreads();
    int more = 0, dup = 0;
    for (int e0 = 0; e0 < scnt; e0 += 128) {  // eight entries per thread in flight
      int x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = e0 + ssub + 16 * j;
        x[j] = e < scnt ? sent[e] : -1;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (x[j] < 0 || (int64_t)x[j] >= tok_lim || (int64_t)x[j] < s0) continue;
        if ((int64_t)x[j] >= s0 + kRTSpan) { more = 1; continue; }
        const int o = (int)((int64_t)x[j] - s0);
        const uint32_t bit = 1u << (o & 31);
        const uint32_t old = atomicOr(&bits[srow][o >> 5], bit);
        dup |= (old & bit) != 0u;
      }
    }
    if (more) s_int[2] = 1;
    if (dup) s_int[3] = 1;
    __syncthreads();
    if (s_int[3]) {  // a row lists a token twice: leave the tile to the per-row kernel
      if (tid == 0) *flag = 0;
      return;
    }
    const bool more_spans = s_int[2] != 0;
    // ---- active windows (ascending, by a workgroup scan) and the span's block-table slice
    {
      const int wi = tid;  // kRTWords == 512 words: one per thread
      uint32_t any = 0u;
#pragma unroll 8
      for (int rr = 0; rr < kRT; ++rr) any |= bits[rr][wi];
      const int act = any != 0u;
      const uint64_t bal = __ballot(act);
      const int before = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) s_wsum[w] = __builtin_popcountll(bal);
      __syncthreads();
      int off = before;
      for (int i = 0; i < w; ++i) off += s_wsum[i];
      if (act) {
        wlist[off] = (uint16_t)wi;
        wany[off] = any;
      }
      if (tid == 511) s_int[4] = off + act;
    }
    const int col0 = (int)(s0 / P.P);
    for (int c = tid; c < kRTBt; c += 512) {
      const int col = col0 + c;
      bt_s[c] = col < P.bt_width ? btr[col] : -1;
    }
    __syncthreads();
    const int nwin = s_int[4];

    // Loads of window list entry k into buffer k % 3: wave w fetches tokens 4w .. 4w+3 (K,
    // then V), 16 lanes per 256-byte row, chunk c into slot c ^ (t & 15).  A token whose page is
    // not in the cache loads the cache's first row (masked below).
    // LDS words read with inline assembly inside the window loop: a plain read would make the
    // compiler wait for every LDS-direct load in flight (two windows' worth).
    auto lds_word = [](const void* p) {
      uint32_t v;
      asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_u32(p))
                   : "memory");
      return v;
    };
    auto win_of = [&](int k) {
      const uint32_t v = lds_word(&wlist[k & ~1]);  // two 16-bit entries per word
      return (int)((k & 1) ? (v >> 16) : (v & 0xFFFFu));
    };
    auto issue = [&](int k) {
      const int t = 4 * w + g4;
      const int64_t tok = s0 + (int64_t)win_of(k) * 32 + t;
      const int c = (int)(tok / P.P) - col0;
      const int page = (int)lds_word(&bt_s[c]);
      const bool ok = tok < tok_lim && page >= 0 && page < P.pages;
      const int64_t off = ok ? ((int64_t)page * P.kv_ps + (int64_t)kvh * P.kv_hs +
                                (int64_t)(tok - (int64_t)(tok / P.P) * P.P) * P.kv_ts) : 0;
      uint8_t* dst = kvt[k % 3][0] + 1024 * w;
      const char* src = kvb + off + 16 * (l16 ^ (t & 15));
      lds_dma16(src, dst);
      lds_dma16(src + 256, dst + kTile * 256);
    };
    if (nwin > 0) issue(0);
    if (nwin > 1) issue(1);
    for (int k = 0; k < nwin; ++k) {
      // Window k's two loads have landed once only window k+1's may be in flight.
      if (k + 1 < nwin) __builtin_amdgcn_s_waitcnt(0x0F72);  // vmcnt(2)
      else __builtin_amdgcn_s_waitcnt(0x0F70);                // vmcnt(0)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();  // window k visible; window k-1's buffer is free
      asm volatile("" ::: "memory");
      if (k + 2 < nwin) issue(k + 2);
      const uint8_t* kt = kvt[k % 3][0];
      const uint8_t* vt = kvt[k % 3][1];
      const int wi = win_of(k);
      // Tokens of the window with a page in the cache (lane l < 32: token l), and the row masks
      // of this lane's two query columns.
      uint32_t valid;
      {
        const int64_t tok = s0 + (int64_t)wi * 32 + (lane & 31);
        const int page = (int)lds_word(&bt_s[(int)(tok / P.P) - col0]);
        valid = (uint32_t)__ballot(tok < tok_lim && page >= 0 && page < P.pages);
      }
      uint32_t rm[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) rm[i] = lds_word(&bits[4 * w + 2 * i + (l16 >> 3)][wi]) & valid;
      const uint32_t anyv = lds_word(&wany[k]) & valid;

      // ---- fragments: K (token blocks bb = 0, 1 of 16, k-steps ks) and, read behind them,
      // V^T through the transposing read (lane (g4, l16) receives dim 16 db + l16 of tokens
      // 4 g4 + j, then 16 + 4 g4 + j, j < 4).
      bf16x8_t kf[2][4];
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const int t = 16 * bb + l16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          asm volatile("ds_read_b128 %0, %1" : "=v"(kf[bb][ks])
                       : "v"(lds_u32(kt + t * 256 + 16 * ((4 * ks + g4) ^ (t & 15)))));
      }
      i16x4_t vlo[8], vhi[8];
      {
        const int tr_t0 = 4 * g4 + (l16 >> 2), tr_t1 = tr_t0 + 16, q4 = l16 & 3;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const int cc = 2 * db + (q4 >> 1), h8 = 8 * (q4 & 1);
          asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(vlo[db])
                       : "v"(lds_u32(vt + tr_t0 * 256 + 16 * (cc ^ (tr_t0 & 15)) + h8)));
          asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(vhi[db])
                       : "v"(lds_u32(vt + tr_t1 * 256 + 16 * (cc ^ (tr_t1 & 15)) + h8)));
        }
      }
      // The K fragments first (the V reads, issued later, complete in order behind them).
      asm volatile("s_waitcnt lgkmcnt(8)" : "+v"(kf[0][0]), "+v"(kf[0][1]), "+v"(kf[0][2]),
                   "+v"(kf[0][3]), "+v"(kf[1][0]), "+v"(kf[1][1]), "+v"(kf[1][2]),
                   "+v"(kf[1][3]));

      // ---- S^T = K . Q^T for both column blocks
      f32x4_t sacc[2][2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          sacc[i][bb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            sacc[i][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[bb][ks], qfr[i][ks],
                                                                   sacc[i][bb], 0, 0, 0);
        }
      // ---- online softmax per query column; P rounded to bf16
      bf16x8_t pfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float z[8];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 16 * bb + 4 * g4 + e;
            z[4 * bb + e] = ((rm[i] >> t) & 1u) ? sacc[i][bb][e] * P.scale_log2 : -INFINITY;
          }
        float tmax = z[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, z[j]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
        const float mn = fmaxf(m[i], tmax);
        float alpha = 1.0f, psum = 0.0f;
        if (mn != -INFINITY) {
          alpha = __builtin_amdgcn_exp2f(m[i] - mn);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            pfr[i][j] = (__bf16)__builtin_amdgcn_exp2f(z[j] - mn);
            psum += (float)pfr[i][j];
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) pfr[i][j] = (__bf16)0.0f;
        }
        m[i] = mn;
        lsum[i] = lsum[i] * alpha + psum;
        if (__ballot(alpha != 1.0f) != 0ull) {
#pragma unroll
          for (int db = 0; db < 8; ++db) acc[i][db] *= alpha;
        }
      }
      // ---- O^T += V^T . P^T for both blocks; V elements of unselected tokens zeroed.  Lane
      // (g4, l16) receives dim 16 db + l16 of tokens 4 g4 + j (lo) and 16 + 4 g4 + j (hi).
      const uint32_t zlo = anyv >> (4 * g4), zhi = anyv >> (16 + 4 * g4);
      const uint32_t mlo0 = ((zlo & 1u) ? 0xFFFFu : 0u) | ((zlo & 2u) ? 0xFFFF0000u : 0u);
      const uint32_t mlo1 = ((zlo & 4u) ? 0xFFFFu : 0u) | ((zlo & 8u) ? 0xFFFF0000u : 0u);
      const uint32_t mhi0 = ((zhi & 1u) ? 0xFFFFu : 0u) | ((zhi & 2u) ? 0xFFFF0000u : 0u);
      const uint32_t mhi1 = ((zhi & 4u) ? 0xFFFFu : 0u) | ((zhi & 8u) ? 0xFFFF0000u : 0u);
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(vlo[0]), "+v"(vlo[1]), "+v"(vlo[2]),
                   "+v"(vlo[3]), "+v"(vlo[4]), "+v"(vlo[5]), "+v"(vlo[6]), "+v"(vlo[7]),
                   "+v"(vhi[0]), "+v"(vhi[1]), "+v"(vhi[2]), "+v"(vhi[3]), "+v"(vhi[4]),
                   "+v"(vhi[5]), "+v"(vhi[6]), "+v"(vhi[7]));
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));
        u32x4v_t u = __builtin_bit_cast(
            u32x4v_t, __builtin_shufflevector(vlo[db], vhi[db], 0, 1, 2, 3, 4, 5, 6, 7));
        u[0] &= mlo0;
        u[1] &= mlo1;
        u[2] &= mhi0;
        u[3] &= mhi1;
        const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, u);
#pragma unroll
        for (int i = 0; i < 2; ++i)
          acc[i][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pfr[i], acc[i][db], 0, 0, 0);
      }
    }
    if (!more_spans) break;
    __syncthreads();  // every wave is done with the span's masks and windows
  }

  // ---- epilogue: lane (g4, l16) of block i holds dims 16 db + 4 g4 + e of row
  // 4w + 2i + l16 / 8, head l16 % 8.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float ltot = lsum[i] + __shfl_xor(lsum[i], 16, kWave) +
                       __shfl_xor(lsum[i], 32, kWave) +
                       __shfl_xor(__shfl_xor(lsum[i], 16, kWave), 32, kWave);
    const int row = row0 + 4 * w + 2 * i + (l16 >> 3);
    const int hq = kvh * G + (l16 & 7);
    const float inv = ltot > 0.0f ? P.v_scale / ltot : 0.0f;
    const uint32_t* gp = P.gate ? reinterpret_cast<const uint32_t*>(
                                      P.gate + (int64_t)row * P.g_rs + (int64_t)hq * P.g_hs)
                                : nullptr;
    uint32_t* op =
        reinterpret_cast<uint32_t*>(P.out + (int64_t)row * P.o_rs + (int64_t)hq * P.o_hs);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = acc[i][db][e] * inv;
      const int d0 = 16 * db + 4 * g4;
      if (gp) {
        const uint32_t g01 = gp[d0 / 2], g23 = gp[d0 / 2 + 1];
        o[0] *= sigmoidf(bf16lo(g01));
        o[1] *= sigmoidf(bf16hi(g01));
        o[2] *= sigmoidf(bf16lo(g23));
        o[3] *= sigmoidf(bf16hi(g23));
      }
      op[d0 / 2] = (f32_to_bf16(o[0]) & 0xFFFFu) | (f32_to_bf16(o[1]) << 16);
      op[d0 / 2 + 1] = (f32_to_bf16(o[2]) & 0xFFFFu) | (f32_to_bf16(o[3]) << 16);
    }
  }
  if (tid == 0) *flag = 1;
}

// Grid (T, Hq), one wavefront.  Lane s reads split s's log-sum-exp while every lane already
// loads dims 2l, 2l+1 of all splits' partials (one round trip for both); the weights are formed
// in-wave, then the partials are combined.  splits <= kMergeMax.
constexpr int kMergeMax = 64;
__global__ __launch_bounds__(64) void gqa_merge_kernel(GqaParams P) {
  const int row = blockIdx.x, hq = blockIdx.y, lane = threadIdx.x;
  const int64_t stride = (int64_t)P.T * P.Hq;   // between splits
  const int64_t pi0 = (int64_t)row * P.Hq + hq;
  const float lse = lane < P.splits ? P.part_lse[lane * stride + pi0] : -INFINITY;
  constexpr int kBatch = 16;
  float o0 = 0.0f, o1 = 0.0f;
  float2 ov[kBatch];
#pragma unroll
  for (int s = 0; s < kBatch; ++s)
    ov[s] = s < P.splits ? reinterpret_cast<const float2*>(P.part_o + (s * stride + pi0) * kHeadDim)[lane]
                         : make_float2(0.0f, 0.0f);
  const float M = wave_max(lse);
  if (M != -INFINITY) {
    const float wgt = lse == -INFINITY ? 0.0f : exp2f(lse - M);
    const float inv = 1.0f / wave_sum(wgt);
#pragma unroll
    for (int s = 0; s < kBatch; ++s) {
      const float ws = __shfl(wgt, s, kWave);
      o0 += ws * ov[s].x;
      o1 += ws * ov[s].y;
    }
    for (int s = kBatch; s < P.splits; ++s) {
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
hipError_t launch_partial(const GqaParams& P, bool f8, bool in_wg, hipStream_t s) {
  // A 1-D grid of 8 * ceil(T * Hkv * splits / 8) workgroups (in-workgroup merge: 8 *
  // ceil(T * Hkv / 8) workgroups of kMergeWaves waves), mapped onto the work by XCD.
  const uint64_t total = (uint64_t)P.T * P.Hkv * (in_wg ? 1 : P.splits);
  if (total > 0xFFFFFFF0ull) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((total + 7) / 8 * 8));
  if (in_wg) {
    hipLaunchKernelGGL((gqa_partial_kernel<G, false, kMergeWaves>), grid, dim3(64 * kMergeWaves),
                       0, s, P);
    return hipGetLastError();
  }
  if (f8)
    hipLaunchKernelGGL((gqa_partial_kernel<G, true>), grid, dim3(64), 0, s, P);
  else
    hipLaunchKernelGGL((gqa_partial_kernel<G, false>), grid, dim3(64), 0, s, P);
  return hipGetLastError();
}

}  // namespace

// Scratch of the allocation-free attention call: the split partials live in this array instead
// of a caller workspace.  Every GPU the library runs on holds its own copy until the process
// ends.  Host code never uses the array's name as an address: the device address of each
// GPU's copy is looked up once with hipGetSymbolAddress and kept per device.
static __device__ __align__(256) uint8_t scratch[kGqaScratchBytes];

hipError_t gqa_scratch(char** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (per_device[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *ptr = static_cast<char*>(per_device[dev]);
  return hipSuccess;
}

GqaPlan gqa_plan(const qsa_gqa_args& a) {
  GqaPlan p{};
  p.tiles = (a.packed_width + kTile - 1) / kTile;
  if (p.tiles < 1) p.tiles = 1;
  int target = a.num_splits;
  const bool bf16 = a.kv_dtype != QSA_DTYPE_FP8_E4M3;
  const int64_t units = (int64_t)a.num_tokens * a.num_kv_heads;  // (row, KV head) pairs
  bool in_wg = bf16 && target > 1 && target <= kMergeWaves;      // forced: 2..8 splits
  if (target <= 0) {
    // Workgroups to aim for, measured on the decode workloads: with bf16 K/V about 768 (three
    // per CU), each split then gathering ~11 tiles of 16 KiB, so that its two dependent
    // round trips before the first gather are amortised; with fp8 K/V (half the bytes per
    // token) about 2048.  More waves than that queue behind the HBM without adding bandwidth.
    const int64_t want = bf16 ? 768 : 2048;
    target = units >= want ? 1 : (int)((want + units - 1) / units);
    // bf16 K/V with 128..256 units: one workgroup of 8 waves per unit, one split per wave,
    // merged in the workgroup (no partials in memory, no merge kernel).  Measured against the
    // split-K plan above on decode batches of 32k-token requests: 128 units 35.9 -> 35.5 us,
    // 192 units 49.5 -> 43.2 us, 256 units (fp8 indexer) 59.5 -> 56.2 us; with fewer units
    // the chip is too empty (64 units: 20.2 -> 28.6 us), with more the workgroups (one per CU:
    // their K/V buffers take 137 KiB of LDS) no longer fit in one round (320 units: 72 -> 84).
    in_wg = bf16 && units >= 128 && units <= 256 && target > 1;
    if (in_wg) target = kMergeWaves;
  }
  if (target > p.tiles) target = p.tiles;
  if (target > kMergeMax) target = kMergeMax;  // the merge reads one split per lane
  p.tiles_per_split = (p.tiles + target - 1) / target;
  p.splits = (p.tiles + p.tiles_per_split - 1) / p.tiles_per_split;
  p.merge_in_wg = in_wg && p.splits > 1;
  p.ws_bytes = 0;
  if (p.splits > 1 && !p.merge_in_wg) {
    const size_t n = (size_t)p.splits * a.num_tokens * a.num_q_heads;
    p.ws_bytes = (n * kHeadDim * sizeof(float) + 255) / 256 * 256 + n * sizeof(float);
  }
  // Row tiles for large prefill calls (bf16 K/V, eight query heads per KV head, one split):
  // a flag per (KV head, tile) after everything else.
  p.row_tiles = 0;
  if (a.row_tiles == 1 && a.kv_dtype == QSA_DTYPE_BF16 && a.num_q_heads == 8 * a.num_kv_heads &&
      p.splits == 1 && a.num_tokens >= kRTMinRows) {
    p.row_tiles = a.num_tokens / kRT;
    p.ws_bytes = (p.ws_bytes + 255) / 256 * 256 +
                 (size_t)p.row_tiles * a.num_kv_heads * sizeof(int32_t);
  }
  return p;
}

hipError_t launch_gqa(const qsa_gqa_args& a, const GqaPlan& plan, char* ws, hipStream_t s,
                      Phase phase) {
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
  const bool f8 = a.kv_dtype == QSA_DTYPE_FP8_E4M3;
  const int64_t elt = f8 ? 1 : 2;
  P.kv = reinterpret_cast<const uint8_t*>(a.kv_cache);
  P.kv_ps = a.kv_page_stride * elt;
  P.kv_hs = a.kv_head_stride * elt;
  P.kv_ts = a.kv_token_stride * elt;
  P.bt = a.block_table;
  P.t2r = a.token_to_req;
  P.packed = a.packed;
  P.p_rs = a.packed_row_stride;
  P.gate = a.gate;
  P.g_rs = a.gate_row_stride;
  P.g_hs = a.gate_head_stride;
  const float scale = a.scale > 0.0f ? a.scale : 1.0f / sqrtf((float)a.head_dim);
  // fp8: K = code * k_scale enters every score once, V = code * v_scale the output once.
  const float k_scale = f8 && a.k_scale > 0.0f ? a.k_scale : 1.0f;
  P.scale_log2 = scale * k_scale * 1.4426950408889634f;
  P.v_scale = f8 && a.v_scale > 0.0f ? a.v_scale : 1.0f;
  P.out = a.out;
  P.o_rs = a.out_row_stride;
  P.o_hs = a.out_head_stride;
  size_t used = 0;
  if (plan.splits > 1 && !plan.merge_in_wg) {
    const size_t n = (size_t)plan.splits * a.num_tokens * a.num_q_heads;
    P.part_o = reinterpret_cast<float*>(ws);
    P.part_lse = reinterpret_cast<float*>(ws + (n * kHeadDim * sizeof(float) + 255) / 256 * 256);
    used = (n * kHeadDim * sizeof(float) + 255) / 256 * 256 + n * sizeof(float);
  }
  P.rt_flags = plan.row_tiles > 0
                   ? reinterpret_cast<int32_t*>(ws + (used + 255) / 256 * 256)
                   : nullptr;
  hipError_t e = hipSuccess;
  if (phase == Phase::kSecond) {  // the merge alone (nothing to merge with one split)
    if (plan.splits == 1 || plan.merge_in_wg) return hipSuccess;
    hipLaunchKernelGGL(gqa_merge_kernel, dim3(P.T, P.Hq), dim3(64), 0, s, P);
    return hipGetLastError();
  }
  if (plan.row_tiles > 0) {  // every flag is written: 1 where the tile's outputs are done
    hipLaunchKernelGGL(gqa_rowtile_kernel<8>, dim3(plan.row_tiles, P.Hkv), dim3(512), 0, s, P);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: e = launch_partial<1>(P, f8, plan.merge_in_wg, s); break;
    case 2: e = launch_partial<2>(P, f8, plan.merge_in_wg, s); break;
    case 4: e = launch_partial<4>(P, f8, plan.merge_in_wg, s); break;
    case 8: e = launch_partial<8>(P, f8, plan.merge_in_wg, s); break;
    case 16: e = launch_partial<16>(P, f8, plan.merge_in_wg, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || plan.splits == 1 || plan.merge_in_wg || phase == Phase::kFirst) return e;
  hipLaunchKernelGGL(gqa_merge_kernel, dim3(P.T, P.Hq), dim3(64), 0, s, P);
  return hipGetLastError();
}

}  // namespace qsa
