// Wave tiles of the vector-unit indexer logits kernels (logits.hip, logits_list.hip): the lane
// layout of a 64-key tile, its loads, and its scoring against head-folded rows.
#pragma once

#include "select.h"

namespace qsa {
namespace logits_tile {
// Lane layout of a 64-key wave tile.  A key's row is split over kLanes lanes of 16 bytes: 8 for
// fp8 (128-byte rows), 16 for bf16 (256-byte rows), so one wave load instruction reads
// 64 / kLanes consecutive rows -- 1 KiB of contiguous cache -- and a tile takes kLoads
// instructions.  Lane `x = lane % kLanes` of group `g = lane / kLanes` holds, in load `it`, dims
// of key `it * (64 / kLanes) + g`: 16x .. 16x+15 (fp8) or 8x .. 8x+7 (bf16).
template <bool FP8>
struct KeyLanes {
  static constexpr int kLanes = FP8 ? 8 : 16;
  static constexpr int kKeysPerLoad = 64 / kLanes;
  static constexpr int kLoads = 64 / kKeysPerLoad;
  static constexpr int kDims = FP8 ? 16 : 8;  // dims per lane per key
};

// Loads tile `tile` of the workgroup (keys tile*256 + w*64 + 0..63) for this lane.  `rows` holds
// the cache row of each of the workgroup's keys (-1: out of range or not visible; such a key
// reads the cache's first row and is masked when scored).  `okm` bit `it` marks load `it` valid.
template <bool FP8>
__device__ __forceinline__ void load_key_tile(const SelectParams& P, const int32_t* rows,
                                              int tile, int w, int lane,
                                              uint32_t (&raw)[KeyLanes<FP8>::kLoads][4],
                                              uint32_t& okm) {
  using K = KeyLanes<FP8>;
  const char* base = reinterpret_cast<const char*>(P.ckv) + (lane % K::kLanes) * 16;
  const int key0 = tile * kLogitsKeysPerWG + w * 64 + lane / K::kLanes;
  int row[K::kLoads];
#pragma unroll
  for (int it = 0; it < K::kLoads; ++it) row[it] = rows[key0 + it * K::kKeysPerLoad];
  // The mask is applied when the tile is scored: a select here would consume the loaded words
  // at once and make the wave wait for them.
  okm = 0;
#pragma unroll
  for (int it = 0; it < K::kLoads; ++it) {
    okm |= (uint32_t)(row[it] >= 0) << it;
    const uint4 x = *reinterpret_cast<const uint4*>(
        base + (int64_t)max(row[it], 0) * (kHeadDim * (FP8 ? 1 : 2)));
    raw[it][0] = x.x;
    raw[it][1] = x.y;
    raw[it][2] = x.z;
    raw[it][3] = x.w;
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the N lanes (8 or 16, aligned) that share a key, on DPP: swap adjacent lanes, then
// lane pairs, then mirror the quads of each half-row, then (N = 16) the halves of the row.
// Every lane ends with the N-lane sum.
template <int N>
__device__ __forceinline__ float group_sum(float d) {
  d += dpp_f32<0xB1>(d);   // quad_perm [1,0,3,2]
  d += dpp_f32<0x4E>(d);   // quad_perm [2,3,0,1]
  d += dpp_f32<0x141>(d);  // row_half_mirror
  if (N == 16) d += dpp_f32<0x140>(d);  // row_mirror
  return d;
}

// Scores the tile in `raw` against NR folded rows (qf: this lane's dims of each row) and writes
// the logits.  After the group sums, lane x of group g keeps the sum of load it = x, so every
// lane ends with one key -- it*(64/kLanes) + g -- and each row is written with one store.
// Updates the lane's running max |k|.  RELU: the NR "rows" are the heads of one row, and its
// logit is the sum over heads of max(0, head product).
template <bool FP8, int NR, bool RELU = false>
__device__ __forceinline__ void score_key_tile(const SelectParams& P,
                                               const uint32_t (&raw)[KeyLanes<FP8>::kLoads][4],
                                               uint32_t okm, const float (&qf)[NR][16], int nr,
                                               int row0, int j0, int vis_max, int lane,
                                               bool track_kmax, float& kmax) {
  using K = KeyLanes<FP8>;
  const int x = lane % K::kLanes, g = lane / K::kLanes;
  // One-hot weight of load `it` for this lane, as arithmetic: a compare would tie up a scalar
  // register pair per load.
  const uint32_t onehot = 1u << x;
  float res[NR];
#pragma unroll
  for (int rr = 0; rr < NR; ++rr) res[rr] = 0.0f;
#pragma unroll
  for (int it = 0; it < K::kLoads; ++it) {
    float k[16];
    const bool ok = (okm >> it) & 1u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t word = raw[it][i];
      if (FP8) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
        k[4 * i] = lo[0];
        k[4 * i + 1] = lo[1];
        k[4 * i + 2] = hi[0];
        k[4 * i + 3] = hi[1];
      } else {
        k[2 * i] = bf16lo(word);
        k[2 * i + 1] = bf16hi(word);
      }
    }
    // A masked key reads the cache's first row, whatever it holds: its values are dropped by
    // selects (never by arithmetic, which a NaN there would survive).
    if (track_kmax) {
      float m = fabsf(k[0]);
#pragma unroll
      for (int i = 1; i < K::kDims; ++i) m = fmaxf(m, fabsf(k[i]));
      kmax = fmaxf(kmax, ok ? m : 0.0f);
    }
#pragma unroll
    for (int rr = 0; rr < NR; ++rr) {
      float d = 0.0f;
#pragma unroll
      for (int i = 0; i < K::kDims; ++i) d = fmaf(qf[rr][i], k[i], d);
      d = group_sum<K::kLanes>(ok ? d : 0.0f);
      res[rr] = fmaf((float)((onehot >> it) & 1u), d, res[rr]);  // exact: one term is d
    }
  }
  // Unconditional buffer stores: a row's record ends at its visible keys (none for a row past
  // nr), so the hardware drops the rest; lanes x >= kLoads hold no key.
  const int j = j0 + x * K::kKeysPerLoad + g;
  if (RELU) {
    float sum = fmaxf(res[0], 0.0f);
#pragma unroll
    for (int rr = 1; rr < NR; ++rr) sum = sum + fmaxf(res[rr], 0.0f);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        P.logits + (int64_t)row0 * P.col_stride, 0, vis_max * 4, 0x00020000);
    const uint32_t off = x < K::kLoads ? (uint32_t)j * 4u : 0xFFFFFFF0u;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sum), rs, off, 0, 0);
    return;
  }
#pragma unroll
  for (int rr = 0; rr < NR; ++rr) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        P.logits + (int64_t)(rr < nr ? row0 + rr : row0) * P.col_stride, 0,
        rr < nr ? vis_max * 4 : 0, 0x00020000);
    const uint32_t off = x < K::kLoads ? (uint32_t)j * 4u : 0xFFFFFFF0u;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(res[rr]), rs, off, 0, 0);
  }
}

}  // namespace logits_tile
}  // namespace qsa
