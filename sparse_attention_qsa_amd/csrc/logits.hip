// Indexer logits on the vector units (decode and short requests): for every row and compressed
// block, the fast float32 score with the index heads folded into Q, sum_h q[h] . k =
// (sum_h q[h]) . k, written to the logits workspace together with the per-128-key bound of
// max |k| that the top-k's error band needs.  Follows the scoring step of QSAIndexer.forward
// (page "vllm.models.qwen4_exp.nvidia.qsa").
#include "select.h"

namespace qsa {
namespace {
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

// Grid (wg_per_req, R), 256 threads.  Workgroup k of request r scores the request's keys
// 1024k .. 1024k+1023 (4 tiles of 256) against every row of the request, NR rows at a time.
// Eight lanes share a key (16 dims each), so one wave load reads eight compressed rows, 128
// contiguous bytes of each.  The cache row of every key and the head-folded rows are staged in
// LDS once; two tiles are in flight from the start and each reload is issued before the other
// buffer's tile is scored.
// RELU: one row at a time, its NR = 8 heads held unfolded as the scorer's rows.
template <bool FP8, int NR, bool RELU = false>
__global__ __launch_bounds__(kLogitsThreads) __attribute__((amdgpu_waves_per_eu(NR >= 4 ? 2 : 4)))
void logits_valu_kernel(SelectParams P) {
  using KL = KeyLanes<FP8>;
  constexpr int kT = kLogitsThreads, kWaves = kLogitsThreads / 64;
  constexpr int kKeys = kLogitsTilesPerWG * kLogitsKeysPerWG;
  static_assert(kLogitsKeysPerWG == kWaves * 64, "a tile is 64 keys per wave");
  __shared__ int32_t rows_s[kKeys];
  __shared__ float qf_s[NR][kHeadDim];
  __shared__ float red[kWaves];
  const int r = blockIdx.y, k = blockIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int jw = k * kKeys;  // first key of the workgroup
  // Block-table entries of this thread's keys jw + tid + kT i: their addresses do not depend
  // on the request metadata, so they are loaded together with it (one round trip).
  int col[kKeys / kT], page[kKeys / kT];
#pragma unroll
  for (int i = 0; i < kKeys / kT; ++i) {
    col[i] = (jw + (int)threadIdx.x + kT * i) / P.Pc;
    page[i] = P.cbt[(int64_t)r * P.cbt_stride + min(col[i], P.cbt_width - 1)];
  }
  // Row range of the request, clamped into [0, T): the metadata is device data the host never
  // saw, so it is not trusted to stay inside the buffers.
  const int q0 = max(0, min(P.qsl[r], P.T));
  const int n = max(0, min(P.qsl[r + 1], P.T) - q0), L = P.seq_lens[r];
  // The MFMA kernel, which runs next, starts its work queues from zero.
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 8) P.work[threadIdx.x] = 0;
  // Requests with many rows are scored by the MFMA kernel; for them this kernel only takes the
  // per-block bound of max |k| the top-k needs (one pass over their keys).
  const bool kmax_only = n > P.mfma_min_rows;  // block-uniform
  const int vis_max = (n > 0 && n <= L) ? min(L / P.c, P.cols) : 0;
  // Barrier without a memory fence (a fence would wait for every load in flight); the LDS
  // writes before it are complete, and global loads are waited for where their data is used.
  auto barrier = [] {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  float kmax = 0.0f;
  if (jw < vis_max) {  // block-uniform
#pragma unroll
    for (int i = 0; i < kKeys / kT; ++i) {
      const int j = jw + threadIdx.x + kT * i;
      const bool ok = j < vis_max && col[i] < P.cbt_width && page[i] >= 0 && page[i] < P.c_pages;
      rows_s[threadIdx.x + kT * i] = ok ? page[i] * P.Pc + (j - col[i] * P.Pc) : -1;
    }
    if (kmax_only) {
      barrier();  // rows_s written
#pragma unroll
      for (int t = 0; t < kLogitsTilesPerWG; ++t) {
        uint32_t a[KL::kLoads][4], ma;
        load_key_tile<FP8>(P, rows_s, t, w, lane, a, ma);
#pragma unroll
        for (int it = 0; it < KL::kLoads; ++it) {
          float m = 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t word = a[it][i];
            if (FP8) {
              const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
              const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
              m = fmaxf(m, fmaxf(fmaxf(fabsf(lo[0]), fabsf(lo[1])),
                                 fmaxf(fabsf(hi[0]), fabsf(hi[1]))));
            } else {
              m = fmaxf(m, fmaxf(fabsf(bf16lo(word)), fabsf(bf16hi(word))));
            }
          }
          kmax = fmaxf(kmax, ((ma >> it) & 1u) ? m : 0.0f);  // masked keys dropped by a select
        }
      }
    }
    for (int rr0 = 0; rr0 < (kmax_only ? 0 : n); rr0 += (RELU ? 1 : NR)) {
      const int nr = RELU ? NR : min(NR, n - rr0);
      // Head-folded Q of the chunk's rows: each of the first nr*128 threads owns one (row, dim)
      // and loads all its heads at once (clamped to Hi - 1, the extra terms added as zero).
      constexpr int kSlots = (NR * kHeadDim + kT - 1) / kT;
      uint32_t v[kSlots][16];  // raw bf16 / e4m3 codes
#pragma unroll
      for (int sl = 0; sl < kSlots; ++sl) {
        const int e = threadIdx.x + kT * sl;
        const int rr = min(e >> 7, nr - 1), d = e & (kHeadDim - 1);
        const int64_t qb = (int64_t)(q0 + rr0 + (RELU ? 0 : rr)) * P.Hi * kHeadDim + d;
#pragma unroll
        for (int h = 0; h < (RELU ? 1 : 16); ++h) {
          // RELU: slot e holds head rr of the one row (clamped to Hi - 1, zeroed below).
          const int64_t idx = qb + min(RELU ? rr : h, P.Hi - 1) * kHeadDim;
          v[sl][h] = FP8 ? (uint32_t)reinterpret_cast<const uint8_t*>(P.q_idx)[idx]
                         : (uint32_t)reinterpret_cast<const uint16_t*>(P.q_idx)[idx];
        }
      }
      // Q first: issued behind the key burst its words would wait several microseconds in
      // the memory queues, and every wave needs them before it can score (and reload).
#pragma unroll
      for (int sl = 0; sl < kSlots; ++sl) {
        auto dec = [](uint32_t x) {
          return FP8 ? e4m3_to_f32_exact((uint8_t)x) : bf16_to_f32((uint16_t)x);
        };
        float f = dec(v[sl][0]);
        if (RELU) {
          if (((int)threadIdx.x + kT * sl) >> 7 >= P.Hi) f = 0.0f;  // a head past Hi
        } else {
#pragma unroll
          for (int h = 1; h < 16; ++h) f = f + (h < P.Hi ? dec(v[sl][h]) : 0.0f);
        }
        v[sl][0] = __float_as_uint(f);
      }
      if (rr0 > 0) barrier();  // the previous chunk's readers are done with qf_s
#pragma unroll
      for (int sl = 0; sl < kSlots; ++sl) {
        const int e = threadIdx.x + kT * sl;
        if (e < nr * kHeadDim) qf_s[e >> 7][e & (kHeadDim - 1)] = __uint_as_float(v[sl][0]);
      }
      barrier();  // rows_s and qf_s written
      float qf[NR][16];
#pragma unroll
      for (int rr = 0; rr < NR; ++rr) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          qf[rr][i] = (rr < nr && i < KL::kDims)
                          ? qf_s[rr][(lane % KL::kLanes) * KL::kDims + i] : 0.0f;
      }
      const bool first = rr0 == 0;
      const int row0 = q0 + rr0;
      // One tile in flight per wave; the other waves of the SIMD (four per SIMD) cover its
      // latency.  The loop is unrolled, so the compiler's vmcnt waits name exactly the tile.
      uint32_t a[KL::kLoads][4], ma;
#pragma unroll
      for (int t = 0; t < kLogitsTilesPerWG; ++t) {
        load_key_tile<FP8>(P, rows_s, t, w, lane, a, ma);
        score_key_tile<FP8, NR, RELU>(P, a, ma, qf, nr, row0,
                                      jw + t * kLogitsKeysPerWG + w * 64, vis_max, lane, first,
                                      kmax);
      }
    }
  }
  kmax = wave_max(kmax);
  if (lane == 0) red[w] = kmax;
  __syncthreads();
  if (threadIdx.x < kKeys / 128) {
    const int blk = k * (kKeys / 128) + threadIdx.x;
    float m = red[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) m = fmaxf(m, red[i]);
    if (blk < P.key_blocks) P.kmax[(int64_t)r * P.key_blocks + blk] = m;
  }
}

template <bool FP8>
hipError_t launch_logits(const SelectParams& P, int rows_per_chunk, hipStream_t s) {
  const dim3 grid(P.key_tiles, P.R);
  if (rows_per_chunk <= 1)
    hipLaunchKernelGGL((logits_valu_kernel<FP8, 1>), grid, dim3(kLogitsThreads), 0, s, P);
  else if (rows_per_chunk <= 2)
    hipLaunchKernelGGL((logits_valu_kernel<FP8, 2>), grid, dim3(kLogitsThreads), 0, s, P);
  else
    hipLaunchKernelGGL((logits_valu_kernel<FP8, 4>), grid, dim3(kLogitsThreads), 0, s, P);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_logits_valu_relu(const SelectParams& P, hipStream_t s) {
  const dim3 grid(P.key_tiles, P.R);
  if (P.fp8)
    hipLaunchKernelGGL((logits_valu_kernel<true, 8, true>), grid, dim3(kLogitsThreads), 0, s, P);
  else
    hipLaunchKernelGGL((logits_valu_kernel<false, 8, true>), grid, dim3(kLogitsThreads), 0, s,
                       P);
  return hipGetLastError();
}

hipError_t launch_logits_valu(const SelectParams& P, int rows_per_chunk, hipStream_t s) {
  return P.fp8 ? launch_logits<true>(P, rows_per_chunk, s)
               : launch_logits<false>(P, rows_per_chunk, s);
}

}  // namespace qsa
