// Indexer logits on the vector units (decode and short requests): for every row and compressed
// block, the fast float32 score with the index heads folded into Q, sum_h q[h] . k =
// (sum_h q[h]) . k, written to the logits workspace together with the per-128-key bound of
// max |k| that the top-k's error band needs.  Follows the scoring step of QSAIndexer.forward
// (page "vllm.models.qwen4_exp.nvidia.qsa").
// This file holds the one-item-per-workgroup kernel and the launchers; the persistent variant
// for grids that do not fit the chip in one round is in logits_list.hip (a translation unit of
// its own: beside it, the compiler schedules this kernel's loads differently).
#include "logits_tile.h"

namespace qsa {
namespace {
using namespace logits_tile;

// Grid (workgroups per request, R), 512 threads (8 waves).  Workgroup k of request r scores the
// request's keys 1024k .. 1024k+1023 (2 tiles of 512; a wave takes 64 keys of each) against
// every row of the request, NR rows at a time.  A key's row is split over 16 lanes (bf16) or 8
// lanes (e4m3) of 16 bytes, so one wave load reads 1 KiB of contiguous cache (the lane layout is
// in logits_tile.h).  The cache row of every key and the head-folded rows are staged in LDS
// once; each wave keeps one tile in flight, the other waves of its SIMD covering the latency.
// RELU: one row at a time, its NR = 8 heads held unfolded as the scorer's rows.
// KMAX: the call also has matrix-core requests, for which this kernel only takes the per-block
// bound of max |k| (a separate instance, so that the decode instances carry no such branch).
// WIN: the call runs in row windows (a logits memory cap): only the rows in [row_lo, row_hi)
// are scored, into logits rows relative to row_lo.
// WIDE (one-row requests, no cap, batches that fill the chip): a workgroup scores 2048 keys as
// 4 tiles, two in flight per wave (the next tile's loads go out before a tile is scored), at 2
// waves per SIMD: the same bytes in flight as 4 waves with one tile each, with the per-workgroup
// round trips for the block table, the metadata and Q paid once per 2048 keys instead of 1024.
// On decode_32k: 30.6 -> 29.6 us; with 8 tiles (half the workgroups) it took 35.5 us.
template <bool FP8, int NR, bool RELU = false, bool KMAX = false, bool WIN = false,
          bool WIDE = false>
__global__ __launch_bounds__(kLogitsThreads)
__attribute__((amdgpu_waves_per_eu((NR >= 4 || WIDE) ? 2 : 4)))
void logits_valu_kernel(SelectParams P) {
  static_assert(!WIDE || (NR == 1 && !RELU && !KMAX && !WIN), "the wide instance is for decode");
  using KL = KeyLanes<FP8>;
  constexpr int kT = kLogitsThreads, kWaves = kLogitsThreads / 64;
  constexpr int kTiles = WIDE ? 2 * kLogitsTilesPerWG : kLogitsTilesPerWG;
  constexpr int kKeys = kTiles * kLogitsKeysPerWG;
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
  // Requests with many rows are scored by the MFMA kernel; for them the KMAX instance only takes
  // the per-block bound of max |k| the top-k needs (one pass over their keys).
  if (!KMAX && n > P.mfma_min_rows) return;  // block-uniform, before any barrier
  const int vis_max = (n > 0 && n <= L) ? min(L / P.c, P.cols) : 0;
  // The request's rows in this window: [rb, re) of its n.
  const int rb = WIN ? min(max(P.row_lo - q0, 0), n) : 0;
  const int re = WIN ? min(max(P.row_hi - q0, 0), n) : n;
  if (WIN && rb >= re) return;  // block-uniform, before any barrier
  // A matrix-core request that began in an earlier window has its max |k| from that window's
  // launch (the bound depends on the keys only), and none of its rows are scored here.
  if (KMAX && WIN && n > P.mfma_min_rows && rb > 0) return;  // block-uniform
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
    if constexpr (KMAX) {
      if (n > P.mfma_min_rows) {  // block-uniform
        barrier();  // rows_s written
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
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
    }
    // (KMAX: the rows of a matrix-core request are not scored here.)
    const int n_scored = KMAX ? (n > P.mfma_min_rows ? rb : re) : re;
    for (int rr0 = rb; rr0 < n_scored; rr0 += (RELU ? 1 : NR)) {
      const int nr = RELU ? NR : min(NR, re - rr0);
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
      if (rr0 > rb) barrier();  // the previous chunk's readers are done with qf_s
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
      const bool first = rr0 == rb;
      const int row0 = q0 + rr0 - (WIN ? P.row_lo : 0);  // logits row (window-relative)
      // One tile in flight per wave (WIDE: two); the other waves of the SIMD cover its
      // latency.  The loops are unrolled, so the compiler's vmcnt waits name exactly the tile.
      if constexpr (WIDE) {
        uint32_t a[2][KL::kLoads][4], ma[2];
        load_key_tile<FP8>(P, rows_s, 0, w, lane, a[0], ma[0]);
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
          if (t + 1 < kTiles)
            load_key_tile<FP8>(P, rows_s, t + 1, w, lane, a[(t + 1) & 1], ma[(t + 1) & 1]);
          score_key_tile<FP8, NR, RELU>(P, a[t & 1], ma[t & 1], qf, nr, row0,
                                        jw + t * kLogitsKeysPerWG + w * 64, vis_max, lane,
                                        first, kmax);
        }
      } else {
        uint32_t a[KL::kLoads][4], ma;
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
          load_key_tile<FP8>(P, rows_s, t, w, lane, a, ma);
          score_key_tile<FP8, NR, RELU>(P, a, ma, qf, nr, row0,
                                        jw + t * kLogitsKeysPerWG + w * 64, vis_max, lane,
                                        first, kmax);
        }
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

// Workgroups the chip holds at once (kCUs, qsa_internal.h): two per CU with up to two rows per
// chunk (four waves per SIMD), one with four or more.

// Workgroups per request of the wide instance (2048 keys each).
int wide_tiles(const SelectParams& P) {
  return (P.cols + 2 * kLogitsTilesPerWG * kLogitsKeysPerWG - 1) /
         (2 * kLogitsTilesPerWG * kLogitsKeysPerWG);
}

// The one-item-per-workgroup grid (rather than the persistent work list) for NR rows per chunk.
bool valu_grid(const SelectParams& P, int nr) {
  const int per_cu = nr >= 4 ? 1 : 2;
  const int64_t dense = (int64_t)P.R * P.key_tiles, resident = (int64_t)kCUs * per_cu;
  return dense <= resident || P.R > kLogitsListReqs;
}

// One-row requests filling the chip with 2048-key workgroups (one per CU): the wide instance.
// Smaller batches keep 1024-key workgroups, which spread over more CUs.
bool wide_applies(const SelectParams& P) {
  const bool windows = P.row_lo > 0 || P.row_hi < P.T;
  return valu_grid(P, 1) && !windows && (int64_t)P.R * wide_tiles(P) >= kCUs;
}

template <bool FP8, int NR, bool RELU, bool KMAX>
hipError_t launch_valu(const SelectParams& P, hipStream_t s) {
  const int per_cu = NR >= 4 ? 1 : 2;
  const int64_t resident = (int64_t)kCUs * per_cu;
  if (valu_grid(P, NR)) {
    const dim3 grid(P.key_tiles, P.R), block(kLogitsThreads);
    const bool windows = P.row_lo > 0 || P.row_hi < P.T;
    if constexpr (NR == 1 && !RELU && !KMAX) {
      if (wide_applies(P)) {
        hipLaunchKernelGGL((logits_valu_kernel<FP8, 1, false, false, false, true>),
                           dim3(wide_tiles(P), P.R), block, 0, s, P);
        return hipGetLastError();
      }
    }
    if (windows)
      hipLaunchKernelGGL((logits_valu_kernel<FP8, NR, RELU, KMAX, true>), grid, block, 0, s, P);
    else
      hipLaunchKernelGGL((logits_valu_kernel<FP8, NR, RELU, KMAX>), grid, block, 0, s, P);
    return hipGetLastError();
  }
  return launch_logits_list(P, NR, RELU, KMAX, (unsigned)resident, s);
}

template <bool FP8>
hipError_t launch_logits(const SelectParams& P, int rows_per_chunk, bool mfma, hipStream_t s) {
  if (mfma)  // the matrix-core kernel scores the requests of more than 16 rows
    return launch_valu<FP8, 4, false, true>(P, s);
  if (rows_per_chunk <= 1) return launch_valu<FP8, 1, false, false>(P, s);
  if (rows_per_chunk <= 2) return launch_valu<FP8, 2, false, false>(P, s);
  return launch_valu<FP8, 4, false, false>(P, s);
}

}  // namespace

bool logits_wide(const SelectParams& P, int rows_per_chunk, bool mfma) {
  return !mfma && !P.relu && rows_per_chunk <= 1 && wide_applies(P);
}

hipError_t launch_logits_valu(const SelectParams& P, int rows_per_chunk, bool mfma,
                              hipStream_t s) {
  return P.fp8 ? launch_logits<true>(P, rows_per_chunk, mfma, s)
               : launch_logits<false>(P, rows_per_chunk, mfma, s);
}

}  // namespace qsa
