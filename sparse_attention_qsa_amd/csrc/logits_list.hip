// Indexer logits on the vector units, persistent variant: the kernel of logits.hip for calls
// whose one-item-per-workgroup grid would not fit the chip in one round (many requests of
// uneven length).  Follows the scoring step of QSAIndexer.forward (page
// "vllm.models.qwen4_exp.nvidia.qsa").
#include "logits_tile.h"

namespace qsa {
namespace {
using namespace logits_tile;

// Work list of the persistent instance: the (request, 1024-key item) pairs that hold visible
// keys, in request order.  Every workgroup derives it from the request metadata (one round
// trip) into LDS as the prefix sums of the requests' item counts, with the requests' row ranges
// and visible keys beside it, then takes items blockIdx.x, blockIdx.x + gridDim.x, ...
// Persistent variant of logits_valu_kernel for grids that do not fit the chip in one round
// (long, uneven requests): workgroups of 512 threads (8 waves).  Item k of request r is the
// request's keys 1024k .. 1024k+1023 (2 tiles of 512; a wave scores 64 keys per tile), scored against every row of the
// request, NR rows at a time.  A key's row is split over 16 lanes (bf16) or 8 lanes (fp8) of 16
// bytes, so every load instruction reads 1 KiB of contiguous cache.  The cache row of every key
// and the head-folded rows are staged in LDS once per item; the block table and the request
// metadata come in one round trip, the folded Q in the next, and the key burst only after Q
// (issued behind it, Q would wait several microseconds in the memory queues).
// The grid holds as many workgroups as the chip runs at once; they walk the work list, so that
// no workgroup is dispatched for keys that do not exist.
// RELU: one row at a time, its NR = 8 heads held unfolded as the scorer's rows.
// KMAX: the call also has matrix-core requests, for which this kernel only takes the per-block
// bound of max |k| (a separate instance, so that the decode instances carry no such branch).
template <bool FP8, int NR, bool RELU = false, bool KMAX = false>
__global__ __launch_bounds__(kLogitsThreads) __attribute__((amdgpu_waves_per_eu(NR >= 4 ? 2 : 4)))
void logits_valu_list_kernel(SelectParams P) {
  using KL = KeyLanes<FP8>;
  constexpr int kT = kLogitsThreads, kWaves = kLogitsThreads / 64;
  constexpr int kKeys = kLogitsTilesPerWG * kLogitsKeysPerWG;
  static_assert(kLogitsKeysPerWG == kWaves * 64, "a tile is 64 keys per wave");
  __shared__ int32_t rows_s[kKeys];
  __shared__ float qf_s[NR][kHeadDim];
  __shared__ float red[kWaves];
  __shared__ int32_t item_end[kLogitsListReqs];  // inclusive prefix sums of the item counts
  __shared__ int32_t req_q0[kLogitsListReqs], req_n[kLogitsListReqs], req_vis[kLogitsListReqs];
  __shared__ int32_t s_tot[kWaves];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // Barrier without a memory fence (a fence would wait for every load in flight); the LDS
  // writes before it are complete, and global loads are waited for where their data is used.
  auto barrier = [] {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // Row range and visible keys of request i, clamped into [0, T): the metadata is device data
  // the host never saw, so it is not trusted to stay inside the buffers.
  auto req_range = [&](int i, int& q0, int& n, int& vis_max) {
    q0 = max(0, min(P.qsl[i], P.T));
    n = max(0, min(P.qsl[i + 1], P.T) - q0);
    const int L = P.seq_lens[i];
    vis_max = (n > 0 && n <= L) ? min(L / P.c, P.cols) : 0;
  };

  auto run_item = [&](const int r, const int k) __attribute__((always_inline)) {
    const int jw = k * kKeys;  // first key of the item
    // Block-table entries of this thread's keys jw + tid + kT i: their addresses do not depend
    // on the request metadata, so they are loaded together with it (one round trip).
    int col[kKeys / kT], page[kKeys / kT];
#pragma unroll
    for (int i = 0; i < kKeys / kT; ++i) {
      col[i] = (jw + (int)threadIdx.x + kT * i) / P.Pc;
      page[i] = P.cbt[(int64_t)r * P.cbt_stride + min(col[i], P.cbt_width - 1)];
    }
    const int q0 = req_q0[r], n = req_n[r], vis_max = req_vis[r];
    // The request's rows in this launch's window (all of them without a logits cap).
    const int rb = min(max(P.row_lo - q0, 0), n), re = min(max(P.row_hi - q0, 0), n);
    // Requests with many rows are scored by the MFMA kernel (none in a call without one); for
    // them this kernel only takes the per-block bound of max |k| the top-k needs (one pass over
    // their keys).
    if (!KMAX && n > P.mfma_min_rows) return;  // block-uniform, before any barrier
    const bool kmax_only = KMAX && n > P.mfma_min_rows;  // block-uniform
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
      for (int rr0 = rb; rr0 < (kmax_only ? rb : re); rr0 += (RELU ? 1 : NR)) {
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
        const int row0 = q0 + rr0 - P.row_lo;  // logits row (window-relative)
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
    // Also the item's last barrier: every wave is done with rows_s and qf_s, which a next item
    // overwrites.
    __syncthreads();
    if (threadIdx.x < kKeys / 128) {
      const int blk = k * (kKeys / 128) + threadIdx.x;
      float m = red[0];
#pragma unroll
      for (int i = 1; i < kWaves; ++i) m = fmaxf(m, red[i]);
      if (blk < P.key_blocks) P.kmax[(int64_t)r * P.key_blocks + blk] = m;
    }
  };

  // The MFMA kernel, which runs next, starts its work queues from zero.
  if (blockIdx.x == 0 && threadIdx.x < 8) P.work[threadIdx.x] = 0;
  {
    // Thread t counts the items of requests t*per .. t*per+per-1; a workgroup scan of the
    // counts (in-wave, then the wave totals) gives every request's end.
    constexpr int kPerMax = kLogitsListReqs / kT;
    const int per = (P.R + kT - 1) / kT, i0 = threadIdx.x * per;
    int cnt[kPerMax];
#pragma unroll
    for (int u = 0; u < kPerMax; ++u) {
      cnt[u] = 0;
      if (u < per && i0 + u < P.R) {
        int q0, n, vm;
        req_range(i0 + u, q0, n, vm);
        // No items for a request without rows in this launch's window.
        if (P.row_hi <= q0 || q0 + n <= P.row_lo) vm = 0;
        cnt[u] = (vm + kKeys - 1) / kKeys;
        req_q0[i0 + u] = q0;
        req_n[i0 + u] = n;
        req_vis[i0 + u] = vm;
      }
    }
    int sum = 0;
#pragma unroll
    for (int u = 0; u < kPerMax; ++u) sum += cnt[u];
    int incl = sum;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int v = __shfl_up(incl, m, 64);
      if (lane >= m) incl += v;
    }
    if (lane == 63) s_tot[w] = incl;
    barrier();
    int run = incl - sum, total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      run += i < w ? s_tot[i] : 0;
      total += s_tot[i];
    }
#pragma unroll
    for (int u = 0; u < kPerMax; ++u) {
      run += cnt[u];
      if (u < per && i0 + u < P.R) item_end[i0 + u] = run;
    }
    barrier();
    for (int item = blockIdx.x; item < total; item += gridDim.x) {
      // The request whose items hold `item`: the first r with item_end[r] > item.
      int lo = 0, hi = P.R - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (item_end[mid] > item) hi = mid; else lo = mid + 1;
      }
      run_item(lo, item - (lo > 0 ? item_end[lo - 1] : 0));
    }
  }
}

}  // namespace

hipError_t launch_logits_list(const SelectParams& P, int nr, bool relu, bool kmax, unsigned grid,
                              hipStream_t s) {
  const dim3 g(grid), b(kLogitsThreads);
  if (kmax) {  // matrix-core requests in the call
    if (P.fp8)
      hipLaunchKernelGGL((logits_valu_list_kernel<true, 4, false, true>), g, b, 0, s, P);
    else
      hipLaunchKernelGGL((logits_valu_list_kernel<false, 4, false, true>), g, b, 0, s, P);
  } else if (P.fp8) {
    if (nr <= 1) hipLaunchKernelGGL((logits_valu_list_kernel<true, 1>), g, b, 0, s, P);
    else if (nr <= 2) hipLaunchKernelGGL((logits_valu_list_kernel<true, 2>), g, b, 0, s, P);
    else hipLaunchKernelGGL((logits_valu_list_kernel<true, 4>), g, b, 0, s, P);
  } else {
    if (nr <= 1) hipLaunchKernelGGL((logits_valu_list_kernel<false, 1>), g, b, 0, s, P);
    else if (nr <= 2) hipLaunchKernelGGL((logits_valu_list_kernel<false, 2>), g, b, 0, s, P);
    else hipLaunchKernelGGL((logits_valu_list_kernel<false, 4>), g, b, 0, s, P);
  }
  return hipGetLastError();
}

}  // namespace qsa
