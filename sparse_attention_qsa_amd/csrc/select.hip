// qsa_index_logits_topk kernels: head-folded indexer logits, block top-k, expansion into the
// packed selection buffer.
//
// Follows QSAIndexer.forward's selection (qsa_select_paged_decode / qsa_select_paged_prefill /
// expand_qsa_block_indices) and the packed-buffer contract of QSAIndexer.output_width /
// packed_output_width (page "vllm.models.qwen4_exp.nvidia.qsa").
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

#include "qsa_internal.h"

namespace qsa {
namespace {

struct SelectParams {
  int T, R, Hi, c, budget, Pc, c_pages, cbt_stride, cbt_width, cols, col_stride, key_tiles;
  int key_blocks;     // 128-key blocks per request in the kmax array
  int mfma_min_rows;  // requests with more rows than this are scored by the MFMA kernel
  bool fp8;
  const int32_t* qsl;
  const int32_t* seq_lens;
  const void* q_idx;
  const void* ckv;
  const int32_t* cbt;
  int32_t* packed;
  int64_t p_rs;
  float* logits;
  float* kmax;  // [R, key_blocks]: an upper bound of max |k| over each block of 128 keys
  int32_t* band_idx;
  double* band_score;
  int* work;  // [8] work counters of the MFMA kernel's queues, zeroed by the VALU kernel
};

__device__ __forceinline__ float load_q_value(const SelectParams& P, int64_t idx) {
  if (P.fp8) return e4m3_to_f32_exact(reinterpret_cast<const uint8_t*>(P.q_idx)[idx]);
  return bf16_to_f32(reinterpret_cast<const uint16_t*>(P.q_idx)[idx]);
}

// ------------------------------------------------------------------------------ logits

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
// Updates the lane's running max |k|.
template <bool FP8, int NR>
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
template <bool FP8, int NR>
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
  // Requests with many rows are scored by the MFMA kernel.
  if (n > P.mfma_min_rows) return;  // block-uniform, before any barrier
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
    for (int rr0 = 0; rr0 < n; rr0 += NR) {
      const int nr = min(NR, n - rr0);
      // Head-folded Q of the chunk's rows: each of the first nr*128 threads owns one (row, dim)
      // and loads all its heads at once (clamped to Hi - 1, the extra terms added as zero).
      constexpr int kSlots = (NR * kHeadDim + kT - 1) / kT;
      uint32_t v[kSlots][16];  // raw bf16 / e4m3 codes
#pragma unroll
      for (int sl = 0; sl < kSlots; ++sl) {
        const int e = threadIdx.x + kT * sl;
        const int rr = min(e >> 7, nr - 1), d = e & (kHeadDim - 1);
        const int64_t qb = (int64_t)(q0 + rr0 + rr) * P.Hi * kHeadDim + d;
#pragma unroll
        for (int h = 0; h < 16; ++h) {
          const int64_t idx = qb + min(h, P.Hi - 1) * kHeadDim;
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
#pragma unroll
        for (int h = 1; h < 16; ++h) f = f + (h < P.Hi ? dec(v[sl][h]) : 0.0f);
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
        score_key_tile<FP8, NR>(P, a, ma, qf, nr, row0, jw + t * kLogitsKeysPerWG + w * 64,
                                vis_max, lane, first, kmax);
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

// ------------------------------------------------------------------------------ prefill logits

// Requests with many rows (chunked prefill) are scored per head on the matrix cores: for a
// tile of 128 rows x 256 keys, S = sum_h Q_h K^T, the head sum taken in the fp32 accumulator
// (bf16 products are exact in fp32).  The fp32 result differs from the canonical float64
// score by at most gamma_{Hi*128} kappa A with u = 2^-23 (any summation order, faithful
// rounding); the top-k's band covers that.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaRows = 128;        // rows per row block
constexpr int kMfmaKeys = 256;        // keys per workgroup (its key tile)
constexpr int kMfmaRowBlocksPerWG = 4;
constexpr int kMfmaMinRows = 16;      // requests with more rows than this take the MFMA kernel

__device__ __forceinline__ void lds_dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// Tiles in LDS hold rows of 256 bytes; row t's 16-byte chunk c sits in slot c ^ (t & 15), so
// that 16 lanes reading chunk c of 16 consecutive rows hit 16 different slots.  They are
// filled by LDS-direct loads: a load writes 4 rows (1 KiB), lane L landing in row L/16, slot
// L%16.
__device__ __forceinline__ const bf16x8_t& tile_chunk(const uint8_t* buf, int t, int c) {
  return *reinterpret_cast<const bf16x8_t*>(buf + t * 256 + 16 * (c ^ (t & 15)));
}
__device__ __forceinline__ uint32_t tile_chunk_addr(const uint8_t* buf, int t, int c) {
  const __attribute__((address_space(3))) uint8_t* p =
      (const __attribute__((address_space(3))) uint8_t*)(buf + t * 256 + 16 * (c ^ (t & 15)));
  return (uint32_t)(uintptr_t)p;
}
// 16-byte LDS read at addr + OFF issued as inline assembly; the caller waits (lgkmcnt)
// before use.
template <int OFF>
__device__ __forceinline__ bf16x8_t lds_read16_off(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds_read offset field is 16 bits");
  bf16x8_t v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}

// Waits until at most n VMEM operations of this wave are outstanding (n from the small set of
// counts the MFMA kernel uses; any other count waits for all).
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 16: __builtin_amdgcn_s_waitcnt(0x4F70); break;
    case 20: __builtin_amdgcn_s_waitcnt(0x4F74); break;
    case 24: __builtin_amdgcn_s_waitcnt(0x4F78); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
}

// Persistent workgroups (one per CU; the LDS use allows no more) take work items -- (request,
// chunk of up to four row blocks, key tile of 256 keys) -- from eight queues, one per XCD:
// queue x holds the (request, row chunk) pairs x, x+8, ..., each with all its key tiles in
// order, so that the workgroups of one XCD work on the same rows at once and share their Q in
// the XCD's L2.  (Workgroup b takes queue b % 8, which is its XCD under round-robin dispatch;
// any other placement only costs locality.)  An item loads its key tile once and keeps the
// key fragments in registers (8 waves, 2 x 4 of 64 rows x 64 keys; per wave 4 x 4
// accumulators of 16 keys x 16 rows, v_mfma_f32_16x16x32_bf16 with the keys as the A operand
// so that a lane ends up with 4 consecutive keys of one row).  The Q slabs (128 rows of one
// head) of its row blocks then stream through four 32 KiB LDS buffers (two of them the key
// tile's), three slabs in flight while one is multiplied.  Stores are unconditional buffer
// stores (out-of-range lanes are dropped by the buffer's bounds), so that every wave issues a
// known number of memory operations and the waits for the slabs are exact.
__global__ __launch_bounds__(512) void logits_mfma_kernel(SelectParams P, int row_blocks) {
  // Four 32 KiB buffers: 0 and 1 hold Q slabs; 2 and 3 hold the key tile (keys 0..127,
  // 128..255) and afterwards two more Q slabs.  Slab sl lives in buffer sl % 4.
  __shared__ __attribute__((aligned(16))) uint8_t lds[4][kMfmaRows * 256];
  uint8_t* const kl = lds[2];
  uint8_t* const kh = lds[3];
  __shared__ float red[2][8];
  __shared__ __attribute__((aligned(4))) uint8_t kok[kMfmaKeys];
  __shared__ int s_item;
  const int key_tiles = (P.cols + kMfmaKeys - 1) / kMfmaKeys;
  const int row_chunks = (row_blocks + kMfmaRowBlocksPerWG - 1) / kMfmaRowBlocksPerWG;
  const int pairs = P.R * row_chunks;
  const int queue = blockIdx.x & 7;
  const int64_t qlen = (int64_t)((pairs - queue + 7) / 8) * key_tiles;  // items of this queue

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int wr = w >> 2, wc = w & 3;  // this wave: rows 64wr .. +63, keys 64wc .. +63
  const char* ckv = reinterpret_cast<const char*>(P.ckv);
  const char* qb = reinterpret_cast<const char*>(P.q_idx);
  // Barrier without a memory fence (a fence would wait for every load in flight); LDS reads
  // are complete before it, and the loads into LDS are waited for explicitly.
  auto barrier = [] {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  for (;;) {
    if (tid == 0) s_item = atomicAdd(&P.work[queue], 1);
    barrier();
    const int64_t item = s_item;
    barrier();  // every wave has read s_item (and is done with the previous item's LDS)
    if (item >= qlen) break;  // workgroup-uniform
    const int g = queue + 8 * (int)(item / key_tiles);
    const int kt = (int)(item % key_tiles);
    const int rc = g % row_chunks, r = g / row_chunks;

    const int q0 = max(0, min(P.qsl[r], P.T));
    const int n = max(0, min(P.qsl[r + 1], P.T) - q0), L = P.seq_lens[r];
    if (n <= P.mfma_min_rows || n > L) continue;  // decode request, or inert rows
    const int key0 = kt * kMfmaKeys;
    const int vis_max = min(L / P.c, P.cols);
    // Row blocks of this chunk that see at least one key of the tile (visibility grows with
    // the row, so they are a suffix of the chunk).
    const int rb_end = min((rc + 1) * kMfmaRowBlocksPerWG, (n + kMfmaRows - 1) / kMfmaRows);
    int rb_first = rc * kMfmaRowBlocksPerWG;
    auto sees_tile = [&](int rb) {
      const int last = min(kMfmaRows, n - rb * kMfmaRows);
      return key0 < min((L - n + rb * kMfmaRows + last) / P.c, P.cols);
    };
    while (rb_first < rb_end && !sees_tile(rb_first)) ++rb_first;
    if (rb_first >= rb_end) continue;

    // ---- key tile (keys key0 .. key0+255), 8 loads per wave (wave w: keys 32w .. 32w+31, in
    // kl for w < 4, else kh); the block-table reads come first, all in flight together.  A
    // key that is not visible or whose page is outside the cache loads the cache's first row
    // and is masked afterwards.
    {
      int page[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int jk = key0 + 32 * w + 4 * i + (lane >> 4);
        const int col = jk < vis_max ? min(jk / P.Pc, P.cbt_width - 1) : 0;
        page[i] = P.cbt[(int64_t)r * P.cbt_stride + col];
      }
      asm volatile("" : "+v"(page[0]), "+v"(page[1]), "+v"(page[2]), "+v"(page[3]),
                   "+v"(page[4]), "+v"(page[5]), "+v"(page[6]), "+v"(page[7]));
      uint8_t* const kdst = w < 4 ? kl : kh;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = 32 * w + 4 * i + (lane >> 4), jk = key0 + j;
        const bool ok = jk < vis_max && jk / P.Pc < P.cbt_width && page[i] >= 0 &&
                        page[i] < P.c_pages;
        const int64_t off = ok ? ((int64_t)page[i] * P.Pc + jk % P.Pc) * kHeadDim * 2 : 0;
        lds_dma16(ckv + off + 16 * ((lane & 15) ^ (j & 15)),
                  kdst + ((32 * w + 4 * i) & 127) * 256);
        if ((lane & 15) == 0) kok[j] = ok;
      }
    }
    // ---- Q slab sl: head sl % Hi of row block rb_first + sl / Hi (rows past the request
    // repeat its last row), 4 loads per wave.
    const int nslabs = (rb_end - rb_first) * P.Hi;
    auto load_q = [&](int sl, uint8_t* dst) {
      const int rb = rb_first + sl / P.Hi, h = sl % P.Hi;
      const int last = min(kMfmaRows, n - rb * kMfmaRows) - 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * w + 4 * i + (lane >> 4);
        const int64_t grow = q0 + rb * kMfmaRows + min(t, last);
        lds_dma16(qb + ((grow * P.Hi + h) * kHeadDim) * 2 + 16 * ((lane & 15) ^ (t & 15)),
                  dst + (16 * w + 4 * i) * 256);
      }
    };
    load_q(0, lds[0]);
    if (nslabs > 1) load_q(1, lds[1]);
    wait_vmcnt(nslabs > 1 ? 4 : 0);  // the key tile and slab 0 have landed
    barrier();

    // ---- max |k| over the valid keys of each 128-key half (upper bounds for the top-k).
    // Consecutive lanes read consecutive dwords; dword d of a half belongs to its key d / 64.
    {
      float km[2] = {0.0f, 0.0f};
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const uint32_t* kw = reinterpret_cast<const uint32_t*>(hf ? kh : kl);
#pragma unroll 8
        for (int i = 0; i < 16; ++i) {
          const int d = tid + 512 * i;
          if (kok[128 * hf + (d >> 6)]) {
            const uint32_t u = kw[d];
            km[hf] = fmaxf(km[hf], fmaxf(fabsf(bf16lo(u)), fabsf(bf16hi(u))));
          }
        }
      }
      km[0] = wave_max(km[0]);
      km[1] = wave_max(km[1]);
      if (lane == 0) {
        red[0][w] = km[0];
        red[1][w] = km[1];
      }
    }
    // ---- this wave's key fragments: keys 64wc + 16kk + lane%16, dims 32ks + 8(lane/16) .. +7
    bf16x8_t kfr[4][4];
    {
      const uint8_t* kt_half = wc < 2 ? kl : kh;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          kfr[kk][ks] = tile_chunk(kt_half, 64 * (wc & 1) + 16 * kk + (lane & 15),
                                   4 * ks + (lane >> 4));
      }
    }
    barrier();  // red[] complete; the key tile is free for slabs 2 and 3
    if (tid < 2 && 2 * kt + tid < P.key_blocks) {
      float m = red[tid][0];
      for (int i = 1; i < 8; ++i) m = fmaxf(m, red[tid][i]);
      P.kmax[(int64_t)r * P.key_blocks + 2 * kt + tid] = m;
    }
    if (nslabs > 2) load_q(2, lds[2]);

    f32x4_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // Bit k of `stored`: the iteration k+1 back wrote its row block (16 stores per wave).
    uint32_t stored = 0;
    // Per-lane LDS addresses of this wave's Q fragments in buffers 0/1 and 2/3 for each K step
    // (row 64wr + lane%16, chunk 4ks + lane/16); the buffer and the row block go in the
    // instruction's offset.
    uint32_t qaddr[2][4];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qaddr[hb][ks] = tile_chunk_addr(lds[2 * hb], 64 * wr + (lane & 15), 4 * ks + (lane >> 4));
    }
    // One slab: wait for it, load slab sl+3 into the buffer slab sl-1 used, multiply, and
    // write the row block when its last head is done.
    auto step = [&](int sl, auto buf_tag) {
      constexpr int kBuf = decltype(buf_tag)::value;
      uint8_t* const next = lds[(kBuf + 3) & 3];
      // Memory operations this wave issued after slab sl's loads: the loads of slabs sl+1
      // and sl+2 (4 each), and the stores of iterations max(0, sl-3) .. sl-1.
      const int dmas = 4 * (min(nslabs - 1, sl + 2) - sl);
      int after = dmas + 16 * __builtin_popcount(stored & 7u);
      if (after > 24) after = dmas;  // fewer than issued: a stricter wait
      wait_vmcnt(after);
      barrier();  // slab sl visible to all waves; slab sl-1's buffer is free
      if (sl + 3 < nslabs) load_q(sl + 3, next);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        // The slab reads are issued as inline assembly, which the compiler's own wait
        // insertion does not track: it would otherwise wait for every load into LDS in
        // flight (including the next slabs') before reading this one, which the wait above
        // already guarantees has landed.
        bf16x8_t qfr[4];
        const uint32_t qa = qaddr[kBuf >> 1][ks];
        qfr[0] = lds_read16_off<(kBuf & 1) * kMfmaRows * 256 + 0 * 4096>(qa);
        qfr[1] = lds_read16_off<(kBuf & 1) * kMfmaRows * 256 + 1 * 4096>(qa);
        qfr[2] = lds_read16_off<(kBuf & 1) * kMfmaRows * 256 + 2 * 4096>(qa);
        qfr[3] = lds_read16_off<(kBuf & 1) * kMfmaRows * 256 + 3 * 4096>(qa);
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(qfr[0]), "+v"(qfr[1]), "+v"(qfr[2]),
                     "+v"(qfr[3]));
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            acc[rr][kk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfr[kk][ks], qfr[rr],
                                                                  acc[rr][kk], 0, 0, 0);
        }
      }
      const bool last_head = sl % P.Hi == P.Hi - 1;
      stored = (stored << 1) | (last_head ? 1u : 0u);
      if (last_head) {
        // ---- row block done.  Accumulator element e of block (rr, kk) is key 64wc + 16kk +
        // 4(lane/16) + e of row 64wr + 16rr + lane%16.  A group of 4 keys is written when its
        // first key is visible to the row (the rest of the group lies inside the row's stride
        // and past its visible keys, which the top-k does not read).
        const int rb = rb_first + sl / P.Hi;
        const int nrows = min(kMfmaRows, n - rb * kMfmaRows);
        const int pbase = L - n + rb * kMfmaRows;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            P.logits + (int64_t)(q0 + rb * kMfmaRows) * P.col_stride, 0,
            nrows * P.col_stride * 4, 0x00020000);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int t = 64 * wr + 16 * rr + (lane & 15);
          const int vis = t < nrows ? min((pbase + t + 1) / P.c, P.cols) : 0;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const int j = 64 * wc + 16 * kk + 4 * (lane >> 4);
            const uint32_t okm = *reinterpret_cast<const uint32_t*>(kok + j);
            f32x4_t v = acc[rr][kk];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (!((okm >> (8 * e)) & 0xFFu)) v[e] = 0.0f;
            }
            const uint32_t off = key0 + j < vis ? (uint32_t)(t * P.col_stride + key0 + j) * 4u
                                                : 0xFFFFFFF0u;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rs, off, 0,
                                                   0);
            acc[rr][kk] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
          }
        }
      }
    };
    for (int sl = 0; sl < nslabs; sl += 4) {
      step(sl, std::integral_constant<int, 0>{});
      if (sl + 1 < nslabs) step(sl + 1, std::integral_constant<int, 1>{});
      if (sl + 2 < nslabs) step(sl + 2, std::integral_constant<int, 2>{});
      if (sl + 3 < nslabs) step(sl + 3, std::integral_constant<int, 3>{});
    }
  }
}

// ------------------------------------------------------------------------------ top-k

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
// zero.  Only the lanes whose partner exists use the result.
template <int N>
__device__ __forceinline__ double row_down(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, 0x100 + N, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), 0x100 + N, 0xF, 0xF,
                                             false);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
template <int N>
__device__ __forceinline__ float row_down(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x100 + N, 0xF, 0xF,
                                                    false));
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
        k0 = e4m3_to_f32_exact(u & 0xFFu);
        k1 = e4m3_to_f32_exact(u >> 8);
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

// Canonical float64 score of compressed row j against the row's Q (held in LDS as floats),
// computed by a group of 16 lanes (l = lane % 16).  Per head the 128 exact products are summed
// by halving: pairs (2i, 2i+1) give v_i; then v_i += v_{i+32} for i < 32, += v_{i+16} for
// i < 16, ..., += v_{i+1} for i < 1.  Lane l holds v_l, v_{l+16}, v_{l+32}, v_{l+48}, so the
// first two halvings are in-lane and the last four take the partner 8, 4, 2, 1 lanes up.
// The heads are then added in order.  The result is valid in lane l = 0.
__device__ double canonical_score16(const SelectParams& P, const float* qrow,
                                    const int32_t* cbt_row, int cw, int j, int l) {
  float k[8];
  key_pairs16(P, cbt_row, cw, j, l, k);
  double s = 0.0;
  for (int h = 0; h < P.Hi; ++h) {
    const float* q = qrow + h * kHeadDim;
    double v[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = l + 16 * t;
      const double p0 = (double)q[2 * i] * (double)k[2 * t];          // exact
      const double p1 = (double)q[2 * i + 1] * (double)k[2 * t + 1];  // exact
      v[t] = p0 + p1;
    }
    double x = (v[0] + v[2]) + (v[1] + v[3]);
    x = x + row_down<8>(x);
    x = x + row_down<4>(x);
    x = x + row_down<2>(x);
    x = x + row_down<1>(x);
    s = (h == 0) ? x : s + x;
  }
  return s;
}

// Head-folded float32 score of compressed row j: (sum_h q_h) . k, the fold held in LDS, by a
// group of 16 lanes; valid in lane l = 0.  Its error is that of the VALU logits.
__device__ float folded_score16(const SelectParams& P, const float* qfold,
                                const int32_t* cbt_row, int cw, int j, int l) {
  float k[8];
  key_pairs16(P, cbt_row, cw, j, l, k);
  float x = 0.0f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int i = l + 16 * t;
    x += qfold[2 * i] * k[2 * t] + qfold[2 * i + 1] * k[2 * t + 1];
  }
  x = x + row_down<8>(x);
  x = x + row_down<4>(x);
  x = x + row_down<2>(x);
  x = x + row_down<1>(x);
  return x;
}

// Top-k kernel configurations: NT threads holding E scores each; the threshold's radix select
// takes PASSES passes of RB-bit digits over the top RB*PASSES bits of the order-preserving key
// (the rest stay unresolved: the threshold lies in one bin's value interval, which the band
// absorbs); bands of up to BAND entries and block-table rows of up to CBT columns live in LDS.
// The decode configurations spend LDS on few, fast rows; the prefill one (many rows) keeps its
// LDS small so that eight rows share a CU.
template <int NT_, int E_, int RB_, int PASSES_, int BAND_, int CBT_>
struct TopkCfg {
  static constexpr int NT = NT_, E = E_, RB = RB_, PASSES = PASSES_, BAND = BAND_, CBT = CBT_;
};
using TopkDecode8 = TopkCfg<512, 8, 12, 2, 1024, 2048>;
using TopkDecode16 = TopkCfg<512, 16, 12, 2, 1024, 2048>;
using TopkDecode32 = TopkCfg<512, 32, 12, 2, 1024, 2048>;
using TopkDecode1k = TopkCfg<1024, 32, 12, 2, 1024, 2048>;
using TopkPrefill = TopkCfg<256, 16, 8, 3, 256, 512>;
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
__global__ __launch_bounds__(C::NT) void topk_kernel(SelectParams P) {
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
  __shared__ float qrow[16 * kHeadDim];
  __shared__ float qfold[kHeadDim];
  __shared__ int32_t band_idx_s[kBandCap];
  __shared__ int32_t band2_idx_s[kBandCap];
  __shared__ double band_score_s[kBandCap];
  __shared__ int32_t cbt_s[kTopkCbtCap];

  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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
  const float* lg = P.logits + (int64_t)row * P.col_stride;
  const int jb = tid * E;
  float sc[E];
#pragma unroll
  for (int i = 0; i < E; i += 4) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (jb + i < P.col_stride) v = *reinterpret_cast<const float4*>(lg + jb + i);
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
  const int any_mine = __syncthreads_or(mine);
  int p = -1, L = 0, n_req = 0, r = -1;
  if (any_mine) {
    r = s_int[0];
    n_req = s_int[2];
    L = s_int[3];
    if (L - n_req >= 0) p = L - n_req + (row - s_int[1]);
  }
  if (p < 0) {  // inert row: no entries, count 0
    for (int col = tid; col <= W; col += NT) out[col] = col < W ? -1 : 0;
    return;
  }
  // seq_lens beyond the max_seq_len the workspace was sized for would overrun the logits
  // row: such rows are clamped (their selection is then undefined but stays in bounds).
  const int vis = min((p + 1) / P.c, P.cols);
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
    const int nt = min(P.key_blocks, (min(L / P.c, P.cols) + 127) / 128);
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
  uint32_t key[E];  // order-preserving keys of the fast scores
#pragma unroll
  for (int i = 0; i < E; ++i) {
    sc[i] = jb + i < vis ? sc[i] : -__builtin_inff();
    key[i] = fkey(sc[i]);
  }
  double qa = 0.0;
#pragma unroll
  for (int k = 0; k < kQPer; ++k) {
    const int i = tid + k * NT;
    if (i < P.Hi * kHeadDim) {
      const float f = P.fp8 ? e4m3_to_f32_exact(qv[k]) : bf16_to_f32((uint16_t)qv[k]);
      qrow[i] = f;
      qa += fabs((double)f);
    }
  }
  const int mask_words = (vis + 31) >> 5;
  for (int i = tid; i < mask_words; i += NT) sel_mask[i] = 0u;

  // ---- radix select.  Thread t reads the counts of bins (bins-1) - t*kPB - i (i < kPB): lower
  // threads own higher bins, so a workgroup prefix sum gives the count above each bin.  The
  // -inf entries land in the lowest bin, below any kb-th largest of the visible blocks.
  // Histograms alternate between two buffers; a pass clears the one the next-but-one uses.
  uint32_t prefix = 0, pmask = 0;
  int krem = kb;
#pragma unroll
  for (int pass = 0; pass < C::PASSES; ++pass) {
    const int shift = 32 - kRadixBits * (pass + 1);
    int* h = hist[pass & 1];
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const uint32_t u = key[i];
      if ((u & pmask) == prefix) atomicAdd(&h[(u >> shift) & (kRadixBins - 1)], 1);
    }
    if (pass >= 1 && pass + 1 < C::PASSES) {  // the buffer of pass + 1 was read by pass - 1
      for (int i = tid; i < kRadixBins; i += NT) hist[(pass + 1) & 1][i] = 0;
    }
    if (pass == 1) {  // the error-bound inputs, reduced over the workgroup below
      const float kmw = wave_max(km);
      double qaw = qa;
#pragma unroll
      for (int mm = 32; mm >= 1; mm >>= 1) qaw += shfl_xor_f64(qaw, mm);
      if (lane == 0) {
        s_flt[w] = kmw;
        s_dbl[w] = qaw;
      }
    }
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
    prefix |= (uint32_t)s_int[4] << shift;
    pmask |= (uint32_t)(kRadixBins - 1) << shift;
    krem = s_int[5];
  }
  // The kb-th largest fast score lies in [T_lo, T_hi], the values of the keys prefix..prefix|255.
  const double T_lo = (double)fval(prefix), T_hi = (double)fval(prefix | kLowMask);
  if (cbt_in_lds) {
#pragma unroll
    for (int k = 0; k < kCbtPer; ++k) {
      const int c = tid + k * NT;
      if (c < cw) cbt_s[c] = cbt_v[k];
    }
  }
  const int32_t* cbt_row = cbt_in_lds ? cbt_s : P.cbt + (int64_t)r * P.cbt_stride;

  // ---- error bound E of the fast scores for this row
  double kappa = 0.0, A = 0.0;
  for (int i = 0; i < kWaves; ++i) {
    kappa = fmax(kappa, (double)s_flt[i]);
    A += s_dbl[i];
  }
  // Bound of the head-folded float32 score (the VALU logits, and the second level below), and
  // of the per-head MFMA score (u = 2^-23 covers any rounding the matrix cores may use).
  const double gam_f = (double)(P.Hi + 130) * 0x1p-24;
  const double E_f = 2.0 * gam_f / (1.0 - gam_f) * kappa * A + 1e-30;
  const bool mfma_row = n_req > P.mfma_min_rows;
  const double gam_m = (double)(P.Hi * kHeadDim + 2) * 0x1p-23;
  const double Ebound = mfma_row ? 2.0 * gam_m / (1.0 - gam_m) * kappa * A + 1e-30 : E_f;
  // Certainly kept above hi, certainly dropped below lo; float32 forms widen the band only.
  const float hi = round_up_f32(T_hi + 2.0 * Ebound), lo = round_down_f32(T_lo - 2.0 * Ebound);

  // ---- classify and collect the band in block order: one workgroup scan of the per-thread
  // counts (band entries in the low half, certain keeps in the high half of a packed int).
  uint32_t keepbits = 0, bandbits = 0;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    keepbits |= (sc[i] > hi ? 1u : 0u) << i;
    bandbits |= (sc[i] <= hi && sc[i] >= lo ? 1u : 0u) << i;
  }
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
  int need = kb - (tot >> 16);
  int nb = tot & 0xFFFF;
  const bool in_lds = nb <= kBandCap;
  int32_t* bidx = in_lds ? band_idx_s : P.band_idx + (int64_t)row * P.col_stride;
  {
    int o = cl_off & 0xFFFF;
    for (uint32_t bits = bandbits; bits; bits &= bits - 1) bidx[o++] = jb + __builtin_ctz(bits);
  }
  if (in_lds) lds_barrier(); else __syncthreads();
  double* bscore = in_lds ? band_score_s : P.band_score + (int64_t)row * P.col_stride;
  const int32_t* band = bidx;
  const int groups = NT / 16;  // 16-lane groups: one band entry each at a time
  const int grp = tid >> 4, l16 = tid & 15;

  if (mfma_row && need > 0) {
    // ---- second level: the band's head-folded float32 scores (error <= E_f) select within
    // the band exactly as the first level selected within the row; the rest of the band goes
    // to the float64 re-scoring.
    for (int d = tid; d < kHeadDim; d += NT) {
      float f = qrow[d];
      for (int hh = 1; hh < P.Hi; ++hh) f = f + qrow[hh * kHeadDim + d];
      qfold[d] = f;
    }
    lds_barrier();
    for (int b0 = 0; b0 < nb; b0 += groups) {
      const int b = b0 + grp;
      const float fs = folded_score16(P, qfold, cbt_row, cw, b < nb ? bidx[b] : -1, l16);
      if (l16 == 0 && b < nb) bscore[b] = fs;
    }
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
                            : reinterpret_cast<int32_t*>(P.logits + (int64_t)row * P.col_stride);
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
    nb = s_int[6];
    band = band2;
  }

  // ---- re-score the band in float64, canonical order (16 lanes per entry)
  for (int b0 = 0; b0 < nb; b0 += groups) {
    const int b = b0 + grp;
    const double s = canonical_score16(P, qrow, cbt_row, cw, b < nb ? band[b] : -1, l16);
    if (l16 == 0 && b < nb) bscore[b] = s;
  }
  if (in_lds) lds_barrier(); else __syncthreads();

  // ---- rank the band: keep its `need` best by (score desc, block asc).  A 16-lane group per
  // entry, each lane comparing against every 16th entry, the counts summed on DPP.
  for (int b0 = 0; b0 < nb; b0 += groups) {
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
  const int sel = min(total, kb), count = sel * P.c + tail;
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
    // col / c through a float reciprocal, corrected to the exact quotient (col < 2^24).
    const float rc = 1.0f / (float)P.c;
    for (int col = tid; col <= W; col += NT) {
      int blk = (int)((float)col * rc), m = col - blk * P.c;
      if (m < 0) { --blk; m += P.c; } else if (m >= P.c) { ++blk; m -= P.c; }
      out[col] = col < sel * P.c ? list[blk] * P.c + m
                                 : (col < count ? vis * P.c + (col - sel * P.c)
                                                : (col < W ? -1 : count));
    }
  } else {
    for (int col = sel * P.c + tid; col <= W; col += NT)
      out[col] = col < count ? vis * P.c + (col - sel * P.c) : (col < W ? -1 : count);
  }
}

template <typename C>
hipError_t launch_topk_kernel(const SelectParams& P, size_t mask_bytes, hipStream_t s) {
  hipLaunchKernelGGL((topk_kernel<C>), dim3(P.T), dim3(C::NT), mask_bytes, s, P);
  return hipGetLastError();
}

}  // namespace

TopkLayout topk_layout(const qsa_topk_args& a) {
  TopkLayout L{};
  const int64_t T = a.num_tokens, R = a.num_requests;
  L.cols = a.max_seq_len / a.compress_ratio;
  if (L.cols < 1) L.cols = 1;
  L.col_stride = (L.cols + 63) / 64 * 64;
  L.key_tiles = (L.cols + kLogitsTilesPerWG * kLogitsKeysPerWG - 1) /
                (kLogitsTilesPerWG * kLogitsKeysPerWG);
  auto align = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t off = 0;
  L.off_logits = off;     off = align(off + (size_t)T * L.col_stride * sizeof(float));
  L.key_blocks = (L.cols + 127) / 128;
  L.off_kmax = off;       off = align(off + (size_t)R * L.key_blocks * sizeof(float));
  L.off_band_idx = off;   off = align(off + (size_t)T * L.col_stride * sizeof(int32_t));
  L.off_band_score = off; off = align(off + (size_t)T * L.col_stride * sizeof(double));
  L.off_work = off;       off = align(off + 8 * sizeof(int));
  L.total = off;
  return L;
}

hipError_t launch_topk(const qsa_topk_args& a, const TopkLayout& L, char* ws, hipStream_t s) {
  SelectParams P{};
  P.T = a.num_tokens;
  P.R = a.num_requests;
  P.Hi = a.num_index_heads;
  P.c = a.compress_ratio;
  P.budget = a.budget;
  P.Pc = a.c_page_size;
  P.c_pages = a.c_pages;
  P.cbt_stride = a.c_block_table_stride;
  P.cbt_width = a.c_block_table_width;
  P.cols = L.cols;
  P.col_stride = L.col_stride;
  P.key_tiles = L.key_tiles;
  P.key_blocks = L.key_blocks;
  P.fp8 = a.index_dtype == QSA_DTYPE_FP8_E4M3;
  P.qsl = a.query_start_loc;
  P.seq_lens = a.seq_lens;
  P.q_idx = a.q_idx;
  P.ckv = a.ckv;
  P.cbt = a.c_block_table;
  P.packed = a.packed;
  P.p_rs = a.packed_row_stride;
  P.logits = reinterpret_cast<float*>(ws + L.off_logits);
  P.kmax = reinterpret_cast<float*>(ws + L.off_kmax);
  P.band_idx = reinterpret_cast<int32_t*>(ws + L.off_band_idx);
  P.band_score = reinterpret_cast<double*>(ws + L.off_band_score);
  P.work = reinterpret_cast<int*>(ws + L.off_work);

  // bf16 requests with more than kMfmaMinRows rows are scored on the matrix cores, the others
  // (and every fp8 request) by the VALU kernel; each kernel skips the other's requests.
  const bool mfma = !P.fp8 && a.max_query_len > kMfmaMinRows;
  P.mfma_min_rows = P.fp8 ? INT32_MAX : kMfmaMinRows;
  const int rows_per_chunk = mfma ? kMfmaMinRows : a.max_query_len;
  hipError_t e = P.fp8 ? launch_logits<true>(P, rows_per_chunk, s)
                       : launch_logits<false>(P, rows_per_chunk, s);
  if (e != hipSuccess) return e;
  if (mfma) {
    // One persistent workgroup per CU (a multiple of 8, one set of queues per XCD).
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cus[dev] == 0) {
      int n = 0;
      if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
          n <= 0)
        n = 256;
      cus[dev] = n;
    }
    const int row_blocks = (a.max_query_len + kMfmaRows - 1) / kMfmaRows;
    const unsigned grid = (unsigned)((cus[dev] + 7) / 8 * 8);
    hipLaunchKernelGGL(logits_mfma_kernel, dim3(grid), dim3(512), 0, s, P, row_blocks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const size_t mask_bytes = (size_t)(L.cols + 31) / 32 * sizeof(uint32_t);
  if (P.T >= kTopkPrefillMinRows && L.cols <= TopkPrefill::NT * TopkPrefill::E)
    return launch_topk_kernel<TopkPrefill>(P, mask_bytes, s);
  if (L.cols <= 512 * 8) return launch_topk_kernel<TopkDecode8>(P, mask_bytes, s);
  if (L.cols <= 512 * 16) return launch_topk_kernel<TopkDecode16>(P, mask_bytes, s);
  if (L.cols <= 512 * 32) return launch_topk_kernel<TopkDecode32>(P, mask_bytes, s);
  return launch_topk_kernel<TopkDecode1k>(P, mask_bytes, s);
}

}  // namespace qsa
