// Fused decode prepare + indexer logits: for a batch of one-row requests whose scoring
// workgroups fit the chip in one round, one launch does the work of qsa_compress (the indexer Q
// prep, the pooling of the group the step completes, the raw-key ring write) and of the
// vector-unit logits kernel (logits.hip), so the step has one launch and one dependency fewer.
// Follows QSAIndexer.forward (page "vllm.models.qwen4_exp.nvidia.qsa"): the prepare of its
// unfused reference path and the scoring of qsa_select_paged_decode.
//
// Grid (workgroups per request, R), 512 threads: workgroup k of request r scores keys
// 2048k .. 2048k+2047 of the request, as logits.hip's wide instance does (or 1024k .. 1024k+1023
// for batches whose 1024-key workgroups fit the chip at one per CU).  Before scoring, it
// computes the row's indexer Q itself (waves 0 .. ceil(Hi/4)-1, one head per 16-lane row, the
// same float64 chain as qsa_compress) into LDS, instead of loading qsa_compress's output; the
// workgroup that holds the key the step completes pools that group (wave 7) and substitutes its
// codes for the cache row it would load; workgroup 0 of each request also writes q_idx and the
// ring (wave 6).  No workgroup reads what another writes in this launch: the substituted key is
// computed where it is scored, and every other scored key is a cache row written before the
// launch.  One-row batches only: row r of the call is request r's row (the host checks that the
// call has one row per request and at most one row in any request).
#include "logits_tile.h"
#include "prep_ops.h"

namespace qsa {
namespace {
using namespace logits_tile;

// TILES: 512-key tiles per workgroup, 4 (the wide layout) or 2 (1024-key workgroups, for
// batches whose workgroups fit the chip at one per CU).
template <bool FP8, int TILES>
__global__ __launch_bounds__(kLogitsThreads) __attribute__((amdgpu_waves_per_eu(2)))
void prep_logits_kernel(SelectParams P, CompressParams C) {
  using KL = KeyLanes<FP8>;
  constexpr int kT = kLogitsThreads, kWaves = kLogitsThreads / 64;
  constexpr int kTiles = TILES;
  static_assert(TILES == 2 || TILES == 4, "two tiles are loaded before the prepare");
  constexpr int kKeys = kTiles * kLogitsKeysPerWG;
  static_assert(kLogitsKeysPerWG == kWaves * 64, "a tile is 64 keys per wave");
  __shared__ int32_t rows_s[kKeys];
  __shared__ float qf_s[kHeadDim];
  // The row's indexer Q codes (head h: the bytes of its q_idx row) and the codes of the key the
  // step completes (the bytes of its cache row), with that key's index in the workgroup.
  __shared__ __attribute__((aligned(16))) uint32_t qc_s[16][kHeadDim / 2];
  __shared__ __attribute__((aligned(16))) uint32_t nk_s[kHeadDim / 2];
  __shared__ int sub_s;
  __shared__ float red[kWaves];
  const int r = blockIdx.y, k = blockIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int jw = k * kKeys;  // first key of the workgroup
  auto barrier = [] {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Indexer Q of a row into qc_s (and q_idx when `store`): waves 0 .. ceil(Hi/4)-1, head
  // 4w + lane/16 on the lane's 16-lane row.  prep_in issues the loads that need only the row;
  // prep_q finishes (the rotation table's loads, the arithmetic, the stores).
  const int nqw = (C.Hi + 3) / 4;
  const int qh = 4 * w + (lane >> 4);
  auto prep_in = [&](int row) {
    return norm_rope_load(C, (int64_t)row * C.Hi + min(qh, C.Hi - 1), (int64_t)C.T * C.Hi,
                          C.Hi, C.qw, lane, [&](int rr, int hh) {
                            return C.q_proj + (int64_t)rr * C.q_rs + hh * 64;
                          });
  };
  auto prep_q = [&](const RowIn& in, const RopeRaw& table, bool store) {
    const int l = lane & 15;
    // The table words pass through here unchanged: nothing that uses them (their widening
    // included) can then move up to the loads, which would wait there for them.
    RopeRaw cs = table;
    asm volatile("" : "+v"(cs.c0), "+v"(cs.s0), "+v"(cs.c1), "+v"(cs.s1));
    float y[8];
    norm_rope_compute(in, cs, C.eps, lane, y);
    if (qh >= C.Hi) return;
    const int64_t v = (int64_t)in.row * C.Hi + qh;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (FP8) {
        const uint16_t code =
            (uint16_t)(f32_to_e4m3(y[2 * kk]) | (f32_to_e4m3(y[2 * kk + 1]) << 8));
        reinterpret_cast<uint16_t*>(qc_s[qh])[l + 16 * kk] = code;
        if (store) reinterpret_cast<uint16_t*>(C.q_idx)[v * 64 + l + 16 * kk] = code;
      } else {
        const uint32_t bits = bf16_pair(y[2 * kk], y[2 * kk + 1]);
        qc_s[qh][l + 16 * kk] = bits;
        if (store) reinterpret_cast<uint32_t*>(C.q_idx)[v * 64 + l + 16 * kk] = bits;
      }
    }
  };

  // ---- one round trip: block-table entries of this thread's keys, the request metadata and
  // the row's Q inputs.
  int col[kKeys / kT], page[kKeys / kT];
#pragma unroll
  for (int i = 0; i < kKeys / kT; ++i) {
    col[i] = (jw + (int)threadIdx.x + kT * i) / P.Pc;
    page[i] = P.cbt[(int64_t)r * P.cbt_stride + min(col[i], P.cbt_width - 1)];
  }
  const int q0 = max(0, min(P.qsl[r], P.T));
  const int n = max(0, min(P.qsl[r + 1], P.T) - q0), L = P.seq_lens[r];
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 8) P.work[threadIdx.x] = 0;
  // By the one-row contract the request's row is row r: its Q inputs go out in the same round
  // trip.
  const int r_row = min(r, P.T - 1);
  // The ring write's inputs (wave 6 of workgroup 0): row r's key and position, the ring page.
  uint32_t ring_key = 0u;
  int64_t ring_pos3 = 0;
  int ring_pg = -1;
  if (w == kWaves - 2 && k == 0) {
    ring_key = C.k_proj[(int64_t)r_row * C.k_rs + lane];
    if (C.mrope && lane < 3) ring_pos3 = C.pos[(int64_t)r_row * 3 + lane];
    ring_pg = C.ring_page[r];
  }
  RowIn qin{};
  if (w < nqw) {
    qin = prep_in(r_row);
    // Waited for here, with the metadata (this round trip completes before the key loads
    // anyway): a wait for them placed after the key loads would wait for those too.
    asm volatile("" ::"v"(qin.u[0]), "v"(qin.u[1]), "v"(qin.u[2]), "v"(qin.u[3]),
                 "v"(qin.wp[0]), "v"(qin.wp[1]), "v"(qin.wp[2]), "v"(qin.wp[3]), "v"(qin.tp.t),
                 "v"(qin.tp.h), "v"(qin.tp.w));
  }
  const int start = L - n;
  const int vis_max = (n > 0 && n <= L) ? min(L / P.c, P.cols) : 0;
  const bool scores = jw < vis_max;  // block-uniform

  // ---- before any key load (a wait for a load also waits for every load issued before it):
  // the Q waves' rotation-table loads; the groups this request's rows complete (wave 7 of the
  // workgroup holding the group's key, the last workgroup for a key past the grid), pooled as
  // qsa_compress does it; the ring write (wave 6 of workgroup 0).
  RopeRaw qcs{};
  if (w < nqw) qcs = norm_rope_table(C, qin, lane);
  if (w == kWaves - 1 && lane == 0) sub_s = -1;  // before this wave's own write below
  // With a 1-D rotation, c <= 8 and one row, the group's loads go out here and its arithmetic
  // runs after the key loads (as the Q waves' does); otherwise the whole group is done here.
  const bool split_group = !C.mrope && C.c <= 8 && n == 1;
  int g_split = -1;
  GroupIn gin{};
  auto publish_group = [&](int g, int gpage, float y0, float y1) {
    if (gpage >= 0 && gpage < C.c_pages)
      store_index_pair(C, C.ckv, (int64_t)gpage * C.Pc + (g % C.Pc), lane, y0, y1);
    if (g >= jw && g < jw + kKeys) {
      if (FP8)
        reinterpret_cast<uint16_t*>(nk_s)[lane] =
            (uint16_t)(f32_to_e4m3(y0) | (f32_to_e4m3(y1) << 8));
      else
        nk_s[lane] = bf16_pair(y0, y1);
      if (lane == 0) sub_s = g - jw;
    }
  };
  if (w == kWaves - 1 && start >= 0) {
    const int rp = C.ring_page[r];
    const bool ring_ok = rp >= 0 && rp < C.ring_pages;
    for (int i = 0; i < n; ++i) {
      const int p = start + i;
      if ((p + 1) % C.c != 0) continue;
      const int g = (p + 1) / C.c - 1;
      if (min(g / kKeys, (int)gridDim.x - 1) != k) continue;
      if (split_group) {
        g_split = g;
        gin = compress_group_load(C, r, q0, start, rp, ring_ok, g, lane);
      } else {
        float y0, y1;
        int gpage;
        compress_group(C, r, q0, start, rp, ring_ok, g, lane, y0, y1, gpage);
        publish_group(g, gpage, y0, y1);
      }
    }
  }
  if (w == kWaves - 2 && k == 0 && start >= 0) {
    if (n == 1 && q0 == r_row) {  // the one-row batch: inputs loaded with the metadata
      const int p = start;
      if (p >= L - C.S && ring_pg >= 0 && ring_pg < C.ring_pages) {
        const int64_t slot = (int64_t)ring_pg * C.S + (p % C.S);
        C.ring[slot * 64 + lane] = ring_key;
        if (C.mrope && lane < 3) C.ring_pos[slot * 3 + lane] = ring_pos3;
      }
    } else {
      for (int i = 0; i < n; ++i) ring_store_row(C, q0 + i, r, start + i, L, lane);
    }
  }

  // ---- the cache rows of the workgroup's keys.  Thread t resolves keys t + 512 i, which are
  // its own wave's keys of every tile, so a wave can load its tiles once its own LDS writes are
  // done: the first two tiles go out before the Q arithmetic and arrive during it.  The loads
  // are unconditional (a workgroup without visible keys loads the cache's first row, masked):
  // behind a branch, the wait for the table words above would also wait for them.
  uint32_t a[2][KL::kLoads][4], ma[2];
#pragma unroll
  for (int i = 0; i < kKeys / kT; ++i) {
    const int j = jw + threadIdx.x + kT * i;
    const bool ok = j < vis_max && col[i] < P.cbt_width && page[i] >= 0 && page[i] < P.c_pages;
    rows_s[threadIdx.x + kT * i] = ok ? page[i] * P.Pc + (j - col[i] * P.Pc) : -1;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  load_key_tile<FP8>(P, rows_s, 0, w, lane, a[0], ma[0]);
  load_key_tile<FP8>(P, rows_s, 1, w, lane, a[1], ma[1]);
  // The row's indexer Q (by the one-row contract, row r), and the split group's arithmetic
  // (its loaded words pass through an empty asm first, as the Q table's do).
  if (w < nqw) prep_q(qin, qcs, k == 0 && r < P.T);
  if (g_split >= 0) {  // wave-uniform
    asm volatile("" : "+v"(gin.page), "+v"(gin.uu[0]), "+v"(gin.uu[1]), "+v"(gin.uu[2]),
                 "+v"(gin.uu[3]), "+v"(gin.uu[4]), "+v"(gin.uu[5]), "+v"(gin.uu[6]),
                 "+v"(gin.uu[7]), "+v"(gin.kw), "+v"(gin.c0), "+v"(gin.s0), "+v"(gin.c1),
                 "+v"(gin.s1));
    float y0, y1;
    compress_group_compute(C, gin, lane, y0, y1);
    publish_group(g_split, gin.page, y0, y1);
  }
  barrier();  // qc_s, nk_s and sub_s written

  float kmax = 0.0f;
  if (scores) {
    const int sub = sub_s;
    // Where the completed key sits in the tiles: tile, wave, load and lane group.
    const int sub_t = sub / kLogitsKeysPerWG, sub_w = (sub % kLogitsKeysPerWG) / 64;
    const int sub_it = (sub % 64) / KL::kKeysPerLoad, sub_g = (sub % 64) % KL::kKeysPerLoad;
    for (int rr0 = 0; rr0 < n; ++rr0) {
      const int row = q0 + rr0;
      if (rr0 > 0) {  // not for a one-row batch: the previous row's readers are done
        barrier();
        load_key_tile<FP8>(P, rows_s, 0, w, lane, a[0], ma[0]);
        load_key_tile<FP8>(P, rows_s, 1, w, lane, a[1], ma[1]);
      }
      if (row != r_row) {  // block-uniform; never for a batch whose row r is request r's
        if (w < nqw) {
          const RowIn in = prep_in(row);
          prep_q(in, norm_rope_table(C, in, lane), false);
        }
        barrier();
      }
      // Head-folded Q: thread d < 128 sums dim d over the heads in order.
      if (threadIdx.x < kHeadDim) {
        const int d = threadIdx.x;
        auto code = [&](int h) {
          return FP8 ? e4m3_to_f32_exact(reinterpret_cast<const uint8_t*>(qc_s[h])[d])
                     : bf16_to_f32(reinterpret_cast<const uint16_t*>(qc_s[h])[d]);
        };
        float f = code(0);
#pragma unroll
        for (int h = 1; h < 16; ++h) f = f + (h < P.Hi ? code(h) : 0.0f);
        qf_s[d] = f;
      }
      barrier();  // qf_s written
      float qf[1][16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        qf[0][i] = i < KL::kDims ? qf_s[(lane % KL::kLanes) * KL::kDims + i] : 0.0f;
      const bool first = rr0 == 0;
      // Two tiles in flight per wave, as in the wide logits instance: tile t + 2 is loaded
      // into t's registers once t is scored.
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        if (sub >= 0 && t == sub_t && w == sub_w) {  // wave-uniform: the completed key's tile
#pragma unroll
          for (int it = 0; it < KL::kLoads; ++it) {
            if (it == sub_it && lane / KL::kLanes == sub_g) {
#pragma unroll
              for (int q = 0; q < 4; ++q) a[t & 1][it][q] = nk_s[4 * (lane % KL::kLanes) + q];
            }
          }
        }
        score_key_tile<FP8, 1, false>(P, a[t & 1], ma[t & 1], qf, 1, row,
                                      jw + t * kLogitsKeysPerWG + w * 64, vis_max, lane, first,
                                      kmax);
        if (t + 2 < kTiles) load_key_tile<FP8>(P, rows_s, t + 2, w, lane, a[t & 1], ma[t & 1]);
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

}  // namespace

namespace {
// The fused kernel's tiles per workgroup for a call: 4 where the plain scoring would use the
// wide layout, 2 where the call's 1024-key workgroups fit the chip at one per CU, else 0 (the
// two calls run instead).
int prep_logits_tiles(const SelectParams& P) {
  if (logits_wide(P, 1, false)) return 4;
  if ((int64_t)P.R * P.key_tiles <= kCUs && P.row_lo == 0 && P.row_hi == P.T) return 2;
  return 0;
}
}  // namespace

bool prep_logits_fusable(const qsa_compress_args& c, const qsa_topk_args& t) {
  // One row per request (row r is request r's: the rows' offsets start at 0 and no request
  // has more than one row), no main-attention prepare, plain-sum aggregation, one window, and
  // the two calls describe the same requests, indexer and compressed cache.
  if (c.main_qkv != nullptr || t.index_agg != QSA_AGG_SUM) return false;
  if (c.num_tokens < 1 || c.num_tokens != c.num_requests || t.num_tokens != c.num_tokens ||
      t.num_requests != c.num_requests || c.max_query_len != 1 || t.max_query_len != 1)
    return false;
  if (c.query_start_loc != t.query_start_loc || c.seq_lens != t.seq_lens ||
      c.q_idx != t.q_idx || c.ckv != t.ckv || c.c_block_table != t.c_block_table ||
      c.c_block_table_stride != t.c_block_table_stride ||
      c.c_block_table_width != t.c_block_table_width || c.c_page_size != t.c_page_size ||
      c.c_pages != t.c_pages || c.num_index_heads != t.num_index_heads ||
      c.compress_ratio != t.compress_ratio || c.index_dtype != t.index_dtype)
    return false;
  // The ring writes cannot alias the group's ring reads (qsa_compress's one-launch plan).
  if ((int64_t)c.max_query_len + c.compress_ratio - 2 >= c.ring_size) return false;
  const TopkLayout L = topk_layout(t);
  if (L.rows != t.num_tokens) return false;
  return prep_logits_tiles(select_params(t, L, nullptr)) != 0;
}

hipError_t launch_prep_logits_topk(const qsa_compress_args& c, const qsa_topk_args& t,
                                   const TopkLayout& L, char* ws, hipStream_t s, Phase phase) {
  const SelectParams P = select_params(t, L, ws);
  const CompressParams C = compress_params(c);
  const int tiles = prep_logits_tiles(P);
  const int keys = tiles * kLogitsKeysPerWG;
  const dim3 grid((P.cols + keys - 1) / keys, P.R), block(kLogitsThreads);
  if (tiles == 4 && P.fp8)
    hipLaunchKernelGGL((prep_logits_kernel<true, 4>), grid, block, 0, s, P, C);
  else if (tiles == 4)
    hipLaunchKernelGGL((prep_logits_kernel<false, 4>), grid, block, 0, s, P, C);
  else if (P.fp8)
    hipLaunchKernelGGL((prep_logits_kernel<true, 2>), grid, block, 0, s, P, C);
  else
    hipLaunchKernelGGL((prep_logits_kernel<false, 2>), grid, block, 0, s, P, C);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || phase == Phase::kFirst) return e;
  return launch_topk_select(P, s);
}

}  // namespace qsa
