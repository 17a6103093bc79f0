// Indexer logits on the matrix cores for requests with many rows (chunked prefill), per index
// head with the head sum in the fp32 accumulator.  Follows the scoring step of
// QSAIndexer.forward (page "vllm.models.qwen4_exp.nvidia.qsa").
#include <type_traits>

#include "select.h"

namespace qsa {
namespace {
// Requests with many rows (chunked prefill) are scored on the matrix cores with the heads
// folded into Q: f = sum_h q_h (float32, heads in order), split into three bf16 terms
// hi = bf16(f), mid = bf16(f - hi), lo = bf16(f - hi - mid) (each difference exact in float32;
// |f - hi - mid - lo| <= 2^-24 |f|), and S = (hi + mid + lo) . k (bf16 products are exact in
// fp32).  The hi products of each 32-dim k-step are summed in an accumulator of their own (32
// terms), the mid and lo products of all dims in one more (their size is 2^-8 of hi's), and the
// five partial sums are added on the vector unit.  Against the exact score sum_h q_h . k the
// result is off by at most C kappa A with
// C = g_fold + (2^-24 + g'_34 (1 + 2^-7) + g'_258 2^-7 + g_4 (1 + 2^-6)) (1 + g_fold)
// (g with u = 2^-24: the fold over Hi-1 additions and the final 4; g' with u = 2^-23: the
// matrix-core sums, whose order and rounding are not specified); the top-k's band covers that.
// One contraction of length 384 instead of one of length 128 per head: fewer matrix-core
// operations than the per-head form and a bound below the vector-unit logits' own.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaRows = 128;         // rows per row block: 8 waves x 16 rows
constexpr int kMfmaKeys = 256;         // keys per tile
constexpr int kMfmaTilesPerItem = 8;   // key tiles per work item (at most)

__device__ __forceinline__ void lds_dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// Key tiles in LDS hold rows of 256 bytes; key t's 16-byte chunk c sits in slot c ^ (t & 15),
// so that 16 lanes reading chunk c of 16 consecutive keys hit 16 different slots.  They are
// filled by LDS-direct loads: a load writes 4 keys (1 KiB), lane L landing in key L/16, slot
// L%16.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Waits until at most n VMEM operations of this wave are outstanding, n rounded down to a
// multiple of 4 (at most 60): rounding down only makes the wait stricter.
__device__ __forceinline__ void wait_vmcnt(int n) {
#define QSA_VMCNT(i)                                                                 \
  case i:                                                                            \
    __builtin_amdgcn_s_waitcnt(((4 * i) & 15) | (((4 * i) >> 4) << 14) | 0x0F70); \
    break;
  switch (n < 0 ? 0 : (n >= 60 ? 15 : n >> 2)) {
    QSA_VMCNT(0) QSA_VMCNT(1) QSA_VMCNT(2) QSA_VMCNT(3) QSA_VMCNT(4) QSA_VMCNT(5)
    QSA_VMCNT(6) QSA_VMCNT(7) QSA_VMCNT(8) QSA_VMCNT(9) QSA_VMCNT(10) QSA_VMCNT(11)
    QSA_VMCNT(12) QSA_VMCNT(13) QSA_VMCNT(14) QSA_VMCNT(15)
  }
#undef QSA_VMCNT
}

// Two float32 values rounded to nearest even as fp16, packed low then high (one
// v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t f16_pack_rne(float lo, float hi) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  const f16x2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// LDS accesses issued as inline assembly, so that the compiler's own wait insertion (which
// cannot tell the targets of the LDS-direct loads apart) does not make them wait for every
// memory operation in flight; each read is waited for before its value is used.
__device__ __forceinline__ uint32_t lds_load_u32(const void* p) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p))
               : "memory");
  return v;
}
__device__ __forceinline__ void lds_store_u32(void* p, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
// Four LDS words at a, b, c, d (byte addresses), one wait.
template <int N>
__device__ __forceinline__ void lds_load_u32x4(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                               int (&o)[N], int k) {
  // Early-clobber outputs: a read's destination must not be the address register of a read
  // issued after it, whose address the returning data could otherwise overwrite.
  asm volatile("ds_read_b32 %0, %4\n\tds_read_b32 %1, %5\n\tds_read_b32 %2, %6\n\t"
               "ds_read_b32 %3, %7\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(o[k]), "=&v"(o[k + 1]), "=&v"(o[k + 2]), "=&v"(o[k + 3])
               : "v"(a), "v"(b), "v"(c), "v"(d)
               : "memory");
}

// Claims the next work item (a returning global atomic issued as inline assembly: the
// compiler would wait for its result at once, and with it for every store in flight).  The
// result is valid after a vmcnt wait that covers it.
__device__ __forceinline__ uint32_t claim_async(int* counter) {
  uint32_t ret;
  asm volatile("global_atomic_add %0, %1, %2, off sc0"
               : "=v"(ret)
               : "v"((uint64_t)(uintptr_t)counter), "v"(1u)
               : "memory");
  return ret;
}

// Persistent workgroups (one per CU; the LDS use allows no more) take work items from one
// queue.  An item is (request, row block of 128 rows, up to `tpi` <= 8 consecutive 256-key
// tiles the block sees); the items of every row block's first tiles come first, the later
// tiles of the longest rows next, so that the big items are claimed first.  The next item is
// claimed when an item starts.
//
// The item's folded Q stays in registers: wave w holds rows 16w .. 16w+15 of the block, the
// three terms of all 128 dims, as the B operand of v_mfma_f32_16x16x32_bf16.  Key tiles
// (64 KiB) stream through two LDS buffers, loaded LDS-direct one tile ahead, so a tile costs
// one barrier.  A wave multiplies a tile four 16-key groups at a time -- 4 x 4 k-steps x 3
// terms of MFMAs into five accumulators per group, the A operand (16 keys x 32 dims) read
// from LDS --
// and stores each group's 16 rows x 16 keys as soon as it is final: the logits leave a store
// per 128 MFMAs instead of in bursts, so that they do not stall the key loads behind them.
// Stores are buffer stores whose range ends at the block's last row; keys a row does not see
// go to an out-of-range offset and are dropped.  The logits leave as fp16, scaled by a power
// of two per row that keeps them in range (rounded to nearest even; the row keeps its
// float32-sized stride): half the bytes of float32, and the top-k's band absorbs the rounding
// (at most 2^-11 of the stored value, or half the smallest subnormal step).
// F8: e4m3 indexer (128-byte key rows): the key codes are converted to bf16 as the fragments are
// read (exact: every e4m3 value is a bf16 value), Q is folded from its codes (exact in fp32),
// and the contraction and its bound are those of the bf16 instance.
template <bool F8>
__global__ __launch_bounds__(512) void logits_mfma_kernel(SelectParams P, int row_blocks,
                                                          int tpi) {
  using frag_t = std::conditional_t<F8, long, bf16x8_t>;  // 8 values of one operand row
  constexpr int kRowB = F8 ? 128 : 256;       // bytes of a key row
  constexpr int kChunks = kRowB / 16;         // its 16-byte chunks
  constexpr int kKeysPerLoad = 1024 / kRowB;  // keys one LDS-direct load instruction fills
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][kMfmaKeys * kRowB];
  __shared__ __attribute__((aligned(16))) uint8_t kok[2][kMfmaKeys];
  // The item's compressed-block-table entries (columns col0 ..), read once per item, so that a
  // tile's loads need no global round trip (whose wait would also drain the logit stores).
  constexpr int kPgCap = kMfmaTilesPerItem * kMfmaKeys + 1;
  __shared__ int32_t pg_s[kPgCap];
  // Per wave, one batch of logits (16 rows x 64 keys, fp16) on its way out: the batch is
  // written here as the matrix-core layout has it (4 keys of one row per lane) and read back
  // as 16-byte row pieces, so that a store instruction writes 8 whole 128-byte row segments
  // instead of 16 rows x 32 bytes.  16-byte chunk c of row r sits in slot c ^ (r & 7).
  __shared__ __attribute__((aligned(16))) uint8_t stg[kMfmaRows / 16][16 * 128];
  __shared__ int s_item[2];
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, l4 = lane >> 4;
  const int key_tiles = (P.cols + kMfmaKeys - 1) / kMfmaKeys;
  const int chunks = (key_tiles + tpi - 1) / tpi;
  // The queue covers the requests whose rows meet this launch's rows [row_lo, row_hi): r_lo ..
  // r_lo + nreq - 1 (the requests' rows are consecutive and in order), and per request at
  // most bw row blocks from rb_first (the first request's block holding row_lo, else 0).  A
  // call that is one window covers every request and row block.
  const bool windowed = P.row_lo > 0 || P.row_hi < P.T;
  int r_lo = 0, nreq = P.R, bw = row_blocks;
  if (windowed) {  // block-uniform
    int before = 0, started = 0;
    for (int b0 = 0; b0 < P.R; b0 += 512) {
      const int i = b0 + tid;
      before += __syncthreads_count(i < P.R && P.qsl[i + 1] <= P.row_lo);
      started += __syncthreads_count(i < P.R && P.qsl[i] < P.row_hi);
    }
    r_lo = before;
    nreq = max(started - before, 0);
    bw = min(row_blocks, (P.row_hi - P.row_lo + kMfmaRows - 1) / kMfmaRows + 1);
  }
  const int per_chunk = nreq * bw;
  const int64_t qlen = (int64_t)per_chunk * chunks;

  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const char* ckv = reinterpret_cast<const char*>(P.ckv);
  const char* qb = reinterpret_cast<const char*>(P.q_idx);
  const __attribute__((address_space(4))) int32_t* qsl_c =
      (const __attribute__((address_space(4))) int32_t*)P.qsl;
  const __attribute__((address_space(4))) int32_t* sl_c =
      (const __attribute__((address_space(4))) int32_t*)P.seq_lens;
  // Barrier without a memory fence (a fence would wait for every load in flight); LDS
  // operations are complete before it, and the loads into LDS are waited for explicitly.
  auto barrier = [] {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // This lane's A-operand address in buffer b for k-step ks: key l16 of the group (the group
  // is an offset of 4 KiB), chunk 4ks + l4.
  // (fp8: the 8 codes of dims 32ks + 8 l4 are half of chunk 2ks + l4/2.)
  uint32_t kaddr[2][4];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      kaddr[b][ks] = F8 ? lds_addr(kbuf[b] + l16 * kRowB + 16 * ((2 * ks + (l4 >> 1)) ^ (l16 & 7)) +
                                   8 * (l4 & 1))
                        : lds_addr(kbuf[b] + l16 * kRowB + 16 * ((4 * ks + l4) ^ l16));
  }

  if (tid == 0) s_item[0] = atomicAdd(&P.work[0], 1);
  __syncthreads();
  for (int it = 0;; ++it) {
    const int64_t item = (int)__builtin_amdgcn_readfirstlane((int)lds_load_u32(&s_item[it & 1]));
    if (item >= qlen) break;  // workgroup-uniform
    uint32_t next = 0;
    if (tid == 0) next = claim_async(&P.work[0]);
    const int chunk = (int)(item / per_chunk), jj = (int)(item % per_chunk);
    const int r = r_lo + jj % nreq;
    const int q0 = max(0, min(qsl_c[r], P.T));
    const int n = max(0, min(qsl_c[r + 1], P.T) - q0), L = sl_c[r];
    const int rb_first = r == r_lo ? max(P.row_lo - q0, 0) / kMfmaRows : 0;
    const int rb = rb_first + (chunk == 0 ? jj / nreq : bw - 1 - jj / nreq);
    int t0 = 0, t1 = 0, nrows = 0, pbase = 0, wlo = 0, whi = 0;
    if (n > P.mfma_min_rows && n <= L && rb * kMfmaRows < n) {
      nrows = min(kMfmaRows, n - rb * kMfmaRows);
      pbase = L - n + rb * kMfmaRows;  // position of the block's first row
      // The block's rows in this launch's window: [wlo, whi) of its nrows.
      const int blk0 = q0 + rb * kMfmaRows;
      wlo = min(max(P.row_lo - blk0, 0), nrows);
      whi = min(max(P.row_hi - blk0, 0), nrows);
      if (wlo >= whi) nrows = 0;
    }
    if (nrows > 0) {
      const int vis_hi = min((pbase + whi) / P.c, P.cols);
      t0 = chunk * tpi;
      t1 = min(t0 + tpi, (vis_hi + kMfmaKeys - 1) / kMfmaKeys);
    }
    if (t0 >= t1) {  // decode request, inert rows, or no tile of this chunk is seen
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the claim has returned
      if (tid == 0) lds_store_u32(&s_item[(it + 1) & 1], next);
      barrier();
      continue;
    }
    const int vis_max = min(L / P.c, P.cols);
    barrier();  // every wave is done with the previous item's buffers
    // Block-table columns of the item's visible keys [t0 * 256, min(t1 * 256, vis_max)).
    const int col0 = (t0 * kMfmaKeys) / P.Pc;
    {
      const int kend = min(t1 * kMfmaKeys, vis_max);
      const int ncol = kend > t0 * kMfmaKeys ? (kend - 1) / P.Pc - col0 + 1 : 0;
      for (int c = tid; c < ncol; c += 512)
        pg_s[c] = P.cbt[(int64_t)r * P.cbt_stride + min(col0 + c, P.cbt_width - 1)];
    }
    barrier();  // the item's pages are in LDS
    // This lane's row of the block and the keys it sees.
    const int trow = 16 * w + l16;  // the row of this lane's matrix-core results
    // The rows this lane stores from the staging buffer: 16 w + (lane / 8) + 8 s, s < 2, keys
    // 8 (lane % 8) .. +7 of each batch; their visible limits and offsets in the window.
    int vis_s[2], roff_s[2];
#pragma unroll
    for (int sr = 0; sr < 2; ++sr) {
      const int br = 16 * w + (lane >> 3) + 8 * sr;
      vis_s[sr] = br >= wlo && br < whi ? min((pbase + br + 1) / P.c, P.cols) : 0;
      roff_s[sr] = (br - wlo) * P.col_stride * 4;
    }
    const uint32_t stg_base = lds_addr(stg[w]);

    // ---- key tile kt into buffer b: LDS-direct loads of 1 KiB, 32 / kKeysPerLoad per wave
    // (wave w: keys 32w .. 32w+31; a load's lane L lands in key L / kChunks, slot L % kChunks);
    // a key that is not visible or whose page is outside the cache loads the cache's first
    // row and is flagged (its logits are written as zero).
    auto load_tile = [&](int kt, int b) __attribute__((always_inline)) {
      constexpr int kL = 32 / kKeysPerLoad;
      const int kin = lane / kChunks, slot = lane % kChunks;
      int page[kL];
      uint32_t pa[kL];
#pragma unroll
      for (int i = 0; i < kL; ++i) {
        const int jk = kt * kMfmaKeys + 32 * w + kKeysPerLoad * i + kin;
        // Visible keys have their column in pg_s; the others are masked below.
        const int ci = jk < vis_max ? jk / P.Pc - col0 : 0;
        pa[i] = lds_addr(&pg_s[ci]);
      }
#pragma unroll
      for (int i = 0; i < kL; i += 4) lds_load_u32x4(pa[i], pa[i + 1], pa[i + 2], pa[i + 3], page, i);
#pragma unroll
      for (int i = 0; i < kL; ++i) {
        const int j = 32 * w + kKeysPerLoad * i + kin, jk = kt * kMfmaKeys + j;
        const bool ok = jk < vis_max && jk / P.Pc < P.cbt_width && page[i] >= 0 &&
                        page[i] < P.c_pages;
        const int64_t off = ok ? ((int64_t)page[i] * P.Pc + jk % P.Pc) * kRowB : 0;
        lds_dma16(ckv + off + 16 * (slot ^ (j & (kChunks - 1))),
                  kbuf[b] + (32 * w + kKeysPerLoad * i) * kRowB);
        if (slot == 0) kok[b][j] = ok;
      }
    };
    load_tile(t0, t0 & 1);

    // ---- folded Q of this wave's rows (rows past the request repeat its last row): lane
    // (l16, l4) holds dims 32 ks + 8 l4 .. +7 of row l16 for each k-step ks, as the hi, mid and
    // lo bf16 terms of f = sum_h q_h (float32, heads in order 0 .. Hi-1).
    bf16x8_t qhi[4], qmid[4], qlo[4];
    // The row's logits are stored as fp16 scaled by 2^-erow: every score satisfies
    // |s| <= kappa * A (kappa = max |k| over the request's keys, from the per-block bounds the
    // vector-unit kernel wrote before this one; A = sum |q| of the row, its heads unfolded), and
    // erow makes kappa * A * 2^-erow < 2^15, inside the fp16 range with room to spare.
    int erow = 0;
    float km = 0.0f;  // this lane's share of kappa, loaded with Q (one round trip)
    {
      const int nkb = min(P.key_blocks, (min(L / P.c, P.cols) + 127) / 128);
      for (int bk = lane; bk < nkb; bk += 64)
        km = fmaxf(km, P.kmax[(int64_t)r * P.key_blocks + bk]);
    }
    {
      const int t = min(trow, nrows - 1);
      float qabs = 0.0f;  // sum |q| over this lane's dims of the row, all heads
      const char* qrow = qb + (int64_t)(q0 + rb * kMfmaRows + t) * P.Hi * kHeadDim * (F8 ? 1 : 2);
      float f[4][8];  // +0 plus the heads in order (a zero's sign changes no score)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[ks][e] = 0.0f;
      }
      // Four heads at a time: their loads for all four k-steps are in flight together.
      for (int hb = 0; hb < P.Hi; hb += 4) {  // workgroup-uniform
        uint4 raw[4][4];
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
          const int h = min(hb + hh, P.Hi - 1);
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            if constexpr (F8) {
              const uint2 u = *reinterpret_cast<const uint2*>(
                  qrow + (int64_t)(h * kHeadDim + 32 * ks + 8 * l4));
              raw[hh][ks] = make_uint4(u.x, u.y, 0u, 0u);
            } else {
              raw[hh][ks] = *reinterpret_cast<const uint4*>(
                  qrow + (int64_t)(h * kHeadDim + 32 * ks + 8 * l4) * 2);
            }
          }
        }
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
          const bool use = hb + hh < P.Hi;  // workgroup-uniform
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            float x[8];
            if constexpr (F8) {
              const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(raw[hh][ks].x, false);
              const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(raw[hh][ks].x, true);
              const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(raw[hh][ks].y, false);
              const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(raw[hh][ks].y, true);
              x[0] = a[0]; x[1] = a[1]; x[2] = b[0]; x[3] = b[1];
              x[4] = c[0]; x[5] = c[1]; x[6] = d[0]; x[7] = d[1];
            } else {
              const uint32_t w4[4] = {raw[hh][ks].x, raw[hh][ks].y, raw[hh][ks].z,
                                      raw[hh][ks].w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                x[2 * e] = __uint_as_float(w4[e] << 16);
                x[2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u);
              }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              f[ks][e] = f[ks][e] + (use ? x[e] : 0.0f);
              qabs = qabs + (use ? fabsf(x[e]) : 0.0f);
            }
          }
        }
      }
      // The row's A: its four lanes' sums (float32 sums of at most 512 terms, widened by 2^-6
      // so that they bound the exact sum), then the exponent.
      qabs = qabs + __shfl_xor(qabs, 16, 64);
      qabs = qabs + __shfl_xor(qabs, 32, 64);
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) km = fmaxf(km, __shfl_xor(km, m, 64));
      const float bound = km * qabs * (1.0f + 0x1p-6f);
      if (!(bound < 0x1p126f)) erow = 127;  // huge or not finite: scaled to nothing
      else erow = max(0, __builtin_amdgcn_frexp_expf(bound) - 15);
      const int grow = q0 + rb * kMfmaRows + trow;  // the call row of this lane's results
      if (l4 == 0 && trow >= wlo && trow < whi) P.lexp[grow - P.row_lo] = erow;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {  // each difference below is exact in float32
          const __bf16 hv = (__bf16)f[ks][e];
          const float r1 = f[ks][e] - (float)hv;
          const __bf16 mv = (__bf16)r1;
          qhi[ks][e] = hv;
          qmid[ks][e] = mv;
          qlo[ks][e] = (__bf16)(r1 - (float)mv);
        }
      }
    }
    // Logits rows are relative to the window: the record starts at the block's first row in
    // it and ends at its last.
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        P.logits + (int64_t)(q0 + rb * kMfmaRows + wlo - P.row_lo) * P.col_stride, 0,
        (whi - wlo) * P.col_stride * 4, 0x00020000);

    // Stores this wave issued while multiplying the previous tile (after this tile's loads,
    // which were issued at the start of that step): they may stay in flight.
    int st_prev = 0;
    for (int kt = t0; kt < t1; ++kt) {
      const int b = kt & 1;
      // Tile kt has landed once only the stores issued after its loads are outstanding.
      wait_vmcnt(st_prev);
      if (kt == t0 && tid == 0) lds_store_u32(&s_item[(it + 1) & 1], next);
      barrier();  // tile kt visible; every wave is done with tile kt-1 (buffer b ^ 1)
      if (kt + 1 < t1) load_tile(kt + 1, b ^ 1);
      int st = 0;
      // Groups of four 16-key blocks; the A fragments of the next k-step are read while the
      // current one is multiplied.
      frag_t kf[2][4];
      // Eight e4m3 codes (one 64-bit fragment) as bf16, exactly.
      auto to_bf16 = [](frag_t v) __attribute__((always_inline)) {
        if constexpr (F8) {
          const uint32_t w0 = (uint32_t)(uint64_t)v, w1 = (uint32_t)((uint64_t)v >> 32);
          const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false);
          const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
          const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false);
          const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
          bf16x8_t r;
          r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)b[0]; r[3] = (__bf16)b[1];
          r[4] = (__bf16)c[0]; r[5] = (__bf16)c[1]; r[6] = (__bf16)d[0]; r[7] = (__bf16)d[1];
          return r;
        } else {
          return v;
        }
      };
      auto read_kf = [&](int kg0, int ks, frag_t (&dst)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (F8)
            asm volatile("ds_read_b64 %0, %1"
                         : "=v"(dst[q])
                         : "v"(kaddr[b][ks] + (uint32_t)(16 * kRowB) * (kg0 + q)));
          else
            asm volatile("ds_read_b128 %0, %1"
                         : "=v"(dst[q])
                         : "v"(kaddr[b][ks] + (uint32_t)(16 * kRowB) * (kg0 + q)));
        }
      };
      read_kf(0, 0, kf[0]);
#pragma unroll
      for (int kg0 = 0; kg0 < 16; kg0 += 4) {
        // ah: the hi products of k-step ks (32 terms each); al: every mid and lo product.
        f32x4_t ah[4][4], al[4];
        const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int q = 0; q < 4; ++q) al[q] = zero;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          frag_t(&cur)[4] = kf[ks & 1];
          asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(cur[0]), "+v"(cur[1]), "+v"(cur[2]),
                       "+v"(cur[3]));
          if (ks < 3) {
            read_kf(kg0, ks + 1, kf[(ks + 1) & 1]);
          } else if (kg0 + 4 < 16) {
            read_kf(kg0 + 4, 0, kf[(ks + 1) & 1]);
          }
          bf16x8_t ka[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) ka[q] = to_bf16(cur[q]);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            ah[q][ks] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[q], qhi[ks], zero, 0, 0, 0);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            al[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[q], qmid[ks], al[q], 0, 0, 0);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            al[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[q], qlo[ks], al[q], 0, 0, 0);
        }
        f32x4_t acc[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[q] = ((ah[q][0] + ah[q][1]) + (ah[q][2] + ah[q][3])) + al[q];
        // Groups kg0 .. kg0+3 are final: element e of group kg is key 16kg + 4(lane/16) + e
        // of row trow; keys that were not loaded are written as zero.
        uint32_t okm[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          asm volatile("ds_read_b32 %0, %1"
                       : "=v"(okm[q])
                       : "v"(lds_addr(&kok[b][16 * (kg0 + q) + 4 * l4])));
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(okm[0]), "+v"(okm[1]), "+v"(okm[2]),
                     "+v"(okm[3]), "+v"(kf[0][0]), "+v"(kf[0][1]), "+v"(kf[0][2]),
                     "+v"(kf[0][3]));
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4_t v = acc[q];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (!((okm[q] >> (8 * e)) & 0xFFu)) v[e] = 0.0f;
          }
          // Keys 16 q + 4 l4 .. +3 of row l16: bytes 32 q + 8 l4 of its 128-byte batch row.
          const u32x2_t pk = {f16_pack_rne(__builtin_amdgcn_ldexpf(v[0], -erow),
                                           __builtin_amdgcn_ldexpf(v[1], -erow)),
                              f16_pack_rne(__builtin_amdgcn_ldexpf(v[2], -erow),
                                           __builtin_amdgcn_ldexpf(v[3], -erow))};
          const uint32_t a = stg_base + l16 * 128 + 16 * ((2 * q + (l4 >> 1)) ^ (l16 & 7)) +
                             8 * (l4 & 1);
          asm volatile("ds_write_b64 %0, %1" ::"v"(a), "v"(pk) : "memory");
        }
        u32x4_t piece[2];
#pragma unroll
        for (int sr = 0; sr < 2; ++sr) {
          const int r16 = (lane >> 3) + 8 * sr, c = lane & 7;
          asm volatile("ds_read_b128 %0, %1"
                       : "=v"(piece[sr])
                       : "v"(stg_base + r16 * 128 + 16 * (c ^ (r16 & 7))));
        }
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(piece[0]), "+v"(piece[1]));
        // A row piece of 8 keys is written when its first key is visible to the row (the rest
        // lies inside the row's stride, past its visible keys, where the top-k does not read).
#pragma unroll
        for (int sr = 0; sr < 2; ++sr) {
          const int j = kt * kMfmaKeys + 16 * kg0 + 8 * (lane & 7);
          const uint32_t off = j < vis_s[sr] ? (uint32_t)(roff_s[sr] + j * 2) : 0xFFFFFFF0u;
          __builtin_amdgcn_raw_buffer_store_b128(piece[sr], rs, off, 0, 0);
          ++st;
        }
      }
      st_prev = st;
    }
  }
}

}  // namespace

// Tiles per item: eight (an item's setup, its claim and its block-table and Q round trips,
// costs about as much as two tiles), halved while the launch's rows would make fewer items
// than there are workgroups (a short call, or one window of a call under a logits cap), so
// that the work still spreads over the chip.
static int mfma_tiles_per_item(const SelectParams& P, unsigned workgroups) {
  const int64_t blocks = ((int64_t)(P.row_hi - P.row_lo) + kMfmaRows - 1) / kMfmaRows;
  const int key_tiles = (P.cols + kMfmaKeys - 1) / kMfmaKeys;
  int tpi = kMfmaTilesPerItem;
  while (tpi > 1 && blocks * ((key_tiles + tpi - 1) / tpi) < (int64_t)workgroups) tpi /= 2;
  return tpi;
}

hipError_t launch_logits_mfma(const SelectParams& P, int max_query_len, hipStream_t s) {
  // One persistent workgroup per CU.
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
  const int row_blocks = (max_query_len + kMfmaRows - 1) / kMfmaRows;
  const unsigned grid = (unsigned)cus[dev];
  const int tpi = mfma_tiles_per_item(P, grid);
  if (P.fp8)
    hipLaunchKernelGGL(logits_mfma_kernel<true>, dim3(grid), dim3(512), 0, s, P, row_blocks,
                       tpi);
  else
    hipLaunchKernelGGL(logits_mfma_kernel<false>, dim3(grid), dim3(512), 0, s, P, row_blocks,
                       tpi);
  return hipGetLastError();
}

}  // namespace qsa
