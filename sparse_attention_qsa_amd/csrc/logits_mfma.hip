// Indexer logits on the matrix cores for requests with many rows (chunked prefill), per index
// head with the head sum in the fp32 accumulator.  Follows the scoring step of
// QSAIndexer.forward (page "vllm.models.qwen4_exp.nvidia.qsa").
#include <type_traits>

#include "select.h"

namespace qsa {
namespace {
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

// LDS accesses issued as inline assembly, so that the compiler's own wait insertion (which
// cannot tell the targets of the LDS-direct loads apart) does not make them wait for every
// memory operation in flight; each read is waited for before its value is used.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ uint32_t lds_load_u32(const void* p) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p))
               : "memory");
  return v;
}
__device__ __forceinline__ void lds_store_u32(void* p, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}

// Claims the next work item of a queue (a returning global atomic issued as inline assembly:
// the compiler would wait for its result at once, and with it for every store in flight).  The
// result is valid after a vmcnt wait that covers it.
__device__ __forceinline__ uint32_t claim_async(int* counter) {
  uint32_t ret;
  asm volatile("global_atomic_add %0, %1, %2, off sc0"
               : "=v"(ret)
               : "v"((uint64_t)(uintptr_t)counter), "v"(1u)
               : "memory");
  return ret;
}

// Largest value over the wavefront (DPP within rows of 16, then the four row results).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}

// Persistent workgroups (one per CU; the LDS use allows no more) take work items -- (request,
// chunk of up to four row blocks, key tile of 256 keys) -- from eight queues, one per XCD:
// queue x holds the (request, row chunk) pairs x, x+8, ..., each with all its key tiles in
// order, so that the workgroups of one XCD work on the same rows at once and share their Q in
// the XCD's L2.  (Workgroup b takes queue b % 8, which is its XCD under round-robin dispatch;
// any other placement only costs locality.)  An item claims the next one when it starts, and
// loads its key tile once and keeps the
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
  __shared__ uint32_t red[2][8];
  __shared__ __attribute__((aligned(16))) uint8_t kok[kMfmaKeys];
  __shared__ int s_item[2];
  const int key_tiles = (P.cols + kMfmaKeys - 1) / kMfmaKeys;
  const int row_chunks = (row_blocks + kMfmaRowBlocksPerWG - 1) / kMfmaRowBlocksPerWG;
  const int pairs = P.R * row_chunks;
  const int queue = blockIdx.x & 7;
  const int64_t qlen = (int64_t)((pairs - queue + 7) / 8) * key_tiles;  // items of this queue

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, l4 = lane >> 4;
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

  if (tid == 0) s_item[0] = atomicAdd(&P.work[queue], 1);
  __syncthreads();
  for (int it = 0;; ++it) {
    const int64_t item = (int)__builtin_amdgcn_readfirstlane((int)lds_load_u32(&s_item[it & 1]));
    if (item >= qlen) break;  // workgroup-uniform
    uint32_t next = 0;
    if (tid == 0) next = claim_async(&P.work[queue]);
    const int g = queue + 8 * (int)(item / key_tiles);
    const int kt = (int)(item % key_tiles);
    const int rc = g % row_chunks, r = g / row_chunks;

    // Request metadata through the scalar cache (vector loads would wait for the stores in
    // flight).
    const __attribute__((address_space(4))) int32_t* qsl_c =
        (const __attribute__((address_space(4))) int32_t*)P.qsl;
    const __attribute__((address_space(4))) int32_t* sl_c =
        (const __attribute__((address_space(4))) int32_t*)P.seq_lens;
    const int q0 = max(0, min(qsl_c[r], P.T));
    const int n = max(0, min(qsl_c[r + 1], P.T) - q0), L = sl_c[r];
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
    if (n > P.mfma_min_rows && n <= L) {
      while (rb_first < rb_end && !sees_tile(rb_first)) ++rb_first;
    } else {
      rb_first = rb_end;  // decode request, or inert rows
    }
    if (rb_first >= rb_end) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the claim has returned
      if (tid == 0) lds_store_u32(&s_item[(it + 1) & 1], next);
      barrier();
      continue;
    }

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
    if (tid == 0) lds_store_u32(&s_item[(it + 1) & 1], next);
    barrier();

    // ---- this wave's key fragments: keys 64wc + 16kk + lane%16, dims 32ks + 8(lane/16) .. +7
    // (row 64(wc%2) + 16kk + lane%16 of its half: slot (4ks + lane/16) ^ (lane%16)), and the
    // validity of those keys.
    bf16x8_t kfr[4][4];
    uint32_t okk[4];
    {
      const uint8_t* kt_half = wc < 2 ? kl : kh;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint32_t a0 = tile_chunk_addr(kt_half, 64 * (wc & 1) + l16, 4 * ks + l4);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          asm volatile("ds_read_b128 %0, %1" : "=v"(kfr[kk][ks]) : "v"(a0 + 4096u * kk));
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        asm volatile("ds_read_u8 %0, %1"
                     : "=v"(okk[kk])
                     : "v"(lds_addr(kok + 64 * wc + 16 * kk + l16)));
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(kfr[0][0]), "+v"(kfr[0][1]), "+v"(kfr[0][2]),
                   "+v"(kfr[0][3]), "+v"(kfr[1][0]), "+v"(kfr[1][1]), "+v"(kfr[1][2]),
                   "+v"(kfr[1][3]), "+v"(okk[0]), "+v"(okk[1]), "+v"(okk[2]), "+v"(okk[3]));
      asm volatile("" : "+v"(kfr[2][0]), "+v"(kfr[2][1]), "+v"(kfr[2][2]), "+v"(kfr[2][3]),
                   "+v"(kfr[3][0]), "+v"(kfr[3][1]), "+v"(kfr[3][2]), "+v"(kfr[3][3]));
    }
    // ---- max |k| over the valid keys of each 128-key half (upper bounds for the top-k's
    // error band), on the bf16 bit patterns (order-preserving for |k|): per wave, then over
    // the two waves of each half.
    {
      uint32_t mk = 0;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        uint32_t m = 0;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const u32x4_t u = __builtin_bit_cast(u32x4_t, kfr[kk][ks]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t x = u[e] & 0x7FFF7FFFu;
            m = max(m, max(x & 0xFFFFu, x >> 16));
          }
        }
        mk = okk[kk] ? max(mk, m) : mk;
      }
      mk = wave_max_u32(mk);
      if (lane == 0 && wr == 0) lds_store_u32(&red[wc >> 1][wc & 1], mk);
    }
    barrier();  // red[] complete; the key tile is free for slabs 2 and 3
    if (tid < 2 && 2 * kt + tid < P.key_blocks) {
      const uint32_t m = max(lds_load_u32(&red[tid][0]), lds_load_u32(&red[tid][1]));
      P.kmax[(int64_t)r * P.key_blocks + 2 * kt + tid] = __uint_as_float(m << 16);
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

}  // namespace

hipError_t launch_logits_mfma(const SelectParams& P, int max_query_len, hipStream_t s) {
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
  const int row_blocks = (max_query_len + kMfmaRows - 1) / kMfmaRows;
  const unsigned grid = (unsigned)((cus[dev] + 7) / 8 * 8);
  hipLaunchKernelGGL(logits_mfma_kernel, dim3(grid), dim3(512), 0, s, P, row_blocks);
  return hipGetLastError();
}

}  // namespace qsa
