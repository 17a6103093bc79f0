// Internal declarations of libqsa: kernel parameter blocks, launchers, and device helpers.
// gfx950 (CDNA4) only: 64-wide wavefronts, OCP fp8, v_dot2c_f32_bf16, bf16/fp8 MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qsa.h"

namespace qsa {

constexpr int kHeadDim = 128;
constexpr int kRotaryDim = 64;
constexpr int kWave = 64;

// ------------------------------------------------------------------------------ launch plans

struct CompressPlan {
  bool fuse_ring;  // ring writes cannot alias this step's ring reads -> one launch
};

// Logits / top-k workspace layout (all offsets in bytes, 256-byte aligned).
struct TopkLayout {
  int32_t cols;           // compressed columns per row (max_seq_len / c, >= 1)
  int32_t col_stride;     // row stride of the per-row arrays (cols rounded up)
  int32_t key_tiles;      // VALU logits workgroups per request (kLogitsTilesPerWG tiles each)
  int32_t key_blocks;     // blocks of 128 keys per request
  int32_t rows;           // rows per window (T without a logits cap): the per-row arrays' rows
  size_t off_logits;      // float  [rows, col_stride] (matrix-core rows: fp16 in the first half)
  size_t off_kmax;        // float  [R, key_blocks]: upper bound of max |k| per block of 128 keys
  size_t off_band_idx;    // int32  [rows, col_stride]
  size_t off_band_score;  // double [rows, col_stride]
  size_t off_work;        // int [8]: work counters of the MFMA kernel
  size_t off_lexp;        // int32  [rows]: scale exponent of each matrix-core row's logits
  size_t total;
};

constexpr int kCUs = 256;              // compute units of an MI355X
constexpr int kLogitsThreads = 512;    // VALU logits workgroup: 8 waves
constexpr int kLogitsKeysPerWG = 512;  // keys per tile: 8 waves x 64 keys
constexpr int kLogitsTilesPerWG = 2;   // tiles walked by one logits workgroup
constexpr int kTopkMaxCols = 32768;    // register-resident top-k: 1024 threads x 32 scores

TopkLayout topk_layout(const qsa_topk_args& a);

struct GqaPlan {
  int32_t tiles;        // ceil(W / 32)
  int32_t splits;       // parts per (row, KV head): workgroups, or waves of one workgroup
  int32_t tiles_per_split;
  bool merge_in_wg;     // the splits are the waves of one workgroup and merged there
  size_t ws_bytes;      // partial outputs + lse when a merge kernel runs, row-tile flags
  int32_t row_tiles;    // tiles of the row-tiled prefill kernel (0: not used)
};

GqaPlan gqa_plan(const qsa_gqa_args& a);

// Launchers (defined next to their kernels).  They assume validated arguments.  A two-kernel
// call runs both phases, or only its first (logits; attention partials) or second (top-k;
// split merge) kernel.
enum class Phase { kAll, kFirst, kSecond };
hipError_t launch_compress(const qsa_compress_args& a, hipStream_t s);
hipError_t launch_topk(const qsa_topk_args& a, const TopkLayout& L, char* ws, hipStream_t s,
                       Phase phase = Phase::kAll);
hipError_t launch_gqa(const qsa_gqa_args& a, const GqaPlan& plan, char* ws, hipStream_t s,
                      Phase phase = Phase::kAll);
// qsa_compress and qsa_index_logits_topk in one scoring launch (prep_logits.hip): whether a
// pair of calls qualifies (one-row requests on the wide vector-unit layout, the two calls
// describing the same requests and caches), and the fused launch (kFirst: without the top-k).
bool prep_logits_fusable(const qsa_compress_args& c, const qsa_topk_args& t);
hipError_t launch_prep_logits_topk(const qsa_compress_args& c, const qsa_topk_args& t,
                                   const TopkLayout& L, char* ws, hipStream_t s,
                                   Phase phase = Phase::kAll);
// The allocation-free attention call's static scratch (gqa.hip): its size, and the device
// address of the current device's copy (looked up on the first call on each device).
constexpr size_t kGqaScratchBytes = size_t(40) << 20;
hipError_t gqa_scratch(char** ptr);
hipError_t launch_diag_e4m3(float* out, hipStream_t s);
hipError_t launch_diag_fp64(const double* in, double* out, int64_t n, hipStream_t s);
hipError_t launch_diag_read(const void* src, const int32_t* idx, int64_t n, int32_t chunk_bytes,
                            uint32_t* sink, hipStream_t s);

// ------------------------------------------------------------------------------ device helpers

__device__ __forceinline__ float bf16lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16hi(uint32_t pair) {
  return __uint_as_float(pair & 0xFFFF0000u);
}
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16 bits, round to nearest even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// double -> float (RNE, hardware) -> bf16 (RNE): the canonical rounding chain.
__device__ __forceinline__ uint32_t f64_to_bf16(double d) { return f32_to_bf16((float)d); }

// bf16-valued float -> OCP e4m3fn code: round to nearest even on the e4m3fn grid extended by
// the would-be value 480 of code 0x7F; a result at or beyond it, or NaN, gives the NaN code.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (!(a == a)) return sign | 0x7Fu;
  if (a < 0.015625f) {                               // below 2^-6: grid step 2^-9
    return sign | (uint32_t)rintf(a * 512.0f);       // 0..8 (8 encodes 2^-6)
  }
  int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;
  if (e > 8) return sign | 0x7Fu;
  int q = (int)rintf(ldexpf(a, 3 - e));             // 8..16
  if (q == 16) { e += 1; q = 8; }
  const int code = (e + 7) * 8 + (q - 8);
  return code >= 0x7F ? (sign | 0x7Fu) : (sign | (uint32_t)code);
}

// e4m3fn code -> value, from the definition (exact; used where float64 exactness matters).
__device__ __forceinline__ float e4m3_to_f32_exact(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  float mag = (e == 0) ? (float)m * 0.001953125f : ldexpf(1.0f + (float)m * 0.125f, (int)e - 7);
  if ((c & 0x7Fu) == 0x7Fu) mag = __uint_as_float(0x7FC00000u);
  return (c & 0x80u) ? -mag : mag;
}

__device__ __forceinline__ double shfl_xor_f64(double v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Stages the row offsets qsl[0..R] in LDS (when they fit) so that request lookups do not
// chain dependent global loads.  Every thread of the block must call it.
constexpr int kQslCap = 2048;
__device__ __forceinline__ const int32_t* stage_qsl(const int32_t* qsl, int R, int32_t* lds) {
  if (R + 1 > kQslCap) return qsl;
  for (int i = threadIdx.x; i <= R; i += blockDim.x) lds[i] = qsl[i];
  __syncthreads();
  return lds;
}

// Request owning `row`, by binary search over the row offsets [R+1]; -1 if none.
__device__ __forceinline__ int find_request(const int32_t* qsl, int R, int row) {
  int lo = 0, hi = R;  // invariant: answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (qsl[mid] <= row) lo = mid; else hi = mid;
  }
  if (R <= 0 || qsl[lo] > row || qsl[lo + 1] <= row) return -1;
  return lo;
}

}  // namespace qsa
