// The indexer prepare of qsa_compress as device functions: the parameter block, the canonical
// float64 chain (RMSNorm with halving sums, NeoX RoPE, the casts) on a wave (one 128-dim vector,
// lane l holding dims 2l, 2l+1) or on a 16-lane row, and the pooling of a completed key group.
// Used by the compress kernels (compress.hip) and by the fused decode prepare + logits kernel
// (prep_logits.hip), so both write the same bytes.  Follows QSAIndexer.forward's unfused
// reference path (page "vllm.models.qwen4_exp.nvidia.qsa") and qsa_compress_groups_with_ratio
// (page "vllm.models.qwen4_exp.nvidia.ops.qsa").
//
// The chain needs floating-point contraction off; this header turns it off for the rest of the
// including file.
#pragma once

#include "qsa_internal.h"

#pragma clang fp contract(off)

namespace qsa {

struct CompressParams {
  int T, R, Hi, c, S, ring_pages, Pc, c_pages, cbt_stride, cbt_width, max_pos;
  int sec_h, sec_w;  // MRoPE sections (H, W); T takes the remaining frequencies
  bool mrope, fp8, fuse_ring;
  const int32_t* qsl;
  const int32_t* seq_lens;
  const uint32_t* q_proj;  // bf16 pairs
  int64_t q_rs;            // row stride in pairs
  const uint32_t* k_proj;
  int64_t k_rs;
  const int64_t* pos;
  const float* cos_sin;
  const uint16_t* qw;
  const uint16_t* kw;
  double eps;
  uint32_t* ring;  // bf16 pairs [ring_pages, S, 64]
  int64_t* ring_pos;
  const int32_t* ring_page;
  void* ckv;
  const int32_t* cbt;
  void* q_idx;
  // main-attention prepare (main == false: none)
  bool main, main_fp8;
  int Hq, Hkv, m_pages, m_P;
  const uint32_t* mqkv;  // bf16 pairs
  int64_t m_rs;          // row stride in pairs
  const uint16_t* mqw;
  const uint16_t* mkw;
  double m_eps;
  uint32_t* mq;  // bf16 pairs [T, Hq, 64]
  void* mcache;
  int64_t m_ps, m_hs, m_ts;  // strides in elements
  const int64_t* slots;
  float k_scale, v_scale;
};

// Position axis (0 = T, 1 = H, 2 = W) of rotary frequency f under interleaved MRoPE.
__device__ __forceinline__ int mrope_axis(int f, int sec_h, int sec_w) {
  if (f % 3 == 1 && f < 3 * sec_h) return 1;
  if (f % 3 == 2 && f < 3 * sec_w) return 2;
  return 0;
}

__device__ __forceinline__ int64_t clamp_pos(int64_t p, int max_pos) {
  return p < 0 ? 0 : (p >= max_pos ? (int64_t)max_pos - 1 : p);
}

// Gemma RMSNorm of the wave's vector (x0, x1 = dims 2l, 2l+1) with weight pair w (bf16 pair),
// rounded float64 -> float32 -> bf16.  Returns the bf16 values as floats.
__device__ __forceinline__ void rmsnorm_pair(float x0f, float x1f, uint32_t wpair, double eps,
                                             float& y0, float& y1) {
  const double x0 = x0f, x1 = x1f;
  double t = x0 * x0 + x1 * x1;  // squares exact; one rounding
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) t = t + shfl_xor_f64(t, m);
  const double var = t / 128.0 + eps;
  const double inv = 1.0 / sqrt(var);
  const double w0 = bf16lo(wpair), w1 = bf16hi(wpair);
  y0 = bf16_to_f32(f64_to_bf16((x0 * inv) * (1.0 + w0)));
  y1 = bf16_to_f32(f64_to_bf16((x1 * inv) * (1.0 + w1)));
}

// cos / sin of the two rotary frequencies of lane l (f0 = 2l mod 32 and f0 + 1), at the
// (clamped) positions posf(f).  Every lane loads (lanes >= 32 duplicate lanes - 32), so the
// loads carry no branch and go out as soon as the positions are known.
struct RopeCS {
  double c0, s0, c1, s1;
};
template <typename PosFn>
__device__ __forceinline__ RopeCS rope_load(const CompressParams& P, int lane, PosFn posf) {
  const int f0 = (2 * lane) & 31;
  const int64_t q0 = posf(f0), q1 = posf(f0 + 1);
  RopeCS cs;
  cs.c0 = P.cos_sin[q0 * 64 + f0];
  cs.s0 = P.cos_sin[q0 * 64 + 32 + f0];
  cs.c1 = P.cos_sin[q1 * 64 + f0 + 1];
  cs.s1 = P.cos_sin[q1 * 64 + 32 + f0 + 1];
  return cs;
}

// NeoX rotation of dims 0..63 (pairs (i, i+32)); dims 64..127 pass through.  Lane l holds dims
// 2l, 2l+1; its partners are in lane l ^ 16.
__device__ __forceinline__ void rope_apply(int lane, float& y0, float& y1, const RopeCS& cs) {
  const float p0 = __shfl_xor(y0, 16, kWave);
  const float p1 = __shfl_xor(y1, 16, kWave);
  if (lane < 32) {
    const double sgn = lane < 16 ? -1.0 : 1.0;  // first half: a*cos - b*sin; second: b*cos + a*sin
    const double r0 = (double)y0 * cs.c0 + sgn * ((double)p0 * cs.s0);
    const double r1 = (double)y1 * cs.c1 + sgn * ((double)p1 * cs.s1);
    y0 = bf16_to_f32(f64_to_bf16(r0));
    y1 = bf16_to_f32(f64_to_bf16(r1));
  }
}

// Positions of a token for the rotation: its three MRoPE axes, or its single position.
struct TokPos {
  int64_t t, h, w;
};
__device__ __forceinline__ int64_t axis_pos(const CompressParams& P, const TokPos& tp, int f) {
  if (!P.mrope) return clamp_pos(tp.t, P.max_pos);
  const int ax = mrope_axis(f, P.sec_h, P.sec_w);
  return clamp_pos(ax == 0 ? tp.t : (ax == 1 ? tp.h : tp.w), P.max_pos);
}

__device__ __forceinline__ void store_index_pair(const CompressParams& P, void* base,
                                                 int64_t vec, int lane, float y0, float y1) {
  if (P.fp8) {
    const uint32_t code = f32_to_e4m3(y0) | (f32_to_e4m3(y1) << 8);
    reinterpret_cast<uint16_t*>(base)[vec * 64 + lane] = (uint16_t)code;
  } else {
    const uint32_t bits = (f32_to_bf16(y0) & 0xFFFFu) | (f32_to_bf16(y1) << 16);
    reinterpret_cast<uint32_t*>(base)[vec * 64 + lane] = bits;
  }
}

// Main-cache fp8 code of x / scale: the quotient rounded to float32, clamped to +-448 (the
// saturating writer), then RNE on the e4m3fn grid.
__device__ __forceinline__ uint32_t scaled_e4m3_sat(float x, float scale) {
  const float q = (float)((double)x / (double)scale);
  if (!(q == q)) return f32_to_e4m3(q);
  return f32_to_e4m3(fminf(fmaxf(q, -448.0f), 448.0f));
}

__device__ __forceinline__ void ring_store_row(const CompressParams& P, int row, int r, int p,
                                               int L, int lane) {
  if (p < L - P.S) return;
  const int rp = P.ring_page[r];
  if (rp < 0 || rp >= P.ring_pages) return;
  const int64_t slot = (int64_t)rp * P.S + (p % P.S);
  P.ring[slot * 64 + lane] = P.k_proj[(int64_t)row * P.k_rs + lane];
  if (P.mrope && lane < 3) P.ring_pos[slot * 3 + lane] = P.pos[(int64_t)row * 3 + lane];
}

// The request owning `row`, found by the whole wave: lane i tests request base + i, loading its
// row interval, length and ring page in the same round trip; the owner's values are broadcast.
struct ReqInfo {
  int r, q0, n, L, rp;
};
__device__ __forceinline__ ReqInfo wave_find_request(const CompressParams& P, int row,
                                                     int lane) {
  ReqInfo ri{-1, 0, 0, 0, -1};
  for (int base = 0; base < P.R; base += kWave) {
    const int i = min(base + lane, P.R - 1);
    const int a = P.qsl[i], b = P.qsl[i + 1], Li = P.seq_lens[i], rpi = P.ring_page[i];
    const uint64_t m = __ballot(base + lane < P.R && a <= row && row < b);
    if (m) {
      const int src = (int)__builtin_ctzll(m);
      ri.r = base + src;
      ri.q0 = __builtin_amdgcn_readlane(a, src);
      ri.n = __builtin_amdgcn_readlane(b, src) - ri.q0;
      ri.L = __builtin_amdgcn_readlane(Li, src);
      ri.rp = __builtin_amdgcn_readlane(rpi, src);
      break;
    }
  }
  return ri;
}

// ---- vectors on 16-lane rows.  Row r = lane / 16 of a wave holds one 128-dim vector; its lane
// l = lane % 16 holds the dim pairs (2i, 2i+1) for i = l, l+16, l+32, l+48 (index k of the
// pair arrays below is i = l + 16k).  The canonical halving sum is then in-lane for its
// strides 32 and 16 (in pairs) and a DPP shift within the row for 8, 4, 2, 1, and the rotation
// partners (d, d+32), d < 32, sit in the same lane: no cross-row data movement at all.

// Value of lane l + N of the same 16-lane row (DPP row_shl); past the row's end: 0 (only lane
// 0's result is used).
template <int N>
__device__ __forceinline__ double row_down_f64(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, 0x100 + N, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), 0x100 + N, 0xF, 0xF,
                                             false);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

// Lane 16r's double, for every lane of row r.
__device__ __forceinline__ double row_broadcast_f64(double x, int lane) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const int lo = (int)(uint32_t)u, hi = (int)(uint32_t)(u >> 32);
  const int r = lane >> 4;
  int blo = __builtin_amdgcn_readlane(lo, 0), bhi = __builtin_amdgcn_readlane(hi, 0);
  const int lo1 = __builtin_amdgcn_readlane(lo, 16), hi1 = __builtin_amdgcn_readlane(hi, 16);
  const int lo2 = __builtin_amdgcn_readlane(lo, 32), hi2 = __builtin_amdgcn_readlane(hi, 32);
  const int lo3 = __builtin_amdgcn_readlane(lo, 48), hi3 = __builtin_amdgcn_readlane(hi, 48);
  blo = r == 1 ? lo1 : (r == 2 ? lo2 : (r == 3 ? lo3 : blo));
  bhi = r == 1 ? hi1 : (r == 2 ? hi2 : (r == 3 ? hi3 : bhi));
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)bhi << 32) | (uint32_t)blo));
}

// Gemma RMSNorm of a row vector (x: this lane's 8 values, pair k in x[2k], x[2k+1]) with the
// weight pairs wp[k], rounded float64 -> float32 -> bf16 (values returned as floats).
__device__ __forceinline__ void rmsnorm_row(const float (&x)[8], const uint32_t (&wp)[4],
                                            double eps, int lane, float (&y)[8]) {
  double v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    v[k] = (double)x[2 * k] * (double)x[2 * k] + (double)x[2 * k + 1] * (double)x[2 * k + 1];
  double t = (v[0] + v[2]) + (v[1] + v[3]);
  t = t + row_down_f64<8>(t);
  t = t + row_down_f64<4>(t);
  t = t + row_down_f64<2>(t);
  t = t + row_down_f64<1>(t);
  t = row_broadcast_f64(t, lane);
  const double var = t / 128.0 + eps;
  const double inv = 1.0 / sqrt(var);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const double w0 = bf16lo(wp[k]), w1 = bf16hi(wp[k]);
    y[2 * k] = bf16_to_f32(f64_to_bf16(((double)x[2 * k] * inv) * (1.0 + w0)));
    y[2 * k + 1] = bf16_to_f32(f64_to_bf16(((double)x[2 * k + 1] * inv) * (1.0 + w1)));
  }
}

// cos / sin of frequencies 2l and 2l+1 (the rotations of dims 2l, 2l+1 with 2l+32, 2l+33).
template <typename PosFn>
__device__ __forceinline__ RopeCS rope_load_row(const CompressParams& P, int l, PosFn posf) {
  const int f0 = 2 * l;
  const int64_t q0 = posf(f0), q1 = posf(f0 + 1);
  RopeCS cs;
  cs.c0 = P.cos_sin[q0 * 64 + f0];
  cs.s0 = P.cos_sin[q0 * 64 + 32 + f0];
  cs.c1 = P.cos_sin[q1 * 64 + f0 + 1];
  cs.s1 = P.cos_sin[q1 * 64 + 32 + f0 + 1];
  return cs;
}

// NeoX rotation in-lane: pair 0 (dims 2l, 2l+1) with pair 1 (dims 2l+32, 2l+33).
__device__ __forceinline__ void rope_row(float (&y)[8], const RopeCS& cs) {
  const double a0 = y[0], a1 = y[1], b0 = y[2], b1 = y[3];
  y[0] = bf16_to_f32(f64_to_bf16(a0 * cs.c0 - b0 * cs.s0));
  y[2] = bf16_to_f32(f64_to_bf16(b0 * cs.c0 + a0 * cs.s0));
  y[1] = bf16_to_f32(f64_to_bf16(a1 * cs.c1 - b1 * cs.s1));
  y[3] = bf16_to_f32(f64_to_bf16(b1 * cs.c1 + a1 * cs.s1));
}

__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  return (f32_to_bf16(a) & 0xFFFFu) | (f32_to_bf16(b) << 16);
}

// The rotary positions of `row`.
__device__ __forceinline__ TokPos row_pos(const CompressParams& P, int row) {
  TokPos tp;
  if (P.mrope) {
    tp = {P.pos[(int64_t)row * 3], P.pos[(int64_t)row * 3 + 1], P.pos[(int64_t)row * 3 + 2]};
  } else {
    tp.t = tp.h = tp.w = P.pos[row];
  }
  return tp;
}

// One Q-type vector per 16-lane row: RMSNorm (weights wt) -> RoPE at the row's positions.
// Loads are clamped to vector n-1 for rows past the end (their results are not stored).  In two
// parts: the loads that need only the vector index (its values, the weights, the row's
// positions), then the rotation table's loads, then the arithmetic.
struct RowIn {
  uint32_t u[4], wp[4];
  TokPos tp;
  int row;
};
template <typename SrcFn>
__device__ __forceinline__ RowIn norm_rope_load(const CompressParams& P, int64_t v, int64_t n,
                                                int heads, const uint16_t* wt, int lane,
                                                SrcFn src) {
  const int l = lane & 15;
  const int64_t vc = v < n ? v : n - 1;
  RowIn in;
  in.row = (int)(vc / heads);
  const uint32_t* s = src(in.row, (int)(vc % heads));
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    in.u[k] = s[l + 16 * k];
    in.wp[k] = reinterpret_cast<const uint32_t*>(wt)[l + 16 * k];
  }
  in.tp = row_pos(P, in.row);
  return in;
}
// The rotation table entries as loaded (float; widened where they are used, so that nothing
// waits for the loads before then).
struct RopeRaw {
  float c0, s0, c1, s1;
};
__device__ __forceinline__ RopeRaw norm_rope_table(const CompressParams& P, const RowIn& in,
                                                   int lane) {
  const int f0 = 2 * (lane & 15);
  const int64_t q0 = axis_pos(P, in.tp, f0), q1 = axis_pos(P, in.tp, f0 + 1);
  return RopeRaw{P.cos_sin[q0 * 64 + f0], P.cos_sin[q0 * 64 + 32 + f0],
                 P.cos_sin[q1 * 64 + f0 + 1], P.cos_sin[q1 * 64 + 32 + f0 + 1]};
}
__device__ __forceinline__ void norm_rope_compute(const RowIn& in, const RopeRaw& raw,
                                                  double eps, int lane, float (&y)[8]) {
  const RopeCS cs{raw.c0, raw.s0, raw.c1, raw.s1};
  float x[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = bf16lo(in.u[k]);
    x[2 * k + 1] = bf16hi(in.u[k]);
  }
  rmsnorm_row(x, in.wp, eps, lane, y);
  rope_row(y, cs);
}
__device__ __forceinline__ void norm_rope_finish(const CompressParams& P, const RowIn& in,
                                                 double eps, int lane, float (&y)[8]) {
  norm_rope_compute(in, norm_rope_table(P, in, lane), eps, lane, y);
}
template <typename SrcFn>
__device__ __forceinline__ void norm_rope_row(const CompressParams& P, int64_t v, int64_t n,
                                              int heads, const uint16_t* wt, double eps,
                                              int lane, SrcFn src, float (&y)[8], int& row) {
  const RowIn in = norm_rope_load(P, v, n, heads, wt, lane, src);
  row = in.row;
  norm_rope_finish(P, in, eps, lane, y);
}

// The compressed row of group g of request r (tokens g*c .. g*c+c-1; those at or after `start`,
// the request's first row of this step, are rows q0 + t - start of the step, earlier ones come
// from the ring, or read as 0 when the request's ring page rp is out of range): the pooled mean,
// rounded to bf16, RMSNorm with the key weights, RoPE at the position of token g*c.  A whole
// wave: lane l gets dims 2l, 2l+1 (y0, y1); `page` is the group's compressed-cache page (-1:
// its column is past the block table; the caller stores the row only for a page in range).
__device__ __forceinline__ void compress_group(const CompressParams& P, int r, int q0, int start,
                                               int rp, bool ring_ok, int g, int lane, float& y0,
                                               float& y1, int& page) {
  const int t0 = g * P.c;
  // Everything the group needs, in one round trip: its keys (this step's rows or the ring),
  // the block-table entry of its compressed row, and its first token's position (1-D: the
  // token index itself, so the cos / sin loads go out at once).
  const int col = g / P.Pc;
  page = col < P.cbt_width ? P.cbt[(int64_t)r * P.cbt_stride + col] : -1;
  TokPos tp;
  if (P.mrope) {
    const bool in_step = t0 >= start;
    const int64_t base = in_step ? (int64_t)(q0 + t0 - start) * 3
                                 : ((int64_t)(ring_ok ? rp : 0) * P.S + (t0 % P.S)) * 3;
    const int64_t* src = in_step ? P.pos : P.ring_pos;
    const bool ok = in_step || ring_ok;
    tp = {ok ? src[base] : 0, ok ? src[base + 1] : 0, ok ? src[base + 2] : 0};
  } else {
    tp.t = tp.h = tp.w = t0;
  }
  const RopeCS cs = rope_load(P, lane, [&](int f) { return axis_pos(P, tp, f); });
  double a0 = 0.0, a1 = 0.0;
  for (int m0 = 0; m0 < P.c; m0 += 8) {
    uint32_t uu[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int t = t0 + m0 + k;
      uint32_t v = 0;
      if (m0 + k < P.c) {
        if (t >= start) {
          v = P.k_proj[(int64_t)(q0 + t - start) * P.k_rs + lane];
        } else if (ring_ok) {
          v = P.ring[((int64_t)rp * P.S + (t % P.S)) * 64 + lane];
        }
      }
      uu[k] = v;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (m0 + k < P.c) {
        const double v0 = bf16lo(uu[k]), v1 = bf16hi(uu[k]);
        if (m0 + k == 0) {
          a0 = v0;
          a1 = v1;
        } else {
          a0 = a0 + v0;
          a1 = a1 + v1;
        }
      }
    }
  }
  const double inv_c = 1.0 / (double)P.c;  // c is a power of two: exact, as is the product
  const float m0f = bf16_to_f32(f64_to_bf16(a0 * inv_c));
  const float m1f = bf16_to_f32(f64_to_bf16(a1 * inv_c));
  rmsnorm_pair(m0f, m1f, reinterpret_cast<const uint32_t*>(P.kw)[lane], P.eps, y0, y1);
  rope_apply(lane, y0, y1, cs);
}

// compress_group in two parts, for a 1-D rotation and c <= 8 (the group's keys fit one batch):
// the loads (its page, its keys, the key weights, the rotation table words of token g*c) and
// the arithmetic, which is compress_group's exactly.
struct GroupIn {
  int page;
  uint32_t uu[8];
  uint32_t kw;
  float c0, s0, c1, s1;
};
__device__ __forceinline__ GroupIn compress_group_load(const CompressParams& P, int r, int q0,
                                                       int start, int rp, bool ring_ok, int g,
                                                       int lane) {
  GroupIn in;
  const int t0 = g * P.c;
  const int col = g / P.Pc;
  in.page = col < P.cbt_width ? P.cbt[(int64_t)r * P.cbt_stride + col] : -1;
  const int f0 = (2 * lane) & 31;
  const int64_t q = clamp_pos(t0, P.max_pos);
  in.c0 = P.cos_sin[q * 64 + f0];
  in.s0 = P.cos_sin[q * 64 + 32 + f0];
  in.c1 = P.cos_sin[q * 64 + f0 + 1];
  in.s1 = P.cos_sin[q * 64 + 32 + f0 + 1];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int t = t0 + k;
    uint32_t v = 0;
    if (k < P.c) {
      if (t >= start) {
        v = P.k_proj[(int64_t)(q0 + t - start) * P.k_rs + lane];
      } else if (ring_ok) {
        v = P.ring[((int64_t)rp * P.S + (t % P.S)) * 64 + lane];
      }
    }
    in.uu[k] = v;
  }
  in.kw = reinterpret_cast<const uint32_t*>(P.kw)[lane];
  return in;
}
__device__ __forceinline__ void compress_group_compute(const CompressParams& P, const GroupIn& in,
                                                       int lane, float& y0, float& y1) {
  double a0 = 0.0, a1 = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < P.c) {
      const double v0 = bf16lo(in.uu[k]), v1 = bf16hi(in.uu[k]);
      if (k == 0) {
        a0 = v0;
        a1 = v1;
      } else {
        a0 = a0 + v0;
        a1 = a1 + v1;
      }
    }
  }
  const double inv_c = 1.0 / (double)P.c;
  const float m0f = bf16_to_f32(f64_to_bf16(a0 * inv_c));
  const float m1f = bf16_to_f32(f64_to_bf16(a1 * inv_c));
  rmsnorm_pair(m0f, m1f, in.kw, P.eps, y0, y1);
  const RopeCS cs{in.c0, in.s0, in.c1, in.s1};
  rope_apply(lane, y0, y1, cs);
}

// The parameter block of a qsa_compress call (arguments already validated).
CompressParams compress_params(const qsa_compress_args& a);

}  // namespace qsa
