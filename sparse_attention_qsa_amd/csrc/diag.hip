// Diagnostic kernels: expose the device arithmetic the exactness of the path rests on, so the
// tests can compare it with the host's IEEE results.
#include "qsa_internal.h"

namespace qsa {
namespace {

// out[0..255]: every e4m3fn code through the hardware converter the logits kernel uses;
// out[256..511]: the same codes through the definitional decoder of the re-scoring path.
__global__ void diag_e4m3_kernel(float* out) {
  const uint32_t c = threadIdx.x;
  const auto v = __builtin_amdgcn_cvt_pk_f32_fp8(c, false);
  out[c] = v[0];
  out[256 + c] = e4m3_to_f32_exact(c);
}

// out[3i] = sqrt(x), out[3i+1] = 1/x, out[3i+2] = 1/sqrt(x), as the RMSNorm chain computes them.
__global__ void diag_fp64_kernel(const double* in, double* out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const double x = in[i];
  const double r = sqrt(x);
  out[3 * i] = r;
  out[3 * i + 1] = 1.0 / x;
  out[3 * i + 2] = 1.0 / r;
}

// Read-bandwidth probe: wave v reads list entries 8v .. 8v+7, then 8(v + waves) .. +7, ... (so a
// streaming read walks contiguous 8-chunk runs), each a chunk of chunk_bytes (entry i at
// i * chunk_bytes, or at idx[i] * chunk_bytes with an index list), 16 bytes per lane, the loads
// of the eight chunks in flight together (the next run's indices are loaded beside them), and
// folds everything it read into one word with XOR (atomically into sink[0]) so that no load is
// dead.
__global__ __launch_bounds__(256) void diag_read_kernel(const uint4* src, const int32_t* idx,
                                                       int64_t n, int32_t chunk_bytes,
                                                       uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / 64);
  const int64_t v = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int per = chunk_bytes / 1024;  // 1 KiB loads per chunk
  uint32_t acc = 0u;
  int64_t cur[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t c = 8 * v + u;
    cur[u] = c < n ? (idx ? (int64_t)idx[c] : c) : -1;
  }
  for (int64_t c0 = 8 * v; c0 < n; c0 += 8 * waves) {
    uint4 x[8][4];
    int64_t nxt[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t c = c0 + 8 * waves + u;
      nxt[u] = c < n ? (idx ? (int64_t)idx[c] : c) : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t c = c0 + u;
      const int64_t base = cur[u] >= 0 ? cur[u] * (chunk_bytes / 16) : 0;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        x[u][k] = (c < n && k < per) ? src[base + 64 * k + lane] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc ^= x[u][k].x ^ x[u][k].y ^ x[u][k].z ^ x[u][k].w;
#pragma unroll
    for (int u = 0; u < 8; ++u) cur[u] = nxt[u];
  }
  for (int m = 32; m >= 1; m >>= 1) acc ^= __shfl_xor(acc, m, kWave);
  if (lane == 0) atomicXor(sink, acc);
}

}  // namespace

hipError_t launch_diag_read(const void* src, const int32_t* idx, int64_t n, int32_t chunk_bytes,
                            uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(diag_read_kernel, dim3(4096), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(src), idx, n, chunk_bytes, sink);
  return hipGetLastError();
}

hipError_t launch_diag_e4m3(float* out, hipStream_t s) {
  hipLaunchKernelGGL(diag_e4m3_kernel, dim3(1), dim3(256), 0, s, out);
  return hipGetLastError();
}

hipError_t launch_diag_fp64(const double* in, double* out, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(diag_fp64_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, in,
                     out, n);
  return hipGetLastError();
}

}  // namespace qsa
