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

}  // namespace

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
