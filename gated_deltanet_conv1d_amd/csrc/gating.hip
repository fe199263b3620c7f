// Fused GDN gating (LightLLM PR #1184 "[model] support Qwen3next", Highlights:
// fused gating; LightLLM #1097 "[model] Support Qwen3next", Highlights
// "Specialized Triton Kernels": fused GDN gating).  Elementwise per (token, V head):
//   g    = -exp(A_log[h]) * softplus(a + dt_bias[h])
//   beta = sigmoid(b)
// HBM-bound and tiny (a and b in, g and beta out); one thread per element.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void gating_kernel(const T* __restrict__ a, const T* __restrict__ b,
                                                     const float* __restrict__ A_log,
                                                     const float* __restrict__ dt_bias, float* __restrict__ g,
                                                     float* __restrict__ beta, int64_t n, int32_t h_v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int h = (int)(i % h_v);
  g[i] = -expf(A_log[h]) * softplusf_(to_f32(a[i]) + dt_bias[h]);
  beta[i] = sigmoidf_(to_f32(b[i]));
}

}  // namespace

hipError_t launch_gating(const GatingArgs& a, hipStream_t st) {
  const int64_t n = a.n_tokens * a.h_v;
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (a.bf16)
    hipLaunchKernelGGL(gating_kernel<bf16>, dim3(blocks), dim3(256), 0, st, (const bf16*)a.a, (const bf16*)a.b,
                       a.A_log, a.dt_bias, a.g, a.beta, n, a.h_v);
  else
    hipLaunchKernelGGL(gating_kernel<float>, dim3(blocks), dim3(256), 0, st, (const float*)a.a,
                       (const float*)a.b, a.A_log, a.dt_bias, a.g, a.beta, n, a.h_v);
  return hipGetLastError();
}

}  // namespace gdn
