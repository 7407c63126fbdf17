// Standalone load statistics and sign-step bias update kernels, one
// workgroup per layer (the arithmetic is in load_balance.hpp).
#include "load_balance.hpp"

namespace moer {
namespace {

__global__ __launch_bounds__(kBalanceThreads) void load_stats_kernel(
    const int32_t* __restrict__ counts, int N, int stride, moer_load_stats_t* out) {
  __shared__ BalanceScratch sh;
  block_load_balance(counts + (size_t)blockIdx.x * stride, N, out + blockIdx.x, nullptr, 0.f, sh);
}

__global__ __launch_bounds__(kBalanceThreads) void bias_update_kernel(
    float* __restrict__ bias, const int32_t* __restrict__ counts, int N, int stride, float u) {
  __shared__ BalanceScratch sh;
  block_load_balance(counts + (size_t)blockIdx.x * stride, N, nullptr, bias + (size_t)blockIdx.x * N,
                     u, sh);
}

}  // namespace

hipError_t launch_load_stats(const int32_t* counts, int L, int N, int stride, moer_load_stats_t* out,
                             hipStream_t s) {
  hipLaunchKernelGGL(load_stats_kernel, dim3(L), dim3(kBalanceThreads), 0, s, counts, N, stride, out);
  return hipGetLastError();
}

hipError_t launch_bias_update(float* bias, const int32_t* counts, int L, int N, int stride,
                              float u, hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(L), dim3(kBalanceThreads), 0, s, bias, counts, N,
                     stride, u);
  return hipGetLastError();
}

}  // namespace moer
