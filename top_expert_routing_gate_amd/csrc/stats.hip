// Standalone load statistics, sign-step bias update and balancing-step
// kernels, one workgroup per layer (the statistics and the sign step share
// their arithmetic with the fused path in load_balance.hpp).
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

// One balancing step of a layer: moving-average loads, then (every `every`
// calls) the sign or proportional rule against the mean load. The mean is
// summed by one thread in ascending expert order in fp64, so the result does
// not depend on the launch shape. Every operation rounds on its own: the
// contract pragma keeps the compiler from fusing the moving average's
// product and sum into one multiply-add (which rounds once, and differs).
__global__ __launch_bounds__(kBalanceThreads) void balance_step_kernel(
    float* __restrict__ bias, const int32_t* __restrict__ counts, int N, int stride, int rule,
    float step, float alpha, float keep, int every, float* __restrict__ loads,
    int32_t* __restrict__ calls) {
#pragma clang fp contract(off)
  __shared__ float sl[kMaxExperts];
  __shared__ double smean;
  const int layer = blockIdx.x;
  const int32_t* c = counts + (size_t)layer * stride;
  float* b = bias + (size_t)layer * N;
  float* ld = loads != nullptr ? loads + (size_t)layer * N : nullptr;
  const int ncall = calls != nullptr ? calls[layer] : 0;
  for (int e = threadIdx.x; e < N; e += blockDim.x) {
    const float ce = (float)c[e];
    float le = ce;
    if (ld != nullptr && ncall != 0) le = alpha * ce + keep * ld[e];
    if (ld != nullptr) ld[e] = le;
    sl[e] = le;
  }
  __syncthreads();
  if ((ncall + 1) % every == 0) {  // the same for every thread of the block
    if (threadIdx.x == 0) {
      double total = 0.0;
      for (int e = 0; e < N; ++e) total += (double)sl[e];
      smean = total / (double)N;
    }
    __syncthreads();
    const double mean = smean;
    for (int e = threadIdx.x; e < N; e += blockDim.x) {
      if (rule == MOER_RULE_SIGN) {
        const double diff = mean - (double)sl[e];
        const float sg = diff > 0.0 ? step : (diff < 0.0 ? -step : 0.f);
        b[e] = b[e] + sg;
      } else if (mean > 0.0) {
        const double rel = ((double)sl[e] - mean) / mean;
        b[e] = b[e] - (float)((double)step * rel);
      }
    }
  }
  if (threadIdx.x == 0 && calls != nullptr) calls[layer] = ncall + 1;
}

}  // namespace

hipError_t launch_balance_step(float* bias, const int32_t* counts, int L, int N, int stride,
                               int rule, float step, float alpha, int every, float* loads,
                               int32_t* calls, hipStream_t s) {
  const float keep = 1.0f - alpha;
  hipLaunchKernelGGL(balance_step_kernel, dim3(L), dim3(kBalanceThreads), 0, s, bias, counts, N,
                     stride, rule, step, alpha, keep, every, loads, calls);
  return hipGetLastError();
}

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
