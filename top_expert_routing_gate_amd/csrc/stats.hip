// Load statistics and the sign-step bias update, one workgroup per layer.
//
// Load statistics ("A minimal experiment in expert-load imbalance", Run the
// example): total, mean = total/N, imbalance = max/mean (0 when the mean is
// 0), capacity = max*N. Also the entropy in bits of the realised load
// distribution ("MoE Routing Entropy vs Expert Saturation", Mathematics) and
// the coefficient of variation std/mean that "DeepSeek V4 MoE load
// balancing" (deployment section) monitors. Integers exactly; the derived
// values in fp64 with fixed-order reductions.
//
// Bias update ("DeepSeek V4 MoE load balancing", auxiliary-loss-free
// balancing): overloaded experts' biases go down, underloaded ones go up, by
// a fixed step u: b_e += u*sign(mean - load_e), the comparison done exactly
// as sign(total - N*load_e) in integers.
#include <math.h>

#include "../../include/moer.h"
#include "moer_internal.hpp"

namespace moer {
namespace {

constexpr int kThreads = 256;

template <typename V, typename Op>
__device__ V block_reduce(V v, V* red, Op op) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] = op(red[threadIdx.x], red[threadIdx.x + o]);
    __syncthreads();
  }
  const V r = red[0];
  __syncthreads();
  return r;
}

struct MaxArg {
  long long v;
  int e;
};

__global__ __launch_bounds__(kThreads) void load_stats_kernel(const int32_t* __restrict__ counts,
                                                              int N, int stride,
                                                              moer_load_stats_t* out) {
  __shared__ long long red_i[kThreads];
  __shared__ double red_d[kThreads];
  __shared__ MaxArg red_m[kThreads];
  const int layer = blockIdx.x;
  const int32_t* c = counts + (size_t)layer * stride;

  long long tot = 0;
  MaxArg best{-1, 0};
  for (int e = threadIdx.x; e < N; e += kThreads) {
    const long long v = c[e];
    tot += v;
    if (v > best.v) best = MaxArg{v, e};
  }
  tot = block_reduce(tot, red_i, [](long long x, long long y) { return x + y; });
  best = block_reduce(best, red_m, [](MaxArg x, MaxArg y) {
    return (y.v > x.v || (y.v == x.v && y.e < x.e)) ? y : x;
  });
  const double mean = (double)tot / (double)N;

  double hpart = 0.0, vpart = 0.0;
  for (int e = threadIdx.x; e < N; e += kThreads) {
    const double v = (double)c[e];
    if (tot > 0 && c[e] > 0) {
      const double q = v / (double)tot;
      hpart -= q * log2(q);
    }
    vpart += (v - mean) * (v - mean);
  }
  const double H = block_reduce(hpart, red_d, [](double x, double y) { return x + y; });
  const double var = block_reduce(vpart, red_d, [](double x, double y) { return x + y; });

  if (threadIdx.x == 0) {
    moer_load_stats_t r;
    r.total = tot;
    r.max_load = best.v;
    r.argmax = best.v > 0 ? best.e : 0;
    r.capacity = best.v * (long long)N;
    r.mean = mean;
    r.imbalance = mean != 0.0 ? (double)best.v / mean : 0.0;
    r.h_load_bits = H;
    r.cv = mean != 0.0 ? sqrt(var / (double)N) / mean : 0.0;
    out[layer] = r;
  }
}

__global__ __launch_bounds__(kThreads) void bias_update_kernel(float* __restrict__ bias,
                                                               const int32_t* __restrict__ counts,
                                                               int N, int stride, float u) {
  __shared__ long long red_i[kThreads];
  const int layer = blockIdx.x;
  const int32_t* c = counts + (size_t)layer * stride;
  long long tot = 0;
  for (int e = threadIdx.x; e < N; e += kThreads) tot += c[e];
  tot = block_reduce(tot, red_i, [](long long x, long long y) { return x + y; });
  for (int e = threadIdx.x; e < N; e += kThreads) {
    const long long diff = tot - (long long)N * c[e];
    const float step = diff > 0 ? u : (diff < 0 ? -u : 0.f);
    float* b = bias + (size_t)layer * N + e;
    *b = *b + step;
  }
}

}  // namespace

hipError_t launch_load_stats(const int32_t* counts, int L, int N, int stride, void* out,
                             hipStream_t s) {
  hipLaunchKernelGGL(load_stats_kernel, dim3(L), dim3(kThreads), 0, s, counts, N, stride,
                     static_cast<moer_load_stats_t*>(out));
  return hipGetLastError();
}

hipError_t launch_bias_update(float* bias, const int32_t* counts, int L, int N, int stride,
                              float u, hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(L), dim3(kThreads), 0, s, bias, counts, N, stride,
                     u);
  return hipGetLastError();
}

}  // namespace moer
