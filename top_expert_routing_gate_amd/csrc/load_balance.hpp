// Workgroup-level load statistics and sign-step bias update (256 threads),
// used by the standalone moer_load_stats / moer_bias_update kernels and by the
// layout's first workgroup when moer_route is asked for them.
//
// Load statistics ("A minimal experiment in expert-load imbalance", Run the
// example): total, mean = total/N, imbalance = max/mean (0 when the mean is
// 0), capacity = max*N; plus the entropy in bits of the realised load
// distribution ("MoE Routing Entropy vs Expert Saturation", Mathematics) and
// the coefficient of variation std/mean that "DeepSeek V4 MoE load
// balancing" (deployment section) monitors. Integers exactly; the derived
// values in fp64 with fixed-order reductions.
//
// Bias update ("DeepSeek V4 MoE load balancing", auxiliary-loss-free
// balancing): overloaded experts' biases go down, underloaded ones go up, by
// a fixed step u: b_e += u*sign(mean - load_e), the comparison done exactly
// as sign(total - N*load_e) in integers; one fp32 rounding per expert.
#pragma once

#include <math.h>

#include "../../include/moer.h"
#include "moer_internal.hpp"

namespace moer {

constexpr int kBalanceThreads = 256;

struct BalanceScratch {
  long long red_i[kBalanceThreads];
  double red_d[kBalanceThreads];
  long long red_v[kBalanceThreads];
  int red_e[kBalanceThreads];
};

template <typename V, typename Op>
__device__ V balance_reduce(V v, V* red, Op op) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int o = kBalanceThreads / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] = op(red[threadIdx.x], red[threadIdx.x + o]);
    __syncthreads();
  }
  const V r = red[0];
  __syncthreads();
  return r;
}

// Sum of c[0..N); every thread receives it.
__device__ inline long long block_count_total(const int32_t* c, int N, BalanceScratch& sh) {
  long long tot = 0;
  for (int e = threadIdx.x; e < N; e += kBalanceThreads) tot += c[e];
  return balance_reduce(tot, sh.red_i, [](long long x, long long y) { return x + y; });
}

// Load statistics of c[0..N) (c may live in LDS or global memory).
__device__ inline void block_load_stats(const int32_t* c, int N, moer_load_stats_t* out,
                                        BalanceScratch& sh) {
  const long long tot = block_count_total(c, N, sh);
  long long bv = -1;
  int be = 0;
  for (int e = threadIdx.x; e < N; e += kBalanceThreads)
    if ((long long)c[e] > bv) { bv = c[e]; be = e; }
  // max with the lowest expert id on ties, fixed pairwise order
  sh.red_v[threadIdx.x] = bv;
  sh.red_e[threadIdx.x] = be;
  __syncthreads();
  for (int o = kBalanceThreads / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      const long long ov = sh.red_v[threadIdx.x + o];
      const int oe = sh.red_e[threadIdx.x + o];
      if (ov > sh.red_v[threadIdx.x] || (ov == sh.red_v[threadIdx.x] && oe < sh.red_e[threadIdx.x])) {
        sh.red_v[threadIdx.x] = ov;
        sh.red_e[threadIdx.x] = oe;
      }
    }
    __syncthreads();
  }
  const long long mx = sh.red_v[0];
  const int am = sh.red_e[0];
  __syncthreads();
  const double mean = (double)tot / (double)N;
  double hpart = 0.0, vpart = 0.0;
  for (int e = threadIdx.x; e < N; e += kBalanceThreads) {
    const double v = (double)c[e];
    if (tot > 0 && c[e] > 0) {
      const double q = v / (double)tot;
      hpart -= q * log2(q);
    }
    vpart += (v - mean) * (v - mean);
  }
  const double H = balance_reduce(hpart, sh.red_d, [](double x, double y) { return x + y; });
  const double var = balance_reduce(vpart, sh.red_d, [](double x, double y) { return x + y; });
  if (threadIdx.x == 0) {
    moer_load_stats_t r;
    r.total = tot;
    r.max_load = mx;
    r.argmax = mx > 0 ? am : 0;
    r.capacity = mx * (long long)N;
    r.mean = mean;
    r.imbalance = mean != 0.0 ? (double)mx / mean : 0.0;
    r.h_load_bits = H;
    r.cv = mean != 0.0 ? sqrt(var / (double)N) / mean : 0.0;
    *out = r;
  }
}

// In-place sign-step update of bias[0..N) from c[0..N).
__device__ inline void block_bias_update(float* bias, const int32_t* c, int N, float u,
                                         BalanceScratch& sh) {
  const long long tot = block_count_total(c, N, sh);
  for (int e = threadIdx.x; e < N; e += kBalanceThreads) {
    const long long diff = tot - (long long)N * c[e];
    const float step = diff > 0 ? u : (diff < 0 ? -u : 0.f);
    bias[e] = bias[e] + step;
  }
}

}  // namespace moer
