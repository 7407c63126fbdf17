// Workgroup-level load statistics and sign-step bias update (256 threads),
// used by the standalone moer_load_stats / moer_bias_update kernels and by the
// layout launch's balance workgroup when moer_route is asked for them.
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
constexpr int kBalanceWaves = kBalanceThreads / kWave;

struct BalanceScratch {
  long long tot[kBalanceWaves];
  unsigned long long best[kBalanceWaves];
  double h[kBalanceWaves];
  double v[kBalanceWaves];
};

// Xor butterfly over the 64 lanes of a wave: every lane ends with the same
// bits (each step combines a lane with its partner using a commutative op).
template <typename V, typename Op>
__device__ __forceinline__ V wave_allreduce(V v, Op op) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v = op(v, __shfl_xor(v, o, kWave));
  return v;
}

// Load statistics (out != nullptr) and/or the sign-step bias update
// (bias != nullptr) of the counts c[0..N) (LDS or global memory). Reductions:
// each thread takes experts tid, tid+256, ... in order, then a butterfly per
// wave, then the four wave results in wave order: fixed, so deterministic.
// The first 256 threads of the workgroup do the work; a larger workgroup's
// other threads only take part in its barriers (same results at any size).
// NW = 1: one wavefront alone (any one: lane = expert), for N <= 64, with no
// barrier; the results are bit for bit those of NW = 4 (there the other
// three waves hold no expert and add exact zeros).
template <int NW = kBalanceWaves>
__device__ inline void block_load_balance(const int32_t* c, int N, moer_load_stats_t* out,
                                          float* bias, float u, BalanceScratch& sh) {
  static_assert(NW == 1 || NW == kBalanceWaves, "one wave or the whole balance group");
  constexpr int kStride = NW == 1 ? kWave : kBalanceThreads;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int tid = NW == 1 ? lane : (int)threadIdx.x;
  const bool worker = tid < kStride;
  const int e_first = worker ? tid : N;
  // first pass: total, and the largest count with the lowest expert id on ties
  // (packed as order-preserving count bits << 32 | ~id, so one unsigned max
  // decides both)
  long long tot = 0;
  unsigned long long best = 0;
  for (int e = e_first; e < N; e += kStride) {
    tot += c[e];
    const unsigned ord = (unsigned)c[e] ^ 0x80000000u;
    const unsigned long long key =
        ((unsigned long long)ord << 32) | (unsigned)(0xFFFFFFFFu - (unsigned)e);
    best = key > best ? key : best;
  }
  tot = wave_allreduce(tot, [](long long x, long long y) { return x + y; });
  best = wave_allreduce(best, [](unsigned long long x, unsigned long long y) { return x > y ? x : y; });
  if constexpr (NW > 1) {
    if (worker && lane == 0) {
      sh.tot[wave] = tot;
      sh.best[wave] = best;
    }
    __syncthreads();
    tot = sh.tot[0];
    best = sh.best[0];
#pragma unroll
    for (int w = 1; w < kBalanceWaves; ++w) {
      tot += sh.tot[w];
      best = sh.best[w] > best ? sh.best[w] : best;
    }
  }

  if (bias != nullptr) {
    for (int e = e_first; e < N; e += kStride) {
      const long long diff = tot - (long long)N * c[e];
      const float step = diff > 0 ? u : (diff < 0 ? -u : 0.f);
      bias[e] = bias[e] + step;
    }
  }
  if (out == nullptr) return;

  // second pass: entropy of the load distribution and the sum of squared deviations
  const double mean = (double)tot / (double)N;
  double hpart = 0.0, vpart = 0.0;
  for (int e = e_first; e < N; e += kStride) {
    const double v = (double)c[e];
    if (tot > 0 && c[e] > 0) {
      const double q = v / (double)tot;
      hpart -= q * log2(q);
    }
    vpart += (v - mean) * (v - mean);
  }
  hpart = wave_allreduce(hpart, [](double x, double y) { return x + y; });
  vpart = wave_allreduce(vpart, [](double x, double y) { return x + y; });
  if constexpr (NW > 1) {
    if (worker && lane == 0) {
      sh.h[wave] = hpart;
      sh.v[wave] = vpart;
    }
    __syncthreads();
  }
  if (tid == 0) {
    double H = hpart, var = vpart;
    if constexpr (NW > 1) {
      H = sh.h[0];
      var = sh.v[0];
#pragma unroll
      for (int w = 1; w < kBalanceWaves; ++w) {
        H += sh.h[w];
        var += sh.v[w];
      }
    }
    const long long mx = (long long)(int)((unsigned)(best >> 32) ^ 0x80000000u);
    const int am = (int)(0xFFFFFFFFu - (unsigned)(best & 0xFFFFFFFFu));
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

}  // namespace moer
