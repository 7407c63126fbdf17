// Forcible load balancing and expert hotspot collection.
//
// MindIE "expert parallelism load balancer" (hiascend.com): forcible load
// balancing replaces the top-k operator's output with indices that load
// every expert equally, which gives the upper bound of what balancing can
// do; the hotspot collection records, per layer and expert, how many tokens
// the expert processed.
//
// The balanced ids walk the experts round-robin over the batch's
// assignments: slot k < K of token t gets (t*K + k + first) mod N, so every
// expert gets T*K/N assignments (within one), and a token's K slots are K
// different experts when K <= N. Shared slots keep ids N..N+n_shared-1.
// Both kernels are elementwise.
#include "moer_internal.hpp"

namespace moer {
namespace {

constexpr int kElemThreads = 256;

__global__ __launch_bounds__(kElemThreads) void balanced_indices_kernel(
    int32_t* __restrict__ idx, int64_t total, int T, int K, int Kt, int N, int start) {
  for (int64_t i = (int64_t)blockIdx.x * kElemThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kElemThreads) {
    const int k = (int)(i % Kt);
    const int64_t t = (i / Kt) % T;
    idx[i] = k < K ? (int32_t)((t * K + k + start) % N) : N + (k - K);
  }
}

__global__ __launch_bounds__(kElemThreads) void hotspot_accumulate_kernel(
    int64_t* __restrict__ hot, const int32_t* __restrict__ counts, int L, int N, int stride) {
  const int64_t i = (int64_t)blockIdx.x * kElemThreads + threadIdx.x;
  if (i >= (int64_t)L * N) return;
  const int64_t l = i / N, e = i % N;
  hot[i] += counts[l * stride + e];
}

unsigned grid_for(int64_t n) {
  const int64_t g = (n + kElemThreads - 1) / kElemThreads;
  return (unsigned)(g < 65536 ? g : 65536);
}

}  // namespace

hipError_t launch_balanced_indices(int32_t* idx, int L, int T, int K, int N, int n_shared,
                                   int start, hipStream_t s) {
  const int Kt = K + n_shared;
  const int64_t total = (int64_t)L * T * Kt;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(balanced_indices_kernel, dim3(grid_for(total)), dim3(kElemThreads), 0, s, idx,
                     total, T, K, Kt, N, start);
  return hipGetLastError();
}

hipError_t launch_hotspot_accumulate(int64_t* hot, const int32_t* counts, int L, int N, int stride,
                                     hipStream_t s) {
  const int64_t total = (int64_t)L * N;
  hipLaunchKernelGGL(hotspot_accumulate_kernel,
                     dim3((unsigned)((total + kElemThreads - 1) / kElemThreads)),
                     dim3(kElemThreads), 0, s, hot, counts, L, N, stride);
  return hipGetLastError();
}

}  // namespace moer
