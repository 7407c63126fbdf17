// Dispatch layout: per-expert counts (the listing's bincount in "MoE Routing
// Entropy vs Expert Saturation"), their exclusive prefix, and a stable
// permutation that groups every (token, slot) assignment by destination
// expert — the grouping dispatch needs ("DeepSeek V4 MoE load balancing",
// DeepEP section). Within an expert, assignments keep (token, slot) order,
// so the result is unique and deterministic.
//
// Two launches per call, both one workgroup per block of kLayoutTokens
// tokens (all layers in one grid):
//  layout_count:   LDS histogram of the block's ids -> cnt[l][blk][Nb];
//                  also folds the score workgroups' column sums of q into
//                  one row per block (for the batch-mean entropy).
//  layout_scatter: every block reads all block histograms of its layer and
//                  derives its base position per expert (prefix over experts
//                  of the totals, plus the prefix over earlier blocks);
//                  in-block stable ranks come from per-64-slot LDS bitmaps
//                  (popcount of lower bits). One extra workgroup per layer
//                  computes the entropy of the batch-mean distribution.
#include <math.h>

#include "moer_internal.hpp"

namespace moer {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxSlotsPerBlock = kLayoutTokens * kMaxSlots;  // 2048
constexpr int kMaxChunks = kMaxSlotsPerBlock / 64;            // 32

__global__ __launch_bounds__(kThreads) void layout_count_kernel(LayoutArgs a) {
  __shared__ int hist[kMaxBuckets];
  const int layer = blockIdx.y;
  const int blk = blockIdx.x;
  const int t0 = blk * kLayoutTokens;
  const int nt = min(kLayoutTokens, a.T - t0);
  const int nslot = nt * a.Kt;
  const size_t base = (size_t)layer * a.T * a.Kt + (size_t)t0 * a.Kt;

  for (int e = threadIdx.x; e < a.Nb; e += kThreads) hist[e] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < nslot; i += kThreads) {
    const int e = a.idx[base + i];
    if (e >= 0 && e < a.Nb) atomicAdd(&hist[e], 1);
    if (a.fill_invalid) a.perm[base + i] = -1;
  }
  __syncthreads();
  int32_t* out = a.cnt + ((size_t)layer * a.nlb + blk) * a.Nb;
  for (int e = threadIdx.x; e < a.Nb; e += kThreads) out[e] = hist[e];

  if (a.colpart2 != nullptr) {
    // rows of the score workgroups covering this block's tokens, summed in order
    const int r0 = t0 / kScoreTokens;
    const int r1 = min(a.nsb, (t0 + nt + kScoreTokens - 1) / kScoreTokens);
    for (int e = threadIdx.x; e < a.N; e += kThreads) {
      float acc = 0.f;
      for (int r = r0; r < r1; ++r) acc += a.colpart[((size_t)layer * a.nsb + r) * a.N + e];
      a.colpart2[((size_t)layer * a.nlb + blk) * a.N + e] = acc;
    }
  }
}

// Exclusive scan of v[0..n) in LDS (n <= 2 * kThreads), deterministic.
__device__ void block_exclusive_scan(int* v, int* tmp, int n) {
  const int tid = threadIdx.x;
  const int i0 = 2 * tid, i1 = 2 * tid + 1;
  const int a0 = i0 < n ? v[i0] : 0;
  const int a1 = i1 < n ? v[i1] : 0;
  tmp[tid] = a0 + a1;
  __syncthreads();
  for (int o = 1; o < kThreads; o <<= 1) {
    const int add = tid >= o ? tmp[tid - o] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  const int excl = tmp[tid] - (a0 + a1);
  __syncthreads();
  if (i0 < n) v[i0] = excl;
  if (i1 < n) v[i1] = excl + a0;
  __syncthreads();
}

__device__ void batch_mean_entropy(const LayoutArgs& a, int layer) {
  __shared__ float red[kThreads];
  // mean_e = (1/T) sum_t q[t][e]; H = entropy of mean / sum(mean)
  float me[kMaxExperts / kThreads];
  float z = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxExperts / kThreads; ++k) {
    const int e = threadIdx.x + k * kThreads;
    float acc = 0.f;
    if (e < a.N)
      for (int b = 0; b < a.nlb; ++b) acc += a.colpart2[((size_t)layer * a.nlb + b) * a.N + e];
    me[k] = a.T > 0 ? acc / (float)a.T : 0.f;
    z += me[k];
  }
  red[threadIdx.x] = z;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  const float Z = red[0];
  __syncthreads();
  float hpart = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxExperts / kThreads; ++k) {
    const float q = Z > 0.f ? me[k] / Z : 0.f;
    hpart -= q > 0.f ? q * log2f(q) : 0.f;
  }
  red[threadIdx.x] = hpart;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.agg_entropy[layer] = a.T > 0 ? red[0] : 0.f;
}

__global__ __launch_bounds__(kThreads) void layout_scatter_kernel(LayoutArgs a) {
  __shared__ int total[2 * kThreads];
  __shared__ int pre[kMaxBuckets];
  __shared__ int scan_tmp[kThreads];
  __shared__ unsigned long long bits[kMaxChunks][kMaxBuckets];
  __shared__ unsigned short chunk_pre[kMaxChunks][kMaxBuckets];

  const int layer = blockIdx.y;
  const int blk = blockIdx.x;
  if (blk == a.nlb) {
    batch_mean_entropy(a, layer);
    return;
  }
  const int Nb = a.Nb;
  const int t0 = blk * kLayoutTokens;
  const int nt = min(kLayoutTokens, a.T - t0);
  const int nslot = nt * a.Kt;
  const int nchunk = (nslot + 63) / 64;
  const size_t lbase = (size_t)layer * a.T * a.Kt;
  const int flat0 = t0 * a.Kt;

  // totals and prefix over earlier blocks, per expert
  const int32_t* cnt = a.cnt + (size_t)layer * a.nlb * Nb;
  for (int e = threadIdx.x; e < 2 * kThreads; e += kThreads) {
    int tot = 0, p = 0;
    if (e < Nb) {
      for (int b = 0; b < a.nlb; ++b) {
        const int c = cnt[(size_t)b * Nb + e];
        tot += c;
        p += b < blk ? c : 0;
      }
      pre[e] = p;
    }
    total[e] = tot;
  }
  for (int c = 0; c < nchunk; ++c)
    for (int e = threadIdx.x; e < Nb; e += kThreads) bits[c][e] = 0ull;
  __syncthreads();
  const int last_count = total[Nb - 1];
  if (blk == 0) {
    for (int e = threadIdx.x; e < Nb; e += kThreads) a.counts[(size_t)layer * Nb + e] = total[e];
  }
  block_exclusive_scan(total, scan_tmp, Nb);  // total[e] := offset of expert e
  if (blk == 0) {
    int32_t* off = a.offsets + (size_t)layer * (Nb + 1);
    for (int e = threadIdx.x; e < Nb; e += kThreads) off[e] = total[e];
    if (threadIdx.x == 0) off[Nb] = total[Nb - 1] + last_count;
  }

  // membership bitmaps: bit i of bits[c][e] <=> slot c*64+i of this block is e
  for (int i = threadIdx.x; i < nslot; i += kThreads) {
    const int e = a.idx[lbase + flat0 + i];
    if (e >= 0 && e < Nb) atomicOr(&bits[i >> 6][e], 1ull << (i & 63));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < Nb; e += kThreads) {
    int run = 0;
    for (int c = 0; c < nchunk; ++c) {
      chunk_pre[c][e] = (unsigned short)run;
      run += __popcll(bits[c][e]);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nslot; i += kThreads) {
    const int e = a.idx[lbase + flat0 + i];
    const int flat = flat0 + i;
    if (e >= 0 && e < Nb) {
      const int c = i >> 6;
      const unsigned long long below = bits[c][e] & ((1ull << (i & 63)) - 1ull);
      const int pos = total[e] + pre[e] + chunk_pre[c][e] + __popcll(below);
      a.perm[lbase + pos] = flat;
      if (a.inv_perm != nullptr) a.inv_perm[lbase + flat] = pos;
    } else if (a.inv_perm != nullptr) {
      a.inv_perm[lbase + flat] = -1;
    }
  }
}

}  // namespace

hipError_t launch_layout(const LayoutArgs& a, int L, hipStream_t s) {
  // a.nlb >= 1 (an empty batch still writes zero counts and offsets)
  hipLaunchKernelGGL(layout_count_kernel, dim3(a.nlb, L), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int extra = a.agg_entropy != nullptr ? 1 : 0;
  hipLaunchKernelGGL(layout_scatter_kernel, dim3(a.nlb + extra, L), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moer
