// Dispatch layout: per-expert counts (the listing's bincount in "MoE Routing
// Entropy vs Expert Saturation"), their exclusive prefix, and a stable
// permutation that groups every (token, slot) assignment by destination
// expert — the grouping dispatch needs ("DeepSeek V4 MoE load balancing",
// DeepEP section). Within an expert, assignments keep (token, slot) order,
// so the result is unique and deterministic.
//
// Histograms per 64-token block, cnt[l][e][b] (uint16, expert-major), come
// from the selection kernel or, for supplied ids, from layout_count below.
// The same kernels add every block histogram into segsum[l][s][e], the
// counts of segment s = 16 consecutive blocks (integer atomics: the sums do
// not depend on the order). layout_scatter runs one workgroup per 64-token
// layout block: an expert's total is the sum of its segments, and its
// assignments before the block are the earlier segments plus the earlier
// blocks of the block's own segment (at most 15 + 14 reads per expert). It
// scans the totals into the offsets and places its assignments; in-block
// stable ranks come from per-64-slot LDS membership bitmaps (popcount of the
// lower bits). Two extra workgroups per layer compute the entropy of the
// batch-mean routing distribution from the per-block column sums of q and,
// when asked, the load statistics and the bias update from the totals.
#include <math.h>

#include "layout_block.hpp"
#include "load_balance.hpp"
#include "moer_internal.hpp"

namespace moer {
namespace {

constexpr int kThreads = 256;
static_assert(kThreads == kBalanceThreads, "the first layout workgroup runs the balance routines");

// Histogram of supplied ids, one workgroup per 64-token block.
__global__ __launch_bounds__(kThreads) void layout_count_kernel(LayoutArgs a) {
  __shared__ int hist[kMaxBuckets];
  const int layer = blockIdx.y;
  if (a.cap_phase == 2 && a.cap_flag[layer] == 0) return;  // the first layout stands
  const int blk = blockIdx.x;
  const int t0 = blk * kRowTokens;
  const int nt = min(kRowTokens, a.T - t0);
  const int nslot = max(nt, 0) * a.Kt;
  const size_t base = (size_t)layer * a.T * a.Kt + (size_t)t0 * a.Kt;

  for (int e = threadIdx.x; e < a.Nb; e += kThreads) hist[e] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < nslot; i += kThreads) {
    const int e = a.idx[base + i];
    if (e >= 0 && e < a.Nb) atomicAdd(&hist[e], 1);
    if (a.fill_invalid) a.perm[base + i] = -1;
  }
  __syncthreads();
  uint16_t* out = a.cnt + (size_t)layer * a.Nb * a.nsb + blk;
  int32_t* seg = a.segsum + ((size_t)layer * a.nseg + blk / kSegBlocks) * a.Nb;
  for (int e = threadIdx.x; e < a.Nb; e += kThreads) {
    out[(size_t)e * a.nsb] = (uint16_t)hist[e];
    if (hist[e] != 0) atomicAdd(&seg[e], hist[e]);
  }
}

// Entropy (bits) of the batch mean of q: thread (quad of experts, row group)
// sums its rows with 16-byte loads; row groups are then added in order.
__device__ void batch_mean_entropy(const LayoutArgs& a, int layer) {
  constexpr int kQuads = kMaxExperts / 4;        // 64 expert quads
  constexpr int kGroups = kThreads / kQuads;     // 4 row groups
  __shared__ float4 part[kGroups][kQuads];
  const int qd = threadIdx.x % kQuads;
  const int rg = threadIdx.x / kQuads;
  const float* cp = a.colpart + (size_t)layer * a.nsb * a.N;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  const int e = qd * 4;
  if (e < a.N) {
    if ((a.N & 3) == 0) {
      // batches of kBatch rows: all their loads in flight before the adds,
      // which still run in row order
      constexpr int kBatch = 32;
      int r = rg;
      for (; r + (kBatch - 1) * kGroups < a.nsb; r += kBatch * kGroups) {
        float4 qv[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
          qv[k] = *reinterpret_cast<const float4*>(cp + (size_t)(r + k * kGroups) * a.N + e);
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          acc.x += qv[k].x; acc.y += qv[k].y; acc.z += qv[k].z; acc.w += qv[k].w;
        }
      }
      for (; r < a.nsb; r += kGroups) {
        const float4 q = *reinterpret_cast<const float4*>(cp + (size_t)r * a.N + e);
        acc.x += q.x; acc.y += q.y; acc.z += q.z; acc.w += q.w;
      }
    } else {
      for (int r = rg; r < a.nsb; r += kGroups) {
        const float* rowp = cp + (size_t)r * a.N;
        acc.x += rowp[e];
        if (e + 1 < a.N) acc.y += rowp[e + 1];
        if (e + 2 < a.N) acc.z += rowp[e + 2];
        if (e + 3 < a.N) acc.w += rowp[e + 3];
      }
    }
  }
  part[rg][qd] = acc;
  __syncthreads();
  // the row groups' sums in group order, then the rest in wavefront 0 alone
  // (lane = expert quad): sums over its 64 lanes by xor butterflies
  // (wave_allreduce), which leave the same value in every lane
  if (rg != 0) return;
  float4 tot = part[0][qd];
  for (int g = 1; g < kGroups; ++g) {
    tot.x += part[g][qd].x; tot.y += part[g][qd].y;
    tot.z += part[g][qd].z; tot.w += part[g][qd].w;
  }
  const float invT = a.T > 0 ? 1.f / (float)a.T : 0.f;
  const float me[4] = {tot.x * invT, tot.y * invT, tot.z * invT, tot.w * invT};
  auto add = [](float x, float y) { return x + y; };
  const float Z = wave_allreduce(me[0] + me[1] + me[2] + me[3], add);
  float hpart = 0.f;
  for (int k = 0; k < 4; ++k) {
    const float q = Z > 0.f ? me[k] / Z : 0.f;
    hpart -= q > 0.f ? q * log2f(q) : 0.f;
  }
  const float H = wave_allreduce(hpart, add);
  if (threadIdx.x == 0) a.agg_entropy[layer] = a.T > 0 ? H : 0.f;
}

// Load statistics and the sign-step bias update of this call's routed counts
// (one workgroup per layer, beside the scatter workgroups).
__device__ void balance_from_histograms(const LayoutArgs& a, int layer, int* total, int* pre) {
  __shared__ BalanceScratch bal;
  load_totals<kThreads>(a, layer, -1, total, pre);
  __syncthreads();
  if (a.cap_phase == 1) {
    // is any routed expert over capacity? then the statistics wait for the
    // final ids
    int over = 0;
    for (int e = threadIdx.x; e < a.N; e += kThreads) over |= total[e] > a.cap ? 1 : 0;
    over = __syncthreads_or(over);
    if (threadIdx.x == 0) a.cap_flag[layer] = over;
    if (over) return;
  }
  if (a.stats == nullptr && a.bias_inout == nullptr) return;
  block_load_balance(total, a.N, a.stats != nullptr ? a.stats + layer : nullptr,
                     a.bias_inout != nullptr ? a.bias_inout + (size_t)layer * a.N : nullptr,
                     a.bias_step, bal);
}

// Workgroups [0, nlb) place 64 tokens each; then, if requested, one
// workgroup for the batch-mean entropy and one for load balancing.
__global__ __launch_bounds__(kThreads, 1) void layout_scatter_kernel(LayoutArgs a) {
  __shared__ ScatterLds sl;
  const int layer = blockIdx.y;
  const int blk = blockIdx.x;
  if (a.cap_phase == 2 && a.cap_flag[layer] == 0) return;  // the first layout stands
  if (blk >= a.nlb) {
    if (blk == a.nlb && a.agg_entropy != nullptr)
      batch_mean_entropy(a, layer);
    else
      balance_from_histograms(a, layer, sl.total, sl.pre);
    return;
  }
  scatter_block<kThreads>(a, layer, blk, sl);
}

}  // namespace

hipError_t launch_layout(const LayoutArgs& a, int L, hipStream_t s) {
  if (a.need_count) {
    hipLaunchKernelGGL(layout_count_kernel, dim3(a.nsb, L), dim3(kThreads), 0, s, a);
    const hipError_t ec = hipGetLastError();
    if (ec != hipSuccess) return ec;
  }
  // a.nlb >= 1 (an empty batch still writes zero counts and offsets)
  const int extra = (a.agg_entropy != nullptr ? 1 : 0) +
                    (a.stats != nullptr || a.bias_inout != nullptr || a.cap_phase == 1 ? 1 : 0);
  hipLaunchKernelGGL(layout_scatter_kernel, dim3(a.nlb + extra, L), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moer
