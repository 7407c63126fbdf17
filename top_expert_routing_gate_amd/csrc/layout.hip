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

#include "load_balance.hpp"
#include "moer_internal.hpp"

namespace moer {
namespace {

constexpr int kThreads = 256;
constexpr int kBlocksPerLayoutBlock = kLayoutTokens / kRowTokens;  // 1
constexpr int kMaxSlotsPerBlock = kLayoutTokens * kMaxSlots;       // 1024
constexpr int kMaxChunks = kMaxSlotsPerBlock / 64;                 // 16
static_assert(kLayoutTokens % kRowTokens == 0, "layout block = whole histogram blocks");
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

// Exclusive scan of v[0..n) in LDS (n <= 2 * kThreads), deterministic:
// each thread adds its pair, waves scan with lane shuffles, then the wave
// totals are added in wave order.
__device__ void block_exclusive_scan(int* v, int* tmp, int n) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int i0 = 2 * tid, i1 = 2 * tid + 1;
  const int a0 = i0 < n ? v[i0] : 0;
  const int a1 = i1 < n ? v[i1] : 0;
  int x = a0 + a1;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    x += lane >= o ? y : 0;
  }
  if (lane == kWave - 1) tmp[wave] = x;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += tmp[w];
  const int excl = base + x - (a0 + a1);
  // each thread rewrites only the two entries it read
  if (i0 < n) v[i0] = excl;
  if (i1 < n) v[i1] = excl + a0;
  __syncthreads();
}

// Entropy (bits) of the batch mean of q: thread (quad of experts, row group)
// sums its rows with 16-byte loads; row groups are then added in order.
__device__ void batch_mean_entropy(const LayoutArgs& a, int layer) {
  constexpr int kQuads = kMaxExperts / 4;        // 64 expert quads
  constexpr int kGroups = kThreads / kQuads;     // 4 row groups
  __shared__ float4 part[kGroups][kQuads];
  __shared__ float red[kThreads];
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
  float me[4] = {0.f, 0.f, 0.f, 0.f};
  float z = 0.f;
  if (rg == 0) {
    float4 tot = part[0][qd];
    for (int g = 1; g < kGroups; ++g) {
      tot.x += part[g][qd].x; tot.y += part[g][qd].y;
      tot.z += part[g][qd].z; tot.w += part[g][qd].w;
    }
    const float invT = a.T > 0 ? 1.f / (float)a.T : 0.f;
    me[0] = tot.x * invT; me[1] = tot.y * invT; me[2] = tot.z * invT; me[3] = tot.w * invT;
    z = me[0] + me[1] + me[2] + me[3];
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
  for (int k = 0; k < 4; ++k) {
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

// total[e] = the layer's assignments of expert e (0 for e >= Nb) and, with
// lb >= 0, pre[e] = those in tokens before layout block lb: the segments
// wholly before it plus the blocks of its own segment before it.
__device__ void load_totals(const LayoutArgs& a, int layer, int lb, int* total, int* pre) {
  constexpr int kMaxSeg = 32;  // segments summed from registers; more take a loop
  const int b_first = lb * kBlocksPerLayoutBlock;
  const int s_own = lb >= 0 ? b_first / kSegBlocks : 0;
  const int32_t* seg = a.segsum + (size_t)layer * a.nseg * a.Nb;
  for (int e = threadIdx.x; e < 2 * kThreads; e += kThreads) {
    int tot = 0, p = 0;
    if (e < a.Nb) {
      for (int s0 = 0; s0 < a.nseg; s0 += kMaxSeg) {
        int v[kMaxSeg];
#pragma unroll
        for (int k = 0; k < kMaxSeg; ++k)
          v[k] = s0 + k < a.nseg ? seg[(size_t)(s0 + k) * a.Nb + e] : 0;
#pragma unroll
        for (int k = 0; k < kMaxSeg; ++k) {
          tot += v[k];
          p += s0 + k < s_own ? v[k] : 0;
        }
      }
      if (lb >= 0) {
        const uint16_t* row = a.cnt + ((size_t)layer * a.Nb + e) * a.nsb;
        const int b0 = s_own * kSegBlocks;
        if ((a.nsb & 7) == 0 && b0 + kSegBlocks <= a.nsb) {
          // the segment's block counts as two 16-byte loads, masked
          static_assert(kSegBlocks == 16, "two uint4 per segment");
          const uint4* r4 = reinterpret_cast<const uint4*>(row + b0);
          const uint4 q0 = r4[0], q1 = r4[1];
          const unsigned w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int b = b0 + 2 * k;
            p += (b < b_first ? (int)(w[k] & 0xFFFF) : 0) + (b + 1 < b_first ? (int)(w[k] >> 16) : 0);
          }
        } else {
          for (int b = b0; b < b_first; ++b) p += row[b];
        }
        pre[e] = p;
      }
    }
    total[e] = tot;
  }
}

// Load statistics and the sign-step bias update of this call's routed counts
// (one workgroup per layer, beside the scatter workgroups).
__device__ void balance_from_histograms(const LayoutArgs& a, int layer, int* total, int* pre) {
  __shared__ BalanceScratch bal;
  load_totals(a, layer, -1, total, pre);
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
  __shared__ int total[2 * kThreads];
  __shared__ int pre[kMaxBuckets];
  __shared__ int scan_tmp[kThreads];
  __shared__ unsigned long long bits[kMaxChunks][kMaxBuckets];
  __shared__ unsigned short chunk_pre[kMaxChunks][kMaxBuckets];

  const int layer = blockIdx.y;
  const int blk = blockIdx.x;
  if (a.cap_phase == 2 && a.cap_flag[layer] == 0) return;  // the first layout stands
  if (blk >= a.nlb) {
    if (blk == a.nlb && a.agg_entropy != nullptr)
      batch_mean_entropy(a, layer);
    else
      balance_from_histograms(a, layer, total, pre);
    return;
  }
  const int Nb = a.Nb;
  const int t0 = blk * kLayoutTokens;
  const int nt = max(0, min(kLayoutTokens, a.T - t0));
  const int nslot = nt * a.Kt;
  const int nchunk = (nslot + 63) / 64;
  const size_t lbase = (size_t)layer * a.T * a.Kt;
  const int flat0 = t0 * a.Kt;

  // the block's ids first: their loads overlap the totals' loads
  constexpr int kIdsPerThread = kMaxSlotsPerBlock / kThreads;
  int ids[kIdsPerThread];
#pragma unroll
  for (int k = 0; k < kIdsPerThread; ++k) {
    const int i = threadIdx.x + k * kThreads;
    ids[k] = i < nslot ? a.idx[lbase + flat0 + i] : -1;
  }
  // per expert: all assignments, and those in tokens before this block
  load_totals(a, layer, blk, total, pre);
  for (int c = 0; c < nchunk; ++c)
    for (int e = threadIdx.x; e < Nb; e += kThreads) bits[c][e] = 0ull;
  __syncthreads();
  const int last_count = total[Nb - 1];
  if (blk == 0)
    for (int e = threadIdx.x; e < Nb; e += kThreads) a.counts[(size_t)layer * Nb + e] = total[e];
  block_exclusive_scan(total, scan_tmp, Nb);  // total[e] := offset of expert e
  if (blk == 0) {
    int32_t* off = a.offsets + (size_t)layer * (Nb + 1);
    for (int e = threadIdx.x; e < Nb; e += kThreads) off[e] = total[e];
    if (threadIdx.x == 0) off[Nb] = total[Nb - 1] + last_count;
  }

  // membership bitmaps: bit i of bits[c][e] <=> slot c*64+i of this block is e
#pragma unroll
  for (int k = 0; k < kIdsPerThread; ++k) {
    const int i = threadIdx.x + k * kThreads;
    const int e = ids[k];
    if (i < nslot && e >= 0 && e < Nb) atomicOr(&bits[i >> 6][e], 1ull << (i & 63));
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
#pragma unroll
  for (int k = 0; k < kIdsPerThread; ++k) {
    const int i = threadIdx.x + k * kThreads;
    if (i >= nslot) break;
    const int e = ids[k];
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
