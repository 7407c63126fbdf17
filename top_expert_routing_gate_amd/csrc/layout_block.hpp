// One layout block (64 tokens) of the dispatch layout: per-expert counts (the
// listing's bincount in "MoE Routing Entropy vs Expert Saturation"), their
// exclusive prefix, and the stable permutation that groups every (token,
// slot) assignment by destination expert ("DeepSeek V4 MoE load balancing",
// DeepEP section: dispatch needs tokens grouped by their expert). Within an
// expert, assignments keep (token, slot) order, so the result is unique.
//
// Inputs: the per-64-token-block histograms cnt[l][e][b] (uint16,
// expert-major) and the per-segment totals segsum[l][s][e] (segment = 16
// consecutive blocks), both complete before these routines run. An expert's
// total is the sum of its segments; its assignments before block b are the
// earlier segments plus the earlier blocks of b's own segment. The totals
// are scanned into offsets, and the block's assignments are placed by
// popcount ranks in per-64-slot LDS membership bitmaps.
//
// Written for any workgroup size NT (a multiple of 64, 256..1024); every
// thread of the workgroup must call these routines (they hold barriers).
#pragma once

#include "moer_internal.hpp"

namespace moer {

constexpr int kMaxSlotsPerBlock = kLayoutTokens * kMaxSlots;  // 1024
constexpr int kMaxChunks = kMaxSlotsPerBlock / 64;            // 16
static_assert(kLayoutTokens == kRowTokens, "a layout block is one histogram block");

// LDS of one layout block.
struct ScatterLds {
  int total[kMaxBuckets];
  int pre[kMaxBuckets];
  int scan_tmp[16];
  unsigned long long bits[kMaxChunks][kMaxBuckets];
  unsigned short chunk_pre[kMaxChunks][kMaxBuckets];
};

// Exclusive scan of v[0..n) in LDS (n <= 2 * NT), deterministic: each thread
// adds its pair, waves scan with lane shuffles, then the wave totals are
// added in wave order.
template <int NT>
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

// No segment totals (16-token histogram blocks): the block counts of every
// expert, eight per 16-byte load, spread over the whole workgroup and added
// into total / pre with LDS integer atomics (any order gives the same sums).
// Layout block lb starts at histogram block lb << hist_shift.
template <int NT>
__device__ void sum_block_counts(const LayoutArgs& a, int layer, int lb, int* total, int* pre) {
  const int hb = lb >= 0 ? lb << a.hist_shift : 0;
  const int nch = (a.nsb + 7) / 8;
  for (int e = threadIdx.x; e < a.Nb; e += NT) {
    total[e] = 0;
    if (lb >= 0) pre[e] = 0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < a.Nb * nch; i += NT) {
    const int e = i / nch, c = i - e * nch;
    const uint16_t* row = a.cnt + ((size_t)layer * a.Nb + e) * a.nsb;
    const int b0 = 8 * c;
    int tot = 0, p = 0;
    if ((a.nsb & 7) == 0) {
      const uint4 w4 = reinterpret_cast<const uint4*>(row)[c];
      const unsigned w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int b = b0 + 2 * m;
        const int c0 = (int)(w[m] & 0xFFFF), c1 = (int)(w[m] >> 16);
        tot += c0 + c1;
        p += (b < hb ? c0 : 0) + (b + 1 < hb ? c1 : 0);
      }
    } else {
      for (int b = b0; b < min(b0 + 8, a.nsb); ++b) {
        const int cb = row[b];
        tot += cb;
        p += b < hb ? cb : 0;
      }
    }
    if (tot != 0) atomicAdd(&total[e], tot);
    if (p != 0) atomicAdd(&pre[e], p);
  }
}

// total[e] = the layer's assignments of expert e (e < Nb) and, with lb >= 0,
// pre[e] = those in tokens before layout block lb: the segments wholly before
// it plus the blocks of its own segment before it (with no segment totals:
// sums of the block counts, above). Complete after the caller's next
// barrier. Every load is issued before any is used (clamped indices, values
// masked afterwards), so the block counts and the segment totals share one
// memory round trip.
template <int NT>
__device__ void load_totals(const LayoutArgs& a, int layer, int lb, int* total, int* pre) {
  constexpr int kSegChunk = 16;  // segment totals loaded at once per expert
  static_assert(kSegBlocks % 8 == 0, "whole 16-byte loads of block counts per segment");
  constexpr int kVec = kSegBlocks / 8;
  if (a.segsum == nullptr) {
    sum_block_counts<NT>(a, layer, lb, total, pre);
    return;
  }
  const int nseg = a.nseg;
  const int s_own = lb >= 0 ? lb / kSegBlocks : 0;
  const int b0 = s_own * kSegBlocks;
  const bool vec = lb >= 0 && (a.nsb & 7) == 0 && b0 + kSegBlocks <= a.nsb;
  for (int e = threadIdx.x; e < a.Nb; e += NT) {
    const uint16_t* row = a.cnt + ((size_t)layer * a.Nb + e) * a.nsb;
    const int32_t* seg = a.segsum + (size_t)layer * nseg * a.Nb;
    uint4 q[kVec];
    if (vec) {
      const uint4* r4 = reinterpret_cast<const uint4*>(row + b0);
#pragma unroll
      for (int k = 0; k < kVec; ++k) q[k] = r4[k];
    }
    int tot = 0, p = 0;
    for (int s0 = 0; s0 < nseg; s0 += kSegChunk) {
      int v[kSegChunk];
#pragma unroll
      for (int k = 0; k < kSegChunk; ++k) v[k] = seg[(size_t)min(s0 + k, nseg - 1) * a.Nb + e];
#pragma unroll
      for (int k = 0; k < kSegChunk; ++k) {
        const bool in = s0 + k < nseg;
        tot += in ? v[k] : 0;
        p += (in && s0 + k < s_own) ? v[k] : 0;
      }
    }
    if (lb >= 0) {
      if (vec) {
        // the own segment's earlier blocks, eight uint16 counts per load
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
          const unsigned w[4] = {q[k].x, q[k].y, q[k].z, q[k].w};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int b = b0 + 8 * k + 2 * m;
            p += (b < lb ? (int)(w[m] & 0xFFFF) : 0) + (b + 1 < lb ? (int)(w[m] >> 16) : 0);
          }
        }
      } else {
        for (int b = b0; b < lb; ++b) p += row[b];
      }
      pre[e] = p;
    }
    total[e] = tot;
  }
}

// Place layout block blk of `layer` (blk < a.nlb): counts and offsets (block
// 0 writes them), perm, inv_perm.
template <int NT>
__device__ void scatter_block(const LayoutArgs& a, int layer, int blk, ScatterLds& sl) {
  const int Nb = a.Nb;
  const int t0 = blk * kLayoutTokens;
  const int nt = max(0, min(kLayoutTokens, a.T - t0));
  const int nslot = nt * a.Kt;
  const int nchunk = (nslot + 63) / 64;
  const size_t lbase = (size_t)layer * a.T * a.Kt;
  const int flat0 = t0 * a.Kt;

  // the block's ids first: their loads overlap the totals' loads
  constexpr int kIdsPerThread = kMaxSlotsPerBlock / NT;
  static_assert(kMaxSlotsPerBlock % NT == 0, "ids split evenly over the threads");
  int ids[kIdsPerThread];
#pragma unroll
  for (int k = 0; k < kIdsPerThread; ++k) {
    const int i = threadIdx.x + k * NT;
    ids[k] = i < nslot ? a.idx[lbase + flat0 + i] : -1;
  }
  // per expert: all assignments, and those in tokens before this block
  load_totals<NT>(a, layer, blk, sl.total, sl.pre);
  for (int c = 0; c < nchunk; ++c)
    for (int e = threadIdx.x; e < Nb; e += NT) sl.bits[c][e] = 0ull;
  __syncthreads();
  const int last_count = sl.total[Nb - 1];
  if (blk == 0)
    for (int e = threadIdx.x; e < Nb; e += NT) a.counts[(size_t)layer * Nb + e] = sl.total[e];
  block_exclusive_scan<NT>(sl.total, sl.scan_tmp, Nb);  // total[e] := offset of expert e
  if (blk == 0) {
    int32_t* off = a.offsets + (size_t)layer * (Nb + 1);
    for (int e = threadIdx.x; e < Nb; e += NT) off[e] = sl.total[e];
    if (threadIdx.x == 0) off[Nb] = sl.total[Nb - 1] + last_count;
  }

  // membership bitmaps: bit i of bits[c][e] <=> slot c*64+i of this block is e
#pragma unroll
  for (int k = 0; k < kIdsPerThread; ++k) {
    const int i = threadIdx.x + k * NT;
    const int e = ids[k];
    if (i < nslot && e >= 0 && e < Nb) atomicOr(&sl.bits[i >> 6][e], 1ull << (i & 63));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < Nb; e += NT) {
    int run = 0;
    for (int c = 0; c < nchunk; ++c) {
      sl.chunk_pre[c][e] = (unsigned short)run;
      run += __popcll(sl.bits[c][e]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kIdsPerThread; ++k) {
    const int i = threadIdx.x + k * NT;
    if (i >= nslot) break;
    const int e = ids[k];
    const int flat = flat0 + i;
    if (e >= 0 && e < Nb) {
      const int c = i >> 6;
      const unsigned long long below = sl.bits[c][e] & ((1ull << (i & 63)) - 1ull);
      const int pos = sl.total[e] + sl.pre[e] + sl.chunk_pre[c][e] + __popcll(below);
      // pos < T * Kt whenever the block counts agree with the ids; the guard
      // keeps a disagreement (a block-count mismatch between kernels) inside
      // the layer's rows, where the parity checks see it
      if ((unsigned)pos < (unsigned)(a.T * a.Kt)) a.perm[lbase + pos] = flat;
      if (a.inv_perm != nullptr) a.inv_perm[lbase + flat] = pos;
    } else if (a.inv_perm != nullptr) {
      a.inv_perm[lbase + flat] = -1;
    }
  }
}

}  // namespace moer
