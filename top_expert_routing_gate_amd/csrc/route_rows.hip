// Standalone selection kernel: one workgroup of 1024 threads routes 64
// tokens (one 16-lane row per token, see route_row.hpp), then writes its
// block's expert histogram (uint16, expert-major [L][Nb][blocks]) and its
// column sums of q ([L][blocks][N]) for the layout kernel. The affinities are
// the sum of the gate GEMM's depth-range partials, added in range order, or
// the given scores.
#include <math.h>

#include "route_row.hpp"

namespace moer {
namespace {

constexpr int kThreads = kRowTokens * kRowLanes;  // 1024: one row per token

template <int EPL, class S>
__device__ __forceinline__ void load_row(const ScoreArgs& a, size_t row_off, size_t split_stride,
                                         int e0, float (&v)[EPL]) {
  // EPL consecutive experts per lane, depth-range partials added in range
  // order; 16-byte loads when the lane's range is whole and aligned. The
  // loads of kBatch ranges are issued before any of them is added, so a
  // router with many ranges waits for ceil(nsplit / kBatch) round trips.
  constexpr int kBatch = EPL >= 16 ? 2 : 4;
  const int N = S::n(a);
#pragma unroll
  for (int j = 0; j < EPL; ++j) v[j] = 0.f;
  if (e0 >= N) return;
  if (EPL % 4 == 0 && e0 + EPL <= N && (N & 3) == 0) {
    constexpr int Q = EPL / 4;
    if constexpr (Q > 0) {
      if (a.nsplit == 2) {  // the common split, without the tail selects
        float4 q0[Q], q1[Q];
        const float4* s0 = reinterpret_cast<const float4*>(a.in + row_off + e0);
        const float4* s1 = reinterpret_cast<const float4*>(a.in + split_stride + row_off + e0);
#pragma unroll
        for (int j = 0; j < Q; ++j) q0[j] = s0[j];
#pragma unroll
        for (int j = 0; j < Q; ++j) q1[j] = s1[j];
#pragma unroll
        for (int j = 0; j < Q; ++j) {
          v[4 * j] = q0[j].x + q1[j].x; v[4 * j + 1] = q0[j].y + q1[j].y;
          v[4 * j + 2] = q0[j].z + q1[j].z; v[4 * j + 3] = q0[j].w + q1[j].w;
        }
        return;
      }
    }
    for (int sp0 = 0; sp0 < a.nsplit; sp0 += kBatch) {
      float4 q[kBatch][Q];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        // ranges past nsplit re-read the last one (not added)
        const int sp = min(sp0 + b, a.nsplit - 1);
        const float4* src = reinterpret_cast<const float4*>(a.in + sp * split_stride + row_off + e0);
#pragma unroll
        for (int j = 0; j < Q; ++j) q[b][j] = src[j];
      }
      // in range order; a range past nsplit leaves v as it is (a select,
      // not a branch, so its load stays with the others)
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const bool first = sp0 + b == 0, in = sp0 + b < a.nsplit;
#pragma unroll
        for (int j = 0; j < Q; ++j) {
          const float4 w = q[b][j];
          v[4 * j] = first ? w.x : (in ? v[4 * j] + w.x : v[4 * j]);
          v[4 * j + 1] = first ? w.y : (in ? v[4 * j + 1] + w.y : v[4 * j + 1]);
          v[4 * j + 2] = first ? w.z : (in ? v[4 * j + 2] + w.z : v[4 * j + 2]);
          v[4 * j + 3] = first ? w.w : (in ? v[4 * j + 3] + w.w : v[4 * j + 3]);
        }
      }
    }
    return;
  }
  for (int sp = 0; sp < a.nsplit; ++sp) {
    const float* src = a.in + sp * split_stride + row_off;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = min(e0 + j, N - 1);
      const float q = (e0 + j < N) ? src[e] : 0.f;
      v[j] = sp == 0 ? q : v[j] + q;
    }
  }
}

template <int EPL, bool GROUPED, int MODE, int LPG, class S>
__global__ __launch_bounds__(kThreads) void route_rows_kernel(ScoreArgs a) {
  __shared__ Cand cand[kRowTokens][kCandStride];
  __shared__ int slot_id[kRowTokens][kMaxSlots];
  __shared__ float slot_s[kRowTokens][kMaxSlots];
  __shared__ int hist[kMaxBuckets];
  constexpr int kWaves = kThreads / kWave;
  __shared__ __attribute__((aligned(16))) float colw[kWaves][kRowLanes * EPL];

  const int N = S::n(a), T = a.T;
  const int Nb = N + S::ns(a);
  const int layer = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int rl = lane & 15;
  const int row = threadIdx.x >> 4;  // row within the workgroup = token slot
  const int t = blockIdx.x * kRowTokens + row;
  const bool live = t < T;

  for (int i = threadIdx.x; i < Nb; i += kThreads) hist[i] = 0;
  LaneConsts<EPL> lc;
  load_lane_consts<EPL, S>(a, layer, MODE != kGiven, lc);
  const size_t row_off = ((size_t)layer * T + (live ? t : 0)) * N;
  const size_t split_stride = (size_t)gridDim.y * T * N;
  float v[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) v[j] = 0.f;
  // The rows' loads go out in two halves: the first half's before the
  // barrier (which also publishes the cleared histogram), the second half's
  // after it. Every workgroup of the launch does the same, so the first
  // halves' data arrives while only half of the launch's loads are in
  // flight, and those rows are routed while the second halves stream in.
  const bool first_half = row < kRowTokens / 2;
  if (live && first_half) load_row<EPL, S>(a, row_off, split_stride, rl * EPL, v);
  __syncthreads();  // histogram cleared; first-half rows loaded
  if (live && !first_half) load_row<EPL, S>(a, row_off, split_stride, rl * EPL, v);

  const RowLds rs{cand[row], slot_id[row], slot_s[row]};
  float q[EPL];
  route_row<EPL, GROUPED, MODE, LPG, S>(a, layer, t, live, v, lc, rs, hist, q);
  block_outputs<EPL, kThreads>(a, layer, N, Nb, q, hist, colw);
}

// Small and mid-sized batches (fewer than 256 blocks of 64 tokens, so fewer
// 64-token workgroups than CUs): TOK = 16 or 32 tokens per workgroup, so the
// batch spreads over more CUs. All 1024 threads first add the depth-range
// partials of the workgroup's tokens into LDS, one 4-expert group of one
// token each, with the loads of up to eight ranges in flight at once and the
// ranges added in order (the sums are bit for bit those of load_row); the
// first TOK rows (TOK / 4 wavefronts) then route from LDS. The histogram
// blocks are TOK tokens and carry no segment totals (the layout kernel sums
// the block counts).
template <int EPL, bool GROUPED, int MODE, int LPG, class S, int TOK>
__global__ __launch_bounds__(kThreads) void route_rows_few_kernel(ScoreArgs a) {
  constexpr int kTok = TOK;
  static_assert(TOK == 16 || TOK == 32, "16 or 32 tokens per workgroup");
  constexpr int kWidth = kRowLanes * EPL;  // experts per row, N rounded up
  constexpr int kGroups = kWidth / 4;      // 4-expert groups per row
  constexpr int kBatch = 8;
  static_assert(kWidth % 4 == 0, "whole 4-expert groups");
  __shared__ Cand cand[kTok][kCandStride];
  __shared__ int slot_id[kTok][kMaxSlots];
  __shared__ float slot_s[kTok][kMaxSlots];
  __shared__ int hist[kMaxBuckets];
  constexpr int kWaves = kThreads / kWave;
  __shared__ __attribute__((aligned(16))) float colw[kWaves][kWidth];
  __shared__ __attribute__((aligned(16))) float hs[kTok][kWidth];

  const int N = S::n(a), T = a.T;
  const int Nb = N + S::ns(a);
  const int layer = blockIdx.y;
  const int rl = threadIdx.x & 15;
  const int row = threadIdx.x >> 4;
  const int t0 = blockIdx.x * kTok;

  for (int i = threadIdx.x; i < Nb; i += kThreads) hist[i] = 0;
  LaneConsts<EPL> lc;
  if (row < kTok) load_lane_consts<EPL, S>(a, layer, MODE != kGiven, lc);
  const size_t split_stride = (size_t)gridDim.y * T * N;
  for (int i = threadIdx.x; i < kTok * kGroups; i += kThreads) {
    const int r = i / kGroups, e = 4 * (i - r * kGroups);
    const size_t off = ((size_t)layer * T + min(t0 + r, T - 1)) * N + e;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (e < N) {
      for (int sp0 = 0; sp0 < a.nsplit; sp0 += kBatch) {
        float q[kBatch][4];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const float* src = a.in + (size_t)min(sp0 + b, a.nsplit - 1) * split_stride + off;
          if ((N & 3) == 0) {
            const float4 f = *reinterpret_cast<const float4*>(src);
            q[b][0] = f.x; q[b][1] = f.y; q[b][2] = f.z; q[b][3] = f.w;
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) q[b][k] = e + k < N ? src[min(k, N - 1 - e)] : 0.f;
          }
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const bool first = sp0 + b == 0, in = sp0 + b < a.nsplit;
#pragma unroll
          for (int k = 0; k < 4; ++k) acc[k] = first ? q[b][k] : (in ? acc[k] + q[b][k] : acc[k]);
        }
      }
    }
    *reinterpret_cast<float4*>(&hs[r][e]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  }
  __syncthreads();  // partial sums in LDS; histogram cleared

  float q[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) q[j] = 0.f;
  if (row < kTok) {  // the first kTok / 4 wavefronts: one row per token
    float v[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) v[j] = hs[row][rl * EPL + j];
    const int t = t0 + row;
    const RowLds rs{cand[row], slot_id[row], slot_s[row]};
    route_row<EPL, GROUPED, MODE, LPG, S>(a, layer, t, t < T, v, lc, rs, hist, q);
  }
  block_outputs<EPL, kThreads>(a, layer, N, Nb, q, hist, colw);
}

template <int EPL, bool GROUPED, int TOK>
auto pick_kernel_few(const ScoreArgs& a) {
  if (!a.apply_score) return route_rows_few_kernel<EPL, GROUPED, kGiven, 0, AnyShape, TOK>;
  if (a.score_fn == 1) return route_rows_few_kernel<EPL, GROUPED, kSigmoid, 0, AnyShape, TOK>;
  return route_rows_few_kernel<EPL, GROUPED, kSoftmax, 0, AnyShape, TOK>;
}

template <int EPL, bool GROUPED, int LPG = 0, class S = AnyShape>
auto pick_kernel(const ScoreArgs& a) {
  if (!a.apply_score) return route_rows_kernel<EPL, GROUPED, kGiven, LPG, S>;
  if (a.score_fn == 1) return route_rows_kernel<EPL, GROUPED, kSigmoid, LPG, S>;
  return route_rows_kernel<EPL, GROUPED, kSoftmax, LPG, S>;
}

// Shapes with kernels of their own (everything fixed at compile time): the
// DeepSeek-V3 router (256 experts, 8 groups of 32, keep 4, top-8) and the
// decode-shaped router (256 experts, top-8 plus one shared slot).
using DeepSeekV3Shape = RowShape<256, 8, 8, 4, 0>;
using DecodeShape = RowShape<256, 8, 1, 1, 1>;

template <int EPL>
hipError_t launch_epl(const ScoreArgs& a, int L, int rows, hipStream_t s) {
  if (rows == 16 || rows == 32) {
    const dim3 grid_few((a.T + rows - 1) / rows, L);
    auto kf = rows == 16
                  ? (a.G > 1 ? pick_kernel_few<EPL, true, 16>(a) : pick_kernel_few<EPL, false, 16>(a))
                  : (a.G > 1 ? pick_kernel_few<EPL, true, 32>(a) : pick_kernel_few<EPL, false, 32>(a));
    hipLaunchKernelGGL(kf, grid_few, dim3(kThreads), 0, s, a);
    return hipGetLastError();
  }
  const dim3 grid((a.T + kRowTokens - 1) / kRowTokens, L);
  // the DeepSeek-V3 geometry (groups of 32 experts, 2 row lanes per group)
  // gets a kernel with the group width fixed at compile time
  const bool two_lane_groups = EPL == 16 && a.G > 1 && a.N / a.G == 2 * EPL;
  auto k = a.G > 1 ? (two_lane_groups ? pick_kernel<EPL, true, 2>(a) : pick_kernel<EPL, true>(a))
                   : pick_kernel<EPL, false>(a);
  if constexpr (EPL == 16) {
    if (DeepSeekV3Shape::matches(a)) k = pick_kernel<EPL, true, 2, DeepSeekV3Shape>(a);
    if (DecodeShape::matches(a)) k = pick_kernel<EPL, false, 0, DecodeShape>(a);
  }
  hipLaunchKernelGGL(k, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int route_rows_epl(int N) {
  int epl = 1;
  while (epl * kRowLanes < N) epl *= 2;
  return epl;
}

bool route_rows_supports(int N, int G) {
  if (N > kMaxExperts) return false;
  if (G <= 1) return true;
  const int gsz = N / G, epl = route_rows_epl(N);
  if (gsz % epl != 0) return false;
  const int lpg = gsz / epl;
  return lpg >= 1 && lpg <= kRowLanes && (lpg & (lpg - 1)) == 0;
}

int route_rows_tokens(int L, int T) {
  const long long blocks = T > 0 ? (long long)L * ((T + kRowTokens - 1) / kRowTokens) : kFewGrid;
  return blocks < kTinyGrid ? 16 : blocks < kFewGrid ? 32 : kRowTokens;
}

hipError_t launch_route_rows(const ScoreArgs& a, int L, hipStream_t s, int rows) {
  switch (route_rows_epl(a.N)) {
    case 1: return launch_epl<1>(a, L, rows, s);
    case 2: return launch_epl<2>(a, L, rows, s);
    case 4: return launch_epl<4>(a, L, rows, s);
    case 8: return launch_epl<8>(a, L, rows, s);
    default: return launch_epl<16>(a, L, rows, s);
  }
}

}  // namespace moer
