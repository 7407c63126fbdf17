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
  // EPL consecutive experts per lane, depth-range partials added in order;
  // 16-byte loads when the lane's range is whole and aligned
  const int N = S::n(a);
#pragma unroll
  for (int j = 0; j < EPL; ++j) v[j] = 0.f;
  if (e0 >= N) return;
  if (EPL % 4 == 0 && e0 + EPL <= N && (N & 3) == 0) {
    for (int sp = 0; sp < a.nsplit; ++sp) {
      const float4* src = reinterpret_cast<const float4*>(a.in + sp * split_stride + row_off + e0);
#pragma unroll
      for (int j = 0; j < EPL / 4; ++j) {
        const float4 q = src[j];
        if (sp == 0) {
          v[4 * j] = q.x; v[4 * j + 1] = q.y; v[4 * j + 2] = q.z; v[4 * j + 3] = q.w;
        } else {
          v[4 * j] += q.x; v[4 * j + 1] += q.y; v[4 * j + 2] += q.z; v[4 * j + 3] += q.w;
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
hipError_t launch_epl(const ScoreArgs& a, int L, hipStream_t s) {
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

hipError_t launch_route_rows(const ScoreArgs& a, int L, hipStream_t s) {
  switch (route_rows_epl(a.N)) {
    case 1: return launch_epl<1>(a, L, s);
    case 2: return launch_epl<2>(a, L, s);
    case 4: return launch_epl<4>(a, L, s);
    case 8: return launch_epl<8>(a, L, s);
    default: return launch_epl<16>(a, L, s);
  }
}

}  // namespace moer
