// Gate GEMM and selection in one launch for routers with at most 16 experts
// (the top-2-of-8 router, the fp32 toy router): one workgroup of 1024 threads
// forms the affinities of 16 tokens against every expert and then routes
// them as the standalone selection kernel does (route_row.hpp: one 16-lane
// DPP row per token, lane j = expert j), writing the same kind of block
// outputs for the layout kernel. With all of a token's experts in one
// workgroup there is no depth-split partial round trip through memory and no
// second launch.
//
// Affinities h = x W_g^T ("MoE Routing Entropy vs Expert Saturation",
// Mathematics): the 16 wavefronts take 16 depth parts (steps dealt
// round-robin) of the same 16 x 16 block and each issues MFMAs with W_g rows
// as the A operand (16 expert rows, zero past N) and x rows as B, from
// operands loaded straight into registers, every load of a part in flight
// before its first MFMA (up to two steps at a time). One load instruction
// covers 64 contiguous bytes of each of the 16 rows. The 16 parts are added
// in part order through LDS.
//  - bf16: a step is 128 deep, four v_mfma_f32_16x16x32_bf16 (bf16 products
//    are exact in fp32 and accumulate in fp32);
//  - fp32: a step is 64 deep, sixteen v_mfma_f32_16x16x4f32.
// The lane's 8-element (bf16) or 4-element (fp32) group g of load i feeds
// the MFMA k-slot g of MFMA i (bf16), or component c of it the k-slot g of
// MFMA (i, c) (fp32): A and B take the same depth for every k-slot, so each
// step's MFMAs together sum its depth range once.
//
// The selection is the same as in the standalone kernel; only its workgroup
// holds 16 tokens (so a launch of T / 16 workgroups fills the chip for the
// few-thousand-token batches these routers see). Its histogram blocks are
// therefore 16 tokens and carry no running segment totals: the layout kernel
// sums the block counts itself, so no counter needs clearing first.
#include <hip/hip_ext.h>
#include <math.h>

#include "route_row.hpp"

namespace moer {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;  // 16 depth parts
constexpr int kTok = kSmallTokens;        // 16 tokens per workgroup
static_assert(kTok == 16 && (kRowTokens >> kSmallShift) == kTok, "16-token blocks");
constexpr int kSmallMaxN = kSmallMaxExperts;
static_assert(kSmallMaxN == kRowLanes, "one row lane per expert");
// the layout sums up to this many block counts per expert (no segment totals)
constexpr int kSmallMaxBlocks = 256;

typedef __bf16 sm_bf16x8 __attribute__((ext_vector_type(8)));
typedef float sm_floatx4 __attribute__((ext_vector_type(4)));

template <bool BF16>
struct StepOf {
  static constexpr int kDepth = BF16 ? 128 : 64;  // elements per step
  static constexpr int kPer = BF16 ? 8 : 4;        // elements per 16-byte load
};

// One step's operands of this lane (row r = lane % 16, group g = lane / 16):
// load i covers elements [s*D + i*D/4 + g*P, +P) of its token row (B) and
// its expert row (A); expert rows past N are zero.
template <bool BF16>
__device__ __forceinline__ void load_step(const uint4* xrow, const uint4* wrow, int s, int g,
                                          uint4 (&xv)[4], uint4 (&wv)[4]) {
  constexpr int D = StepOf<BF16>::kDepth, P = StepOf<BF16>::kPer;
#pragma unroll
  for (int i = 0; i < 4; ++i) xv[i] = xrow[(s * D + i * (D / 4) + g * P) / P];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    wv[i] = wrow != nullptr ? wrow[(s * D + i * (D / 4) + g * P) / P] : uint4{0u, 0u, 0u, 0u};
}

template <bool BF16>
__device__ __forceinline__ void mfma_step(const uint4 (&xv)[4], const uint4 (&wv)[4],
                                          sm_floatx4& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (BF16) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(sm_bf16x8, wv[i]),
                                                    __builtin_bit_cast(sm_bf16x8, xv[i]), acc, 0,
                                                    0, 0);
    } else {
      const float xs[4] = {__uint_as_float(xv[i].x), __uint_as_float(xv[i].y),
                           __uint_as_float(xv[i].z), __uint_as_float(xv[i].w)};
      const float ws[4] = {__uint_as_float(wv[i].x), __uint_as_float(wv[i].y),
                           __uint_as_float(wv[i].z), __uint_as_float(wv[i].w)};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ws[c], xs[c], acc, 0, 0, 0);
    }
  }
}

// The wavefront's 16x16 block over depth part w (steps w, w + 16, ...): lane
// l holds experts 4*(l/16) .. +3 of token l%16.
template <bool BF16>
__device__ __forceinline__ sm_floatx4 part_affinities(const uint4* xrow, const uint4* wrow, int d,
                                                      int w) {
  const int g = (threadIdx.x & 63) >> 4;
  const int nsteps = d / StepOf<BF16>::kDepth;
  sm_floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = w; s < nsteps; s += 2 * kWaves) {
    uint4 x0[4], w0[4], x1[4], w1[4];
    const bool two = s + kWaves < nsteps;
    load_step<BF16>(xrow, wrow, s, g, x0, w0);
    if (two) load_step<BF16>(xrow, wrow, s + kWaves, g, x1, w1);
    mfma_step<BF16>(x0, w0, acc);
    if (two) mfma_step<BF16>(x1, w1, acc);
  }
  return acc;
}

template <bool BF16, bool GROUPED, int MODE>
__global__ __launch_bounds__(kThreads) void route_small_kernel(ScoreArgs a, const void* x,
                                                               const void* W, int d) {
  __shared__ Cand cand[kTok][kCandStride];
  __shared__ int slot_id[kTok][kMaxSlots];
  __shared__ float slot_s[kTok][kMaxSlots];
  __shared__ int hist[kMaxBuckets];
  __shared__ __attribute__((aligned(16))) float colw[kWaves][kRowLanes];
  __shared__ __attribute__((aligned(16))) float part_h[kWaves][kTok][kSmallMaxN];

  const int N = a.N, T = a.T;
  const int Nb = N + a.n_shared;
  const int layer = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int r = threadIdx.x & 15;    // token row of the MFMA block / row lane = expert
  const int row = threadIdx.x >> 4;  // routing row (rows < kTok hold the tokens)
  const int t0 = blockIdx.x * kTok;

  for (int i = threadIdx.x; i < Nb; i += kThreads) hist[i] = 0;
  LaneConsts<1> lc;
  if (row < kTok) load_lane_consts<1>(a, layer, true, lc);

  {
    // tokens past T read row T - 1 (their results are never stored)
    const int tt = min(t0 + r, T - 1);
    const size_t esz = BF16 ? 2 : 4;
    const uint4* xrow = reinterpret_cast<const uint4*>(static_cast<const char*>(x) +
                                                       ((size_t)layer * T + tt) * d * esz);
    const uint4* wrow = r < N ? reinterpret_cast<const uint4*>(static_cast<const char*>(W) +
                                                               ((size_t)layer * N + r) * d * esz)
                              : nullptr;
    const sm_floatx4 acc = part_affinities<BF16>(xrow, wrow, d, wave);
    const int g = (threadIdx.x & 63) >> 4;
    *reinterpret_cast<sm_floatx4*>(&part_h[wave][r][4 * g]) = acc;
  }
  __syncthreads();  // every part stored; the histogram cleared

  float q[1] = {0.f};
  if (row < kTok) {  // wavefronts 0-3: one row per token
    float v[1] = {0.f};
#pragma unroll
    for (int p = 0; p < kWaves; ++p) v[0] += part_h[p][row][r];
    const int t = t0 + row;
    const RowLds rs{cand[row], slot_id[row], slot_s[row]};
    route_row<1, GROUPED, MODE>(a, layer, t, t < T, v, lc, rs, hist, q);
  }
  block_outputs<1, kThreads>(a, layer, N, Nb, q, hist, colw);
}

template <bool BF16, bool GROUPED>
auto pick(const ScoreArgs& a) {
  return a.score_fn == 1 ? route_small_kernel<BF16, GROUPED, kSigmoid>
                         : route_small_kernel<BF16, GROUPED, kSoftmax>;
}

}  // namespace

bool route_small_eligible(bool bf16, int T, int d, int N, int G, bool aligned) {
  if (T < 1 || T > kSmallMaxBlocks * kTok || N > kSmallMaxN || !route_rows_supports(N, G) ||
      d < 1 || !aligned)
    return false;
  return d % (bf16 ? StepOf<true>::kDepth : StepOf<false>::kDepth) == 0;
}

hipError_t launch_route_small(const ScoreArgs& a, const void* x, const void* W, int d, bool bf16,
                              int L, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const dim3 grid((a.T + kTok - 1) / kTok, L);
  auto k = bf16 ? (a.G > 1 ? pick<true, true>(a) : pick<true, false>(a))
                : (a.G > 1 ? pick<false, true>(a) : pick<false, false>(a));
  hipExtLaunchKernelGGL(k, grid, dim3(kThreads), 0, s, ev0, ev1, 0, a, x, W, d);
  return hipGetLastError();
}

}  // namespace moer
