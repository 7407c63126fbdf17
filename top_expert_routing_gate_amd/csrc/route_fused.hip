// One co-resident launch for the whole router pass of a large batch: gate
// GEMM, scores, group-limited top-k, weights, entropy, histograms, and then
// (after a grid-wide barrier) the dispatch layout, the batch-mean entropy,
// the load statistics and the bias update.
//
// The method per token is the one route_row.hpp implements (pages cited
// there): h = x · W_g ("MoE Routing Entropy vs Expert Saturation",
// Mathematics), sigmoid or softmax scores, key = s + b (auxiliary-loss-free
// balancing, "DeepSeek V4 MoE load balancing"), group-limited top-k
// ("DeepSeek-V3 Group-Limited Expert Routing", s.1 and s.3), renormalised
// weights and routing entropy; the layout and balance steps are those of
// layout_block.hpp and load_balance.hpp.
//
// Work split. Each tile is 128 tokens x all experts; its depth d is split in
// two halves, and each half is one workgroup (256 workgroups for the
// 16k-token batch: one per CU). The two workgroups of a tile each own 64 of
// its tokens. After the GEMM main loop a workgroup keeps its own tokens'
// partial affinities in LDS and stores the partner's half to an exchange
// buffer; once both halves are published, it adds the partner's partial
// (h = part0 + part1: two terms, so the sum is the same in either order and
// equal to the separate selection kernel's), routes its 64 tokens from LDS,
// and writes its block histogram and column sums. A grid barrier then makes
// every histogram visible, and each workgroup places its own 64-token layout
// block. Compared with separate launches this writes and re-reads half the
// partial affinities, and saves two kernel boundaries.
//
// Synchronisation needs every workgroup of the launch to be resident at
// once: the host launches this kernel only when the occupancy calculator
// says the whole grid fits. Waits are bounded in time: a wait that runs out
// (which only a violated residency assumption could cause) gives up, so the
// launch always ends. Counters start at zero (a fill kernel clears them
// before the launch); releases and acquires are agent-scope atomics, which
// write back and invalidate the L2 of the die (the two halves of a tile run
// on different dies).
#include <math.h>

#include <atomic>

#include "gemm_pipeline.hpp"
#include "layout_block.hpp"
#include "load_balance.hpp"
#include "route_row.hpp"

namespace moer {
namespace {

constexpr int kBT = 128, kBE = 256, kWT = 2, kWE = 2, kNP = 4, kNStage = 3;
using Pipe = GemmPipeline<kBT, kBE, kWT, kWE, kNP, kNStage>;
constexpr int kFThreads = Pipe::kThreads;        // 512
constexpr int kFWaves = kFThreads / kWave;       // 8
constexpr int kSplit = 2;                        // depth halves per tile
constexpr int kSub = kBT / kSplit;               // tokens routed per workgroup
constexpr int kEPL = 16;                         // experts per row lane (N in (128, 256])
constexpr int kPassRows = kFWaves * 4;           // token rows routed at once
constexpr int kPasses = kSub / kPassRows;        // 2
static_assert(kSub == kRowTokens, "a workgroup's tokens are one histogram block");
static_assert(kBT / kWT == kSub, "a consumer row of waves owns one token half");
static_assert(kPasses * kPassRows == kSub, "whole passes");

// LDS after the GEMM main loop (carved from the ring).
constexpr int kHRowBytes = kMaxExperts * 4;                 // one token's affinities
constexpr int kOffH = 0;                                    // [kSub][256] fp32, swizzled
constexpr int kOffCand = kOffH + kSub * kHRowBytes;         // [kPassRows][kCandStride]
constexpr int kOffSlotId = kOffCand + kPassRows * kCandStride * (int)sizeof(Cand);
constexpr int kOffSlotS = kOffSlotId + kPassRows * kMaxSlots * 4;
constexpr int kOffHist = kOffSlotS + kPassRows * kMaxSlots * 4;
constexpr int kOffColw = kOffHist + kMaxBuckets * 4;        // [kFWaves][256] fp32
constexpr int kRouteLds = kOffColw + kFWaves * kMaxExperts * 4;
// after the grid barrier
constexpr int kOffScatter = 0;
constexpr int kOffBal = 64 * 1024;
constexpr int kOffRed = kOffBal + 256;
static_assert(kRouteLds <= (int)Pipe::kRingBytes, "routing scratch fits in the ring");
static_assert(sizeof(ScatterLds) <= kOffBal && kOffRed + kFThreads * 4 <= (int)Pipe::kRingBytes,
              "layout scratch fits in the ring");
static_assert(sizeof(BalanceScratch) <= 256, "balance scratch");

// Chunk (4 experts) c4 of token row r lives at chunk c4 ^ ((c4 >> 4) & 3) ^
// (r & 15) of the row: the GEMM's accumulator stores (16 token rows, one
// chunk column) and the routing reads (16 consecutive lanes of one row, every
// fourth chunk) both spread over all 16 chunk positions of 256 bytes.
__device__ __forceinline__ int h_chunk(int r, int c4) { return c4 ^ ((c4 >> 4) & 3) ^ (r & 15); }

struct FusedArgs {
  const uint16_t* x;   // [L][T][d] bf16
  const uint16_t* W;   // [L][N][d] bf16
  float* part;         // [2][L][T][N] exchange: half s's partial for the partner's tokens
  int32_t* sync;       // [n_tiles] pair counters, [L] entropy tickets, [1] grid counter
  float* colmean;      // [L][N] batch-mean q per expert
  ScoreArgs sa;        // selection outputs and constants (in / nsplit unused)
  LayoutArgs la;       // layout outputs (cnt, segsum, colpart shared with sa)
  int L, T, d, N, n_tt, n_work, per_xcd;
  int layout;          // 1: run the layout phase here (else a separate launch does)
  long long spin_ticks;  // wait bound in s_memrealtime ticks (100 MHz)
};

// Spin until *p >= target (agent scope), bounded in time; then acquire.
__device__ __forceinline__ void wait_at_least(int32_t* p, int target, long long ticks) {
  const long long t0 = (long long)__builtin_amdgcn_s_memrealtime();
  while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    __builtin_amdgcn_s_sleep(2);
    if ((long long)__builtin_amdgcn_s_memrealtime() - t0 > ticks) break;
  }
  __atomic_thread_fence(__ATOMIC_ACQUIRE);  // agent scope: invalidates the die's caches
}

// Every wave's stores have completed (vmcnt also counts stores on this
// architecture); then the workgroup meets.
__device__ __forceinline__ void stores_done_barrier() {
  __builtin_amdgcn_s_waitcnt(wait_imm(0));
  __syncthreads();
}

template <bool GROUPED, int MODE, int LPG>
__global__ __launch_bounds__(kFThreads, 1) void route_fused_kernel(FusedArgs f) {
  __shared__ u32x4 ring[kNStage][Pipe::kStageSlots];
  GemmWork w;
  if (!decode_work(f.n_tt, 1, kSplit, f.n_work, f.per_xcd, w)) return;
  const int layer = w.layer;
  const int t0 = w.tt * kBT;
  const int krange = f.d / kSplit;
  const int nk = krange / kKStage;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int T = f.T, N = f.N;
  char* lds = reinterpret_cast<char*>(&ring[0][0]);

  // ---- gate GEMM over this workgroup's depth half ----------------------------
  floatx4 acc[Pipe::ME][Pipe::MT];
  if (wave >= Pipe::kConsumers) {
    Pipe::produce(ring, f.x + (size_t)layer * T * f.d, f.W + (size_t)layer * N * f.d, t0, 0, T,
                  N, f.d, w.ks * krange, nk, wave - Pipe::kConsumers);
  } else {
    Pipe::consume(ring, nk, wave / kWE, wave % kWE, acc);
  }
  __syncthreads();  // the ring is free

  // ---- exchange: own tokens to LDS, the partner's to the exchange buffer ----
  const int sub0 = w.ks * kSub;  // first own token within the tile
  int* hist = reinterpret_cast<int*>(lds + kOffHist);
  for (int e = threadIdx.x; e < kMaxBuckets; e += kFThreads) hist[e] = 0;
  if (wave < Pipe::kConsumers) {
    const int wt = wave / kWE, we = wave % kWE;
    if (wt * (kBT / kWT) == sub0) {
      u32x4* hrow = reinterpret_cast<u32x4*>(lds + kOffH);
#pragma unroll
      for (int i = 0; i < Pipe::ME; ++i) {
        const int c4 = Pipe::acc_expert(we, i) / 4;
#pragma unroll
        for (int j = 0; j < Pipe::MT; ++j) {
          const int r = Pipe::acc_token(wt, j) - sub0;
          hrow[r * (kHRowBytes / 16) + h_chunk(r, c4)] = __builtin_bit_cast(u32x4, acc[i][j]);
        }
      }
    } else {
      Pipe::store(acc, f.part + ((size_t)w.ks * f.L + layer) * T * N, t0, 0, T, N, wt, we);
    }
  }
  const int tile = layer * f.n_tt + w.tt;
  stores_done_barrier();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(&f.sync[tile], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    wait_at_least(&f.sync[tile], kSplit, f.spin_ticks);
  }
  __syncthreads();

  // ---- routing of the own 64 tokens (two passes of 32 rows) ------------------
  const ScoreArgs& a = f.sa;
  const int rl = lane & 15;
  const int prow = threadIdx.x >> 4;  // row within a pass
  const float* other = f.part + ((size_t)(1 - w.ks) * f.L + layer) * T * N;
  float4 pv[kPasses][kEPL / 4];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int t = t0 + sub0 + p * kPassRows + prow;
    const float4* src = reinterpret_cast<const float4*>(other + (size_t)min(t, T - 1) * N) + rl * 4;
#pragma unroll
    for (int q = 0; q < kEPL / 4; ++q)
      pv[p][q] = rl * kEPL < N ? src[q] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  LaneConsts<kEPL> lc;
  load_lane_consts<kEPL>(a, layer, true, lc);
  Cand* cand = reinterpret_cast<Cand*>(lds + kOffCand);
  int* slot_id = reinterpret_cast<int*>(lds + kOffSlotId);
  float* slot_s = reinterpret_cast<float*>(lds + kOffSlotS);
  const RowLds rs{cand + prow * kCandStride, slot_id + prow * kMaxSlots, slot_s + prow * kMaxSlots};
  const u32x4* hrow = reinterpret_cast<const u32x4*>(lds + kOffH);
  float cs[kEPL];
#pragma unroll
  for (int j = 0; j < kEPL; ++j) cs[j] = 0.f;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int r = p * kPassRows + prow;
    const int t = t0 + sub0 + r;
    const bool live = t < T;
    float v[kEPL];
#pragma unroll
    for (int q = 0; q < kEPL / 4; ++q) {
      const floatx4 own = __builtin_bit_cast(floatx4, hrow[r * (kHRowBytes / 16) + h_chunk(r, rl * 4 + q)]);
      v[4 * q + 0] = own[0] + pv[p][q].x;
      v[4 * q + 1] = own[1] + pv[p][q].y;
      v[4 * q + 2] = own[2] + pv[p][q].z;
      v[4 * q + 3] = own[3] + pv[p][q].w;
    }
    float qv[kEPL];
    route_row<kEPL, GROUPED, MODE, LPG>(a, layer, t, live, v, lc, rs, hist, qv);
    if (a.colpart != nullptr) {
      // the wavefront's column sums of q over its 4 rows, as in the
      // separate selection kernel, accumulated over the passes in order
#pragma unroll
      for (int j = 0; j < kEPL; ++j) {
        const auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(qv[j]),
                                                         __float_as_uint(qv[j]), false, false);
        const float pair = __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
        const auto h2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair),
                                                         __float_as_uint(pair), false, false);
        cs[j] += __uint_as_float(h2[0]) + __uint_as_float(h2[1]);
      }
    }
  }
  float* colw = reinterpret_cast<float*>(lds + kOffColw);
  if (a.colpart != nullptr && lane < kRowLanes) {
#pragma unroll
    for (int j = 0; j < kEPL; ++j) colw[wave * kMaxExperts + rl * kEPL + j] = cs[j];
  }
  __syncthreads();

  // ---- block histogram, segment totals, column sums --------------------------
  const int Nb = N + a.n_shared;
  const int blk = (t0 + sub0) / kRowTokens;  // this workgroup's histogram / layout block
  const int nsb = (T + kRowTokens - 1) / kRowTokens;
  if (blk < nsb) {
    uint16_t* out = a.cnt + (size_t)layer * Nb * nsb + blk;
    const int nseg = (nsb + kSegBlocks - 1) / kSegBlocks;
    int32_t* seg = a.segsum + ((size_t)layer * nseg + blk / kSegBlocks) * Nb;
    for (int e = threadIdx.x; e < Nb; e += kFThreads) {
      out[(size_t)e * nsb] = (uint16_t)hist[e];
      if (hist[e] != 0) atomicAdd(&seg[e], hist[e]);
    }
    if (a.colpart != nullptr) {
      for (int e = threadIdx.x; e < N; e += kFThreads) {
        float s = colw[e];
#pragma unroll
        for (int ww = 1; ww < kFWaves; ++ww) s += colw[ww * kMaxExperts + e];
        a.colpart[((size_t)layer * nsb + blk) * N + e] = s;
      }
    }
  }
  if (!f.layout) return;

  // ---- grid barrier: every histogram, total and column sum is published -----
  int32_t* grid_ctr = f.sync + (size_t)f.L * f.n_tt + f.L;
  stores_done_barrier();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(grid_ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    wait_at_least(grid_ctr, f.n_work, f.spin_ticks);
  }
  __syncthreads();

  // ---- layout block --------------------------------------------------------
  const LayoutArgs& la = f.la;
  ScatterLds& sl = *reinterpret_cast<ScatterLds*>(lds + kOffScatter);
  if (blk < la.nlb) scatter_block<kFThreads>(la, layer, blk, sl);

  // ---- batch-mean entropy: column e of the layer summed by its e-th block ---
  const int n_blk = kSplit * f.n_tt;  // workgroups (= blocks) of the layer
  const int lw = blk;                 // this workgroup's index within its layer
  if (la.agg_entropy != nullptr && lw < N) {
    float* red = reinterpret_cast<float*>(lds + kOffRed);
    const float invT = T > 0 ? 1.f / (float)T : 0.f;
    for (int e = lw; e < N; e += n_blk) {
      // block order within each thread, threads in a fixed tree
      float s = 0.f;
      for (int b = threadIdx.x; b < nsb; b += kFThreads) s += la.colpart[((size_t)layer * nsb + b) * N + e];
      red[threadIdx.x] = s;
      __syncthreads();
      for (int o = kFThreads / 2; o > 0; o >>= 1) {
        if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
      }
      if (threadIdx.x == 0) f.colmean[(size_t)layer * N + e] = red[0] * invT;
      __syncthreads();
    }
    const int n_part = min(N, n_blk);
    int32_t* ticket = f.sync + (size_t)f.L * f.n_tt + layer;
    __shared__ int last;
    stores_done_barrier();
    if (threadIdx.x == 0) {
      last = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
             n_part - 1;
    }
    __syncthreads();
    if (last) {
      // the last column in: entropy (bits) of the normalised batch mean
      const float m = threadIdx.x < N ? f.colmean[(size_t)layer * N + threadIdx.x] : 0.f;
      red[threadIdx.x] = m;
      __syncthreads();
      for (int o = kFThreads / 2; o > 0; o >>= 1) {
        if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
      }
      const float Z = red[0];
      __syncthreads();
      const float q = Z > 0.f ? m / Z : 0.f;
      red[threadIdx.x] = q > 0.f ? -q * log2f(q) : 0.f;
      __syncthreads();
      for (int o = kFThreads / 2; o > 0; o >>= 1) {
        if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
      }
      if (threadIdx.x == 0) la.agg_entropy[layer] = T > 0 ? red[0] : 0.f;
    }
  }

  // ---- load statistics and bias update: the layer's last block ---------------
  if (lw == n_blk - 1 && (la.stats != nullptr || la.bias_inout != nullptr)) {
    __syncthreads();
    load_totals<kFThreads>(la, layer, -1, sl.total, sl.pre);
    __syncthreads();
    BalanceScratch& bal = *reinterpret_cast<BalanceScratch*>(lds + kOffBal);
    block_load_balance(sl.total, N, la.stats != nullptr ? la.stats + layer : nullptr,
                       la.bias_inout != nullptr ? la.bias_inout + (size_t)layer * N : nullptr,
                       la.bias_step, bal);
  }
}

constexpr int kVariants = 6;
const void* variant_fn(int v) {
  switch (v) {
    case 0: return reinterpret_cast<const void*>(&route_fused_kernel<false, kSigmoid, 0>);
    case 1: return reinterpret_cast<const void*>(&route_fused_kernel<true, kSigmoid, 2>);
    case 2: return reinterpret_cast<const void*>(&route_fused_kernel<true, kSigmoid, 0>);
    case 3: return reinterpret_cast<const void*>(&route_fused_kernel<false, kSoftmax, 0>);
    case 4: return reinterpret_cast<const void*>(&route_fused_kernel<true, kSoftmax, 2>);
    default: return reinterpret_cast<const void*>(&route_fused_kernel<true, kSoftmax, 0>);
  }
}

// Which kernel variant routes a shape: the score function, and for groups
// whether a group is two row lanes (the DeepSeek-V3 geometry, fixed at
// compile time) or any other width.
int pick_variant(int score_fn, int N, int G) {
  const int base = score_fn == 1 ? 0 : 3;
  if (G <= 1) return base;
  return base + (N / G == 2 * kEPL ? 1 : 2);
}

// Workgroups of a variant that fit on the current device at once (computed
// once per device and variant; 0 when the runtime cannot say).
int resident_capacity(int v) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices][kVariants];  // capacity + 1; 0 = not known yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int got = cache[dev][v].load(std::memory_order_relaxed);
  if (got > 0) return got - 1;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, variant_fn(v), kFThreads, 0) !=
          hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  got = per_cu * cus;
  cache[dev][v].store(got + 1, std::memory_order_relaxed);
  return got;
}

}  // namespace

bool route_fused_eligible(int L, int T, int d, int N, int G) {
  // N a multiple of 16: a row lane's experts are all present or all absent
  if (T <= 0 || N <= kMaxExperts / 2 || N > kMaxExperts || N % kEPL != 0) return false;
  if (d % (kKStage * kSplit) != 0) return false;
  if (route_rows_epl(N) != kEPL || !route_rows_supports(N, G)) return false;
  const long long n_work = (long long)L * ((T + kBT - 1) / kBT) * kSplit;
  if (n_work > (1 << 20)) return false;
  // both score functions' variants must fit the whole grid at once
  const int cap = min(resident_capacity(pick_variant(1, N, G)), resident_capacity(pick_variant(0, N, G)));
  return n_work <= (long long)cap;
}

int route_fused_sync_ints(int L, int T) { return L * ((T + kBT - 1) / kBT) + L + 1; }

hipError_t launch_route_fused(const void* x, const void* w, float* part, int32_t* sync,
                              float* colmean, const ScoreArgs& sa, const LayoutArgs& la, int L,
                              int T, int d, int N, bool layout, hipStream_t s) {
  FusedArgs f{};
  f.x = static_cast<const uint16_t*>(x);
  f.W = static_cast<const uint16_t*>(w);
  f.part = part;
  f.sync = sync;
  f.colmean = colmean;
  f.sa = sa;
  f.la = la;
  f.L = L;
  f.T = T;
  f.d = d;
  f.N = N;
  f.n_tt = (T + kBT - 1) / kBT;
  f.n_work = L * f.n_tt * kSplit;
  f.per_xcd = (f.n_work + 7) / 8;
  f.layout = layout ? 1 : 0;
  f.spin_ticks = 20000000LL;  // 0.2 s at 100 MHz
  void* args[] = {&f};
  return hipLaunchKernel(variant_fn(pick_variant(sa.score_fn, N, sa.G)), dim3(8 * f.per_xcd),
                         dim3(kFThreads), args, 0, s);
}

}  // namespace moer
