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
// as the A operand (16 expert rows, zero past N) and x rows as B, every load
// of a part in flight before its first MFMA (up to two steps at a time). A
// step is 256 bytes of each row. Its loads cover whole 128-byte lines, four
// rows of 256 bytes per instruction, into registers; the wavefront then
// passes them through its own LDS tile to the MFMA fragment layout (one row
// per lane, 64 bytes of it per instruction). Loaded in that layout directly,
// each instruction would touch sixteen half lines, and a CU's loads would
// take about twice as long. The tiles take 128 KB of LDS, so a CU holds one
// workgroup at a time. The 16 parts are added in part order through LDS.
//  - bf16: a step is 128 deep, four v_mfma_f32_16x16x32_bf16 (bf16 products
//    are exact in fp32 and accumulate in fp32);
//  - fp32: a step is 64 deep, sixteen v_mfma_f32_16x16x4f32.
// The lane's 8-element (bf16) or 4-element (fp32) group g of fragment i
// (16-byte chunk 4i + g of its row) feeds the MFMA k-slot g of MFMA i
// (bf16), or component c of it the k-slot g of MFMA (i, c) (fp32): A and B
// take the same depth for every k-slot, so each step's MFMAs together sum
// its depth range once.
//
// The selection is the same as in the standalone kernel; only its workgroup
// holds 16 tokens (so a launch of T / 16 workgroups fills the chip for the
// few-thousand-token batches these routers see). Its histogram blocks are
// therefore 16 tokens and carry no running segment totals: the layout kernel
// sums the block counts itself, so no counter needs clearing first.
//
// A layer of at most kWholeTokens tokens takes one workgroup for the whole
// call (route_layer_kernel): it routes all its tokens at once, and with the
// whole layer's histogram in its own LDS it then does the layout kernel's
// work as well (counts, offsets, the stable permutation and its inverse, the
// entropy of the batch mean of q, the load statistics and the bias update),
// so the call is one launch.
#include <hip/hip_ext.h>
#include <math.h>

#include "load_balance.hpp"
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

// One step's whole-line loads: load i is row 4i + lane/16, chunk lane%16 of
// the step's 256 bytes, at a base the whole wavefront shares (the step's
// first byte in the block's first row) plus the lane's 32-bit offset ox[i] /
// ow[i]. W_g takes the first NW loads (NW * 4 >= N rows). Rows past the
// last (x rows past rows_x, W_g rows past N within those loads) read the
// last row again, so no branch surrounds a load and nothing uses a loaded
// value before the tile write: the loads stay in flight together, and the
// waits before the tile writes count them exactly. The tile reads zero the
// W_g rows past N.
struct StepLines {  // named fields, so the values stay in registers
  uint4 x0, x1, x2, x3, w0, w1, w2, w3;
};
template <int NW>
__device__ __forceinline__ StepLines load_lines(const char* xs, const char* ws,
                                                const uint32_t (&ox)[4],
                                                const uint32_t (&ow)[4]) {
  const auto ld = [](const char* p) { return *reinterpret_cast<const uint4*>(p); };
  StepLines L{};
  L.x0 = ld(xs + ox[0]);
  L.x1 = ld(xs + ox[1]);
  L.x2 = ld(xs + ox[2]);
  L.x3 = ld(xs + ox[3]);
  L.w0 = ld(ws + ow[0]);
  if constexpr (NW > 1) L.w1 = ld(ws + ow[1]);
  if constexpr (NW > 2) L.w2 = ld(ws + ow[2]);
  if constexpr (NW > 3) L.w3 = ld(ws + ow[3]);
  return L;
}

// The wavefront's LDS tile for one step: 16 rows x 16 chunks of 16 bytes, x
// rows (tokens) then W_g rows (experts). Chunk c of row r sits at chunk
// c ^ r of the row, so the whole-line writes (16 lanes: one row, every
// chunk) and the fragment reads (16 lanes: every row, one chunk) both fall
// on distinct banks.
constexpr int kTileChunks = 16 * 16;
struct StepTile {
  uint4 x[kTileChunks];
  uint4 w[kTileChunks];
};

// One step through the tile: the lane's whole-line chunks (load i: row
// 4i + lane/16, chunk lane%16) are written to the tile, and the fragments
// read back are exactly those load_step would have loaded (MFMA i, k-slot g:
// chunk 4i + g of row lane%16), so the MFMAs and h are the same bit for bit.
// W_g rows past N are read as zero (the tile holds a repeat of row N - 1
// there, or nothing). Rows of the tile are private to the
// wavefront, and its LDS operations complete in order: no barrier.
template <bool BF16, int NW>
__device__ __forceinline__ void staged_mfma_step(const StepLines L, int N, StepTile& tile,
                                                 sm_floatx4& acc) {
  const int lane = threadIdx.x & 63;
  const int a = lane >> 4, kc = lane & 15;  // as loaded: row 4i + a, chunk kc
  const int r = lane & 15, g = lane >> 4;   // as used: row r, k-slot g
  const uint4 xl[4] = {L.x0, L.x1, L.x2, L.x3}, wl[4] = {L.w0, L.w1, L.w2, L.w3};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * i + a;
    tile.x[row * 16 + (kc ^ row)] = xl[i];
    if (i < NW) tile.w[row * 16 + (kc ^ row)] = wl[i];  // later loads hold no row below N
  }
  uint4 xv[4], wv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = (4 * i + g) ^ r;
    xv[i] = tile.x[r * 16 + c];
    wv[i] = r < N ? tile.w[r * 16 + c] : uint4{0u, 0u, 0u, 0u};
  }
  // (the next step's tile writes stay after these reads: the compiler cannot
  // tell the lane-dependent addresses apart, and the LDS keeps the order)
  mfma_step<BF16>(xv, wv, acc);
}

// part_affinities with whole-line loads staged through the wavefront's LDS
// tile. xblk: the first of the block's rows_x token rows (later rows read
// the last one; their results are never stored); wblk: W_g's N rows; rowb:
// bytes per row. NW: W_g load instructions per step (4 * NW >= N); ALL_TWO:
// every pass of every wavefront has two steps (the step count a multiple of
// 2 * kWaves), so the second step's loads need no condition either.
template <bool BF16, int NW, bool ALL_TWO>
__device__ __forceinline__ sm_floatx4 part_affinities_staged(const char* xblk, int rows_x,
                                                             const char* wblk, int N,
                                                             size_t rowb, int d, int w,
                                                             StepTile& tile) {
  const int nsteps = d / StepOf<BF16>::kDepth;
  const int lane = threadIdx.x & 63;
  uint32_t ox[4], ow[4];  // 16 rows of at most 2^27 bytes (checked by the host)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * i + (lane >> 4);
    ox[i] = (uint32_t)(min(row, rows_x - 1) * rowb) + (uint32_t)(lane & 15) * 16u;
    ow[i] = (uint32_t)(min(row, N - 1) * rowb) + (uint32_t)(lane & 15) * 16u;
  }
  sm_floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = w; s < nsteps; s += 2 * kWaves) {
    const bool two = ALL_TWO || s + kWaves < nsteps;  // the same for the whole wavefront
    const size_t s1 = (size_t)s * 256, s2 = (size_t)(s + kWaves) * 256;
    const StepLines l0 = load_lines<NW>(xblk + s1, wblk + s1, ox, ow);
    const StepLines l1 = two ? load_lines<NW>(xblk + s2, wblk + s2, ox, ow) : StepLines{};
    __builtin_amdgcn_sched_barrier(0);  // both steps' loads before any tile work
    staged_mfma_step<BF16, NW>(l0, N, tile, acc);
    if (two) staged_mfma_step<BF16, NW>(l1, N, tile, acc);
  }
  return acc;
}

// The wavefront's 16x16 block over depth part w (steps w, w + 16, ...): lane
// l holds experts 4*(l/16) .. +3 of token l%16. Operands loaded straight in
// the fragment layout (the one-workgroup layer kernel, whose parts are at
// most one step).
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
  // each wavefront's step tile; afterwards its part of h (16 x 16 fp32)
  __shared__ StepTile tiles[kWaves];
  static_assert(sizeof(StepTile) >= kTok * kSmallMaxN * sizeof(float), "part fits the tile");

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
    const size_t esz = BF16 ? 2 : 4;
    const char* xblk = static_cast<const char*>(x) + ((size_t)layer * T + t0) * d * esz;
    const char* wblk = static_cast<const char*>(W) + (size_t)layer * N * d * esz;
    // the part index as a wavefront-uniform value, so each step's base is too
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const int rows = min(kTok, T - t0);
    const size_t rowb = (size_t)d * esz;
    const bool all_two = (d / StepOf<BF16>::kDepth) % (2 * kWaves) == 0;
    sm_floatx4 acc;
#define MOER_PARTS(NW)                                                                          \
    acc = all_two ? part_affinities_staged<BF16, NW, true>(xblk, rows, wblk, N, rowb, d, wu,    \
                                                           tiles[wu])                           \
                  : part_affinities_staged<BF16, NW, false>(xblk, rows, wblk, N, rowb, d, wu,   \
                                                            tiles[wu]);
    if (N <= 4) {
      MOER_PARTS(1)
    } else if (N <= 8) {
      MOER_PARTS(2)
    } else {
      MOER_PARTS(4)
    }
#undef MOER_PARTS
    const int g = (threadIdx.x & 63) >> 4;
    // the part goes where this wavefront's tile was (its own reads are done)
    float(*part)[kSmallMaxN] = reinterpret_cast<float(*)[kSmallMaxN]>(&tiles[wave]);
    *reinterpret_cast<sm_floatx4*>(&part[r][4 * g]) = acc;
  }
  __syncthreads();  // every part stored; the histogram cleared

  float q[1] = {0.f};
  if (row < kTok) {  // wavefronts 0-3: one row per token
    float v[1] = {0.f};
#pragma unroll
    for (int p = 0; p < kWaves; ++p)
      v[0] += reinterpret_cast<const float(*)[kSmallMaxN]>(&tiles[p])[row][r];
    const int t = t0 + row;
    const RowLds rs{cand[row], slot_id[row], slot_s[row]};
    route_row<1, GROUPED, MODE>(a, layer, t, t < T, v, lc, rs, hist, q);
  }
  block_outputs<1, kThreads>(a, layer, N, Nb, q, hist, colw);
}

constexpr int kMaxBucketsSmall = 2 * kSmallMaxN;  // N <= 16 plus at most 15 shared slots
constexpr int kWholeChunks = kWholeTokens * kMaxSlots / 64;  // 64-slot chunks of a layer

// The layout of a layer routed by one workgroup (route_layer_kernel), from
// its LDS histogram and chosen slots (hist, slot_id: complete after the
// caller's barrier); qsum: this thread's q. The same outputs as the layout
// kernel (layout.hip, layout_block.hpp, load_balance.hpp), computed the same
// way:
//  - counts = the histogram; offsets = its exclusive prefix;
//  - perm / inv_perm: the stable order by (expert, token, slot), slot i of
//    the layer at offset[e] + the earlier slots of expert e, counted with
//    per-64-slot membership bitmaps (popcounts of the lower bits);
//  - the entropy of the batch mean of q: column sums of q per wavefront
//    (wave_column_sums), the wavefronts added in order, then the entropy in
//    one wavefront with xor butterflies;
//  - load statistics and the sign-step bias update (block_load_balance, in
//    one wavefront).
template <int RL>
__device__ void whole_layer_layout(const ScoreArgs& a, const LayoutArgs& la, int layer,
                                   float qsum, const int* hist,
                                   const int (*slot_id)[kMaxSlots]) {
  __shared__ unsigned long long bits[kWholeChunks][kMaxBucketsSmall];
  __shared__ int pos0[kWholeChunks][kMaxBucketsSmall];  // first position of chunk c's slots of e
  __shared__ int off[kMaxBucketsSmall + 1];
  __shared__ float colw[kWaves][kSmallMaxN];
  __shared__ BalanceScratch bal;
  const int N = a.N, T = a.T, Nb = la.Nb, Kt = la.Kt;
  const int M = T * Kt;  // <= kThreads
  const int i = threadIdx.x;
  const int lane = i & 63;
  const size_t lbase = (size_t)layer * M;

  for (int k = i; k < kWholeChunks * kMaxBucketsSmall; k += kThreads)
    (&bits[0][0])[k] = 0ull;
  // the wavefront's column sums of q over its 64 / RL rows (lane = expert)
  {
    const float qv[1] = {qsum};
    float cs[1];
    wave_column_sums<1, RL>(qv, cs);
    if (lane < RL) colw[i >> 6][lane] = cs[0];
  }
  if (i == 0) {  // offsets: exclusive prefix of the counts
    int run = 0;
    for (int e = 0; e < Nb; ++e) {
      off[e] = run;
      run += hist[e];
    }
    off[Nb] = run;
  }
  // slot i of the layer (token i / Kt, slot i % Kt): the id route_row wrote
  int e_i = -1;
  if (i < M) {
    const int t = i / Kt, k = i - t * Kt;
    e_i = k < a.K ? min(max(slot_id[t][k], 0), N - 1) : N + (k - a.K);
  }
  __syncthreads();
  if (e_i >= 0) atomicOr(&bits[i >> 6][e_i], 1ull << (i & 63));
  if (i < Nb) {
    la.counts[(size_t)layer * Nb + i] = hist[i];
    la.offsets[(size_t)layer * (Nb + 1) + i] = off[i];
  }
  if (i == 0) la.offsets[(size_t)layer * (Nb + 1) + Nb] = off[Nb];
  __syncthreads();
  const int nchunk = (M + 63) / 64;
  if (i < Nb) {
    int run = off[i];
    for (int c = 0; c < nchunk; ++c) {
      pos0[c][i] = run;
      run += __popcll(bits[c][i]);
    }
  }
  __syncthreads();
  if (e_i >= 0) {
    const int c = i >> 6;
    const int pos = pos0[c][e_i] + __popcll(bits[c][e_i] & ((1ull << (i & 63)) - 1ull));
    la.perm[lbase + pos] = i;
    if (la.inv_perm != nullptr) la.inv_perm[lbase + i] = pos;
  }
  // after the last barrier, beside the scatter: the batch-mean entropy in the
  // last wavefront, the load statistics and bias update in the one before
  // (one wave each, no barrier; at most 16 experts, lane = expert)
  const int wave = i >> 6;
  if (la.agg_entropy != nullptr && wave == kWaves - 1) {
    float tot = 0.f;
    if (lane < N) {
      tot = colw[0][lane];
      for (int w = 1; w < kWaves; ++w) tot += colw[w][lane];
    }
    const float me = lane < N ? tot * (T > 0 ? 1.f / (float)T : 0.f) : 0.f;
    auto add = [](float x, float y) { return x + y; };
    const float Z = wave_allreduce(me, add);
    const float qm = Z > 0.f ? me / Z : 0.f;
    const float H = wave_allreduce(qm > 0.f ? -qm * log2f(qm) : 0.f, add);
    if (lane == 0) la.agg_entropy[layer] = T > 0 ? H : 0.f;
  }
  if ((la.stats != nullptr || la.bias_inout != nullptr) && wave == kWaves - 2)
    block_load_balance<1>(hist, N, la.stats != nullptr ? la.stats + layer : nullptr,
                          la.bias_inout != nullptr ? la.bias_inout + (size_t)layer * N : nullptr,
                          la.bias_step, bal);
}

// One workgroup per layer of at most kWholeTokens tokens (kWholeTokensWide
// for more than 8 experts) and a short depth (at most kWholeSteps steps, so
// each depth part is at most one step). Wavefront w forms depth parts w / 4,
// w / 4 + 4, ... of token block w % 4: each (block, part) with the same
// steps, in the same order, as the 16-token kernel, and the parts are added
// in the same order, so every h is bit for bit the one the 16-token kernel
// forms; the blocks' loads go out together. Every token is then routed at
// once, in rows of RL lanes, the fewest that hold the router's N experts (4,
// 8 or 16): T * RL / 64 of the workgroup's wavefronts route. Then the
// workgroup does the layout. Measured against 16-token workgroups on several
// CUs plus the layout launch: ahead up to 64 tokens in 4- and 8-lane rows,
// up to 32 in 16-lane rows.
template <bool BF16, bool GROUPED, int MODE, int RL>
__global__ __launch_bounds__(kThreads) void route_layer_kernel(ScoreArgs a, const void* x,
                                                               const void* W, int d,
                                                               LayoutArgs la) {
  __shared__ Cand cand[kWholeTokens][kCandStride];
  __shared__ int slot_id[kWholeTokens][kMaxSlots];
  __shared__ float slot_s[kWholeTokens][kMaxSlots];
  __shared__ int hist[kMaxBuckets];
  __shared__ __attribute__((aligned(16))) float part_h[kWaves][kWholeTokens][kSmallMaxN];
  static_assert(kThreads / RL >= kWholeTokens, "one row per token of the layer");

  const int N = a.N, T = a.T;
  const int Nb = N + a.n_shared;
  const int layer = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int r = threadIdx.x & 15;     // token row of the MFMA block
  const int row = threadIdx.x / RL;   // routing row = token
  const int rl = threadIdx.x & (RL - 1);  // row lane = expert
  const int ntb = (T + kTok - 1) / kTok;

  for (int i = threadIdx.x; i < Nb; i += kThreads) hist[i] = 0;
  LaneConsts<1> lc;
  load_lane_consts<1, AnyShape, RL>(a, layer, true, lc);
  {
    const size_t esz = BF16 ? 2 : 4;
    const uint4* wrow = r < N ? reinterpret_cast<const uint4*>(static_cast<const char*>(W) +
                                                               ((size_t)layer * N + r) * d * esz)
                              : nullptr;
    const int g = (threadIdx.x & 63) >> 4;
    const int tb = wave & 3;
    if (tb < ntb) {  // ntb <= kWholeTokens / 16 <= 4
      // tokens past T read row T - 1 (their results are never stored)
      const int tt = min(tb * kTok + r, T - 1);
      const uint4* xrow = reinterpret_cast<const uint4*>(static_cast<const char*>(x) +
                                                         ((size_t)layer * T + tt) * d * esz);
#pragma unroll
      for (int p = wave >> 2; p < kWaves; p += 4) {
        const sm_floatx4 acc = part_affinities<BF16>(xrow, wrow, d, p);
        *reinterpret_cast<sm_floatx4*>(&part_h[p][tb * kTok + r][4 * g]) = acc;
      }
    }
  }
  __syncthreads();  // every part stored; the histogram cleared

  float q[1] = {0.f};
  if (row < ntb * kTok) {  // the wavefronts of the token blocks (rows past T route, unused)
    float v[1] = {0.f};
#pragma unroll
    for (int p = 0; p < kWaves; ++p) v[0] += part_h[p][row][rl];
    const RowLds rs{cand[row], slot_id[row], slot_s[row]};
    route_row<1, GROUPED, MODE, 0, AnyShape, RL>(a, layer, row, row < T, v, lc, rs, hist, q);
  }
  __syncthreads();  // every row routed: histogram and slots complete
  whole_layer_layout<RL>(a, la, layer, q[0], hist, slot_id);
}

template <bool BF16, bool GROUPED, int RL>
auto pick_layer_rl(const ScoreArgs& a) {
  return a.score_fn == 1 ? route_layer_kernel<BF16, GROUPED, kSigmoid, RL>
                         : route_layer_kernel<BF16, GROUPED, kSoftmax, RL>;
}
template <bool BF16, bool GROUPED>
auto pick_layer(const ScoreArgs& a) {
  return a.N <= 4 ? pick_layer_rl<BF16, GROUPED, 4>(a)
                  : (a.N <= 8 ? pick_layer_rl<BF16, GROUPED, 8>(a)
                              : pick_layer_rl<BF16, GROUPED, 16>(a));
}

template <bool BF16, bool GROUPED>
auto pick(const ScoreArgs& a) {
  return a.score_fn == 1 ? route_small_kernel<BF16, GROUPED, kSigmoid>
                         : route_small_kernel<BF16, GROUPED, kSoftmax>;
}

}  // namespace

bool route_layer_eligible(bool bf16, int T, int d, int N) {
  return T >= 1 && T <= (N <= 8 ? kWholeTokens : kWholeTokensWide) && N <= kSmallMaxN &&
         d <= kWholeSteps * (bf16 ? StepOf<true>::kDepth : StepOf<false>::kDepth);
}

bool route_small_eligible(bool bf16, int T, int d, int N, int G, bool aligned) {
  if (T < 1 || T > kSmallMaxBlocks * kTok || N > kSmallMaxN || !route_rows_supports(N, G) ||
      d < 1 || !aligned)
    return false;
  // the staged loads address a block's 16 rows with 32-bit offsets
  if ((long long)kTok * d * (bf16 ? 2 : 4) > (1LL << 31)) return false;
  return d % (bf16 ? StepOf<true>::kDepth : StepOf<false>::kDepth) == 0;
}

hipError_t launch_route_small(const ScoreArgs& a, const void* x, const void* W, int d, bool bf16,
                              int L, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1,
                              const LayoutArgs* whole) {
  if (whole != nullptr) {
    if (!route_layer_eligible(bf16, a.T, d, a.N) || whole->Nb > kMaxBucketsSmall ||
        a.T * whole->Kt > kWholeTokens * kMaxSlots)
      return hipErrorInvalidValue;
    auto k = bf16 ? (a.G > 1 ? pick_layer<true, true>(a) : pick_layer<true, false>(a))
                  : (a.G > 1 ? pick_layer<false, true>(a) : pick_layer<false, false>(a));
    hipExtLaunchKernelGGL(k, dim3(1, L), dim3(kThreads), 0, s, ev0, ev1, 0, a, x, W, d, *whole);
    return hipGetLastError();
  }
  const dim3 grid((a.T + kTok - 1) / kTok, L);
  auto k = bf16 ? (a.G > 1 ? pick<true, true>(a) : pick<true, false>(a))
                : (a.G > 1 ? pick<false, true>(a) : pick<false, false>(a));
  hipExtLaunchKernelGGL(k, grid, dim3(kThreads), 0, s, ev0, ev1, 0, a, x, W, d);
  return hipGetLastError();
}

}  // namespace moer
