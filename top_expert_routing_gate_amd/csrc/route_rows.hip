// Scoring, bias-aware group-limited top-k, combine weights, routing entropy
// and the per-block expert histogram, with one 16-lane DPP row per token.
//
// The method, per token (pages cited by title and section):
//  1. scores: sigmoid s = 1/(1+exp(-h)) ("DeepSeek V4 MoE load balancing",
//     token routing: sigmoid gating) or softmax p = exp(h)/sum exp(h)
//     ("MoE Routing Entropy vs Expert Saturation", Mathematics); the given
//     scores in SCORES mode. h = sum of the GEMM's depth-range partials (in
//     range order) + the optional logit offset.
//  2. key = s + b in fp32 (auxiliary-loss-free balancing: the bias steers the
//     decision only); -0 is made +0.
//  3. G > 1 ("DeepSeek-V3 Group-Limited Expert Routing", s.1 and s.3): group
//     score = fp32 sum of the group's two largest keys; the Gk best groups
//     (score desc, group id asc) stay eligible.
//  4. the K best eligible keys (key desc, expert id asc) fill slots 0..K-1
//     in that order; shared experts (same page, s.4) take slots K..Kt-1 with
//     weight 1.
//  5. weights: chosen unbiased scores over their sum (the top-k
//     renormalisation of the dailyaiworld listing).
//  6. entropy in bits of q = s / sum s (Mathematics section); column sums of
//     q per workgroup feed the batch-mean entropy.
//
// Layout on the GPU: a wavefront is 4 rows of 16 lanes; row r handles one
// token and lane j of the row holds experts [j*EPL, (j+1)*EPL). Every
// cross-lane step stays inside the row and is a DPP operation (quad
// permutes, half-row and row mirrors, row shifts and rotations), so no
// shuffle goes through the LDS crossbar.
//
// Exact top-K without K argmax rounds:
//  - lo = the K-th largest of the row's per-lane top-2 eligible keys; these
//    are keys of distinct eligible experts, so lo is at most the K-th largest
//    eligible key: every chosen expert has key >= lo.
//  - the eligible keys >= lo (typically K to K+4 of 256) are compacted into
//    LDS as packed 64-bit words (orderable key bits, then inverted id), at
//    positions from a row prefix scan of per-lane counts;
//  - a candidate's slot is the number of candidates whose packed word is
//    larger, i.e. that beat it under (key desc, id asc); slots < K are kept.
// The result does not depend on the order candidates were written in.
#include <math.h>

#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

#include "moer_internal.hpp"

namespace moer {
namespace {

constexpr int kRowLanes = 16;
constexpr int kThreads = kRowTokens * kRowLanes;  // 1024: one row per token

// ---- DPP helpers (row = 16 lanes) -------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                            0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
// row shift right by n with zero fill (bound_ctrl)
template <int N_>
__device__ __forceinline__ int shr_zero(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0x110 + N_, 0xF, 0xF, true);
}

constexpr int kXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kMirror = 0x140;     // lane i <-> 15-i within 16

// All 16 lanes of a row receive max / min / sum of the row (bitwise equal in
// every lane: each step combines a lane with a partner that combines the same
// two operands).
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp_f<kXor1>(v));
  v = fmaxf(v, dpp_f<kXor2>(v));
  v = fmaxf(v, dpp_f<kHalfMirror>(v));
  return fmaxf(v, dpp_f<kMirror>(v));
}
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_f<kXor1>(v);
  v += dpp_f<kXor2>(v);
  v += dpp_f<kHalfMirror>(v);
  return v + dpp_f<kMirror>(v);
}
__device__ __forceinline__ int row_max_i(int v) {
  v = max(v, dpp_i<kXor1>(v));
  v = max(v, dpp_i<kXor2>(v));
  v = max(v, dpp_i<kHalfMirror>(v));
  return max(v, dpp_i<kMirror>(v));
}
// inclusive prefix sum over the row
__device__ __forceinline__ int row_scan(int v) {
  v += shr_zero<1>(v);
  v += shr_zero<2>(v);
  v += shr_zero<4>(v);
  return v + shr_zero<8>(v);
}

// Orderable encoding: larger word <=> larger key, then smaller expert id.
__device__ __forceinline__ unsigned long long pack_key(float key, int e) {
  const unsigned f = __builtin_bit_cast(unsigned, key);
  const unsigned u = (f & 0x80000000u) ? ~f : (f | 0x80000000u);
  return ((unsigned long long)u << 32) | (unsigned)(0xFFFF - e);
}

template <int EPL>
__device__ __forceinline__ void load_row(const ScoreArgs& a, size_t row_off, size_t split_stride,
                                         int e0, float (&v)[EPL]) {
  // EPL consecutive experts per lane, depth-range partials added in order;
  // 16-byte loads when the lane's range is whole and aligned
#pragma unroll
  for (int j = 0; j < EPL; ++j) v[j] = 0.f;
  if (e0 >= a.N) return;
  if (EPL % 4 == 0 && e0 + EPL <= a.N && (a.N & 3) == 0) {
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
      const int e = min(e0 + j, a.N - 1);
      const float q = (e0 + j < a.N) ? src[e] : 0.f;
      v[j] = sp == 0 ? q : v[j] + q;
    }
  }
}

// Score modes: the scores are given, or sigmoid / softmax of the affinities.
enum { kGiven = 0, kSigmoid = 1, kSoftmax = 2 };

// Hardware transcendentals (v_exp_f32, v_rcp_f32, v_log_f32: about 1 ulp):
// the affinities already carry ~1e-6 GEMM rounding, so the scores only need
// to be accurate well inside the 1e-3 weight and 1e-4 entropy tolerances.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
constexpr float kLog2e = 1.4426950408889634f;

// Score of one affinity (same instructions wherever it is used, so a score
// re-derived later is bitwise the one the selection saw).
template <int MODE>
__device__ __forceinline__ float score_of(float v, float m, float inv_z) {
  if (MODE == kGiven) return v;
  if (MODE == kSigmoid) return rcp_hw(1.f + exp2_hw(-v * kLog2e));
  return exp2_hw((v - m) * kLog2e) * inv_z;
}

template <int EPL, bool GROUPED, int MODE>
__global__ __launch_bounds__(kThreads) void route_rows_kernel(ScoreArgs a) {
  extern __shared__ unsigned long long smem[];
  const int N = a.N, K = a.K, T = a.T;
  const int Kt = K + a.n_shared;
  const int Nb = N + a.n_shared;
  const int layer = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int rl = lane & 15;             // lane within the row
  const int row = threadIdx.x >> 4;     // row within the workgroup = token slot
  const int t = blockIdx.x * kRowTokens + row;
  const bool live = t < T;
  const int e0 = rl * EPL;
  const float NEG_INF = -__builtin_inff();

  // LDS: candidates [rows][N+1] (the pad word staggers rows across banks) |
  // slot ids [rows][16] | histogram [Nb]. The candidate area is reused at the
  // end for the per-wave column sums of q.
  const int cstride = a.N + 1;
  unsigned long long* cand = smem + (size_t)row * cstride;
  int* slot_id = reinterpret_cast<int*>(smem + (size_t)kRowTokens * cstride) + row * kMaxSlots;
  int* hist = reinterpret_cast<int*>(smem + (size_t)kRowTokens * cstride) + kRowTokens * kMaxSlots;
  for (int i = threadIdx.x; i < Nb; i += kThreads) hist[i] = 0;

  // 1. affinities / scores
  const size_t row_off = ((size_t)layer * T + (live ? t : 0)) * N;
  const size_t split_stride = (size_t)gridDim.y * T * N;
  float v[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) v[j] = 0.f;
  if (live) load_row<EPL>(a, row_off, split_stride, e0, v);
  if (rl < kMaxSlots) slot_id[rl] = 0;
  const bool full = e0 + EPL <= N;  // every expert of this lane exists
  if (MODE != kGiven) {
    if (a.offset != nullptr) {
#pragma unroll
      for (int j = 0; j < EPL; ++j) v[j] += a.offset[min(e0 + j, N - 1)];
    }
    if (live && a.h_out != nullptr) {
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (e0 + j < N) a.h_out[row_off + e0 + j] = v[j];
    }
  }
  float m = 0.f, inv_z = 1.f;
  if (MODE == kSoftmax) {
    float lm = NEG_INF;
#pragma unroll
    for (int j = 0; j < EPL; ++j) lm = fmaxf(lm, (full || e0 + j < N) ? v[j] : NEG_INF);
    m = row_max(lm);
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) z += (full || e0 + j < N) ? exp2_hw((v[j] - m) * kLog2e) : 0.f;
    inv_z = rcp_hw(row_sum(z));
  }
  float s[EPL], key[EPL];
  if (full) {
    const float* bias = a.bias != nullptr ? a.bias + (size_t)layer * N + e0 : nullptr;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      s[j] = score_of<MODE>(v[j], m, inv_z);
      key[j] = (s[j] + (bias != nullptr ? bias[j] : 0.f)) + 0.f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = e0 + j;
      const float b = (a.bias != nullptr && e < N) ? a.bias[(size_t)layer * N + e] : 0.f;
      s[j] = e < N ? score_of<MODE>(v[j], m, inv_z) : 0.f;
      key[j] = e < N ? (s[j] + b) + 0.f : NEG_INF;
    }
  }

  // 6. entropy of q = s / sum s, and this token's q for the column sums
  float ssum = 0.f, slog = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    ssum += s[j];
    slog += s[j] > 0.f ? s[j] * log2_hw(s[j]) : 0.f;
  }
  ssum = row_sum(ssum);
  slog = row_sum(slog);
  if (live && rl == 0 && a.tok_entropy != nullptr)
    a.tok_entropy[(size_t)layer * T + t] = ssum > 0.f ? log2f(ssum) - slog / ssum : 0.f;
  const float inv_s = (live && ssum > 0.f) ? 1.f / ssum : 0.f;

  // 3. group-limited eligibility
  bool eligible = true;
  if (GROUPED) {
    const int lpg = (N / a.G) / EPL;       // lanes per group (power of two, <= 16)
    const int g = rl / lpg;
    float m1 = key[0], m2 = NEG_INF;
#pragma unroll
    for (int j = 1; j < EPL; ++j) {
      m2 = fmaxf(m2, fminf(m1, key[j]));
      m1 = fmaxf(m1, key[j]);
    }
    // merge the group's lanes (lanes of a group are aligned, lpg a power of 2)
    auto merge = [&](float b1, float b2) {
      const float n2 = fmaxf(fminf(m1, b1), fmaxf(m2, b2));
      m1 = fmaxf(m1, b1);
      m2 = n2;
    };
    if (lpg >= 2) merge(dpp_f<kXor1>(m1), dpp_f<kXor1>(m2));
    if (lpg >= 4) merge(dpp_f<kXor2>(m1), dpp_f<kXor2>(m2));
    if (lpg >= 8) merge(dpp_f<kHalfMirror>(m1), dpp_f<kHalfMirror>(m2));
    if (lpg >= 16) merge(dpp_f<kMirror>(m1), dpp_f<kMirror>(m2));
    const float gs = (g < a.G) ? m1 + m2 : NEG_INF;
    const int gid = g < a.G ? g : 0x7FFF;
    // rank among the row's groups: rotate (score, id) by whole groups
    int rank = 0;
#define MOER_ROT(n)                                                                  \
    if ((n) % lpg == 0) {                                                            \
      const float og = dpp_f<0x120 + (n)>(gs);                                       \
      const int oid = dpp_i<0x120 + (n)>(gid);                                       \
      rank += (oid < a.G && (og > gs || (og == gs && oid < gid))) ? 1 : 0;           \
    }
    MOER_ROT(1) MOER_ROT(2) MOER_ROT(3) MOER_ROT(4) MOER_ROT(5) MOER_ROT(6) MOER_ROT(7)
    MOER_ROT(8) MOER_ROT(9) MOER_ROT(10) MOER_ROT(11) MOER_ROT(12) MOER_ROT(13) MOER_ROT(14)
    MOER_ROT(15)
#undef MOER_ROT
    eligible = g < a.G && rank < a.Gk;
  }

  // lo: K-th largest of the eligible lanes' two largest keys (keys of up to 32
  // distinct eligible experts, so lo is at most the K-th largest eligible key)
  float l1 = NEG_INF, l2 = NEG_INF;
  if (eligible) {
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      l2 = fmaxf(l2, fminf(l1, key[j]));
      l1 = fmaxf(l1, key[j]);
    }
  }
  int c1 = 1 + (l2 >= l1 ? 1 : 0), c2 = 2;  // values >= l1 / >= l2, own pair included
#define MOER_CGE(n)                                          \
  {                                                          \
    const float o1 = dpp_f<0x120 + (n)>(l1);                 \
    const float o2 = dpp_f<0x120 + (n)>(l2);                 \
    c1 += (o1 >= l1 ? 1 : 0) + (o2 >= l1 ? 1 : 0);           \
    c2 += (o1 >= l2 ? 1 : 0) + (o2 >= l2 ? 1 : 0);           \
  }
  MOER_CGE(1) MOER_CGE(2) MOER_CGE(3) MOER_CGE(4) MOER_CGE(5) MOER_CGE(6) MOER_CGE(7)
  MOER_CGE(8) MOER_CGE(9) MOER_CGE(10) MOER_CGE(11) MOER_CGE(12) MOER_CGE(13) MOER_CGE(14)
  MOER_CGE(15)
#undef MOER_CGE
  const float lo = row_max(fmaxf(c1 >= K ? l1 : NEG_INF, c2 >= K ? l2 : NEG_INF));

  // candidates: eligible keys >= lo, compacted by a row prefix scan
  unsigned bits = 0;
  if (eligible) {
#pragma unroll
    for (int j = 0; j < EPL; ++j) bits |= (key[j] >= lo && key[j] > NEG_INF) ? 1u << j : 0u;
  }
  const int mine = __builtin_popcount(bits);
  const int incl = row_scan(mine);
  const int count = row_max_i(incl);
  int pos = incl - mine;
#pragma unroll
  for (int j = 0; j < EPL; ++j)
    if (bits & (1u << j)) cand[pos++] = pack_key(key[j], e0 + j);
  // A row's candidates, slots and weights are private to its wavefront and a
  // wavefront's LDS operations complete in order: no workgroup barrier here.

  // 4. slot of each candidate = number of candidates that beat it
  for (int c = rl; c < count; c += kRowLanes) {
    const unsigned long long my = cand[c];
    int r = 0;
#pragma unroll 4
    for (int i = 0; i < count; ++i) r += cand[i] > my ? 1 : 0;
    if (r < K) slot_id[r] = 0xFFFF - (int)(my & 0xFFFF);
  }

  // 5. weights over the chosen slots (re-derived scores, same instructions)
  int my_e = 0;
  float my_s = 0.f;
  if (rl < K) {
    my_e = min(max(slot_id[rl], 0), N - 1);  // always in range, even for non-finite input
    if (live) {
      const size_t o = row_off + my_e;
      float hv = a.in[o];
      for (int sp = 1; sp < a.nsplit; ++sp) hv += a.in[sp * split_stride + o];
      if (MODE != kGiven && a.offset != nullptr) hv += a.offset[my_e];
      my_s = score_of<MODE>(hv, m, inv_z);
    }
  }
  const float zsel = row_sum(rl < K ? my_s : 0.f);

  // column sums of q over the wavefront's 4 tokens (rows): rows 0+1 and 2+3,
  // then the two pairs; both lanes of a pair add the same two operands, so
  // every lane ends with the bitwise-same sum
  float colq[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const float q = s[j] * inv_s;
    const float h = q + __shfl_xor(q, 16, kWave);
    colq[j] = h + __shfl_xor(h, 32, kWave);
  }

  __syncthreads();  // histogram cleared, every wavefront done with its candidates
  if (live && rl < Kt) {
    const size_t o = ((size_t)layer * T + t) * Kt + rl;
    if (rl < K) {
      a.idx[o] = my_e;
      a.w[o] = zsel > 0.f ? my_s / zsel : 1.f / (float)K;
      atomicAdd(&hist[my_e], 1);
    } else {
      a.idx[o] = N + (rl - K);
      a.w[o] = 1.f;
      atomicAdd(&hist[N + (rl - K)], 1);
    }
  }
  float* colw = reinterpret_cast<float*>(smem);  // [wave][j*16 + lane] in the candidate area
  const int wave = threadIdx.x >> 6;
  if (a.colpart != nullptr) {
    // every lane stores (the 4 rows of a wavefront store identical sums), so
    // the lane exchanges above are never moved under a lane-dependent branch
#pragma unroll
    for (int j = 0; j < EPL; ++j) colw[wave * (kRowLanes * EPL) + j * kRowLanes + rl] = colq[j];
  }
  __syncthreads();
  if (a.cnt != nullptr) {
    uint16_t* out = a.cnt + (size_t)layer * Nb * gridDim.x + blockIdx.x;
    for (int e = threadIdx.x; e < Nb; e += kThreads) out[(size_t)e * gridDim.x] = (uint16_t)hist[e];
  }
  if (a.colpart != nullptr) {
    constexpr int kWavesPerBlock = kThreads / kWave;
    for (int e = threadIdx.x; e < N; e += kThreads) {
      const int idx = (e % EPL) * kRowLanes + e / EPL;
      float acc = colw[idx];
#pragma unroll
      for (int w = 1; w < kWavesPerBlock; ++w) acc += colw[w * (kRowLanes * EPL) + idx];
      a.colpart[((size_t)layer * gridDim.x + blockIdx.x) * N + e] = acc;
    }
  }
}

template <int EPL, bool GROUPED>
auto pick_kernel(const ScoreArgs& a) {
  if (!a.apply_score) return route_rows_kernel<EPL, GROUPED, kGiven>;
  if (a.score_fn == 1) return route_rows_kernel<EPL, GROUPED, kSigmoid>;
  return route_rows_kernel<EPL, GROUPED, kSoftmax>;
}

// Raise a kernel's dynamic LDS limit to what any N needs, once per kernel and
// device (the attribute call is a host round trip; launches are hot).
hipError_t allow_max_lds(const void* kernel) {
  static std::mutex mu;
  static std::vector<std::pair<const void*, int>> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& kd : done)
    if (kd.first == kernel && kd.second == dev) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)route_rows_lds_bytes(kMaxExperts));
  if (e == hipSuccess) done.emplace_back(kernel, dev);
  return e;
}

template <int EPL>
hipError_t launch_epl(const ScoreArgs& a, int L, hipStream_t s) {
  const dim3 grid((a.T + kRowTokens - 1) / kRowTokens, L);
  const size_t lds = route_rows_lds_bytes(a.N);
  auto k = a.G > 1 ? pick_kernel<EPL, true>(a) : pick_kernel<EPL, false>(a);
  const hipError_t e = allow_max_lds((const void*)k);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, grid, dim3(kThreads), lds, s, a);
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

size_t route_rows_lds_bytes(int N) {
  // candidates (64-bit per expert per row, one pad word per row), reused at
  // the end for the per-wave column sums; slot ids; histogram
  const int epl = route_rows_epl(N);
  const size_t cand = std::max((size_t)kRowTokens * (N + 1) * 8,
                               (size_t)(kThreads / kWave) * kRowLanes * epl * 4);
  return cand + (size_t)kRowTokens * kMaxSlots * 4 + kMaxBuckets * 4;
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
