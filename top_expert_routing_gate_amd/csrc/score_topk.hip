// Scoring, bias-aware group-limited top-k, combine weights and per-token
// routing entropy: one wavefront per token, E consecutive experts per lane
// (E = 4 for N <= 256, 2 for N <= 128, 1 for N <= 64), all N scores held in
// registers.
//
// Steps, per token, in the order the pages give them:
//  1. scores: sigmoid s = 1/(1+exp(-h)) ("DeepSeek V4 MoE load balancing",
//     token routing: sigmoid gating) or softmax p = exp(h)/sum exp(h)
//     ("MoE Routing Entropy vs Expert Saturation", Mathematics); in SCORES
//     mode the scores are given.
//  2. key = s + b in fp32 (auxiliary-loss-free balancing: the bias enters the
//     routing decision only); -0 is made +0.
//  3. G > 1 ("DeepSeek-V3 Group-Limited Expert Routing", s.1 and s.3): the N
//     keys are G contiguous groups; group score = fp32 sum of the group's two
//     largest keys; the Gk best groups (score desc, group id asc) stay
//     eligible, the others are masked out. Groups that are a power-of-two
//     number of lanes merge their lanes' top-2 by shuffles; any other group
//     size (any N/G >= 2) goes through LDS: a lane scans whole groups.
//  4. K rounds of a wave-wide argmax over the eligible keys, ordered by
//     (key desc, expert id asc); the winner of round r fills slot r.
//  5. Shared experts (same page, s.4: counted as routed slots) fill slots
//     K..Kt-1 with ids N.. and weight 1.
//  6. weights = chosen unbiased scores / their sum (the listing's top-k
//     renormalisation; the weighted combine of the routing section).
//  7. entropy of q = s / sum_e s in bits (Mathematics section), per token;
//     each workgroup also writes the column sums of q over its tokens for
//     the batch-mean entropy.
#include <math.h>

#include "moer_internal.hpp"

namespace moer {
namespace {

constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Lane-aligned groups: every group is a power-of-two number of whole lanes.
bool score_topk_lane_groups(int N, int G) {
  const int gsz = N / G, E = experts_per_lane(N);
  return gsz % E == 0 && ((gsz / E) & (gsz / E - 1)) == 0 && gsz / E <= kWave;
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Group stage: none, lane-aligned power-of-two groups (shuffles), or any
// group size (the wave's keys and group scores in LDS).
enum { kNoGroups = 0, kLaneGroups = 1, kAnyGroups = 2 };

// Orders the wave's LDS writes before its later LDS reads at compile time; a
// wavefront's LDS operations are performed in program order.
__device__ __forceinline__ void wave_lds_order() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

template <int E, int GMODE>
__global__ __launch_bounds__(kWavesPerBlock * kWave) void score_topk_kernel(ScoreArgs a) {
  constexpr bool GROUPED = GMODE != kNoGroups;
  constexpr int kGW = GMODE == kAnyGroups ? kWavesPerBlock : 1;
  __shared__ float colsum[kWavesPerBlock][kMaxExperts];
  __shared__ float gkey[kGW][GMODE == kAnyGroups ? kMaxExperts : 1];       // the token's keys
  __shared__ float gscore[kGW][GMODE == kAnyGroups ? kMaxExperts / 2 : 1]; // group scores
  __shared__ int gkeep[kGW][GMODE == kAnyGroups ? kMaxExperts / 2 : 1];    // group eligible

  const int layer = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int N = a.N, K = a.K, T = a.T;
  const int Kt = K + a.n_shared;
  const float NEG_INF = -__builtin_inff();

  float bias_r[E];
  float off_r[E];
  float col[E];
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int e = lane * E + j;
    bias_r[j] = (a.bias != nullptr && e < N) ? a.bias[(size_t)layer * N + e] : 0.f;
    // logit-space bias: added to the logits with the offset (offset + b, one
    // fp32 rounding, as in the row kernel); the keys are then the scores
    off_r[j] = (a.offset != nullptr && e < N) ? a.offset[e] : 0.f;
    if (a.bias_logit) {
      off_r[j] += bias_r[j];
      bias_r[j] = 0.f;
    }
    col[j] = 0.f;
  }

  // Group geometry (GROUPED only): group size, and for lane-aligned groups
  // the lanes per group and this lane's group.
  const int gsz = GROUPED ? N / a.G : N;
  const int lpg = GMODE == kLaneGroups ? gsz / E : kWave;
  const int my_group = GMODE == kLaneGroups ? lane / lpg : 0;

  const int tbase = blockIdx.x * kRowTokens;
  for (int tt = wave; tt < kRowTokens; tt += kWavesPerBlock) {
    const int t = tbase + tt;
    if (t >= T) break;
    const size_t row_off = ((size_t)layer * T + t) * N;
    const size_t split_stride = (size_t)gridDim.y * T * N;

    // affinities: partial sums over depth ranges added in order, then the offset
    float v[E];
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int e = lane * E + j;
      float acc = 0.f;
      if (e < N) {
        acc = a.in[row_off + e];
        for (int sp = 1; sp < a.nsplit; ++sp) acc += a.in[sp * split_stride + row_off + e];
        if (a.offset != nullptr || (a.bias_logit && a.bias != nullptr)) acc += off_r[j];
        if (a.h_out != nullptr) a.h_out[row_off + e] = acc;
      }
      v[j] = acc;
    }

    // 1. scores
    float s[E];
    if (!a.apply_score) {
#pragma unroll
      for (int j = 0; j < E; ++j) s[j] = (lane * E + j < N) ? v[j] : 0.f;
    } else if (a.score_fn == 1) {
#pragma unroll
      for (int j = 0; j < E; ++j) s[j] = (lane * E + j < N) ? 1.f / (1.f + expf(-v[j])) : 0.f;
    } else {
      float m = NEG_INF;
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (lane * E + j < N) m = fmaxf(m, v[j]);
      m = wave_max(m);
      float z = 0.f;
#pragma unroll
      for (int j = 0; j < E; ++j) {
        s[j] = (lane * E + j < N) ? expf(v[j] - m) : 0.f;
        z += s[j];
      }
      z = wave_sum(z);
#pragma unroll
      for (int j = 0; j < E; ++j) s[j] = s[j] / z;
    }

    // 2. biased keys
    float key[E];
#pragma unroll
    for (int j = 0; j < E; ++j) {
      key[j] = (lane * E + j < N) ? (s[j] + bias_r[j]) + 0.f : NEG_INF;
    }

    // 3. group-limited eligibility
    if (GMODE == kAnyGroups) {
      const int gw = GMODE == kAnyGroups ? wave : 0;
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (lane * E + j < N) gkey[gw][lane * E + j] = key[j];
      wave_lds_order();
      // lane g (and g + 64) scores whole groups: the sum of the two largest keys
      for (int g = lane; g < a.G; g += kWave) {
        const float* gk = &gkey[gw][g * gsz];
        float m1 = gk[0], m2 = NEG_INF;
        for (int i = 1; i < gsz; ++i) {
          m2 = fmaxf(m2, fminf(m1, gk[i]));
          m1 = fmaxf(m1, gk[i]);
        }
        gscore[gw][g] = m1 + m2;
      }
      wave_lds_order();
      // rank among all groups under (score desc, group id asc)
      for (int g = lane; g < a.G; g += kWave) {
        const float gs = gscore[gw][g];
        int rank = 0;
        for (int o = 0; o < a.G; ++o) {
          const float og = gscore[gw][o];
          rank += (og > gs || (og == gs && o < g)) ? 1 : 0;
        }
        gkeep[gw][g] = rank < a.Gk ? 1 : 0;
      }
      wave_lds_order();
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const int e = lane * E + j;
        if (e < N && gkeep[gw][e / gsz] == 0) key[j] = NEG_INF;
      }
      wave_lds_order();  // the next token's key writes come after these reads
    } else if (GMODE == kLaneGroups) {
      float m1 = key[0], m2 = NEG_INF;
#pragma unroll
      for (int j = 1; j < E; ++j) {
        m2 = fmaxf(m2, fminf(m1, key[j]));
        m1 = fmaxf(m1, key[j]);
      }
      for (int o = 1; o < lpg; o <<= 1) {
        const float b1 = __shfl_xor(m1, o, kWave);
        const float b2 = __shfl_xor(m2, o, kWave);
        const float n2 = fmaxf(fminf(m1, b1), fmaxf(m2, b2));
        m1 = fmaxf(m1, b1);
        m2 = n2;
      }
      const float gs = m1 + m2;
      int rank = 0;
      for (int g = 0; g < a.G; ++g) {
        const float og = readlane_f(gs, g * lpg);
        rank += (og > gs || (og == gs && g < my_group)) ? 1 : 0;
      }
      if (rank >= a.Gk) {
#pragma unroll
        for (int j = 0; j < E; ++j) key[j] = NEG_INF;
      }
    }

    // keys and scores for the capacity-limited rounds (candidates beyond top-K)
    if (a.key_out != nullptr) {
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const int e = lane * E + j;
        if (e < N) {
          a.key_out[row_off + e] = key[j];
          a.s_out[row_off + e] = s[j];
        }
      }
    }

    // 4. top-K rounds
    int sel_e[kMaxSlots];
    float sel_s[kMaxSlots];
#pragma unroll
    for (int r = 0; r < kMaxSlots; ++r) {
      sel_e[r] = 0;
      sel_s[r] = 0.f;
      if (r >= K) continue;
      float bv = key[0];
      int bj = 0;
      float bs = s[0];
#pragma unroll
      for (int j = 1; j < E; ++j) {
        if (key[j] > bv) { bv = key[j]; bj = j; bs = s[j]; }
      }
      const float M = wave_max(bv);
      // lanes past the experts hold -inf keys: they may tie M only when every
      // real key is -inf or NaN (non-finite input, unspecified result); the
      // winner is then a real expert all the same
      const unsigned long long hit = __ballot(bv == M && lane * E < N);
      const int L = hit ? __builtin_ctzll(hit) : 0;
      const int jw = __builtin_amdgcn_readlane(bj, L);
      sel_e[r] = min(L * E + jw, N - 1);
      sel_s[r] = readlane_f(bs, L);
      if (lane == L) {
#pragma unroll
        for (int j = 0; j < E; ++j)
          if (j == jw) key[j] = NEG_INF;
      }
    }

    // 6. renormalised weights (all lanes hold the same slot values)
    float z = 0.f;
#pragma unroll
    for (int r = 0; r < kMaxSlots; ++r)
      if (r < K) z += sel_s[r];
    if (lane < Kt) {
      int my_e = N + (lane - K);
      float my_w = 1.f;
#pragma unroll
      for (int r = 0; r < kMaxSlots; ++r) {
        if (r < K && lane == r) {
          my_e = sel_e[r];
          my_w = z > 0.f ? sel_s[r] / z : 1.f / (float)K;
        }
      }
      const size_t o = ((size_t)layer * T + t) * Kt + lane;
      a.idx[o] = my_e;
      a.w[o] = my_w;
    }

    // 7. entropy of q = s / sum s, and column sums of q
    if (a.tok_entropy != nullptr || a.colpart != nullptr) {
      float ssum = 0.f, slog = 0.f;
#pragma unroll
      for (int j = 0; j < E; ++j) {
        ssum += s[j];
        slog += s[j] > 0.f ? s[j] * log2f(s[j]) : 0.f;
      }
      ssum = wave_sum(ssum);
      slog = wave_sum(slog);
      if (a.tok_entropy != nullptr && lane == 0)
        a.tok_entropy[(size_t)layer * T + t] = ssum > 0.f ? log2f(ssum) - slog / ssum : 0.f;
      if (ssum > 0.f) {
        const float inv = 1.f / ssum;
#pragma unroll
        for (int j = 0; j < E; ++j) col[j] += s[j] * inv;
      }
    }
  }

  if (a.colpart != nullptr) {
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int e = lane * E + j;
      if (e < kMaxExperts) colsum[wave][e] = col[j];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < N; e += blockDim.x) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < kWavesPerBlock; ++w) acc += colsum[w][e];
      a.colpart[((size_t)layer * gridDim.x + blockIdx.x) * N + e] = acc;
    }
  }
}

template <int E>
hipError_t launch_e(const ScoreArgs& a, int L, hipStream_t s) {
  dim3 grid((a.T + kRowTokens - 1) / kRowTokens, L);
  const dim3 block(kWavesPerBlock * kWave);
  if (a.G > 1 && score_topk_lane_groups(a.N, a.G))
    hipLaunchKernelGGL((score_topk_kernel<E, kLaneGroups>), grid, block, 0, s, a);
  else if (a.G > 1)
    hipLaunchKernelGGL((score_topk_kernel<E, kAnyGroups>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((score_topk_kernel<E, kNoGroups>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score_topk(const ScoreArgs& a, int L, hipStream_t s) {
  switch (experts_per_lane(a.N)) {
    case 4: return launch_e<4>(a, L, s);
    case 2: return launch_e<2>(a, L, s);
    default: return launch_e<1>(a, L, s);
  }
}

}  // namespace moer
