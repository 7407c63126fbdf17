// Per-token routing on one 16-lane DPP row: scores, bias-aware group-limited
// top-k, combine weights, routing entropy and the block histogram.
//
// The method, per token (pages cited by title and section):
//  1. scores: sigmoid s = 1/(1+exp(-h)) ("DeepSeek V4 MoE load balancing",
//     token routing: sigmoid gating) or softmax p = exp(h)/sum exp(h)
//     ("MoE Routing Entropy vs Expert Saturation", Mathematics); the given
//     scores in SCORES mode. h includes the optional logit offset.
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
//  6. entropy in bits of q = s / sum s (Mathematics section); q is returned
//     for the callers' column sums (batch-mean entropy).
//
// Layout: a wavefront is 4 rows of 16 lanes; the row handles one token and
// lane j of the row holds experts [j*EPL, (j+1)*EPL). Every cross-lane step
// stays inside the row and is a DPP operation (quad permutes, half-row and
// row mirrors, row shifts and rotations).
//
// Exact top-K without K argmax rounds:
//  - lo = the K-th largest of the row's per-lane top-2 eligible keys; these
//    are keys of distinct eligible experts, so lo is at most the K-th largest
//    eligible key: every chosen expert has key >= lo.
//  - the eligible keys >= lo (typically K to K+4) are compacted into LDS as
//    packed 64-bit words (orderable key bits, then inverted id) with their
//    scores, at positions from a row prefix scan of per-lane counts;
//  - a candidate's slot is the number of candidates whose packed word is
//    larger, i.e. that beat it under (key desc, id asc); slots < K are kept.
//  - when more than kCandCap keys reach lo (heavy ties), the row instead runs
//    K rounds of a row-wide maximum over the untaken eligible packed words.
// Both give the unique answer under (key desc, id asc).
#pragma once

#include <math.h>

#include "moer_internal.hpp"

namespace moer {

constexpr int kRowLanes = 16;
constexpr int kCandCap = 32;                // candidates ranked in LDS per token
constexpr int kCandStride = kCandCap + 1;   // entries per row; the pad staggers banks

// ---- DPP helpers ------------------------------------------------------------
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
constexpr int kXor3 = 0x1B;        // quad_perm [3,2,1,0]
constexpr int kHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kMirror = 0x140;     // lane i <-> 15-i within 16

// Rows of RL lanes: 16 (one token per 16-lane DPP row), 8 or 4 (two or four
// tokens per DPP row; only the one-workgroup small-router kernel, whose
// rows hold at most RL experts, uses them). Every lane of a row receives
// max / min / sum of the row (bitwise equal in every lane: each step
// combines a lane with a partner that combines the same two operands).
template <int RL = kRowLanes>
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp_f<kXor1>(v));
  v = fmaxf(v, dpp_f<kXor2>(v));
  if constexpr (RL >= 8) v = fmaxf(v, dpp_f<kHalfMirror>(v));
  if constexpr (RL == 16) v = fmaxf(v, dpp_f<kMirror>(v));
  return v;
}
template <int RL = kRowLanes>
__device__ __forceinline__ float row_min(float v) {
  v = fminf(v, dpp_f<kXor1>(v));
  v = fminf(v, dpp_f<kXor2>(v));
  if constexpr (RL >= 8) v = fminf(v, dpp_f<kHalfMirror>(v));
  if constexpr (RL == 16) v = fminf(v, dpp_f<kMirror>(v));
  return v;
}
template <int RL = kRowLanes>
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_f<kXor1>(v);
  v += dpp_f<kXor2>(v);
  if constexpr (RL >= 8) v += dpp_f<kHalfMirror>(v);
  if constexpr (RL == 16) v += dpp_f<kMirror>(v);
  return v;
}
template <int RL = kRowLanes>
__device__ __forceinline__ int row_max_i(int v) {
  v = max(v, dpp_i<kXor1>(v));
  v = max(v, dpp_i<kXor2>(v));
  if constexpr (RL >= 8) v = max(v, dpp_i<kHalfMirror>(v));
  if constexpr (RL == 16) v = max(v, dpp_i<kMirror>(v));
  return v;
}
// inclusive prefix sum over the row. In 4- and 8-lane rows a shift that
// would cross into the previous token adds nothing; each shift is taken
// with every lane active (a DPP read from a lane that EXEC disables returns
// 0) and masked afterwards.
template <int RL = kRowLanes>
__device__ __forceinline__ int row_scan(int v) {
  if constexpr (RL == 16) {
    v += shr_zero<1>(v);
    v += shr_zero<2>(v);
    v += shr_zero<4>(v);
    return v + shr_zero<8>(v);
  } else {
    const int sub = threadIdx.x & (RL - 1);
    const int d1 = shr_zero<1>(v);
    v += sub >= 1 ? d1 : 0;
    const int d2 = shr_zero<2>(v);
    v += sub >= 2 ? d2 : 0;
    if constexpr (RL == 8) {
      const int d4 = shr_zero<4>(v);
      v += sub >= 4 ? d4 : 0;
    }
    return v;
  }
}
// row maximum of 64-bit words held as (hi, lo) halves
template <int CTRL>
__device__ __forceinline__ void max_step_u64(unsigned& hi, unsigned& lo) {
  const unsigned oh = (unsigned)dpp_i<CTRL>((int)hi);
  const unsigned ol = (unsigned)dpp_i<CTRL>((int)lo);
  if (oh > hi || (oh == hi && ol > lo)) {
    hi = oh;
    lo = ol;
  }
}
template <int RL = kRowLanes>
__device__ __forceinline__ unsigned long long row_max_u64(unsigned long long v) {
  unsigned hi = (unsigned)(v >> 32), lo = (unsigned)v;
  max_step_u64<kXor1>(hi, lo);
  max_step_u64<kXor2>(hi, lo);
  if constexpr (RL >= 8) max_step_u64<kHalfMirror>(hi, lo);
  if constexpr (RL == 16) max_step_u64<kMirror>(hi, lo);
  return ((unsigned long long)hi << 32) | lo;
}
// Every other lane of a 4- or 8-lane row once: xor 1, 2, 3 inside the quad,
// then (8 lanes) the other quad through the half mirror (lane i <-> 7 - i)
// and xor 1, 2, 3 of that. out[0 .. RL-2] receive v from those lanes.
template <int RL>
__device__ __forceinline__ void row_partners(int v, int (&out)[RL - 1]) {
  out[0] = dpp_i<kXor1>(v);
  out[1] = dpp_i<kXor2>(v);
  out[2] = dpp_i<kXor3>(v);
  if constexpr (RL == 8) {
    const int m = dpp_i<kHalfMirror>(v);
    out[3] = m;
    out[4] = dpp_i<kXor1>(m);
    out[5] = dpp_i<kXor2>(m);
    out[6] = dpp_i<kXor3>(m);
  }
}

// Orderable encoding: larger word <=> larger key, then smaller expert id.
// -0 and +0 are the same key: -0 is mapped to +0 here, where the order bits
// are formed (plain float compares already treat them as equal).
__device__ __forceinline__ unsigned long long pack_key(float key, int e) {
  unsigned f = __builtin_bit_cast(unsigned, key);
  f = f == 0x80000000u ? 0u : f;
  const unsigned u = (f & 0x80000000u) ? ~f : (f | 0x80000000u);
  return ((unsigned long long)u << 32) | (unsigned)(0xFFFF - e);
}

// Score modes: the scores are given, or sigmoid / softmax of the affinities.
enum { kGiven = 0, kSigmoid = 1, kSoftmax = 2 };

// Router shape, fixed at compile time for the geometries that get kernels
// of their own (0, or -1 for the shared slots, = taken from the arguments):
// experts N, routed slots K, groups G, groups kept Gk, shared slots.
template <int N_ = 0, int K_ = 0, int G_ = 0, int GK_ = 0, int NS_ = -1>
struct RowShape {
  __device__ static int n(const ScoreArgs& a) { return N_ > 0 ? N_ : a.N; }
  __device__ static int k(const ScoreArgs& a) { return K_ > 0 ? K_ : a.K; }
  __device__ static int g(const ScoreArgs& a) { return G_ > 0 ? G_ : a.G; }
  __device__ static int gk(const ScoreArgs& a) { return GK_ > 0 ? GK_ : a.Gk; }
  __device__ static int ns(const ScoreArgs& a) { return NS_ >= 0 ? NS_ : a.n_shared; }
  static bool matches(const ScoreArgs& a) {
    return (N_ == 0 || a.N == N_) && (K_ == 0 || a.K == K_) && (G_ == 0 || a.G == G_) &&
           (GK_ == 0 || a.Gk == GK_) && (NS_ < 0 || a.n_shared == NS_);
  }
};
using AnyShape = RowShape<>;

// Hardware transcendentals (v_exp_f32, v_rcp_f32, v_log_f32: about 1 ulp):
// the affinities already carry ~1e-6 GEMM rounding, so the scores only need
// to be accurate well inside the 1e-3 weight and 1e-4 entropy tolerances.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
constexpr float kLog2e = 1.4426950408889634f;

template <int MODE>
__device__ __forceinline__ float score_of(float v, float m, float inv_z) {
  if (MODE == kGiven) return v;
  if (MODE == kSigmoid) return rcp_hw(1.f + exp2_hw(-v * kLog2e));
  return exp2_hw((v - m) * kLog2e) * inv_z;
}

// LDS scratch of one token row. A candidate is one 16-byte entry written by
// one store: its first 8 bytes are a 64-bit word whose low half is
// 0xFFFF - expert id and high half the key's order bits, so that one
// unsigned 64-bit compare orders (key desc, id asc); then the score.
struct alignas(16) Cand {
  unsigned id_inv, key, score, pad;
};
__device__ __forceinline__ unsigned long long cand_word(const Cand& c) {
  return *reinterpret_cast<const unsigned long long*>(&c);
}
struct RowLds {
  Cand* cand;    // [kCandStride]
  int* slot_id;  // [kMaxSlots]
  float* slot_s; // [kMaxSlots]
};
// Order bits of a key: for keys all > 0 the raw bits already order them;
// otherwise flip negatives (and set the sign of non-negatives).
__device__ __forceinline__ unsigned order_bits(float key, bool all_positive) {
  unsigned f = __builtin_bit_cast(unsigned, key);
  if (all_positive) return f;
  f = f == 0x80000000u ? 0u : f;  // -0 is +0
  return (f & 0x80000000u) ? ~f : (f | 0x80000000u);
}

// The lane's per-expert constants of a layer, loaded once (and early, so
// their latency hides under the affinity loads): selection bias and logit
// offset of experts e0 .. e0+EPL-1 (0 past N or when absent). With a
// logit-space bias the bias is folded into the offset (offset + b, one fp32
// rounding) and the selection bias is zero.
template <int EPL>
struct LaneConsts {
  float bias[EPL];
  float offset[EPL];
};
template <int EPL, class S = AnyShape, int RL = kRowLanes>
__device__ __forceinline__ void load_lane_consts(const ScoreArgs& a, int layer, bool with_offset,
                                                 LaneConsts<EPL>& c) {
  const int N = S::n(a);
  const int e0 = (threadIdx.x & (RL - 1)) * EPL;
  const float* b = a.bias != nullptr ? a.bias + (size_t)layer * N : nullptr;
  const float* o = with_offset ? a.offset : nullptr;
  auto fill = [&](const float* src, float (&dst)[EPL]) {
    if (src != nullptr && EPL % 4 == 0 && e0 + EPL <= N && (N & 3) == 0) {
#pragma unroll
      for (int j = 0; j < EPL / 4; ++j) {
        const float4 f = reinterpret_cast<const float4*>(src + e0)[j];
        dst[4 * j] = f.x; dst[4 * j + 1] = f.y; dst[4 * j + 2] = f.z; dst[4 * j + 3] = f.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < EPL; ++j) dst[j] = (src != nullptr && e0 + j < N) ? src[e0 + j] : 0.f;
    }
  };
  fill(b, c.bias);
  fill(o, c.offset);
  if (a.bias_logit) {  // the bias joins the logit offset; the keys are the scores
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      c.offset[j] += c.bias[j];
      c.bias[j] = 0.f;
    }
  }
}

// Route token t of `layer` (live = t < T). v: the lane's EPL affinities (or
// given scores), already summed over depth ranges, without the logit offset.
// LPG: lanes per expert group when fixed at compile time, 0 = from a.G at
// run time (GROUPED only). hist: the block histogram in LDS (cleared, and
// the clearing made visible by a barrier, before the call). q: this lane's
// q = s / sum s (0 when dead). All 16 lanes of the row must call together;
// rows are independent.
template <int EPL, bool GROUPED, int MODE, int LPG = 0, class S = AnyShape, int RL = kRowLanes>
__device__ __forceinline__ void route_row(const ScoreArgs& a, int layer, int t, bool live,
                                          float (&v)[EPL], const LaneConsts<EPL>& lc,
                                          const RowLds& rs, int* hist, float (&q)[EPL]) {
  const int N = S::n(a), K = S::k(a), T = a.T;
  const int G = S::g(a), Gk = S::gk(a);
  const int Kt = K + S::ns(a);
  const int rl = threadIdx.x & (RL - 1);  // lane within the row
  const int e0 = rl * EPL;
  const bool full = e0 + EPL <= N;  // every expert of this lane exists
  const float NEG_INF = -__builtin_inff();
  const size_t row_off = ((size_t)layer * T + (live ? t : 0)) * N;

  for (int sl = rl; sl < kMaxSlots; sl += RL) {
    rs.slot_id[sl] = 0;
    rs.slot_s[sl] = 0.f;
  }
  // 1. affinities (+ offset) and scores
  if (MODE != kGiven) {
    if (a.offset != nullptr || (a.bias_logit && a.bias != nullptr)) {
#pragma unroll
      for (int j = 0; j < EPL; ++j) v[j] += lc.offset[j];
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
    m = row_max<RL>(lm);
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) z += (full || e0 + j < N) ? exp2_hw((v[j] - m) * kLog2e) : 0.f;
    inv_z = rcp_hw(row_sum<RL>(z));
  }
  // scores, keys, and each expert's entropy term s*log2(s) (from quantities
  // the score already has where possible)
  float s[EPL], key[EPL], ent[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const bool in = full || e0 + j < N;
    if (MODE == kSigmoid) {
      const float tj = 1.f + exp2_hw(-v[j] * kLog2e);  // s = 1/t, log2 s = -log2 t
      s[j] = in ? rcp_hw(tj) : 0.f;
      ent[j] = -s[j] * log2_hw(fminf(tj, __FLT_MAX__));  // s = 0 when t overflows
    } else if (MODE == kSoftmax) {
      const float aj = (v[j] - m) * kLog2e;  // log2 p = aj + log2(inv_z)
      s[j] = in ? exp2_hw(aj) * inv_z : 0.f;
      ent[j] = s[j] * aj;  // the log2(inv_z) * sum(p) part is added after the sum
    } else {
      s[j] = in ? v[j] : 0.f;
      ent[j] = s[j] > 0.f ? s[j] * log2_hw(s[j]) : 0.f;
    }
    key[j] = in ? s[j] + lc.bias[j] : NEG_INF;
  }

  // 6. entropy of q = s / sum s: H = log2(S) - (sum s log2 s) / S
  float ssum = 0.f, slog = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    ssum += s[j];
    slog += ent[j];
  }
  ssum = row_sum<RL>(ssum);
  slog = row_sum<RL>(slog);
  if (MODE == kSoftmax) slog += log2_hw(inv_z) * ssum;
  // hardware reciprocal and log2 (about 1 ulp each), well inside the 1e-4
  // bit entropy tolerance
  const float rs_sum = ssum > 0.f ? rcp_hw(ssum) : 0.f;
  if (live && rl == 0 && a.tok_entropy != nullptr)
    a.tok_entropy[(size_t)layer * T + t] = ssum > 0.f ? log2_hw(ssum) - slog * rs_sum : 0.f;
  const float inv_s = live ? rs_sum : 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) q[j] = s[j] * inv_s;

  // the lane's two largest keys (used by both the group stage and the bound)
  // (lt1 >= lt2 throughout: the new second largest of {lt1, lt2, k} is the
  // median of the three)
  float lt1 = key[0], lt2 = NEG_INF;
#pragma unroll
  for (int j = 1; j < EPL; ++j) {
    lt2 = __builtin_amdgcn_fmed3f(lt1, lt2, key[j]);
    lt1 = fmaxf(lt1, key[j]);
  }

  // 3. group-limited eligibility
  bool eligible = true;
  float group_m2 = NEG_INF;  // second largest key of this lane's group
  if (GROUPED) {
    const int lpg = LPG > 0 ? LPG : (N / G) / EPL;  // lanes per group (power of two, <= RL)
    const int g = rl / lpg;
    float m1 = lt1, m2 = lt2;
    // merge the group's lanes (lanes of a group are aligned, lpg a power of 2)
    auto merge = [&](float b1, float b2) {
      const float n2 = fmaxf(fminf(m1, b1), fmaxf(m2, b2));
      m1 = fmaxf(m1, b1);
      m2 = n2;
    };
    if (lpg >= 2) merge(dpp_f<kXor1>(m1), dpp_f<kXor1>(m2));
    if (lpg >= 4) merge(dpp_f<kXor2>(m1), dpp_f<kXor2>(m2));
    if (RL >= 8 && lpg >= 8) merge(dpp_f<kHalfMirror>(m1), dpp_f<kHalfMirror>(m2));
    if (RL == 16 && lpg >= 16) merge(dpp_f<kMirror>(m1), dpp_f<kMirror>(m2));
    // the group as one orderable word: score order bits, then the inverted
    // group id, so one unsigned compare orders (score desc, id asc); lanes
    // past the last group hold 0 and beat no group. (A NaN group score sorts
    // above +inf.)
    const unsigned ghi = g < G ? order_bits(m1 + m2, false) : 0u;
    const unsigned glo = g < G ? (unsigned)(0xFFFF - g) : 0u;
    const unsigned long long gkey = ((unsigned long long)ghi << 32) | glo;
    int rank = 0;
    if constexpr (RL == 16) {
      // rank among the row's groups: rotate the words by whole groups
#define MOER_ROT(n)                                                                  \
      if ((n) % lpg == 0) {                                                          \
        const unsigned oh = (unsigned)dpp_i<0x120 + (n)>((int)ghi);                  \
        const unsigned ol = (unsigned)dpp_i<0x120 + (n)>((int)glo);                  \
        rank += ((((unsigned long long)oh << 32) | ol) > gkey) ? 1 : 0;              \
      }
      MOER_ROT(1) MOER_ROT(2) MOER_ROT(3) MOER_ROT(4) MOER_ROT(5) MOER_ROT(6) MOER_ROT(7)
      MOER_ROT(8) MOER_ROT(9) MOER_ROT(10) MOER_ROT(11) MOER_ROT(12) MOER_ROT(13) MOER_ROT(14)
      MOER_ROT(15)
#undef MOER_ROT
      eligible = g < G && rank < Gk;
    } else {
      // every other lane of the row once: a better group is counted once per
      // lane it spans (lpg), the own group's lanes never (equal words)
      int ph[RL - 1], pl[RL - 1];
      row_partners<RL>((int)ghi, ph);
      row_partners<RL>((int)glo, pl);
#pragma unroll
      for (int i = 0; i < RL - 1; ++i)
        rank += ((((unsigned long long)(unsigned)ph[i] << 32) | (unsigned)pl[i]) > gkey) ? 1 : 0;
      eligible = g < G && rank < Gk * lpg;
    }
    group_m2 = m2;
  }

  // keys and scores for the capacity-limited rounds (candidates beyond top-K)
  if (live && a.key_out != nullptr) {
    float ko[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) ko[j] = eligible ? key[j] + 0.f : NEG_INF;  // -0 -> +0
    if (EPL % 4 == 0 && full && (N & 3) == 0) {  // 16-byte stores
#pragma unroll
      for (int j = 0; j < EPL; j += 4) {
        *reinterpret_cast<float4*>(a.key_out + row_off + e0 + j) =
            make_float4(ko[j], ko[j + 1], ko[j + 2], ko[j + 3]);
        *reinterpret_cast<float4*>(a.s_out + row_off + e0 + j) =
            make_float4(s[j], s[j + 1], s[j + 2], s[j + 3]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        if (e0 + j < N) {
          a.key_out[row_off + e0 + j] = ko[j];
          a.s_out[row_off + e0 + j] = s[j];
        }
      }
    }
  }

  // lo: a key that at least K distinct eligible experts reach, so every chosen
  // expert has key >= lo.
  float lo;
  if (GROUPED && 2 * Gk == K) {
    // the kept groups' two largest keys are exactly K such experts: lo is
    // the smallest of them (the groups' second keys)
    lo = row_min<RL>(eligible ? group_m2 : __builtin_inff());
  } else {
    // the K-th largest of the eligible lanes' two largest keys (up to 32)
    const float l1 = eligible ? lt1 : NEG_INF, l2 = eligible ? lt2 : NEG_INF;
    int c1 = 1 + (l2 >= l1 ? 1 : 0), c2 = 2;  // values >= l1 / >= l2, own pair included
    auto count_ge = [&](float o1, float o2) {
      c1 += (o1 >= l1 ? 1 : 0) + (o2 >= l1 ? 1 : 0);
      c2 += (o1 >= l2 ? 1 : 0) + (o2 >= l2 ? 1 : 0);
    };
    if constexpr (RL == 16) {
#define MOER_CGE(n) count_ge(dpp_f<0x120 + (n)>(l1), dpp_f<0x120 + (n)>(l2));
      MOER_CGE(1) MOER_CGE(2) MOER_CGE(3) MOER_CGE(4) MOER_CGE(5) MOER_CGE(6) MOER_CGE(7)
      MOER_CGE(8) MOER_CGE(9) MOER_CGE(10) MOER_CGE(11) MOER_CGE(12) MOER_CGE(13) MOER_CGE(14)
      MOER_CGE(15)
#undef MOER_CGE
    } else {
      int p1[RL - 1], p2[RL - 1];
      row_partners<RL>(__float_as_int(l1), p1);
      row_partners<RL>(__float_as_int(l2), p2);
#pragma unroll
      for (int i = 0; i < RL - 1; ++i) count_ge(__int_as_float(p1[i]), __int_as_float(p2[i]));
    }
    lo = row_max<RL>(fmaxf(c1 >= K ? l1 : NEG_INF, c2 >= K ? l2 : NEG_INF));
  }

  // candidates: eligible keys >= lo (lo is finite: at least K finite keys
  // reach it; the clamp keeps absent experts' -inf keys out regardless)
  const float lo_f = fmaxf(lo, -__FLT_MAX__);
  unsigned bits = 0;
  if (eligible) {
#pragma unroll
    for (int j = 0; j < EPL; ++j) bits |= key[j] >= lo_f ? 1u << j : 0u;
  }
  const int mine = __builtin_popcount(bits);
  const int incl = row_scan<RL>(mine);
  const int count = row_max_i<RL>(incl);
  // A row's candidates and slots are private to its wavefront, and a
  // wavefront's LDS operations complete in order: no barrier is needed.
  if (count <= kCandCap) {
    // 4. compact, then slot = number of candidates that beat this one
    const bool all_positive = lo > 0.f;  // every candidate key >= lo
    int pos = incl - mine;
    if (all_positive) {
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (bits & (1u << j)) {
          rs.cand[pos] = Cand{(unsigned)(0xFFFF - (e0 + j)), __builtin_bit_cast(unsigned, key[j]),
                              __builtin_bit_cast(unsigned, s[j]), 0u};
          ++pos;
        }
    } else {
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (bits & (1u << j)) {
          rs.cand[pos] = Cand{(unsigned)(0xFFFF - (e0 + j)), order_bits(key[j], false),
                              __builtin_bit_cast(unsigned, s[j]), 0u};
          ++pos;
        }
    }
    for (int c = rl; c < count; c += RL) {
      const unsigned long long my = cand_word(rs.cand[c]);
      int r = 0;
#pragma unroll 4
      for (int i = 0; i < count; ++i) r += cand_word(rs.cand[i]) > my ? 1 : 0;
      if (r < K) {
        rs.slot_id[r] = 0xFFFF - (int)(my & 0xFFFF);
        rs.slot_s[r] = __builtin_bit_cast(float, rs.cand[c].score);
      }
    }
  } else {
    // heavy ties: K rounds of the row-wide best untaken candidate
    unsigned taken = 0;
    for (int r = 0; r < K; ++r) {
      unsigned long long best = 0;
      int bj = -1;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        if (!((bits >> j) & 1u) || ((taken >> j) & 1u)) continue;
        const unsigned long long pk = pack_key(key[j], e0 + j);
        if (pk > best) {
          best = pk;
          bj = j;
        }
      }
      const unsigned long long win = row_max_u64<RL>(best);
      if (bj >= 0 && best == win) {  // expert ids are unique: one owner lane
        taken |= 1u << bj;
        rs.slot_id[r] = e0 + bj;
        float sb = 0.f;
#pragma unroll
        for (int j = 0; j < EPL; ++j) sb = j == bj ? s[j] : sb;
        rs.slot_s[r] = sb;
      }
    }
  }

  // 5. weights over the chosen slots, then the outputs and the histogram
  // (lane rl takes slots rl, rl + RL, ...: one slot per lane in 16-lane rows)
  constexpr int kSlotsPerLane = kMaxSlots / RL;
  int my_e[kSlotsPerLane];
  float my_s[kSlotsPerLane];
  float zpart = 0.f;
#pragma unroll
  for (int h = 0; h < kSlotsPerLane; ++h) {
    const int sl = rl + h * RL;
    my_e[h] = 0;
    my_s[h] = 0.f;
    if (sl < K) {
      my_e[h] = min(max(rs.slot_id[sl], 0), N - 1);  // in range even for non-finite input
      my_s[h] = rs.slot_s[sl];
      zpart = h == 0 ? my_s[h] : zpart + my_s[h];
    }
  }
  const float zsel = row_sum<RL>(zpart);
  if (live) {
#pragma unroll
    for (int h = 0; h < kSlotsPerLane; ++h) {
      const int sl = rl + h * RL;
      if (sl >= Kt) continue;
      const size_t o = ((size_t)layer * T + t) * Kt + sl;
      if (sl < K) {
        a.idx[o] = my_e[h];
        a.w[o] = zsel > 0.f ? my_s[h] / zsel : 1.f / (float)K;
        atomicAdd(&hist[my_e[h]], 1);
      } else {
        a.idx[o] = N + (sl - K);
        a.w[o] = 1.f;
        atomicAdd(&hist[N + (sl - K)], 1);
      }
    }
  }
}

// The column sums of q over the 64 / RL rows of this wavefront (zero for
// rows past T), left in lanes 0 .. RL-1 (lane rl: experts rl*EPL ..): in
// 4- and 8-lane rows first the tokens of each 16-lane DPP row (rotations by
// 8, then 4), then (row0 + row1) + (row2 + row3) of the DPP rows by lane
// swaps between rows and between wave halves. Every lane adds its operands
// in a fixed order, so the sums are deterministic.
template <int EPL, int RL = kRowLanes>
__device__ __forceinline__ void wave_column_sums(const float (&q)[EPL], float (&cs)[EPL]) {
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    float x = q[j];
    if constexpr (RL <= 8) x += dpp_f<0x128>(x);  // row_ror:8
    if constexpr (RL == 4) x += dpp_f<0x124>(x);  // row_ror:4
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    const float pair = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair),
                                                    false, false);
    cs[j] = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  }
}

// The block outputs of a selection workgroup of NT threads (NT / 16 rows, one
// 64-token histogram block per workgroup, blockIdx.x = block), once every row
// has been routed: the block's expert histogram cnt[l][e][b], its running
// segment totals, and its column sums of q. colw: LDS [NT / 64][16 * EPL].
// Every thread of the workgroup must call (it holds a barrier).
template <int EPL, int NT>
__device__ __forceinline__ void block_outputs(const ScoreArgs& a, int layer, int N, int Nb,
                                              const float (&q)[EPL], const int* hist,
                                              float (*colw)[kRowLanes * EPL]) {
  constexpr int kWaves = NT / kWave;
  const int lane = threadIdx.x & 63;
  const int rl = lane & 15;
  if (a.colpart != nullptr) {
    // the wavefront's column sums of q over its 4 rows (zero for tokens past T)
    float cs[EPL];
    wave_column_sums<EPL>(q, cs);
    if (lane < kRowLanes) {
#pragma unroll
      for (int j = 0; j < EPL; ++j) colw[threadIdx.x >> 6][rl * EPL + j] = cs[j];
    }
  }
  __syncthreads();
  if (a.cnt != nullptr) {
    uint16_t* out = a.cnt + (size_t)layer * Nb * gridDim.x + blockIdx.x;
    for (int e = threadIdx.x; e < Nb; e += NT) out[(size_t)e * gridDim.x] = (uint16_t)hist[e];
  }
  if (a.segsum != nullptr) {
    // running totals per segment of blocks (integer adds: any order, same sum)
    const int nseg = (gridDim.x + kSegBlocks - 1) / kSegBlocks;
    int32_t* seg = a.segsum + ((size_t)layer * nseg + blockIdx.x / kSegBlocks) * Nb;
    for (int e = threadIdx.x; e < Nb; e += NT)
      if (hist[e] != 0) atomicAdd(&seg[e], hist[e]);
  }
  if (a.colpart != nullptr) {
    // the block's column sums: the wavefronts' sums in wavefront order
    for (int e = threadIdx.x; e < N; e += NT) {
      float acc = colw[0][e];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) acc += colw[w][e];
      a.colpart[((size_t)layer * gridDim.x + blockIdx.x) * N + e] = acc;
    }
  }
}

}  // namespace moer
