// Internal declarations shared by the router's HIP sources (not part of the
// public ABI; the public ABI is include/moer.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moer {

constexpr int kWave = 64;           // CDNA wavefront width
constexpr int kMaxExperts = 256;    // N
constexpr int kMaxSlots = 16;       // Kt
constexpr int kMaxBuckets = kMaxExperts + kMaxSlots;
constexpr int kScoreTokens = 16;    // tokens per score_topk workgroup
constexpr int kLayoutTokens = 128;  // tokens per layout workgroup

// Everything a score/select launch needs (passed by value).
struct ScoreArgs {
  const float* in;        // [L][T][N] affinities h (apply_score) or scores s
  const float* bias;      // [L][N] or nullptr
  int32_t* idx;           // [L][T][Kt]
  float* w;               // [L][T][Kt]
  float* tok_entropy;     // [L][T] or nullptr
  float* colpart;         // [L][nsb][N] per-workgroup sums of q, or nullptr
  int T, N, K, G, Gk, n_shared, score_fn, apply_score;
};

struct LayoutArgs {
  const int32_t* idx;     // [L][T][Kt]
  int32_t* cnt;           // workspace [L][nlb][Nb]
  const float* colpart;   // [L][nsb][N] or nullptr
  float* colpart2;        // [L][nlb][N] or nullptr
  float* agg_entropy;     // [L] or nullptr
  int32_t* counts;        // [L][Nb]
  int32_t* offsets;       // [L][Nb+1]
  int32_t* perm;          // [L][T*Kt]
  int32_t* inv_perm;      // [L][T*Kt] or nullptr
  int T, Kt, Nb, N, nlb, nsb, fill_invalid;
};

hipError_t launch_gate_gemm_bf16(const void* x, const void* w, const float* offset, float* h,
                                 int L, int T, int d, int N, hipStream_t s);
hipError_t launch_gate_gemm_f32(const float* x, const float* w, const float* offset, float* h,
                                int L, int T, int d, int N, hipStream_t s);
hipError_t launch_score_topk(const ScoreArgs& a, int L, hipStream_t s);
hipError_t launch_layout(const LayoutArgs& a, int L, hipStream_t s);
hipError_t launch_load_stats(const int32_t* counts, int L, int N, int stride, void* out,
                             hipStream_t s);
hipError_t launch_bias_update(float* bias, const int32_t* counts, int L, int N, int stride,
                              float u, hipStream_t s);

// Experts held per lane by the one-wave-per-token selection.
inline int experts_per_lane(int N) { return N > 128 ? 4 : (N > 64 ? 2 : 1); }

}  // namespace moer
