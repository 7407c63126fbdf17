// Internal declarations shared by the router's HIP sources (not part of the
// public ABI; the public ABI is include/moer.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moer.h"

namespace moer {

constexpr int kWave = 64;           // CDNA wavefront width
constexpr int kMaxExperts = 256;    // N
constexpr int kMaxSlots = 16;       // Kt
constexpr int kMaxBuckets = kMaxExperts + kMaxSlots;
constexpr int kRowTokens = 64;      // tokens per selection workgroup (= histogram block)
constexpr int kLayoutTokens = 64;   // tokens per scatter workgroup (1 histogram block)
constexpr int kSegBlocks = 16;       // histogram blocks per segment of the running totals

// Everything a score/select launch needs (passed by value).
struct ScoreArgs {
  const float* in;        // [nsplit][L][T][N] partial affinities (apply_score) or scores s
  const float* offset;    // [N] logit offset added to h, or nullptr
  float* h_out;           // [L][T][N] summed affinities, or nullptr
  const float* bias;      // [L][N] or nullptr
  int32_t* idx;           // [L][T][Kt]
  float* w;               // [L][T][Kt]
  float* tok_entropy;     // [L][T] or nullptr
  float* colpart;         // [L][nsb][N] sums of q per 64-token block, or nullptr
  uint16_t* cnt;          // [L][Nb][nsb] expert counts per 64-token block, or nullptr
  int32_t* segsum;        // [L][nseg][Nb] += the block counts (zero beforehand), or nullptr
  int T, N, K, G, Gk, n_shared, score_fn, apply_score, nsplit;
  int bias_logit;         // 1: the bias is added to the logits (with the offset)
  float* key_out;         // [L][T][N] selection keys, -inf outside the kept groups, or nullptr
  float* s_out;           // [L][T][N] scores (the weights' numerators), or nullptr
};

struct LayoutArgs {
  const int32_t* idx;     // [L][T][Kt]
  uint16_t* cnt;          // [L][Nb][nsb] expert counts per 64-token block
  int32_t* segsum;        // [L][nseg][Nb] expert counts per segment of kSegBlocks blocks
  const float* colpart;   // [L][nsb][N] or nullptr
  float* agg_entropy;     // [L] or nullptr
  int32_t* counts;        // [L][Nb]
  int32_t* offsets;       // [L][Nb+1]
  int32_t* perm;          // [L][T*Kt]
  int32_t* inv_perm;      // [L][T*Kt] or nullptr
  moer_load_stats_t* stats;  // [L] or nullptr
  float* bias_inout;      // [L][N] updated in place, or nullptr
  float bias_step;
  int T, Kt, Nb, N, nlb, nsb, nseg, fill_invalid, need_count;
  // histogram blocks per layout block = 1 << hist_shift (> 0 only for
  // 16-token histogram blocks, which carry no segment totals: segsum null)
  int hist_shift;
  // capacity-limited routing: phase 1 = the layout of the top-K ids (one
  // balance workgroup per layer sets cap_flag[l] when a routed expert holds
  // more than cap, and does the statistics / bias update only when none
  // does); phase 2 = the layout of the final ids (skipped, like the rest of
  // the capacity pass, for layers whose flag is 0)
  int cap, cap_phase;
  int32_t* cap_flag;      // [L]
};

// Depth ranges the bf16 gate GEMM splits d into (its partial sums are
// part[0..ksplit) [L][T][N]); 1 for fp32 inputs.
int gate_gemm_ksplit(int dtype_bf16, int L, int T, int d, int N);
// zero[0..n_zero) is cleared by the launch before any of its tiles finish
// (for counters the next kernels of the call accumulate into).
// ev0 / ev1 (may be null): profiling events recorded at the GEMM kernel's
// start and end.
hipError_t launch_gate_gemm_bf16(const void* x, const void* w, float* part, int L, int T, int d,
                                 int N, int ksplit, int32_t* zero, int n_zero, hipStream_t s,
                                 hipEvent_t ev0, hipEvent_t ev1);
// Whether launch_gate_gemm_bf16 takes the pipelined kernel (which clears
// `zero` itself) for this shape; otherwise clear it with launch_zero_ints.
bool gate_gemm_clears(int L, int T, int d, int N, int ksplit);
hipError_t launch_zero_ints(int32_t* p, int n, hipStream_t s);
hipError_t launch_gate_gemm_f32(const float* x, const float* w, float* h, int L, int T, int d,
                                int N, int32_t* zero, int n_zero, hipStream_t s);
hipError_t launch_score_topk(const ScoreArgs& a, int L, hipStream_t s);
// 16-token histogram blocks (the small-batch selection kernel and the
// one-launch small-router kernel): four per 64-token layout block.
constexpr int kSmallTokens = 16;
constexpr int kSmallShift = 2;  // kRowTokens / kSmallTokens = 4 blocks per layout block
constexpr int kSmallMaxExperts = 16;

// Row-per-token selection (writes the block histograms itself). rows: the
// tokens per workgroup and histogram block, route_rows_tokens(L, T): 64, or
// 16 / 32 for batches of fewer than kTinyGrid / kFewGrid 64-token blocks;
// blocks of 16 or 32 tokens carry no segment totals (ScoreArgs and LayoutArgs
// segsum null, LayoutArgs hist_shift = log2(64 / rows)).
constexpr int kTinyGrid = 64;
constexpr int kFewGrid = 256;
int route_rows_epl(int N);
bool route_rows_supports(int N, int G);
int route_rows_tokens(int L, int T);
hipError_t launch_route_rows(const ScoreArgs& a, int L, hipStream_t s, int rows);
// Gate GEMM and selection in one launch for at most 16 experts and 4096
// tokens (bf16 with d a multiple of 128, or fp32 with d a multiple of 64;
// x and W_g 16-byte aligned). Its histogram blocks are kSmallTokens tokens
// (cnt [L][Nb][ceil(T / kSmallTokens)], colpart likewise) and carry no
// segment totals: ScoreArgs segsum null, LayoutArgs segsum null with
// hist_shift = kSmallShift. ev0 / ev1 (optional) bracket the launch.
// With whole != nullptr (route_layer_eligible: layers of at most
// kWholeTokens tokens for routers of at most 8 experts, kWholeTokensWide for
// at most 16, and at most kWholeSteps depth steps of 128 (bf16) or 64
// (fp32); no capacity limit): one workgroup per layer that also writes the
// layout outputs of *whole (counts, offsets, perm, inv_perm, batch-mean
// entropy, load statistics, bias update), so no layout launch follows.
constexpr int kWholeTokens = 64;
constexpr int kWholeTokensWide = 32;
constexpr int kWholeSteps = 4;
bool route_small_eligible(bool bf16, int T, int d, int N, int G, bool aligned);
bool route_layer_eligible(bool bf16, int T, int d, int N);
hipError_t launch_route_small(const ScoreArgs& a, const void* x, const void* W, int d, bool bf16,
                              int L, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1,
                              const LayoutArgs* whole = nullptr);
hipError_t launch_layout(const LayoutArgs& a, int L, hipStream_t s);
// Fused router pass (gate GEMM in two depth halves exchanging partials
// pairwise, selection from LDS, then the layout after a grid barrier): can it
// take this bf16 router (128 < N <= 256, N % 16 == 0, d % 128 == 0, its
// whole grid resident at once)? Its exchange buffer is [2][L][T][N] fp32.
bool route_fused_eligible(int L, int T, int d, int N, int G);
// Counters the fused pass needs zeroed before its launch.
int route_fused_sync_ints(int L, int T);
hipError_t launch_route_fused(const void* x, const void* w, float* part, int32_t* sync,
                              float* colmean, const ScoreArgs& sa, const LayoutArgs& la, int L,
                              int T, int d, int N, bool layout, hipStream_t s);
hipError_t launch_load_stats(const int32_t* counts, int L, int N, int stride, moer_load_stats_t* out,
                             hipStream_t s);
hipError_t launch_bias_update(float* bias, const int32_t* counts, int L, int N, int stride,
                              float u, hipStream_t s);

// Local dispatch / weighted combine (token-major, one wavefront per token).
hipError_t launch_dispatch(const void* x, int64_t row_bytes, int L, int T, int Kt,
                           const int32_t* inv_perm, void* out, hipStream_t s);
hipError_t launch_combine(const void* eo, int eo_bf16, const float* w, const int32_t* inv_perm,
                          int L, int T, int Kt, int d, void* y, int y_bf16, hipStream_t s);

// Capacity-limited routing (after the selection and the first layout).
// Rounds 1..kCapGridRounds are ranked by the layout kernels (all of the
// chip); the rest by one workgroup per layer.
constexpr int kCapGridRounds = 2;
struct CapRound {
  int32_t* prop;            // [L][T*K] proposals of the round (-1: none / no candidate)
  int32_t* mask;            // [L][T] slots proposing in the round (bit k)
  uint16_t* cnt;            // layout of the proposals (grid rounds only)
  int32_t* segsum;
  int32_t* counts;          // [L][N]
  int32_t* offsets;         // [L][N+1]
  int32_t* perm;            // [L][T*K]
  int32_t* inv;             // [L][T*K] position of each proposal in its expert's bucket
};
struct CapArgs {
  int32_t* idx;             // [L][T][Kt] top-K in, capacity-limited out (-1 = dropped)
  float* w;                 // [L][T][Kt] weights, renormalised for changed tokens
  const int32_t* inv_perm;  // [L][T*Kt] first layout (round 0 ranks)
  const int32_t* offsets;   // [L][Nb+1] first layout
  const float* key;         // [L][T][N] selection keys, -inf when not eligible
  const float* s;           // [L][T][N] scores
  uint8_t* ranked;          // [L][T][256] candidate lists (tokens with a rejection)
  int32_t* n_el;            // [L][T] list lengths (0 = token not affected)
  int32_t* next;            // [L][T] next candidate position
  uint8_t* changed;         // [L][T] token's slots changed
  int32_t* list0;           // [L][T*K] pending slots, two buffers
  int32_t* list1;
  int32_t* stats;           // [L][2] rerouted, dropped, or nullptr
  const int32_t* flag;      // [L] the layer has an expert over capacity
  CapRound round[kCapGridRounds + 1];  // round[r] = round r+1
  int32_t* list_e;          // [L][T*K] first workgroup round's list: proposed experts
  int32_t* part;            // [rounds][L][accept workgroups][3] rerouted / dropped / pending
  int32_t* segsum;          // [L][nseg][Nb] cleared for the final layout
  int L, T, N, K, Kt, Nb, cap, nseg, nsb, nlb;
  int G, Gk;                // expert groups and groups kept (eligible experts <= Gk*N/G)
};
hipError_t launch_capacity(const CapArgs& c, hipStream_t s);

// Balancing step with rule, moving-average loads and period (one
// workgroup per layer).
hipError_t launch_balance_step(float* bias, const int32_t* counts, int L, int N, int stride,
                               int rule, float step, float alpha, int every, float* loads,
                               int32_t* calls, hipStream_t s);

// Forcible-balance expert ids and hotspot accumulation (elementwise).
hipError_t launch_balanced_indices(int32_t* idx, int L, int T, int K, int N, int n_shared,
                                   int start, hipStream_t s);
hipError_t launch_hotspot_accumulate(int64_t* hot, const int32_t* counts, int L, int N, int stride,
                                     hipStream_t s);

// Experts held per lane by the one-wave-per-token selection.
inline int experts_per_lane(int N) { return N > 128 ? 4 : (N > 64 ? 2 : 1); }

}  // namespace moer
