/*
 * moero.h — CPU oracle for the Mixture-of-Experts router.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link or
 * call this code: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it. It shares no code with the HIP library.
 *
 * Plain, slow and obviously correct: fp64 wherever the pages do not fix a
 * precision; fp32 only where the routing decision itself is defined on fp32
 * values (selection keys, group scores, the bias update), so that a GPU given
 * the same fp32 scores must reproduce the decision bit for bit.
 *
 * Sources (the five web pages the method is described on):
 *  [P1] dailyaiworld.com, "MoE Routing Entropy vs Expert Saturation:
 *       Optimizing DeepSeek V4 Load Balancing" — section "The Mathematics:
 *       Router Entropy and Gating Imbalance" (logits h = x·W_g, softmax,
 *       Shannon routing entropy in bits) and the code listing "Dynamic Expert
 *       Bias Routing Controller" (top-k, renormalisation, bincount, bias).
 *  [P2] blog.hotdry.top, "DeepSeek V4 MoE load balancing" — sections on
 *       token routing / top-K (sigmoid gating, weighted combine) and on
 *       auxiliary-loss-free balancing (per-expert bias added to the affinity
 *       score for the routing decision; lowered when overloaded, raised when
 *       underloaded); deployment section (std/mean of activation frequency).
 *  [P3] cnnetsun.cn, "DeepSeek-V3 Group-Limited Expert Routing" — section 1
 *       (256 experts in 8 groups of 32, keep the best 4 groups, pick 8 of
 *       their 128), section 3 (Gate.forward: view scores as groups, top-k
 *       groups, mask the other groups, top-k experts), section 4 (decode:
 *       no groups, the shared expert counted as a routed slot, 9 per token).
 *  [P4] tech-blog-chi.vercel.app, "A minimal experiment in expert-load
 *       imbalance" — "Run the example" (total, mean, max/mean imbalance,
 *       capacity = max·N) and "Expected output" (the worked example).
 *  [P5] hiascend.com, MindIE "expert parallelism load balancer" — forcible
 *       load balancing: replace the top-k output by supplied indices.
 */
#ifndef MOERO_H
#define MOERO_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MOERO_SOFTMAX = 0, MOERO_SIGMOID = 1 };

typedef struct {
  int32_t T;            /* tokens */
  int32_t N;            /* routed experts */
  int32_t K;            /* routed experts chosen per token */
  int32_t n_groups;     /* G: contiguous expert groups (1 = no group limit) */
  int32_t topk_groups;  /* Gk: groups kept per token */
  int32_t n_shared;     /* shared-expert slots appended after the K routed */
} moero_cfg;

typedef struct {
  int64_t total, max_load, argmax, capacity;
  double mean, imbalance, h_load_bits, cv;
} moero_stats;

/* Gate affinities, [P1] Mathematics: h[t][e] = sum_k x[t][k]*W[e][k] (+ o[e]).
 * x [T][d], W [N][d] (fp32 holding exactly the bf16/fp32 input values),
 * offset [N] or NULL; h [T][N] fp64, summed in ascending k. */
void moero_affinities(const float* x, const float* W, const float* offset,
                      int32_t T, int32_t d, int32_t N, double* h);

/* Scores from affinities: softmax over experts ([P1] Mathematics) or the
 * element-wise logistic sigmoid ([P2] routing section). fp64 in and out. */
void moero_scores(const double* h, int32_t T, int32_t N, int32_t score_fn, double* s);

/* Selection for every token ([P3] s.1/s.3/s.4, [P2] bias, [P1] renorm).
 * s32 [T][N]: the fp32 scores the decision is taken on; s64 [T][N]: the same
 * scores at full precision (weights, entropy); bias [N] or NULL.
 * Outputs (each may be NULL): idx [T][Kt] int32, w [T][Kt] fp32,
 * tok_H [T] fp64 bits, gap [T] fp64 (smallest score margin that decides the
 * selection or its order; +inf when nothing competes). Returns 0, or -1 when
 * the configuration is invalid. */
int moero_select(const moero_cfg* cfg, const float* s32, const double* s64,
                 const float* bias, int32_t* idx, float* w, double* tok_H,
                 double* gap);

/* Capacity-limited routing ([P1] production testing section: a hard token
 * capacity per expert; the excess goes to secondary candidates). Rounds of
 * proposals: round 0 proposes each token's top-K; each round, an expert
 * accepts proposals in (token, slot) order while it holds fewer than cap;
 * a rejected slot proposes the token's next eligible candidate (decision
 * order of moero_select) in the next round, or is dropped (id -1, weight 0)
 * when none is left. Slots keep their positions; shared slots are not
 * limited. Weights: unbiased scores of the placed routed slots renormalised.
 * Inputs as moero_select; outputs idx, w [T][Kt] (nullable), and the counts
 * of rerouted and dropped slots. Returns -1 on an invalid configuration. */
int moero_capacity_route(const moero_cfg* cfg, const float* s32, const double* s64,
                         const float* bias, int32_t cap, int32_t* idx, float* w,
                         int64_t* n_rerouted, int64_t* n_dropped);

/* Aggregate routing entropy ([P1] Mathematics and compute_routing_entropy):
 * the entropy in bits of the batch-mean of the per-token distributions
 * q[t][e] = s[t][e] / sum_e s[t][e]. 0 for T == 0. */
double moero_agg_entropy(const double* s64, int32_t T, int32_t N);

/* Dispatch layout over Nb buckets for idx [T][Kt]: counts [Nb], exclusive
 * offsets [Nb+1], perm [T*Kt] ordered by (expert, token, slot) holding flat
 * slot ids t*Kt+k, and inv_perm [T*Kt] (may be NULL). Entries outside
 * [0, Nb) are not placed; their inv_perm is -1 and the unused tail of perm
 * is -1. */
void moero_layout(const int32_t* idx, int32_t T, int32_t Kt, int32_t Nb,
                  int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm);

/* Load statistics over routed experts [P4] Run the example, [P1] entropy,
 * [P2] deployment section (std/mean). */
void moero_load_stats(const int32_t* counts, int32_t N, moero_stats* out);

/* Sign-step bias update ([P2] auxiliary-loss-free balancing):
 * b[e] += u * sign(mean_load - load[e]), sign(0) = 0, in fp32. */
void moero_bias_update(float* bias, const int32_t* counts, int32_t N, float u);

/* Local dispatch ([P2] DeepEP section: tokens go to the experts they were
 * routed to, grouped by destination; on one device that is a gather into
 * expert-contiguous order). For every position pos of the layout with
 * perm[pos] >= 0, row pos of x_out is the row of token perm[pos] / Kt of x.
 * Rows are row_bytes bytes (copied, not converted); rows whose perm entry is
 * -1 are not written. */
void moero_dispatch(const void* x, int64_t row_bytes, int32_t T, int32_t Kt,
                    const int32_t* perm, void* x_out);

/* Weighted combine ([P2] token routing: the layer output is the sum of the
 * chosen experts' outputs weighted by the routing weights; [P2] DeepEP
 * section: combine returns them to token order). out [T*Kt][d] holds one
 * expert-output row per layout position (fp64 copies of the exact values),
 * w [T][Kt] the fp32 weights: y[t] = sum over the slots k of token t that
 * have a position (perm[pos] == t*Kt + k) of w[t][k] * out[pos], in fp64.
 * A slot with no position contributes nothing. */
void moero_combine(const double* out, const float* w, const int32_t* perm,
                   int32_t T, int32_t Kt, int32_t d, double* y);

/* Forcible load balancing ([P5]: the top-k output is replaced by indices
 * that load every expert equally, as an upper bound for balancing): slot k
 * < K of token t gets expert (t*K + k + first) mod N, the n_shared shared
 * slots get N..N+n_shared-1. idx is [T][K + n_shared]. */
void moero_balanced_indices(int32_t T, int32_t K, int32_t N, int32_t n_shared, int32_t first,
                            int32_t* idx);

/* Expert hotspot collection ([P5]: per layer and expert, the number of
 * tokens the expert processed): hot[l][e] += counts[l*stride + e] for
 * e < N, over n_layers layers. */
void moero_hotspot_accumulate(int64_t* hot, const int32_t* counts, int32_t n_layers, int32_t N,
                              int32_t stride);

/* Logit-space selection bias ([P1] listing "Dynamic Expert Bias Routing
 * Controller": the bias is added to the raw logits, and the scores, the
 * top-k, the weights and the entropy all come from the compensated logits):
 * h[t][e] += b[e] in fp64. */
void moero_logit_bias(double* h, const float* b, int32_t T, int32_t N);

/* One balancing step with a selectable rule, smoothing and period
 * ([P1] listing: proportional update; [P2] auxiliary-loss-free section:
 * sign-style direction, moving-average load statistics, update period).
 *   loads: l_e = counts_e on the first call (calls == 0 or loads NULL),
 *          else l_e = alpha*counts_e + (1-alpha)*l_e (fp32, no fused ops);
 *   rule, on every `every`-th call (calls+1 divisible by every):
 *     mean = (sum over e of l_e, in fp64, ascending e) / N
 *     SIGN (0):         b_e += step * sign(mean - l_e)          (fp32 add)
 *     PROPORTIONAL (1): b_e -= (float)(step * ((l_e - mean) / mean)) when
 *                       mean > 0 (fp64 divide and multiply, one rounding to
 *                       fp32, then the fp32 subtraction)
 *   *calls += 1 (when calls is not NULL).
 * counts [N] int32; loads [N] fp32 state or NULL (then alpha must be 1);
 * calls: one counter or NULL (then every must be 1). */
void moero_balance_step(float* bias, const int32_t* counts, int32_t N, int32_t rule, float step,
                        float alpha, int32_t every, float* loads, int32_t* calls);

int moero_num_threads(void);
/* Threads the OpenMP loops use from now on (timing at one core). */
void moero_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
