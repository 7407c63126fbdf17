/*
 * moer.h — C ABI of the MI355X (gfx950) Mixture-of-Experts router.
 *
 * Three calls make up the router's hot path:
 *   moer_route        gate affinities -> scores -> bias-aware group-limited
 *                     top-k -> combine weights -> routing entropy ->
 *                     dispatch layout (counts, offsets, stable permutation);
 *                     optionally a per-expert capacity with rerouting, and
 *                     the two calls below fused in
 *   moer_load_stats   load statistics of the realised per-expert counts
 *   moer_bias_update  sign-step update of the per-expert selection bias
 * and around it:
 *   moer_balance_step        other balancing rules (proportional update,
 *                            moving-average loads, update period)
 *   moer_dispatch /          the single-device dispatch of token rows to their
 *   moer_combine             experts and the weighted combine back
 *   moer_balanced_indices    forcible-balance expert ids (an upper bound)
 *   moer_hotspot_accumulate  per-layer, per-expert token counts over batches
 *
 * The method is the one described on these web pages (cited by title and
 * section throughout):
 *  - "MoE Routing Entropy vs Expert Saturation: Optimizing DeepSeek V4 Load
 *    Balancing" (dailyaiworld.com): section "The Mathematics: Router Entropy
 *    and Gating Imbalance" (h = x·W_g, softmax, Shannon entropy in bits) and
 *    the listing "Dynamic Expert Bias Routing Controller" (top-k,
 *    renormalised weights, per-expert bincount, bias buffer).
 *  - "DeepSeek V4 MoE load balancing" (blog.hotdry.top): token routing and
 *    top-K section (sigmoid gating, weighted combine), auxiliary-loss-free
 *    balancing section (per-expert bias added to the affinity score for the
 *    routing decision; lowered for overloaded, raised for underloaded
 *    experts), DeepEP section (dispatch groups tokens by destination expert).
 *  - "DeepSeek-V3 Group-Limited Expert Routing" (cnnetsun.cn): section 1
 *    (256 experts in 8 groups of 32; keep the best 4 groups; choose 8 experts
 *    among their 128), section 3 (Gate.forward: view the scores as groups,
 *    top-k groups, mask the rest, top-k experts), section 4 (decode: no
 *    group limit; the shared expert counts as a routed slot, 9 per token).
 *  - "A minimal experiment in expert-load imbalance" (tech-blog-chi):
 *    "Run the example" (imbalance = max/mean, capacity = max x experts).
 *  - MindIE "expert parallelism load balancer" (hiascend.com): forcible
 *    balancing replaces the top-k output with supplied indices.
 *
 * Conventions for every call
 *  - All array arguments are DEVICE pointers, owned by the caller, row-major
 *    and contiguous. The library allocates nothing and keeps no state other
 *    than a thread-local error string; scratch memory is the caller's
 *    workspace (size from moer_route_workspace_bytes).
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls only
 *    enqueue work on it and never wait for the device; outputs are valid
 *    once the stream has reached them.
 *  - Arguments are validated on the host before anything is enqueued. On
 *    error nothing is enqueued, the status is returned and moer_last_error()
 *    says why. Nothing throws across this ABI.
 *  - Identical inputs give bitwise-identical outputs (fixed reduction
 *    orders, no floating-point atomics).
 *  - Inputs must be finite; NaN or infinite scores give unspecified (but
 *    memory-safe) results.
 */
#ifndef MOER_H
#define MOER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOER_ABI_VERSION 2
#define MOER_MAX_EXPERTS 256 /* N */
#define MOER_MAX_SLOTS 16    /* Kt = K + n_shared */

typedef enum {
  MOER_OK = 0,
  MOER_EINVAL = 1,       /* invalid argument (see moer_last_error) */
  MOER_EUNSUPPORTED = 2, /* reserved: valid, but a shape the kernels do not take
                            (every descriptor that validates has a kernel today) */
  MOER_EWORKSPACE = 3,   /* workspace missing or smaller than required */
  MOER_EHIP = 4          /* the HIP runtime refused a launch */
} moer_status;

typedef enum {
  MOER_SOFTMAX = 0, /* p_e = exp(h_e) / sum_j exp(h_j)  (dailyaiworld, Mathematics) */
  MOER_SIGMOID = 1  /* s_e = 1 / (1 + exp(-h_e))        (hotdry, token routing)    */
} moer_score_fn;

typedef enum { MOER_BF16 = 0, MOER_F32 = 1 } moer_dtype;

typedef enum {
  MOER_BIAS_SCORE = 0, /* key = s + b for the selection only; weights and
                          entropy from the unbiased scores (hotdry,
                          auxiliary-loss-free balancing) */
  MOER_BIAS_LOGIT = 1  /* b added to the logits: scores, selection, weights
                          and entropy all from h + b (dailyaiworld listing
                          "Dynamic Expert Bias Routing Controller"); HIDDEN
                          input only */
} moer_bias_mode;

typedef enum {
  MOER_RULE_SIGN = 0,        /* b_e += step * sign(mean - load_e)          */
  MOER_RULE_PROPORTIONAL = 1 /* b_e -= step * (load_e - mean) / mean       */
} moer_bias_rule;

typedef enum {
  MOER_IN_HIDDEN = 0,  /* x and W_g given: full path from the gate GEMM      */
  MOER_IN_SCORES = 1,  /* fp32 scores s [L][T][N] given: the GEMM is skipped */
  MOER_IN_INDICES = 2  /* expert ids idx_in [L][T][Kt] given (MindIE's
                          forcible balancing): only the layout is built      */
} moer_input;

/* Shape of one call. n_layers independent routers (each with its own x,
 * W_g and bias) are processed by one call. */
typedef struct {
  int32_t n_layers;    /* L >= 1 */
  int32_t T;           /* tokens per layer, >= 0 (0 = empty batch) */
  int32_t d;           /* hidden size (HIDDEN mode); bf16 needs d % 8 == 0 */
  int32_t N;           /* routed experts, 1..256 */
  int32_t K;           /* routed experts chosen per token, 1..N */
  int32_t n_groups;    /* G: N/G contiguous experts per group (any N/G >= 2 that
                          divides N); 1 = no limit */
  int32_t topk_groups; /* Gk: groups kept per token, 1..G, Gk*(N/G) >= K */
  int32_t n_shared;    /* shared-expert slots appended after the K routed */
  int32_t score_fn;    /* moer_score_fn */
  int32_t dtype;       /* moer_dtype of x and W_g (HIDDEN mode) */
  int32_t input;       /* moer_input */
  int32_t bias_mode;   /* moer_bias_mode (0 = MOER_BIAS_SCORE) */
  int32_t capacity;    /* 0 = unlimited; else the most assignments a routed
                          expert takes per layer (dailyaiworld, production
                          testing: 1.25 x T*K/N, rounded up). Slots beyond it
                          move to the token's next candidates, in rounds (see
                          moer_route); HIDDEN or SCORES input */
} moer_route_desc;

/* Per-layer record written by moer_load_stats (device memory, 64 bytes). */
typedef struct {
  int64_t total;      /* sum of counts over the N routed experts */
  int64_t max_load;   /* largest count */
  int64_t argmax;     /* expert with the largest count (lowest id on ties) */
  int64_t capacity;   /* max_load * N: fixed per-expert capacity that fits */
  double mean;        /* total / N */
  double imbalance;   /* max_load / mean, 0 when mean == 0 */
  double h_load_bits; /* entropy (bits) of counts/total, 0 when total == 0 */
  double cv;          /* population std of counts / mean, 0 when mean == 0 */
} moer_load_stats_t;

/* Buffers of one call (device pointers; Kt = K + n_shared, Nb = N + n_shared).
 * "req" = required in the modes that produce it; "opt" = may be NULL. */
typedef struct {
  const void* x;             /* HIDDEN: [L][T][d] bf16 or fp32 hidden states;
                                bf16: 16-byte aligned */
  const void* w_gate;        /* HIDDEN: [L][N][d] gate weights, same dtype;
                                row e is expert e's vector (nn.Linear layout);
                                bf16: 16-byte aligned */
  const float* scores;       /* SCORES: [L][T][N] fp32 scores s (or p),
                                16-byte aligned */
  const int32_t* idx_in;     /* INDICES: [L][T][Kt] expert ids; ids outside
                                [0, Nb) are not placed (see perm) */
  const float* bias;         /* opt [L][N] fp32 selection bias b_e (NULL = 0),
                                16-byte aligned */
  const float* logit_offset; /* opt [N] fp32 added to every layer's h (HIDDEN),
                                16-byte aligned */
  float* h_out;              /* opt [L][T][N] fp32 affinities h (HIDDEN) */
  float* topk_w;             /* req [L][T][Kt] combine weights (not INDICES) */
  float* tok_entropy;        /* opt [L][T] per-token routing entropy, bits */
  float* agg_entropy;        /* opt [L] entropy of the batch-mean distribution */
  int32_t* topk_idx;         /* req [L][T][Kt] expert ids (not INDICES) */
  int32_t* counts;           /* req [L][Nb] assignments per expert */
  int32_t* offsets;          /* req [L][Nb+1] exclusive prefix of counts;
                                offsets[Nb] = assignments placed */
  int32_t* perm;             /* req [L][T*Kt] flat slot ids t*Kt+k ordered by
                                (expert, token, slot); positions past
                                offsets[Nb] hold -1 */
  int32_t* inv_perm;         /* opt [L][T*Kt] position of each slot in perm,
                                -1 for ids that were not placed */
  void* ev_gemm_begin;       /* opt hipEvent_t pair for profiling the gate  */
  void* ev_gemm_end;         /* GEMM: the bf16 kernel's launch records them
                                at its own start and end (the dispatch's
                                timestamps); other gate kernels are
                                bracketed by records on the stream. Routers
                                of at most 16 experts whose GEMM and
                                selection share one launch: that launch's
                                start and end */
  moer_load_stats_t* load_stats; /* opt [L]: what moer_load_stats gives for this
                                    call's counts (fused, no extra launch) */
  float* bias_update;        /* opt [L][N]: moer_bias_update applied in place
                                with this call's counts and step bias_update_u,
                                after the selection has read `bias` (so it may
                                be the same buffer): the auxiliary-loss-free
                                balancing step of one training iteration */
  float bias_update_u;       /* step u >= 0 for bias_update */
  int32_t* cap_stats;        /* opt [L][2] with a capacity: slots placed on
                                another expert than their first choice, and
                                slots dropped (no candidate left) */
  void* ev_select_wait;      /* opt hipEvent_t: the selection (and everything
                                after it) waits for this event, the gate GEMM
                                does not. Lets a loop overlap the next batch's
                                GEMM with this batch's selection and layout:
                                call i+1 on a second stream, with its own
                                workspace, waiting for an event recorded after
                                call i (whose bias update it then sees) */
} moer_route_io;


/* Bytes of workspace moer_route needs for `desc` (0 on an invalid desc). */
size_t moer_route_workspace_bytes(const moer_route_desc* desc);

/* The router: for each layer l and token t
 *   h      = x[t] . W_g^T (+ logit_offset)         fp32 accumulation (MFMA)
 *   s      = softmax(h) or sigmoid(h)              (or the given scores)
 *   key_e  = s_e + b_e                             fp32, selection only
 *   if G > 1: group score = sum of the group's two largest keys; keep the
 *             Gk best groups (score desc, group id asc); others ineligible
 *   slots 0..K-1 = the K best eligible keys (key desc, expert id asc)
 *   slots K..Kt-1 = shared experts N..Nb-1 with weight 1
 *   w_k    = s_k / sum of the chosen s            (unbiased scores)
 *   tok_entropy = entropy (bits) of s / sum_e s over the N experts
 *   agg_entropy = entropy (bits) of the mean over tokens of s / sum_e s
 * then the dispatch layout over Nb buckets (counts, offsets, perm,
 * inv_perm), stable in (token, slot) order within an expert.
 * With desc->capacity = c > 0 the routed slots are then limited to c per
 * expert, in rounds: round 0 is the top-K above; in every round an expert
 * accepts that round's proposals in (token, slot) order while it holds
 * fewer than c, and each rejected slot proposes its token's next eligible
 * candidate (decision order; a token's rejected slots in slot order) in the
 * next round, or is dropped (id -1, weight 0) when none is left. Slots keep
 * their positions; the weights are renormalised over the placed routed
 * slots; entropies are those of the scores; the layout, load statistics and
 * bias update use the final ids.
 * Workspace: device memory of at least moer_route_workspace_bytes(desc)
 * bytes, any contents; it is clobbered. Returns MOER_OK or an error status
 * (MOER_EINVAL also for a pointer below 16-byte alignment where the field
 * above asks for it).
 * Kernel choice (results are the same up to the rounding of h, bit for bit
 * where only the selection kernel differs); environment variables, read at
 * every call, override it for testing and profiling:
 *   MOER_ROUTE_SMALL=0  routers of at most 16 experts use the separate gate
 *                       GEMM and selection launches instead of one launch;
 *   MOER_ROUTE_TINY=0   batches of fewer than 256 blocks of 64 tokens use
 *                       64-token selection workgroups instead of 16 or 32;
 *   MOER_ROUTE_WHOLE=0  layers of at most 64 tokens (routers of at most 8
 *                       experts) or 32 (at most 16) with d at most 512 (bf16)
 *                       or 256 (fp32) keep a separate layout launch instead
 *                       of one workgroup per layer that also writes the
 *                       layout outputs;
 *   MOER_ROUTE_FUSED=1|2|3  the co-resident fused pass for the large bf16
 *                       routers it takes (off by default: slower here). */
moer_status moer_route(const moer_route_desc* desc, const moer_route_io* io,
                       void* workspace, size_t workspace_bytes, void* stream);

/* moer_route for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same call and results, with the scratch memory taken from a static array
 * of MOER_NOALLOC_SCRATCH_BYTES that each GPU holds from the library's load
 * until the process ends, instead of a caller workspace. Nothing is
 * allocated or freed. Every call on a GPU shares that GPU's array: calls
 * that overlap on one GPU (on different streams, or from different threads)
 * race and give undefined results. The first call on a device looks the
 * array up on that device (the current device; the stream, if not NULL,
 * must belong to it). Returns MOER_EWORKSPACE when the router needs more
 * scratch than the array holds (moer_route_workspace_bytes(desc) >
 * MOER_NOALLOC_SCRATCH_BYTES: e.g. a capacity limit on a large batch),
 * MOER_EINVAL for a stream of another device, else as moer_route. */
#define MOER_NOALLOC_SCRATCH_BYTES ((size_t)40 << 20)
moer_status moer_route_noalloc(const moer_route_desc* desc, const moer_route_io* io,
                               void* stream);

/* Load statistics ("A minimal experiment in expert-load imbalance", Run the
 * example; entropy per the dailyaiworld Mathematics section; std/mean per
 * the hotdry deployment section) of counts[l*stride + e], e < N, for each of
 * n_layers layers, written to out_dev[l] (device memory). stride >= N. */
moer_status moer_load_stats(const int32_t* counts, int32_t n_layers, int32_t N,
                            int32_t stride, moer_load_stats_t* out_dev, void* stream);

/* Sign-step bias update (hotdry, auxiliary-loss-free balancing), in place:
 *   bias[l*N + e] += u * sign(mean_l - counts[l*stride + e])
 * with mean_l = (sum_e counts) / N compared exactly (in integers) and
 * sign(0) = 0; one fp32 rounding per expert. stride >= N. */
moer_status moer_bias_update(float* bias, const int32_t* counts, int32_t n_layers,
                             int32_t N, int32_t stride, float u, void* stream);

/* Local dispatch (hotdry "DeepSeek V4 MoE load balancing", DeepEP section:
 * dispatch carries each token to the experts it was routed to; on one device
 * that is a gather into the layout's expert-contiguous order). For every
 * layer l, token t and slot k whose position p = inv_perm[l][t*Kt + k] lies
 * in [0, T*Kt):
 *   x_out[l][p] = x[l][t]        (a row of row_bytes bytes, copied as is)
 * so the rows of expert e end up at offsets[e] .. offsets[e+1]-1, tokens
 * ascending. Rows of x_out that no slot names are not written.
 *   x        [L][T] rows of row_bytes, device, 16-byte aligned
 *   inv_perm [L][T*Kt] int32, device (moer_route's inv_perm); entries that
 *            are negative or >= T*Kt are skipped
 *   x_out    [L][T*Kt] rows of row_bytes, device, 16-byte aligned; must not
 *            overlap x
 * row_bytes > 0 and a multiple of 16; 1 <= Kt <= 16; T*Kt < 2^31. Reads each
 * x row once and writes Kt rows. MOER_EINVAL on a bad argument. */
moer_status moer_dispatch(const void* x, int64_t row_bytes, int32_t n_layers, int32_t T,
                          int32_t Kt, const int32_t* inv_perm, void* x_out, void* stream);

/* Weighted combine (hotdry, token routing section: the layer output is the
 * sum of the chosen experts' outputs weighted by the routing weights; DeepEP
 * section: combine returns them to token order):
 *   y[l][t] = sum over slots k of token t with a position p (as in
 *             moer_dispatch) of w[l][t][k] * expert_out[l][p]
 * accumulated in fp32 in slot order (one fused multiply-add per term),
 * rounded once to y's dtype (bf16: round to nearest even). A token with no
 * placed slot gets a zero row.
 *   expert_out [L][T*Kt][d] in out_dtype (MOER_BF16 or MOER_F32), device,
 *              16-byte aligned: one expert-output row per layout position
 *   w          [L][T][Kt] fp32 (moer_route's topk_w; shared slots weigh 1)
 *   inv_perm   [L][T*Kt] int32, as in moer_dispatch
 *   y          [L][T][d] in y_dtype (MOER_BF16 or MOER_F32), device,
 *              16-byte aligned; must not overlap the inputs
 * d > 0 and a multiple of 8; 1 <= Kt <= 16; T*Kt < 2^31. Reads Kt rows and
 * writes one row per token. MOER_EINVAL on a bad argument. */
moer_status moer_combine(const void* expert_out, moer_dtype out_dtype, const float* w,
                         const int32_t* inv_perm, int32_t n_layers, int32_t T, int32_t Kt,
                         int32_t d, void* y, moer_dtype y_dtype, void* stream);

/* Forcible load balancing (MindIE "expert parallelism load balancer":
 * the top-k output replaced by indices that balance the experts exactly, an
 * upper bound for load balancing; not a routing decision). Writes
 *   idx[l][t][k] = (t*K + k + first) mod N      for k < K
 *   idx[l][t][K + j] = N + j                     for the n_shared shared slots
 * into idx [L][T][K + n_shared] int32 (device), ready for moer_route's
 * INDICES mode. Every expert gets T*K/N assignments per layer (within one);
 * a token's K routed ids are distinct. 1 <= K <= N <= 256, K + n_shared <=
 * 16, T*(K + n_shared) < 2^31; `first` is any integer (taken mod N). */
moer_status moer_balanced_indices(int32_t* idx, int32_t n_layers, int32_t T, int32_t K, int32_t N,
                                  int32_t n_shared, int32_t first, void* stream);

/* Expert hotspot collection (MindIE balancer: per layer and expert, the
 * number of tokens the expert processed): hot[l][e] += counts[l*stride + e]
 * for e < N. hot [L][N] int64 and counts (e.g. moer_route's [L][Nb]) are
 * device memory; stride >= N. Call once per batch; copy `hot` to the host
 * whenever a hotspot table is written. */
moer_status moer_hotspot_accumulate(int64_t* hot, const int32_t* counts, int32_t n_layers,
                                    int32_t N, int32_t stride, void* stream);

/* Balancing rule with smoothing and a period (dailyaiworld listing:
 * proportional update with a decay factor; hotdry auxiliary-loss-free
 * section: direction-only update, loads smoothed by a moving average, the
 * bias updated every so many steps). */
typedef struct {
  int32_t rule;  /* moer_bias_rule */
  float step;    /* u (SIGN) or the decay factor gamma (PROPORTIONAL), >= 0 */
  float alpha;   /* moving-average weight of the new counts, in (0, 1];
                    1 = the loads are this call's counts */
  int32_t every; /* apply the rule on every `every`-th call, >= 1 */
} moer_balance_cfg;

/* One balancing step per layer l (one call per training step):
 *   loads[l][e] = counts[l][e]                             on the first call
 *                 (calls[l] == 0) or when loads is NULL,
 *               = alpha*counts + (1-alpha)*loads[l][e]     otherwise (fp32,
 *                 two products and a sum, no fused multiply-add)
 *   if (calls[l] + 1) % every == 0:
 *     mean = (sum over e < N of loads[l][e], in fp64, ascending e) / N
 *     SIGN:         bias[l][e] += step * sign(mean - loads[l][e])
 *     PROPORTIONAL: bias[l][e] -= (float)(step * ((loads[l][e] - mean)
 *                   / mean)) (fp64, one rounding), no change when mean == 0
 *   calls[l] += 1
 * bias [L][N] fp32, in place; counts [L][stride] int32 (stride >= N, e.g.
 * moer_route's counts); loads [L][N] fp32 caller state (required when
 * alpha < 1); calls [L] int32 caller state (required when every > 1). Zero
 * both before the first call. With alpha = 1, every = 1 and SIGN this is
 * moer_bias_update (the comparison agrees with the integer one). */
moer_status moer_balance_step(float* bias, const int32_t* counts, int32_t n_layers, int32_t N,
                              int32_t stride, const moer_balance_cfg* cfg, float* loads,
                              int32_t* calls, void* stream);

const char* moer_status_str(moer_status status);
const char* moer_last_error(void);
int moer_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOER_H */
