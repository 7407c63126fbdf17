/*
 * moero.c — CPU oracle for the Mixture-of-Experts router.
 *
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
 * CPU-baseline leg call it; the product path never does. It shares no code,
 * header or table with the HIP library. Build: gcc -O2 -fopenmp
 * -ffp-contract=off (no fused multiply-add, no fast-math), so every fp32
 * operation below is one IEEE rounding.
 *
 * Each function follows the steps of the method in the order the pages give
 * them; the page and section are named above each one (see moero.h for the
 * page list [P1]..[P5]).
 *
 * Pinning (what checks this file against something other than itself) is
 * done by the CPU tests: the [P4] worked example, entropy closed forms,
 * brute-force enumeration of group-limited top-k, library special cases
 * (fp64 matmul/softmax/sigmoid/stable sort), the bias closed form, and for
 * dispatch/combine the bucket-membership properties and the closed form of a
 * combine over experts that only scale their rows.
 */
#include "moero.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int moero_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void moero_set_num_threads(int n) {
#ifdef _OPENMP
  omp_set_num_threads(n > 0 ? n : 1);
#else
  (void)n;
#endif
}

/* [P1] Mathematics: routing logits h_i = x·W_g, with W_g's rows the expert
 * vectors ([P2] routing: similarity of the hidden state with every expert's
 * embedding vector). The optional per-expert offset is added to the logit
 * (used to plant "celebrity" experts). */
void moero_affinities(const float* x, const float* W, const float* offset,
                      int32_t T, int32_t d, int32_t N, double* h) {
#pragma omp parallel for schedule(static)
  for (int32_t t = 0; t < T; ++t) {
    const float* xt = x + (size_t)t * d;
    for (int32_t e = 0; e < N; ++e) {
      const float* we = W + (size_t)e * d;
      double acc = 0.0;
      for (int32_t k = 0; k < d; ++k) acc += (double)xt[k] * (double)we[k];
      if (offset) acc += (double)offset[e];
      h[(size_t)t * N + e] = acc;
    }
  }
}

/* [P1] Mathematics: p(e_i|x) = exp(h_i) / sum_j exp(h_j) (evaluated with the
 * row maximum subtracted, which leaves p unchanged); [P2] routing: sigmoid
 * gating s_i = 1 / (1 + exp(-h_i)), element-wise. */
void moero_scores(const double* h, int32_t T, int32_t N, int32_t score_fn, double* s) {
#pragma omp parallel for schedule(static)
  for (int32_t t = 0; t < T; ++t) {
    const double* ht = h + (size_t)t * N;
    double* st = s + (size_t)t * N;
    if (score_fn == MOERO_SOFTMAX) {
      double m = ht[0];
      for (int32_t e = 1; e < N; ++e) m = ht[e] > m ? ht[e] : m;
      double z = 0.0;
      for (int32_t e = 0; e < N; ++e) { st[e] = exp(ht[e] - m); z += st[e]; }
      for (int32_t e = 0; e < N; ++e) st[e] /= z;
    } else {
      for (int32_t e = 0; e < N; ++e) st[e] = 1.0 / (1.0 + exp(-ht[e]));
    }
  }
}

/* Ranking record: a value with the id it belongs to. Order: value
 * descending, id ascending on equal values (the tie rule; -0 equals +0). */
typedef struct { float v; int32_t id; } ranked;

static int by_value_desc_id_asc(const void* pa, const void* pb) {
  const ranked* a = (const ranked*)pa;
  const ranked* b = (const ranked*)pb;
  if (a->v > b->v) return -1;
  if (a->v < b->v) return 1;
  return (a->id > b->id) - (a->id < b->id);
}

/* Shannon entropy in bits of the distribution q_e = s_e / sum_e s_e
 * ([P1] Mathematics: H(P) = -sum p log2 p), with 0·log 0 = 0. */
static double entropy_bits_of(const double* s, int32_t N) {
  double z = 0.0;
  for (int32_t e = 0; e < N; ++e) z += s[e];
  if (!(z > 0.0)) return 0.0;
  double H = 0.0;
  for (int32_t e = 0; e < N; ++e) {
    double q = s[e] / z;
    if (q > 0.0) H -= q * log2(q);
  }
  return H;
}

static int cfg_valid(const moero_cfg* c) {
  if (c->T < 0 || c->N < 1 || c->K < 1 || c->K > c->N) return 0;
  if (c->n_groups < 1 || c->N % c->n_groups != 0) return 0;
  if (c->topk_groups < 1 || c->topk_groups > c->n_groups) return 0;
  if (c->n_groups > 1 && c->N / c->n_groups < 2) return 0;
  if (c->topk_groups * (c->N / c->n_groups) < c->K) return 0;
  if (c->n_shared < 0) return 0;
  return 1;
}

/* Steps 1-3 of the per-token decision (see moero_select): the biased
 * keys, the group-limited eligibility, and the eligible experts ranked by
 * (key descending, id ascending) into cand[0..n). Returns n; lowers
 * *margin to the gap between the Gk-th and the next group score. */
static int32_t rank_token(const float* st, const float* bias, int32_t N, int32_t G, int32_t Gk,
                          ranked* cand, ranked* grp, ranked* mem, float* key, char* kept,
                          double* margin) {
  const int32_t gsz = N / G;
  /* 1. biased keys */
  for (int32_t e = 0; e < N; ++e) {
    volatile float k = st[e] + (bias ? bias[e] : 0.0f);
    key[e] = k + 0.0f;
  }
  /* 2. group-limited eligibility */
  if (G > 1) {
    for (int32_t g = 0; g < G; ++g) {
      for (int32_t j = 0; j < gsz; ++j) {
        mem[j].v = key[g * gsz + j];
        mem[j].id = g * gsz + j;
      }
      qsort(mem, (size_t)gsz, sizeof(ranked), by_value_desc_id_asc);
      volatile float gs = mem[0].v + mem[1].v;
      grp[g].v = gs + 0.0f;
      grp[g].id = g;
    }
    qsort(grp, (size_t)G, sizeof(ranked), by_value_desc_id_asc);
    memset(kept, 0, (size_t)G);
    for (int32_t r = 0; r < Gk; ++r) kept[grp[r].id] = 1;
    if (Gk < G) {
      double dg = (double)grp[Gk - 1].v - (double)grp[Gk].v;
      if (dg < *margin) *margin = dg;
    }
  } else {
    kept[0] = 1;
  }
  /* 3. eligible experts, ranked */
  int32_t n_el = 0;
  for (int32_t e = 0; e < N; ++e) {
    if (kept[e / gsz]) { cand[n_el].v = key[e]; cand[n_el].id = e; ++n_el; }
  }
  qsort(cand, (size_t)n_el, sizeof(ranked), by_value_desc_id_asc);
  return n_el;
}

/* Per-token routing decision.
 *  1. key_e = s_e + b_e in fp32 ([P2] auxiliary-loss-free balancing: the
 *     bias is added to the affinity score for the routing decision only);
 *     -0 is made +0 so that equal keys compare equal bit for bit.
 *  2. With G > 1 groups ([P3] s.1, s.3): view the N keys as G contiguous
 *     groups of N/G; a group's score is the fp32 sum of its two largest keys;
 *     keep the Gk best groups (score descending, group id ascending); experts
 *     of the other groups cannot be chosen.
 *  3. Top-K of the eligible keys, key descending, expert id ascending on
 *     ties ([P1] torch.topk in the listing; [P3] s.3 final top-k); slots hold
 *     the experts in that order.
 *  4. Shared experts ([P3] s.4: counted as routed slots) take slots K..Kt-1
 *     with ids N..N+n_shared-1 and weight 1.
 *  5. Weights: the chosen experts' unbiased scores renormalised to sum 1
 *     ([P1] listing: renormalise top-k weights; [P2] routing: weighted sum
 *     by affinity), in fp64, stored as fp32.
 *  6. Per-token entropy of q = s / sum s over the N routed experts.
 *  7. Decision margin ("gap"): the smallest of the K-th minus (K+1)-th
 *     eligible key, the Gk-th minus (Gk+1)-th group score, and the key gaps
 *     between adjacent slots — the distance to a different answer. */
int moero_select(const moero_cfg* cfg, const float* s32, const double* s64,
                 const float* bias, int32_t* idx, float* w, double* tok_H,
                 double* gap) {
  if (!cfg_valid(cfg)) return -1;
  const int32_t T = cfg->T, N = cfg->N, K = cfg->K, G = cfg->n_groups;
  const int32_t Gk = cfg->topk_groups, Kt = K + cfg->n_shared;
  const int32_t gsz = N / G;
  int failed = 0;
#pragma omp parallel
  {
    ranked* cand = (ranked*)malloc(sizeof(ranked) * (size_t)N);
    ranked* grp = (ranked*)malloc(sizeof(ranked) * (size_t)G);
    ranked* mem = (ranked*)malloc(sizeof(ranked) * (size_t)gsz);
    float* key = (float*)malloc(sizeof(float) * (size_t)N);
    char* kept = (char*)malloc((size_t)G);
    if (!cand || !grp || !mem || !key || !kept) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(static)
      for (int32_t t = 0; t < T; ++t) {
        const float* st = s32 + (size_t)t * N;
        const double* sd = s64 + (size_t)t * N;
        double margin = INFINITY;
        const int32_t n_el = rank_token(st, bias, N, G, Gk, cand, grp, mem, key, kept, &margin);
        for (int32_t k = 0; k + 1 < K; ++k) {
          double dk = (double)cand[k].v - (double)cand[k + 1].v;
          if (dk < margin) margin = dk;
        }
        if (n_el > K) {
          double dk = (double)cand[K - 1].v - (double)cand[K].v;
          if (dk < margin) margin = dk;
        }
        /* 5. renormalised unbiased weights */
        double z = 0.0;
        for (int32_t k = 0; k < K; ++k) z += sd[cand[k].id];
        for (int32_t k = 0; k < K; ++k) {
          if (idx) idx[(size_t)t * Kt + k] = cand[k].id;
          if (w) w[(size_t)t * Kt + k] = (float)(z > 0.0 ? sd[cand[k].id] / z : 1.0 / K);
        }
        /* 4. shared slots */
        for (int32_t j = 0; j < cfg->n_shared; ++j) {
          if (idx) idx[(size_t)t * Kt + K + j] = N + j;
          if (w) w[(size_t)t * Kt + K + j] = 1.0f;
        }
        /* 6. per-token entropy */
        if (tok_H) tok_H[t] = entropy_bits_of(sd, N);
        if (gap) gap[t] = margin;
      }
    }
    free(cand); free(grp); free(mem); free(key); free(kept);
  }
  return failed ? -1 : 0;
}

/* Capacity-limited routing ([P1] production testing: a hard per-expert
 * token capacity, 1.25 x T*K/N in the page's setting; tokens beyond it go
 * to their next candidate experts). Read here as rounds of proposals:
 *  - every token's candidates are its eligible experts in decision order
 *    (steps 1-3 of moero_select); round 0 proposes its top-K (slot k ->
 *    candidate k);
 *  - in each round an expert accepts that round's proposals in (token,
 *    slot) order while it holds fewer than `cap` assignments, and rejects
 *    the rest; accepted assignments are never revisited;
 *  - a rejected slot proposes the token's next unused candidate (a token's
 *    rejected slots take them in slot order) in the next round, or is
 *    dropped (id -1, weight 0) when none is left;
 *  - rounds repeat until nothing is pending.
 * Slot k keeps its position; shared slots are not limited (ids N+j,
 * weight 1). Weights are the placed routed slots' unbiased scores
 * renormalised (fp64, stored as fp32; 1/n_placed when they sum to 0).
 * Writes idx [T][Kt], w [T][Kt] (either may be NULL), and the numbers of
 * slots placed on another expert than their first proposal and of slots
 * dropped. Returns -1 on an invalid configuration. */
int moero_capacity_route(const moero_cfg* cfg, const float* s32, const double* s64,
                         const float* bias, int32_t cap, int32_t* idx, float* w,
                         int64_t* n_rerouted, int64_t* n_dropped) {
  if (!cfg_valid(cfg)) return -1;
  const int32_t T = cfg->T, N = cfg->N, K = cfg->K, G = cfg->n_groups;
  const int32_t Gk = cfg->topk_groups, Kt = K + cfg->n_shared;
  const int32_t gsz = N / G;
  const int64_t A = (int64_t)T * K;
  enum { PENDING = 0, ACCEPTED = 1, REJECTED = 2, DROPPED = 3 };
  int32_t* list = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1) * (size_t)N);
  int32_t* n_el = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  int32_t* next = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  int32_t* prop = (int32_t*)malloc(sizeof(int32_t) * (size_t)(A > 0 ? A : 1));
  char* state = (char*)malloc((size_t)(A > 0 ? A : 1));
  int32_t* held = (int32_t*)calloc((size_t)N, sizeof(int32_t));
  ranked* cand = (ranked*)malloc(sizeof(ranked) * (size_t)N);
  ranked* grp = (ranked*)malloc(sizeof(ranked) * (size_t)G);
  ranked* mem = (ranked*)malloc(sizeof(ranked) * (size_t)gsz);
  float* key = (float*)malloc(sizeof(float) * (size_t)N);
  char* kept = (char*)malloc((size_t)G);
  if (!list || !n_el || !next || !prop || !state || !held || !cand || !grp || !mem || !key ||
      !kept)
    return -1;
  /* candidates; round 0 proposes the top-K */
  for (int32_t t = 0; t < T; ++t) {
    double margin = INFINITY;
    n_el[t] = rank_token(s32 + (size_t)t * N, bias, N, G, Gk, cand, grp, mem, key, kept, &margin);
    for (int32_t r = 0; r < n_el[t]; ++r) list[(size_t)t * N + r] = cand[r].id;
    for (int32_t k = 0; k < K; ++k) {
      prop[(size_t)t * K + k] = list[(size_t)t * N + k];
      state[(size_t)t * K + k] = PENDING;
    }
    next[t] = K;
  }
  int64_t pending = A;
  while (pending > 0) {
    /* accept in (token, slot) order up to the capacity */
    for (int64_t a = 0; a < A; ++a) {
      if (state[a] != PENDING) continue;
      const int32_t e = prop[a];
      if (held[e] < cap) { held[e] += 1; state[a] = ACCEPTED; }
      else state[a] = REJECTED;
    }
    /* rejected slots take the next candidates, in slot order per token */
    pending = 0;
    for (int64_t a = 0; a < A; ++a) {
      if (state[a] != REJECTED) continue;
      const int32_t t = (int32_t)(a / K);
      if (next[t] < n_el[t]) {
        prop[a] = list[(size_t)t * N + next[t]];
        next[t] += 1;
        state[a] = PENDING;
        ++pending;
      } else {
        state[a] = DROPPED;
      }
    }
  }
  int64_t rerouted = 0, dropped = 0;
  for (int32_t t = 0; t < T; ++t) {
    const double* sd = s64 + (size_t)t * N;
    double z = 0.0;
    int32_t placed = 0;
    for (int32_t k = 0; k < K; ++k) {
      const int64_t a = (int64_t)t * K + k;
      if (state[a] == DROPPED) { ++dropped; continue; }
      if (prop[a] != list[(size_t)t * N + k]) ++rerouted;
      z += sd[prop[a]];
      ++placed;
    }
    for (int32_t k = 0; k < K; ++k) {
      const int64_t a = (int64_t)t * K + k;
      const int dropped_slot = state[a] == DROPPED;
      if (idx) idx[(size_t)t * Kt + k] = dropped_slot ? -1 : prop[a];
      if (w)
        w[(size_t)t * Kt + k] = dropped_slot ? 0.0f
                                : (float)(z > 0.0 ? sd[prop[a]] / z : 1.0 / placed);
    }
    for (int32_t j = 0; j < cfg->n_shared; ++j) {
      if (idx) idx[(size_t)t * Kt + K + j] = N + j;
      if (w) w[(size_t)t * Kt + K + j] = 1.0f;
    }
  }
  if (n_rerouted) *n_rerouted = rerouted;
  if (n_dropped) *n_dropped = dropped;
  free(list); free(n_el); free(next); free(prop); free(state); free(held);
  free(cand); free(grp); free(mem); free(key); free(kept);
  return 0;
}

/* [P1] compute_routing_entropy: average the routing distributions over the
 * batch, then take the entropy (bits) of that mean distribution. */
double moero_agg_entropy(const double* s64, int32_t T, int32_t N) {
  if (T <= 0) return 0.0;
  double* mean = (double*)calloc((size_t)N, sizeof(double));
  if (!mean) return NAN;
  for (int32_t t = 0; t < T; ++t) {
    const double* sd = s64 + (size_t)t * N;
    double z = 0.0;
    for (int32_t e = 0; e < N; ++e) z += sd[e];
    if (z > 0.0)
      for (int32_t e = 0; e < N; ++e) mean[e] += sd[e] / z;
  }
  for (int32_t e = 0; e < N; ++e) mean[e] /= (double)T;
  double H = entropy_bits_of(mean, N);
  free(mean);
  return H;
}

/* Dispatch layout: [P1] listing's bincount of the selected experts, then an
 * exclusive prefix over experts, then every (token, slot) placed in expert
 * order and, within an expert, in token (then slot) order — the grouping by
 * destination expert that dispatch needs ([P2] DeepEP section). */
void moero_layout(const int32_t* idx, int32_t T, int32_t Kt, int32_t Nb,
                  int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm) {
  const int64_t A = (int64_t)T * Kt;
  for (int32_t e = 0; e < Nb; ++e) counts[e] = 0;
  for (int64_t a = 0; a < A; ++a)
    if (idx[a] >= 0 && idx[a] < Nb) counts[idx[a]] += 1;
  offsets[0] = 0;
  for (int32_t e = 0; e < Nb; ++e) offsets[e + 1] = offsets[e] + counts[e];
  for (int64_t a = 0; a < A; ++a) {
    perm[a] = -1;
    if (inv_perm) inv_perm[a] = -1;
  }
  int64_t pos = 0;
  for (int32_t e = 0; e < Nb; ++e) {
    for (int64_t a = 0; a < A; ++a) {
      if (idx[a] == e) {
        perm[pos] = (int32_t)a;
        if (inv_perm) inv_perm[a] = (int32_t)pos;
        ++pos;
      }
    }
  }
}

/* [P2] DeepEP section: dispatch. Walk the layout in its own (expert-major)
 * order and fetch each position's token row. */
void moero_dispatch(const void* x, int64_t row_bytes, int32_t T, int32_t Kt,
                    const int32_t* perm, void* x_out) {
  const int64_t A = (int64_t)T * Kt;
  for (int64_t pos = 0; pos < A; ++pos) {
    if (perm[pos] < 0) continue;
    const int64_t t = perm[pos] / Kt;
    memcpy((char*)x_out + pos * row_bytes, (const char*)x + t * row_bytes, (size_t)row_bytes);
  }
}

/* [P2] token routing and DeepEP section: weighted combine. Each layout
 * position adds its expert-output row, times the weight of the slot it
 * serves, to that slot's token. */
void moero_combine(const double* out, const float* w, const int32_t* perm,
                   int32_t T, int32_t Kt, int32_t d, double* y) {
  const int64_t A = (int64_t)T * Kt;
  for (int64_t i = 0; i < (int64_t)T * d; ++i) y[i] = 0.0;
  for (int64_t pos = 0; pos < A; ++pos) {
    const int32_t slot = perm[pos];
    if (slot < 0) continue;
    const int64_t t = slot / Kt;
    const double wk = (double)w[slot];
    for (int32_t j = 0; j < d; ++j) y[t * d + j] += wk * out[pos * d + j];
  }
}

/* [P5] forcible load balancing: consecutive assignments of the batch walk
 * the experts round-robin, so every expert receives the same number (within
 * one) and a token's K routed slots are K different experts when K <= N. */
void moero_balanced_indices(int32_t T, int32_t K, int32_t N, int32_t n_shared, int32_t first,
                            int32_t* idx) {
  const int32_t Kt = K + n_shared;
  int64_t start = first % N;
  if (start < 0) start += N;
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t k = 0; k < K; ++k)
      idx[(int64_t)t * Kt + k] = (int32_t)(((int64_t)t * K + k + start) % N);
    for (int32_t j = 0; j < n_shared; ++j) idx[(int64_t)t * Kt + K + j] = N + j;
  }
}

/* [P5] hotspot collection: add this batch's per-expert token counts. */
void moero_hotspot_accumulate(int64_t* hot, const int32_t* counts, int32_t n_layers, int32_t N,
                              int32_t stride) {
  for (int32_t l = 0; l < n_layers; ++l)
    for (int32_t e = 0; e < N; ++e) hot[(int64_t)l * N + e] += counts[(int64_t)l * stride + e];
}

/* [P1] listing: the dynamic bias is added to the raw gate logits before
 * the softmax, so every later step sees the compensated logits. */
void moero_logit_bias(double* h, const float* b, int32_t T, int32_t N) {
  for (int32_t t = 0; t < T; ++t)
    for (int32_t e = 0; e < N; ++e) h[(int64_t)t * N + e] += (double)b[e];
}

/* [P1] listing (proportional rule: lower an overloaded expert's bias by the
 * decay times its relative load error) and [P2] auxiliary-loss-free section
 * (direction-only rule; a moving average smooths the load statistics; the
 * bias is updated every so many steps). */
void moero_balance_step(float* bias, const int32_t* counts, int32_t N, int32_t rule, float step,
                        float alpha, int32_t every, float* loads, int32_t* calls) {
  const int32_t ncall = calls ? *calls : 0;
  float* l = (float*)malloc((size_t)N * sizeof(float));
  const float keep = 1.0f - alpha;
  for (int32_t e = 0; e < N; ++e) {
    volatile float ce = (float)counts[e];
    if (loads == NULL || ncall == 0) {
      l[e] = ce;
    } else {
      volatile float fresh = alpha * ce;
      volatile float old = keep * loads[e];
      volatile float sum = fresh + old;
      l[e] = sum;
    }
    if (loads) loads[e] = l[e];
  }
  if ((ncall + 1) % every == 0) {
    double total = 0.0;
    for (int32_t e = 0; e < N; ++e) total += (double)l[e];
    const double mean = total / (double)N;
    for (int32_t e = 0; e < N; ++e) {
      if (rule == 0) {
        const double diff = mean - (double)l[e];
        const float s = diff > 0 ? step : (diff < 0 ? -step : 0.0f);
        volatile float nb = bias[e] + s;
        bias[e] = nb;
      } else if (mean > 0.0) {
        const double rel = ((double)l[e] - mean) / mean;
        const float delta = (float)((double)step * rel);
        volatile float nb = bias[e] - delta;
        bias[e] = nb;
      }
    }
  }
  if (calls) *calls = ncall + 1;
  free(l);
}

/* [P4] Run the example: total, mean = total / N, imbalance = max / mean
 * (0 when the mean is 0), capacity = max · N. Added: argmax (lowest expert on
 * ties); load entropy in bits of counts/total ([P1] Mathematics applied to
 * the realised load); coefficient of variation = population std / mean
 * ([P2] deployment section monitors std relative to the mean). */
void moero_load_stats(const int32_t* counts, int32_t N, moero_stats* out) {
  int64_t total = 0, mx = 0, am = 0;
  for (int32_t e = 0; e < N; ++e) {
    total += counts[e];
    if (counts[e] > mx) { mx = counts[e]; am = e; }
  }
  if (N > 0 && mx == 0) am = 0;
  out->total = total;
  out->max_load = mx;
  out->argmax = am;
  out->capacity = mx * (int64_t)N;
  out->mean = N > 0 ? (double)total / (double)N : 0.0;
  out->imbalance = out->mean != 0.0 ? (double)mx / out->mean : 0.0;
  double H = 0.0;
  if (total > 0) {
    for (int32_t e = 0; e < N; ++e) {
      if (counts[e] > 0) {
        double q = (double)counts[e] / (double)total;
        H -= q * log2(q);
      }
    }
  }
  out->h_load_bits = H;
  double var = 0.0;
  for (int32_t e = 0; e < N; ++e) {
    double dlt = (double)counts[e] - out->mean;
    var += dlt * dlt;
  }
  var = N > 0 ? var / (double)N : 0.0;
  out->cv = out->mean != 0.0 ? sqrt(var) / out->mean : 0.0;
}

/* [P2] auxiliary-loss-free balancing: after each step, lower the bias of
 * overloaded experts and raise it for underloaded ones, by a fixed step u:
 * b_e += u · sign(mean_load − load_e). The comparison is made exactly, in
 * integers, as sign(total − N·load_e). */
void moero_bias_update(float* bias, const int32_t* counts, int32_t N, float u) {
  int64_t total = 0;
  for (int32_t e = 0; e < N; ++e) total += counts[e];
  for (int32_t e = 0; e < N; ++e) {
    int64_t diff = total - (int64_t)N * counts[e];
    float step = diff > 0 ? u : (diff < 0 ? -u : 0.0f);
    volatile float nb = bias[e] + step;
    bias[e] = nb;
  }
}
