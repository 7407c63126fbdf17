// Host side of the C ABI (include/moer.h): argument validation, workspace
// carving, and the stream-ordered launch sequence. No host synchronisation,
// no allocation, no global state besides the thread-local error string.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/moer.h"
#include "moer_internal.hpp"

// Scratch memory of moer_route_noalloc: one array per GPU, allocated with
// the code object when the library is loaded on a device and held until the
// process ends. Host code never passes this name to a kernel (on the host it
// is only a stand-in symbol); it uses the device address that
// hipGetSymbolAddress returns for the current device.
constexpr size_t kNoAllocScratchBytes = MOER_NOALLOC_SCRATCH_BYTES;  // 40 MiB
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

thread_local char g_err[512] = "";

moer_status fail(moer_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

moer_status ok() {
  g_err[0] = '\0';
  return MOER_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }


bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

moer_status check_rows(int32_t n_layers, int32_t T, int32_t Kt) {
  if (n_layers < 1 || T < 0) return fail(MOER_EINVAL, "need n_layers >= 1 and T >= 0");
  if (Kt < 1 || Kt > MOER_MAX_SLOTS)
    return fail(MOER_EINVAL, "Kt must be in [1, %d] (got %d)", MOER_MAX_SLOTS, Kt);
  if ((int64_t)T * Kt >= ((int64_t)1 << 31)) return fail(MOER_EINVAL, "T * Kt must be < 2^31");
  return MOER_OK;
}

// Workspace regions (byte offsets) for a validated descriptor.
struct Plan {
  int Kt, Nb, nsb, nlb, ksplit;
  int nsb_small;  // 16-token histogram blocks (small routers, small batches; 0: none)
  int nseg;
  int nsync;  // fused pass counters, stored right after the segment totals
  size_t off_h, off_colpart, off_cnt, off_seg, off_colmean, total;
  // capacity-limited routing
  size_t off_key, off_s, off_ranked, off_nel, off_next, off_changed, off_list0, off_list1,
      off_inv, off_flag, off_liste, off_rd;
  struct Round {
    size_t prop, mask, cnt, segsum, counts, offsets, perm, inv;
  } round[moer::kCapGridRounds + 1];
};

Plan make_plan(const moer_route_desc& d, bool hidden, bool want_agg) {
  Plan p{};
  const size_t L = (size_t)d.n_layers;
  p.Kt = d.K + d.n_shared;
  p.Nb = d.N + d.n_shared;
  p.nsb = (d.T + moer::kRowTokens - 1) / moer::kRowTokens;
  p.nlb = d.T > 0 ? (d.T + moer::kLayoutTokens - 1) / moer::kLayoutTokens : 1;
  p.ksplit = hidden ? moer::gate_gemm_ksplit(d.dtype == MOER_BF16, d.n_layers, d.T, d.d, d.N) : 1;
  // routers the one-launch small kernel or the few-token selection kernel may
  // take: room for their blocks of 16 (or 32) tokens
  p.nsb_small = (hidden && d.N <= moer::kSmallMaxExperts) ||
                        moer::route_rows_tokens(d.n_layers, d.T) < moer::kRowTokens
                    ? (d.T + moer::kSmallTokens - 1) / moer::kSmallTokens : 0;
  const size_t nsb_room = (size_t)std::max(p.nsb, p.nsb_small);
  size_t o = 0;
  p.off_h = o;  // partial affinities of the gate GEMM
  if (hidden) o += align_up((size_t)p.ksplit * L * d.T * d.N * sizeof(float));
  p.off_colpart = o;  // column sums of q per histogram block
  if (want_agg) o += align_up(L * nsb_room * d.N * sizeof(float) + 16);
  p.off_cnt = o;  // expert histograms per histogram block (uint16)
  o += align_up(L * p.Nb * nsb_room * sizeof(uint16_t) + 16);
  p.nseg = (p.nsb + moer::kSegBlocks - 1) / moer::kSegBlocks;
  p.off_seg = o;  // expert counts per segment of histogram blocks, then the
                  // fused pass's counters (one zero fill clears both)
  p.nsync = hidden ? moer::route_fused_sync_ints(d.n_layers, d.T) : 0;
  o += align_up((L * p.nseg * p.Nb + p.nsync) * sizeof(int32_t) + 16);
  p.off_colmean = o;  // fused pass: batch-mean q per expert
  if (hidden && want_agg) o += align_up(L * d.N * sizeof(float) + 16);
  if (d.capacity > 0 && d.input != MOER_IN_INDICES) {
    const size_t LT = L * (size_t)d.T;
    p.off_key = o;      // selection keys, -inf outside the kept groups
    o += align_up(LT * d.N * sizeof(float) + 16);
    p.off_s = o;        // scores
    o += align_up(LT * d.N * sizeof(float) + 16);
    p.off_ranked = o;   // candidate lists, 256 ids per token
    o += align_up(LT * moer::kMaxExperts + 16);
    p.off_nel = o;
    o += align_up(LT * sizeof(int32_t) + 16);
    p.off_next = o;
    o += align_up(LT * sizeof(int32_t) + 16);
    p.off_changed = o;
    o += align_up(LT + 16);
    p.off_list0 = o;    // pending slots (two buffers)
    o += align_up(LT * d.K * sizeof(int32_t) + 16);
    p.off_list1 = o;
    o += align_up(LT * d.K * sizeof(int32_t) + 16);
    p.off_inv = o;      // the first layout's inv_perm when the caller has none
    o += align_up(LT * p.Kt * sizeof(int32_t) + 16);
    p.off_flag = o;     // layers with an expert over capacity
    o += align_up(L * sizeof(int32_t) + 16);
    p.off_liste = o;    // the workgroup rounds' first list: proposed experts
    o += align_up(LT * d.K * sizeof(int32_t) + 16);
    p.off_rd = o;       // rerouted / dropped / left pending, per accept workgroup
    o += align_up(moer::kCapGridRounds * L * ((d.T + 63) / 64) * 3 * sizeof(int32_t) + 16);
    for (int r = 0; r <= moer::kCapGridRounds; ++r) {  // per round: proposals ...
      Plan::Round& q = p.round[r];
      q.prop = o;
      o += align_up(LT * d.K * sizeof(int32_t) + 16);
      q.mask = o;
      o += align_up(LT * sizeof(int32_t) + 16);
      if (r == moer::kCapGridRounds) break;
      q.cnt = o;        // ... and, for the grid rounds, their layout
      o += align_up(L * d.N * p.nsb * sizeof(uint16_t) + 16);
      q.segsum = o;
      o += align_up(L * p.nseg * d.N * sizeof(int32_t) + 16);
      q.counts = o;
      o += align_up(L * d.N * sizeof(int32_t) + 16);
      q.offsets = o;
      o += align_up(L * (d.N + 1) * sizeof(int32_t) + 16);
      q.perm = o;
      o += align_up(LT * d.K * sizeof(int32_t) + 16);
      q.inv = o;
      o += align_up(LT * d.K * sizeof(int32_t) + 16);
    }
  }
  p.total = o;
  return p;
}

// Fused router pass, chosen by the environment variable MOER_ROUTE_FUSED:
// 0 (the default) = never; 1 = for the batches whose separate gate GEMM also
// splits d in two (tiles enough to fill the chip); 2 = the same with the
// layout as a separate launch; 3 = for every shape it can take. Off by
// default: on MI355X its in-kernel synchronisation costs more than the
// kernel boundaries it removes (the 16k-token batch: 126 us with it, 82 us
// without).
int fused_mode() {
  const char* v = getenv("MOER_ROUTE_FUSED");
  if (v == nullptr || *v == '\0') return 0;
  return atoi(v);
}

// One-launch gate GEMM + selection for routers with at most 16 experts,
// chosen by the environment variable MOER_ROUTE_SMALL: on (the default)
// unless it is "0", which keeps such routers on the separate gate GEMM and
// selection launches.
bool small_enabled() {
  const char* v = getenv("MOER_ROUTE_SMALL");
  return v == nullptr || strcmp(v, "0") != 0;
}

// One workgroup per layer that also writes the layout outputs, for layers of
// at most moer::kWholeTokens tokens and a short depth on the one-launch
// small-router kernel (moer::route_layer_eligible),
// chosen by the environment variable MOER_ROUTE_WHOLE: on (the default)
// unless it is "0", which keeps the layout launch.
bool whole_enabled() {
  const char* v = getenv("MOER_ROUTE_WHOLE");
  return v == nullptr || strcmp(v, "0") != 0;
}

// 16- or 32-token selection workgroups for small batches
// (route_rows_tokens), chosen by the environment variable MOER_ROUTE_TINY:
// on (the default) unless it is "0", which keeps every batch on 64-token
// workgroups.
bool tiny_enabled() {
  const char* v = getenv("MOER_ROUTE_TINY");
  return v == nullptr || strcmp(v, "0") != 0;
}

// Which selection kernel takes this shape: 1 = one 16-lane row per token,
// 2 = one wavefront per token (any group size).
int selection_path(const moer_route_desc& d) {
  return moer::route_rows_supports(d.N, d.n_groups) ? 1 : 2;
}

moer_status validate_desc(const moer_route_desc* d) {
  if (d == nullptr) return fail(MOER_EINVAL, "desc is NULL");
  if (d->n_layers < 1) return fail(MOER_EINVAL, "n_layers must be >= 1 (got %d)", d->n_layers);
  if (d->T < 0) return fail(MOER_EINVAL, "T must be >= 0 (got %d)", d->T);
  if (d->N < 1 || d->N > MOER_MAX_EXPERTS)
    return fail(MOER_EINVAL, "N must be in [1, %d] (got %d)", MOER_MAX_EXPERTS, d->N);
  if (d->K < 1 || d->K > d->N) return fail(MOER_EINVAL, "K must be in [1, N] (got %d)", d->K);
  if (d->n_shared < 0) return fail(MOER_EINVAL, "n_shared must be >= 0");
  if (d->K + d->n_shared > MOER_MAX_SLOTS)
    return fail(MOER_EINVAL, "K + n_shared must be <= %d", MOER_MAX_SLOTS);
  if ((long long)d->T * (d->K + d->n_shared) >= (1LL << 31))
    return fail(MOER_EINVAL, "T * (K + n_shared) must be < 2^31");
  if (d->n_groups < 1 || d->N % d->n_groups != 0)
    return fail(MOER_EINVAL, "n_groups must divide N (N=%d, n_groups=%d)", d->N, d->n_groups);
  if (d->topk_groups < 1 || d->topk_groups > d->n_groups)
    return fail(MOER_EINVAL, "topk_groups must be in [1, n_groups]");
  const int gsz = d->N / d->n_groups;
  if (d->n_groups > 1 && gsz < 2)
    return fail(MOER_EINVAL, "groups need at least 2 experts (top-2 group score)");
  if ((long long)d->topk_groups * gsz < d->K)
    return fail(MOER_EINVAL, "topk_groups * N/n_groups must be >= K");
  if (d->score_fn != MOER_SOFTMAX && d->score_fn != MOER_SIGMOID)
    return fail(MOER_EINVAL, "unknown score_fn %d", d->score_fn);
  if (d->input != MOER_IN_HIDDEN && d->input != MOER_IN_SCORES && d->input != MOER_IN_INDICES)
    return fail(MOER_EINVAL, "unknown input mode %d", d->input);
  if (d->input == MOER_IN_HIDDEN) {
    if (d->dtype != MOER_BF16 && d->dtype != MOER_F32)
      return fail(MOER_EINVAL, "unknown dtype %d", d->dtype);
    if (d->d < 1) return fail(MOER_EINVAL, "d must be >= 1 (got %d)", d->d);
    if (d->dtype == MOER_BF16 && d->d % 8 != 0)
      return fail(MOER_EINVAL, "bf16 inputs need d %% 8 == 0 (got %d)", d->d);
    if ((long long)d->T * d->d >= (1LL << 40) || (long long)d->N * d->d >= (1LL << 40))
      return fail(MOER_EINVAL, "hidden size too large");
  }
  if (d->bias_mode != MOER_BIAS_SCORE && d->bias_mode != MOER_BIAS_LOGIT)
    return fail(MOER_EINVAL, "unknown bias_mode %d", d->bias_mode);
  if (d->bias_mode == MOER_BIAS_LOGIT && d->input != MOER_IN_HIDDEN)
    return fail(MOER_EINVAL, "a logit-space bias needs HIDDEN input (the logits)");
  if (d->capacity < 0) return fail(MOER_EINVAL, "capacity must be >= 0 (got %d)", d->capacity);
  if (d->capacity > 0 && d->input == MOER_IN_INDICES)
    return fail(MOER_EINVAL, "a capacity needs HIDDEN or SCORES input (the candidates)");
  return MOER_OK;
}

}  // namespace

extern "C" {

int moer_abi_version(void) { return MOER_ABI_VERSION; }

const char* moer_last_error(void) { return g_err; }

const char* moer_status_str(moer_status s) {
  switch (s) {
    case MOER_OK: return "MOER_OK";
    case MOER_EINVAL: return "MOER_EINVAL";
    case MOER_EUNSUPPORTED: return "MOER_EUNSUPPORTED";
    case MOER_EWORKSPACE: return "MOER_EWORKSPACE";
    case MOER_EHIP: return "MOER_EHIP";
  }
  return "MOER_UNKNOWN";
}

size_t moer_route_workspace_bytes(const moer_route_desc* desc) {
  if (validate_desc(desc) != MOER_OK) return 0;
  // Upper bound over the optional outputs: h in workspace and the entropy
  // partials are always budgeted.
  return make_plan(*desc, desc->input == MOER_IN_HIDDEN, desc->input != MOER_IN_INDICES).total;
}

moer_status moer_route(const moer_route_desc* desc, const moer_route_io* io, void* workspace,
                       size_t workspace_bytes, void* stream) {
  moer_status st = validate_desc(desc);
  if (st != MOER_OK) return st;
  if (io == nullptr) return fail(MOER_EINVAL, "io is NULL");
  const moer_route_desc& d = *desc;
  const bool hidden = d.input == MOER_IN_HIDDEN;
  const bool scores = d.input == MOER_IN_SCORES;
  const bool indices = d.input == MOER_IN_INDICES;
  // Arrays whose size is proportional to T may be NULL for an empty batch.
  const bool some = d.T > 0;
  if (hidden && some && (io->x == nullptr || io->w_gate == nullptr))
    return fail(MOER_EINVAL, "HIDDEN input needs x and w_gate");
  if (scores && some && io->scores == nullptr)
    return fail(MOER_EINVAL, "SCORES input needs scores");
  if (indices && some && io->idx_in == nullptr)
    return fail(MOER_EINVAL, "INDICES input needs idx_in");
  if (!indices && some && (io->topk_idx == nullptr || io->topk_w == nullptr))
    return fail(MOER_EINVAL, "topk_idx and topk_w are required");
  if (io->counts == nullptr || io->offsets == nullptr || (some && io->perm == nullptr))
    return fail(MOER_EINVAL, "counts, offsets and perm are required");
  // 16-byte vector loads (the gate GEMM's DMA; four experts per load of
  // scores, bias and logit offset)
  if (hidden && some && d.dtype == MOER_BF16 && (!aligned16(io->x) || !aligned16(io->w_gate)))
    return fail(MOER_EINVAL, "x and w_gate must be 16-byte aligned");
  if (scores && some && !aligned16(io->scores))
    return fail(MOER_EINVAL, "scores must be 16-byte aligned");
  if ((io->bias != nullptr && !aligned16(io->bias)) ||
      (io->logit_offset != nullptr && !aligned16(io->logit_offset)))
    return fail(MOER_EINVAL, "bias and logit_offset must be 16-byte aligned");
  if ((io->ev_gemm_begin == nullptr) != (io->ev_gemm_end == nullptr))
    return fail(MOER_EINVAL, "ev_gemm_begin and ev_gemm_end go together");
  if (io->bias_update != nullptr &&
      (!(io->bias_update_u == io->bias_update_u) || io->bias_update_u < 0.f ||
       io->bias_update_u == __builtin_inff()))
    return fail(MOER_EINVAL, "bias_update_u must be finite and >= 0");

  const bool want_agg = !indices && io->agg_entropy != nullptr;
  const bool capped = d.capacity > 0 && !indices;
  const Plan p = make_plan(d, hidden, want_agg);
  if (workspace == nullptr && p.total > 0) return fail(MOER_EWORKSPACE, "workspace is NULL");
  if (workspace_bytes < p.total)
    return fail(MOER_EWORKSPACE, "workspace too small: need %zu bytes, got %zu", p.total,
                workspace_bytes);

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int L = d.n_layers;
  hipError_t he = hipSuccess;
#define MOER_CHECK(expr)                                                        \
  do {                                                                          \
    he = (expr);                                                                \
    if (he != hipSuccess)                                                       \
      return fail(MOER_EHIP, "%s: %s", #expr, hipGetErrorString(he));           \
  } while (0)

  int32_t* segsum = reinterpret_cast<int32_t*>(ws + p.off_seg);
  const int n_seg = L * p.nseg * p.Nb;
  float* colpart = want_agg ? reinterpret_cast<float*>(ws + p.off_colpart) : nullptr;
  uint16_t* cnt = reinterpret_cast<uint16_t*>(ws + p.off_cnt);
  const int path = indices ? 0 : selection_path(d);

  // a2-a6 arguments: scores, selection, weights, entropy, block histograms
  moer::ScoreArgs a{};
  a.in = hidden ? reinterpret_cast<const float*>(ws + p.off_h) : io->scores;
  a.offset = hidden ? io->logit_offset : nullptr;
  a.h_out = hidden ? io->h_out : nullptr;
  a.nsplit = p.ksplit;
  a.bias = io->bias;
  a.idx = io->topk_idx;
  a.w = io->topk_w;
  a.tok_entropy = io->tok_entropy;
  a.colpart = colpart;
  a.T = d.T;
  a.N = d.N;
  a.K = d.K;
  a.G = d.n_groups;
  a.Gk = d.topk_groups;
  a.n_shared = d.n_shared;
  a.score_fn = d.score_fn;
  a.apply_score = hidden ? 1 : 0;
  a.bias_logit = d.bias_mode == MOER_BIAS_LOGIT ? 1 : 0;
  if (capped) {
    a.key_out = reinterpret_cast<float*>(ws + p.off_key);
    a.s_out = reinterpret_cast<float*>(ws + p.off_s);
  }
  a.cnt = path == 1 ? cnt : nullptr;
  a.segsum = path == 1 ? segsum : nullptr;

  // a6-a8 (+ batch-mean entropy, statistics, bias update) arguments: layout
  moer::LayoutArgs la{};
  la.idx = indices ? io->idx_in : io->topk_idx;
  la.cnt = cnt;
  la.segsum = segsum;
  la.nseg = p.nseg;
  la.colpart = colpart;
  la.agg_entropy = want_agg ? io->agg_entropy : nullptr;
  la.counts = io->counts;
  la.offsets = io->offsets;
  la.perm = io->perm;
  int32_t* inv_perm = io->inv_perm;
  if (capped && inv_perm == nullptr) inv_perm = reinterpret_cast<int32_t*>(ws + p.off_inv);
  la.inv_perm = inv_perm;
  la.T = d.T;
  la.Kt = p.Kt;
  la.Nb = p.Nb;
  la.N = d.N;
  la.nlb = p.nlb;
  la.nsb = p.nsb;
  la.stats = io->load_stats;
  la.bias_inout = io->bias_update;
  la.bias_step = io->bias_update_u;
  int32_t* cap_flag = capped ? reinterpret_cast<int32_t*>(ws + p.off_flag) : nullptr;
  if (capped && d.T > 0) {
    // statistics and bias update only for layers no expert overflows; the
    // others wait for the final ids
    la.cap = d.capacity;
    la.cap_phase = 1;
    la.cap_flag = cap_flag;
  }
  la.fill_invalid = indices ? 1 : 0;
  la.need_count = (path != 1 && d.T > 0) ? 1 : 0;

  // The fused pass (one co-resident launch after a fill kernel) takes the
  // large bf16 routers it was built for; every other shape, the capacity
  // limit and a split selection stream take the separate launches below.
  const int fused = fused_mode();
  if (fused != 0 && hidden && d.dtype == MOER_BF16 && d.T > 0 && !capped &&
      io->ev_select_wait == nullptr && p.ksplit >= 2 && (fused == 3 || p.ksplit == 2) &&
      moer::route_fused_eligible(L, d.T, d.d, d.N, d.n_groups)) {
    MOER_CHECK(moer::launch_zero_ints(segsum, n_seg + p.nsync, s));
    if (io->ev_gemm_begin) MOER_CHECK(hipEventRecord(static_cast<hipEvent_t>(io->ev_gemm_begin), s));
    MOER_CHECK(moer::launch_route_fused(io->x, io->w_gate, reinterpret_cast<float*>(ws + p.off_h),
                                        segsum + n_seg,
                                        reinterpret_cast<float*>(ws + p.off_colmean), a, la, L,
                                        d.T, d.d, d.N, fused != 2, s));
    if (io->ev_gemm_end) MOER_CHECK(hipEventRecord(static_cast<hipEvent_t>(io->ev_gemm_end), s));
    if (fused == 2) MOER_CHECK(moer::launch_layout(la, L, s));
    return ok();
  }

  // Routers with at most 16 experts: every expert of a token fits one
  // workgroup, which forms the affinities and routes them in one launch.
  if (hidden && d.T > 0 && !capped && path == 1 && io->ev_select_wait == nullptr &&
      small_enabled() &&
      moer::route_small_eligible(d.dtype == MOER_BF16, d.T, d.d, d.N, d.n_groups,
                                 aligned16(io->x) && aligned16(io->w_gate))) {
    a.segsum = nullptr;  // the layout sums the block counts itself
    la.segsum = nullptr;
    la.nsb = (d.T + moer::kSmallTokens - 1) / moer::kSmallTokens;  // its 16-token blocks
    la.hist_shift = moer::kSmallShift;
    // a layer of at most kWholeTokens tokens: one workgroup does the layout too
    const bool whole =
        moer::route_layer_eligible(d.dtype == MOER_BF16, d.T, d.d, d.N) && whole_enabled();
    MOER_CHECK(moer::launch_route_small(a, io->x, io->w_gate, d.d, d.dtype == MOER_BF16, L, s,
                                        static_cast<hipEvent_t>(io->ev_gemm_begin),
                                        static_cast<hipEvent_t>(io->ev_gemm_end),
                                        whole ? &la : nullptr));
    if (!whole) MOER_CHECK(moer::launch_layout(la, L, s));
    return ok();
  }

  // Small batches: 16- or 32-token selection workgroups, whose histogram
  // blocks carry no segment totals (the layout sums the block counts).
  int rows = moer::kRowTokens;
  if (path == 1 && !capped && tiny_enabled()) rows = moer::route_rows_tokens(L, d.T);
  if (rows < moer::kRowTokens) {
    a.segsum = nullptr;
    la.segsum = nullptr;
    la.nsb = (d.T + rows - 1) / rows;
    la.hist_shift = rows == moer::kSmallTokens ? moer::kSmallShift : 1;
  }

  // segment counters start at zero: cleared by the gate GEMM when the
  // pipelined bf16 kernel or the fp32 kernel runs, else by a fill kernel
  const bool gemm_clears =
      hidden && d.T > 0 &&
      (d.dtype == MOER_BF16 ? moer::gate_gemm_clears(L, d.T, d.d, d.N, p.ksplit) : true);
  if (!gemm_clears) MOER_CHECK(moer::launch_zero_ints(segsum, n_seg, s));

  // a1: gate affinities (depth-range partial sums in the workspace)
  if (hidden && d.T > 0) {
    float* hbuf = reinterpret_cast<float*>(ws + p.off_h);
    hipEvent_t ev0 = static_cast<hipEvent_t>(io->ev_gemm_begin);
    hipEvent_t ev1 = static_cast<hipEvent_t>(io->ev_gemm_end);
    if (d.dtype == MOER_BF16) {
      MOER_CHECK(moer::launch_gate_gemm_bf16(io->x, io->w_gate, hbuf, L, d.T, d.d, d.N, p.ksplit,
                                             gemm_clears ? segsum : nullptr,
                                             gemm_clears ? n_seg : 0, s, ev0, ev1));
    } else {
      if (ev0) MOER_CHECK(hipEventRecord(ev0, s));
      MOER_CHECK(moer::launch_gate_gemm_f32(static_cast<const float*>(io->x),
                                            static_cast<const float*>(io->w_gate), hbuf, L, d.T,
                                            d.d, d.N,
                                            gemm_clears ? segsum : nullptr,
                                            gemm_clears ? n_seg : 0, s));
      if (ev1) MOER_CHECK(hipEventRecord(ev1, s));
    }
  }
  if (io->ev_select_wait != nullptr)
    MOER_CHECK(hipStreamWaitEvent(s, static_cast<hipEvent_t>(io->ev_select_wait), 0));

  if (!indices && d.T > 0) {
    if (path == 1)
      MOER_CHECK(moer::launch_route_rows(a, L, s, rows));
    else
      MOER_CHECK(moer::launch_score_topk(a, L, s));
  }
  MOER_CHECK(moer::launch_layout(la, L, s));

  if (capped && d.T > 0) {
    // later rounds of the capacity limit, then the layout of the final ids
    moer::CapArgs c{};
    c.idx = io->topk_idx;
    c.w = io->topk_w;
    c.inv_perm = inv_perm;
    c.offsets = io->offsets;
    c.key = reinterpret_cast<const float*>(ws + p.off_key);
    c.s = reinterpret_cast<const float*>(ws + p.off_s);
    c.ranked = reinterpret_cast<uint8_t*>(ws + p.off_ranked);
    c.n_el = reinterpret_cast<int32_t*>(ws + p.off_nel);
    c.next = reinterpret_cast<int32_t*>(ws + p.off_next);
    c.changed = reinterpret_cast<uint8_t*>(ws + p.off_changed);
    c.list0 = reinterpret_cast<int32_t*>(ws + p.off_list0);
    c.list1 = reinterpret_cast<int32_t*>(ws + p.off_list1);
    c.stats = io->cap_stats;
    c.flag = cap_flag;
    auto i32 = [&](size_t o) { return reinterpret_cast<int32_t*>(ws + o); };
    for (int r = 0; r <= moer::kCapGridRounds; ++r) {
      const Plan::Round& q = p.round[r];
      c.round[r].prop = i32(q.prop);
      c.round[r].mask = i32(q.mask);
      if (r == moer::kCapGridRounds) break;
      c.round[r].cnt = reinterpret_cast<uint16_t*>(ws + q.cnt);
      c.round[r].segsum = i32(q.segsum);
      c.round[r].counts = i32(q.counts);
      c.round[r].offsets = i32(q.offsets);
      c.round[r].perm = i32(q.perm);
      c.round[r].inv = i32(q.inv);
    }
    c.list_e = i32(p.off_liste);
    c.part = i32(p.off_rd);
    c.segsum = segsum;
    c.nseg = p.nseg;
    c.nsb = p.nsb;
    c.nlb = p.nlb;
    c.G = d.n_groups;
    c.Gk = d.topk_groups;
    c.L = L;
    c.T = d.T;
    c.N = d.N;
    c.K = d.K;
    c.Kt = p.Kt;
    c.Nb = p.Nb;
    c.cap = d.capacity;
    MOER_CHECK(moer::launch_capacity(c, s));
    la.inv_perm = io->inv_perm;
    la.colpart = nullptr;
    la.agg_entropy = nullptr;
    la.fill_invalid = 1;
    la.need_count = 1;
    la.cap_phase = 2;
    MOER_CHECK(moer::launch_layout(la, L, s));
  } else if (capped && io->cap_stats != nullptr) {
    MOER_CHECK(moer::launch_zero_ints(io->cap_stats, 2 * L, s));
  }
#undef MOER_CHECK
  return ok();
}

moer_status moer_route_noalloc(const moer_route_desc* desc, const moer_route_io* io,
                               void* stream) {
  moer_status st = validate_desc(desc);
  if (st != MOER_OK) return st;
  const size_t need = moer_route_workspace_bytes(desc);
  if (need > kNoAllocScratchBytes)
    return fail(MOER_EWORKSPACE,
                "moer_route_noalloc: this router needs %zu bytes of scratch; the static scratch "
                "holds %zu (use moer_route with a workspace)",
                need, kNoAllocScratchBytes);
  int dev = 0;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return fail(MOER_EHIP, "hipGetDevice: %s", hipGetErrorString(he));
  if (stream != nullptr) {
    int sdev = -1;
    he = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (he != hipSuccess) return fail(MOER_EHIP, "hipStreamGetDevice: %s", hipGetErrorString(he));
    if (sdev != dev)
      return fail(MOER_EINVAL, "moer_route_noalloc: the stream is on device %d, the current "
                  "device is %d", sdev, dev);
  }
  // the scratch array's device address, looked up once per device with that
  // device current (each device holds its own copy at its own address)
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOER_EUNSUPPORTED, "moer_route_noalloc: device %d beyond %d", dev, kMaxDevices);
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (ptr[dev] == nullptr) {
      void* p = nullptr;
      he = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (he != hipSuccess || p == nullptr)
        return fail(MOER_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(he));
      ptr[dev] = p;
    }
    ws = ptr[dev];
  }
  return moer_route(desc, io, ws, kNoAllocScratchBytes, stream);
}

moer_status moer_load_stats(const int32_t* counts, int32_t n_layers, int32_t N, int32_t stride,
                            moer_load_stats_t* out_dev, void* stream) {
  if (counts == nullptr || out_dev == nullptr)
    return fail(MOER_EINVAL, "counts and out_dev are required");
  if (n_layers < 1 || N < 1 || stride < N)
    return fail(MOER_EINVAL, "need n_layers >= 1, N >= 1, stride >= N");
  hipError_t he = moer::launch_load_stats(counts, n_layers, N, stride, out_dev,
                                          static_cast<hipStream_t>(stream));
  if (he != hipSuccess) return fail(MOER_EHIP, "load_stats launch: %s", hipGetErrorString(he));
  return ok();
}

moer_status moer_bias_update(float* bias, const int32_t* counts, int32_t n_layers, int32_t N,
                             int32_t stride, float u, void* stream) {
  if (bias == nullptr || counts == nullptr)
    return fail(MOER_EINVAL, "bias and counts are required");
  if (n_layers < 1 || N < 1 || stride < N)
    return fail(MOER_EINVAL, "need n_layers >= 1, N >= 1, stride >= N");
  if (!(u == u) || u < 0.f || u == __builtin_inff())
    return fail(MOER_EINVAL, "u must be finite and >= 0");
  hipError_t he = moer::launch_bias_update(bias, counts, n_layers, N, stride, u,
                                           static_cast<hipStream_t>(stream));
  if (he != hipSuccess) return fail(MOER_EHIP, "bias_update launch: %s", hipGetErrorString(he));
  return ok();
}

moer_status moer_dispatch(const void* x, int64_t row_bytes, int32_t n_layers, int32_t T,
                          int32_t Kt, const int32_t* inv_perm, void* x_out, void* stream) {
  const moer_status st = check_rows(n_layers, T, Kt);
  if (st != MOER_OK) return st;
  if (row_bytes <= 0 || row_bytes % 16 != 0)
    return fail(MOER_EINVAL, "row_bytes must be a positive multiple of 16 (got %lld)",
                (long long)row_bytes);
  if (T == 0) return ok();
  if (x == nullptr || inv_perm == nullptr || x_out == nullptr)
    return fail(MOER_EINVAL, "x, inv_perm and x_out are required");
  if (!aligned16(x) || !aligned16(x_out))
    return fail(MOER_EINVAL, "x and x_out must be 16-byte aligned");
  hipError_t he = moer::launch_dispatch(x, row_bytes, n_layers, T, Kt, inv_perm, x_out,
                                        static_cast<hipStream_t>(stream));
  if (he != hipSuccess) return fail(MOER_EHIP, "dispatch launch: %s", hipGetErrorString(he));
  return ok();
}

moer_status moer_combine(const void* expert_out, moer_dtype out_dtype, const float* w,
                         const int32_t* inv_perm, int32_t n_layers, int32_t T, int32_t Kt,
                         int32_t d, void* y, moer_dtype y_dtype, void* stream) {
  const moer_status st = check_rows(n_layers, T, Kt);
  if (st != MOER_OK) return st;
  if (d < 1 || d % 8 != 0) return fail(MOER_EINVAL, "d must be a positive multiple of 8 (got %d)", d);
  if ((out_dtype != MOER_BF16 && out_dtype != MOER_F32) || (y_dtype != MOER_BF16 && y_dtype != MOER_F32))
    return fail(MOER_EINVAL, "out_dtype and y_dtype must be MOER_BF16 or MOER_F32");
  if (T == 0) return ok();
  if (expert_out == nullptr || w == nullptr || inv_perm == nullptr || y == nullptr)
    return fail(MOER_EINVAL, "expert_out, w, inv_perm and y are required");
  if (!aligned16(expert_out) || !aligned16(y))
    return fail(MOER_EINVAL, "expert_out and y must be 16-byte aligned");
  hipError_t he = moer::launch_combine(expert_out, out_dtype == MOER_BF16, w, inv_perm, n_layers,
                                       T, Kt, d, y, y_dtype == MOER_BF16,
                                       static_cast<hipStream_t>(stream));
  if (he != hipSuccess) return fail(MOER_EHIP, "combine launch: %s", hipGetErrorString(he));
  return ok();
}

moer_status moer_balanced_indices(int32_t* idx, int32_t n_layers, int32_t T, int32_t K, int32_t N,
                                  int32_t n_shared, int32_t first, void* stream) {
  if (N < 1 || N > MOER_MAX_EXPERTS)
    return fail(MOER_EINVAL, "N must be in [1, %d] (got %d)", MOER_MAX_EXPERTS, N);
  if (K < 1 || K > N) return fail(MOER_EINVAL, "K must be in [1, N] (got %d)", K);
  if (n_shared < 0) return fail(MOER_EINVAL, "n_shared must be >= 0");
  const moer_status st = check_rows(n_layers, T, K + n_shared);
  if (st != MOER_OK) return st;
  if (T == 0) return ok();
  if (idx == nullptr) return fail(MOER_EINVAL, "idx is required");
  int start = first % N;
  if (start < 0) start += N;
  hipError_t he = moer::launch_balanced_indices(idx, n_layers, T, K, N, n_shared, start,
                                                static_cast<hipStream_t>(stream));
  if (he != hipSuccess) return fail(MOER_EHIP, "balanced_indices launch: %s", hipGetErrorString(he));
  return ok();
}

moer_status moer_hotspot_accumulate(int64_t* hot, const int32_t* counts, int32_t n_layers,
                                    int32_t N, int32_t stride, void* stream) {
  if (hot == nullptr || counts == nullptr) return fail(MOER_EINVAL, "hot and counts are required");
  if (n_layers < 1 || N < 1 || stride < N)
    return fail(MOER_EINVAL, "need n_layers >= 1, N >= 1, stride >= N");
  hipError_t he = moer::launch_hotspot_accumulate(hot, counts, n_layers, N, stride,
                                                  static_cast<hipStream_t>(stream));
  if (he != hipSuccess) return fail(MOER_EHIP, "hotspot launch: %s", hipGetErrorString(he));
  return ok();
}

moer_status moer_balance_step(float* bias, const int32_t* counts, int32_t n_layers, int32_t N,
                              int32_t stride, const moer_balance_cfg* cfg, float* loads,
                              int32_t* calls, void* stream) {
  if (bias == nullptr || counts == nullptr || cfg == nullptr)
    return fail(MOER_EINVAL, "bias, counts and cfg are required");
  if (n_layers < 1 || N < 1 || N > MOER_MAX_EXPERTS || stride < N)
    return fail(MOER_EINVAL, "need n_layers >= 1, 1 <= N <= %d, stride >= N", MOER_MAX_EXPERTS);
  if (cfg->rule != MOER_RULE_SIGN && cfg->rule != MOER_RULE_PROPORTIONAL)
    return fail(MOER_EINVAL, "unknown rule %d", cfg->rule);
  if (!(cfg->step >= 0.f) || cfg->step == __builtin_inff())
    return fail(MOER_EINVAL, "step must be finite and >= 0");
  if (!(cfg->alpha > 0.f && cfg->alpha <= 1.f)) return fail(MOER_EINVAL, "alpha must be in (0, 1]");
  if (cfg->every < 1) return fail(MOER_EINVAL, "every must be >= 1");
  if (cfg->alpha < 1.f && loads == nullptr)
    return fail(MOER_EINVAL, "alpha < 1 needs the loads state");
  if (cfg->every > 1 && calls == nullptr) return fail(MOER_EINVAL, "every > 1 needs the calls state");
  hipError_t he = moer::launch_balance_step(bias, counts, n_layers, N, stride, cfg->rule, cfg->step,
                                            cfg->alpha, cfg->every, loads, calls,
                                            static_cast<hipStream_t>(stream));
  if (he != hipSuccess) return fail(MOER_EHIP, "balance_step launch: %s", hipGetErrorString(he));
  return ok();
}

}  // extern "C"
