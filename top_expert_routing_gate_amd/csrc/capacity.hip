// Capacity-limited routing.
//
// "MoE Routing Entropy vs Expert Saturation" (dailyaiworld), production
// testing section: every expert gets a hard token capacity (1.25 x T*K/N in
// the page's setting) and the tokens beyond it are routed to secondary
// candidate experts. Read as rounds of proposals:
//   round 0  every token proposes its top-K (the ordinary decision);
//   a round  each expert accepts that round's proposals in (token, slot)
//            order while it holds fewer than `cap` assignments, and rejects
//            the rest; accepted assignments stay;
//   then     every rejected slot proposes its token's next unused candidate
//            (eligible experts in decision order, a token's rejected slots
//            in slot order), or is dropped (id -1) when none is left;
// until nothing is pending. Shared slots are not limited.
//
// Kernels, after the selection (which wrote the masked keys and the scores)
// and the first layout (whose bucket ranks decide round 0, and which flags
// the layers with an expert over capacity; the other layers skip all of
// this):
//  1. cap_rank_kernel (one wavefront per token): a token with a slot past
//     its expert's capacity sorts its eligible experts (a 256-entry bitonic
//     sort of (key, id) across the wavefront) into its candidate list, and
//     makes its round-1 proposals.
//  2. Rounds 1 and 2 use the whole chip: the layout kernels rank each
//     round's proposals within their experts in (token, slot) order (the
//     stable counting sort the router's layout already is), and
//     cap_accept_kernel (one thread per token) accepts those whose rank fits
//     under what the expert holds, and makes the rejected slots' next
//     proposals.
//  3. cap_rounds_kernel (one workgroup per layer): the remaining rounds,
//     which are small. The pending slots form a list in (token, slot) order;
//     it is walked in chunks of 1024, one slot per thread: the slot's next
//     candidate comes from its token's list, its rank among the chunk's
//     proposals to the same expert from per-expert bitmaps in LDS
//     (popcounts, so the order is the list order), and the experts' running
//     counts carry the rank across chunks. Rejected slots are compacted, in
//     order, into the next round's list.
//  4. cap_weights_kernel: renormalised weights of the tokens that changed.
// The layout is then rebuilt from the final ids.
#include "moer_internal.hpp"

namespace moer {
namespace {

constexpr int kRankWaves = 4;          // tokens per workgroup in cap_rank_kernel
constexpr int kSortN = 256;            // bitonic sort width (>= N)
constexpr int kRoundThreads = 1024;    // cap_rounds_kernel workgroup = list chunk
constexpr int kChunkWords = kRoundThreads / 32;

__device__ __forceinline__ uint32_t float_order(float f) {  // monotone in f
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  const int lo = __shfl_xor((int)(uint32_t)v, m, kWave);
  const int hi = __shfl_xor((int)(uint32_t)(v >> 32), m, kWave);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ unsigned long long shfl_u64(unsigned long long v, int src) {
  const int lo = __shfl((int)(uint32_t)v, src, kWave);
  const int hi = __shfl((int)(uint32_t)(v >> 32), src, kWave);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Per-token candidate lists for tokens with a slot rejected in round 0.
// SN: sort width, a power of two >= the most experts a token can be eligible
// for (the kept groups' experts); the eligible entries are packed into the
// first SN places before the sort.
template <int SN>
__global__ __launch_bounds__(kRankWaves* kWave) void cap_rank_kernel(CapArgs c) {
  static_assert(SN >= kWave && SN <= kSortN, "sort width");
  __shared__ unsigned long long pack[kRankWaves][SN];
  const int lane = threadIdx.x & 63;
  const int layer = blockIdx.y;
  {
    // clear the grid rounds' segment totals
    const int64_t g = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * gridDim.y * blockDim.x;
    const int64_t nseg = (int64_t)c.L * c.nseg * c.N;
    for (int r = 0; r < kCapGridRounds; ++r)
      for (int64_t i = g; i < nseg; i += stride) c.round[r].segsum[i] = 0;
  }
  const int t = blockIdx.x * kRankWaves + (threadIdx.x >> 6);
  if (t >= c.T || c.flag[layer] == 0) return;
  const int N = c.N, K = c.K, Kt = c.Kt;
  const size_t tok = (size_t)layer * c.T + t;
  const int32_t* off = c.offsets + (size_t)layer * (c.Nb + 1);
  bool rejected = false;
  if (lane < K) {
    const size_t slot = tok * Kt + lane;
    const int e = c.idx[slot];
    const int p = c.inv_perm[slot];
    rejected = e >= 0 && e < N && p - off[e] >= c.cap;
  }
  const unsigned long long rmask = __ballot(rejected);
  const int n_rej = __builtin_popcountll(rmask);
  if (lane == 0) {
    c.changed[tok] = 0;
    c.round[0].mask[tok] = (int32_t)rmask;
    c.next[tok] = K + n_rej;  // round 1 takes candidates K .. K + n_rej - 1
  }
  if (rmask == 0) {
    if (lane < K) c.round[0].prop[tok * K + lane] = -1;
    return;
  }

  // (order(key), 0xFFFF - id): larger = earlier in decision order; 0 = not
  // eligible (or absent). Eligible entries are packed (in expert order) into
  // the wavefront's LDS row, then element i of the sort is pack[i].
  const float* key = c.key + tok * N;
  unsigned long long* row = pack[threadIdx.x >> 6];
  int n_el = 0;
#pragma unroll
  for (int r = 0; r < kSortN / kWave; ++r) {
    const int e = r * kWave + lane;
    const float k = e < N ? key[e] : -__builtin_inff();
    // eligible: not -inf (masked or absent) and not NaN. Decided on the bits:
    // the float compare k > -inf has been lowered as an ordered compare for
    // the store below and an unordered one for the ballot, which counted NaN
    // keys that were never stored.
    const uint32_t kb = __float_as_uint(k);
    const bool el = kb != 0xFF800000u && (kb & 0x7FFFFFFFu) <= 0x7F800000u;
    const unsigned long long m = __ballot(el);
    const int pos = n_el + __builtin_popcountll(m & ((1ull << lane) - 1ull));
    // more than SN only with non-finite scores (unspecified results): stay in bounds
    if (el && pos < SN) row[pos] = ((unsigned long long)float_order(k) << 16) | (unsigned)(0xFFFF - e);
    n_el += __builtin_popcountll(m);  // the same in every lane
  }
  n_el = n_el < SN ? n_el : SN;
  // a wavefront's LDS operations complete in order; keep the compiler from
  // moving the reads above the writes
  asm volatile("" ::: "memory");
  unsigned long long v[SN / kWave];
#pragma unroll
  for (int r = 0; r < SN / kWave; ++r) {
    const int i = r * kWave + lane;
    v[r] = i < n_el ? row[i] : 0ull;
  }
  // bitonic sort, descending, of element i = r*64 + lane
#pragma unroll
  for (int k = 2; k <= SN; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= kWave) {
        const int rj = j / kWave;
#pragma unroll
        for (int r = 0; r < SN / kWave; ++r) {
          if (r & rj) continue;
          const int i = r * kWave + lane;
          const bool desc = (i & k) == 0;
          const unsigned long long a = v[r], b = v[r | rj];
          const bool sw = desc ? (a < b) : (a > b);
          v[r] = sw ? b : a;
          v[r | rj] = sw ? a : b;
        }
      } else {
#pragma unroll
        for (int r = 0; r < SN / kWave; ++r) {
          const int i = r * kWave + lane;
          const unsigned long long o = shfl_xor_u64(v[r], j);
          const bool lower = (lane & j) == 0;
          const bool desc = (i & k) == 0;
          const bool take_max = lower == desc;
          v[r] = take_max ? (o > v[r] ? o : v[r]) : (o < v[r] ? o : v[r]);
        }
      }
    }
  }
  uint8_t* list = c.ranked + tok * kMaxExperts;
#pragma unroll
  for (int r = 0; r < SN / kWave; ++r) {
    const int i = r * kWave + lane;
    if (i < n_el) list[i] = (uint8_t)(0xFFFF - (unsigned)(v[r] & 0xFFFF));
  }
  if (lane == 0) c.n_el[tok] = n_el;
  // round 1: the j-th rejected slot (slot order) proposes candidate K + j
  // (the shuffles run in every lane; only rejected slots store)
  const int j = __builtin_popcountll(rmask & ((1ull << lane) - 1ull));
  const int ci = rejected ? K + j : 0;
  int e = -1;
#pragma unroll
  for (int r = 0; r < SN / kWave; ++r) {
    const unsigned long long x = shfl_u64(v[r], ci & 63);  // element ci
    if (r == (ci >> 6)) e = (int)(0xFFFF - (unsigned)(x & 0xFFFF));
  }
  if (lane < K) c.round[0].prop[tok * K + lane] = (rejected && ci < n_el) ? e : -1;
}

// What expert e holds before grid round r (0-based): the first layout's
// count, then each earlier round's proposals, every step capped.
__device__ __forceinline__ int held_before(const CapArgs& c, int layer, int e, int r) {
  const int32_t* o0 = c.offsets + (size_t)layer * (c.Nb + 1);
  int h = min(o0[e + 1] - o0[e], c.cap);
  for (int i = 0; i < r; ++i) {
    const int32_t* oi = c.round[i].offsets + (size_t)layer * (c.N + 1);
    h = min(h + (oi[e + 1] - oi[e]), c.cap);
  }
  return h;
}

// Grid round r (0-based): accept the round's proposals whose rank within
// their expert fits under what the expert holds; the rejected slots of a
// token take its next candidates, in slot order, as the next round's
// proposals. One thread per token.
constexpr int kAcceptThreads = 64;  // small workgroups: the work is latency, spread it wide

__global__ __launch_bounds__(kAcceptThreads) void cap_accept_kernel(CapArgs c, int r) {
  __shared__ int held[kMaxExperts];
  const int layer = blockIdx.y;
  const int t = blockIdx.x * kAcceptThreads + threadIdx.x;
  if (c.flag[layer] == 0) return;
  const int K = c.K, Kt = c.Kt;
  for (int e = threadIdx.x; e < c.N; e += kAcceptThreads) held[e] = held_before(c, layer, e, r);
  __syncthreads();
  int rerouted = 0, dropped = 0, pending = 0;
  if (t < c.T) {
    const size_t tok = (size_t)layer * c.T + t;
    const CapRound& cur = c.round[r];
    const CapRound& nxt = c.round[r + 1];
    const int m = cur.mask[tok];
    int nx = c.next[tok];
    const int ne = c.n_el[tok];
    const int32_t* off = cur.offsets + (size_t)layer * (c.N + 1);
    // every slot's proposal, rank and bucket start loaded together (the
    // latency chain is three loads deep, not three per slot)
    int pe[kMaxSlots], pos[kMaxSlots], base[kMaxSlots];
#pragma unroll
    for (int k = 0; k < kMaxSlots; ++k) {
      const bool on = k < K && ((m >> k) & 1);
      pe[k] = on ? cur.prop[tok * K + k] : -1;
      pos[k] = on ? cur.inv[tok * K + k] : 0;
    }
#pragma unroll
    for (int k = 0; k < kMaxSlots; ++k) base[k] = pe[k] >= 0 ? off[pe[k]] : 0;
    int rej = 0;
    bool touched = false;
#pragma unroll
    for (int k = 0; k < kMaxSlots; ++k) {
      if (k >= K || !((m >> k) & 1)) continue;
      const int e = pe[k];
      if (e < 0) {
        c.idx[tok * Kt + k] = -1;
        touched = true;
        ++dropped;
      } else if (held[e] + (pos[k] - base[k]) < c.cap) {
        c.idx[tok * Kt + k] = e;
        touched = true;
        ++rerouted;
      } else {
        rej |= 1 << k;
      }
    }
    if (touched) c.changed[tok] = 1;
    const uint8_t* list = c.ranked + tok * kMaxExperts;
    for (int k = 0; k < K; ++k) {
      int e = -1;
      if ((rej >> k) & 1) {
        e = nx < ne ? (int)list[nx] : -1;
        ++nx;
      }
      nxt.prop[tok * K + k] = e;
    }
    if (rej) c.next[tok] = nx;
    nxt.mask[tok] = rej;
    pending = __builtin_popcount(rej);
  }
  // this workgroup's (one wavefront's) reroute / drop / still-pending counts,
  // summed later by cap_rounds_kernel (one atomic per workgroup on the same
  // three counters serialised at the cache)
  static_assert(kAcceptThreads == kWave, "one wavefront per workgroup");
  for (int o = 32; o > 0; o >>= 1) {
    rerouted += __shfl_xor(rerouted, o, kWave);
    dropped += __shfl_xor(dropped, o, kWave);
    pending += __shfl_xor(pending, o, kWave);
  }
  if (threadIdx.x == 0) {
    int32_t* part = c.part + (((size_t)r * c.L + layer) * gridDim.x + blockIdx.x) * 3;
    part[0] = rerouted;
    part[1] = dropped;
    part[2] = pending;
  }
}

// Exclusive prefix of `flag` over the workgroup (in thread order); returns
// the thread's offset and sets *total.
__device__ __forceinline__ int block_prefix(int flag, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long m = __ballot(flag);
  const int below = __builtin_popcountll(m & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[wave] = __builtin_popcountll(m);
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < kRoundThreads / kWave; ++w) {
    const int c = wsum[w];
    base += w < wave ? c : 0;
    tot += c;
  }
  __syncthreads();  // wsum may be reused
  *total = tot;
  return base + below;
}

struct RoundsLds {
  int held[kMaxExperts];
  int run[kMaxExperts];
  unsigned bits[kMaxExperts][kChunkWords];  // proposals of the chunk per expert
  int wsum[kRoundThreads / kWave];
  int red[2][kRoundThreads / kWave];
};

__global__ __launch_bounds__(kRoundThreads) void cap_rounds_kernel(CapArgs c) {
  __shared__ RoundsLds sh;
  const int layer = blockIdx.x;
  const int N = c.N, K = c.K, Kt = c.Kt, T = c.T, cap = c.cap;
  const int tid = threadIdx.x;
  const int64_t A = (int64_t)T * K;
  int32_t* idx = c.idx + (size_t)layer * T * Kt;
  int32_t* next = c.next + (size_t)layer * T;
  const int32_t* n_el = c.n_el + (size_t)layer * T;
  const uint8_t* ranked = c.ranked + (size_t)layer * T * kMaxExperts;
  uint8_t* changed = c.changed + (size_t)layer * T;
  int32_t* lists[2] = {c.list0 + (size_t)layer * A, c.list1 + (size_t)layer * A};

  // the grid rounds' counts (one record per accept workgroup); rounds are
  // left only where they left slots pending
  int grid_rr = 0, grid_dr = 0, grid_pend = 0;
  if (c.flag[layer] != 0) {
    const int nwg = (T + kAcceptThreads - 1) / kAcceptThreads;
    for (int r = 0; r < kCapGridRounds; ++r) {
      const int32_t* part = c.part + ((size_t)r * c.L + layer) * nwg * 3;
      for (int w = tid; w < nwg; w += kRoundThreads) {
        grid_rr += part[3 * w];
        grid_dr += part[3 * w + 1];
        if (r == kCapGridRounds - 1) grid_pend += part[3 * w + 2];
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    grid_rr += __shfl_xor(grid_rr, o, kWave);
    grid_dr += __shfl_xor(grid_dr, o, kWave);
    grid_pend += __shfl_xor(grid_pend, o, kWave);
  }
  if ((tid & 63) == 0) {
    sh.red[0][tid >> 6] = grid_rr;
    sh.red[1][tid >> 6] = grid_dr;
    sh.wsum[tid >> 6] = grid_pend;
  }
  __syncthreads();
  grid_rr = grid_dr = grid_pend = 0;
  for (int w = 0; w < kRoundThreads / kWave; ++w) {
    grid_rr += sh.red[0][w];
    grid_dr += sh.red[1][w];
    grid_pend += sh.wsum[w];
  }
  __syncthreads();  // red and wsum are reused
  const bool any_over = c.flag[layer] != 0 && grid_pend != 0;
  int rerouted = 0, dropped = 0;
  if (any_over) {
    for (int e = tid; e < N; e += kRoundThreads) sh.held[e] = held_before(c, layer, e, kCapGridRounds);
    // the pending slots after the grid rounds, in (token, slot) order, from
    // the per-token masks: each wavefront takes 64 tokens, 16 per pass
    int P = 0;
    const int lane = tid & 63, wave = tid >> 6;
    const int32_t* mask = c.round[kCapGridRounds].mask + (size_t)layer * T;
    const int32_t* prop = c.round[kCapGridRounds].prop + (size_t)layer * A;
    int32_t* le = c.list_e + (size_t)layer * A;
    constexpr int kBatch = 16;  // passes whose masks are loaded together
    int mb[kBatch];
    for (int t0 = 0; t0 < T; t0 += kRoundThreads) {
      const int q = (t0 / kRoundThreads) % kBatch;
      if (q == 0) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int tu = t0 + u * kRoundThreads + wave * kWave + lane;
          mb[u] = tu < T ? mask[tu] : 0;
        }
      }
      const int t = t0 + wave * kWave + lane;
      int m = 0;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) m = u == q ? mb[u] : m;
      const int n = __builtin_popcount(m);
      int x = n;  // inclusive scan over the wavefront's tokens
      for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o, kWave);
        x += lane >= o ? y : 0;
      }
      if (lane == kWave - 1) sh.wsum[wave] = x;
      __syncthreads();
      int base = P, tot = 0;
      for (int w = 0; w < kRoundThreads / kWave; ++w) {
        base += w < wave ? sh.wsum[w] : 0;
        tot += sh.wsum[w];
      }
      int pos = base + x - n;
      for (int k = 0; k < K; ++k) {
        if (!((m >> k) & 1)) continue;
        const int a = t * K + k;
        lists[0][pos] = a;
        le[pos] = prop[a];
        ++pos;
      }
      __syncthreads();  // wsum is reused
      P += tot;
    }
    int cur = 0;
    bool first = true;  // proposals made by the last grid round
    while (P > 0) {  // P is the same in every thread
      // run[e]: this round's proposals to e in the chunks already walked
      for (int x = tid; x < N; x += kRoundThreads) sh.run[x] = 0;
      int Pn = 0;
      for (int i0 = 0; i0 < P; i0 += kRoundThreads) {
        const int i = i0 + tid;
        const int32_t* list = lists[cur];
        // advance: the slot's ordinal among its token's pending slots picks
        // the candidate; the token's last pending slot moves the pointer on
        int a = -1, t = -1, e = -1, new_next = -1;
        if (i < P && first) {
          a = list[i];
          t = a / K;
          e = le[i];
        } else if (i < P) {
          a = list[i];
          t = a / K;
          int ord = 0;
          for (int d = 1; d < K && i - d >= 0; ++d) {
            if (list[i - d] / K != t) break;
            ++ord;
          }
          const int ci = next[t] + ord;
          e = ci < n_el[t] ? (int)ranked[(size_t)t * kMaxExperts + ci] : -1;
          const bool last = (i + 1 >= P) || (list[i + 1] / K != t);
          if (last) new_next = ci + 1;
        }
        for (int w = tid; w < kMaxExperts * kChunkWords; w += kRoundThreads)
          (&sh.bits[0][0])[w] = 0u;
        __syncthreads();  // every read of next[] of this chunk is done
        if (new_next >= 0) next[t] = new_next;
        if (e >= 0) atomicOr(&sh.bits[e][tid >> 5], 1u << (tid & 31));
        __syncthreads();
        // accept while held + earlier proposals to the expert < cap
        int rej = 0;
        if (i < P) {
          const int64_t slot = (int64_t)t * Kt + a % K;
          if (e < 0) {
            idx[slot] = -1;
            changed[t] = 1;
            ++dropped;
          } else {
            int rank = __builtin_popcount(sh.bits[e][tid >> 5] & ((1u << (tid & 31)) - 1u));
            for (int w = 0; w < (tid >> 5); ++w) rank += __builtin_popcount(sh.bits[e][w]);
            if (sh.held[e] + sh.run[e] + rank < cap) {
              idx[slot] = e;
              changed[t] = 1;
              ++rerouted;
            } else {
              rej = 1;
            }
          }
        }
        __syncthreads();  // ranks read before the running counts move
        for (int x = tid; x < N; x += kRoundThreads) {
          int n = 0;
          for (int w = 0; w < kChunkWords; ++w) n += __builtin_popcount(sh.bits[x][w]);
          sh.run[x] += n;
        }
        int total;
        const int pos = block_prefix(rej, sh.wsum, &total);
        if (rej) lists[cur ^ 1][Pn + pos] = a;
        Pn += total;
      }
      for (int x = tid; x < N; x += kRoundThreads) {
        const int h = sh.held[x] + sh.run[x];
        sh.held[x] = h < cap ? h : cap;
      }
      __syncthreads();
      P = Pn;
      cur ^= 1;
      first = false;
    }
  }
  if (c.flag[layer] != 0) {
    // the final layout counts into cleared segment totals
    int32_t* seg = c.segsum + (size_t)layer * c.nseg * c.Nb;
    for (int x = tid; x < c.nseg * c.Nb; x += kRoundThreads) seg[x] = 0;
  }
  // counts of rerouted and dropped slots
  if (c.stats != nullptr) {
    int r = rerouted, d = dropped;
    for (int o = 32; o > 0; o >>= 1) {
      r += __shfl_xor(r, o, kWave);
      d += __shfl_xor(d, o, kWave);
    }
    if ((tid & 63) == 0) {
      sh.red[0][tid >> 6] = r;
      sh.red[1][tid >> 6] = d;
    }
    __syncthreads();
    if (tid == 0) {
      int rs = 0, ds = 0;
      for (int w = 0; w < kRoundThreads / kWave; ++w) {
        rs += sh.red[0][w];
        ds += sh.red[1][w];
      }
      c.stats[2 * layer] = rs + grid_rr;  // the grid rounds' counts too
      c.stats[2 * layer + 1] = ds + grid_dr;
    }
  }
}

// Weights of the tokens whose slots changed: the placed routed slots'
// scores over their sum (1/placed when the sum is 0); dropped slots 0.
__global__ __launch_bounds__(kAcceptThreads) void cap_weights_kernel(CapArgs c) {
  const int64_t tok = (int64_t)blockIdx.x * kAcceptThreads + threadIdx.x;
  if (tok >= (int64_t)c.L * c.T || c.flag[tok / c.T] == 0 || !c.changed[tok]) return;
  const int32_t* id = c.idx + tok * c.Kt;
  const float* s = c.s + tok * c.N;
  float z = 0.f;
  int placed = 0;
  for (int k = 0; k < c.K; ++k) {
    if (id[k] < 0) continue;
    z += s[id[k]];
    ++placed;
  }
  float* w = c.w + tok * c.Kt;
  for (int k = 0; k < c.K; ++k)
    w[k] = id[k] < 0 ? 0.f : (z > 0.f ? s[id[k]] / z : 1.f / (float)placed);
}

}  // namespace

hipError_t launch_capacity(const CapArgs& c, hipStream_t s) {
  if (c.T == 0) return hipSuccess;
  // sort width: the most experts a token can be eligible for, rounded up
  const int grid_x = (c.T + kRankWaves - 1) / kRankWaves;
  const int elig = c.G > 1 ? c.Gk * (c.N / c.G) : c.N;
  if (elig <= 64)
    hipLaunchKernelGGL(cap_rank_kernel<64>, dim3(grid_x, c.L), dim3(kRankWaves * kWave), 0, s, c);
  else if (elig <= 128)
    hipLaunchKernelGGL(cap_rank_kernel<128>, dim3(grid_x, c.L), dim3(kRankWaves * kWave), 0, s, c);
  else
    hipLaunchKernelGGL(cap_rank_kernel<256>, dim3(grid_x, c.L), dim3(kRankWaves * kWave), 0, s, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int r = 0; r < kCapGridRounds; ++r) {
    // rank the round's proposals within their experts: the layout kernels
    LayoutArgs la{};
    la.idx = c.round[r].prop;
    la.cnt = c.round[r].cnt;
    la.segsum = c.round[r].segsum;
    la.counts = c.round[r].counts;
    la.offsets = c.round[r].offsets;
    la.perm = c.round[r].perm;
    la.inv_perm = c.round[r].inv;
    la.T = c.T;
    la.Kt = c.K;
    la.Nb = c.N;
    la.N = c.N;
    la.nlb = c.nlb;
    la.nsb = c.nsb;
    la.nseg = c.nseg;
    la.need_count = 1;
    la.cap_phase = 2;  // layers without an expert over capacity skip
    la.cap_flag = const_cast<int32_t*>(c.flag);
    e = launch_layout(la, c.L, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(cap_accept_kernel, dim3((c.T + kAcceptThreads - 1) / kAcceptThreads, c.L),
                       dim3(kAcceptThreads), 0, s, c, r);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(cap_rounds_kernel, dim3(c.L), dim3(kRoundThreads), 0, s, c);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)c.L * c.T;
  hipLaunchKernelGGL(cap_weights_kernel, dim3((unsigned)((n + kAcceptThreads - 1) / kAcceptThreads)),
                     dim3(kAcceptThreads), 0, s, c);
  return hipGetLastError();
}

}  // namespace moer
