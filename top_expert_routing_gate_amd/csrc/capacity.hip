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
// and the first layout (whose bucket ranks decide round 0):
//  1. cap_rank_kernel (one wavefront per token): a token with a slot past
//     its expert's capacity sorts its eligible experts (a 256-entry bitonic
//     sort of (key, id) across the wavefront) into its candidate list.
//  2. cap_rounds_kernel (one workgroup per layer): every later round. The
//     pending slots form a list in (token, slot) order; it is walked in
//     chunks of 1024, one slot per thread: the slot's next candidate comes
//     from its token's list, its rank among the chunk's proposals to the
//     same expert from per-expert bitmaps in LDS (popcounts, so the order is
//     the list order), and the experts' running counts carry the rank across
//     chunks. Rejected slots are compacted, in order, into the next round's
//     list.
//  3. cap_weights_kernel: renormalised weights of the tokens that changed.
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

// Per-token candidate lists for tokens with a slot rejected in round 0.
__global__ __launch_bounds__(kRankWaves* kWave) void cap_rank_kernel(CapArgs c) {
  const int lane = threadIdx.x & 63;
  const int layer = blockIdx.y;
  const int t = blockIdx.x * kRankWaves + (threadIdx.x >> 6);
  if (t >= c.T) return;
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
  const bool affected = __ballot(rejected) != 0;
  if (lane == 0) {
    c.changed[tok] = 0;
    c.next[tok] = K;
    if (!affected) c.n_el[tok] = 0;
  }
  if (!affected) return;

  // (order(key), 0xFFFF - id): larger = earlier in decision order; 0 = not
  // eligible (or absent)
  unsigned long long v[kSortN / kWave];
  const float* key = c.key + tok * N;
  int n_el = 0;
#pragma unroll
  for (int r = 0; r < kSortN / kWave; ++r) {
    const int e = r * kWave + lane;
    const float k = e < N ? key[e] : -__builtin_inff();
    const bool el = k > -__builtin_inff();
    v[r] = el ? ((unsigned long long)float_order(k) << 16) | (unsigned)(0xFFFF - e) : 0ull;
    n_el += el ? 1 : 0;
  }
  // bitonic sort, descending, of element i = r*64 + lane
#pragma unroll
  for (int k = 2; k <= kSortN; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= kWave) {
        const int rj = j / kWave;
#pragma unroll
        for (int r = 0; r < kSortN / kWave; ++r) {
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
        for (int r = 0; r < kSortN / kWave; ++r) {
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
  for (int o = 32; o > 0; o >>= 1) n_el += __shfl_xor(n_el, o, kWave);
  uint8_t* list = c.ranked + tok * kMaxExperts;
#pragma unroll
  for (int r = 0; r < kSortN / kWave; ++r) {
    const int i = r * kWave + lane;
    if (i < n_el) list[i] = (uint8_t)(0xFFFF - (unsigned)(v[r] & 0xFFFF));
  }
  if (lane == 0) c.n_el[tok] = n_el;
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
  int off[kMaxExperts + 1];
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
  const int32_t* off = c.offsets + (size_t)layer * (c.Nb + 1);
  int32_t* idx = c.idx + (size_t)layer * T * Kt;
  const int32_t* inv = c.inv_perm + (size_t)layer * T * Kt;
  int32_t* next = c.next + (size_t)layer * T;
  const int32_t* n_el = c.n_el + (size_t)layer * T;
  const uint8_t* ranked = c.ranked + (size_t)layer * T * kMaxExperts;
  uint8_t* changed = c.changed + (size_t)layer * T;
  int32_t* lists[2] = {c.list0 + (size_t)layer * A, c.list1 + (size_t)layer * A};

  for (int e = tid; e <= N; e += kRoundThreads) sh.off[e] = off[e];
  __syncthreads();
  int over = 0;
  for (int e = tid; e < N; e += kRoundThreads) {
    const int n = sh.off[e + 1] - sh.off[e];
    sh.held[e] = n < cap ? n : cap;
    over |= n > cap ? 1 : 0;
  }
  const bool any_over = __syncthreads_or(over) != 0;
  int rerouted = 0, dropped = 0;
  if (any_over) {
    // round 0's rejections, compacted in (token, slot) order
    int P = 0;
    for (int64_t a0 = 0; a0 < A; a0 += kRoundThreads) {
      const int64_t a = a0 + tid;
      int rej = 0;
      if (a < A) {
        const int64_t slot = (a / K) * Kt + a % K;
        const int e = idx[slot];
        rej = (e >= 0 && e < N && inv[slot] - sh.off[e] >= cap) ? 1 : 0;
      }
      int total;
      const int pos = block_prefix(rej, sh.wsum, &total);
      if (rej) lists[0][P + pos] = (int32_t)a;
      P += total;
    }
    int cur = 0;
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
        if (i < P) {
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
    }
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
      c.stats[2 * layer] = rs;
      c.stats[2 * layer + 1] = ds;
    }
  }
}

// Weights of the tokens whose slots changed: the placed routed slots'
// scores over their sum (1/placed when the sum is 0); dropped slots 0.
__global__ __launch_bounds__(256) void cap_weights_kernel(CapArgs c) {
  const int64_t tok = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (tok >= (int64_t)c.L * c.T || !c.changed[tok]) return;
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
  hipLaunchKernelGGL(cap_rank_kernel, dim3((c.T + kRankWaves - 1) / kRankWaves, c.L),
                     dim3(kRankWaves * kWave), 0, s, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cap_rounds_kernel, dim3(c.L), dim3(kRoundThreads), 0, s, c);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)c.L * c.T;
  hipLaunchKernelGGL(cap_weights_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, c);
  return hipGetLastError();
}

}  // namespace moer
