// Local dispatch and weighted combine: the single-device part of moving
// tokens to their experts and back.
//
// hotdry "DeepSeek V4 MoE load balancing", DeepEP section: dispatch sends
// each token's hidden state to the experts it was routed to, combine brings
// the expert results back to the token. Same page, token routing section:
// the layer output is the sum of the chosen experts' outputs, each weighted
// by its routing weight. On one device both steps are permutations through
// the dispatch layout (perm / inv_perm of the router).
//
// Both kernels walk tokens, not layout positions, so every token row is read
// once by dispatch and written once by combine:
//   dispatch: read x[t] (one row), write it to the Kt positions inv_perm
//             names (Kt rows);
//   combine:  read the Kt expert-output rows of token t, write y[t].
// One wavefront per token; the token's Kt positions and weights sit one per
// lane and are broadcast with readlane. Rows are moved in 16-byte chunks,
// lane-interleaved, with several chunks per lane in flight before the first
// use. Both are HBM-bound copies: no LDS, no cross-wave traffic.
//
// Cache policy, measured on MI355X at 16384 tokens x 7168 x top-8: the
// dispatched rows are written with non-temporal stores (they are not read
// again by this kernel; 5.9 TB/s against 5.0 with plain stores), and the
// expert-output rows the combine gathers are read with non-temporal loads
// (each is read once; 5.55 TB/s against 4.9). Non-temporal loads in the
// dispatch and non-temporal stores of y were slower.
#include "moer_internal.hpp"

namespace moer {
namespace {

constexpr int kTokWaves = 4;         // tokens (wavefronts) per workgroup
constexpr int kDispatchUnroll = 8;   // 16-byte chunks per lane in flight (dispatch)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Wave-uniform token index of this wavefront.
__device__ __forceinline__ int64_t wave_token() {
  return (int64_t)blockIdx.x * kTokWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Copy chunks c0 + u*64 + lane (u < kDispatchUnroll) of one token row to
// each of its placed positions; kTail checks the row end.
template <bool kTail>
__device__ __forceinline__ void dispatch_group(const u32x4* src, u32x4* dst_layer, int64_t chunks,
                                               int64_t c0, int lane, int Kt, int my_pos) {
  u32x4 v[kDispatchUnroll];
#pragma unroll
  for (int u = 0; u < kDispatchUnroll; ++u) {
    // in the tail, lanes past the row end re-read its last chunk (unused)
    const int64_t c = c0 + u * kWave + lane;
    v[u] = src[kTail && c >= chunks ? chunks - 1 : c];
  }
  for (int k = 0; k < Kt; ++k) {
    const int p = __builtin_amdgcn_readlane(my_pos, k);
    if (p < 0) continue;
    u32x4* dst = dst_layer + (int64_t)p * chunks;
#pragma unroll
    for (int u = 0; u < kDispatchUnroll; ++u) {
      const int64_t c = c0 + u * kWave + lane;
      if (!kTail || c < chunks) __builtin_nontemporal_store(v[u], dst + c);
    }
  }
}

__global__ __launch_bounds__(kTokWaves* kWave) void dispatch_kernel(
    const u32x4* __restrict__ x, int64_t chunks, int64_t n_tok, int T, int Kt,
    const int32_t* __restrict__ inv_perm, u32x4* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t g = wave_token();
  if (g >= n_tok) return;
  const int64_t rows = (int64_t)T * Kt;  // layout positions per layer
  int my_pos = -1;
  if (lane < Kt) {
    const int p = inv_perm[g * Kt + lane];
    my_pos = (p >= 0 && p < rows) ? p : -1;
  }
  const u32x4* src = x + g * chunks;
  u32x4* dst_layer = out + (g / T) * rows * chunks;
  constexpr int kGroup = kWave * kDispatchUnroll;
  int64_t c0 = 0;
  for (; c0 + kGroup <= chunks; c0 += kGroup)
    dispatch_group<false>(src, dst_layer, chunks, c0, lane, Kt, my_pos);
  if (c0 < chunks) dispatch_group<true>(src, dst_layer, chunks, c0, lane, Kt, my_pos);
}

// Eight consecutive elements (one chunk of the combine) as loaded; they are
// widened to fp32 only when used, so the loads in flight hold raw bits.
template <typename TIn>
struct Raw8;
template <>
struct Raw8<uint16_t> {  // bf16
  u32x4 r;
  __device__ __forceinline__ void load(const uint16_t* p) {
    r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  __device__ __forceinline__ float at(int e) const {
    const uint32_t word = r[e >> 1];
    return __uint_as_float((e & 1) ? (word & 0xFFFF0000u) : (word << 16));
  }
};
template <>
struct Raw8<float> {
  u32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 4));
  }
  __device__ __forceinline__ float at(int e) const { return __uint_as_float(e < 4 ? a[e] : b[e - 4]); }
};

__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));  // round to nearest even
}

__device__ __forceinline__ void store8(uint16_t* p, const float (&a)[8]) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = bf16_bits(a[2 * i]) | (bf16_bits(a[2 * i + 1]) << 16);
  *reinterpret_cast<u32x4*>(p) = r;
}

__device__ __forceinline__ void store8(float* p, const float (&a)[8]) {
  u32x4 r0, r1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r0[i] = __float_as_uint(a[i]);
    r1[i] = __float_as_uint(a[4 + i]);
  }
  *reinterpret_cast<u32x4*>(p) = r0;
  *reinterpret_cast<u32x4*>(p + 4) = r1;
}

// y[g] = sum over slots k (in slot order) of w[g][k] * eo[pos_k], fp32 fma,
// one rounding to TOut at the end. KT (the slot count) is a template
// parameter so that every slot's loads are issued together, unconditionally:
// a slot without a position reads row 0 of its layer (in bounds) and skips
// its multiply-add. Each lane keeps about 16 chunk loads in flight.
template <typename TIn, typename TOut, int KT>
__global__ __launch_bounds__(kTokWaves* kWave) void combine_kernel(
    const TIn* __restrict__ eo, const float* __restrict__ w, const int32_t* __restrict__ inv_perm,
    int64_t n_tok, int T, int d, TOut* __restrict__ y) {
  constexpr int U = (sizeof(TIn) == 2 ? 16 : 8) / KT > 0 ? (sizeof(TIn) == 2 ? 16 : 8) / KT : 1;
  const int lane = threadIdx.x & 63;
  const int64_t g = wave_token();
  if (g >= n_tok) return;
  const int64_t rows = (int64_t)T * KT;
  int my_pos = -1;
  float my_w = 0.f;
  if (lane < KT) {
    const int p = inv_perm[g * KT + lane];
    my_pos = (p >= 0 && p < rows) ? p : -1;
    my_w = w[g * KT + lane];
  }
  int pos[KT];
  float wt[KT];
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    pos[k] = __builtin_amdgcn_readlane(my_pos, k);
    wt[k] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), k));
  }
  const TIn* layer_rows = eo + (g / T) * rows * d;
  TOut* yrow = y + g * d;
  const int n8 = d / 8;
  for (int c0 = 0; c0 < n8; c0 += kWave * U) {
    Raw8<TIn> v[KT][U];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      const TIn* row = layer_rows + (int64_t)(pos[k] < 0 ? 0 : pos[k]) * d;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // lanes past the row end re-read its last chunk (in bounds, unused)
        const int c = min(c0 + u * kWave + lane, n8 - 1);
        v[k][u].load(row + (int64_t)c * 8);
      }
    }
    float acc[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[u][e] = 0.f;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      if (pos[k] < 0) continue;
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[u][e] = fmaf(wt[k], v[k][u].at(e), acc[u][e]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave + lane;
      if (c < n8) store8(yrow + (int64_t)c * 8, acc[u]);
    }
  }
}

template <typename TIn, typename TOut, int KT>
hipError_t launch_combine_k(const void* eo, const float* w, const int32_t* inv_perm, int L, int T,
                            int Kt, int d, void* y, hipStream_t s) {
  if (Kt != KT) {
    if constexpr (KT < kMaxSlots)
      return launch_combine_k<TIn, TOut, KT + 1>(eo, w, inv_perm, L, T, Kt, d, y, s);
    return hipErrorInvalidValue;
  } else {
    const int64_t n_tok = (int64_t)L * T;
    const int64_t grid = (n_tok + kTokWaves - 1) / kTokWaves;
    hipLaunchKernelGGL((combine_kernel<TIn, TOut, KT>), dim3((unsigned)grid),
                       dim3(kTokWaves * kWave), 0, s, static_cast<const TIn*>(eo), w, inv_perm,
                       n_tok, T, d, static_cast<TOut*>(y));
    return hipGetLastError();
  }
}

}  // namespace

hipError_t launch_dispatch(const void* x, int64_t row_bytes, int L, int T, int Kt,
                           const int32_t* inv_perm, void* out, hipStream_t s) {
  const int64_t n_tok = (int64_t)L * T;
  if (n_tok == 0) return hipSuccess;
  const int64_t grid = (n_tok + kTokWaves - 1) / kTokWaves;
  hipLaunchKernelGGL(dispatch_kernel, dim3((unsigned)grid), dim3(kTokWaves * kWave), 0, s,
                     static_cast<const u32x4*>(x), row_bytes / 16, n_tok, T, Kt, inv_perm,
                     static_cast<u32x4*>(out));
  return hipGetLastError();
}

hipError_t launch_combine(const void* eo, int eo_bf16, const float* w, const int32_t* inv_perm,
                          int L, int T, int Kt, int d, void* y, int y_bf16, hipStream_t s) {
  if ((int64_t)L * T == 0) return hipSuccess;
  if (eo_bf16)
    return y_bf16 ? launch_combine_k<uint16_t, uint16_t, 1>(eo, w, inv_perm, L, T, Kt, d, y, s)
                  : launch_combine_k<uint16_t, float, 1>(eo, w, inv_perm, L, T, Kt, d, y, s);
  return y_bf16 ? launch_combine_k<float, uint16_t, 1>(eo, w, inv_perm, L, T, Kt, d, y, s)
                : launch_combine_k<float, float, 1>(eo, w, inv_perm, L, T, Kt, d, y, s);
}

}  // namespace moer
