// Gate affinities h = x · W_g^T as fp32 partial sums over split ranges of d
// ("MoE Routing Entropy vs Expert Saturation", Mathematics: h_i = x · W_g;
// W_g is [N][d], one row per expert).
//
// The depth d is split into `ksplit` equal ranges; range s writes
// part[s][l][t][e]. The selection kernel adds the ranges in order s = 0, 1,
// ... (and the logit offset), so the result is deterministic. The pipelined
// tile (gemm_pipeline.hpp) needs d to be a multiple of 64 per range; other d
// take the register-staged kernel below, fp32 inputs a plain FMA kernel.
#include <hip/hip_ext.h>

#include "gemm_pipeline.hpp"

namespace moer {
namespace {

// Partial affinities leave through an LDS transpose as whole rows (true) or
// straight from the accumulators (false).
constexpr bool kStoreViaLds = true;

// ---------------------------------------------------------------------------
// Pipelined kernel: producer waves stream the tiles, consumer waves run the
// MFMAs and store the depth range's partial affinities.
template <int BT, int BE, int WT, int WE, int NP, int NSTAGE>
__global__ __launch_bounds__((WT * WE + NP) * kWave, 1) void gate_gemm_dma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, float* __restrict__ part,
    int L, int T, int d, int N, int ksplit, int n_tt, int n_te, int n_work, int per_xcd,
    int32_t* __restrict__ zero, int n_zero) {
  using P = GemmPipeline<BT, BE, WT, WE, NP, NSTAGE>;
  __shared__ u32x4 ring[NSTAGE][P::kStageSlots];
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < n_zero; i += P::kThreads) zero[i] = 0;
  GemmWork w;
  if (!decode_work(n_tt, n_te, ksplit, n_work, per_xcd, w)) return;
  const int t0 = w.tt * BT, e0 = w.te * BE;
  const int krange = d / ksplit;
  const int nk = krange / kKStage;
  x += (size_t)w.layer * T * d;
  W += (size_t)w.layer * N * d;
  const int wave = threadIdx.x >> 6;
  float* out = part + ((size_t)w.ks * L + w.layer) * T * N;
  floatx4 acc[P::ME][P::MT];
  if (wave >= P::kConsumers) {
    P::produce(ring, x, W, t0, e0, T, N, d, w.ks * krange, nk, wave - P::kConsumers);
    if (!kStoreViaLds) return;
  } else {
    P::consume(ring, nk, wave / WE, wave % WE, acc);
    if (!kStoreViaLds) {
      P::store(acc, out, t0, e0, T, N, wave / WE, wave % WE);
      return;
    }
  }
  __syncthreads();  // the ring is free
  P::store_tile_lds(ring, acc, out, t0, e0, T, N);
}

// ---------------------------------------------------------------------------
// General kernel (any d with d % 8 == 0): register-staged, double-buffered
// LDS, zero-filled tails. One depth range (ksplit = 1).
template <int BE, int BT, int WE, int WT>
__global__ __launch_bounds__(WE * WT * kWave) void gate_gemm_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, float* __restrict__ h, int T,
    int d, int N) {
  constexpr int kThreads = WE * WT * kWave;
  constexpr int kRows = BE + BT;
  constexpr int kStageChunks = kRows * kChunks;
  constexpr int kPerThread = (kStageChunks + kThreads - 1) / kThreads;
  constexpr int ME = BE / WE / 16;
  constexpr int MT = BT / WT / 16;
  static_assert(BE % (WE * 16) == 0 && BT % (WT * 16) == 0, "tile shape");

  __shared__ u32x4 lds[2][kStageChunks];

  const int layer = blockIdx.z;
  x += (size_t)layer * T * d;
  W += (size_t)layer * N * d;
  h += (size_t)layer * T * N;
  const int t0 = blockIdx.x * BT;
  const int e0 = blockIdx.y * BE;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int we = wave / WT;
  const int wt = wave % WT;

  const uint16_t* src[kPerThread];
  int dst[kPerThread];
  int col[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int c = tid + i * kThreads;
    src[i] = nullptr;
    dst[i] = -1;
    col[i] = 0;
    if (c < kStageChunks) {
      const int r = c / kChunks;
      const int q = c % kChunks;
      dst[i] = r * kChunks + (q ^ (r & 7));
      col[i] = q * 8;
      if (r < BE) {
        if (e0 + r < N) src[i] = W + (size_t)(e0 + r) * d;
      } else {
        if (t0 + r - BE < T) src[i] = x + (size_t)(t0 + r - BE) * d;
      }
    }
  }

  u32x4 stage[kPerThread];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int k = k0 + col[i];
      if (src[i] != nullptr && k < d)
        stage[i] = *reinterpret_cast<const u32x4*>(src[i] + k);
      else
        stage[i] = u32x4{0, 0, 0, 0};
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i)
      if (dst[i] >= 0) lds[buf][dst[i]] = stage[i];
  };

  floatx4 acc[ME][MT];
#pragma unroll
  for (int i = 0; i < ME; ++i)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nk = (d + kKStage - 1) / kKStage;
  fetch(0);
  commit(0);
  __syncthreads();

  const int frow = lane & 15;
  const int fq = lane >> 4;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) fetch((kt + 1) * kKStage);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 a[ME], b[MT];
#pragma unroll
      for (int i = 0; i < ME; ++i) {
        const int r = (we * ME + i) * 16 + frow;
        const int q = kk * 4 + fq;
        a[i] = __builtin_bit_cast(bf16x8, lds[buf][r * kChunks + (q ^ (r & 7))]);
      }
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const int r = BE + (wt * MT + j) * 16 + frow;
        const int q = kk * 4 + fq;
        b[j] = __builtin_bit_cast(bf16x8, lds[buf][r * kChunks + (q ^ (r & 7))]);
      }
#pragma unroll
      for (int i = 0; i < ME; ++i)
#pragma unroll
        for (int j = 0; j < MT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) commit(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < ME; ++i) {
    const int e = e0 + (we * ME + i) * 16 + 4 * fq;
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int t = t0 + (wt * MT + j) * 16 + frow;
      if (t >= T) continue;
      float* dst_row = h + (size_t)t * N;
      if (e + 3 < N && (N & 3) == 0) {
        *reinterpret_cast<floatx4*>(dst_row + e) = acc[i][j];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (e + r < N) dst_row[e + r] = acc[i][j][r];
      }
    }
  }
}

// fp32 inputs (small routers): one thread per (token, expert) dot product,
// summed in ascending k. Rows are read as 16-byte vectors, eight per
// operand in flight, when d allows (the sum order is the same).
__global__ __launch_bounds__(256) void gate_gemm_f32_kernel(const float* __restrict__ x,
                                                            const float* __restrict__ W,
                                                            float* __restrict__ h, int T, int d,
                                                            int N, int32_t* __restrict__ zero,
                                                            int n_zero) {
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int z = threadIdx.x; z < n_zero; z += blockDim.x) zero[z] = 0;
  const int layer = blockIdx.y;
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)T * N) return;
  const int t = (int)(i / N);
  const int e = (int)(i % N);
  const float* xt = x + ((size_t)layer * T + t) * d;
  const float* we = W + ((size_t)layer * N + e) * d;
  float acc = 0.f;
  int k = 0;
  if ((d & 3) == 0 && ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(W)) & 15) == 0) {
    const float4* x4 = reinterpret_cast<const float4*>(xt);
    const float4* w4 = reinterpret_cast<const float4*>(we);
#pragma unroll 8
    for (int k4 = 0; k4 < d / 4; ++k4) {
      const float4 a = x4[k4], b = w4[k4];
      acc = __builtin_fmaf(a.x, b.x, acc);
      acc = __builtin_fmaf(a.y, b.y, acc);
      acc = __builtin_fmaf(a.z, b.z, acc);
      acc = __builtin_fmaf(a.w, b.w, acc);
    }
    k = d;
  }
  for (; k < d; ++k) acc = __builtin_fmaf(xt[k], we[k], acc);
  h[((size_t)layer * T + t) * N + e] = acc;
}

// ev0 / ev1 (may be null): recorded by the launch itself at the kernel's
// start and end (the dispatch's own timestamps), for profiling.
template <int BT, int BE, int WT, int WE, int NP, int NSTAGE>
hipError_t launch_dma(const void* x, const void* w, float* part, int L, int T, int d, int N,
                      int ksplit, int32_t* zero, int n_zero, hipStream_t s, hipEvent_t ev0,
                      hipEvent_t ev1) {
  const int n_tt = (T + BT - 1) / BT;
  const int n_te = (N + BE - 1) / BE;
  const int n_work = L * ksplit * n_te * n_tt;
  const int per_xcd = (n_work + 7) / 8;
  hipExtLaunchKernelGGL((gate_gemm_dma_kernel<BT, BE, WT, WE, NP, NSTAGE>), dim3(8 * per_xcd),
                        dim3((WT * WE + NP) * kWave), 0, s, ev0, ev1, 0,
                        static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), part, L,
                        T, d, N, ksplit, n_tt, n_te, n_work, per_xcd, zero, n_zero);
  return hipGetLastError();
}

template <int BE, int BT, int WE, int WT>
hipError_t launch_tile(const void* x, const void* w, float* h, int L, int T, int d, int N,
                       hipStream_t s) {
  dim3 grid((T + BT - 1) / BT, (N + BE - 1) / BE, L);
  hipLaunchKernelGGL((gate_gemm_bf16_kernel<BE, BT, WE, WT>), grid, dim3(WE * WT * kWave), 0, s,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), h, T, d,
                     N);
  return hipGetLastError();
}

// Tile of the pipelined kernel: 64 tokens x 32 experts for small routers,
// and for batches too small to give the 128 x 256 tile 32 work items (a
// one-layer decode batch: its one 128 x 256 tile would leave all but a few
// CUs idle); 128 x 256 otherwise.
bool small_tile(int L, int T, int N) {
  return N <= 32 || (long long)L * ((T + 127) / 128) * ((N + 255) / 256) < 32;
}
constexpr int kMaxSplit = 16;  // depth ranges at most
// 128 x 128 for large routers with decode-sized layers (at most two
// 128-token tiles per layer, so W_g streams from HBM rather than being
// re-read from L2) whose batch gives the 128 x 256 tile fewer than 128 work
// items (the 64-layer decode batch): twice the tiles, so half the depth
// ranges, and half the partial affinities written and read back.
bool mid_tile(int L, int T, int N) {
  return !small_tile(L, T, N) && N > 128 && (T + 127) / 128 <= 2 &&
         (long long)L * ((T + 127) / 128) * ((N + 255) / 256) < 128;
}

}  // namespace

int gate_gemm_ksplit(int dtype_bf16, int L, int T, int d, int N) {
  if (!dtype_bf16 || T == 0 || d % kKStage != 0) return 1;
  const bool small = small_tile(L, T, N);
  const int bt = small ? 64 : 128;
  const int be = small ? 32 : (mid_tile(L, T, N) ? 128 : 256);
  const long long tiles = (long long)L * ((T + bt - 1) / bt) * ((N + be - 1) / be);
  int ks = 1;
  while (ks < kMaxSplit && tiles * ks < 256 && d % (kKStage * ks * 2) == 0) ks *= 2;
  return ks;
}

bool gate_gemm_clears(int L, int T, int d, int N, int ksplit) {
  return L > 0 && T > 0 && d % (kKStage * ksplit) == 0;
}

__global__ void zero_ints_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_zero_ints(int32_t* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_ints_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_gate_gemm_bf16(const void* x, const void* w, float* part, int L, int T, int d,
                                 int N, int ksplit, int32_t* zero, int n_zero, hipStream_t s,
                                 hipEvent_t ev0, hipEvent_t ev1) {
  if (d % (kKStage * ksplit) == 0) {
    if (mid_tile(L, T, N))
      return launch_dma<128, 128, 2, 2, 4, 3>(x, w, part, L, T, d, N, ksplit, zero, n_zero, s, ev0,
                                              ev1);
    if (small_tile(L, T, N))
      return launch_dma<64, 32, 4, 1, 4, 3>(x, w, part, L, T, d, N, ksplit, zero, n_zero, s, ev0,
                                            ev1);
    return launch_dma<128, 256, 2, 2, 4, 3>(x, w, part, L, T, d, N, ksplit, zero, n_zero, s, ev0,
                                            ev1);
  }
  if (ksplit != 1) return hipErrorInvalidValue;
  hipError_t e = ev0 != nullptr ? hipEventRecord(ev0, s) : hipSuccess;
  if (e == hipSuccess)
    e = N <= 16 ? launch_tile<16, 64, 1, 4>(x, w, part, L, T, d, N, s)
                : launch_tile<64, 128, 1, 4>(x, w, part, L, T, d, N, s);
  if (e == hipSuccess && ev1 != nullptr) e = hipEventRecord(ev1, s);
  return e;
}

hipError_t launch_gate_gemm_f32(const float* x, const float* w, float* h, int L, int T, int d,
                                int N, int32_t* zero, int n_zero, hipStream_t s) {
  const long long n = (long long)T * N;
  dim3 grid((unsigned)((n + 255) / 256), L);
  hipLaunchKernelGGL(gate_gemm_f32_kernel, grid, dim3(256), 0, s, x, w, h, T, d, N, zero, n_zero);
  return hipGetLastError();
}

}  // namespace moer
