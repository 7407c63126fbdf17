// Gate affinities h = x · W_g^T (+ per-expert logit offset), fp32 result.
//
// "MoE Routing Entropy vs Expert Saturation" (dailyaiworld), Mathematics:
// the routing logits are h_i = x · W_g; its listing builds the gate as
// nn.Linear(hidden, experts, bias=False), i.e. W_g is [N][d] with one row
// per expert — the layout used here, so both operands are contiguous in the
// reduction dimension d.
//
// bf16 path: v_mfma_f32_16x16x32_bf16 (bf16 products are exact in fp32, the
// sum is accumulated in fp32). The MFMA "A" operand is a 16-expert slice of
// W_g and "B" a 16-token slice of x, so the 16x16 result block holds
// D[e][t]; lane l owns experts 4*(l/16)..+3 of token l%16 and writes them
// as one 16-byte store into h[t][e..e+3].
#include "moer_internal.hpp"

namespace moer {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kKStage = 64;              // reduction depth per LDS stage
constexpr int kChunks = kKStage / 8;     // 16-byte chunks per staged row

// One workgroup computes a BE-expert x BT-token tile over the full depth d.
// Waves are arranged WE x WT; each owns (BE/WE) x (BT/WT) in 16x16 blocks.
// Staging: both operand tiles go through LDS, double-buffered, 16-byte
// chunks swizzled by (chunk ^ row%8) so the MFMA fragment reads of 8
// consecutive rows hit 8 distinct 16-byte bank groups.
template <int BE, int BT, int WE, int WT>
__global__ __launch_bounds__(WE * WT * kWave) void gate_gemm_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W,
    const float* __restrict__ offset, float* __restrict__ h, int T, int d, int N) {
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

  // Global source of each chunk this thread stages (row pointer or null).
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

  const int frow = lane & 15;   // fragment row within a 16-row block
  const int fq = lane >> 4;     // fragment chunk (8 values of the reduction)
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

  // Epilogue: lane owns D[e..e+3][t].
#pragma unroll
  for (int i = 0; i < ME; ++i) {
    const int e = e0 + (we * ME + i) * 16 + 4 * fq;
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int t = t0 + (wt * MT + j) * 16 + frow;
      if (t >= T) continue;
      float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      if (offset != nullptr) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (e + r < N) v[r] += offset[e + r];
      }
      float* dst_row = h + (size_t)t * N;
      if (e + 3 < N && (N & 3) == 0) {
        *reinterpret_cast<floatx4*>(dst_row + e) = floatx4{v[0], v[1], v[2], v[3]};
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (e + r < N) dst_row[e + r] = v[r];
      }
    }
  }
}

// fp32 inputs (small routers): one thread per (token, expert) dot product,
// summed in ascending k.
__global__ __launch_bounds__(256) void gate_gemm_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ W, const float* __restrict__ offset,
    float* __restrict__ h, int T, int d, int N) {
  const int layer = blockIdx.y;
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)T * N) return;
  const int t = (int)(i / N);
  const int e = (int)(i % N);
  const float* xt = x + ((size_t)layer * T + t) * d;
  const float* we = W + ((size_t)layer * N + e) * d;
  float acc = 0.f;
  for (int k = 0; k < d; ++k) acc = __builtin_fmaf(xt[k], we[k], acc);
  if (offset != nullptr) acc += offset[e];
  h[((size_t)layer * T + t) * N + e] = acc;
}

template <int BE, int BT, int WE, int WT>
hipError_t launch_tile(const void* x, const void* w, const float* offset, float* h, int L, int T,
                       int d, int N, hipStream_t s) {
  dim3 grid((T + BT - 1) / BT, (N + BE - 1) / BE, L);
  hipLaunchKernelGGL((gate_gemm_bf16_kernel<BE, BT, WE, WT>), grid, dim3(WE * WT * kWave), 0, s,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), offset, h,
                     T, d, N);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_gemm_bf16(const void* x, const void* w, const float* offset, float* h,
                                 int L, int T, int d, int N, hipStream_t s) {
  if (N <= 16) return launch_tile<16, 64, 1, 4>(x, w, offset, h, L, T, d, N, s);
  const long long big_tiles = (long long)L * ((T + 63) / 64) * ((N + 255) / 256);
  if (N > 128 && big_tiles >= 256) return launch_tile<256, 64, 4, 1>(x, w, offset, h, L, T, d, N, s);
  return launch_tile<64, 128, 1, 4>(x, w, offset, h, L, T, d, N, s);
}

hipError_t launch_gate_gemm_f32(const float* x, const float* w, const float* offset, float* h,
                                int L, int T, int d, int N, hipStream_t s) {
  const long long n = (long long)T * N;
  dim3 grid((unsigned)((n + 255) / 256), L);
  hipLaunchKernelGGL(gate_gemm_f32_kernel, grid, dim3(256), 0, s, x, w, offset, h, T, d, N);
  return hipGetLastError();
}

}  // namespace moer
