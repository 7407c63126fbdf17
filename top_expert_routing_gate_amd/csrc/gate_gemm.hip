// Gate affinities h = x · W_g^T as fp32 partial sums over split ranges of d.
//
// "MoE Routing Entropy vs Expert Saturation" (dailyaiworld), Mathematics:
// the routing logits are h_i = x · W_g; its listing builds the gate as
// nn.Linear(hidden, experts, bias=False), i.e. W_g is [N][d] with one row
// per expert — the layout used here, so both operands are contiguous in the
// reduction dimension d.
//
// bf16 products are exact in fp32 and are accumulated in fp32 by
// v_mfma_f32_16x16x32_bf16. The MFMA "A" operand is a 16-expert slice of W_g
// and "B" a 16-token slice of x, so a 16x16 result block holds D[e][t]: lane
// l owns experts 4*(l/16)..+3 of token l%16 and stores them as one 16-byte
// write. The depth d is split into `ksplit` equal ranges; range s writes
// part[s][l][t][e]. The selection kernel adds the ranges in order s = 0, 1,
// ... (and the logit offset), so the result is deterministic.
#include "moer_internal.hpp"

namespace moer {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kKStage = 64;           // reduction depth per LDS stage (bf16)
constexpr int kChunks = kKStage / 8;  // 16-byte chunks per staged row

// s_waitcnt immediate (gfx9 encoding) for vmcnt <= n and lgkmcnt == 0: this
// wave's DMA stages up to the wanted one have landed and its own LDS reads
// have completed.
constexpr int wait_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }
constexpr int kNoVmWait = 63;  // vmcnt field at its maximum: wait for LDS only

// Workgroup barrier that orders LDS traffic at compile time only (asm memory
// clobbers); the hardware side is the explicit s_waitcnt before it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Pipelined kernel (d a multiple of 64 * ksplit).
//
// Workgroup tile: BT tokens x BE experts over one depth range. The
// workgroup's waves have two roles:
//  - WT x WE consumer waves, each owning (BT/WT) x (BE/WE) in 16x16 MFMA
//    blocks, read operand fragments from LDS and issue the MFMAs;
//  - NP producer waves stream the operand tiles into an NSTAGE-deep LDS ring
//    with global_load_lds_dwordx4 (no VGPR staging).
// Splitting the roles matters on CDNA: a wave that issues a long run of
// loads stalls in the issue stage while the memory pipeline back-pressures,
// and a wave's MFMAs cannot issue past its own stalled loads. With separate
// waves the matrix cores run while the producers wait.
//
// Each producer instruction fills 64 consecutive 16-byte LDS slots, and each
// lane fetches the global chunk that belongs in its slot under the XOR
// swizzle slot(r, q) = r*8 + (q ^ (r%8)), which makes the 16-byte fragment
// reads of 8 consecutive rows conflict-free. Rows past T or N are clamped to
// the last valid row (their results are never stored); d must be a multiple
// of the stage depth so no chunk is partial.
//
// One workgroup barrier per stage orders the ring: before barrier k the
// producers wait until their stage-k loads have landed, and the consumers
// have finished reading stage k-1; after it the consumers read stage k and
// the producers refill the buffer of stage k-1 with stage k+NSTAGE-1.
//
// Workgroups are numbered so that consecutive tiles of one (layer, depth
// range) land on the same XCD (dispatch is round-robin over the 8 XCDs):
// every XCD then streams one part of W_g through its own L2.
template <int BT, int BE, int WT, int WE, int NP, int NSTAGE>
__global__ __launch_bounds__((WT * WE + NP) * kWave, 1) void gate_gemm_dma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, float* __restrict__ part,
    int L, int T, int d, int N, int ksplit, int n_tt, int n_te, int n_work, int per_xcd) {
  constexpr int kConsumers = WT * WE;
  constexpr int kRows = BT + BE;
  constexpr int kStageSlots = kRows * kChunks;
  constexpr int kLoads = kStageSlots / (NP * kWave);  // DMA instructions per producer per stage
  constexpr int MT = BT / WT / 16;
  constexpr int ME = BE / WE / 16;
  static_assert(kStageSlots % (NP * kWave) == 0, "stage must split evenly over the producers");
  static_assert((NSTAGE - 2) * kLoads <= 63, "outstanding loads must fit the vmcnt field");
  static_assert(BT % (WT * 16) == 0 && BE % (WE * 16) == 0, "tile shape");

  __shared__ u32x4 ring[NSTAGE][kStageSlots];

  // XCD-aware work index: dispatch slot b runs on XCD b % 8.
  const int b = blockIdx.x;
  const int work = (b % 8) * per_xcd + b / 8;
  if (work >= n_work) return;
  int rest = work;
  const int tt = rest % n_tt; rest /= n_tt;
  const int te = rest % n_te; rest /= n_te;
  const int ks = rest % ksplit; rest /= ksplit;
  const int layer = rest;

  const int t0 = tt * BT, e0 = te * BE;
  const int krange = d / ksplit;
  const int kbeg = ks * krange;
  const int nk = krange / kKStage;
  x += (size_t)layer * T * d;
  W += (size_t)layer * N * d;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  if (wave >= kConsumers) {
    // ---- producer ----
    const int pw = wave - kConsumers;
    const uint16_t* src[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int slot = (i * NP + pw) * kWave + lane;
      const int r = slot / kChunks;
      const int q = (slot % kChunks) ^ (r & 7);
      const uint16_t* row = r < BT ? x + (size_t)min(t0 + r, T - 1) * d
                                   : W + (size_t)min(e0 + r - BT, N - 1) * d;
      src[i] = row + kbeg + q * 8;
    }
    auto issue = [&](int stage_k, int buf) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(src[i] + stage_k * kKStage),
                                         LDS_PTR(&ring[buf][(i * NP + pw) * kWave]), 16, 0, 0);
    };
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s)
      if (s < nk) issue(s, s);
    for (int k = 0; k < nk; ++k) {
      // stage k has landed once at most the later issued stages are pending
      if (k + NSTAGE - 2 < nk)
        __builtin_amdgcn_s_waitcnt(wait_imm((NSTAGE - 2) * kLoads));
      else
        __builtin_amdgcn_s_waitcnt(wait_imm(0));
      ring_barrier();
      if (k + NSTAGE - 1 < nk) issue(k + NSTAGE - 1, (k + NSTAGE - 1) % NSTAGE);
    }
    return;
  }

  // ---- consumer ----
  const int wt = wave / WE;
  const int we = wave % WE;
  floatx4 acc[ME][MT];
#pragma unroll
  for (int i = 0; i < ME; ++i)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int frow = lane & 15;
  const int fq = lane >> 4;
  for (int k = 0; k < nk; ++k) {
    // own fragment reads of stage k-1 complete before its buffer is refilled
    __builtin_amdgcn_s_waitcnt(wait_imm(kNoVmWait));
    ring_barrier();
    const u32x4* buf = ring[k % NSTAGE];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 a[ME], bb[MT];
      const int q = kk * 4 + fq;
#pragma unroll
      for (int i = 0; i < ME; ++i) {
        const int r = BT + (we * ME + i) * 16 + frow;
        a[i] = __builtin_bit_cast(bf16x8, buf[r * kChunks + (q ^ (r & 7))]);
      }
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const int r = (wt * MT + j) * 16 + frow;
        bb[j] = __builtin_bit_cast(bf16x8, buf[r * kChunks + (q ^ (r & 7))]);
      }
#pragma unroll
      for (int i = 0; i < ME; ++i)
#pragma unroll
        for (int j = 0; j < MT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
    }
  }

  float* out = part + ((size_t)ks * L + layer) * T * N;
#pragma unroll
  for (int i = 0; i < ME; ++i) {
    const int e = e0 + (we * ME + i) * 16 + 4 * fq;
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int t = t0 + (wt * MT + j) * 16 + frow;
      if (t >= T) continue;
      float* row = out + (size_t)t * N;
      if (e + 3 < N && (N & 3) == 0) {
        *reinterpret_cast<floatx4*>(row + e) = acc[i][j];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (e + r < N) row[e + r] = acc[i][j][r];
      }
    }
  }
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
// summed in ascending k.
__global__ __launch_bounds__(256) void gate_gemm_f32_kernel(const float* __restrict__ x,
                                                            const float* __restrict__ W,
                                                            float* __restrict__ h, int T, int d,
                                                            int N) {
  const int layer = blockIdx.y;
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)T * N) return;
  const int t = (int)(i / N);
  const int e = (int)(i % N);
  const float* xt = x + ((size_t)layer * T + t) * d;
  const float* we = W + ((size_t)layer * N + e) * d;
  float acc = 0.f;
  for (int k = 0; k < d; ++k) acc = __builtin_fmaf(xt[k], we[k], acc);
  h[((size_t)layer * T + t) * N + e] = acc;
}

template <int BT, int BE, int WT, int WE, int NP, int NSTAGE>
hipError_t launch_dma(const void* x, const void* w, float* part, int L, int T, int d, int N,
                      int ksplit, hipStream_t s) {
  const int n_tt = (T + BT - 1) / BT;
  const int n_te = (N + BE - 1) / BE;
  const int n_work = L * ksplit * n_te * n_tt;
  const int per_xcd = (n_work + 7) / 8;
  hipLaunchKernelGGL((gate_gemm_dma_kernel<BT, BE, WT, WE, NP, NSTAGE>), dim3(8 * per_xcd),
                     dim3((WT * WE + NP) * kWave), 0, s, static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(w), part, L, T, d, N, ksplit, n_tt, n_te,
                     n_work, per_xcd);
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

// Tile of the pipelined kernel for a router with N experts.
bool small_n(int N) { return N <= 32; }

}  // namespace

int gate_gemm_ksplit(int dtype_bf16, int L, int T, int d, int N) {
  if (!dtype_bf16 || T == 0 || d % kKStage != 0) return 1;
  const int bt = small_n(N) ? 64 : 128;
  const int be = small_n(N) ? 32 : 256;
  const long long tiles = (long long)L * ((T + bt - 1) / bt) * ((N + be - 1) / be);
  int ks = 1;
  while (ks < 8 && tiles * ks < 256 && d % (kKStage * ks * 2) == 0) ks *= 2;
  return ks;
}

hipError_t launch_gate_gemm_bf16(const void* x, const void* w, float* part, int L, int T, int d,
                                 int N, int ksplit, hipStream_t s) {
  if (d % (kKStage * ksplit) == 0) {
    if (small_n(N)) return launch_dma<64, 32, 4, 1, 4, 3>(x, w, part, L, T, d, N, ksplit, s);
    return launch_dma<128, 256, 2, 2, 4, 3>(x, w, part, L, T, d, N, ksplit, s);
  }
  if (ksplit != 1) return hipErrorInvalidValue;
  if (N <= 16) return launch_tile<16, 64, 1, 4>(x, w, part, L, T, d, N, s);
  return launch_tile<64, 128, 1, 4>(x, w, part, L, T, d, N, s);
}

hipError_t launch_gate_gemm_f32(const float* x, const float* w, float* h, int L, int T, int d,
                                int N, hipStream_t s) {
  const long long n = (long long)T * N;
  dim3 grid((unsigned)((n + 255) / 256), L);
  hipLaunchKernelGGL(gate_gemm_f32_kernel, grid, dim3(256), 0, s, x, w, h, T, d, N);
  return hipGetLastError();
}

}  // namespace moer
