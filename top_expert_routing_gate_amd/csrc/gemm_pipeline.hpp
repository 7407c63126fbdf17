// Pipelined bf16 gate GEMM tile (d a multiple of 64 per depth range): the
// producer/consumer main loop of the gate GEMM.
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
// l owns experts 4*(l/16)..+3 of token l%16 (16-byte stores).
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
// the last valid row (their results are never used); d must be a multiple of
// the stage depth so no chunk is partial.
//
// One workgroup barrier per stage orders the ring: before barrier k the
// producers wait until their stage-k loads have landed, and the consumers
// have finished reading stage k-1; after it the consumers read stage k and
// the producers refill the buffer of stage k-1 with stage k+NSTAGE-1.
#pragma once

#include "moer_internal.hpp"

namespace moer {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define MOER_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kKStage = 64;           // reduction depth per LDS stage (bf16)
constexpr int kNonTemporal = 2;       // cache-policy operand of a load: the nt bit
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

// Work item of a launch: workgroup b runs on XCD b % 8 (round-robin
// dispatch); consecutive items of one (layer, depth range) go to one XCD so
// that XCD streams one part of W_g through its own L2.
struct GemmWork {
  int tt, te, ks, layer;
};
__device__ __forceinline__ bool decode_work(int n_tt, int n_te, int ksplit, int n_work,
                                            int per_xcd, GemmWork& w) {
  const int b = blockIdx.x;
  const int work = (b % 8) * per_xcd + b / 8;
  if (work >= n_work) return false;
  int rest = work;
  w.tt = rest % n_tt; rest /= n_tt;
  w.te = rest % n_te; rest /= n_te;
  w.ks = rest % ksplit; rest /= ksplit;
  w.layer = rest;
  return true;
}

template <int BT, int BE, int WT, int WE, int NP, int NSTAGE>
struct GemmPipeline {
  static constexpr int kConsumers = WT * WE;
  static constexpr int kThreads = (WT * WE + NP) * kWave;
  static constexpr int kRows = BT + BE;
  static constexpr int kStageSlots = kRows * kChunks;
  static constexpr int kLoads = kStageSlots / (NP * kWave);  // per producer per stage
  // instruction i of a producer covers rows ((i*NP + pw)*64 + lane)/8: the
  // first kXLoads of them are x rows, the rest W_g rows
  static constexpr int kXLoads = BT * kChunks / (NP * kWave);
  static constexpr int MT = BT / WT / 16;
  static constexpr int ME = BE / WE / 16;
  static constexpr size_t kRingBytes = (size_t)NSTAGE * kStageSlots * sizeof(u32x4);
  static_assert(kStageSlots % (NP * kWave) == 0, "stage must split evenly over the producers");
  static_assert((BT * kChunks) % (NP * kWave) == 0, "x rows must fill whole instructions");
  static_assert((NSTAGE - 2) * kLoads <= 63, "outstanding loads must fit the vmcnt field");
  static_assert(BT % (WT * 16) == 0 && BE % (WE * 16) == 0, "tile shape");

  // Producer wave pw: stream depth [kbeg, kbeg + nk*64) of x rows t0.. and
  // W rows e0.. (x, W already offset to the layer) into the ring.
  __device__ static void produce(u32x4 (*ring)[kStageSlots], const uint16_t* x,
                                 const uint16_t* W, int t0, int e0, int T, int N, int d,
                                 int kbeg, int nk, int pw) {
    const int lane = threadIdx.x & 63;
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
    // x rows are read once: their loads carry the non-temporal hint, which
    // streams them through the L2 with less disturbance of the W_g rows
    // every workgroup of the die re-reads
    auto issue = [&](int stage_k, int buf) {
#pragma unroll
      for (int i = 0; i < kXLoads; ++i)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(src[i] + stage_k * kKStage),
                                         MOER_LDS_PTR(&ring[buf][(i * NP + pw) * kWave]), 16, 0,
                                         kNonTemporal);
#pragma unroll
      for (int i = kXLoads; i < kLoads; ++i)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(src[i] + stage_k * kKStage),
                                         MOER_LDS_PTR(&ring[buf][(i * NP + pw) * kWave]), 16, 0,
                                         0);
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
  }

  // Consumer wave (wt, we): accumulate its (BT/WT) x (BE/WE) block.
  __device__ static void consume(u32x4 (*ring)[kStageSlots], int nk, int wt, int we,
                                 floatx4 (&acc)[ME][MT]) {
    const int lane = threadIdx.x & 63;
    const int frow = lane & 15;
    const int fq = lane >> 4;
#pragma unroll
    for (int i = 0; i < ME; ++i)
#pragma unroll
      for (int j = 0; j < MT; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
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
  }

  // Token row (within the tile) and first expert of the lane's accumulator
  // block (i, j): experts e .. e+3 of token t.
  __device__ static int acc_token(int wt, int j) { return (wt * MT + j) * 16 + (threadIdx.x & 15); }
  __device__ static int acc_expert(int we, int i) {
    return (we * ME + i) * 16 + 4 * ((threadIdx.x & 63) >> 4);
  }

  // Transpose the consumers' blocks through LDS (the ring, free once every
  // wave has passed the barrier before this call): every wave of the
  // workgroup then stores whole token rows, 1 KB per instruction (eight full
  // 128-byte lines), instead of 64-byte pieces of sixteen rows. Chunk c
  // (four experts) of token row r sits at chunk c ^ (r % 16) of the row (the
  // row's chunk count, when below 16), so both the accumulator writes
  // (sixteen rows, one chunk column) and the row reads hit different 16-byte
  // bank groups. Every wave calls this.
  static constexpr int kTileChunks = BE / 4;  // 16-byte chunks per token row
  static constexpr int kSwz = (kTileChunks < 16 ? kTileChunks : 16) - 1;
  static_assert((size_t)BT * BE * 4 <= kRingBytes, "the tile fits in the ring");
  static_assert((kTileChunks & (kTileChunks - 1)) == 0, "power-of-two chunks per row");
  __device__ static void store_tile_lds(u32x4 (*ring)[kStageSlots], const floatx4 (&acc)[ME][MT],
                                        float* out, int t0, int e0, int T, int N) {
    u32x4* tile = &ring[0][0];
    const int wave = threadIdx.x >> 6;
    if (wave < kConsumers) {
      const int wt = wave / WE, we = wave % WE;
#pragma unroll
      for (int i = 0; i < ME; ++i) {
        const int c = acc_expert(we, i) / 4;
#pragma unroll
        for (int j = 0; j < MT; ++j) {
          const int r = acc_token(wt, j);
          tile[r * kTileChunks + (c ^ (r & kSwz))] = __builtin_bit_cast(u32x4, acc[i][j]);
        }
      }
    }
    __syncthreads();
    constexpr int kWaves = kThreads / kWave;
    constexpr int kRowsPerPass = kWaves * kWave / kTileChunks;  // token rows stored at once
    const int lane_row = threadIdx.x / kTileChunks;
    const int c = threadIdx.x % kTileChunks;
    const int e = e0 + 4 * c;
    for (int r = lane_row; r < BT; r += kRowsPerPass) {
      const int t = t0 + r;
      if (t >= T) break;
      const floatx4 v = __builtin_bit_cast(floatx4, tile[r * kTileChunks + (c ^ (r & kSwz))]);
      float* row = out + (size_t)t * N;
      if (e + 3 < N && (N & 3) == 0) {
        *reinterpret_cast<floatx4*>(row + e) = v;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (e + q < N) row[e + q] = v[q];
      }
    }
  }

  // Store the consumer's block to out[t][e] (row stride N), rows < T only.
  __device__ static void store(const floatx4 (&acc)[ME][MT], float* out, int t0, int e0, int T,
                               int N, int wt, int we) {
#pragma unroll
    for (int i = 0; i < ME; ++i) {
      const int e = e0 + acc_expert(we, i);
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const int t = t0 + acc_token(wt, j);
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
};

}  // namespace moer
