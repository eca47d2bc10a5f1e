// The K loop of every 256 x 256 tile kernel: C[a_row, b_row] += sum_k A[a_row, k] B[b_row, k]
// with both operands contiguous along K (bf16 or fp32), fp32 accumulation on MFMA.
//
// Data movement (gfx950):
//   - K advances 64 bytes per stage (32 bf16 / 16 fp32 values per row);
//   - each stage's A and B panels (256 rows x 64 B = 16 KiB each) are copied from global
//     memory straight into LDS by the direct-to-LDS loads (global_load_lds_dwordx4, 16 B per
//     lane, no registers), three stages ahead, into a ring of four LDS stages (128 KiB);
//   - a wave instruction fills 1 KiB of LDS = 16 rows; lane i lands at byte 16 i of it, so
//     the XOR swizzle of the 16-byte chunks is applied on the global side: lane i fetches
//     the logical chunk that belongs at its physical slot;
//   - MFMA fragments are double-buffered in registers: the reads of the next half-stage are
//     in flight while the current half-stage's 16 MFMAs issue;
//   - one barrier per stage, between the two MFMA halves, publishes the next stage.
#pragma once

#include "common.hpp"

namespace rlk {

constexpr int kKBytes = 64;                    // K bytes per row per stage
constexpr int kRing = 4;                       // LDS stages
constexpr int kPanel = kTile * kKBytes;        // 16 KiB
constexpr int kDmaPerWave = kPanel / 1024 / 4; // wave instructions per panel per wave = 4

struct RingSmem {
  uint8_t a[kRing][kPanel];
  uint8_t b[kRing][kPanel];
};

// 2-bit chunk swizzle of panel row r (4 chunks of 16 B per 64 B row).  Any 8 consecutive
// rows, and any 16 consecutive rows, read at one logical chunk hit distinct 16-byte bank
// groups.
__device__ __forceinline__ int ring_swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// Row of panel slot q (0..3) that this lane fills, and the logical chunk it fetches.
__device__ __forceinline__ int dma_row(int q, int wave, int lane) { return (wave * 4 + q) * 16 + (lane >> 2); }
__device__ __forceinline__ int dma_chunk(int q, int wave, int lane) {
  return (lane & 3) ^ ring_swz(dma_row(q, wave, lane));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ lds_ptr_t to_lds(void* p) {
  return (lds_ptr_t)((__attribute__((address_space(3))) uint8_t*)(p));
}

// s_waitcnt with vmcnt = n (0..63) and lgkmcnt = 0 (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Wait until at most n of this wave's global loads are outstanding and all its LDS reads
// have returned, then a workgroup barrier.  No instruction may be scheduled across it (MFMAs
// included: they touch no memory, so a memory clobber alone would let the compiler move them
// past it); every MFMA issued before it keeps the matrix pipe busy while the wave waits.
template <int n>
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  wait_vm_lgkm0<n>();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Instruction-class masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedDsRead = 0x100;

// a_src[q] / b_src[q]: this lane's source for panel slot q at K = 0 (row pointer plus
// 16 * dma_chunk); each stage adds 64 bytes.  nk stages.  On return all waves have passed a
// barrier after their last LDS read.
template <bool kBF16>
__device__ __forceinline__ void ring_mainloop(RingSmem& sm, const uint8_t* const (&a_src)[4],
                                              const uint8_t* const (&b_src)[4], int nk, Acc& acc) {
  if (nk <= 0) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wa = (wave & 1) * kWaveTile;
  const int wb = (wave >> 1) * kWaveTile;
  const int fr = lane & 31;
  const int g = ring_swz(fr);  // the same for every 32-row block
  const int off0 = fr * kKBytes + 16 * ((0 + (lane >> 5)) ^ g);
  const int off1 = fr * kKBytes + 16 * ((2 + (lane >> 5)) ^ g);

  auto dma = [&](int k) {
    const int buf = k & (kRing - 1);
    const size_t koff = (size_t)k * kKBytes;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds(a_src[q] + koff, to_lds(&sm.a[buf][(wave * 4 + q) * 1024]),
                                       16, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds(b_src[q] + koff, to_lds(&sm.b[buf][(wave * 4 + q) * 1024]),
                                       16, 0, 0);
  };
  auto frag = [&](int k, int off, u32x4 (&fa)[4], u32x4 (&fb)[4]) {
    const uint8_t* pa = sm.a[k & (kRing - 1)] + wa * kKBytes + off;
    const uint8_t* pb = sm.b[k & (kRing - 1)] + wb * kKBytes + off;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = *reinterpret_cast<const u32x4*>(pa + i * 32 * kKBytes);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = *reinterpret_cast<const u32x4*>(pb + j * 32 * kKBytes);
  };
  auto mma = [&](const u32x4 (&fa)[4], const u32x4 (&fb)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mma_step<kBF16>(acc.c[i][j], fa[i], fb[j]);
  };
  // Issue order inside a half-stage: one MFMA, one LDS read (and one DMA), repeated, so the
  // reads and loads for later stages hide behind the MFMAs.
  auto interleave = [&](bool with_dma) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      if (with_dma) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, kBF16 ? 8 : 32, 0);
  };

  u32x4 a0[4], b0[4], a1[4], b1[4];
  if (nk < 4) {
    // short K: every stage is in LDS before the first MFMA
    for (int k = 0; k < nk; ++k) dma(k);
    stage_barrier<0>();
    for (int k = 0; k < nk; ++k) {
      frag(k, off0, a0, b0);
      frag(k, off1, a1, b1);
      mma(a0, b0);
      mma(a1, b1);
    }
    stage_barrier<0>();
    return;
  }
  dma(0);
  dma(1);
  dma(2);
  stage_barrier<16>();
  frag(0, off0, a0, b0);
  int k = 0;
  for (; k + 3 < nk; ++k) {
    dma(k + 3);
    frag(k, off1, a1, b1);
    mma(a0, b0);
    interleave(true);
    stage_barrier<16>();  // stage k + 1 landed (k + 2 and k + 3 may still be in flight)
    frag(k + 1, off0, a0, b0);
    mma(a1, b1);
    interleave(false);
  }
  // last three stages: no more loads to issue
  frag(k, off1, a1, b1);
  mma(a0, b0);
  interleave(false);
  stage_barrier<8>();
  frag(k + 1, off0, a0, b0);
  mma(a1, b1);
  interleave(false);
  ++k;
  frag(k, off1, a1, b1);
  mma(a0, b0);
  interleave(false);
  stage_barrier<0>();
  frag(k + 1, off0, a0, b0);
  mma(a1, b1);
  interleave(false);
  ++k;
  frag(k, off1, a1, b1);
  mma(a0, b0);
  interleave(false);
  stage_barrier<0>();
  mma(a1, b1);
}

}  // namespace rlk
