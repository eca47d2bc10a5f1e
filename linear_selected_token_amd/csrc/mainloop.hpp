// The ring K loop and the persistent tile driver shared by the tile kernels.
//
// The loop computes C[a_row, b_row] += sum_k A[a_row, k] B[b_row, k] for one 256 x 256 tile,
// with both operands contiguous along K (bf16 or fp32) and fp32 accumulation on MFMA.
//
// Data movement (gfx950):
//   - K advances 128 bytes per stage (64 bf16 / 32 fp32 values per row).  The direct-to-LDS
//     loads (global_load_lds_dwordx4, 16 B per lane, no registers) then move whole 128-byte
//     lines, 8 rows per wave instruction; with 64-byte row pieces they move half as many
//     bytes per clock, because every line touched is only half used;
//   - the A panel (256 rows x 128 B = 32 KiB) has a ring of three stages and is loaded two
//     stages ahead; the B panel has a ring of two and is loaded one stage ahead.  Together
//     they fill the 160 KiB of LDS.  (A is the operand that misses in L2 when the tile
//     order streams it; B panels are shared by many tiles in flight.)
//   - a wave instruction fills 1 KiB of LDS = 8 rows; lane i lands at byte 16 i of it, so the
//     XOR swizzle of the 16-byte chunks is applied on the global side: lane i fetches the
//     logical chunk that belongs at its physical slot;
//   - MFMA fragments are double-buffered in registers: the reads of the next 32-byte K slice
//     are in flight while the current slice's MFMAs issue;
//   - issuing a load stalls the issuing wave for tens of cycles; with two waves per SIMD
//     the other wave keeps the matrix pipe busy meanwhile;
//   - one barrier per stage publishes the next stage and frees the oldest buffers.
#pragma once

#include "common.hpp"

namespace rlk {

constexpr int kKBytes = 128;                       // K bytes per row per stage
constexpr int kRingA = 3;                          // LDS stages of the A panel
constexpr int kRingB = 2;                          // LDS stages of the B panel
constexpr int kPanel = kTile * kKBytes;            // 32 KiB
constexpr int kDmaPerWave = kPanel / 1024 / kWaves;  // load instructions per panel per wave (4)

struct RingSmem {
  uint8_t a[kRingA][kPanel];
  uint8_t b[kRingB][kPanel];
};
static_assert(sizeof(RingSmem) == 160 * 1024, "the rings fill the LDS");

// Chunk swizzle of panel row r (8 chunks of 16 B per 128 B row): bits 1-3 of the row.  With
// it the fragment reads of the loop (32 consecutive rows per lane half, the halves one chunk
// apart) measure zero LDS bank conflicts on gfx950 (SQ_LDS_BANK_CONFLICT).
__device__ __forceinline__ int ring_swz(int r) { return (r >> 1) & 7; }

// Row of panel slot q (0 .. kDmaPerWave-1) that this lane fills, and the logical chunk it
// fetches.
__device__ __forceinline__ int dma_row(int q, int wave, int lane) {
  return (wave * kDmaPerWave + q) * 8 + (lane >> 3);
}
__device__ __forceinline__ int dma_chunk(int q, int wave, int lane) {
  return (lane & 7) ^ ring_swz(dma_row(q, wave, lane));
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
// past it).
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

// Load sources of one tile: this lane's 16-byte chunk of panel row dma_row(q) at K = 0.
struct TileSrc {
  const uint8_t* a[kDmaPerWave];
  const uint8_t* b[kDmaPerWave];
};

// Loads of panel slots q in [q0, q0 + n) of stage k.
__device__ __forceinline__ void dma_panel(uint8_t* panel, const uint8_t* const (&src)[kDmaPerWave],
                                          int k, int q0, int n) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const size_t koff = (size_t)k * kKBytes;
#pragma unroll
  for (int q = q0; q < q0 + n; ++q)
    __builtin_amdgcn_global_load_lds(src[q] + koff, to_lds(panel + (wave * kDmaPerWave + q) * 1024),
                                     16, 0, 0);
}
__device__ __forceinline__ void dma_a(RingSmem& sm, const TileSrc& t, int k, int q0 = 0,
                                      int n = kDmaPerWave) {
  dma_panel(sm.a[k % kRingA], t.a, k, q0, n);
}
__device__ __forceinline__ void dma_b(RingSmem& sm, const TileSrc& t, int k, int q0 = 0,
                                      int n = kDmaPerWave) {
  dma_panel(sm.b[k % kRingB], t.b, k, q0, n);
}

// The loads a tile's K loop expects in flight when it starts, in this order: A stage 0,
// B stage 0, A stage 1.  May be issued early (for example under the previous tile's
// epilogue) once every wave has passed the previous loop's final barrier.
__device__ __forceinline__ void ring_prologue(RingSmem& sm, const TileSrc& t, int nk) {
  if (nk <= 0) return;
  dma_a(sm, t, 0);
  dma_b(sm, t, 0);
  if (nk > 1) dma_a(sm, t, 1);
}

// nk stages of the tile whose ring_prologue was issued.  On return all waves have passed a
// barrier after their last LDS read, so the next tile's prologue may be issued.
template <bool kBF16>
__device__ __forceinline__ void ring_mainloop(RingSmem& sm, const TileSrc& t, int nk, Acc& acc) {
  if (nk <= 0) return;
  constexpr int kHalf = kDmaPerWave / 2;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wa = wave_a0(wave);
  const int wb = wave_b0(wave);
  const int fr = lane & 31;
  const int g = ring_swz(fr);  // the same for every 32-row block
  int off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) off[s] = fr * kKBytes + 16 * ((2 * s + (lane >> 5)) ^ g);

  auto frag = [&](int k, int s, u32x4 (&fa)[kBlkA], u32x4 (&fb)[kBlkB]) {
    const uint8_t* pa = sm.a[k % kRingA] + wa * kKBytes + off[s];
    const uint8_t* pb = sm.b[k % kRingB] + wb * kKBytes + off[s];
#pragma unroll
    for (int i = 0; i < kBlkA; ++i) fa[i] = *reinterpret_cast<const u32x4*>(pa + i * 32 * kKBytes);
#pragma unroll
    for (int j = 0; j < kBlkB; ++j) fb[j] = *reinterpret_cast<const u32x4*>(pb + j * 32 * kKBytes);
  };
  auto mma = [&](const u32x4 (&fa)[kBlkA], const u32x4 (&fb)[kBlkB]) {
#pragma unroll
    for (int i = 0; i < kBlkA; ++i)
#pragma unroll
      for (int j = 0; j < kBlkB; ++j) mma_step<kBF16>(acc.c[i][j], fa[i], fb[j]);
  };
  // Issue order inside one K slice (8 MFMA steps): the 6 LDS reads of the next slice go
  // between the first MFMAs, the slice's loads (0 or kHalf) between later ones.  Each slice
  // is its own scheduling region (sched_barrier at the end): otherwise the compiler pulls
  // MFMAs of the next slice up behind the LDS reads that feed them, which collapses the
  // register double-buffering into read-wait-MFMA chains.
  auto interleave = [&](int n_dma) {
#pragma unroll
    for (int m = 0; m < kBlkA * kBlkB; ++m) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, kBF16 ? 1 : 4, 0);
      if (m < kBlkA + kBlkB) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      if (m < n_dma) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Stage k with its first slice in (a0, b0).  Loads: B stage k + 1 in slices 0-1, A stage
  // k + 2 in slices 2-3 (slice 3 runs after the barrier; A's ring slot for k + 2 stays free
  // until stage k + 2).  The first slice of stage k + 1 is read after the barrier.
  u32x4 a0[kBlkA], b0[kBlkB], a1[kBlkA], b1[kBlkB];
  auto stage = [&](int k, bool dma_b_next, bool dma_a_next) {
    if (dma_b_next) dma_b(sm, t, k + 1, 0, kHalf);
    frag(k, 1, a1, b1);
    mma(a0, b0);
    interleave(dma_b_next ? kHalf : 0);
    if (dma_b_next) dma_b(sm, t, k + 1, kHalf, kHalf);
    frag(k, 2, a0, b0);
    mma(a1, b1);
    interleave(dma_b_next ? kHalf : 0);
    if (dma_a_next) dma_a(sm, t, k + 2, 0, kHalf);
    frag(k, 3, a1, b1);
    mma(a0, b0);
    interleave(dma_a_next ? kHalf : 0);
  };

  // stage 0 visible: A0 and B0 landed (A1 may still be in flight)
  if (nk > 1) stage_barrier<kDmaPerWave>();
  else stage_barrier<0>();
  frag(0, 0, a0, b0);
  int k = 0;
  for (; k + 2 < nk; ++k) {
    stage(k, true, true);
    stage_barrier<kHalf>();  // A k+1, B k+1 landed; half of A k+2 may be in flight
    dma_a(sm, t, k + 2, kHalf, kHalf);
    frag(k + 1, 0, a0, b0);
    mma(a1, b1);
    interleave(kHalf);
  }
  if (k + 1 < nk) {  // stage nk - 2: only B nk - 1 left to load
    stage(k, true, false);
    stage_barrier<0>();
    frag(k + 1, 0, a0, b0);
    mma(a1, b1);
    interleave(0);
    ++k;
  }
  stage(k, false, false);  // last stage
  stage_barrier<0>();
  mma(a1, b1);
}

// Persistent tile driver.  Tiles u = virtual_tile(round, blockIdx.x, gridDim.x) for
// round = 0, 1, ... while u < n_tiles.  setup(u, src, ctx) prepares a tile's load sources
// and its epilogue context; epilogue(ctx, acc) consumes the accumulators (registers and
// global memory only, no LDS).  The next tile's first loads are issued before the current
// tile's epilogue, so their latency hides behind it.
template <bool kBF16, class Ctx, class Setup, class Epilogue>
__device__ __forceinline__ void persistent_tiles(RingSmem& sm, int n_tiles, int nk, Setup setup,
                                                 Epilogue epilogue) {
  int round = 0;
  int u = virtual_tile(round, blockIdx.x, gridDim.x);
  if (u >= n_tiles) return;
  TileSrc src;
  Ctx ctx;
  setup(u, src, ctx);
  ring_prologue(sm, src, nk);
  while (true) {
    Acc acc;
    zero_acc(acc);
    ring_mainloop<kBF16>(sm, src, nk, acc);
    const int un = virtual_tile(++round, blockIdx.x, gridDim.x);
    const bool more = un < n_tiles;
    Ctx cur = ctx;
    if (more) {
      setup(un, src, ctx);
      ring_prologue(sm, src, nk);
    }
    epilogue(cur, acc);
    if (!more) break;
  }
}

}  // namespace rlk
