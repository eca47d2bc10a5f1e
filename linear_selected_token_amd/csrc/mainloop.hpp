// The ring K loop and the persistent tile driver shared by the tile kernels.
//
// The loop computes C[a_row, b_row] += sum_k A[a_row, k] B[b_row, k] for one 256 x 256 tile,
// with both operands contiguous along K (bf16 or fp32) and fp32 accumulation on MFMA.
//
// Data movement (gfx950):
//   - K advances 128 bytes per stage (64 bf16 / 32 fp32 values per row).  The direct-to-LDS
//     loads (buffer_load_dwordx4 ... lds, 16 B per lane, no registers) then move whole 128-byte
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

// K-strided ("T") panels, for an operand stored with K as its row index (K-rows of M
// values): a stage holds 64 K-rows of the tile's 256 M values, 512 B per K-row.  Chunk c
// (16 B = 8 M values) of K-row kk sits at physical chunk c ^ tswz(kk), so the transposing
// fragment reads (4 K-rows x 16 M values per 16-lane group) hit distinct banks.  A wave's
// load q fills K-rows 2 (wave kDmaPerWave + q) + (lane >> 5), the lane at physical chunk
// lane & 31.
__device__ __forceinline__ int tswz(int kk) { return 4 * (kk & 3); }
__device__ __forceinline__ int tdma_row(int q, int wave, int lane) {
  return 2 * (wave * kDmaPerWave + q) + (lane >> 5);
}
__device__ __forceinline__ int tdma_chunk(int q, int wave, int lane) {
  return (lane & 31) ^ tswz(tdma_row(q, wave, lane));
}
// Byte offset in a T panel of this lane's first transposing read for the 32-row M block at
// m0, K slice 0: K-row 8 (lane >> 5) + ((lane & 15) >> 2), M values m0 + 16 ((lane >> 4) & 1)
// + 4 (lane & 3) .. + 3.  K slice s adds 16 s K-rows, the second read of a fragment 4 more;
// neither changes kk & 3, so both are plain offsets.
__device__ __forceinline__ int tfrag_off(int m0, int lane) {
  const int kk = 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int m = m0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  return kk * 512 + (((m >> 3) ^ tswz(kk)) << 4) + (m & 7) * 2;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// One MFMA fragment from a T panel: two transposing reads give this lane 4 + 4 consecutive K
// values of its M row (within a 16-lane group, lane i receives element e of the 4-element
// words loaded by lanes 4e .. 4e + 3, i.e. K-row e at M value i).
__device__ __forceinline__ u32x4 tfrag_read(const uint8_t* p) {
  const lds_i16x4* q = (const lds_i16x4*)((__attribute__((address_space(3))) uint8_t*)(p));
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_i16x4*>(q));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_i16x4*>(q + 4 * 512 / 8));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
  const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
  u32x4 r;
  r.x = l2.x;
  r.y = l2.y;
  r.z = h2.x;
  r.w = h2.y;
  return r;
}

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

// A scheduling fence: nothing moves across it, so code between two fences issues in
// program order relative to the code around it.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// Load sources of one tile.  Each operand is a uniform base address (kept in scalar
// registers), advanced by a_kstep / b_kstep bytes per K stage, plus this lane's byte offset,
// per panel slot q, of the 16-byte chunk it loads at stage 0 (K-contiguous panels: row
// dma_row(q), kstep 128; T panels: K-row tdma_row(q), kstep 64 K-rows).  The loads are
// buffer loads (raw, unswizzled) whose range check returns zeros for any offset at or past
// the operand's remaining bytes, so a load can never touch memory outside its operand, and
// rows past the end of an operand read as zeros.
struct TileSrc {
  int nk;  // K stages of the tile
  const uint8_t* a;
  const uint8_t* b;
  uint64_t a_bytes, b_bytes;  // readable bytes from each base
  uint32_t a_kstep, b_kstep;  // bytes per K stage
  uint32_t ao[kDmaPerWave];
  uint32_t bo[kDmaPerWave];
};

// The same value in every lane, held in scalar registers.
__device__ __forceinline__ const uint8_t* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

// Readable bytes of an operand from a base.
__device__ __forceinline__ uint64_t operand_bytes(size_t n) { return (uint64_t)n; }

// Buffer descriptor word 3 for raw (untyped, unswizzled) loads on gfx9-family parts.
constexpr int kRawBufferWord3 = 0x00020000;

// Loads of panel slots q in [q0, q0 + n) of stage k, as buffer_load_dwordx4 ... lds (16 B per
// lane; lane i lands at byte 16 i of the slot's 1 KiB, the slot's LDS address in M0).
//
// kAsm == false (no K-strided panel in the loop): the compiler intrinsic, with the tile's base
// fixed and the stage's offset k * kstep as the scalar offset.
//
// kAsm == true (a K-strided panel is read with transposing LDS reads): inline assembly.  Issued
// through the intrinsic, a load into LDS makes the compiler drain every outstanding load
// (s_waitcnt vmcnt(0)) before each transposing read of the same shared object, although the
// ring slot being read is never one being filled.  The explicit waits of stage_barrier order
// the loads against the reads instead; the memory clobber keeps LDS reads from moving across
// a load, and waits the compiler computes for its own loads can only over-wait, because vmcnt
// retires in order.  The base advances k * kstep bytes per stage (64-bit, so K-strided
// operands of any size stay addressable), and the descriptor's byte count shrinks with it so
// that rows past the operand's end still read as zeros.  A stage's first row always lies
// inside the operand, so the remaining byte count is positive.
typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
template <bool kAsm>
__device__ __forceinline__ void dma_panel(uint8_t* panel, const uint8_t* base, uint64_t bytes,
                                          uint32_t kstep, const uint32_t (&off)[kDmaPerWave],
                                          int k, int q0, int n) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if constexpr (!kAsm) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(base), (short)0, (int)(bytes < 0x7fffffffu ? bytes : 0x7fffffffu),
        kRawBufferWord3);
    const int koff = k * (int)kstep;
#pragma unroll
    for (int q = q0; q < q0 + n; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, to_lds(panel + (wave * kDmaPerWave + q) * 1024), 16, (int)off[q], koff, 0, 0);
  } else {
    const uint64_t koff = (uint64_t)(uint32_t)k * kstep;
    const uint64_t left = bytes - koff;
    const uint64_t addr = reinterpret_cast<uint64_t>(base) + koff;
    u32x4s rs;  // raw buffer descriptor: base, stride 0, byte count, word 3
    rs.x = (uint32_t)addr;
    rs.y = (uint32_t)(addr >> 32) & 0xffffu;
    rs.z = (uint32_t)(left >> 31) != 0 ? 0x7fffffffu : (uint32_t)left;
    rs.w = (uint32_t)kRawBufferWord3;
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(to_lds(panel));
#pragma unroll
    for (int q = q0; q < q0 + n; ++q) {
      const uint32_t m0 = lds0 + (uint32_t)((wave * kDmaPerWave + q) * 1024);
      // M0 (the slot's LDS address) is an input bound to that register, so the compiler
      // writes it and knows it is read; the s_nop is the wait state the hardware needs between
      // a write of M0 and a load into LDS that uses it.
      asm volatile(
          "s_nop 0\n\t"
          "buffer_load_dwordx4 %0, %1, 0 offen lds"
          :
          : "v"(off[q]), "s"(rs), "{m0}"(m0)
          : "memory");
    }
  }
}
template <bool kAsm = false>
__device__ __forceinline__ void dma_a(RingSmem& sm, const TileSrc& t, int k, int q0 = 0,
                                      int n = kDmaPerWave) {
  dma_panel<kAsm>(sm.a[k % kRingA], t.a, t.a_bytes, t.a_kstep, t.ao, k, q0, n);
}
template <bool kAsm = false>
__device__ __forceinline__ void dma_b(RingSmem& sm, const TileSrc& t, int k, int q0 = 0,
                                      int n = kDmaPerWave) {
  dma_panel<kAsm>(sm.b[k % kRingB], t.b, t.b_bytes, t.b_kstep, t.bo, k, q0, n);
}

// The loads a tile's K loop expects in flight when it starts, in this order: A stage 0,
// B stage 0, the first half of B stage 1, A stage 1.  May be issued early (for example
// under the previous tile's epilogue) once every wave has passed the previous loop's final
// barrier.
template <bool kAsm = false>
__device__ __forceinline__ void ring_prologue(RingSmem& sm, const TileSrc& t, int nk) {
  if (nk <= 0) return;
  dma_a<kAsm>(sm, t, 0);
  dma_b<kAsm>(sm, t, 0);
  if (nk > 1) {
    dma_b<kAsm>(sm, t, 1, 0, kDmaPerWave / 2);
    dma_a<kAsm>(sm, t, 1);
  }
}

// nk stages of the tile whose ring_prologue was issued.  On return all waves have passed a
// barrier after their last LDS read, so the next tile's prologue may be issued.
//
// A stage is four 32-byte K slices.  Each slice issues its kBlkA x kBlkB MFMAs in a fixed
// order with, between them, the LDS fragment reads of the next slice (in the order that
// slice consumes them, so its first MFMA waits only for the first two reads) and up to
// kHalf direct-to-LDS loads (one after every other MFMA, so no wave issues a burst of
// loads while its matrix pipe drains).  Every instruction group is fenced: the order below
// is the issue order.
template <bool kBF16, bool kTA, bool kTB>
__device__ __forceinline__ void ring_mainloop(RingSmem& sm, const TileSrc& t, int nk, Acc& acc) {
  static_assert(kBF16 || (!kTA && !kTB), "T panels hold bf16 operands");
  constexpr bool kAsm = kTA || kTB;
  if (nk <= 0) return;
  constexpr int kHalf = kDmaPerWave / 2;
  constexpr int kReads = kBlkA + kBlkB;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wa = wave_a0(wave);
  const int wb = wave_b0(wave);
  const int fr = lane & 31;
  const int g = ring_swz(fr);  // the same for every 32-row block
  int off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) off[s] = fr * kKBytes + 16 * ((2 * s + (lane >> 5)) ^ g);
  int toa[kBlkA], tob[kBlkB];  // T panels: per-block offsets of the transposing reads
#pragma unroll
  for (int i = 0; i < kBlkA; ++i) toa[i] = kTA ? tfrag_off(wa + 32 * i, lane) : 0;
#pragma unroll
  for (int j = 0; j < kBlkB; ++j) tob[j] = kTB ? tfrag_off(wb + 32 * j, lane) : 0;

  auto frag_a = [&](int k, int s, int i) __attribute__((always_inline)) -> u32x4 {
    if constexpr (kTA)
      return tfrag_read(sm.a[k % kRingA] + toa[i] + s * 16 * 512);
    else
      return *reinterpret_cast<const u32x4*>(sm.a[k % kRingA] + wa * kKBytes + off[s] +
                                             i * 32 * kKBytes);
  };
  auto frag_b = [&](int k, int s, int j) __attribute__((always_inline)) -> u32x4 {
    if constexpr (kTB)
      return tfrag_read(sm.b[k % kRingB] + tob[j] + s * 16 * 512);
    else
      return *reinterpret_cast<const u32x4*>(sm.b[k % kRingB] + wb * kKBytes + off[s] +
                                             j * 32 * kKBytes);
  };
  // Fragment read e of slice s of stage k: a[0], b[0 .. kBlkB), a[1 .. kBlkA).
  auto read1 = [&](int k, int s, int e, u32x4 (&fa)[kBlkA], u32x4 (&fb)[kBlkB]) {
    if (e == 0)
      fa[0] = frag_a(k, s, 0);
    else if (e <= kBlkB)
      fb[e - 1] = frag_b(k, s, e - 1);
    else
      fa[e - kBlkB] = frag_a(k, s, e - kBlkB);
  };
  // One slice: MFMAs on (ca, cb); if rd, the reads of slice (k2, s2) into (na, nb); the n
  // loads dma(0 .. n).
  auto slice = [&](const u32x4 (&ca)[kBlkA], const u32x4 (&cb)[kBlkB], bool rd, int k2, int s2,
                   u32x4 (&na)[kBlkA], u32x4 (&nb)[kBlkB], int n, auto&& dma) {
    int r = 0;
#pragma unroll
    for (int m = 0; m < kBlkA * kBlkB; ++m) {
      mma_step<kBF16>(acc.c[m / kBlkB][m % kBlkB], ca[m / kBlkB], cb[m % kBlkB]);
      fence();
      if ((m & 1) == 0 && (m >> 1) < n) {
        dma(m >> 1);
        fence();
      }
      if (rd && r < kReads) {
        read1(k2, s2, r, na, nb);
        ++r;
        fence();
      }
    }
#pragma unroll
    for (; rd && r < kReads; ++r) read1(k2, s2, r, na, nb);
    fence();
  };
  auto no_dma = [&](int) {};

  u32x4 a0[kBlkA], b0[kBlkB], a1[kBlkA], b1[kBlkB];
  // A ring slot is free once every wave has passed the barrier after its last fragment
  // read, so each load goes out right after the barrier that frees its slot:
  //   slice 3 of stage k - 1 (after barrier k - 1) and slice 0 of stage k: B stage k + 1,
  //     which stage k + 1 reads after barrier k (about one stage in flight);
  //   slices 1 and 2 of stage k: A stage k + 2 (about one and a half stages in flight).
  // Barrier k waits until only A stage k + 2 may still be in flight.
  auto stage = [&](int k, bool more_b, bool more_a) {  // slices 0-2 of stage k
    auto db = [&](int q) { dma_b<kAsm>(sm, t, k + 1, kHalf + q, 1); };
    auto da0 = [&](int q) { dma_a<kAsm>(sm, t, k + 2, q, 1); };
    auto da1 = [&](int q) { dma_a<kAsm>(sm, t, k + 2, kHalf + q, 1); };
    slice(a0, b0, true, k, 1, a1, b1, more_b ? kHalf : 0, db);
    slice(a1, b1, true, k, 2, a0, b0, more_a ? kHalf : 0, da0);
    slice(a0, b0, true, k, 3, a1, b1, more_a ? kHalf : 0, da1);
  };

  // stage 0 visible: A0 and B0 landed (half of B1 and A1 may still be in flight)
  if (nk > 1) stage_barrier<kHalf + kDmaPerWave>();
  else stage_barrier<0>();
#pragma unroll
  for (int e = 0; e < kReads; ++e) read1(0, 0, e, a0, b0);
  fence();
  int k = 0;
  for (; k + 2 < nk; ++k) {
    stage(k, true, true);
    stage_barrier<kDmaPerWave>();  // A k+1, B k+1 landed; A k+2 may be in flight
    const int kk = k;
    auto db = [&](int q) { dma_b<kAsm>(sm, t, kk + 2, q, 1); };
    slice(a1, b1, true, k + 1, 0, a0, b0, kHalf, db);
  }
  if (k + 1 < nk) {  // stage nk - 2: only the second half of B nk - 1 left to load
    stage(k, true, false);
    stage_barrier<0>();
    slice(a1, b1, true, k + 1, 0, a0, b0, 0, no_dma);
    ++k;
  }
  stage(k, false, false);  // last stage
  stage_barrier<0>();
  slice(a1, b1, false, 0, 0, a0, b0, 0, no_dma);
}

// virtual_tile, except that a last, partial round (fewer than grid tiles left) is dealt out
// across the XCDs: tile round * grid + b, and work-group b runs on XCD b % 8.  Each XCD then
// gets its share of that round, which matters when the work-groups go on to other work.
__device__ __forceinline__ int virtual_tile_spread(int round, int b, int grid, int n_tiles) {
  if ((round + 1) * grid > n_tiles) return round * grid + b;
  return virtual_tile(round, b, grid);
}

// Persistent tile driver.  Tiles u = virtual_tile(round, blockIdx.x, gridDim.x) for
// round = 0, 1, ... while u < n_tiles.  setup(u, src, ctx) prepares a tile's load sources
// (including its number of K stages) and its epilogue context; epilogue(ctx, acc) consumes
// the accumulators (registers and global memory only, no LDS).  The next tile's first
// loads are issued before the current tile's epilogue, so their latency hides behind it.
//
// kSpreadTail: the last, partial round is dealt out across the XCDs (virtual_tile_spread).
template <bool kBF16, class Ctx, bool kTA = false, bool kTB = false, bool kSpreadTail = false,
          class Setup, class Epilogue>
__device__ __forceinline__ void persistent_tiles(RingSmem& sm, int n_tiles, Setup setup,
                                                 Epilogue epilogue) {
  auto tile_of = [&](int round) __attribute__((always_inline)) {
    return kSpreadTail ? virtual_tile_spread(round, blockIdx.x, gridDim.x, n_tiles)
                       : virtual_tile(round, blockIdx.x, gridDim.x);
  };
  int round = 0;
  int u = tile_of(round);
  if (u >= n_tiles) return;
  TileSrc src;
  Ctx ctx;
  setup(u, src, ctx);
  ring_prologue<kTA || kTB>(sm, src, src.nk);
  while (true) {
    Acc acc;
    zero_acc(acc);
    ring_mainloop<kBF16, kTA, kTB>(sm, src, src.nk, acc);
    const int un = tile_of(++round);
    const bool more = un < n_tiles;
    Ctx cur = ctx;
    if (more) {
      setup(un, src, ctx);
      ring_prologue<kTA || kTB>(sm, src, src.nk);
    }
    epilogue(cur, acc);
    if (!more) break;
  }
}

// Tiles claimed at run time instead of by a fixed rule.  The work-group's XCD x = blockIdx.x & 7
// hands out claim numbers i = 0, 1, ... from counter[x] (one atomic add per tile, by one
// lane); claim i is virtual tile (i / per) * grid + x * per + i % per with per = grid / 8, and
// past the full rounds tile full * grid + 8 (i - full * per) + x: the tiles
// virtual_tile_spread gives XCD x, in the same order.  So the tiles in flight on an XCD are
// still the ones that share its L2, while work-groups that finished earlier work sooner take
// more of them.  Every claim number is handed out once and an XCD's tiles increase with it, so
// each tile below n_tiles is computed exactly once and a work-group stops at its first claim
// past n_tiles.  The claim is broadcast through the first word of the A ring while the ring is
// idle (every wave has passed the barrier after its last fragment read and no load into LDS is
// in flight); the counters must be zero when the launch starts.
__device__ __forceinline__ int claim_tile(RingSmem& sm, int* counter, int n_tiles) {
  int* slot = reinterpret_cast<int*>(sm.a[0]);
  if (threadIdx.x == 0) {
    const int grid = gridDim.x;
    int u;
    if ((grid & 7) == 0) {
      const int x = blockIdx.x & 7;
      const int per = grid >> 3;
      const int full = n_tiles / grid;  // full rounds
      const int i = atomicAdd(counter + x, 1);
      u = i < full * per ? (i / per) * grid + x * per + i % per
                         : full * grid + 8 * (i - full * per) + x;
    } else {
      u = atomicAdd(counter, 1);
    }
    *slot = u;
  }
  __syncthreads();
  const int u = __builtin_amdgcn_readfirstlane(*slot);
  __syncthreads();  // every wave has read the slot before it is written or loaded into again
  return u;
}

// persistent_tiles with claimed tiles (see claim_tile); the same setup / epilogue contract.
template <bool kBF16, class Ctx, bool kTA = false, bool kTB = false, class Setup, class Epilogue>
__device__ __forceinline__ void claimed_tiles(RingSmem& sm, int n_tiles, int* counter, Setup setup,
                                              Epilogue epilogue) {
  int u = claim_tile(sm, counter, n_tiles);
  if (u >= n_tiles) return;
  TileSrc src;
  Ctx ctx;
  setup(u, src, ctx);
  ring_prologue<kTA || kTB>(sm, src, src.nk);
  while (true) {
    Acc acc;
    zero_acc(acc);
    ring_mainloop<kBF16, kTA, kTB>(sm, src, src.nk, acc);
    const int un = claim_tile(sm, counter, n_tiles);
    const bool more = un < n_tiles;
    Ctx cur = ctx;
    if (more) {
      setup(un, src, ctx);
      ring_prologue<kTA || kTB>(sm, src, src.nk);
    }
    epilogue(cur, acc);
    if (!more) break;
  }
}

}  // namespace rlk
