// Shared device code for the gfx950 kernels: vector types, the MFMA step, the LDS layout
// of a tile stage and the double-buffered K loop that every GEMM-shaped kernel runs.
//
// Tile geometry (constants of the build, never derived from N):
//   - a work-group of 256 threads = 4 wave64s computes a 256 x 256 fp32 tile C = A B^T,
//     where A and B are 256-row panels whose rows are contiguous along K;
//   - wave w owns the 128 x 128 quadrant (rows 128*(w&1), columns 128*(w>>1)) as a 4 x 4
//     grid of 32x32 MFMA blocks, 256 fp32 accumulators per lane;
//   - K advances 128 bytes per stage (64 bf16 or 32 fp32 values per row); each stage
//     holds A and B panels of 256 rows x 128 bytes in LDS (32 KiB each), two stages are
//     double-buffered (128 KiB of the 160 KiB LDS).
//
// MFMA 32x32 output layout: lane l holds column (l & 31); its register r holds row
// 8*(r/4) + 4*(l/32) + (r%4).  A and B fragments are 16 bytes per lane: row (l & 31) of
// the block, K-chunk (l / 32) of the current 32-byte K slice.  A and B use the same
// K assignment, so each output is the dot product of its own row of A and row of B, in a
// K order that is the same for every output element.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;      // threads per work-group (4 wave64)
constexpr int kTile = 256;         // rows of A and of B per tile
constexpr int kWaveTile = 128;     // rows of A / of B per wave quadrant
constexpr int kStageBytes = 128;   // K bytes per row per stage
constexpr int kPanelBytes = kTile * kStageBytes;  // 32 KiB
constexpr int kLoadsPerThread = kPanelBytes / 16 / kThreads;  // 8 chunks of 16 B per panel

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Physical 16-byte chunk of logical chunk c in panel row r.  Eight consecutive rows read
// at the same logical chunk land on eight distinct chunk positions, so a 16-lane group of
// a ds_read_b128 touches every bank once.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }

__device__ __forceinline__ int panel_offset(int r, int c) { return r * kStageBytes + 16 * swz(r, c); }

// One K slice of 32 bytes: acc += A_frag * B_frag.
template <bool kBF16>
__device__ __forceinline__ void mma_step(f32x16& acc, const u32x4& a, const u32x4& b) {
  if constexpr (kBF16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  } else {
    // Cast the whole vector, then take named elements: a bit_cast of a single vector
    // element (a[e]) is lowered to element 0 by this compiler.
    const f32x4 af = __builtin_bit_cast(f32x4, a);
    const f32x4 bf = __builtin_bit_cast(f32x4, b);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af.x, bf.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af.y, bf.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af.z, bf.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af.w, bf.w, acc, 0, 0, 0);
  }
}

struct Acc {
  f32x16 c[4][4];  // [A block i][B block j]
};

__device__ __forceinline__ void zero_acc(Acc& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.c[i][j][r] = 0.f;
}

// Row (within the 256-row tile) of this thread's q-th 16-byte load, and its logical chunk.
__device__ __forceinline__ int load_row(int q, int tid) { return q * 32 + (tid >> 3); }
__device__ __forceinline__ int load_chunk(int tid) { return tid & 7; }

// LDS for one tile kernel: [stage][panel A|B][32 KiB].
struct TileSmem {
  uint8_t buf[2][2][kPanelBytes];
};

// Double-buffered K loop.  a_src[q] / b_src[q] point at this thread's 16-byte chunk of
// panel row load_row(q) at K = 0; each stage advances them by 128 bytes.  `nk` stages.
// On return every wave has passed a barrier after its last LDS read, so the caller may
// reuse the shared memory.
template <bool kBF16>
__device__ __forceinline__ void mainloop(TileSmem& sm, const uint8_t* const (&a_src)[kLoadsPerThread],
                                         const uint8_t* const (&b_src)[kLoadsPerThread], int nk,
                                         Acc& acc) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wa = (wave & 1) * kWaveTile;   // A rows of this wave
  const int wb = (wave >> 1) * kWaveTile;  // B rows of this wave
  const int chunk = load_chunk(tid);

  u32x4 ra[kLoadsPerThread], rb[kLoadsPerThread];
  int st_off[kLoadsPerThread];
#pragma unroll
  for (int q = 0; q < kLoadsPerThread; ++q) st_off[q] = panel_offset(load_row(q, tid), chunk);

  // fragment read offsets (row part), K chunk added per step
  const int frow = lane & 31;
  const int fhalf = lane >> 5;

  auto gload = [&](int k) {
    const size_t off = (size_t)k * kStageBytes;
#pragma unroll
    for (int q = 0; q < kLoadsPerThread; ++q) {
      ra[q] = *reinterpret_cast<const u32x4*>(a_src[q] + off);
      rb[q] = *reinterpret_cast<const u32x4*>(b_src[q] + off);
    }
  };
  auto sstore = [&](int s) {
#pragma unroll
    for (int q = 0; q < kLoadsPerThread; ++q) {
      *reinterpret_cast<u32x4*>(&sm.buf[s][0][st_off[q]]) = ra[q];
      *reinterpret_cast<u32x4*>(&sm.buf[s][1][st_off[q]]) = rb[q];
    }
  };
  auto compute = [&](int s) {
    const uint8_t* pa = sm.buf[s][0];
    const uint8_t* pb = sm.buf[s][1];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = 2 * ks + fhalf;
      u32x4 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const u32x4*>(pa + panel_offset(wa + 32 * i + frow, c));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fb[j] = *reinterpret_cast<const u32x4*>(pb + panel_offset(wb + 32 * j + frow, c));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mma_step<kBF16>(acc.c[i][j], fa[i], fb[j]);
    }
  };

  if (nk <= 0) return;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int k = 0; k < nk; ++k) {
    const int s = k & 1;
    if (k + 1 < nk) gload(k + 1);
    compute(s);
    if (k + 1 < nk) sstore(s ^ 1);
    __syncthreads();
  }
}

// Output coordinates of accumulator register r of block (i, j) for this lane, relative to
// the wave quadrant: row within the A quadrant, column within the B quadrant.
__device__ __forceinline__ int acc_row(int i, int r, int lane) {
  return 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int j, int lane) { return 32 * j + (lane & 31); }

// Persistent-grid tile order.  Work-groups are dispatched round-robin over the 8 XCDs, so
// group b runs on XCD b % 8.  The virtual tile index gives each XCD 32 consecutive virtual
// tiles per round; virtual tiles walk bands of `band` B-tiles (tokens), A-tile-major inside
// a band, so the work-groups of one XCD share a few A panels and a few B panels in its L2.
__device__ __forceinline__ int virtual_tile(int round, int b, int grid) {
  if ((grid & 7) == 0) return round * grid + (b & 7) * (grid >> 3) + (b >> 3);
  return round * grid + b;
}

__device__ __forceinline__ void tile_coords(int u, int nA, int nB, int band, int& ta, int& tb) {
  const int nfull = nB / band;
  const int full_tiles = nfull * band * nA;
  if (u < full_tiles) {
    const int bi = u / (band * nA);
    const int w = u - bi * band * nA;
    ta = w / band;
    tb = bi * band + (w - ta * band);
  } else {
    const int rem = nB - nfull * band;
    const int w = u - full_tiles;
    ta = w / rem;
    tb = nfull * band + (w - ta * rem);
  }
}

}  // namespace rlk
