// Shared device code for the gfx950 kernels: vector types, tile geometry, the MFMA step and
// the persistent tile order.
//
// Tile geometry (constants of the build, never derived from N):
//   - a work-group of 512 threads = 8 wave64s (two per SIMD) computes a 256 x 256 fp32 tile
//     C[a, b] = sum_k A[a, k] B[b, k], where A and B are 256-row panels contiguous along K;
//   - wave w owns A rows 128*(w&1) .. +128 and B rows 64*(w>>1) .. +64, a 4 x 2 grid of
//     32x32 MFMA blocks: 128 fp32 accumulators per lane, so two waves fit one SIMD and the
//     matrix pipe keeps running while one of them stalls on a load or LDS read.
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
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;                 // wave64s per work-group
constexpr int kThreads = 64 * kWaves;     // 512
constexpr int kTile = 256;                // rows of A and of B per tile
constexpr int kWaveA = 128;               // A rows per wave
constexpr int kWaveB = 64;                // B rows per wave
constexpr int kBlkA = kWaveA / 32;        // 32-row MFMA blocks per wave along A (4)
constexpr int kBlkB = kWaveB / 32;        // along B (2)

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int wave_a0(int wave) { return (wave & 1) * kWaveA; }
__device__ __forceinline__ int wave_b0(int wave) { return (wave >> 1) * kWaveB; }

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
  f32x16 c[kBlkA][kBlkB];  // [A block i][B block j]
};

__device__ __forceinline__ void zero_acc(Acc& acc) {
#pragma unroll
  for (int i = 0; i < kBlkA; ++i)
#pragma unroll
    for (int j = 0; j < kBlkB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.c[i][j][r] = 0.f;
}

// Output coordinates of accumulator register r of block (i, j) for this lane, relative to
// the wave's sub-tile: row within its A rows, column within its B rows.
__device__ __forceinline__ int acc_row(int i, int r, int lane) {
  return 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int j, int lane) { return 32 * j + (lane & 31); }

// Persistent-grid tile order.  Work-groups are dispatched round-robin over the 8 XCDs, so
// group b runs on XCD b % 8.  The virtual tile index gives each XCD 32 consecutive virtual
// tiles per round; virtual tiles walk bands of `band` B-tiles, A-tile-major inside a band,
// so the work-groups of one XCD share a few A panels and a few B panels in its L2.
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
