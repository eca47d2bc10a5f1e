// Forward kernels of the fused linear log-prob.
//
// The forward streams the vocabulary in tiles and keeps only per-row softmax statistics,
// never the [N, V] logits (RL-Kernel Roadmap (2026), P0.2, "Fused CE LogProb without
// materializing logits": the forward path streams vocab blocks with online softmax).
//
//   fwd_tiles: persistent grid over (vocabulary tile x token tile) pairs.  Each 256 x 256
//              tile is z = W_tile h_tile^T on bf16 (or fp32) MFMA with fp32 accumulation over
//              the whole hidden dimension in one fixed K order.  Its epilogue folds 1/T and
//              log2(e) into one multiply, and for every token and every 128-entry vocabulary
//              column writes the column maximum and the sum of 2^(z*log2e - max).  The tile
//              that holds a token's target also writes that target logit.
//   fwd_merge: per token, combines the columns in one fixed order into lse and logp.
//
// Batch invariance (RL-Kernel Roadmap (2026), P0.2, "Batch-Invariant Deterministic
// LogProb": no atomics, fixed reduction topology and block partition, per-row reduction
// independent of the batch): the vocabulary tiling is a build constant; a token's column
// statistics depend only on its own h row, the W tile and the fixed K order; the lane and
// register order of every reduction is the same for every token position; the merge walks
// the columns in the same fixed association for every token.
#include "common.hpp"
#include "kernels.hpp"
#include "mainloop.hpp"

namespace rlk {

namespace {

struct FwdCtx {
  int vq;      // first vocabulary entry of this wave's quadrant
  int tok[kBlkB];  // compacted token index of each of this lane's token columns
  int tgt[kBlkB];  // their targets (-1: none or out of range)
};

template <bool kBF16>
__global__ __launch_bounds__(kThreads) void fwd_tiles_kernel(FwdTileArgs a) {
  __shared__ RingSmem sm;
  const int Na = *a.n_active;
  const int nTokTiles = (Na + kTile - 1) / kTile;
  const int nVocTiles = (a.V + kTile - 1) / kTile;
  const int band = nTokTiles < 8 ? nTokTiles : 8;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const size_t row_bytes = (size_t)a.H * (kBF16 ? 2 : 4);
  const int nk = (int)(row_bytes / kKBytes);
  const float c2 = a.inv_t * kLog2e;
  const int wv = wave_a0(wave);  // vocabulary offset of the wave sub-tile
  const int wt = wave_b0(wave);  // token offset of the wave sub-tile

  auto setup = [&](int u, TileSrc& src, FwdCtx& c) {
    int vt, tt;
    tile_coords(u, nVocTiles, nTokTiles, band, vt, tt);
    const int vbase = vt * kTile;
    const int tbase = tt * kTile;
    src.nk = nk;
    src.a_kstep = src.b_kstep = kKBytes;
    src.a = uniform_ptr(static_cast<const uint8_t*>(a.W) + (size_t)vbase * row_bytes);
    src.b = uniform_ptr(a.h);
    src.a_bytes = operand_bytes((size_t)(a.V - vbase) * row_bytes);
    src.b_bytes = operand_bytes((size_t)a.N * row_bytes);
#pragma unroll
    for (int q = 0; q < kDmaPerWave; ++q) {
      const int r = dma_row(q, wave, lane);
      const int ch = dma_chunk(q, wave, lane);
      const int v = min(vbase + r, a.V - 1);
      const int t = a.idx[min(tbase + r, Na - 1)];
      src.ao[q] = (uint32_t)((size_t)(v - vbase) * row_bytes) + 16 * ch;
      src.bo[q] = (uint32_t)((size_t)t * row_bytes) + 16 * ch;
    }
    c.vq = vbase + wv;
#pragma unroll
    for (int j = 0; j < kBlkB; ++j) {
      c.tok[j] = tbase + wt + acc_col(j, lane);
      // target as a row of this W (out of range or in another vocabulary shard: none)
      const int y = c.tok[j] < Na ? a.targets[a.idx[c.tok[j]]] - a.vstart : -1;
      c.tgt[j] = (y >= 0 && y < a.V) ? y : -1;
    }
  };

  // Per token column: statistics of this wave's 128 vocabulary entries.
  auto epilogue = [&](const FwdCtx& c, Acc& acc) {
    const int vq = c.vq;
    if (vq >= a.V) return;  // quadrant entirely past the vocabulary
    const int col = (a.vstart + vq) / kVocabPartial;  // global partial column (kWaveA == kVocabPartial)
    const bool tail = vq + kWaveA > a.V;
    const int half4 = 4 * (lane >> 5);
#pragma unroll
    for (int j = 0; j < kBlkB; ++j) {
      // target capture (rare: only when some lane's target falls in this quadrant)
      const int d = c.tgt[j] - vq - half4;
      float zsel = 0.f;
      bool hit = false;
      if (__builtin_amdgcn_ballot_w64(c.tgt[j] >= vq && c.tgt[j] < vq + kWaveA)) {
#pragma unroll
        for (int i = 0; i < kBlkA; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool m = (d == 32 * i + 8 * (r >> 2) + (r & 3));
            zsel = m ? acc.c[i][j][r] : zsel;
            hit = hit || m;
          }
      }
      // Column maximum in log2 units.  c2 > 0 and rounding is monotonic, so the maximum of
      // the scaled logits is the scaled maximum of the accumulators: take it on the raw
      // values (entries past the vocabulary set to -inf in place), then form each exponent
      // with one fma.
      if (tail) {
#pragma unroll
        for (int i = 0; i < kBlkA; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (vq + acc_row(i, r, lane) >= a.V) acc.c[i][j][r] = -INFINITY;
      }
      float am = -INFINITY;
#pragma unroll
      for (int i = 0; i < kBlkA; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) am = fmaxf(am, acc.c[i][j][r]);
      am = fmaxf(am, __shfl_xor(am, 32));
      const float mx = am * c2;
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
      for (int i = 0; i < kBlkA; ++i)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          s0 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc.c[i][j][r + 0], c2, -mx));
          s1 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc.c[i][j][r + 1], c2, -mx));
          s2 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc.c[i][j][r + 2], c2, -mx));
          s3 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc.c[i][j][r + 3], c2, -mx));
        }
      float s = (s0 + s1) + (s2 + s3);
      s = s + __shfl_xor(s, 32);
      const int ti = c.tok[j];
      if (ti < Na) {
        if (lane < 32) {
          a.part_max[(size_t)col * a.N + ti] = mx;
          a.part_sum[(size_t)col * a.N + ti] = s;
        }
        if (hit) a.target_logit[ti] = zsel * a.inv_t;
      }
    }
  };

  persistent_tiles<kBF16, FwdCtx>(sm, nTokTiles * nVocTiles, setup, epilogue);
}

// One work-group of 256 threads merges 32 compacted rows: thread (row = tid & 31,
// slice = tid >> 5) walks columns slice, slice + 8, ... in ascending order; the eight slice
// sums are added in a fixed tree.
__global__ __launch_bounds__(256) void fwd_merge_kernel(MergeArgs a) {
  __shared__ float red[8][33];
  const int Na = *a.n_active;
  const int i0 = blockIdx.x * 32;
  if (i0 >= Na) return;
  const int r = threadIdx.x & 31;
  const int sl = threadIdx.x >> 5;
  const int i = i0 + r;
  const bool ok = i < Na;
  const int J = (a.V + kVocabPartial - 1) / kVocabPartial;

  float m = -INFINITY;
  if (ok)
    for (int j = sl; j < J; j += 8) m = fmaxf(m, a.part_max[(size_t)j * a.N + i]);
  red[sl][r] = m;
  __syncthreads();
  float M = red[0][r];
#pragma unroll
  for (int k = 1; k < 8; ++k) M = fmaxf(M, red[k][r]);
  __syncthreads();

  float s = 0.f;
  if (ok)
    for (int j = sl; j < J; j += 8) {
      const size_t o = (size_t)j * a.N + i;
      s += a.part_sum[o] * __builtin_amdgcn_exp2f(a.part_max[o] - M);
    }
  red[sl][r] = s;
  __syncthreads();
  if (sl == 0 && ok) {
    const float S = ((red[0][r] + red[1][r]) + (red[2][r] + red[3][r])) +
                    ((red[4][r] + red[5][r]) + (red[6][r] + red[7][r]));
    const float lse = (M + __builtin_amdgcn_logf(S)) * kLn2;
    const int t = a.idx[i];
    a.logp[t] = a.target_logit[i] - lse;
    if (a.lse) a.lse[t] = lse;
  }
}

}  // namespace

hipError_t launch_fwd_tiles(const FwdTileArgs& a, bool bf16, int grid, hipStream_t stream) {
  if (bf16)
    hipLaunchKernelGGL(fwd_tiles_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(fwd_tiles_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd_merge(const MergeArgs& a, hipStream_t stream) {
  const int grid = (int)((a.N + 31) / 32);
  hipLaunchKernelGGL(fwd_merge_kernel, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rlk
