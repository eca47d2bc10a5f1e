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
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "mainloop.hpp"

namespace rlk {

namespace {

// The 16-bit codes of two entries' exponents d = acc c2 - mx <= 0 (log2 units): -d 2^9 rounded
// half up and clamped to [0, 65535], as one fma per entry with k1 = -c2 2^9 and
// k2 = mx 2^9 + 1/2, then truncation (a -inf entry past the vocabulary gives 65535; the
// column maximum's own rounding residual gives 0).  Two codes per word, the first in the low
// half.
__device__ __forceinline__ uint32_t pack_dcode(float acc_lo, float acc_hi, float k1, float k2) {
  const float lo = __builtin_amdgcn_fmed3f(__builtin_fmaf(acc_lo, k1, k2), 0.f, 65535.f);
  const float hi = __builtin_amdgcn_fmed3f(__builtin_fmaf(acc_hi, k1, k2), 0.f, 65535.f);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pk_u16((uint32_t)lo, (uint32_t)hi));
}

struct FwdCtx {
  int vq;      // first vocabulary entry of this wave's quadrant
  int tok[kBlkB];  // compacted token index of each of this lane's token columns
  int tgt[kBlkB];  // their targets (-1: none or out of range)
};

// Epilogue modes.  The column maximum and sum are computed the same way in every mode.
//   kFwdPlain    column max and sum, target logit.
//   kFwdEntropy  also part_w = sum_v e_v max(d_v, -126) with d_v = x_v - max (log2 units)
//                and e_v = 2^d_v; the clamp only touches terms whose e_v is 0 (entries past
//                the vocabulary, or underflowed), so the column's sum_v e_v x_v is
//                part_w + max * part_sum.
//   kFwdStoreD   the plain statistics and target, and d = x - max of every entry of the tile
//                (the exponent the column sum adds up, <= 0) into dbuf as a 16-bit code,
//                -d 2^9 rounded and clamped to [0, 65535]: steps of 2^-9 over (-128, 0], so the
//                p = 2^(d + max - lse) it gives back carries at most 2^-10 ln 2 relative error
//                whatever d is (entries with d <= -128 have p < 2^-128).  Token-major rows of
//                d_pitch codes, entry v of the vocabulary at column v, one row per compacted
//                token of the launch (padded token columns included).  The fused forward +
//                backward turns these rows into dL/dz once lse is known, in place of a second
//                pass of the GEMM.
//   kFwdStoreDEnt kFwdStoreD plus the entropy statistic of kFwdEntropy (the fused call with an
//                entropy bonus).
template <bool kBF16, int kMode>
__global__ __launch_bounds__(kThreads) void fwd_tiles_kernel(FwdTileArgs a) {
  constexpr bool kEnt = kMode == kFwdEntropy || kMode == kFwdStoreDEnt;
  constexpr bool kStoreD = kMode == kFwdStoreD || kMode == kFwdStoreDEnt;
  __shared__ RingSmem sm;
  const int Na = *a.n_active;
  const int nTokTiles = (Na + kTile - 1) / kTile;
  const int nVocTiles = (a.V + kTile - 1) / kTile;
  // bands of 8 token tiles; up to 12 token tiles (a token block of the fused call) take one
  // band, instead of a band of 8 and a narrow remainder band whose work-groups share few panels
  const int band = nTokTiles <= 12 ? nTokTiles : 8;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const size_t row_bytes = (size_t)a.H * (kBF16 ? 2 : 4);
  const int nk = (int)(row_bytes / kKBytes);
  const float c2 = a.inv_t * kLog2e;
  const int wv = wave_a0(wave);  // vocabulary offset of the wave sub-tile
  const int wt = wave_b0(wave);  // token offset of the wave sub-tile
  const size_t pst = a.pstride > 0 ? (size_t)a.pstride : (size_t)a.N;  // partial column stride

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
      // values (entries past the vocabulary read as -inf), then form each exponent with one
      // fma.  The -inf is applied where a value is read, and only in the quadrant that holds
      // the vocabulary's end: the body is instantiated with and without the mask (written
      // into the accumulators in place, it made the store-code epilogues spill).
      const int lim = a.V - vq - half4;  // local rows >= lim are past the vocabulary
      auto column = [&](auto masked) __attribute__((always_inline)) {
        auto val = [&](int i, int r) __attribute__((always_inline)) -> float {
          const float x = acc.c[i][j][r];
          if constexpr (decltype(masked)::value)
            return 32 * i + 8 * (r >> 2) + (r & 3) >= lim ? -INFINITY : x;
          else
            return x;
        };
        float am = -INFINITY;
#pragma unroll
        for (int i = 0; i < kBlkA; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) am = fmaxf(am, val(i, r));
        am = fmaxf(am, __shfl_xor(am, 32));
        const float mx = am * c2;
        float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
        float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 0.f;
#pragma unroll
        for (int i = 0; i < kBlkA; ++i)
#pragma unroll
          for (int r = 0; r < 16; r += 4) {
            const float d0 = __builtin_fmaf(val(i, r + 0), c2, -mx);
            const float d1 = __builtin_fmaf(val(i, r + 1), c2, -mx);
            const float d2 = __builtin_fmaf(val(i, r + 2), c2, -mx);
            const float d3 = __builtin_fmaf(val(i, r + 3), c2, -mx);
            const float e0 = __builtin_amdgcn_exp2f(d0);
            const float e1 = __builtin_amdgcn_exp2f(d1);
            const float e2 = __builtin_amdgcn_exp2f(d2);
            const float e3 = __builtin_amdgcn_exp2f(d3);
            s0 += e0;
            s1 += e1;
            s2 += e2;
            s3 += e3;
            if constexpr (kEnt) {
              w0 = __builtin_fmaf(e0, fmaxf(d0, -126.f), w0);
              w1 = __builtin_fmaf(e1, fmaxf(d1, -126.f), w1);
              w2 = __builtin_fmaf(e2, fmaxf(d2, -126.f), w2);
              w3 = __builtin_fmaf(e3, fmaxf(d3, -126.f), w3);
            }
          }
        float s = (s0 + s1) + (s2 + s3);
        s = s + __shfl_xor(s, 32);
        float w = 0.f;
        if constexpr (kEnt) {
          w = (w0 + w1) + (w2 + w3);
          w = w + __shfl_xor(w, 32);
        }
        const int ti = c.tok[j];
        if constexpr (kStoreD) {
          // codes of the wave's 128 entries for this token column, 16 bytes per lane: per 32-entry
          // block, v_permlane32_swap on the packed groups (2h, 2h + 1) hands lane l entries
          // 16 h + 0..7 and lane l + 32 entries 16 h + 8..15 of the same token (as for dL/dz).
          // Rows of padded token columns (ti >= Na, still inside the block's rows) are written
          // too and never read as d.
          uint16_t* drow = a.dbuf + (size_t)ti * a.d_pitch + vq;
          const float k1 = -c2 * 512.f;
          const float k2 = __builtin_fmaf(mx, 512.f, 0.5f);
#pragma unroll
          for (int i = 0; i < kBlkA; ++i) {
            u32x2 pk[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              pk[g][0] = pack_dcode(val(i, 4 * g + 0), val(i, 4 * g + 1), k1, k2);
              pk[g][1] = pack_dcode(val(i, 4 * g + 2), val(i, 4 * g + 3), k1, k2);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const auto s0 =
                  __builtin_amdgcn_permlane32_swap(pk[2 * h][0], pk[2 * h + 1][0], false, false);
              const auto s1 =
                  __builtin_amdgcn_permlane32_swap(pk[2 * h][1], pk[2 * h + 1][1], false, false);
              u32x4 q;
              q.x = s0[0];
              q.y = s1[0];
              q.z = s0[1];
              q.w = s1[1];
              *reinterpret_cast<u32x4*>(drow + 32 * i + 16 * h + 8 * (lane >> 5)) = q;
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (ti < Na) {
          if (lane < 32) {
            a.part_max[col * pst + ti] = mx;
            a.part_sum[col * pst + ti] = s;
            if constexpr (kEnt) a.part_w[col * pst + ti] = w;
          }
          if (hit) a.target_logit[ti] = zsel * a.inv_t;
        }
      };
      if (tail) column(std::true_type{});
      else column(std::false_type{});
    }
  };

  persistent_tiles<kBF16, FwdCtx>(sm, nTokTiles * nVocTiles, setup, epilogue);
}

// One work-group of 256 threads merges 32 compacted rows: thread (row = tid & 31,
// slice = tid >> 5) walks columns slice, slice + 8, ... in ascending order; the eight slice
// sums are added in a fixed tree.
template <bool kEnt>
__global__ __launch_bounds__(256) void fwd_merge_kernel(MergeArgs a) {
  __shared__ float red[8][33];
  __shared__ float wred[8][33];
  constexpr int kU = 8;  // columns in flight per thread (the walk order is unchanged)
  const int Na = *a.n_active;
  const int i0 = blockIdx.x * 32;
  if (i0 >= Na) return;
  const int r = threadIdx.x & 31;
  const int sl = threadIdx.x >> 5;
  const int i = i0 + r;
  const bool ok = i < Na;
  const int J = (a.V + kVocabPartial - 1) / kVocabPartial;
  const float* pmax = a.part_max + i;
  const float* psum = a.part_sum + i;
  const size_t N = a.N;

  float m = -INFINITY;
  if (ok) {
    int j = sl;
    for (; j + 8 * (kU - 1) < J; j += 8 * kU) {
      float x[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) x[u] = pmax[(size_t)(j + 8 * u) * N];
#pragma unroll
      for (int u = 0; u < kU; ++u) m = fmaxf(m, x[u]);
    }
    for (; j < J; j += 8) m = fmaxf(m, pmax[(size_t)j * N]);
  }
  red[sl][r] = m;
  __syncthreads();
  float M = red[0][r];
#pragma unroll
  for (int k = 1; k < 8; ++k) M = fmaxf(M, red[k][r]);
  __syncthreads();

  // column j adds part_sum 2^(part_max - M) to s and, for the entropy, sum_v 2^(x_v - M)
  // (x_v - M) over the column to w; columns sl, sl + 8, ... in ascending order
  float s = 0.f, w = 0.f;
  auto add = [&](float pm, float ps, float pw) __attribute__((always_inline)) {
    const float f = __builtin_amdgcn_exp2f(pm - M);
    s += ps * f;
    if constexpr (kEnt) w += (pw + (pm - M) * ps) * f;
  };
  if (ok) {
    int j = sl;
    for (; j + 8 * (kU - 1) < J; j += 8 * kU) {
      float x[kU], y[kU], z[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const size_t o = (size_t)(j + 8 * u) * N;
        x[u] = pmax[o];
        y[u] = psum[o];
        z[u] = kEnt ? a.part_w[o + i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) add(x[u], y[u], z[u]);
    }
    for (; j < J; j += 8) {
      const size_t o = (size_t)j * N;
      add(pmax[o], psum[o], kEnt ? a.part_w[o + i] : 0.f);
    }
  }
  red[sl][r] = s;
  wred[sl][r] = w;
  __syncthreads();
  if (sl == 0 && ok) {
    const float S = ((red[0][r] + red[1][r]) + (red[2][r] + red[3][r])) +
                    ((red[4][r] + red[5][r]) + (red[6][r] + red[7][r]));
    const float log2S = __builtin_amdgcn_logf(S);
    const float lse = (M + log2S) * kLn2;
    const int t = a.idx[i];
    a.logp[t] = a.target_logit[i] - lse;
    if (a.lse) a.lse[t] = lse;
    if constexpr (kEnt) {
      // H = lse - E_p[z] = ln2 (log2 S - E_p[x - M]) in log2 units x = z log2 e
      const float A = ((wred[0][r] + wred[1][r]) + (wred[2][r] + wred[3][r])) +
                      ((wred[4][r] + wred[5][r]) + (wred[6][r] + wred[7][r]));
      // rounding can leave a near-certain token a few ulp below zero; the entropy is >= 0
      a.entropy[t] = fmaxf((log2S - A / S) * kLn2, 0.f);
    }
  }
}

}  // namespace

template <int kMode>
void launch_mode(const FwdTileArgs& a, bool bf16, int grid, hipStream_t stream) {
  if (bf16)
    hipLaunchKernelGGL((fwd_tiles_kernel<true, kMode>), dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_tiles_kernel<false, kMode>), dim3(grid), dim3(kThreads), 0, stream, a);
}

hipError_t launch_fwd_tiles(const FwdTileArgs& a, bool bf16, int grid, hipStream_t stream,
                            int mode) {
  switch (mode) {
    case kFwdPlain: launch_mode<kFwdPlain>(a, bf16, grid, stream); break;
    case kFwdEntropy: launch_mode<kFwdEntropy>(a, bf16, grid, stream); break;
    case kFwdStoreD:
      if (!bf16) return hipErrorInvalidValue;
      hipLaunchKernelGGL((fwd_tiles_kernel<true, kFwdStoreD>), dim3(grid), dim3(kThreads), 0,
                         stream, a);
      break;
    case kFwdStoreDEnt:
      if (!bf16) return hipErrorInvalidValue;
      hipLaunchKernelGGL((fwd_tiles_kernel<true, kFwdStoreDEnt>), dim3(grid), dim3(kThreads), 0,
                         stream, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fwd_merge(const MergeArgs& a, hipStream_t stream) {
  const int grid = (int)((a.N + 31) / 32);
  if (a.part_w)
    hipLaunchKernelGGL(fwd_merge_kernel<true>, dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(fwd_merge_kernel<false>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rlk
