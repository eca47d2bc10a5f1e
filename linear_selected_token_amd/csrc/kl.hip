// Full-vocabulary KL between a teacher and a student LM head (RL-Kernel Roadmap (2026),
// operator backlog: chunked full-vocabulary / distillation KL fused with the LM head,
// forward and reverse).
//
//   kl_tiles    persistent grid over (vocabulary tile x token tile) pairs.  Per tile, the
//               teacher's z_t = W_t h_t^T and then the student's z_s = W_s h_s^T, each on
//               MFMA with fp32 accumulation over its whole hidden dimension in one fixed K
//               order (the forward tile kernel's loop).  The teacher's accumulators wait in
//               the work-group's scratch slot while the student's are formed; the student's
//               epilogue pairs the two entry by entry, in log2 units x = z log2 e:
//                 forward: per token and 128-entry column, both heads' column maximum m and
//                   sum of 2^(x - m), and the cross terms
//                     wf = sum_v 2^(x_t - m_t) (x_t - x_s)   (forward KL)
//                     wr = sum_v 2^(x_s - m_s) (x_s - x_t)   (reverse KL)
//                 backward: for L = sum_t (f_t KL_fwd,t + r_t KL_rev,t), the student's
//                     dL/dz = (f_t / T)(p_s - p_t) + (r_t / T) p_s (ln p_s - ln p_t - KL_rev)
//                   rounded to bf16 in the token-major layout the dL/dh and dL/dW GEMMs read.
//               No logits of either head reach memory.
//   kl_merge    per token, in the forward merge's fixed association: both heads' M and S,
//                 KL_fwd = ln2 (A_f / S_t - (M_t + log2 S_t) + (M_s + log2 S_s))
//                 KL_rev = ln2 (A_r / S_s - (M_s + log2 S_s) + (M_t + log2 S_t))
//               with A_f = sum_j 2^(m_t,j - M_t) wf_j and A_r likewise.
//
// Every reduction is a fixed in-lane order followed by a fixed xor tree, and the columns
// are merged in one fixed order, so a token's results depend only on its own rows.
#include "common.hpp"
#include "aux_kernels.hpp"
#include "kernels.hpp"
#include "mainloop.hpp"

namespace rlk {

namespace {

// Two floats to packed bf16, round to nearest even.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

struct KlCtx {
  int vbase, tbase;  // first vocabulary entry (of the launch) and first compacted token
  int tok[kBlkB];    // this lane's token columns (compacted index within the block)
};

// kGrad: the backward's dL/dz (kF / kR: the forward / reverse term is present); otherwise
// the forward's column statistics.
template <bool kBF16, bool kGrad, bool kF, bool kR>
__global__ __launch_bounds__(kThreads) void kl_tiles_kernel(KlTileArgs a) {
  __shared__ RingSmem sm;
  const int Na = *a.n_active;
  const int nTokTiles = (Na + kTile - 1) / kTile;
  const int nVocTiles = (a.V + kTile - 1) / kTile;
  const int n_tiles = nTokTiles * nVocTiles;
  const int band = nTokTiles <= 12 ? nTokTiles : 8;  // as the forward tile kernel's order
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const size_t es = kBF16 ? 2 : 4;
  const size_t rb_t = (size_t)a.H_t * es;
  const size_t rb_s = (size_t)a.H_s * es;
  const float c2 = a.inv_t * kLog2e;
  const int wv = wave_a0(wave);  // vocabulary offset of the wave sub-tile
  const int wt = wave_b0(wave);  // token offset of the wave sub-tile
  const int half4 = 4 * (lane >> 5);
  // this lane's 32 vectors in the work-group's slot: vector e at slot[64 e]
  f32x4* slot = reinterpret_cast<f32x4*>(a.scratch) +
                ((size_t)blockIdx.x * kWaves + wave) * (kBlkA * kBlkB * 4 * 64) + lane;

  // load sources of one head's GEMM for the tile at (vbase, tbase): rows of W past the launch's
  // vocabulary repeat its last row (the epilogue drops them), token rows past the block repeat
  // its last token (their columns are dropped or zeroed)
  auto head_src = [&](const void* W, const void* h, size_t rb, const KlCtx& c, TileSrc& src) {
    src.nk = (int)(rb / kKBytes);
    src.a_kstep = src.b_kstep = kKBytes;
    src.a = uniform_ptr(static_cast<const uint8_t*>(W) + (size_t)c.vbase * rb);
    src.b = uniform_ptr(h);
    src.a_bytes = operand_bytes((size_t)(a.V - c.vbase) * rb);
    src.b_bytes = operand_bytes((size_t)a.N * rb);
#pragma unroll
    for (int q = 0; q < kDmaPerWave; ++q) {
      const int r = dma_row(q, wave, lane);
      const int ch = dma_chunk(q, wave, lane);
      const int v = min(c.vbase + r, a.V - 1);
      const int t = a.idx[min(c.tbase + r, Na - 1)];
      src.ao[q] = (uint32_t)((size_t)(v - c.vbase) * rb) + 16 * ch;
      src.bo[q] = (uint32_t)((size_t)t * rb) + 16 * ch;
    }
  };
  auto setup = [&](int u, KlCtx& c) {
    int vt, tt;
    tile_coords(u, nVocTiles, nTokTiles, band, vt, tt);
    c.vbase = vt * kTile;
    c.tbase = tt * kTile;
#pragma unroll
    for (int j = 0; j < kBlkB; ++j) c.tok[j] = c.tbase + wt + acc_col(j, lane);
  };

  // The teacher's accumulators of block (i, j), group g, go to vector 4 (i kBlkB + j) + g; for
  // the forward, each token column's maximum over the wave's vocabulary rows (log2 units; rows
  // past the vocabulary left out) is taken on the way.
  auto stash = [&](const KlCtx& c, const Acc& acc, float (&mt)[kBlkB]) {
    const int lim = a.V - c.vbase - wv - half4;  // row offsets >= lim are past the vocabulary
    const bool tail = c.vbase + wv + kWaveA > a.V;  // wave-uniform
#pragma unroll
    for (int j = 0; j < kBlkB; ++j) {
      float am = -INFINITY;
#pragma unroll
      for (int i = 0; i < kBlkA; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v;
          v.x = acc.c[i][j][4 * g + 0];
          v.y = acc.c[i][j][4 * g + 1];
          v.z = acc.c[i][j][4 * g + 2];
          v.w = acc.c[i][j][4 * g + 3];
          slot[64 * ((i * kBlkB + j) * 4 + g)] = v;
          if constexpr (!kGrad) {
            if (tail) {
              const int o = 32 * i + 8 * g;
              v.x = o + 0 < lim ? v.x : -INFINITY;
              v.y = o + 1 < lim ? v.y : -INFINITY;
              v.z = o + 2 < lim ? v.z : -INFINITY;
              v.w = o + 3 < lim ? v.w : -INFINITY;
            }
            am = fmaxf(fmaxf(am, v.x), fmaxf(v.y, fmaxf(v.z, v.w)));
          }
        }
      if constexpr (!kGrad) mt[j] = fmaxf(am, __shfl_xor(am, 32)) * c2;
    }
  };

  // The teacher's accumulators of block (i, j), as the student's are laid out.
  auto unstash = [&](int i, int j, float (&tv)[16]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 v = slot[64 * ((i * kBlkB + j) * 4 + g)];
      tv[4 * g + 0] = v.x;
      tv[4 * g + 1] = v.y;
      tv[4 * g + 2] = v.z;
      tv[4 * g + 3] = v.w;
    }
  };

  // Per token column j of the student's accumulators in acc.  Entry (i, r) is vocabulary row
  // vq + acc_row(i, r, lane), at row offset 32 i + 8 (r >> 2) + (r & 3) from this lane's first.
  // The teacher's blocks are read back one ahead of the one in use.
  auto epilogue = [&](const KlCtx& c, Acc& acc, const float (&mt)[kBlkB]) {
    const int vq = c.vbase + wv;
    if (vq >= a.V) return;  // quadrant entirely past the vocabulary
    const bool tail = vq + kWaveA > a.V;  // wave-uniform
    const int lim = a.V - vq - half4;
    float tv[2][16];
    unstash(0, 0, tv[0]);
#pragma unroll
    for (int j = 0; j < kBlkB; ++j) {
      const int ti = c.tok[j];
      if constexpr (!kGrad) {
        // entries past the vocabulary: -inf in the student's maximum, no term in the sums
        float am = -INFINITY;
        if (tail) {
#pragma unroll
          for (int i = 0; i < kBlkA; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * i + 8 * (r >> 2) + (r & 3) >= lim) acc.c[i][j][r] = -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < kBlkA; ++i)
#pragma unroll
          for (int r = 0; r < 16; r += 2)
            am = fmaxf(am, fmaxf(acc.c[i][j][r], acc.c[i][j][r + 1]));
        const float ms = fmaxf(am, __shfl_xor(am, 32)) * c2;
        // wf and wr are summed in accumulator units: wf = c2 sum et (t - s), wr = c2 sum es (s - t)
        float st = 0.f, ss = 0.f, wf = 0.f, wr = 0.f;
#pragma unroll
        for (int i = 0; i < kBlkA; ++i) {
          const int cb = (j * kBlkA + i) & 1;
          if (j * kBlkA + i + 1 < kBlkA * kBlkB)
            unstash((i + 1) % kBlkA, j + (i + 1) / kBlkA, tv[cb ^ 1]);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float t = tv[cb][r];
            const float s_ = acc.c[i][j][r];  // -inf past the vocabulary
            const float et = __builtin_amdgcn_exp2f(__builtin_fmaf(t, c2, -mt[j]));
            const float e_s = __builtin_amdgcn_exp2f(__builtin_fmaf(s_, c2, -ms));
            float d = t - s_;
            if (tail) d = 32 * i + 8 * (r >> 2) + (r & 3) < lim ? d : 0.f;
            st += tail && !(32 * i + 8 * (r >> 2) + (r & 3) < lim) ? 0.f : et;
            ss += e_s;
            wf = __builtin_fmaf(et, d, wf);
            wr = __builtin_fmaf(e_s, -d, wr);
          }
        }
        float o[4] = {st, ss, wf * c2, wr * c2};
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] += __shfl_xor(o[q], 32);
        if (ti < Na && lane < 32) {
          const size_t at = (size_t)((a.vstart + vq) / kVocabPartial) * a.pstride + ti;
          a.t_max[at] = mt[j];
          a.t_sum[at] = o[0];
          a.s_max[at] = ms;
          a.s_sum[at] = o[1];
          a.wf[at] = o[2];
          a.wr[at] = o[3];
        }
      } else {
        // dL/dz of every entry, 0 past the vocabulary and in padded token columns; stored as
        // the backward's logits pass stores it (per 32-entry block, v_permlane32_swap hands
        // lane l entries 16 h + 0..7 and lane l + 32 entries 16 h + 8..15 of the same token)
        const bool act = ti < Na;
        const int t = act ? a.idx[ti] : 0;
        const float lse2s = act ? a.lse_s[t] * kLog2e : 0.f;
        const float lse2t = act ? a.lse_t[t] * kLog2e : 0.f;
        const float cf = (kF && act) ? a.coef_f[t] * a.inv_t : 0.f;
        const float cr = (kR && act) ? a.coef_r[t] * a.inv_t : 0.f;
        const float klr = (kR && act) ? a.kl_rev[t] : 0.f;
        const int lj = act ? lim : 0;  // entries at row offset >= lj are 0
        const bool zero_some = tail || !act;
#pragma unroll
        for (int i = 0; i < kBlkA; ++i) {
          const int cb = (j * kBlkA + i) & 1;
          if (j * kBlkA + i + 1 < kBlkA * kBlkB)
            unstash((i + 1) % kBlkA, j + (i + 1) / kBlkA, tv[cb ^ 1]);
          u32x2 pk[4];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float G[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * g + e;
              const float ls = __builtin_fmaf(acc.c[i][j][r], c2, -lse2s);  // log2 p_s
              const float lt = __builtin_fmaf(tv[cb][r], c2, -lse2t);
              const float ps = __builtin_amdgcn_exp2f(ls);
              float gv = 0.f;
              if constexpr (kF) gv = cf * (ps - __builtin_amdgcn_exp2f(lt));
              if constexpr (kR) gv = __builtin_fmaf(cr * ps, __builtin_fmaf(ls - lt, kLn2, -klr), gv);
              if (zero_some) gv = (32 * i + 8 * g + e < lj) ? gv : 0.f;
              G[e] = gv;
            }
            pk[g][0] = pack2(G[0], G[1]);
            pk[g][1] = pack2(G[2], G[3]);
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
            const int vl = vq + 32 * i + 16 * h + 8 * (lane >> 5);  // first of 8
            *reinterpret_cast<u32x4*>(a.Gv + (size_t)ti * a.gv_pitch + vl) = q;
          }
        }
      }
    }
  };

  // The persistent walk (the tile driver of the forward kernel, with two GEMMs per tile): the
  // student's first loads go out before the teacher's accumulators are stashed, the next tile's
  // teacher loads before the epilogue.
  int round = 0;
  int u = virtual_tile(round, blockIdx.x, gridDim.x);
  if (u >= n_tiles) return;
  TileSrc src;
  KlCtx ctx;
  setup(u, ctx);
  head_src(a.W_t, a.h_t, rb_t, ctx, src);
  ring_prologue(sm, src, src.nk);
  while (true) {
    Acc acc;
    zero_acc(acc);
    ring_mainloop<kBF16, false, false>(sm, src, src.nk, acc);  // teacher
    head_src(a.W_s, a.h_s, rb_s, ctx, src);
    ring_prologue(sm, src, src.nk);
    float mt[kBlkB];
    stash(ctx, acc, mt);
    zero_acc(acc);
    ring_mainloop<kBF16, false, false>(sm, src, src.nk, acc);  // student
    const int un = virtual_tile(++round, blockIdx.x, gridDim.x);
    const bool more = un < n_tiles;
    const KlCtx cur = ctx;
    if (more) {
      setup(un, ctx);
      head_src(a.W_t, a.h_t, rb_t, ctx, src);
      ring_prologue(sm, src, src.nk);
    }
    epilogue(cur, acc, mt);
    if (!more) break;
  }
}

// 32 compacted rows per work-group of 256 threads; thread (row = tid & 31, slice = tid >> 5)
// walks columns slice, slice + 8, ... in ascending order, the 8 slices are added in a fixed
// tree (the forward merge's association).
__global__ __launch_bounds__(256) void kl_merge_kernel(KlArgs a) {
  __shared__ float red[6][8][33];
  const int Na = *a.n_active;
  const int r = threadIdx.x & 31;
  const int sl = threadIdx.x >> 5;
  const int i = blockIdx.x * 32 + r;
  const bool ok = i < Na;
  const int J = (a.V + 127) / 128;
  constexpr int kU = 8;  // columns in flight per thread (the walk order is unchanged)
  float mt = -INFINITY, ms = -INFINITY;
  if (ok) {
    int j = sl;
    for (; j + 8 * (kU - 1) < J; j += 8 * kU) {
      float xt[kU], xs[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        xt[u] = a.t_max[(size_t)(j + 8 * u) * a.N + i];
        xs[u] = a.s_max[(size_t)(j + 8 * u) * a.N + i];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        mt = fmaxf(mt, xt[u]);
        ms = fmaxf(ms, xs[u]);
      }
    }
    for (; j < J; j += 8) {
      mt = fmaxf(mt, a.t_max[(size_t)j * a.N + i]);
      ms = fmaxf(ms, a.s_max[(size_t)j * a.N + i]);
    }
  }
  red[0][sl][r] = mt;
  red[1][sl][r] = ms;
  __syncthreads();
  float Mt = red[0][0][r], Ms = red[1][0][r];
#pragma unroll
  for (int k = 1; k < 8; ++k) {
    Mt = fmaxf(Mt, red[0][k][r]);
    Ms = fmaxf(Ms, red[1][k][r]);
  }
  __syncthreads();
  float st = 0.f, ss = 0.f, af = 0.f, ar = 0.f;
  auto add = [&](size_t o) __attribute__((always_inline)) {
    const float ft = __builtin_amdgcn_exp2f(a.t_max[o] - Mt);
    const float fs = __builtin_amdgcn_exp2f(a.s_max[o] - Ms);
    st += a.t_sum[o] * ft;
    ss += a.s_sum[o] * fs;
    af += a.wf[o] * ft;
    ar += a.wr[o] * fs;
  };
  if (ok) {
    int j = sl;
    for (; j + 8 * (kU - 1) < J; j += 8 * kU) {
#pragma unroll
      for (int u = 0; u < kU; ++u) add((size_t)(j + 8 * u) * a.N + i);
    }
    for (; j < J; j += 8) add((size_t)j * a.N + i);
  }
  red[2][sl][r] = st;
  red[3][sl][r] = ss;
  red[4][sl][r] = af;
  red[5][sl][r] = ar;
  __syncthreads();
  if (sl == 0 && ok) {
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float (*x)[33] = red[2 + q];
      v[q] = ((x[0][r] + x[1][r]) + (x[2][r] + x[3][r])) + ((x[4][r] + x[5][r]) + (x[6][r] + x[7][r]));
    }
    const float lt2 = Mt + __builtin_amdgcn_logf(v[0]);  // lse_t in log2 units
    const float ls2 = Ms + __builtin_amdgcn_logf(v[1]);
    const int t = a.idx[i];
    // KL >= 0; rounding can leave a near-zero divergence a few ulp below it
    a.kl_fwd[t] = fmaxf((v[2] / v[0] - lt2 + ls2) * kLn2, 0.f);
    a.kl_rev[t] = fmaxf((v[3] / v[1] - ls2 + lt2) * kLn2, 0.f);
    if (a.lse_s) a.lse_s[t] = ls2 * kLn2;
    if (a.lse_t) a.lse_t[t] = lt2 * kLn2;
  }
}

}  // namespace

hipError_t launch_kl_tiles(const KlTileArgs& a, bool bf16, bool grad, int grid, hipStream_t stream) {
  if (grid > kKlSlots) grid = kKlSlots;
  if (!grad) {
    if (bf16)
      hipLaunchKernelGGL((kl_tiles_kernel<true, false, false, false>), dim3(grid), dim3(kThreads), 0,
                         stream, a);
    else
      hipLaunchKernelGGL((kl_tiles_kernel<false, false, false, false>), dim3(grid), dim3(kThreads), 0,
                         stream, a);
  } else if (!bf16) {
    return hipErrorInvalidValue;  // the backward is bf16 only
  } else if (a.coef_f && a.coef_r) {
    hipLaunchKernelGGL((kl_tiles_kernel<true, true, true, true>), dim3(grid), dim3(kThreads), 0,
                       stream, a);
  } else if (a.coef_r) {
    hipLaunchKernelGGL((kl_tiles_kernel<true, true, false, true>), dim3(grid), dim3(kThreads), 0,
                       stream, a);
  } else {
    hipLaunchKernelGGL((kl_tiles_kernel<true, true, true, false>), dim3(grid), dim3(kThreads), 0,
                       stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_kl_merge(const KlArgs& a, hipStream_t stream) {
  const int blocks = (a.N + 31) / 32;
  if (blocks > 0) hipLaunchKernelGGL(kl_merge_kernel, dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rlk
