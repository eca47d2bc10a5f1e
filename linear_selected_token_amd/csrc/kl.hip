// Full-vocabulary KL between a teacher and a student LM head (RL-Kernel Roadmap (2026),
// operator backlog: chunked full-vocabulary / distillation KL fused with the LM head,
// forward and reverse).
//
// The vocabulary is walked in chunks of kBwdChunk entries.  Per chunk, each head's tile
// kernel (fwd_tiles_kernel in its kFwdStoreX mode, run as a vocabulary shard) writes its
// column statistics and x = z log2 e of the chunk, token-major, into a chunk buffer; the
// kernels below pair the two buffers entry by entry.  At most one chunk of each head's
// logits exists at a time.
//
//   kl_cross    per token and 128-entry column:
//                 wf = sum_v 2^(x_t - m_t) (x_t - x_s)   (forward KL's cross term)
//                 wr = sum_v 2^(x_s - m_s) (x_s - x_t)   (reverse KL's)
//               with m_t, m_s the columns' maxima.
//   kl_merge    per token, in the forward merge's fixed association: both heads' M and S,
//                 KL_fwd = ln2 (A_f / S_t - (M_t + log2 S_t) + (M_s + log2 S_s))
//                 KL_rev = ln2 (A_r / S_s - (M_s + log2 S_s) + (M_t + log2 S_t))
//               with A_f = sum_j 2^(m_t,j - M_t) wf_j and A_r likewise.
//   kl_grad     the backward's dL/dz of one chunk for L = sum_t (f_t KL_fwd,t + r_t KL_rev,t),
//               rounded to bf16 in the token-major layout the dL/dh and dL/dW GEMMs read (Gv):
//                 (f_t / T)(p_s - p_t) + (r_t / T) p_s (ln p_s - ln p_t - KL_rev)
//
// Every reduction is a fixed in-lane order followed by a fixed xor tree, and the columns
// are merged in one fixed order, so a token's results depend only on its own rows.
#include "common.hpp"
#include "aux_kernels.hpp"
#include "kernels.hpp"

namespace rlk {

namespace {

// One work-group of 4 waves per compacted token row; each 32-lane half of a wave takes one
// 128-entry column (4 entries per lane), so a wave step covers 2 columns.  A half takes its
// columns two at a time (both columns' loads issued before either is reduced); the chunk
// buffers are read once, with non-temporal loads.
__global__ __launch_bounds__(256) void kl_cross_kernel(KlArgs a, int c0) {
  const int Na = *a.n_active;
  const int i = blockIdx.x;
  if (i >= Na) return;
  const int vc = min(kBwdChunk, a.V - c0);
  const int ncol = (vc + 127) / 128;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const float* xs_row = a.xs + (size_t)i * kXPitch;
  const float* xt_row = a.xt + (size_t)i * kXPitch;
  auto ld = [&](const float* r, int v0) __attribute__((always_inline)) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(r + v0));
  };
  auto col_terms = [&](int jc, const f32x4& xs, const f32x4& xt, float ms,
                       float mt) __attribute__((always_inline)) {
    const int col = c0 / 128 + jc;
    const int v0 = jc * 128 + 4 * l32;
    const float s4[4] = {xs.x, xs.y, xs.z, xs.w};
    const float t4[4] = {xt.x, xt.y, xt.z, xt.w};
    float wf = 0.f, wr = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (v0 + e < vc) {  // entries past the vocabulary hold -inf in both buffers
        const float d = t4[e] - s4[e];
        wf = __builtin_fmaf(__builtin_amdgcn_exp2f(t4[e] - mt), d, wf);
        wr = __builtin_fmaf(__builtin_amdgcn_exp2f(s4[e] - ms), -d, wr);
      }
    }
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) {
      wf += __shfl_xor(wf, o);
      wr += __shfl_xor(wr, o);
    }
    if (l32 == 0) {
      a.wf[(size_t)col * a.N + i] = wf;
      a.wr[(size_t)col * a.N + i] = wr;
    }
  };
  for (int jc = 2 * wave + half; jc < ncol; jc += 16) {
    const bool two = jc + 8 < ncol;
    const int colA = c0 / 128 + jc, colB = colA + 8;
    const f32x4 xsA = ld(xs_row, jc * 128 + 4 * l32), xtA = ld(xt_row, jc * 128 + 4 * l32);
    f32x4 xsB = {0.f, 0.f, 0.f, 0.f}, xtB = {0.f, 0.f, 0.f, 0.f};
    float msB = 0.f, mtB = 0.f;
    if (two) {
      xsB = ld(xs_row, (jc + 8) * 128 + 4 * l32);
      xtB = ld(xt_row, (jc + 8) * 128 + 4 * l32);
      msB = a.s_max[(size_t)colB * a.N + i];
      mtB = a.t_max[(size_t)colB * a.N + i];
    }
    const float msA = a.s_max[(size_t)colA * a.N + i];
    const float mtA = a.t_max[(size_t)colA * a.N + i];
    col_terms(jc, xsA, xtA, msA, mtA);
    if (two) col_terms(jc + 8, xsB, xtB, msB, mtB);
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

// Two floats to packed bf16, round to nearest even.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// One work-group per row of Gv (rows up to the active count rounded to the tile, the rest
// exit); each thread forms 4 consecutive entries per step, two steps at a time (both steps'
// non-temporal loads issued first).  Rows past the active count and
// entries past the vocabulary are written as 0, since the GEMMs that follow read them.
// kF / kR: the forward / reverse KL term is present (coef_f / coef_r given).
template <bool kF, bool kR>
__global__ __launch_bounds__(256) void kl_grad_kernel(KlArgs a, int c0) {
  const int Na = *a.n_active;
  const int i = blockIdx.x;
  const int rows = (Na + 255) / 256 * 256;
  if (i >= rows) return;
  const int vc = min(kBwdChunk, a.V - c0);
  const int vt = (vc + 255) / 256 * 256;  // entries the tiles of the chunk cover
  const bool act = i < Na;
  float lse2s = 0.f, lse2t = 0.f, cf = 0.f, cr = 0.f, klr = 0.f;
  if (act) {
    const int t = a.idx[i];
    lse2s = a.lse_s_in[t] * kLog2e;
    lse2t = a.lse_t_in[t] * kLog2e;
    if constexpr (kF) cf = a.coef_f[t] * a.inv_t;
    if constexpr (kR) {
      cr = a.coef_r[t] * a.inv_t;
      klr = a.kl_rev_in[t];
    }
  }
  const float* xs_row = a.xs + (size_t)i * kXPitch;
  const float* xt_row = a.xt + (size_t)i * kXPitch;
  uint16_t* g_row = a.Gv + (size_t)i * kGvPitch;
  auto grad4 = [&](int v0, const f32x4& xs, const f32x4& xt) __attribute__((always_inline)) {
    float G[4] = {0.f, 0.f, 0.f, 0.f};
    if (act && v0 < vc) {
      const float s4[4] = {xs.x, xs.y, xs.z, xs.w};
      const float t4[4] = {xt.x, xt.y, xt.z, xt.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (v0 + e < vc) {
          const float ls = s4[e] - lse2s;  // log2 p_s
          const float lt = t4[e] - lse2t;
          const float ps = __builtin_amdgcn_exp2f(ls);
          float g = 0.f;
          if constexpr (kF) g = cf * (ps - __builtin_amdgcn_exp2f(lt));
          if constexpr (kR) g = __builtin_fmaf(cr * ps, __builtin_fmaf(ls - lt, kLn2, -klr), g);
          G[e] = g;
        }
      }
    }
    u32x2 pk;
    pk[0] = pack2(G[0], G[1]);
    pk[1] = pack2(G[2], G[3]);
    *reinterpret_cast<u32x2*>(g_row + v0) = pk;
  };
  auto ld = [&](const float* r, int v0) __attribute__((always_inline)) {
    return (act && v0 < vc) ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(r + v0))
                            : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  for (int v0 = 4 * threadIdx.x; v0 < vt; v0 += 2048) {
    const int v1 = v0 + 1024;
    const f32x4 xs0 = ld(xs_row, v0), xt0 = ld(xt_row, v0);
    const f32x4 xs1 = ld(xs_row, v1), xt1 = ld(xt_row, v1);
    grad4(v0, xs0, xt0);
    if (v1 < vt) grad4(v1, xs1, xt1);
  }
}

}  // namespace

hipError_t launch_kl_cross(const KlArgs& a, int c0, int rows, hipStream_t stream) {
  if (rows > 0) hipLaunchKernelGGL(kl_cross_kernel, dim3(rows), dim3(256), 0, stream, a, c0);
  return hipGetLastError();
}

hipError_t launch_kl_merge(const KlArgs& a, hipStream_t stream) {
  const int blocks = (a.N + 31) / 32;
  if (blocks > 0) hipLaunchKernelGGL(kl_merge_kernel, dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_kl_grad(const KlArgs& a, int c0, int rows, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (a.coef_f && a.coef_r)
    hipLaunchKernelGGL((kl_grad_kernel<true, true>), dim3(rows), dim3(256), 0, stream, a, c0);
  else if (a.coef_r)
    hipLaunchKernelGGL((kl_grad_kernel<false, true>), dim3(rows), dim3(256), 0, stream, a, c0);
  else
    hipLaunchKernelGGL((kl_grad_kernel<true, false>), dim3(rows), dim3(256), 0, stream, a, c0);
  return hipGetLastError();
}

}  // namespace rlk
