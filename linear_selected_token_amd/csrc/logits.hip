// Selected-token log-prob from logits that already exist: the reference-scoring sibling of
// the fused path (RL-Kernel integration roadmap for vime, "Operator Integration Plan", logp
// Reference Scoring: a deterministic policy with a fixed row-local reduction topology, a
// fixed launch configuration and an explicit log-softmax contract).
//
// The contract is the fused forward's: for every active token and every 128-entry vocabulary
// column, the column maximum and the sum of 2^(z log2 e - max) in log2 units, with z = logit
// / T applied once, followed by the fused forward's fixed-order merge.  The kernel is a pure
// HBM stream: one work-group of 4 waves per active token row keeps its row's column
// statistics in LDS (8 bytes per column) and merges them itself; each wave step reads
// 4 KiB of the row (four 16-byte non-temporal loads per lane: the row is read once), i.e. 16
// bf16 columns (16 lanes each) or 8 fp32 columns (32 lanes each), and the next step's loads
// are issued before the current step is reduced.  Every reduction is a fixed in-lane order
// followed by a fixed xor tree, so a row's results depend only on that row.
#include "common.hpp"
#include "kernels.hpp"

namespace rlk {

namespace {

template <bool kBF16>
__device__ __forceinline__ float logit_at(const uint8_t* row, int v) {
  if constexpr (kBF16) {
    const uint32_t b = reinterpret_cast<const uint16_t*>(row)[v];
    return __builtin_bit_cast(float, b << 16);
  } else {
    return reinterpret_cast<const float*>(row)[v];
  }
}

template <bool kBF16>
__global__ __launch_bounds__(256) void logits_logp_kernel(LogitsArgs a) {
  extern __shared__ float col_stats[];       // [2][J]: column max, then column sum
  constexpr int kPer = kBF16 ? 8 : 4;        // values per lane per 16-byte load
  constexpr int kGroup = 128 / kPer;         // lanes per column: 16 (bf16) or 32 (fp32)
  constexpr int kCols = 64 / kGroup;         // columns per wave step
  constexpr int kUnroll = 4;                 // wave steps per loop iteration
  const int Na = *a.n_active;
  const int i = blockIdx.x;
  if (i >= Na) return;
  const int t = a.idx[i];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const size_t esize = kBF16 ? 2 : 4;
  const uint8_t* row = static_cast<const uint8_t*>(a.logits) + (size_t)t * a.ld * esize;
  const float c2 = a.inv_t * kLog2e;
  const int J = (a.V + 127) / 128;
  float* cmax = col_stats;
  float* csum = col_stats + J;
  // the target logit, requested first so that its latency hides behind the row's stream
  float zy = 0.f;
  if (threadIdx.x == 0) {
    const int y = a.targets[t];
    zy = (y >= 0 && y < a.V) ? logit_at<kBF16>(row, y) * a.inv_t : NAN;
  }

  // 1. Column statistics.  Wave w takes column blocks w, w + 4, ... of kCols columns each;
  // the raw 16-byte loads of the next kUnroll blocks are in flight while the current ones are
  // reduced (two register buffers).
  constexpr int kStep = 4 * kCols * kUnroll;  // columns per work-group iteration
  auto load = [&](int jb, u32x4 (&raw)[kUnroll]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = jb + u * 4 * kCols + lane / kGroup;
      const int v0 = j * 128 + (lane % kGroup) * kPer;
      // v0 and ld are multiples of kPer, so the 16 bytes stay inside the row's ld entries
      raw[u] = (j < J && v0 < a.V) ? __builtin_nontemporal_load(
                                       reinterpret_cast<const u32x4*>(row + (size_t)v0 * esize))
                                   : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto reduce = [&](int jb, const u32x4 (&raw)[kUnroll]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = jb + u * 4 * kCols + lane / kGroup;
      const int v0 = j * 128 + (lane % kGroup) * kPer;
      float x[kPer];
      if constexpr (kBF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = __builtin_bit_cast(float, raw[u][e] << 16);
          x[2 * e + 1] = __builtin_bit_cast(float, raw[u][e] & 0xffff0000u);
        }
      } else {
        // cast the whole vector: a bit_cast of one vector element is lowered to element 0
        const f32x4 f = __builtin_bit_cast(f32x4, raw[u]);
        x[0] = f.x;
        x[1] = f.y;
        x[2] = f.z;
        x[3] = f.w;
      }
      // entries past the vocabulary (and lanes past the last column) count as -inf
#pragma unroll
      for (int e = 0; e < kPer; ++e)
        if (j >= J || v0 + e >= a.V) x[e] = -INFINITY;
      // column maximum on the raw logits (c2 > 0, rounding monotonic), in log2 units
      float m = x[0];
#pragma unroll
      for (int e = 1; e < kPer; ++e) m = fmaxf(m, x[e]);
#pragma unroll
      for (int o = kGroup / 2; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      const float mx = m * c2;
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < kPer; ++e) s += __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], c2, -mx));
#pragma unroll
      for (int o = kGroup / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o);
      if (lane % kGroup == 0 && j < J) {
        cmax[j] = mx;
        csum[j] = s;
      }
    }
  };
  u32x4 r0[kUnroll], r1[kUnroll];
  int jb = wave * kCols;
  load(jb, r0);
  while (jb < J) {
    load(jb + kStep, r1);
    reduce(jb, r0);
    jb += kStep;
    if (jb >= J) break;
    load(jb + kStep, r0);
    reduce(jb, r1);
    jb += kStep;
  }
  __syncthreads();

  // 2. The merge of the fused forward (fwd_merge_kernel), in the same association: slice
  // sl = 0..7 adds the columns sl, sl + 8, ... in ascending order, s = fma(sum_j, 2^(max_j -
  // M), s), and the 8 slice sums are added in one fixed tree.  The maximum M (exact in any
  // order) and the factors 2^(max_j - M) are formed by all threads; only the eight ordered
  // sums run serially, with their LDS reads batched ahead of the chain.
  __shared__ float red[8];
  float m = -INFINITY;
  for (int j = threadIdx.x; j < J; j += 256) m = fmaxf(m, cmax[j]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  for (int j = threadIdx.x; j < J; j += 256) cmax[j] = __builtin_amdgcn_exp2f(cmax[j] - M);
  __syncthreads();
  const int sl = threadIdx.x;
  if (sl < 8) {
    float s = 0.f;
    int j = sl;
    constexpr int kB = 8;  // columns per batch of LDS reads
    for (; j + 8 * (kB - 1) < J; j += 8 * kB) {
      float c[kB], e[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        c[u] = csum[j + 8 * u];
        e[u] = cmax[j + 8 * u];
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) s = __builtin_fmaf(c[u], e[u], s);
    }
    for (; j < J; j += 8) s = __builtin_fmaf(csum[j], cmax[j], s);
    red[sl] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const float S = ((red[0] + red[1]) + (red[2] + red[3])) + ((red[4] + red[5]) + (red[6] + red[7]));
    const float lse = (M + __builtin_amdgcn_logf(S)) * kLn2;
    a.logp[t] = zy - lse;
    if (a.lse) a.lse[t] = lse;
  }
}

}  // namespace

hipError_t launch_logits_logp(const LogitsArgs& a, bool bf16, hipStream_t stream) {
  const int grid = a.N > 0 ? a.N : 1;
  const size_t lds = 2 * sizeof(float) * (size_t)((a.V + 127) / 128);
  if (bf16)
    hipLaunchKernelGGL(logits_logp_kernel<true>, dim3(grid), dim3(256), lds, stream, a);
  else
    hipLaunchKernelGGL(logits_logp_kernel<false>, dim3(grid), dim3(256), lds, stream, a);
  return hipGetLastError();
}

}  // namespace rlk
