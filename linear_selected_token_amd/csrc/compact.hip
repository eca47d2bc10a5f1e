// Active-row compaction: the positions of the active tokens in ascending order.
//
// Only active response tokens are scored (RL-Kernel integration roadmap for vime,
// "Consistency Contract": prompt and padding tokens are excluded from every aggregate).
// Compacting them first means inactive rows never enter a product, so their contents
// cannot reach any result, and the tile grid covers only active rows.
//
// One work-group of 1024 threads walks the mask in blocks of 4096 tokens; each block is an
// exclusive scan (wave64 shuffles, then the 16 wave totals in order), so the output order
// is the token order and the result is deterministic.
#include "common.hpp"
#include "kernels.hpp"

namespace rlk {

namespace {

__global__ __launch_bounds__(1024) void compact_kernel(CompactArgs a) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int base = 0;
  for (int t0 = 0; t0 < a.N; t0 += 4096) {
    int f[4];
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t = t0 + 4 * tid + k;
      f[k] = 0;
      if (t < a.N) {
        f[k] = a.mask[t] != 0;
        if (a.target_logit) a.target_logit[t] = __builtin_nanf("");
        if (!f[k]) {
          if (a.logp) a.logp[t] = 0.f;
          if (a.lse) a.lse[t] = 0.f;
          if (a.entropy) a.entropy[t] = 0.f;
          if (a.extra) a.extra[t] = 0.f;
        }
      }
      cnt += f[k];
    }
    int x = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int wpre = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int v = wsum[w];
      wpre += (w < wave) ? v : 0;
      total += v;
    }
    int o = base + wpre + x - cnt;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (f[k]) a.idx[o++] = t0 + 4 * tid + k;
    base += total;
    __syncthreads();
  }
  if (tid == 0) *a.n_active = base;
}

}  // namespace

hipError_t launch_compact(const CompactArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rlk
