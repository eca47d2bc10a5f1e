// Active-row compaction: the positions of the active tokens in ascending order.
//
// Only active response tokens are scored (RL-Kernel integration roadmap for vime,
// "Consistency Contract": prompt and padding tokens are excluded from every aggregate).
// Compacting them first means inactive rows never enter a product, so their contents
// cannot reach any result, and the tile grid covers only active rows.
//
// One work-group of 1024 threads walks the mask in blocks of 4096 tokens; each block is an
// exclusive scan (wave64 shuffles, then the 16 wave totals in order), so the output order
// is the token order and the result is deterministic.  On request it also cuts the compacted
// indices into the backward's token blocks (fixed blocks of the capacity, or the active tokens
// cut into equal blocks of at most the capacity), so later kernels read their block's count on
// the device; select_block copies one balanced block's indices for the kernels that follow.
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
  if (tid < a.nblk) {
    const int cap = a.block_cap;
    if (a.block_count) {
      const int n = base - tid * cap;
      a.block_count[tid] = n < 0 ? 0 : (n < cap ? n : cap);
    }
    if (a.block_desc) {
      // ceil(Na / cap) blocks of one size (a multiple of 256, at most cap), the last shorter
      const int nb = (base + cap - 1) / cap;
      const int size = nb > 0 ? ((base + nb - 1) / nb + 255) / 256 * 256 : 0;
      const int first = tid < nb ? tid * size : 0;
      const int n = tid < nb ? base - first : 0;
      a.block_desc[2 * tid] = n < 0 ? 0 : (n < size ? n : size);
      a.block_desc[2 * tid + 1] = first < base ? first : 0;
    }
  }
}

__global__ __launch_bounds__(256) void select_block_kernel(const int32_t* idx, const int32_t* desc,
                                                           int b, int32_t* bidx, int32_t* bn) {
  const int n = desc[2 * b];
  const int first = desc[2 * b + 1];
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) bidx[i] = idx[first + i];
  if (blockIdx.x == 0 && threadIdx.x == 0) *bn = n;
}

}  // namespace

hipError_t launch_compact(const CompactArgs& a, hipStream_t stream) {
  if (a.nblk > 1024 || (a.nblk > 0 && (a.block_cap <= 0 || a.block_cap % 256 != 0)))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_select_block(const int32_t* idx, const int32_t* desc, int b, int cap,
                               int32_t* bidx, int32_t* bn, hipStream_t stream) {
  const int grid = (cap + 255) / 256;
  hipLaunchKernelGGL(select_block_kernel, dim3(grid), dim3(256), 0, stream, idx, desc, b, bidx, bn);
  return hipGetLastError();
}

}  // namespace rlk
