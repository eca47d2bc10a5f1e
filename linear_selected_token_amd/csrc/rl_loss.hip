// Loss fragments and diagnostics that consume the selected-token log-prob (RL-Kernel
// integration roadmap for vime, "RL Loss Operators: ratio_kl, GRPO/PPO/DPO Loss Fragments":
// optional fused ratio / KL fragments whose contract fixes mask handling, dtype and the
// reduction order; and the minimum dlogp diagnostics of its "Consistency Contract").
//
// ratio_kl_loss: one thread per 4 tokens, fp32 per-token arithmetic, so each token's loss,
// gradient and ratio depend only on that token's inputs.  The masked sums are fp64: every
// work-group of kLossBlock tokens reduces its tokens in one fixed tree, and one work-group
// adds the group partials in a fixed order (no atomics), so the sums are deterministic for
// a given N.
//
// dlogp_diagnostics: dlogp = a - b is formed in fp64 (exact for two fp32 inputs of similar
// magnitude), the sums in fp64 as above; the percentiles of |dlogp| come from an exact
// radix select over the fp64 bit patterns (non-negative doubles order like their bits):
// eight passes of one byte each, most significant first, each counting with integer
// atomics (exact, so order-independent) the keys that match the prefix selected so far
// (ranks with equal prefixes share one count), then one work-group scans the counts and
// stores each rank's extended prefix and remaining rank for the next pass.
#include <math.h>

#include "common.hpp"
#include "aux_kernels.hpp"
#include "kernels.hpp"

namespace rlk {

namespace {

constexpr int kRThreads = 256;

// Fixed-order tree over kRThreads values of 4 doubles in LDS; the result lands in v[0].
__device__ __forceinline__ void tree4(double (*v)[4]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int s = kRThreads / 2; s >= 1; s >>= 1) {
    __syncthreads();
    if (tid < s)
#pragma unroll
      for (int k = 0; k < 4; ++k) v[tid][k] = v[tid][k] + v[tid + s][k];
  }
  __syncthreads();
}

__global__ __launch_bounds__(kRThreads) void loss_kernel(LossArgs a) {
  __shared__ double red[kRThreads][4];
  const int tid = threadIdx.x;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int k = 0; k < kLossBlock / kRThreads; ++k) {
    const int t = blockIdx.x * kLossBlock + k * kRThreads + tid;
    if (t >= a.N) break;
    float loss = 0.f, badv = 0.f, ratio = 0.f;
    if (a.mask[t]) {
      const float lp = a.logp[t];
      const float A = a.adv[t];
      const float r = expf(lp - a.old_logp[t]);
      const float rc = fminf(fmaxf(r, 1.f - a.eps_lo), 1.f + a.eps_hi);
      const float un = -A * r;
      const float cl = -A * rc;
      const bool clipped = cl > un;
      float pg = clipped ? cl : un;
      float g = clipped ? 0.f : -A * r;  // dL/dlogp of the policy-gradient term
      float kl = 0.f;
      if (a.ref_logp) {
        const float d = a.ref_logp[t] - lp;
        const float e = expf(d);
        kl = (e - 1.f) - d;
        g = __builtin_fmaf(a.beta, 1.f - e, g);
        pg = __builtin_fmaf(a.beta, kl, pg);
      }
      loss = a.scale * pg;
      badv = -a.scale * g;
      ratio = r;
      acc[0] += (double)loss;
      acc[1] += clipped ? 1.0 : 0.0;
      acc[2] += (double)kl;
      acc[3] += 1.0;
    }
    a.loss[t] = loss;
    a.bwd_adv[t] = badv;
    if (a.ratio) a.ratio[t] = ratio;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) red[tid][k] = acc[k];
  tree4(red);
  if (tid < 4) a.part[(size_t)blockIdx.x * 4 + tid] = red[0][tid];
}

// One work-group: thread s adds partials s, s + 256, ... in ascending order, then one tree.
__global__ __launch_bounds__(kRThreads) void sum4_kernel(const double* part, int nblk,
                                                          double* out) {
  __shared__ double red[kRThreads][4];
  const int tid = threadIdx.x;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int j = tid; j < nblk; j += kRThreads)
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] += part[(size_t)j * 4 + k];
#pragma unroll
  for (int k = 0; k < 4; ++k) red[tid][k] = acc[k];
  tree4(red);
  if (tid < 4) out[tid] = red[0][tid];
}

// ---------------------------------------------------------------- diagnostics

__device__ __forceinline__ uint64_t key_of(double x) { return __builtin_bit_cast(uint64_t, x); }

// The 6 ranks whose order statistics the three percentiles need: floor and ceil of
// q (n - 1) / 100 for q = 50, 90, 99.
__device__ __forceinline__ void percentile_ranks(int n, int64_t* rk, double* frac) {
  const int qs[3] = {50, 90, 99};
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const double pos = (double)((int64_t)qs[i] * (n - 1)) / 100.0;
    const int64_t lo = (int64_t)floor(pos);
    rk[2 * i] = lo;
    rk[2 * i + 1] = lo + 1 < n ? lo + 1 : n - 1;
    frac[i] = pos - (double)lo;
  }
}

// Ranks whose selected prefixes are equal share one histogram: the first such rank owns it.
__device__ __forceinline__ int prefix_owner(const uint64_t* pf, int r) {
  int o = r;
  for (int q = r - 1; q >= 0; --q)
    if (pf[q] == pf[r]) o = q;
  return o;
}

// keys, per-block sums (|d|, exp(d), clipped, exp(d) - 1 - d) and the block's largest key
// with its first token.
__global__ __launch_bounds__(kRThreads) void diag_keys_kernel(DiagArgs a) {
  __shared__ double red[kRThreads][4];
  __shared__ uint64_t mk[kRThreads];
  __shared__ int mt[kRThreads];
  const int tid = threadIdx.x;
  const int Na = *a.n_active;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  uint64_t best = 0;
  int best_t = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < kLossBlock / kRThreads; ++k) {
    const int i = blockIdx.x * kLossBlock + k * kRThreads + tid;
    if (i >= Na) break;
    const int t = a.idx[i];
    const double d = (double)a.a[t] - (double)a.b[t];
    const double ad = fabs(d);
    const uint64_t key = key_of(ad);
    a.keys[i] = key;
    const double e = exp(d);
    acc[0] += ad;
    acc[1] += e;
    acc[2] += fabs(e - 1.0) > (double)a.eps ? 1.0 : 0.0;
    acc[3] += (e - 1.0) - d;
    // tokens are visited in ascending order, so a strictly larger key is needed to move
    if (key > best || best_t == 0x7fffffff) {
      best = key;
      best_t = t;
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) red[tid][k] = acc[k];
  mk[tid] = best;
  mt[tid] = best_t;
  tree4(red);
  // fixed tree for the maximum; ties go to the smaller token index
#pragma unroll
  for (int s = kRThreads / 2; s >= 1; s >>= 1) {
    if (tid < s) {
      const uint64_t k2 = mk[tid + s];
      const int t2 = mt[tid + s];
      if (t2 != 0x7fffffff && (mt[tid] == 0x7fffffff || k2 > mk[tid] ||
                               (k2 == mk[tid] && t2 < mt[tid]))) {
        mk[tid] = k2;
        mt[tid] = t2;
      }
    }
    __syncthreads();
  }
  if (tid < 4) a.part[(size_t)blockIdx.x * 4 + tid] = red[0][tid];
  if (tid == 0) {
    a.pmax[blockIdx.x] = mk[0];
    a.ptok[blockIdx.x] = mt[0];
  }
}

// Clears the histograms and starts the selection: empty prefixes, the ranks themselves.
__global__ __launch_bounds__(kRThreads) void diag_zero_kernel(DiagArgs a) {
  const int n = 8 * kDiagRanks * 256;
  for (int e = blockIdx.x * kRThreads + threadIdx.x; e < n; e += gridDim.x * kRThreads)
    a.hist[e] = 0;
  if (blockIdx.x == 0 && threadIdx.x < kDiagRanks) {
    const int Na = *a.n_active;
    int64_t rk[kDiagRanks];
    double frac[3];
    percentile_ranks(Na > 0 ? Na : 1, rk, frac);
    a.sel_prefix[threadIdx.x] = 0;
    a.sel_rank[threadIdx.x] = rk[threadIdx.x];
  }
}

// Pass p: per rank, count the keys that match the selected prefix, by their byte p.
__global__ __launch_bounds__(kRThreads) void diag_hist_kernel(DiagArgs a, int pass) {
  __shared__ int cnt[kDiagRanks][256];
  __shared__ uint64_t pf[kDiagRanks];
  __shared__ int own[kDiagRanks];
  const int tid = threadIdx.x;
  const int Na = *a.n_active;
  for (int e = tid; e < kDiagRanks * 256; e += kRThreads) (&cnt[0][0])[e] = 0;
  if (tid < kDiagRanks) pf[tid] = a.sel_prefix[tid];
  __syncthreads();
  if (tid < kDiagRanks) own[tid] = prefix_owner(pf, tid);
  __syncthreads();
  const int shift = 56 - 8 * pass;
  const uint64_t hi_mask = pass == 0 ? 0 : (~0ull << (shift + 8));
  for (int i = blockIdx.x * kRThreads + tid; i < Na; i += gridDim.x * kRThreads) {
    const uint64_t key = a.keys[i];
    const int d = (int)((key >> shift) & 255);
#pragma unroll
    for (int r = 0; r < kDiagRanks; ++r)
      if (own[r] == r && (key & hi_mask) == pf[r]) atomicAdd(&cnt[r][d], 1);
  }
  __syncthreads();
  int* h = a.hist + (size_t)pass * kDiagRanks * 256;
  for (int e = tid; e < kDiagRanks * 256; e += kRThreads) {
    const int c = (&cnt[0][0])[e];
    if (c) atomicAdd(h + e, c);
  }
}

// One work-group, after pass `pass`: for each rank, the byte of that pass under which its order
// statistic lies (an inclusive scan of the owner's 256 counts) and the rank left inside it.
__global__ __launch_bounds__(256) void diag_select_kernel(DiagArgs a, int pass) {
  __shared__ int cum[256];
  __shared__ uint64_t pf[kDiagRanks];
  const int tid = threadIdx.x;
  if (tid < kDiagRanks) pf[tid] = a.sel_prefix[tid];
  __syncthreads();
  for (int r = 0; r < kDiagRanks; ++r) {
    const int o = prefix_owner(pf, r);
    const int64_t k = a.sel_rank[r];
    cum[tid] = a.hist[((size_t)pass * kDiagRanks + o) * 256 + tid];
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int v = tid >= off ? cum[tid - off] : 0;
      __syncthreads();
      cum[tid] += v;
      __syncthreads();
    }
    const int64_t below = tid > 0 ? cum[tid - 1] : 0;
    if (k >= below && k < (int64_t)cum[tid]) {  // exactly one byte holds rank k
      a.sel_prefix[r] = pf[r] | ((uint64_t)tid << (56 - 8 * pass));
      a.sel_rank[r] = k - below;
    }
    __syncthreads();
  }
}

// One work-group: the sums, the maximum and the percentiles.
__global__ __launch_bounds__(kRThreads) void diag_final_kernel(DiagArgs a, int nblk) {
  __shared__ double red[kRThreads][4];
  __shared__ uint64_t mk[kRThreads];
  __shared__ int mt[kRThreads];
  __shared__ double ostat[kDiagRanks];
  const int tid = threadIdx.x;
  const int Na = *a.n_active;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  uint64_t best = 0;
  int best_t = 0x7fffffff;
  for (int j = tid; j < nblk; j += kRThreads) {
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] += a.part[(size_t)j * 4 + k];
    const int t = a.ptok[j];
    if (t != 0x7fffffff && (best_t == 0x7fffffff || a.pmax[j] > best ||
                            (a.pmax[j] == best && t < best_t))) {
      best = a.pmax[j];
      best_t = t;
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) red[tid][k] = acc[k];
  mk[tid] = best;
  mt[tid] = best_t;
  tree4(red);
#pragma unroll
  for (int s = kRThreads / 2; s >= 1; s >>= 1) {
    if (tid < s) {
      const uint64_t k2 = mk[tid + s];
      const int t2 = mt[tid + s];
      if (t2 != 0x7fffffff && (mt[tid] == 0x7fffffff || k2 > mk[tid] ||
                               (k2 == mk[tid] && t2 < mt[tid]))) {
        mk[tid] = k2;
        mt[tid] = t2;
      }
    }
    __syncthreads();
  }
  int64_t rk[kDiagRanks];
  double frac[3];
  percentile_ranks(Na > 0 ? Na : 1, rk, frac);
  if (tid < kDiagRanks) ostat[tid] = __builtin_bit_cast(double, a.sel_prefix[tid]);
  __syncthreads();
  if (tid == 0) {
    double* o = a.out;
    if (Na == 0) {
      for (int k = 0; k < kDiagOut; ++k) o[k] = 0.0;
      *a.worst = -1;
      return;
    }
    const double n = (double)Na;
    o[0] = n;
    o[1] = red[0][0] / n;
    o[2] = __builtin_bit_cast(double, mk[0]);
    for (int i = 0; i < 3; ++i) {
      const double lo = ostat[2 * i], hi = ostat[2 * i + 1];
      o[3 + i] = lo + frac[i] * (hi - lo);
    }
    o[6] = red[0][1] / n;
    o[7] = red[0][2] / n;
    o[8] = red[0][3] / n;
    *a.worst = mt[0];
  }
}

}  // namespace

hipError_t launch_ratio_kl_loss(const LossArgs& a, double* sums, hipStream_t stream) {
  const int nblk = (a.N + kLossBlock - 1) / kLossBlock;
  if (nblk > 0)
    hipLaunchKernelGGL(loss_kernel, dim3(nblk), dim3(kRThreads), 0, stream, a);
  if (sums) hipLaunchKernelGGL(sum4_kernel, dim3(1), dim3(kRThreads), 0, stream, a.part, nblk, sums);
  return hipGetLastError();
}

hipError_t launch_dlogp_diagnostics(const DiagArgs& a, hipStream_t stream) {
  const int nblk = (a.N + kLossBlock - 1) / kLossBlock;  // enough for every active token
  const int nb = nblk > 0 ? nblk : 1;
  hipLaunchKernelGGL(diag_keys_kernel, dim3(nb), dim3(kRThreads), 0, stream, a);
  hipLaunchKernelGGL(diag_zero_kernel, dim3(8), dim3(kRThreads), 0, stream, a);
  const int hb = nb < 1024 ? nb : 1024;
  for (int p = 0; p < 8; ++p) {
    hipLaunchKernelGGL(diag_hist_kernel, dim3(hb), dim3(kRThreads), 0, stream, a, p);
    hipLaunchKernelGGL(diag_select_kernel, dim3(1), dim3(256), 0, stream, a, p);
  }
  hipLaunchKernelGGL(diag_final_kernel, dim3(1), dim3(kRThreads), 0, stream, a, nb);
  return hipGetLastError();
}

}  // namespace rlk
