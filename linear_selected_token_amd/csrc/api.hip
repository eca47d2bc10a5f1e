// C ABI of the library: argument checks, workspace carving and kernel launches on the
// caller's stream.  The operation and its contract are described in include/rlk.h.
#include <hip/hip_runtime.h>

#include <math.h>

#include <atomic>
#include <cstdio>
#include <string>

#include "aux_kernels.hpp"
#include "kernels.hpp"
#include "rlk.h"
#include "validate.hpp"

static_assert(rlk::kBwdChunkEntries == rlk::kBwdChunk && rlk::kBwdDhPieces == rlk::kDhPieces,
              "host workspace layout and device chunking agree");
static_assert(rlk::kKlScratchBytes == (size_t)rlk::kKlSlots * rlk::kKlSlotFloats * 4,
              "the KL scratch size the host carves is the one the tile kernel addresses");

namespace rlk {
namespace {

// Compute units of each device, read once (the only state the library keeps).
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

hipError_t persistent_grid(int* grid) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int cus = (dev >= 0 && dev < kMaxDevices) ? g_cus[dev].load(std::memory_order_relaxed) : 0;
  if (cus <= 0) {
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) g_cus[dev].store(cus, std::memory_order_relaxed);
  }
  // one work-group per CU; a multiple of 8 keeps the XCD-aware tile order exact
  *grid = cus >= 8 ? (cus & ~7) : cus;
  return hipSuccess;
}

// Scratch of rlk_linear_logp_fwd_noalloc: the forward's workspace in a static device array, so
// that the call needs no allocation.  Each device holds its own copy (at its own address) from
// the time the library's code is loaded on it until the process ends.  In host code the name
// `scratch` is a host-side stand-in, never a device address: kernels get the address that
// hipGetSymbolAddress returns for the current device, read once per device.
constexpr size_t kNoAllocScratchBytes = RLK_NOALLOC_SCRATCH_BYTES;
static_assert(kNoAllocScratchBytes % 256 == 0, "the forward's workspace is carved in 256-byte units");
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
std::atomic<uintptr_t> g_scratch[kMaxDevices];

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  uintptr_t p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == 0) {
    void* q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (q == nullptr || reinterpret_cast<uintptr_t>(q) % 256 != 0) return hipErrorInvalidSymbol;
    p = reinterpret_cast<uintptr_t>(q);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = reinterpret_cast<void*>(p);
  return hipSuccess;
}

inline rlk_status_t dev_status(hipError_t e) { return e == hipSuccess ? RLK_SUCCESS : RLK_ERROR_DEVICE; }

template <class T>
T* carve(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

const char* build_info_string() {
  // written once (thread-safe static initialisation), from the build's constants
  static const std::string s = [] {
    char buf[768];
    snprintf(buf, sizeof buf,
             "rlk linear_logp | arch gfx950 | compiler " __clang_version__
             " | tile 256x256, K stage 128 B, 8 wave64 x 128x64, mfma 32x32x16 bf16 / 32x32x2 f32"
             " | vocab partial 128 | merge 8 strided slices + fixed tree"
             " | bwd chunk %d, dh split at %d"
             " | fused fwd+bwd: one dh/dW launch per token block, dh in the two halves of V"
             " (each rounded up to 64)"
             " | bwd token blocks: equal blocks of at most the largest multiple of 256 tokens whose"
             " buffers (%zu + %zu H bytes per token) fit %zu bytes",
             kBwdChunk, kDhSplitK, bwd_bytes_per_token(0), (bwd_bytes_per_token(1 << 10) - bwd_bytes_per_token(0)) >> 10,
             kBwdBlockBudget);
    return std::string(buf);
  }();
  return s.c_str();
}

// The backward behind rlk_linear_logp_bwd and rlk_linear_logp_bwd_entropy (ent_coef and
// entropy null for the former).
rlk_status_t run_bwd(const void* h, const void* W, const int32_t* targets, const uint8_t* mask,
                     int64_t N, int64_t H, int64_t V, int dtype, float temperature,
                     const float* adv, const float* lse, const float* ent_coef,
                     const float* entropy, float* dh, float* dW, void* workspace,
                     size_t workspace_bytes, void* stream) {
  rlk_status_t s = check_bwd(h, W, targets, mask, N, H, V, dtype, temperature, adv, lse, dh, dW,
                             workspace, workspace_bytes);
  if (s != RLK_SUCCESS) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (N == 0) {
    // nothing to differentiate: dL/dW = 0 (a fill kernel, not a memset node)
    return dev_status(launch_zero(dW, (size_t)V * (size_t)H, st));
  }
  int grid = 0;
  if (persistent_grid(&grid) != hipSuccess) return RLK_ERROR_DEVICE;
  const BwdLayout L = bwd_layout(N, H);
  BwdArgs a{};
  a.h = h;
  a.W = W;
  a.targets = targets;
  a.adv = adv;
  a.lse = lse;
  a.ent_coef = ent_coef;
  a.entropy = entropy;
  int32_t* idx = carve<int32_t>(workspace, L.idx);
  int32_t* na = carve<int32_t>(workspace, L.n_active);
  int32_t* desc = carve<int32_t>(workspace, L.block_desc);
  int32_t* bidx = carve<int32_t>(workspace, L.bidx);
  int32_t* bn = carve<int32_t>(workspace, L.bn);
  a.N = (int)N;
  a.H = (int)H;
  a.V = (int)V;
  a.Npad = (int)bwd_npad(N, H);
  a.inv_t = (float)(1.0 / (double)temperature);
  a.dh = dh;
  a.dW = dW;
  a.hT = carve<uint16_t>(workspace, L.hT);
  a.Gv = carve<uint16_t>(workspace, L.Gv);
  a.dhp[0] = nullptr;  // piece 0 accumulates in dh's rows
  for (int q = 1; q < kDhPieces; ++q) a.dhp[q] = carve<float>(workspace, L.dhp[q]);
  a.sched = carve<int>(workspace, L.sched);
  a.idx = bidx;
  a.n_active = bn;
  const int nblk = bwd_blocks(N, H);
  CompactArgs c{mask, idx, na, nullptr, nullptr, nullptr, (int)N};
  c.block_desc = desc;
  c.nblk = nblk;
  c.block_cap = (int)bwd_token_cap(H);
  hipError_t e = launch_compact(c, st);
  if (e != hipSuccess) return RLK_ERROR_DEVICE;
  e = launch_zero(dh, (size_t)N * (size_t)H, st);  // inactive rows stay 0
  if (e != hipSuccess) return RLK_ERROR_DEVICE;
  const int nchunks = (int)((V + kBwdChunk - 1) / kBwdChunk);
  for (int b = 0; b < nblk; ++b) {
    // the block's compacted indices and count, copied for the kernels that follow
    e = launch_select_block(idx, desc, b, a.Npad, bidx, bn, st);
    if (e != hipSuccess) return RLK_ERROR_DEVICE;
    e = launch_bwd_transpose(a, st);
    if (e != hipSuccess) return RLK_ERROR_DEVICE;
    for (int c0 = 0; c0 < nchunks; ++c0) {
      e = launch_bwd_chunk(a, c0, grid, b > 0, st);
      if (e != hipSuccess) return RLK_ERROR_DEVICE;
    }
    e = launch_bwd_finish(a, st);
    if (e != hipSuccess) return RLK_ERROR_DEVICE;
  }
  return RLK_SUCCESS;
}


// The fused forward + backward behind rlk_linear_logp_fwd_bwd.  Per token block: the forward
// tile kernel with the statistics and the 16-bit code of every entry's d stored, the merge (logp and lse
// of the block's tokens, the same bits as rlk_linear_logp_fwd), d turned into dL/dz in place,
// then the backward's dL/dh and dL/dW GEMMs over the vocabulary chunks, reading dL/dz from the
// block's rows.  No GEMM is run twice.
//
// With `loss` (rlk_linear_ppo_fwd_bwd) the upstream gradient comes from the clipped policy-
// gradient loss on the fresh logp: after each block's merge the loss fragment runs over every
// token (the block's tokens now have their final logp; the others are recomputed by their own
// block) and its -dloss/dlogp takes the place of adv in the dz pass; a last run after the final
// block gives every token's loss and ratio and the fixed-order sums.
struct FusedLoss {
  LossArgs args;  // logp, mask and N filled in here; part: the loss fragment's partial sums
  double* sums;   // may be null
};

// With `ent_coef` (rlk_linear_logp_fwd_bwd_entropy) the forward also keeps the entropy
// statistic, the merge writes each token's entropy, and the dz pass adds the entropy bonus's
// term.
rlk_status_t run_fused(const void* h, const void* W, const int32_t* targets, const uint8_t* mask,
                       int64_t N, int64_t H, int64_t V, int dtype, float temperature,
                       const float* adv, float* logp, float* lse, float* dh, float* dW,
                       void* workspace, size_t workspace_bytes, void* stream,
                       FusedLoss* loss = nullptr, const float* ent_coef = nullptr,
                       float* entropy = nullptr) {
  const bool ent = ent_coef != nullptr;
  rlk_status_t s = check_fused(h, W, targets, mask, N, H, V, dtype, temperature, adv, logp, lse,
                               dh, dW, workspace, workspace_bytes, ent);
  if (s != RLK_SUCCESS) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (loss) {
    loss->args.logp = logp;
    loss->args.mask = mask;
    loss->args.N = (int)N;
    adv = loss->args.bwd_adv;  // the dz pass reads -dloss/dlogp
  }
  if (N == 0) {
    if (loss && launch_ratio_kl_loss(loss->args, loss->sums, st) != hipSuccess)
      return RLK_ERROR_DEVICE;
    return dev_status(launch_zero(dW, (size_t)V * (size_t)H, st));
  }
  int grid = 0;
  if (persistent_grid(&grid) != hipSuccess) return RLK_ERROR_DEVICE;
  // the largest block capacity the given workspace holds (check_fused made sure one does)
  const int64_t cap64 = fused_cap_for_workspace(N, H, V, workspace_bytes, ent);
  const FusedLayout L = fused_layout_cap(N, H, V, cap64, ent);
  const int np = (int)fused_npad_cap(N, cap64);
  const int cap = (int)cap64;
  const int nblk = fused_blocks_cap(N, cap64);
  const float inv_t = (float)(1.0 / (double)temperature);
  int32_t* idx = carve<int32_t>(workspace, L.idx);
  int32_t* na = carve<int32_t>(workspace, L.n_active);
  int32_t* desc = carve<int32_t>(workspace, L.block_desc);
  int32_t* bidx = carve<int32_t>(workspace, L.bidx);
  int32_t* bn = carve<int32_t>(workspace, L.bn);
  float* zy = carve<float>(workspace, L.target_logit);
  float* pm = carve<float>(workspace, L.part_max);
  float* ps = carve<float>(workspace, L.part_sum);
  uint16_t* X = carve<uint16_t>(workspace, L.X);

  FwdTileArgs f{h, W, targets, bidx, bn, (int)N, (int)H, (int)V, inv_t, pm, ps, zy, 0};
  f.pstride = np;
  f.dbuf = X;
  f.d_pitch = (int)fused_pitch(V);
  MergeArgs m{pm, ps, zy, bidx, bn, np, (int)V, logp, lse};  // N = np: the partials' stride
  DzArgs z{X, (int)fused_pitch(V), pm, np, bidx, bn, targets, adv, lse, (int)V, inv_t};
  if (ent) {
    float* pw = carve<float>(workspace, L.part_w);
    f.part_w = pw;
    m.part_w = pw;
    m.entropy = entropy;
    z.ent_coef = ent_coef;
    z.entropy = entropy;
  }
  BwdArgs a{};
  a.h = h;
  a.W = W;
  a.targets = targets;
  a.adv = adv;
  a.lse = lse;
  a.idx = bidx;
  a.n_active = bn;
  a.N = (int)N;
  a.H = (int)H;
  a.V = (int)V;
  a.Npad = np;
  a.inv_t = inv_t;
  a.dh = dh;
  a.dW = dW;
  a.hT = carve<uint16_t>(workspace, L.hT);
  a.Gv = X;
  a.gv_pitch = (int)fused_pitch(V);
  a.gv_full = true;
  a.dhp[0] = nullptr;  // piece 0 accumulates in dh's rows
  for (int q = 1; q < kDhPieces; ++q) a.dhp[q] = carve<float>(workspace, L.dhp[q]);
  a.sched = carve<int>(workspace, L.sched);

  // logp, lse (and the entropy) are zeroed at every token (the merge writes the active ones)
  CompactArgs c{mask, idx, na, nullptr, logp, lse, (int)N, entropy};
  c.block_desc = desc;
  c.nblk = nblk;
  c.block_cap = cap;
  hipError_t e = launch_compact(c, st);
  if (e != hipSuccess) return RLK_ERROR_DEVICE;
  e = launch_zero(dh, (size_t)N * (size_t)H, st);  // inactive rows stay 0
  if (e != hipSuccess) return RLK_ERROR_DEVICE;
  for (int b = 0; b < nblk; ++b) {
    e = launch_select_block(idx, desc, b, np, bidx, bn, st);
    if (e != hipSuccess) return RLK_ERROR_DEVICE;
    // a target outside [0, V) is never captured: its logp stays NaN, as in the forward
    e = launch_fill(zy, (size_t)np, NAN, st);
    if (e != hipSuccess) return RLK_ERROR_DEVICE;
    e = launch_fwd_tiles(f, true, grid, st, ent ? kFwdStoreDEnt : kFwdStoreD);
    if (e != hipSuccess) return RLK_ERROR_DEVICE;
    e = launch_fwd_merge(m, st);
    if (e != hipSuccess) return RLK_ERROR_DEVICE;
    if (loss) {
      e = launch_ratio_kl_loss(loss->args, nullptr, st);
      if (e != hipSuccess) return RLK_ERROR_DEVICE;
    }
    e = launch_dz_from_d(z, st);
    if (e != hipSuccess) return RLK_ERROR_DEVICE;
    e = launch_bwd_transpose(a, st);
    if (e != hipSuccess) return RLK_ERROR_DEVICE;
    // dL/dz of every column is in place: both GEMMs of the whole vocabulary in one launch
    e = launch_bwd_whole_gemms(a, grid, b > 0, st);
    if (e != hipSuccess) return RLK_ERROR_DEVICE;
    e = launch_bwd_finish_whole(a, st);
    if (e != hipSuccess) return RLK_ERROR_DEVICE;
  }
  if (loss) return dev_status(launch_ratio_kl_loss(loss->args, loss->sums, st));
  return RLK_SUCCESS;
}

}  // namespace
}  // namespace rlk

using namespace rlk;

extern "C" {

const char* rlk_status_string(int status) {
  switch (status) {
    case RLK_SUCCESS: return "RLK_SUCCESS";
    case RLK_ERROR_INVALID_VALUE: return "RLK_ERROR_INVALID_VALUE: invalid argument";
    case RLK_ERROR_UNSUPPORTED: return "RLK_ERROR_UNSUPPORTED: unsupported dtype, shape or alignment";
    case RLK_ERROR_WORKSPACE: return "RLK_ERROR_WORKSPACE: workspace too small";
    case RLK_ERROR_DEVICE: return "RLK_ERROR_DEVICE: HIP launch or runtime failure";
    default: return "unknown rlk status";
  }
}

const char* rlk_build_info(void) { return build_info_string(); }

int64_t rlk_num_vocab_partials(int64_t V) { return num_partials(V); }

rlk_status_t rlk_linear_logp_fwd_workspace_size(int64_t N, int64_t H, int64_t V, int dtype,
                                                size_t* bytes) {
  if (!bytes) return RLK_ERROR_INVALID_VALUE;
  rlk_status_t s = check_shape(N, H, V, dtype);
  if (s != RLK_SUCCESS) return s;
  *bytes = fwd_layout(N, V).total;
  return RLK_SUCCESS;
}

rlk_status_t rlk_linear_logp_fwd_entropy_workspace_size(int64_t N, int64_t H, int64_t V,
                                                        int dtype, size_t* bytes) {
  if (!bytes) return RLK_ERROR_INVALID_VALUE;
  rlk_status_t s = check_shape(N, H, V, dtype);
  if (s != RLK_SUCCESS) return s;
  *bytes = fwd_layout(N, V, true).total;
  return RLK_SUCCESS;
}

rlk_status_t rlk_linear_logp_bwd_workspace_size(int64_t N, int64_t H, int64_t V, int dtype,
                                                size_t* bytes) {
  if (!bytes) return RLK_ERROR_INVALID_VALUE;
  rlk_status_t s = check_shape(N, H, V, dtype);
  if (s != RLK_SUCCESS) return s;
  if (dtype != RLK_BF16 || H % 256 != 0) return RLK_ERROR_UNSUPPORTED;
  *bytes = bwd_layout(N, H).total;
  return RLK_SUCCESS;
}

rlk_status_t rlk_compact_active(const uint8_t* mask, int64_t N, int32_t* idx, int32_t* n_active,
                                float* target_logit, float* logp, float* lse, void* stream) {
  if (N < 0) return RLK_ERROR_INVALID_VALUE;
  if (N > kMaxTokens) return RLK_ERROR_UNSUPPORTED;
  if (!n_active) return RLK_ERROR_INVALID_VALUE;
  if (N > 0 && (!mask || !idx)) return RLK_ERROR_INVALID_VALUE;
  if (!aligned(idx, 4) || !aligned(n_active, 4) || (target_logit && !aligned(target_logit, 4)) ||
      (logp && !aligned(logp, 4)) || (lse && !aligned(lse, 4)))
    return RLK_ERROR_UNSUPPORTED;
  CompactArgs a{mask, idx, n_active, target_logit, logp, lse, (int)N};
  return dev_status(launch_compact(a, static_cast<hipStream_t>(stream)));
}

rlk_status_t rlk_linear_logp_partials_shard(const void* h, const void* W, const int32_t* targets,
                                            const int32_t* idx, const int32_t* n_active,
                                            int64_t N, int64_t H, int64_t V, int64_t vocab_start,
                                            int64_t V_global, int dtype, float temperature,
                                            float* part_max, float* part_sum,
                                            float* target_logit, void* stream) {
  rlk_status_t s = check_shape(N, H, V, dtype);
  if (s != RLK_SUCCESS) return s;
  s = check_temperature(temperature);
  if (s != RLK_SUCCESS) return s;
  s = check_shard(V, vocab_start, V_global);
  if (s != RLK_SUCCESS) return s;
  if (N == 0) return RLK_SUCCESS;
  if (!h || !W || !targets || !idx || !n_active || !part_max || !part_sum || !target_logit)
    return RLK_ERROR_INVALID_VALUE;
  if (!aligned(h, 16) || !aligned(W, 16) || !aligned(targets, 4) || !aligned(idx, 4) ||
      !aligned(n_active, 4) || !aligned(part_max, 4) || !aligned(part_sum, 4) ||
      !aligned(target_logit, 4))
    return RLK_ERROR_UNSUPPORTED;
  int grid = 0;
  hipError_t e = persistent_grid(&grid);
  if (e != hipSuccess) return RLK_ERROR_DEVICE;
  FwdTileArgs a{h, W, targets, idx, n_active, (int)N, (int)H, (int)V,
                (float)(1.0 / (double)temperature), part_max, part_sum, target_logit,
                (int)vocab_start};
  return dev_status(
      launch_fwd_tiles(a, dtype == RLK_BF16, grid, static_cast<hipStream_t>(stream), kFwdPlain));
}

rlk_status_t rlk_linear_logp_partials(const void* h, const void* W, const int32_t* targets,
                                      const int32_t* idx, const int32_t* n_active, int64_t N,
                                      int64_t H, int64_t V, int dtype, float temperature,
                                      float* part_max, float* part_sum, float* target_logit,
                                      void* stream) {
  return rlk_linear_logp_partials_shard(h, W, targets, idx, n_active, N, H, V, 0, V, dtype,
                                        temperature, part_max, part_sum, target_logit, stream);
}

rlk_status_t rlk_linear_logp_merge(const float* part_max, const float* part_sum,
                                   const float* target_logit, const int32_t* idx,
                                   const int32_t* n_active, int64_t N, int64_t V, float* logp,
                                   float* lse, void* stream) {
  if (N < 0 || V <= 0) return RLK_ERROR_INVALID_VALUE;
  if (N > kMaxTokens || V > kMaxVocab) return RLK_ERROR_UNSUPPORTED;
  if (N == 0) return RLK_SUCCESS;
  if (!part_max || !part_sum || !target_logit || !idx || !n_active || !logp)
    return RLK_ERROR_INVALID_VALUE;
  if (!aligned(part_max, 4) || !aligned(part_sum, 4) || !aligned(target_logit, 4) ||
      !aligned(idx, 4) || !aligned(n_active, 4) || !aligned(logp, 4) || (lse && !aligned(lse, 4)))
    return RLK_ERROR_UNSUPPORTED;
  MergeArgs a{part_max, part_sum, target_logit, idx, n_active, (int)N, (int)V, logp, lse};
  return dev_status(launch_fwd_merge(a, static_cast<hipStream_t>(stream)));
}

rlk_status_t rlk_logp_from_logits_workspace_size(int64_t N, int64_t V, size_t* bytes) {
  if (!bytes) return RLK_ERROR_INVALID_VALUE;
  if (N < 0 || V <= 0) return RLK_ERROR_INVALID_VALUE;
  if (N > kMaxTokens || V > kMaxLogitsVocab) return RLK_ERROR_UNSUPPORTED;
  *bytes = logits_layout(N).total;
  return RLK_SUCCESS;
}

rlk_status_t rlk_logp_from_logits(const void* logits, int64_t ld, const int32_t* targets,
                                  const uint8_t* mask, int64_t N, int64_t V, int dtype,
                                  float temperature, float* logp, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  rlk_status_t s = check_logits(logits, N, V, ld, dtype, temperature, targets, mask, logp, lse,
                                workspace, workspace_bytes);
  if (s != RLK_SUCCESS || N == 0) return s;
  const LogitsLayout L = logits_layout(N);
  int32_t* idx = carve<int32_t>(workspace, L.idx);
  int32_t* na = carve<int32_t>(workspace, L.n_active);
  s = rlk_compact_active(mask, N, idx, na, nullptr, logp, lse, stream);
  if (s != RLK_SUCCESS) return s;
  LogitsArgs a{logits, targets, idx, na, (int)N, (int)V, (int)ld,
               (float)(1.0 / (double)temperature), logp, lse};
  return dev_status(launch_logits_logp(a, dtype == RLK_BF16, static_cast<hipStream_t>(stream)));
}

rlk_status_t rlk_linear_logp_fwd(const void* h, const void* W, const int32_t* targets,
                                 const uint8_t* mask, int64_t N, int64_t H, int64_t V, int dtype,
                                 float temperature, float* logp, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  rlk_status_t s = check_fwd(h, W, targets, mask, N, H, V, dtype, temperature, logp, lse,
                             workspace, workspace_bytes);
  if (s != RLK_SUCCESS || N == 0) return s;
  const FwdLayout L = fwd_layout(N, V);
  int32_t* idx = carve<int32_t>(workspace, L.idx);
  int32_t* na = carve<int32_t>(workspace, L.n_active);
  float* zy = carve<float>(workspace, L.target_logit);
  float* pm = carve<float>(workspace, L.part_max);
  float* ps = carve<float>(workspace, L.part_sum);
  s = rlk_compact_active(mask, N, idx, na, zy, logp, lse, stream);
  if (s != RLK_SUCCESS) return s;
  s = rlk_linear_logp_partials(h, W, targets, idx, na, N, H, V, dtype, temperature, pm, ps, zy,
                               stream);
  if (s != RLK_SUCCESS) return s;
  return rlk_linear_logp_merge(pm, ps, zy, idx, na, N, V, logp, lse, stream);
}

rlk_status_t rlk_linear_logp_fwd_noalloc(const void* h, const void* W, const int32_t* targets,
                                         const uint8_t* mask, int64_t N, int64_t H, int64_t V,
                                         int dtype, float temperature, float* logp, float* lse,
                                         void* stream) {
  // every argument check first, against a stand-in for the scratch (256-byte aligned, non-null)
  rlk_status_t s = check_fwd(h, W, targets, mask, N, H, V, dtype, temperature, logp, lse,
                             reinterpret_cast<void*>(uintptr_t(256)), kNoAllocScratchBytes);
  if (s != RLK_SUCCESS || N == 0) return s;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return RLK_ERROR_DEVICE;
  return rlk_linear_logp_fwd(h, W, targets, mask, N, H, V, dtype, temperature, logp, lse, ws,
                             kNoAllocScratchBytes, stream);
}

rlk_status_t rlk_linear_logp_fwd_entropy(const void* h, const void* W, const int32_t* targets,
                                         const uint8_t* mask, int64_t N, int64_t H, int64_t V,
                                         int dtype, float temperature, float* logp, float* lse,
                                         float* entropy, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  rlk_status_t s = check_fwd(h, W, targets, mask, N, H, V, dtype, temperature, logp, lse,
                             workspace, workspace_bytes, true);
  if (s != RLK_SUCCESS || N == 0) return s;
  if (!entropy) return RLK_ERROR_INVALID_VALUE;
  if (!aligned(entropy, 4)) return RLK_ERROR_UNSUPPORTED;
  const FwdLayout L = fwd_layout(N, V, true);
  int32_t* idx = carve<int32_t>(workspace, L.idx);
  int32_t* na = carve<int32_t>(workspace, L.n_active);
  float* zy = carve<float>(workspace, L.target_logit);
  float* pm = carve<float>(workspace, L.part_max);
  float* ps = carve<float>(workspace, L.part_sum);
  float* pw = carve<float>(workspace, L.part_w);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the compaction zeroes logp and lse at every token; entropy gets the same treatment
  CompactArgs c{mask, idx, na, zy, logp, lse, (int)N, entropy};
  hipError_t e = launch_compact(c, st);
  if (e != hipSuccess) return RLK_ERROR_DEVICE;
  int grid = 0;
  e = persistent_grid(&grid);
  if (e != hipSuccess) return RLK_ERROR_DEVICE;
  FwdTileArgs a{h, W, targets, idx, na, (int)N, (int)H, (int)V,
                (float)(1.0 / (double)temperature), pm, ps, zy, 0, pw};
  e = launch_fwd_tiles(a, dtype == RLK_BF16, grid, st, kFwdEntropy);
  if (e != hipSuccess) return RLK_ERROR_DEVICE;
  MergeArgs m{pm, ps, zy, idx, na, (int)N, (int)V, logp, lse, pw, entropy};
  return dev_status(launch_fwd_merge(m, st));
}

rlk_status_t rlk_ratio_kl_loss_workspace_size(int64_t N, size_t* bytes) {
  if (!bytes || N < 0) return RLK_ERROR_INVALID_VALUE;
  if (N > kMaxTokens) return RLK_ERROR_UNSUPPORTED;
  *bytes = loss_workspace(N);
  return RLK_SUCCESS;
}

rlk_status_t rlk_ratio_kl_loss(const float* logp, const float* old_logp, const float* ref_logp,
                               const float* adv, const uint8_t* mask, int64_t N, float eps_lo,
                               float eps_hi, float beta, float scale, float* loss,
                               float* bwd_adv, float* ratio, double* sums, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (N < 0) return RLK_ERROR_INVALID_VALUE;
  if (N > kMaxTokens) return RLK_ERROR_UNSUPPORTED;
  if (!(eps_lo >= 0.f && eps_lo < 1.f) || !(eps_hi >= 0.f && eps_hi <= 1e30f) ||
      !(fabsf(beta) <= 1e30f) || !(fabsf(scale) <= 1e30f))
    return RLK_ERROR_INVALID_VALUE;
  if (N > 0 && (!logp || !old_logp || !adv || !mask || !loss || !bwd_adv))
    return RLK_ERROR_INVALID_VALUE;
  if (!workspace) return RLK_ERROR_INVALID_VALUE;
  if (!aligned(logp, 4) || !aligned(old_logp, 4) || !aligned(ref_logp, 4) || !aligned(adv, 4) ||
      !aligned(loss, 4) || !aligned(bwd_adv, 4) || !aligned(ratio, 4) || !aligned(sums, 8) ||
      !aligned(workspace, 256))
    return RLK_ERROR_UNSUPPORTED;
  if (workspace_bytes < loss_workspace(N)) return RLK_ERROR_WORKSPACE;
  LossArgs a{logp, old_logp, ref_logp, adv, mask, (int)N, eps_lo, eps_hi, beta, scale, loss,
             bwd_adv, ratio, static_cast<double*>(workspace)};
  return dev_status(launch_ratio_kl_loss(a, sums, static_cast<hipStream_t>(stream)));
}

rlk_status_t rlk_dlogp_diagnostics_workspace_size(int64_t N, size_t* bytes) {
  if (!bytes || N < 0) return RLK_ERROR_INVALID_VALUE;
  if (N > kMaxTokens) return RLK_ERROR_UNSUPPORTED;
  *bytes = diag_layout(N).total;
  return RLK_SUCCESS;
}

rlk_status_t rlk_dlogp_diagnostics(const float* logp_a, const float* logp_b,
                                   const uint8_t* mask, int64_t N, float clip_eps, double* out,
                                   int64_t* worst, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (N < 0) return RLK_ERROR_INVALID_VALUE;
  if (N > kMaxTokens) return RLK_ERROR_UNSUPPORTED;
  if (!(clip_eps >= 0.f && clip_eps <= 1e30f)) return RLK_ERROR_INVALID_VALUE;
  if (!out || !worst || !workspace) return RLK_ERROR_INVALID_VALUE;
  if (N > 0 && (!logp_a || !logp_b || !mask)) return RLK_ERROR_INVALID_VALUE;
  if (!aligned(logp_a, 4) || !aligned(logp_b, 4) || !aligned(out, 8) || !aligned(worst, 8) ||
      !aligned(workspace, 256))
    return RLK_ERROR_UNSUPPORTED;
  if (workspace_bytes < diag_layout(N).total) return RLK_ERROR_WORKSPACE;
  const DiagLayout L = diag_layout(N);
  int32_t* idx = carve<int32_t>(workspace, L.idx);
  int32_t* na = carve<int32_t>(workspace, L.n_active);
  hipStream_t st = static_cast<hipStream_t>(stream);
  CompactArgs c{mask, idx, na, nullptr, nullptr, nullptr, (int)N};
  hipError_t e = launch_compact(c, st);
  if (e != hipSuccess) return RLK_ERROR_DEVICE;
  DiagArgs a{logp_a, logp_b, idx, na, (int)N, clip_eps,
             carve<uint64_t>(workspace, L.keys), carve<double>(workspace, L.part),
             carve<uint64_t>(workspace, L.pmax), carve<int>(workspace, L.ptok),
             carve<int>(workspace, L.hist), carve<uint64_t>(workspace, L.sel),
             carve<int64_t>(workspace, L.sel + 8 * kDiagRanks), out, worst};
  return dev_status(launch_dlogp_diagnostics(a, st));
}

rlk_status_t rlk_linear_kl_fwd_workspace_size(int64_t N, int64_t H_s, int64_t H_t, int64_t V,
                                              int dtype, size_t* bytes) {
  if (!bytes) return RLK_ERROR_INVALID_VALUE;
  rlk_status_t s = check_shape(N, H_s, V, dtype);
  if (s == RLK_SUCCESS) s = check_shape(N, H_t, V, dtype);
  if (s != RLK_SUCCESS) return s;
  if (kl_fwd_blocks(N, V) > 1024) return RLK_ERROR_UNSUPPORTED;  // the compaction's bound
  *bytes = kl_fwd_layout(N, V).total;
  return RLK_SUCCESS;
}

rlk_status_t rlk_linear_kl_fwd_workspace_size_for_block(int64_t N, int64_t H_s, int64_t H_t,
                                                        int64_t V, int dtype,
                                                        int64_t block_tokens, size_t* bytes) {
  if (!bytes) return RLK_ERROR_INVALID_VALUE;
  rlk_status_t s = check_shape(N, H_s, V, dtype);
  if (s == RLK_SUCCESS) s = check_shape(N, H_t, V, dtype);
  if (s != RLK_SUCCESS) return s;
  if (block_tokens <= 0 || block_tokens % 256 != 0) return RLK_ERROR_INVALID_VALUE;
  const int64_t top = ((N > 0 ? N : 1) + 255) / 256 * 256;
  const int64_t cap = block_tokens < top ? block_tokens : top;
  if (bwd_blocks_cap(N, cap) > 1024) return RLK_ERROR_UNSUPPORTED;
  *bytes = kl_fwd_layout_cap(N, V, cap).total;
  return RLK_SUCCESS;
}

rlk_status_t rlk_linear_kl_fwd(const void* h_s, const void* W_s, const void* h_t,
                               const void* W_t, const uint8_t* mask, int64_t N, int64_t H_s,
                               int64_t H_t, int64_t V, int dtype, float temperature,
                               float* kl_fwd, float* kl_rev, float* lse_s, float* lse_t,
                               void* workspace, size_t workspace_bytes, void* stream) {
  rlk_status_t s = check_kl(h_s, W_s, h_t, W_t, mask, N, H_s, H_t, V, dtype, temperature,
                            workspace);
  if (s != RLK_SUCCESS || N == 0) return s;
  if (!kl_fwd || !kl_rev) return RLK_ERROR_INVALID_VALUE;
  if (!aligned(kl_fwd, 4) || !aligned(kl_rev, 4) || !aligned(lse_s, 4) || !aligned(lse_t, 4))
    return RLK_ERROR_UNSUPPORTED;
  // the block capacity is the largest the workspace holds (at most 1024 blocks)
  const int64_t cap64 = kl_fwd_cap_for_workspace(N, V, workspace_bytes);
  if (cap64 == 0) return RLK_ERROR_WORKSPACE;
  const KlLayout L = kl_fwd_layout_cap(N, V, cap64);
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* idx = carve<int32_t>(workspace, L.idx);
  int32_t* na = carve<int32_t>(workspace, L.n_active);
  int32_t* counts = carve<int32_t>(workspace, L.block_count);
  const int nblk = bwd_blocks_cap(N, cap64);
  const int cap = (int)cap64;
  const int np = (int)bwd_npad_cap(N, cap64);
  CompactArgs c{mask, idx, na, nullptr, kl_fwd, lse_s, (int)N, kl_rev, lse_t};
  c.block_count = counts;
  c.nblk = nblk;
  c.block_cap = cap;
  hipError_t e = launch_compact(c, st);
  if (e != hipSuccess) return RLK_ERROR_DEVICE;
  int grid = 0;
  if (persistent_grid(&grid) != hipSuccess) return RLK_ERROR_DEVICE;
  KlTileArgs t{};
  t.h_s = h_s;
  t.W_s = W_s;
  t.h_t = h_t;
  t.W_t = W_t;
  t.N = (int)N;
  t.H_s = (int)H_s;
  t.H_t = (int)H_t;
  t.V = (int)V;
  t.vstart = 0;
  t.inv_t = (float)(1.0 / (double)temperature);
  t.scratch = carve<float>(workspace, L.scratch);
  t.t_max = carve<float>(workspace, L.tmax);
  t.t_sum = carve<float>(workspace, L.tsum);
  t.s_max = carve<float>(workspace, L.smax);
  t.s_sum = carve<float>(workspace, L.ssum);
  t.wf = carve<float>(workspace, L.wf);
  t.wr = carve<float>(workspace, L.wr);
  t.pstride = np;
  KlArgs k{};
  k.N = np;  // the row stride of the block's statistics
  k.V = (int)V;
  k.t_max = t.t_max;
  k.t_sum = t.t_sum;
  k.s_max = t.s_max;
  k.s_sum = t.s_sum;
  k.wf = t.wf;
  k.wr = t.wr;
  k.kl_fwd = kl_fwd;
  k.kl_rev = kl_rev;
  k.lse_s = lse_s;
  k.lse_t = lse_t;
  // Per token block (the fixed partition: compacted indices b * cap ..; the statistics hold
  // one block's rows): both heads over the whole vocabulary in one launch, then the block's
  // merge writes its tokens' results.
  for (int b = 0; b < nblk; ++b) {
    const size_t t0 = (size_t)b * cap;
    t.idx = k.idx = idx + t0;
    t.n_active = k.n_active = counts + b;
    e = launch_kl_tiles(t, dtype == RLK_BF16, false, grid, st);
    if (e != hipSuccess) return RLK_ERROR_DEVICE;
    e = launch_kl_merge(k, st);
    if (e != hipSuccess) return RLK_ERROR_DEVICE;
  }
  return RLK_SUCCESS;
}

rlk_status_t rlk_linear_kl_bwd_workspace_size(int64_t N, int64_t H_s, int64_t H_t, int64_t V,
                                              int dtype, size_t* bytes) {
  if (!bytes) return RLK_ERROR_INVALID_VALUE;
  rlk_status_t s = check_shape(N, H_s, V, dtype);
  if (s == RLK_SUCCESS) s = check_shape(N, H_t, V, dtype);
  if (s != RLK_SUCCESS) return s;
  if (dtype != RLK_BF16 || H_s % 256 != 0) return RLK_ERROR_UNSUPPORTED;
  *bytes = kl_bwd_bytes(N, H_s);
  return RLK_SUCCESS;
}

rlk_status_t rlk_linear_kl_bwd(const void* h_s, const void* W_s, const void* h_t,
                               const void* W_t, const uint8_t* mask, int64_t N, int64_t H_s,
                               int64_t H_t, int64_t V, int dtype, float temperature,
                               const float* coef_fwd, const float* coef_rev, const float* lse_s,
                               const float* lse_t, const float* kl_rev, float* dh_s,
                               float* dW_s, void* workspace, size_t workspace_bytes,
                               void* stream) {
  rlk_status_t s = check_kl(h_s, W_s, h_t, W_t, mask, N, H_s, H_t, V, dtype, temperature,
                            workspace);
  if (s != RLK_SUCCESS) return s;
  if (dtype != RLK_BF16 || H_s % 256 != 0) return RLK_ERROR_UNSUPPORTED;
  if (!dW_s) return RLK_ERROR_INVALID_VALUE;
  if (!aligned(dW_s, 4)) return RLK_ERROR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (N == 0) return dev_status(launch_zero(dW_s, (size_t)V * (size_t)H_s, st));
  if ((!coef_fwd && !coef_rev) || !lse_s || !lse_t || !dh_s || (coef_rev && !kl_rev))
    return RLK_ERROR_INVALID_VALUE;
  if (!aligned(coef_fwd, 4) || !aligned(coef_rev, 4) || !aligned(lse_s, 4) || !aligned(lse_t, 4) ||
      !aligned(kl_rev, 4) ||
      !aligned(dh_s, 16))
    return RLK_ERROR_UNSUPPORTED;
  if (workspace_bytes < kl_bwd_bytes(N, H_s)) return RLK_ERROR_WORKSPACE;
  int grid = 0;
  if (persistent_grid(&grid) != hipSuccess) return RLK_ERROR_DEVICE;
  const BwdLayout L = kl_bwd_layout(N, H_s);
  const int64_t cap = kl_bwd_token_cap(H_s);
  const float inv_t = (float)(1.0 / (double)temperature);
  int32_t* idx = carve<int32_t>(workspace, L.idx);
  int32_t* na = carve<int32_t>(workspace, L.n_active);
  int32_t* desc = carve<int32_t>(workspace, L.block_desc);
  int32_t* bidx = carve<int32_t>(workspace, L.bidx);
  int32_t* bn = carve<int32_t>(workspace, L.bn);
  BwdArgs a{};
  a.h = h_s;
  a.W = W_s;
  a.N = (int)N;
  a.H = (int)H_s;
  a.V = (int)V;
  a.Npad = (int)bwd_npad_cap(N, cap);
  a.inv_t = inv_t;
  a.dh = dh_s;
  a.dW = dW_s;
  a.hT = carve<uint16_t>(workspace, L.hT);
  a.Gv = carve<uint16_t>(workspace, L.Gv);
  a.dhp[0] = nullptr;  // piece 0 accumulates in dh_s's rows
  for (int q = 1; q < kDhPieces; ++q) a.dhp[q] = carve<float>(workspace, L.dhp[q]);
  a.sched = carve<int>(workspace, L.sched);
  a.idx = bidx;
  a.n_active = bn;
  KlTileArgs t{};
  t.h_s = h_s;
  t.h_t = h_t;
  t.idx = bidx;
  t.n_active = bn;
  t.N = (int)N;
  t.H_s = (int)H_s;
  t.H_t = (int)H_t;
  t.inv_t = inv_t;
  t.scratch = carve<float>(workspace, L.total);
  t.lse_s = lse_s;
  t.lse_t = lse_t;
  t.kl_rev = kl_rev;
  t.coef_f = coef_fwd;
  t.coef_r = coef_rev;
  t.Gv = a.Gv;
  t.gv_pitch = kGvPitch;
  const int nblk = bwd_blocks_cap(N, cap);
  CompactArgs c{mask, idx, na, nullptr, nullptr, nullptr, (int)N};
  c.block_desc = desc;
  c.nblk = nblk;
  c.block_cap = (int)cap;
  hipError_t e = launch_compact(c, st);
  if (e != hipSuccess) return RLK_ERROR_DEVICE;
  e = launch_zero(dh_s, (size_t)N * (size_t)H_s, st);  // inactive rows stay 0
  if (e != hipSuccess) return RLK_ERROR_DEVICE;
  const int nchunks = (int)((V + kBwdChunk - 1) / kBwdChunk);
  for (int b = 0; b < nblk; ++b) {
    // the token block's compacted indices and count, copied for the kernels that follow
    e = launch_select_block(idx, desc, b, a.Npad, bidx, bn, st);
    if (e != hipSuccess) return RLK_ERROR_DEVICE;
    e = launch_bwd_transpose(a, st);
    if (e != hipSuccess) return RLK_ERROR_DEVICE;
    for (int ch = 0; ch < nchunks; ++ch) {
      const int64_t c0 = (int64_t)ch * kBwdChunk;
      // dL/dz of the chunk from both heads' tiles, then its dL/dh and dL/dW
      t.W_s = static_cast<const uint8_t*>(W_s) + (size_t)c0 * H_s * 2;
      t.W_t = static_cast<const uint8_t*>(W_t) + (size_t)c0 * H_t * 2;
      t.V = (int)(V - c0 < kBwdChunk ? V - c0 : kBwdChunk);
      t.vstart = (int)c0;
      e = launch_kl_tiles(t, true, true, grid, st);
      if (e != hipSuccess) return RLK_ERROR_DEVICE;
      e = launch_bwd_chunk_gemms(a, ch, grid, b > 0, st);
      if (e != hipSuccess) return RLK_ERROR_DEVICE;
    }
    e = launch_bwd_finish(a, st);
    if (e != hipSuccess) return RLK_ERROR_DEVICE;
  }
  return RLK_SUCCESS;
}

rlk_status_t rlk_linear_logp_bwd(const void* h, const void* W, const int32_t* targets,
                                 const uint8_t* mask, int64_t N, int64_t H, int64_t V, int dtype,
                                 float temperature, const float* adv, const float* lse,
                                 float* dh, float* dW, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return run_bwd(h, W, targets, mask, N, H, V, dtype, temperature, adv, lse, nullptr, nullptr,
                 dh, dW, workspace, workspace_bytes, stream);
}

rlk_status_t rlk_linear_logp_bwd_entropy(const void* h, const void* W, const int32_t* targets,
                                         const uint8_t* mask, int64_t N, int64_t H, int64_t V,
                                         int dtype, float temperature, const float* adv,
                                         const float* ent_coef, const float* lse,
                                         const float* entropy, float* dh, float* dW,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  if (N > 0 && (!ent_coef || !entropy)) return RLK_ERROR_INVALID_VALUE;
  if (!aligned(ent_coef, 4) || !aligned(entropy, 4)) return RLK_ERROR_UNSUPPORTED;
  return run_bwd(h, W, targets, mask, N, H, V, dtype, temperature, adv, lse, ent_coef, entropy,
                 dh, dW, workspace, workspace_bytes, stream);
}

rlk_status_t rlk_linear_logp_fwd_bwd_workspace_size(int64_t N, int64_t H, int64_t V, int dtype,
                                                    size_t* bytes) {
  if (!bytes) return RLK_ERROR_INVALID_VALUE;
  rlk_status_t s = check_shape(N, H, V, dtype);
  if (s != RLK_SUCCESS) return s;
  if (dtype != RLK_BF16 || H % 256 != 0 || fused_blocks(N, H, V) > 1024)
    return RLK_ERROR_UNSUPPORTED;
  *bytes = fused_layout(N, H, V).total;
  return RLK_SUCCESS;
}

rlk_status_t rlk_linear_logp_fwd_bwd_workspace_size_for_block(int64_t N, int64_t H, int64_t V,
                                                              int dtype, int64_t block_tokens,
                                                              size_t* bytes) {
  if (!bytes || block_tokens < 0) return RLK_ERROR_INVALID_VALUE;
  rlk_status_t s = check_shape(N, H, V, dtype);
  if (s != RLK_SUCCESS) return s;
  if (dtype != RLK_BF16 || H % 256 != 0 || fused_blocks(N, H, V) > 1024)
    return RLK_ERROR_UNSUPPORTED;
  const int64_t n = N > 0 ? N : 1;
  if (block_tokens == 0) block_tokens = fused_token_cap(H, V);  // the default's blocks
  const int64_t want = ((block_tokens < n ? block_tokens : n) + 255) / 256 * 256;
  if (bwd_blocks_cap(N, want) > 1024) return RLK_ERROR_UNSUPPORTED;
  *bytes = fused_layout_cap(N, H, V, want).total;
  return RLK_SUCCESS;
}

rlk_status_t rlk_linear_logp_fwd_bwd(const void* h, const void* W, const int32_t* targets,
                                     const uint8_t* mask, int64_t N, int64_t H, int64_t V,
                                     int dtype, float temperature, const float* adv, float* logp,
                                     float* lse, float* dh, float* dW, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return run_fused(h, W, targets, mask, N, H, V, dtype, temperature, adv, logp, lse, dh, dW,
                   workspace, workspace_bytes, stream);
}

rlk_status_t rlk_linear_logp_fwd_bwd_entropy_workspace_size(int64_t N, int64_t H, int64_t V,
                                                            int dtype, size_t* bytes) {
  if (!bytes) return RLK_ERROR_INVALID_VALUE;
  rlk_status_t s = check_shape(N, H, V, dtype);
  if (s != RLK_SUCCESS) return s;
  if (dtype != RLK_BF16 || H % 256 != 0 || fused_blocks(N, H, V, true) > 1024)
    return RLK_ERROR_UNSUPPORTED;
  *bytes = fused_layout(N, H, V, true).total;
  return RLK_SUCCESS;
}

rlk_status_t rlk_linear_logp_fwd_bwd_entropy(const void* h, const void* W,
                                             const int32_t* targets, const uint8_t* mask,
                                             int64_t N, int64_t H, int64_t V, int dtype,
                                             float temperature, const float* adv,
                                             const float* ent_coef, float* logp, float* lse,
                                             float* entropy, float* dh, float* dW,
                                             void* workspace, size_t workspace_bytes,
                                             void* stream) {
  if (N > 0 && (!ent_coef || !entropy)) return RLK_ERROR_INVALID_VALUE;
  if (!aligned(ent_coef, 4) || !aligned(entropy, 4)) return RLK_ERROR_UNSUPPORTED;
  // (N == 0: only dL/dW is written; ent_coef selects the layout, so a stand-in is passed)
  const float* ec = ent_coef ? ent_coef : reinterpret_cast<const float*>(uintptr_t(256));
  return run_fused(h, W, targets, mask, N, H, V, dtype, temperature, adv, logp, lse, dh, dW,
                   workspace, workspace_bytes, stream, nullptr, ec, entropy);
}

rlk_status_t rlk_linear_ppo_fwd_bwd_workspace_size(int64_t N, int64_t H, int64_t V, int dtype,
                                                   size_t* bytes) {
  if (!bytes) return RLK_ERROR_INVALID_VALUE;
  size_t f = 0;
  rlk_status_t s = rlk_linear_logp_fwd_bwd_workspace_size(N, H, V, dtype, &f);
  if (s != RLK_SUCCESS) return s;
  *bytes = loss_workspace(N) + f;
  return RLK_SUCCESS;
}

rlk_status_t rlk_linear_ppo_fwd_bwd(const void* h, const void* W, const int32_t* targets,
                                    const uint8_t* mask, int64_t N, int64_t H, int64_t V,
                                    int dtype, float temperature, const float* old_logp,
                                    const float* ref_logp, const float* adv, float eps_lo,
                                    float eps_hi, float beta, float scale, float* logp,
                                    float* lse, float* loss, float* bwd_adv, float* ratio,
                                    double* sums, float* dh, float* dW, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  // the loss fragment's own checks (as rlk_ratio_kl_loss), then the fused call's
  if (!(eps_lo >= 0.f && eps_lo < 1.f) || !(eps_hi >= 0.f && eps_hi <= 1e30f) ||
      !(fabsf(beta) <= 1e30f) || !(fabsf(scale) <= 1e30f))
    return RLK_ERROR_INVALID_VALUE;
  if (N > 0 && (!old_logp || !adv || !loss || !bwd_adv)) return RLK_ERROR_INVALID_VALUE;
  if (!aligned(old_logp, 4) || !aligned(ref_logp, 4) || !aligned(adv, 4) || !aligned(loss, 4) ||
      !aligned(bwd_adv, 4) || !aligned(ratio, 4) || !aligned(sums, 8) || !aligned(workspace, 256))
    return RLK_ERROR_UNSUPPORTED;
  const size_t lw = loss_workspace(N > 0 ? N : 0);
  if (!workspace) return RLK_ERROR_INVALID_VALUE;
  if (workspace_bytes < lw) return RLK_ERROR_WORKSPACE;
  FusedLoss fl;
  fl.args = LossArgs{nullptr, old_logp, ref_logp, adv, nullptr, 0, eps_lo, eps_hi, beta, scale,
                     loss, bwd_adv, ratio, static_cast<double*>(workspace)};
  fl.sums = sums;
  // adv is checked by the fused call as its upstream gradient; the loss replaces it there
  return run_fused(h, W, targets, mask, N, H, V, dtype, temperature, adv, logp, lse, dh, dW,
                   static_cast<uint8_t*>(workspace) + lw, workspace_bytes - lw, stream, &fl);
}

}  // extern "C"
