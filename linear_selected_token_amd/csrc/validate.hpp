// Host-side argument checks of the C ABI.  Pure functions: no HIP call, no device access,
// so every error path is decided before anything is enqueued.
#pragma once

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "rlk.h"

namespace rlk {

constexpr int64_t kMaxTokens = int64_t(1) << 22;
constexpr int64_t kMaxVocab = int64_t(1) << 22;
constexpr int64_t kMaxHidden = int64_t(1) << 16;
// The tile loads gather token rows of h with 32-bit buffer offsets from its base.
constexpr int64_t kMaxHiddenStateBytes = (int64_t(1) << 31) - 1;

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int64_t num_partials(int64_t V) { return V <= 0 ? 0 : (V + 127) / 128; }

inline int elt_size(int dtype) { return dtype == RLK_BF16 ? 2 : 4; }

// Shapes, dtype and temperature shared by every entry point.
inline rlk_status_t check_shape(int64_t N, int64_t H, int64_t V, int dtype) {
  if (N < 0 || H <= 0 || V <= 0) return RLK_ERROR_INVALID_VALUE;
  if (dtype != RLK_BF16 && dtype != RLK_FP32) return RLK_ERROR_UNSUPPORTED;
  if (H % 64 != 0) return RLK_ERROR_UNSUPPORTED;
  if (N > kMaxTokens || V > kMaxVocab || H > kMaxHidden) return RLK_ERROR_UNSUPPORTED;
  if (N * H * elt_size(dtype) > kMaxHiddenStateBytes) return RLK_ERROR_UNSUPPORTED;
  return RLK_SUCCESS;
}

// A vocabulary shard [vocab_start, vocab_start + V) of a vocabulary of V_global entries.  Its
// partial columns must be whole columns of the full vocabulary: it starts on a column boundary
// and, unless it is the last shard, ends on one.
inline rlk_status_t check_shard(int64_t V, int64_t vocab_start, int64_t V_global) {
  if (vocab_start < 0 || V_global <= 0 || vocab_start + V > V_global)
    return RLK_ERROR_INVALID_VALUE;
  if (V_global > kMaxVocab) return RLK_ERROR_UNSUPPORTED;
  if (vocab_start % 128 != 0) return RLK_ERROR_UNSUPPORTED;
  if (V % 128 != 0 && vocab_start + V != V_global) return RLK_ERROR_UNSUPPORTED;
  return RLK_SUCCESS;
}

inline rlk_status_t check_temperature(float T) {
  if (!isfinite(T) || !(T > 0.f)) return RLK_ERROR_INVALID_VALUE;
  // 1/T must be finite and nonzero in fp32
  const float inv = (float)(1.0 / (double)T);
  if (!isfinite(inv) || inv == 0.f) return RLK_ERROR_INVALID_VALUE;
  return RLK_SUCCESS;
}

// Workspace layout of the forward: idx[N] | n_active | target_logit[N] | part_max | part_sum.
struct FwdLayout {
  size_t idx, n_active, target_logit, part_max, part_sum, part_w, total;
};

// entropy: also room for the per-column entropy statistic (part_w)
inline FwdLayout fwd_layout(int64_t N, int64_t V, bool entropy = false) {
  FwdLayout L;
  const size_t n = (size_t)(N > 0 ? N : 1);
  const size_t np = (size_t)num_partials(V);
  size_t o = 0;
  L.idx = o;          o = align_up(o + 4 * n, 256);
  L.n_active = o;     o = align_up(o + 4, 256);
  L.target_logit = o; o = align_up(o + 4 * n, 256);
  L.part_max = o;     o = align_up(o + 4 * n * np, 256);
  L.part_sum = o;     o = align_up(o + 4 * n * np, 256);
  L.part_w = o;       if (entropy) o = align_up(o + 4 * n * np, 256);
  L.total = o;
  return L;
}

// Loss fragments: the per-work-group partial sums.
inline size_t loss_workspace(int64_t N) {
  const size_t nblk = (size_t)((N + 1023) / 1024);
  return align_up(32 * (nblk > 0 ? nblk : 1), 256);
}

struct DiagLayout {
  size_t idx, n_active, keys, part, pmax, ptok, hist, sel, total;
};

inline DiagLayout diag_layout(int64_t N) {
  DiagLayout L;
  const size_t n = (size_t)(N > 0 ? N : 1);
  const size_t nblk = (n + 1023) / 1024;
  size_t o = 0;
  L.idx = o;      o = align_up(o + 4 * n, 256);
  L.n_active = o; o = align_up(o + 4, 256);
  L.keys = o;     o = align_up(o + 8 * n, 256);
  L.part = o;     o = align_up(o + 32 * nblk, 256);
  L.pmax = o;     o = align_up(o + 8 * nblk, 256);
  L.ptok = o;     o = align_up(o + 4 * nblk, 256);
  L.hist = o;     o = align_up(o + 4 * 8 * 6 * 256, 256);
  L.sel = o;      o = align_up(o + 16 * 6, 256);
  L.total = o;
  return L;
}

constexpr int64_t kBwdChunkEntries = 32768;
constexpr int kBwdDhPieces = 2;  // dL/dh pieces of a full chunk (16384 entries each): the first
                                 // accumulates in dh, the other in the workspace

// The backward takes the active tokens in blocks (compacted order) and its buffers hold one
// block: per token of capacity, a row of the bf16 dL/dz chunk, three fp32 dL/dh piece rows
// (the first piece accumulates in dh itself) and a bf16 column of the transposed h.  The
// capacity is the largest multiple of 256 tokens whose buffers fit this budget (at least 256):
// 11008 tokens at H = 4096, 8960 at H = 7168.
constexpr size_t kBwdBlockBudget = 1000000000;  // bytes

inline size_t bwd_bytes_per_token(int64_t H) {
  return 2 * (size_t)(kBwdChunkEntries + 64) + 4 * (kBwdDhPieces - 1) * (size_t)H + 2 * (size_t)H;
}

inline int64_t bwd_token_cap(int64_t H) {
  const int64_t c = (int64_t)(kBwdBlockBudget / bwd_bytes_per_token(H > 0 ? H : 1)) / 256 * 256;
  return c < 256 ? 256 : c;
}

// Token blocks of at most cap tokens (a multiple of 256) for N tokens (an upper bound: it
// assumes every token is active; blocks past the active tokens do nothing), and the block
// buffers' rows: min(N, cap) rounded up to the 256-token tile.
inline int bwd_blocks_cap(int64_t N, int64_t cap) {
  return (int)(((N > 0 ? N : 1) + cap - 1) / cap);
}

inline int64_t bwd_npad_cap(int64_t N, int64_t cap) {
  const int64_t n = N <= 0 ? 1 : (N < cap ? N : cap);
  return (n + 255) / 256 * 256;
}

// At most 586 blocks of the backward's capacity for the shapes check_shape accepts (N <= 2^22
// and h <= 2^31 bytes bound N by the capacity's H).
inline int bwd_blocks(int64_t N, int64_t H) { return bwd_blocks_cap(N, bwd_token_cap(H)); }
inline int64_t bwd_npad(int64_t N, int64_t H) { return bwd_npad_cap(N, bwd_token_cap(H)); }

// Workspace layout of the backward: idx[N] | n_active | block_desc[blocks][2] | bidx[Npad] |
// bn | sched[8] | hT[H, Npad] | Gv[Npad, chunk] (bf16) | dhp[1 ..][Npad, H] (fp32).
struct BwdLayout {
  size_t idx, n_active, block_desc, bidx, bn, sched, hT, Gv, dhp[kBwdDhPieces], total;
};

inline BwdLayout bwd_layout_cap(int64_t N, int64_t H, int64_t cap) {
  BwdLayout L;
  const size_t n = (size_t)(N > 0 ? N : 1);
  const size_t np = (size_t)bwd_npad_cap(N, cap);
  const size_t c = (size_t)kBwdChunkEntries;
  size_t o = 0;
  L.idx = o;        o = align_up(o + 4 * n, 256);
  L.n_active = o;   o = align_up(o + 4, 256);
  L.block_desc = o; o = align_up(o + 8 * (size_t)bwd_blocks_cap(N, cap), 256);
  L.bidx = o;       o = align_up(o + 4 * np, 256);
  L.bn = o;         o = align_up(o + 4, 256);
  L.sched = o;      o = align_up(o + 4 * 8, 256);
  L.hT = o;         o = align_up(o + 2 * (size_t)H * np, 256);
  L.Gv = o;         o = align_up(o + 2 * np * (c + 64), 256);  // rows of kGvPitch entries
  L.dhp[0] = 0;     // piece 0 accumulates in dh's rows
  for (int q = 1; q < kBwdDhPieces; ++q) {
    L.dhp[q] = o;
    o = align_up(o + 4 * np * (size_t)H, 256);
  }
  L.total = o;
  return L;
}

inline BwdLayout bwd_layout(int64_t N, int64_t H) { return bwd_layout_cap(N, H, bwd_token_cap(H)); }

// The fused forward + backward keeps, per token of a block, the 16-bit d code of every vocabulary
// entry (one row of roundup(V, 256) + 64 entries, turned into bf16 dL/dz in place), the
// block's column statistics (max and sum per 128-entry column), its target logit, a bf16 column
// of the transposed h and the fp32 dL/dh piece rows past the first.  Blocks hold the largest
// multiple of 256 tokens whose buffers fit the backward's budget (at least 256): 2816 tokens
// for H = 4096, V = 151936.
inline int64_t fused_pitch(int64_t V) { return (V + 255) / 256 * 256 + 64; }

// ent: with an entropy bonus, a third statistic per column (4 bytes per 128 entries more).
inline size_t fused_bytes_per_token(int64_t H, int64_t V, bool ent = false) {
  return 2 * (size_t)fused_pitch(V) + (ent ? 12 : 8) * (size_t)num_partials(V) + 4 +
         4 * (kBwdDhPieces - 1) * (size_t)H + 2 * (size_t)H + 8;
}

inline int64_t fused_token_cap(int64_t H, int64_t V, bool ent = false) {
  const int64_t c =
      (int64_t)(kBwdBlockBudget / fused_bytes_per_token(H > 0 ? H : 1, V > 0 ? V : 1, ent)) /
      256 * 256;
  return c < 256 ? 256 : (c > kMaxTokens ? kMaxTokens : c);
}

// Blocks of at most cap tokens (a multiple of 256) for N tokens, and the block buffers' rows.
inline int fused_blocks_cap(int64_t N, int64_t cap) {
  return (int)(((N > 0 ? N : 1) + cap - 1) / cap);
}

inline int64_t fused_npad_cap(int64_t N, int64_t cap) {
  const int64_t n = N <= 0 ? 1 : (N < cap ? N : cap);
  return (n + 255) / 256 * 256;
}

inline int fused_blocks(int64_t N, int64_t H, int64_t V, bool ent = false) {
  return fused_blocks_cap(N, fused_token_cap(H, V, ent));
}

inline int64_t fused_npad(int64_t N, int64_t H, int64_t V, bool ent = false) {
  return fused_npad_cap(N, fused_token_cap(H, V, ent));
}

// Workspace layout of the fused forward + backward: idx[N] | n_active | block_desc[blocks][2] |
// bidx[Npad] | bn | sched[8] | target_logit[Npad] | part_max[J][Npad] | part_sum[J][Npad] |
// hT[H, Npad] | X[Npad, pitch] (d codes, then bf16 dL/dz) | dhp[1 ..][Npad, H] (fp32).
struct FusedLayout {
  size_t idx, n_active, block_desc, bidx, bn, sched, target_logit, part_max, part_sum, part_w,
      hT, X, dhp[kBwdDhPieces], total;
};

// The layout for blocks of at most cap tokens (fused_layout: the budget's capacity); ent adds
// the entropy statistic part_w[J][Npad] (else its size is 0).
inline FusedLayout fused_layout_cap(int64_t N, int64_t H, int64_t V, int64_t cap,
                                    bool ent = false) {
  FusedLayout L;
  const size_t n = (size_t)(N > 0 ? N : 1);
  const size_t np = (size_t)fused_npad_cap(N, cap);
  const size_t jn = 4 * np * (size_t)num_partials(V);
  size_t o = 0;
  L.idx = o;          o = align_up(o + 4 * n, 256);
  L.n_active = o;     o = align_up(o + 4, 256);
  L.block_desc = o;   o = align_up(o + 8 * (size_t)fused_blocks_cap(N, cap), 256);
  L.bidx = o;         o = align_up(o + 4 * np, 256);
  L.bn = o;           o = align_up(o + 4, 256);
  L.sched = o;        o = align_up(o + 4 * 8, 256);
  L.target_logit = o; o = align_up(o + 4 * np, 256);
  L.part_max = o;     o = align_up(o + jn, 256);
  L.part_sum = o;     o = align_up(o + jn, 256);
  L.part_w = o;       if (ent) o = align_up(o + jn, 256);
  L.hT = o;           o = align_up(o + 2 * (size_t)H * np, 256);
  L.X = o;            o = align_up(o + 2 * np * (size_t)fused_pitch(V), 256);
  L.dhp[0] = 0;       // piece 0 accumulates in dh's rows
  for (int q = 1; q < kBwdDhPieces; ++q) {
    L.dhp[q] = o;
    o = align_up(o + 4 * np * (size_t)H, 256);
  }
  L.total = o;
  return L;
}

inline FusedLayout fused_layout(int64_t N, int64_t H, int64_t V, bool ent = false) {
  return fused_layout_cap(N, H, V, fused_token_cap(H, V, ent), ent);
}

// The block capacity a workspace of ws_bytes allows: the largest multiple of 256 tokens, at most
// N rounded up to 256 (one block) and leaving at most 1024 blocks, whose layout fits ws_bytes;
// 0 if none does.  The budget's workspace gives the budget's capacity; a larger one buys fewer,
// larger blocks, a smaller one more, smaller blocks.
inline int64_t fused_cap_for_workspace(int64_t N, int64_t H, int64_t V, size_t ws_bytes,
                                       bool ent = false) {
  const int64_t n = N > 0 ? N : 1;
  const int64_t top = (n + 255) / 256 * 256;
  const int64_t low = (n + 1024 * 256 - 1) / (1024 * 256) * 256;  // ceil(n / 1024), to 256
  for (int64_t cap = top; cap >= low; cap -= 256)
    if (fused_layout_cap(N, H, V, cap, ent).total <= ws_bytes) return cap;
  return 0;
}

// Workspace of the log-prob from existing logits: idx[N] | n_active.
struct LogitsLayout {
  size_t idx, n_active, total;
};

inline LogitsLayout logits_layout(int64_t N) {
  LogitsLayout L;
  const size_t n = (size_t)(N > 0 ? N : 1);
  L.idx = 0;
  L.n_active = align_up(4 * n, 256);
  L.total = align_up(L.n_active + 4, 256);
  return L;
}

// The logits path keeps a row's column statistics in LDS (8 bytes per 128-entry column), at
// most 64000 bytes: up to 8000 columns.
constexpr int64_t kMaxLogitsVocab = int64_t(128) * 8000;

// Existing logits [N, ld] with V <= ld entries per row: rows are addressed in 16-byte units.
inline rlk_status_t check_logits(const void* logits, int64_t N, int64_t V, int64_t ld, int dtype,
                                 float T, const int32_t* targets, const uint8_t* mask,
                                 const float* logp, const float* lse, const void* ws,
                                 size_t ws_bytes) {
  if (N < 0 || V <= 0 || ld < V) return RLK_ERROR_INVALID_VALUE;
  if (dtype != RLK_BF16 && dtype != RLK_FP32) return RLK_ERROR_UNSUPPORTED;
  if (N > kMaxTokens || V > kMaxLogitsVocab || ld > (int64_t(1) << 24)) return RLK_ERROR_UNSUPPORTED;
  if ((ld * elt_size(dtype)) % 16 != 0) return RLK_ERROR_UNSUPPORTED;
  const float inv = (float)(1.0 / (double)T);
  if (!isfinite(T) || !(T > 0.f) || !isfinite(inv) || inv == 0.f) return RLK_ERROR_INVALID_VALUE;
  if (N == 0) return RLK_SUCCESS;
  if (!logits || !targets || !mask || !logp || !ws) return RLK_ERROR_INVALID_VALUE;
  if (!aligned(logits, 16) || !aligned(targets, 4) || !aligned(logp, 4) ||
      (lse && !aligned(lse, 4)) || !aligned(ws, 256))
    return RLK_ERROR_UNSUPPORTED;
  if (ws_bytes < logits_layout(N).total) return RLK_ERROR_WORKSPACE;
  return RLK_SUCCESS;
}

inline rlk_status_t check_fwd(const void* h, const void* W, const int32_t* targets,
                              const uint8_t* mask, int64_t N, int64_t H, int64_t V, int dtype,
                              float T, const float* logp, const float* lse, const void* ws,
                              size_t ws_bytes, bool entropy = false) {
  rlk_status_t s = check_shape(N, H, V, dtype);
  if (s != RLK_SUCCESS) return s;
  s = check_temperature(T);
  if (s != RLK_SUCCESS) return s;
  if (N == 0) return RLK_SUCCESS;
  if (!h || !W || !targets || !mask || !logp || !ws) return RLK_ERROR_INVALID_VALUE;
  if (!aligned(h, 16) || !aligned(W, 16) || !aligned(targets, 4) || !aligned(logp, 4) ||
      (lse && !aligned(lse, 4)) || !aligned(ws, 256))
    return RLK_ERROR_UNSUPPORTED;
  if (ws_bytes < fwd_layout(N, V, entropy).total) return RLK_ERROR_WORKSPACE;
  return RLK_SUCCESS;
}

inline rlk_status_t check_bwd(const void* h, const void* W, const int32_t* targets,
                              const uint8_t* mask, int64_t N, int64_t H, int64_t V, int dtype,
                              float T, const float* adv, const float* lse, const float* dh,
                              const float* dW, const void* ws, size_t ws_bytes) {
  rlk_status_t s = check_shape(N, H, V, dtype);
  if (s != RLK_SUCCESS) return s;
  s = check_temperature(T);
  if (s != RLK_SUCCESS) return s;
  if (dtype != RLK_BF16 || H % 256 != 0) return RLK_ERROR_UNSUPPORTED;
  if (!dW) return RLK_ERROR_INVALID_VALUE;
  if (N == 0) return RLK_SUCCESS;  // dW is still zeroed by the caller-visible contract
  if (!h || !W || !targets || !mask || !adv || !lse || !dh || !ws) return RLK_ERROR_INVALID_VALUE;
  if (!aligned(h, 16) || !aligned(W, 16) || !aligned(targets, 4) || !aligned(adv, 4) ||
      !aligned(lse, 4) || !aligned(dh, 16) || !aligned(dW, 4) || !aligned(ws, 256))
    return RLK_ERROR_UNSUPPORTED;
  if (ws_bytes < bwd_layout(N, H).total) return RLK_ERROR_WORKSPACE;
  return RLK_SUCCESS;
}

inline rlk_status_t check_fused(const void* h, const void* W, const int32_t* targets,
                                const uint8_t* mask, int64_t N, int64_t H, int64_t V, int dtype,
                                float T, const float* adv, const float* logp, const float* lse,
                                const float* dh, const float* dW, const void* ws,
                                size_t ws_bytes, bool ent = false) {
  rlk_status_t s = check_shape(N, H, V, dtype);
  if (s != RLK_SUCCESS) return s;
  s = check_temperature(T);
  if (s != RLK_SUCCESS) return s;
  if (dtype != RLK_BF16 || H % 256 != 0) return RLK_ERROR_UNSUPPORTED;
  if (fused_blocks(N, H, V, ent) > 1024) return RLK_ERROR_UNSUPPORTED;  // the compaction's bound
  if (!dW) return RLK_ERROR_INVALID_VALUE;
  if (N == 0) return RLK_SUCCESS;
  if (!h || !W || !targets || !mask || !adv || !logp || !lse || !dh || !ws)
    return RLK_ERROR_INVALID_VALUE;
  if (!aligned(h, 16) || !aligned(W, 16) || !aligned(targets, 4) || !aligned(adv, 4) ||
      !aligned(logp, 4) || !aligned(lse, 4) || !aligned(dh, 16) || !aligned(dW, 4) ||
      !aligned(ws, 256))
    return RLK_ERROR_UNSUPPORTED;
  if (fused_cap_for_workspace(N, H, V, ws_bytes, ent) == 0) return RLK_ERROR_WORKSPACE;
  return RLK_SUCCESS;
}

// Full-vocabulary KL.  The tile kernel keeps the teacher's accumulators of a tile in a scratch
// slot per work-group while the student's are formed: 256 slots of 8 x 128 x 64 floats (the
// launch's grid is at most 256 work-groups).
constexpr size_t kKlScratchBytes = (size_t)256 * 8 * 128 * 64 * 4;  // 64 MiB

// The KL forward takes the active tokens in blocks of its own: per token of capacity, a row of
// the six column-statistics arrays (both heads' maxima and sums, both cross terms), 24
// ceil(V / 128) bytes.  The capacity is the largest multiple of 256 tokens whose rows fit the
// backward's budget beside the scratch (at least 256): 32512 tokens at V = 151936.
inline size_t kl_fwd_bytes_per_token(int64_t V) { return 24 * (size_t)num_partials(V); }

inline int64_t kl_fwd_token_cap(int64_t V) {
  const int64_t c = (int64_t)((kBwdBlockBudget - kKlScratchBytes) /
                              kl_fwd_bytes_per_token(V > 0 ? V : 1)) / 256 * 256;
  return c < 256 ? 256 : (c > kMaxTokens ? kMaxTokens : c);
}

inline int kl_fwd_blocks(int64_t N, int64_t V) { return bwd_blocks_cap(N, kl_fwd_token_cap(V)); }
inline int64_t kl_fwd_npad(int64_t N, int64_t V) { return bwd_npad_cap(N, kl_fwd_token_cap(V)); }

struct KlLayout {
  size_t idx, n_active, block_count, tmax, tsum, smax, ssum, wf, wr, scratch, total;
};

// idx[N] | n_active | block_count[blocks] | six [J][Npad] statistics | scratch, for blocks of at
// most cap tokens (a multiple of 256)
inline KlLayout kl_fwd_layout_cap(int64_t N, int64_t V, int64_t cap) {
  KlLayout L;
  const size_t n = (size_t)(N > 0 ? N : 1);
  const int64_t np = bwd_npad_cap(N, cap);
  const size_t jn = 4 * (size_t)np * (size_t)num_partials(V);
  size_t o = 0;
  L.idx = o;      o = align_up(o + 4 * n, 256);
  L.n_active = o; o = align_up(o + 4, 256);
  L.block_count = o; o = align_up(o + 4 * (size_t)bwd_blocks_cap(N, cap), 256);
  L.tmax = o;     o = align_up(o + jn, 256);
  L.tsum = o;     o = align_up(o + jn, 256);
  L.smax = o;     o = align_up(o + jn, 256);
  L.ssum = o;     o = align_up(o + jn, 256);
  L.wf = o;       o = align_up(o + jn, 256);
  L.wr = o;       o = align_up(o + jn, 256);
  L.scratch = o;  o += kKlScratchBytes;
  L.total = o;
  return L;
}

inline KlLayout kl_fwd_layout(int64_t N, int64_t V) {
  return kl_fwd_layout_cap(N, V, kl_fwd_token_cap(V));
}

// The block capacity a KL forward workspace of ws bytes gives: the largest multiple of 256
// tokens, at most N rounded up to 256 and leaving at most 1024 blocks, whose layout fits; 0 if
// none does.  The default workspace gives kl_fwd_token_cap(V) (or one block for fewer tokens).
inline int64_t kl_fwd_cap_for_workspace(int64_t N, int64_t V, size_t ws) {
  const int64_t n = N > 0 ? N : 1;
  const int64_t top = (n + 255) / 256 * 256;
  const int64_t low = (n + 1024 * 256 - 1) / (1024 * 256) * 256;  // ceil(n / 1024), to 256
  for (int64_t cap = top; cap >= low; cap -= 256)
    if (kl_fwd_layout_cap(N, V, cap).total <= ws) return cap;
  return 0;
}

// The KL backward takes the active tokens in the backward's blocks, of a capacity whose
// buffers fit the budget beside the scratch: 10240 tokens at H_s = 4096.
inline int64_t kl_bwd_token_cap(int64_t H) {
  const int64_t c = (int64_t)((kBwdBlockBudget - kKlScratchBytes) /
                              bwd_bytes_per_token(H > 0 ? H : 1)) / 256 * 256;
  return c < 256 ? 256 : c;
}

// The backward's layout for that capacity, then the scratch.
inline BwdLayout kl_bwd_layout(int64_t N, int64_t H) {
  return bwd_layout_cap(N, H, kl_bwd_token_cap(H));
}
inline size_t kl_bwd_bytes(int64_t N, int64_t H) {
  return kl_bwd_layout(N, H).total + kKlScratchBytes;
}

inline rlk_status_t check_kl(const void* hs, const void* Ws, const void* ht, const void* Wt,
                             const uint8_t* mask, int64_t N, int64_t Hs, int64_t Ht, int64_t V,
                             int dtype, float T, const void* ws) {
  rlk_status_t s = check_shape(N, Hs, V, dtype);
  if (s != RLK_SUCCESS) return s;
  s = check_shape(N, Ht, V, dtype);
  if (s != RLK_SUCCESS) return s;
  s = check_temperature(T);
  if (s != RLK_SUCCESS) return s;
  if (N == 0) return RLK_SUCCESS;
  if (!hs || !Ws || !ht || !Wt || !mask || !ws) return RLK_ERROR_INVALID_VALUE;
  if (!aligned(hs, 16) || !aligned(Ws, 16) || !aligned(ht, 16) || !aligned(Wt, 16) ||
      !aligned(ws, 256))
    return RLK_ERROR_UNSUPPORTED;
  return RLK_SUCCESS;
}

}  // namespace rlk
