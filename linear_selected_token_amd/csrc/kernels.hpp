// Kernel argument blocks and launchers (host-visible, internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlk {

constexpr int kVocabPartial = 128;  // vocabulary entries per partial-statistics column
constexpr int kBwdChunk = 32768;    // vocabulary entries per backward chunk (build constant)
constexpr int kDhSplitK = 16384;    // dL/dh sums each chunk's first and second 16384 entries apart
// Row pitch (entries) of the token-major chunk buffers: the chunk plus 128 bytes, so that the
// rows a wave writes at once (32 tokens) do not all start at the same 64 KiB-aligned offset.
constexpr int kGvPitch = kBwdChunk + 64;  // bf16 dL/dz
constexpr int kXPitch = kBwdChunk + 32;   // fp32 x of the KL path

struct CompactArgs {
  const uint8_t* mask;
  int32_t* idx;
  int32_t* n_active;
  float* target_logit;  // [N], set to NaN (may be null)
  float* logp;          // may be null: 0 at inactive tokens
  float* lse;           // may be null: 0 at inactive tokens
  int N;
  float* entropy = nullptr;  // may be null: 0 at inactive tokens
  float* extra = nullptr;    // may be null: 0 at inactive tokens
};

struct FwdTileArgs {
  const void* h;
  const void* W;
  const int32_t* targets;
  const int32_t* idx;
  const int32_t* n_active;
  int N, H, V;
  float inv_t;
  float* part_max;
  float* part_sum;
  float* target_logit;
  int vstart;  // global vocabulary index of W row 0 (a multiple of kVocabPartial)
  float* part_w = nullptr;  // [J][N] entropy statistic per column (kFwdEntropy)
  float* xbuf = nullptr;    // [Npad][kXPitch] x = z log2 e of one vocabulary chunk (kFwdStoreX)
};

enum FwdMode { kFwdPlain = 0, kFwdEntropy = 1, kFwdStoreX = 2 };

struct MergeArgs {
  const float* part_max;
  const float* part_sum;
  const float* target_logit;
  const int32_t* idx;
  const int32_t* n_active;
  int N, V;
  float* logp;
  float* lse;
  const float* part_w = nullptr;  // entropy statistics, or null
  float* entropy = nullptr;       // [N], written at active tokens when part_w is given
};

// Log-prob from existing logits rows.
struct LogitsArgs {
  const void* logits;     // [N, ld] bf16 or fp32; entries 0 .. V-1 of each row are the logits
  const int32_t* targets;
  const int32_t* idx;
  const int32_t* n_active;
  int N, V, ld;
  float inv_t;
  float* logp;            // [N], written at active tokens
  float* lse;             // [N] or null
};

// Backward buffers (bf16 stored as uint16_t).
struct BwdArgs {
  const void* h;          // [N, H] bf16
  const void* W;          // [V, H] bf16
  const int32_t* targets; // [N]
  const float* adv;       // [N]
  const float* lse;       // [N]
  const int32_t* idx;     // [N] compacted active positions
  const int32_t* n_active;
  int N, H, V, Npad;      // Npad: token capacity of the G / hT buffers (multiple of 256)
  float inv_t;
  float* dh;              // [N, H]
  float* dW;              // [V, H]
  uint16_t* hT;           // [H, Npad]   compacted h, transposed, zero past Na
  uint16_t* Gv;           // [Npad, kGvPitch] dL/dz of the chunk, token-major
  float* dh1;             // [Npad, H] dL/dh from the second half of every chunk, compacted rows
  // entropy bonus (both null without it): L gains -sum_t mask_t c_t H_t
  const float* ent_coef = nullptr;  // [N] c_t
  const float* entropy = nullptr;   // [N] H_t from the entropy forward
};

// Loss fragments on the log-prob (per-token, then fixed-order fp64 sums).
constexpr int kLossBlock = 1024;  // tokens per work-group
constexpr int kDiagRanks = 6;     // order statistics behind the 50/90/99th percentiles
constexpr int kDiagOut = 9;       // doubles written by the diagnostics

struct LossArgs {
  const float* logp;
  const float* old_logp;
  const float* ref_logp;  // may be null: no KL term
  const float* adv;
  const uint8_t* mask;
  int N;
  float eps_lo, eps_hi, beta, scale;
  float* loss;     // [N]
  float* bwd_adv;  // [N] -dL/dlogp
  float* ratio;    // [N] or null
  double* part;    // [ceil(N / kLossBlock)][4]
};

struct DiagArgs {
  const float* a;
  const float* b;
  const int32_t* idx;
  const int32_t* n_active;
  int N;
  float eps;
  uint64_t* keys;   // [N] bit patterns of |dlogp| of the active tokens, compacted
  double* part;     // [nblk][4]
  uint64_t* pmax;   // [nblk]
  int* ptok;        // [nblk]
  int* hist;        // [8][kDiagRanks][256]
  uint64_t* sel_prefix;  // [kDiagRanks] bytes selected so far, most significant first
  int64_t* sel_rank;     // [kDiagRanks] rank left under that prefix
  double* out;      // [kDiagOut]
  int64_t* worst;
};

// Full-vocabulary KL between a student (s) and a teacher (t) head.
struct KlArgs {
  const int32_t* idx;
  const int32_t* n_active;
  int N, V;
  float inv_t;
  const float* xs;     // [Npad][kXPitch] student x of the current chunk
  const float* xt;     // teacher
  const float* s_max;  // [J][N] column statistics
  const float* s_sum;
  const float* t_max;
  const float* t_sum;
  float* wf;           // [J][N] forward-KL cross term per column
  float* wr;           // reverse
  float* kl_fwd;       // [N] outputs of the merge
  float* kl_rev;
  float* lse_s;        // may be null
  float* lse_t;        // may be null
  // backward
  const float* lse_s_in;
  const float* lse_t_in;
  const float* kl_rev_in;  // reverse KL only
  const float* coef;       // [N] c_t
  uint16_t* Gv;            // [Npad][kGvPitch]
};

hipError_t launch_compact(const CompactArgs& a, hipStream_t stream);
hipError_t launch_fwd_tiles(const FwdTileArgs& a, bool bf16, int grid, hipStream_t stream,
                            int mode);
hipError_t launch_fwd_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_logits_logp(const LogitsArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_ratio_kl_loss(const LossArgs& a, double* sums, hipStream_t stream);
hipError_t launch_dlogp_diagnostics(const DiagArgs& a, hipStream_t stream);
hipError_t launch_kl_cross(const KlArgs& a, int c0, int rows, hipStream_t stream);
hipError_t launch_kl_merge(const KlArgs& a, hipStream_t stream);
hipError_t launch_kl_grad(const KlArgs& a, int c0, int rows, bool reverse, hipStream_t stream);

// Backward phases.
hipError_t launch_zero(float* p, size_t n, hipStream_t stream);
hipError_t launch_bwd_prepare(const BwdArgs& a, hipStream_t stream);          // dh = 0, hT
hipError_t launch_bwd_chunk(const BwdArgs& a, int chunk, int grid, hipStream_t stream);
// dL/dh and dL/dW of one chunk from a Gv written elsewhere
hipError_t launch_bwd_chunk_gemms(const BwdArgs& a, int chunk, int grid, hipStream_t stream);
hipError_t launch_bwd_finish(const BwdArgs& a, hipStream_t stream);          // dh += dh1

}  // namespace rlk
