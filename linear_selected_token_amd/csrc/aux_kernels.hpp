// Argument blocks and launchers of the kernels that sit beside the fused log-prob: the loss
// fragments, the dlogp diagnostics and the full-vocabulary KL (host-visible, internal to the
// library).  Kept apart from kernels.hpp so that the forward tile kernel's sources do not
// change with them.
#pragma once

#include "kernels.hpp"

namespace rlk {

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
//
// The tile kernel runs both heads' GEMMs on the same 256 x 256 (vocabulary x token) tile, the
// teacher's first; the teacher's fp32 accumulators wait in the work-group's scratch slot
// (kKlSlotFloats floats, written and read back by the same lanes) while the student's are
// formed, and the student's epilogue pairs the two entry by entry.
constexpr int kKlSlots = 256;                     // scratch slots: the launch's grid is at most this
constexpr int kKlSlotFloats = 8 * 128 * 64;       // per work-group: 8 waves x 128 accumulators x 64 lanes

struct KlTileArgs {
  const void* h_s;  // [N][H_s] student hidden states (bf16 or fp32)
  const void* W_s;  // the launch's first vocabulary row of the student head, [V][H_s]
  const void* h_t;  // teacher
  const void* W_t;
  const int32_t* idx;       // the block's compacted token indices
  const int32_t* n_active;  // the block's token count
  int N, H_s, H_t;
  int V;       // vocabulary entries of the launch (rows of W_s and W_t from their bases)
  int vstart;  // global index of the launch's first entry (a multiple of 256)
  float inv_t;
  float* scratch;  // [kKlSlots][kKlSlotFloats]
  // forward: per token of the block and 128-entry column, [J][pstride]: each head's column
  // maximum (log2 units) and sum, and the two cross terms
  float* t_max;
  float* t_sum;
  float* s_max;
  float* s_sum;
  float* wf;
  float* wr;
  int pstride;
  // backward: dL/dz of the launch's entries for the block's tokens, bf16, [rows][gv_pitch]
  const float* lse_s;   // [N] natural-log lse of each head, from the forward
  const float* lse_t;
  const float* kl_rev;  // [N] with coef_r only
  const float* coef_f;  // [N] dL/dKL_fwd per token, or null
  const float* coef_r;  // [N] dL/dKL_rev per token, or null (not both null)
  uint16_t* Gv;
  int gv_pitch;
};

// The per-token merge of the block's column statistics.
struct KlArgs {
  const int32_t* idx;
  const int32_t* n_active;
  int N, V;            // N: the statistics' column stride
  const float* s_max;  // [J][N] column statistics
  const float* s_sum;
  const float* t_max;
  const float* t_sum;
  const float* wf;     // [J][N] forward-KL cross term per column
  const float* wr;     // reverse
  float* kl_fwd;       // [N] outputs of the merge
  float* kl_rev;
  float* lse_s;        // may be null
  float* lse_t;        // may be null
};

hipError_t launch_ratio_kl_loss(const LossArgs& a, double* sums, hipStream_t stream);
hipError_t launch_dlogp_diagnostics(const DiagArgs& a, hipStream_t stream);
// mode: false the forward statistics, true the backward's dL/dz; grid at most kKlSlots
hipError_t launch_kl_tiles(const KlTileArgs& a, bool bf16, bool grad, int grid, hipStream_t stream);
hipError_t launch_kl_merge(const KlArgs& a, hipStream_t stream);

}  // namespace rlk
