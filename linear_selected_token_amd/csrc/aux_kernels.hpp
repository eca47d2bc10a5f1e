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
  const float* kl_rev_in;  // with coef_r only
  const float* coef_f;     // [N] dL/dKL_fwd per token, or null
  const float* coef_r;     // [N] dL/dKL_rev per token, or null (not both null)
  uint16_t* Gv;            // [Npad][kGvPitch]
};

hipError_t launch_ratio_kl_loss(const LossArgs& a, double* sums, hipStream_t stream);
hipError_t launch_dlogp_diagnostics(const DiagArgs& a, hipStream_t stream);
hipError_t launch_kl_cross(const KlArgs& a, int c0, int rows, hipStream_t stream);
hipError_t launch_kl_merge(const KlArgs& a, hipStream_t stream);
hipError_t launch_kl_grad(const KlArgs& a, int c0, int rows, hipStream_t stream);

}  // namespace rlk
