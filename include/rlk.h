/*
 * rlk.h -- C ABI of the fused linear log-prob for AMD Instinct MI355X (gfx950).
 *
 * The operation (RL-Kernel Roadmap (2026), P0.2 "Fused CE LogProb without materializing
 * logits + fused backward"; RL-Kernel integration roadmap for vime, "Operator Integration
 * Plan", linear_logp): given hidden states h[N,H], the LM-head weight W[V,H], target ids
 * y[N], an active mask and a temperature T, compute for every active token t
 *
 *     z[t,v]  = (h_t . W_v) / T
 *     lse[t]  = log sum_v exp(z[t,v])
 *     logp[t] = z[t, y_t] - lse[t]
 *
 * without forming the [N,V] logits.  The backward pass of L = -sum_t mask_t adv_t logp_t
 * recomputes the logits tile by tile (the roadmap's "chunked backward" that trades compute
 * for memory) and returns dL/dh and dL/dW.
 *
 * Also exported, under the same conventions: the forward with each token's entropy and the
 * backward with an entropy bonus; the log-prob from logits that already exist; the forward
 * and reverse full-vocabulary KL between a student and a teacher head, with its backward; the
 * clipped policy-gradient loss fragment with a KL penalty and the dlogp diagnostics; and the
 * building blocks of the forward (compaction, per-column partials, vocabulary shards, merge).
 *
 * Batch invariance (RL-Kernel Roadmap (2026), P0.2 "Batch-Invariant Deterministic
 * LogProb"; vime roadmap, "Consistency Contract"): a token's logp, lse and dL/dh row are
 * bit-identical whatever else is in the batch, in whatever order, with whatever padding
 * and active-mask density, on repeat runs and on any stream, for one build of this library
 * (rlk_build_info names the build).  No atomics touch results; the vocabulary tiling and
 * every reduction order are constants of the build, independent of N.  dL/dW is a sum over
 * tokens: it is deterministic run to run and does not depend on padding or inactive rows.
 *
 * Conventions for every entry point:
 *   - Every array argument is a DEVICE pointer owned by the caller (the `bytes` result of
 *     the *_workspace_size queries is the only host pointer).  Arrays are dense and
 *     row-major.  Hidden states and weights must be 16-byte aligned, the workspace 256-byte
 *     aligned, float and int32 arrays 4-byte aligned, double and int64 arrays 8-byte.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  All work is
 *     enqueued on it; nothing blocks the host; results are valid once the stream reaches
 *     that point.  The library never allocates or frees device memory.
 *   - dtype: RLK_BF16 (h and W hold bf16) or RLK_FP32 (float).  Accumulation is fp32.
 *   - Size limits (beyond them: RLK_ERROR_UNSUPPORTED): N <= 2^22, V <= 2^22, H <= 2^16,
 *     H a multiple of 64, and h at most 2^31 - 1 bytes (N * H * element size), because the
 *     tile loads address token rows with 32-bit offsets from h.
 *   - Every argument check happens on the host before anything is enqueued, so a call
 *     that returns an error has written nothing.  N == 0 returns RLK_SUCCESS at once.
 *   - An active token whose target is outside [0, V) gets logp = NaN (checking it on the
 *     host would need a device-to-host copy); its lse is still correct, and in the
 *     backward its dL/dz has no target term (only -g_t p[t,v]).
 *   - Inactive tokens (mask == 0) are never read into the products; their h rows and
 *     targets may hold anything.  Their logp and lse are 0 and their dL/dh row is 0.
 *   - Calls are reentrant: the only shared state is read-only device properties.
 *     Calls that share a workspace must be ordered by the caller (same stream).
 */
#ifndef RLK_H_
#define RLK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RLK_SUCCESS = 0,
  RLK_ERROR_INVALID_VALUE = 1, /* NULL required pointer, N < 0, H or V <= 0, T not finite or <= 0 */
  RLK_ERROR_UNSUPPORTED = 2,   /* dtype, H % 64 != 0, misalignment, sizes beyond the limits */
  RLK_ERROR_WORKSPACE = 3,     /* workspace smaller than the *_workspace_size query */
  RLK_ERROR_DEVICE = 4         /* a HIP launch or runtime call failed */
} rlk_status_t;

typedef enum { RLK_BF16 = 0, RLK_FP32 = 1 } rlk_dtype_t;

/* Width, in vocabulary entries, of one partial-statistics column (see
 * rlk_linear_logp_partials).  A constant of the build. */
#define RLK_VOCAB_PARTIAL 128

/* Static description of a status code.  Never NULL. */
const char* rlk_status_string(int status);

/* Build fingerprint: target architecture, compiler, tile constants.  The bitwise
 * batch-invariance claim holds per fingerprint (vime roadmap, "Consistency Contract",
 * deterministic operator claim).  Never NULL. */
const char* rlk_build_info(void);

/* Number of partial-statistics columns for a vocabulary of V entries:
 * ceil(V / RLK_VOCAB_PARTIAL).  Returns 0 for V <= 0. */
int64_t rlk_num_vocab_partials(int64_t V);

/* Workspace bytes needed by rlk_linear_logp_fwd / rlk_linear_logp_bwd for N tokens
 * (an upper bound: it assumes every token is active).  Host-only, no device work.
 * The forward's grows with N (8 bytes per token and 128-entry vocabulary column).  The
 * backward's stops growing past one token block (see rlk_linear_logp_bwd): about 1e9 bytes at
 * most, plus 4 bytes of index per token. */
rlk_status_t rlk_linear_logp_fwd_workspace_size(int64_t N, int64_t H, int64_t V, int dtype,
                                                size_t* bytes);
rlk_status_t rlk_linear_logp_bwd_workspace_size(int64_t N, int64_t H, int64_t V, int dtype,
                                                size_t* bytes);

/* Forward: selected-token log-prob.
 *   h        [N,H]  dtype     hidden states
 *   W        [V,H]  dtype     LM-head weight
 *   targets  [N]    int32     target ids; must lie in [0,V) where mask != 0
 *   mask     [N]    uint8     0 = inactive (prompt, padding), nonzero = active
 *   temperature               finite and > 0; the logits are divided by it exactly once
 *   logp     [N]    float     out: z[t,y_t] - lse[t] at active tokens, 0 elsewhere
 *   lse      [N]    float     out (may be NULL): log-sum-exp of z[t,:], 0 at inactive tokens;
 *                             rlk_linear_logp_bwd takes it back
 *   workspace / workspace_bytes: device scratch of at least
 *                             rlk_linear_logp_fwd_workspace_size bytes; its contents on
 *                             entry do not matter.
 * Equivalent to rlk_compact_active + rlk_linear_logp_partials + rlk_linear_logp_merge on
 * buffers carved out of the workspace. */
rlk_status_t rlk_linear_logp_fwd(const void* h, const void* W, const int32_t* targets,
                                 const uint8_t* mask, int64_t N, int64_t H, int64_t V, int dtype,
                                 float temperature, float* logp, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* The forward without a workspace argument, for callers that cannot allocate device memory
 * (code under stream capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * library's own scratch serves as the workspace: a static device array of
 * RLK_NOALLOC_SCRATCH_BYTES per device, held from the time the library's code is loaded on a
 * device until the process ends; the call allocates and frees nothing.
 *   h, W, targets, mask, N, H, V, dtype, temperature, logp, lse: as for rlk_linear_logp_fwd;
 *                             the outputs are bit-identical to rlk_linear_logp_fwd's.
 * The forward's workspace must fit the scratch: rlk_linear_logp_fwd_workspace_size(N, H, V)
 * <= RLK_NOALLOC_SCRATCH_BYTES (about 9.5 KB per token at V = 151936, i.e. up to ~7000 tokens;
 * about 2 KB per token at V = 32000), else RLK_ERROR_WORKSPACE and nothing is written.  Every
 * call on a device shares that device's scratch and leaves its contents there; each call
 * overwrites everything it reads (nothing needs to start at zero).  Calls that overlap on one
 * device (several host threads or streams at once) race on the scratch: the caller orders
 * them, for example on one stream. */
#define RLK_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
rlk_status_t rlk_linear_logp_fwd_noalloc(const void* h, const void* W, const int32_t* targets,
                                         const uint8_t* mask, int64_t N, int64_t H, int64_t V,
                                         int dtype, float temperature, float* logp, float* lse,
                                         void* stream);

/* Forward with the entropy of each active token's distribution, in the same pass:
 * entropy[t] = -sum_v p[t,v] log p[t,v] with p[t,:] = softmax(z[t,:]), z = h W^T / T (the
 * entropy statistic the RL-Kernel Roadmap (2026) lists next to the fused log-prob, "operator
 * backlog"; vime roadmap, "Fast and Consistency Compatibility", entropy without
 * materialising the logits).
 *   h, W, targets, mask, N, H, V, dtype, temperature, logp, lse: as for rlk_linear_logp_fwd;
 *                             logp and lse are bit-identical to what rlk_linear_logp_fwd
 *                             returns for the same inputs
 *   entropy  [N]    float     out: the entropy at active tokens (natural log, clamped at 0
 *                             against rounding), 0 elsewhere
 *   workspace: at least rlk_linear_logp_fwd_entropy_workspace_size bytes (the forward's
 *              workspace plus one more float per token and 128-entry vocabulary column).
 * Per active token and vocabulary column the tile epilogue also forms
 * sum_v 2^(x_v - m) (x_v - m) (x = z log2 e, m the column maximum); the merge rescales these
 * to the global maximum M in the forward's fixed association and returns
 * ln 2 * (log2 S - sum_v 2^(x_v - M) (x_v - M) / S), S = sum_v 2^(x_v - M).  Batch-invariant
 * like logp. */
rlk_status_t rlk_linear_logp_fwd_entropy_workspace_size(int64_t N, int64_t H, int64_t V,
                                                        int dtype, size_t* bytes);
rlk_status_t rlk_linear_logp_fwd_entropy(const void* h, const void* W, const int32_t* targets,
                                         const uint8_t* mask, int64_t N, int64_t H, int64_t V,
                                         int dtype, float temperature, float* logp, float* lse,
                                         float* entropy, void* workspace, size_t workspace_bytes,
                                         void* stream);

/* Selected-token log-prob from logits that already exist: the reference-scoring sibling of
 * the fused path, with the same log-softmax contract (RL-Kernel integration roadmap for vime,
 * "Operator Integration Plan", logp Reference Scoring: a deterministic policy with a fixed
 * row-local reduction topology and an explicit max / sum-exp contract).
 *   logits   [N, ld] dtype    row t holds the logits of token t in entries 0 .. V-1 (entries
 *                             V .. ld-1 are ignored); ld >= V, ld * element size a multiple
 *                             of 16 bytes, logits 16-byte aligned
 *   targets, mask, temperature, logp, lse: as for rlk_linear_logp_fwd (z = logit / T)
 *   workspace: at least rlk_logp_from_logits_workspace_size bytes (the active-row index).
 * V is at most 1,024,000 (a row's column statistics are kept on chip).
 * Per active token and 128-entry vocabulary column the column maximum and sum-exp are formed
 * in log2 units exactly as in rlk_linear_logp_partials, then merged in the association of
 * rlk_linear_logp_merge: a token's result depends only on its own row and is bit-identical in
 * any batch.  An active token whose target is outside [0, V) gets logp = NaN. */
rlk_status_t rlk_logp_from_logits_workspace_size(int64_t N, int64_t V, size_t* bytes);
rlk_status_t rlk_logp_from_logits(const void* logits, int64_t ld, const int32_t* targets,
                                  const uint8_t* mask, int64_t N, int64_t V, int dtype,
                                  float temperature, float* logp, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Backward of L = -sum_t mask_t * adv_t * logp_t (bf16 only, H a multiple of 256).
 *   h, W, targets, mask, N, H, V, dtype, temperature: exactly as passed to the forward
 *   adv      [N]    float     per-token advantage (the upstream gradient is -adv_t at
 *                             active tokens; pass adv = -dL/dlogp for another loss)
 *   lse      [N]    float     the forward's lse output for the same inputs
 *   dh       [N,H]  float     out, overwritten: dL/dh; rows of inactive tokens are 0.
 *                             16-byte aligned (it also serves as one of the partial sums)
 *   dW       [V,H]  float     out, overwritten: dL/dW
 *   workspace: at least rlk_linear_logp_bwd_workspace_size bytes.
 * The vocabulary is walked in fixed chunks; per chunk the logits are recomputed on MFMA,
 * turned into dL/dz (rounded to bf16), and multiplied into dh (accumulated in fp32 in a fixed
 * order of vocabulary pieces) and into the chunk's rows of dW.  The active tokens are taken in
 * blocks of equal size (the last shorter), at most the largest multiple of 256 tokens whose
 * buffers (65664 + 6 H bytes per token) fit 1e9 bytes: 11008 tokens at H = 4096, 8960 at
 * H = 7168.  The workspace holds one block, so it does not grow with N past that.  A token's
 * dL/dh row does not depend on the block it falls in (bit-identical in any batch); dL/dW is
 * the sum of the blocks' sums in ascending block order (deterministic, and independent of
 * padding and inactive rows). */
rlk_status_t rlk_linear_logp_bwd(const void* h, const void* W, const int32_t* targets,
                                 const uint8_t* mask, int64_t N, int64_t H, int64_t V, int dtype,
                                 float temperature, const float* adv, const float* lse,
                                 float* dh, float* dW, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Forward and backward in one call (bf16 only, H a multiple of 256): logp and lse as
 * rlk_linear_logp_fwd returns them (the same bits), and dL/dh, dL/dW of
 * L = -sum_t mask_t * adv_t * logp_t as rlk_linear_logp_bwd defines them, for a loss whose
 * upstream gradient is known before the forward (RL-Kernel Roadmap (2026), P0.2: fused linear
 * log-prob with a fused backward).  Instead of recomputing the logits for the backward, each
 * token block's forward keeps d = x - m (x = z log2 e / T, m the maximum over the token's
 * 128-entry vocabulary column, so d <= 0) of every entry as a 16-bit code, round(-d 2^9)
 * clamped to 65535, and turns it into dL/dz once lse is known: three GEMMs per step instead of
 * four.  The code moves each p by at most 2^-10 ln 2 relative, whatever d is (entries with
 * d <= -128 have p < 2^-128); dL/dz is rounded to bf16 as in the two-call path, whose dh and
 * dW differ from these only by such rounding.  With every column's dL/dz in place, one launch
 * per block runs both GEMMs over the whole vocabulary; dL/dh sums the two halves of the
 * vocabulary apart and then adds them (the two-call path sums 16384-entry pieces of 32768-entry
 * chunks), a split fixed by V alone.
 *   h, W, targets, mask, N, H, V, dtype, temperature, adv: as for rlk_linear_logp_bwd
 *   logp [N] float  out: as rlk_linear_logp_fwd
 *   lse  [N] float  out (required: the gradient pass reads it back)
 *   dh   [N,H] float out, overwritten: dL/dh (inactive rows 0), 16-byte aligned
 *   dW   [V,H] float out, overwritten: dL/dW
 *   workspace: rlk_linear_logp_fwd_bwd_workspace_size bytes by default.  The active tokens
 *   are taken in blocks of equal size (the last shorter) of at most the largest multiple of 256
 *   tokens whose buffers fit the workspace given: per token a row of roundup(V, 256) + 64
 *   two-byte entries, the column statistics (8 bytes per 128 entries) and 6 H + 12 bytes.  The
 *   default size is that of blocks which fit 1e9 bytes, 2816 tokens at H = 4096, V = 151936
 *   (0.96 GB), so it does not grow past one block; RLK_ERROR_WORKSPACE when not even 256-token
 *   blocks (at most 1024 of them) fit.
 * A token's logp, lse and dL/dh row are the same bits in any batch, whatever block it falls in;
 * dL/dW is the sum of the blocks' sums in ascending block order.  The size query returns
 * RLK_ERROR_UNSUPPORTED when N would need more than 1024 blocks of the default size. */
rlk_status_t rlk_linear_logp_fwd_bwd_workspace_size(int64_t N, int64_t H, int64_t V, int dtype,
                                                    size_t* bytes);
/* The workspace sets the block size: a larger one than rlk_linear_logp_fwd_bwd_workspace_size
 * buys fewer, larger blocks (at most one for all N tokens), a smaller one trades speed for
 * memory with more, smaller blocks.  This query gives the bytes for blocks of block_tokens
 * tokens (rounded up to 256; 0: the default's blocks; block_tokens >= N: one block), e.g.
 * 3.38 GB for blocks of 9984 tokens at N = 16384, H = 4096, V = 151936 (one block for up to
 * 9984 active tokens), or RLK_ERROR_UNSUPPORTED past 1024 blocks.  logp, lse and dL/dh do not
 * depend on the block size; dL/dW sums the blocks in ascending order, so its rounding does. */
rlk_status_t rlk_linear_logp_fwd_bwd_workspace_size_for_block(int64_t N, int64_t H, int64_t V,
                                                              int dtype, int64_t block_tokens,
                                                              size_t* bytes);
rlk_status_t rlk_linear_logp_fwd_bwd(const void* h, const void* W, const int32_t* targets,
                                     const uint8_t* mask, int64_t N, int64_t H, int64_t V,
                                     int dtype, float temperature, const float* adv, float* logp,
                                     float* lse, float* dh, float* dW, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* rlk_linear_logp_fwd_bwd with an entropy bonus: logp, lse and entropy as
 * rlk_linear_logp_fwd_entropy returns them (the same bits), and the gradients of
 * L = -sum_t mask_t (adv_t logp_t + c_t H_t) as rlk_linear_logp_bwd_entropy defines them, formed
 * from the forward's stored logit codes (the entropy's statistic rides along in the forward;
 * the dz pass adds c_t p (ln p + H_t) / T).
 *   ent_coef [N] float  c_t;   entropy [N] float  out
 *   the rest as for rlk_linear_logp_fwd_bwd; the workspace (and so the token blocks) holds one
 *   more statistic per 128 vocabulary entries: rlk_linear_logp_fwd_bwd_entropy_workspace_size
 *   bytes by default (still 2816 tokens per block at H = 4096, V = 151936). */
rlk_status_t rlk_linear_logp_fwd_bwd_entropy_workspace_size(int64_t N, int64_t H, int64_t V,
                                                            int dtype, size_t* bytes);
rlk_status_t rlk_linear_logp_fwd_bwd_entropy(const void* h, const void* W,
                                             const int32_t* targets, const uint8_t* mask,
                                             int64_t N, int64_t H, int64_t V, int dtype,
                                             float temperature, const float* adv,
                                             const float* ent_coef, float* logp, float* lse,
                                             float* entropy, float* dh, float* dW,
                                             void* workspace, size_t workspace_bytes,
                                             void* stream);

/* rlk_linear_logp_fwd_bwd for the clipped policy-gradient loss with a KL penalty
 * (rlk_ratio_kl_loss), whose gradient depends on the fresh logp: the loss fragment runs after
 * each token block's merge and its -dloss/dlogp drives that block's gradient pass, so one call
 * gives what rlk_linear_logp_fwd, rlk_ratio_kl_loss and rlk_linear_logp_bwd give in sequence
 * (RL-Kernel integration roadmap for vime, "RL Loss Operators": ratio_kl / GRPO / PPO loss
 * fragments fused with linear_logp).
 *   h, W, targets, mask, N, H, V, dtype, temperature: as for rlk_linear_logp_fwd_bwd
 *   old_logp, ref_logp, adv, eps_lo, eps_hi, beta, scale: as for rlk_ratio_kl_loss (ref_logp
 *              may be NULL: no KL term)
 *   logp, lse  out: the forward's bits
 *   loss, bwd_adv, ratio, sums  out: the bits rlk_ratio_kl_loss gives for this logp (ratio and
 *              sums may be NULL)
 *   dh, dW     out: gradients of sum_t loss_t (dL/dlogp_t = -bwd_adv_t), as rlk_linear_logp_fwd_bwd
 *              forms them
 *   workspace: rlk_linear_ppo_fwd_bwd_workspace_size bytes by default, never NULL (the loss
 *              fragment's partial sums, then the fused call's workspace, whose size sets the
 *              token blocks as there). */
rlk_status_t rlk_linear_ppo_fwd_bwd_workspace_size(int64_t N, int64_t H, int64_t V, int dtype,
                                                   size_t* bytes);
rlk_status_t rlk_linear_ppo_fwd_bwd(const void* h, const void* W, const int32_t* targets,
                                    const uint8_t* mask, int64_t N, int64_t H, int64_t V,
                                    int dtype, float temperature, const float* old_logp,
                                    const float* ref_logp, const float* adv, float eps_lo,
                                    float eps_hi, float beta, float scale, float* logp,
                                    float* lse, float* loss, float* bwd_adv, float* ratio,
                                    double* sums, float* dh, float* dW, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* Backward of the policy-gradient loss with an entropy bonus (bf16 only),
 *   L = -sum_t mask_t (adv_t logp_t + c_t H_t)
 * with H_t the entropy of softmax(z[t,:]) (RL-Kernel Roadmap (2026), "operator backlog":
 * fused entropy / entropy-bonus kernel).  dL/dz[t,v] = -adv_t (delta(v, y_t) - p[t,v]) +
 * c_t p[t,v] (log p[t,v] + H_t); the rest is rlk_linear_logp_bwd's chunked walk.
 *   h, W, targets, mask, N, H, V, dtype, temperature, adv, lse, dh, dW, workspace: as for
 *                             rlk_linear_logp_bwd (same workspace size)
 *   ent_coef [N]    float     c_t, the entropy-bonus weight of each token (masked tokens
 *                             ignore it)
 *   entropy  [N]    float     H_t as returned by rlk_linear_logp_fwd_entropy for the same
 *                             inputs (lse likewise)
 * With c = 0 the result equals rlk_linear_logp_bwd's up to the rounding of one extra fma
 * per logit. */
rlk_status_t rlk_linear_logp_bwd_entropy(const void* h, const void* W, const int32_t* targets,
                                         const uint8_t* mask, int64_t N, int64_t H, int64_t V,
                                         int dtype, float temperature, const float* adv,
                                         const float* ent_coef, const float* lse,
                                         const float* entropy, float* dh, float* dW,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* ---- Full-vocabulary KL between a student and a teacher LM head (RL-Kernel Roadmap (2026),
 * operator backlog: chunked full-vocabulary / distillation KL fused with the LM head, forward
 * and reverse, beyond the sampled-token path).
 *   h_s [N,H_s], W_s [V,H_s]   student hidden states and LM head (dtype)
 *   h_t [N,H_t], W_t [V,H_t]   teacher (the same dtype, vocabulary and temperature)
 *   z_s = h_s W_s^T / T, z_t = h_t W_t^T / T, p = softmax(z)
 *   kl_fwd[t] = sum_v p_t (log p_t - log p_s),  kl_rev[t] = sum_v p_s (log p_s - log p_t)
 * at active tokens, 0 elsewhere (both clamped at 0 against rounding).  One tile kernel forms
 * both heads' logits for each 256 x 256 (vocabulary x token) tile, the teacher's first (its
 * fp32 tile waits in a per-work-group scratch slot, never as logits in memory), and pairs them
 * in the student's epilogue into per-column statistics: each head's maximum and sum and the two
 * cross terms; a fixed-order merge per token gives the results.  The active tokens are taken
 * in blocks (compacted order) of the largest multiple of 256 tokens whose statistics fit the
 * workspace given (at most 1024 blocks).  Batch-invariant like logp.  H_s and H_t: multiples
 * of 64; each h at most 2^31 - 1 bytes.
 *   lse_s, lse_t [N] float     out (may be NULL): each head's log-sum-exp, which the backward
 *                              takes back
 *   workspace: rlk_linear_kl_fwd_workspace_size bytes (blocks of the largest multiple of 256
 *              tokens whose six float statistics of ceil(V/128) per token fit 1e9 bytes beside
 *              the 64 MiB scratch: 32512 tokens at V = 151936, so 0.53 GB at N = 16384; past one
 *              block only the 4-byte index per token grows), or
 *              rlk_linear_kl_fwd_workspace_size_for_block bytes for blocks of block_tokens (a
 *              positive multiple of 256): a smaller workspace trades memory for more launches.
 *              RLK_ERROR_WORKSPACE when not even 256-token blocks (within 1024 blocks) fit;
 *              the size queries return RLK_ERROR_UNSUPPORTED past 1024 blocks. */
rlk_status_t rlk_linear_kl_fwd_workspace_size(int64_t N, int64_t H_s, int64_t H_t, int64_t V,
                                              int dtype, size_t* bytes);
rlk_status_t rlk_linear_kl_fwd_workspace_size_for_block(int64_t N, int64_t H_s, int64_t H_t,
                                                        int64_t V, int dtype,
                                                        int64_t block_tokens, size_t* bytes);
rlk_status_t rlk_linear_kl_fwd(const void* h_s, const void* W_s, const void* h_t,
                               const void* W_t, const uint8_t* mask, int64_t N, int64_t H_s,
                               int64_t H_t, int64_t V, int dtype, float temperature,
                               float* kl_fwd, float* kl_rev, float* lse_s, float* lse_t,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Backward of L = sum_t mask_t (coef_fwd_t kl_fwd[t] + coef_rev_t kl_rev[t]) into the student
 * (bf16, H_s a multiple of 256); the teacher is frozen.  Per vocabulary chunk of 32768 entries,
 * the forward's tile kernel forms both heads' logits again and its epilogue writes
 * dL/dz_s = (coef_fwd (p_s - p_t) + coef_rev p_s (log p_s - log p_t - kl_rev)) / T, rounded to
 * bf16; the chunk's dL/dh_s and dL/dW_s follow as in rlk_linear_logp_bwd, over token blocks of
 * the largest multiple of 256 tokens whose buffers fit 1e9 bytes beside the scratch (10240 at
 * H_s = 4096).
 *   coef_fwd, coef_rev [N] float   dL/dkl_fwd and dL/dkl_rev per token; either may be NULL (that
 *                                  term is absent), not both
 *   lse_s, lse_t [N] and (with coef_rev) kl_rev [N]: from rlk_linear_kl_fwd
 *   dh_s [N,H_s], dW_s [V,H_s] float   out, overwritten (dh_s 16-byte aligned)
 *   workspace: rlk_linear_kl_bwd_workspace_size bytes: the backward's buffers for one block and
 *              the 64 MiB scratch (within 1e9 bytes but for the 4-byte index per token). */
rlk_status_t rlk_linear_kl_bwd_workspace_size(int64_t N, int64_t H_s, int64_t H_t, int64_t V,
                                              int dtype, size_t* bytes);
rlk_status_t rlk_linear_kl_bwd(const void* h_s, const void* W_s, const void* h_t,
                               const void* W_t, const uint8_t* mask, int64_t N, int64_t H_s,
                               int64_t H_t, int64_t V, int dtype, float temperature,
                               const float* coef_fwd, const float* coef_rev, const float* lse_s,
                               const float* lse_t, const float* kl_rev, float* dh_s,
                               float* dW_s, void* workspace, size_t workspace_bytes,
                               void* stream);

/* ---- Loss fragments that consume the log-prob (RL-Kernel integration roadmap for vime,
 * "RL Loss Operators: ratio_kl, GRPO/PPO/DPO Loss Fragments": optional fused ratio / KL
 * fragments whose contract states mask handling, aggregation, dtype and reduction order).
 * Every pointer is device memory; all per-token arrays are [N] float32 unless stated. */

/* Per-token clipped policy-gradient loss with a KL penalty towards a reference policy:
 *   r_t   = exp(logp_t - old_logp_t)
 *   pg_t  = max(-A_t r_t, -A_t clip(r_t, 1 - eps_lo, 1 + eps_hi))
 *   kl_t  = exp(d_t) - 1 - d_t with d_t = ref_logp_t - logp_t (the function the pages use
 *           for approx_kl0; a non-negative estimate of KL(policy || reference))
 *   loss_t    = scale * (pg_t + beta * kl_t)                 at active tokens, else 0
 *   bwd_adv_t = -dloss_t/dlogp_t = scale * (A_t r_t [unclipped] - beta (1 - exp(d_t)))
 *               (0 where the clipped term is the larger one), ready to be passed as `adv`
 *               to rlk_linear_logp_bwd, which differentiates -sum adv * logp
 *   ratio_t   = r_t at active tokens, else 0 (ratio may be NULL)
 *   sums      double[4] (may be NULL): sum_t loss_t, the number of clipped tokens,
 *             sum_t kl_t, the number of active tokens
 * ref_logp NULL: no KL term (beta ignored).  The caller owns the aggregation: scale is applied
 * per token (for a token mean pass 1 / number of active tokens).  Per-token values are fp32
 * and depend only on the token's own inputs; the sums are fp64 in a fixed order for a given
 * N.  eps_lo must lie in [0, 1), eps_hi >= 0, beta and scale finite (else INVALID_VALUE).
 * workspace: rlk_ratio_kl_loss_workspace_size bytes (256-byte aligned). */
rlk_status_t rlk_ratio_kl_loss_workspace_size(int64_t N, size_t* bytes);
rlk_status_t rlk_ratio_kl_loss(const float* logp, const float* old_logp, const float* ref_logp,
                               const float* adv, const uint8_t* mask, int64_t N, float eps_lo,
                               float eps_hi, float beta, float scale, float* loss,
                               float* bwd_adv, float* ratio, double* sums, void* workspace,
                               size_t workspace_bytes, void* stream);

/* dlogp diagnostics over the active tokens (vime roadmap, "Consistency Contract", minimum
 * diagnostics), dlogp_t = logp_a_t - logp_b_t formed in fp64:
 *   out[0] active tokens   out[1] mean |dlogp|   out[2] max |dlogp|
 *   out[3..5] 50th, 90th, 99th percentile of |dlogp| (linear interpolation between the
 *             order statistics at floor and ceil of q (n - 1) / 100; the order statistics
 *             are exact, found by radix selection)
 *   out[6] mean ratio0 = exp(dlogp)   out[7] clipfrac0 = fraction with |ratio0 - 1| > clip_eps
 *   out[8] approx_kl0 = mean(exp(dlogp) - 1 - dlogp)
 *   worst: the first token index of largest |dlogp| (-1 when no token is active)
 * With no active token every out[] entry is 0.  out (double[9]) and worst are device
 * memory, written on the stream.  workspace: rlk_dlogp_diagnostics_workspace_size bytes. */
rlk_status_t rlk_dlogp_diagnostics_workspace_size(int64_t N, size_t* bytes);
rlk_status_t rlk_dlogp_diagnostics(const float* logp_a, const float* logp_b,
                                   const uint8_t* mask, int64_t N, float clip_eps, double* out,
                                   int64_t* worst, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* ---- Building blocks of the forward (the same kernels rlk_linear_logp_fwd runs).  They
 * expose the per-vocabulary-slice statistics so that slices computed elsewhere (for
 * example on other devices holding other vocabulary shards) can be merged in a fixed
 * order (vime roadmap, linear_logp "RL-Kernel backend": explicit local max, global max,
 * local sum-exp, global sum-exp, selected target logit and final downcast). */

/* Active-row compaction: idx[0..Na) = the positions t with mask[t] != 0, ascending;
 * *n_active = Na (device int32).  Also sets target_logit[0..N) = NaN and, when logp/lse
 * are non-NULL, writes 0 to logp[t] and lse[t] at inactive t (active entries are left for
 * the merge).  idx [N] int32, n_active [1] int32, target_logit [N] float. */
rlk_status_t rlk_compact_active(const uint8_t* mask, int64_t N, int32_t* idx, int32_t* n_active,
                                float* target_logit, float* logp, float* lse, void* stream);

/* Partial statistics of the compacted rows.  For compacted row i < Na (token idx[i]) and
 * vocabulary column j (entries [128 j, min(V, 128 j + 128))):
 *   part_max[j*N + i] = max_v  z[idx[i], v] * log2(e)
 *   part_sum[j*N + i] = sum_v  2^(z[idx[i], v] * log2(e) - part_max[j*N + i])
 * and target_logit[i] = z[idx[i], y] for the one column that holds y = targets[idx[i]]
 * (left untouched if y is out of range).  part_max and part_sum are
 * [rlk_num_vocab_partials(V), N] float, row stride N. */
rlk_status_t rlk_linear_logp_partials(const void* h, const void* W, const int32_t* targets,
                                      const int32_t* idx, const int32_t* n_active, int64_t N,
                                      int64_t H, int64_t V, int dtype, float temperature,
                                      float* part_max, float* part_sum, float* target_logit,
                                      void* stream);

/* Partial statistics for one vocabulary shard, for vocabulary-parallel scoring (RL-Kernel
 * integration roadmap for vime, "Operator Integration Plan", linear_logp: the hook passes the
 * local vocabulary start and the global vocabulary size, and the backend makes the
 * vocabulary-shard merge of local max, local sum-exp and target logit explicit).
 *   W            [V,H] dtype   rows vocab_start .. vocab_start + V - 1 of the full LM head
 *   vocab_start               global index of W's first row; a multiple of RLK_VOCAB_PARTIAL
 *   V_global                  size of the full vocabulary; vocab_start + V <= V_global, and V
 *                             is a multiple of RLK_VOCAB_PARTIAL unless the shard ends at
 *                             V_global (the last shard)
 *   part_max, part_sum        the full-vocabulary arrays, [rlk_num_vocab_partials(V_global), N]:
 *                             this call writes the shard's columns vocab_start / 128 ..
 *   target_logit [N]          written for tokens whose target lies in this shard, untouched
 *                             for the others (rlk_compact_active sets it to NaN first)
 * Other arguments as for rlk_linear_logp_partials, which is this call with vocab_start = 0
 * and V_global = V.  Once every shard has run (in any order, on any streams ordered before
 * the merge), rlk_linear_logp_merge with V_global gives logp and lse bit-identical to the
 * single-call forward: a column's statistics are the same arithmetic whichever call computes
 * it.  Errors: RLK_ERROR_INVALID_VALUE for a shard outside [0, V_global),
 * RLK_ERROR_UNSUPPORTED for a shard that would split a column. */
rlk_status_t rlk_linear_logp_partials_shard(const void* h, const void* W, const int32_t* targets,
                                            const int32_t* idx, const int32_t* n_active,
                                            int64_t N, int64_t H, int64_t V, int64_t vocab_start,
                                            int64_t V_global, int dtype, float temperature,
                                            float* part_max, float* part_sum,
                                            float* target_logit, void* stream);

/* Fixed-order merge: for i < Na, M = max_j part_max[j*N+i], S = sum_j part_sum[j*N+i] *
 * 2^(part_max[j*N+i] - M) in one fixed association over j = 0..J-1 (J =
 * rlk_num_vocab_partials(V)), lse = (M + log2 S) * ln 2, logp = target_logit[i] - lse;
 * both are written at position idx[i] (lse may be NULL). */
rlk_status_t rlk_linear_logp_merge(const float* part_max, const float* part_sum,
                                   const float* target_logit, const int32_t* idx,
                                   const int32_t* n_active, int64_t N, int64_t V, float* logp,
                                   float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RLK_H_ */
