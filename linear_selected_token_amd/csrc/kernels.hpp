// Kernel argument blocks and launchers (host-visible, internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlk {

constexpr int kVocabPartial = 128;  // vocabulary entries per partial-statistics column
// Vocabulary entries per backward chunk, and per dL/dh piece of a chunk (build constants; a
// token's dL/dh bits depend on them, never on N).
#define RLK_BWD_CHUNK 32768
#define RLK_DH_SPLIT 16384
constexpr int kBwdChunk = RLK_BWD_CHUNK;  // vocabulary entries per backward chunk
constexpr int kDhSplitK = RLK_DH_SPLIT;   // dL/dh sums each piece of a chunk apart
constexpr int kDhPieces = kBwdChunk / kDhSplitK;  // pieces of a full chunk
// dL/dh pieces when one launch covers the whole vocabulary (the fused forward + backward, whose
// dL/dz buffer holds every column): the K extent (V rounded up to 64) in two halves, each
// rounded up to 64 entries (one piece when that covers it).  A rule of V alone, so a token's
// dL/dh bits never depend on the batch; two pieces put the same K on a tile's critical path as
// the chunked pieces (half the vocabulary).
__host__ __device__ constexpr int whole_dh_split(int V) {
  return (((V + 63) / 64 * 64) / 2 + 63) / 64 * 64;
}
static_assert(kDhPieces >= 2, "the whole-vocabulary split needs the second piece buffer");
// The backward (and the KL paths) take the active tokens in blocks of at most a capacity the
// host derives from H (a multiple of 256, at most 65536), in compacted order: its buffers hold
// one block, so the workspace does not grow past that many tokens.
// Row pitch (entries) of the token-major chunk buffers: the chunk plus 128 bytes, so that the
// rows a wave writes at once (32 tokens) do not all start at the same 64 KiB-aligned offset.
constexpr int kGvPitch = kBwdChunk + 64;  // bf16 dL/dz

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
  // Token blocks of at most block_cap compacted indices (block_cap a multiple of 256), for
  // nblk blocks (the host's bound, at most 1024):
  //   block_count [nblk]     fixed blocks b * block_cap ...: active tokens of each (may be null)
  //   block_desc  [nblk][2]  balanced blocks (count, first compacted index): the active tokens
  //                          cut into ceil(Na / block_cap) blocks of one size, a multiple of 256
  //                          but for the last (may be null)
  int32_t* block_count = nullptr;
  int32_t* block_desc = nullptr;
  int nblk = 0;
  int block_cap = 0;
};

// Copies block b of the balanced partition: bidx[0 .. count) = idx[first ..], *bn = count.
hipError_t launch_select_block(const int32_t* idx, const int32_t* desc, int b, int cap,
                               int32_t* bidx, int32_t* bn, hipStream_t stream);

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
  int pstride = 0;          // column stride of part_max / part_sum / part_w (0: N)
  uint16_t* dbuf = nullptr; // [rows][d_pitch] 16-bit code of d = x - column max (kFwdStoreD)
  int d_pitch = 0;          // entries per dbuf row
};

enum FwdMode { kFwdPlain = 0, kFwdEntropy = 1, kFwdStoreD = 3, kFwdStoreDEnt = 4 };

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
  uint16_t* Gv;           // [Npad, gv_pitch] dL/dz of the chunk, token-major
  float* dhp[kDhPieces];  // [Npad, H] each for q >= 1: dL/dh from piece q of every chunk,
                          // compacted rows; piece 0 accumulates in place in dh's own rows
  int* sched;             // [8] tile-claim counters of the dL/dW section (zeroed per launch)
  // A token block: idx and n_active hold the block's compacted indices and its count (at most
  // Npad), so every kernel sees the block as a batch of its own.
  // entropy bonus (both null without it): L gains -sum_t mask_t c_t H_t
  const float* ent_coef = nullptr;  // [N] c_t
  const float* entropy = nullptr;   // [N] H_t from the entropy forward
  int gv_pitch = kGvPitch;  // entries per Gv row
  // false: a Gv row holds one chunk (entry v - c0 of the chunk at c0); true: the whole
  // vocabulary (entry v), so the chunk at c0 starts at column c0 of every row
  bool gv_full = false;
};

// dL/dz of a token block from its stored d (fwd tiles in kFwdStoreD), in place: the 16-bit
// codes of X become bf16 dL/dz, with zeros in the padded rows and past the vocabulary.
struct DzArgs {
  uint16_t* X;             // [rows][pitch]
  int pitch;               // entries per row
  const float* part_max;   // [J][pstride] column maxima (log2 units) of the block's tokens
  int pstride;
  const int32_t* idx;      // the block's compacted indices (positions in [0, N))
  const int32_t* n_active; // the block's token count
  const int32_t* targets;  // [N]
  const float* adv;        // [N]
  const float* lse;        // [N] natural-log lse, written by the merge
  int V;
  float inv_t;
  // entropy bonus (both null without it): dL/dz gains c_t p (ln p + H_t)
  const float* ent_coef = nullptr;  // [N] c_t
  const float* entropy = nullptr;   // [N] H_t, written by the merge
};

hipError_t launch_compact(const CompactArgs& a, hipStream_t stream);
hipError_t launch_fwd_tiles(const FwdTileArgs& a, bool bf16, int grid, hipStream_t stream,
                            int mode);
hipError_t launch_fwd_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_logits_logp(const LogitsArgs& a, bool bf16, hipStream_t stream);

// Backward phases.
hipError_t launch_zero(float* p, size_t n, hipStream_t stream);
hipError_t launch_bwd_transpose(const BwdArgs& a, hipStream_t stream);  // hT of the block
// accum_dw: add the block's dL/dW to what earlier blocks stored (the first block stores)
hipError_t launch_bwd_chunk(const BwdArgs& a, int chunk, int grid, bool accum_dw,
                            hipStream_t stream);
// dL/dh and dL/dW of one chunk from a Gv written elsewhere
hipError_t launch_bwd_chunk_gemms(const BwdArgs& a, int chunk, int grid, bool accum_dw,
                                  hipStream_t stream);
hipError_t launch_bwd_finish(const BwdArgs& a, hipStream_t stream);  // dh[idx] = sum of pieces
// With Gv holding every column (gv_full): dL/dh and dL/dW of the whole vocabulary in one launch,
// dL/dh in the whole_dh_split pieces; then their sum into dh[idx].
hipError_t launch_bwd_whole_gemms(const BwdArgs& a, int grid, bool accum_dw, hipStream_t stream);
hipError_t launch_bwd_finish_whole(const BwdArgs& a, hipStream_t stream);
hipError_t launch_fill(float* p, size_t n, float value, hipStream_t stream);
hipError_t launch_dz_from_d(const DzArgs& a, hipStream_t stream);

}  // namespace rlk
