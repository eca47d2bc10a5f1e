// Backward kernels of the fused linear log-prob: L = -sum_t mask_t adv_t logp_t.
//
// The backward recomputes the logits tile by tile instead of storing them (RL-Kernel
// Roadmap (2026), P0.2: "the backward path recomputes tiles to trade compute for memory
// instead of storing full logits/probabilities"); the only saved state is lse[N].  With
// g_t = -adv_t at active tokens and p = softmax(z_t):
//
//   dL/dz[t,v] = g_t (delta(v, y_t) - p[t,v])
//   dL/dh_t    = (1/T) sum_v dL/dz[t,v] W_v
//   dL/dW_v    = (1/T) sum_t dL/dz[t,v] h_t
//
// With an entropy bonus, L = -sum_t mask_t (adv_t logp_t + c_t H_t) and dL/dz gains
// c_t p[t,v] (log p[t,v] + H_t), the derivative of -c_t H_t = c_t sum_v p log p through the
// softmax; H_t comes from the entropy forward.
//
// The vocabulary is walked in chunks of kBwdChunk entries, in ascending order.  Per chunk:
//   dlogits      the forward tile GEMM again, epilogue G = (g_t / T)(delta - p) rounded to
//                bf16 and stored token-major (Gv);
//   dh_chunk     Gv W[chunk] in K pieces of kDhSplitK entries (fp32 accumulation; two per
//                full chunk): Gv is the first operand, W the second, read as a K-strided
//                panel (rows past V as zeros); a tile is 256 tokens x 256 hidden
//                columns.  Piece q is added to dhp[q] (compacted
//                rows), in chunk order; the pieces are independent tiles, so a chunk fills the
//                machine even when few tokens are active;
//   dw_chunk     dW[chunk rows]^T = hT Gv  (K = the active tokens in ascending order; hT is
//                the first operand, Gv the second, read as a K-strided panel, so a lane's four
//                consecutive accumulator rows are four consecutive hidden columns of one dW row,
//                written 16 bytes at a time).
// dh_chunk and dw_chunk run as the two sections of one launch (grad_chunk_kernel): the
// dL/dW tiles are claimed at run time, so they fill the last round of dL/dh tiles.
// The fused forward + backward has dL/dz of the whole vocabulary in place for a token block at
// once, so there one launch per block covers every column (grad_whole_kernel): dL/dh in two
// pieces, the two halves of the vocabulary (whole_dh_split), each tile summing its whole half,
// and dL/dW over every vocabulary row; the finish then adds the second half to the first.  A
// token's dL/dh is again a sum fixed by V alone (it differs in rounding from the chunked one).
// The active tokens are taken in blocks (compacted order, at most the buffers' capacity, all of
// one size but the last), each block a batch of its own for every kernel here (idx and
// n_active hold the block's indices and count), so the buffers hold one block and the workspace
// stops growing with N.  dh is zeroed once (its inactive rows stay 0).  Per block: hT = the
// block's h rows transposed; per chunk the three steps above, the first chunk's dL/dh tiles
// storing into the token's dh row (piece 0) and the piece buffers and later chunks adding to
// them, the first block's dL/dW tiles storing and later blocks adding; after the last chunk,
// bwd_finish adds the other pieces to dh[idx[m]] in ascending order.  The chunks and
// pieces are build constants, so a token's dh row is the same sum in the same order in every
// batch, whatever block it falls in; dW sums the blocks in ascending order.
#include "common.hpp"
#include "kernels.hpp"
#include "mainloop.hpp"

namespace rlk {

namespace {

// Two floats to packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ---------------------------------------------------------------- transpose of the active h rows

// hT[k][i] = h[idx[i]][k] for i < Na, 0 for Na <= i < Npad.  Grid (Npad / 64, H / 256), four
// waves per work-group, each wave one 64-token x 64-column block.  Lane (tb, kb) = (lane & 7,
// lane >> 3) loads 8 columns of 8 token rows as eight 16-byte vectors, transposes the 8 x 8
// block of bf16 in registers and stores 8 hT rows of 8 tokens: both the loads and the stores
// are 128 contiguous bytes per 8 lanes, with no LDS.
__global__ __launch_bounds__(256) void transpose_h_kernel(BwdArgs a) {
  const int Na = *a.n_active;
  const int lane = threadIdx.x & 63;
  const int tb = lane & 7, kb = lane >> 3;
  const int i0 = blockIdx.x * 64 + 8 * tb;                        // first of this lane's tokens
  const int k0 = blockIdx.y * 256 + (threadIdx.x >> 6) * 64 + 8 * kb;  // first of its columns
  const uint16_t* h = static_cast<const uint16_t*>(a.h);
  u32x4 in[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int i = i0 + q;
    in[q] = u32x4{0u, 0u, 0u, 0u};
    if (i < Na) in[q] = *reinterpret_cast<const u32x4*>(h + (size_t)a.idx[i] * a.H + k0);
  }
#pragma unroll
  for (int p = 0; p < 8; ++p) {  // column k0 + p: element p of every token's vector
    const int sh = 16 * (p & 1);
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {  // tokens 2t (low half) and 2t + 1 (high half)
      const uint32_t lo = (in[2 * t][p >> 1] >> sh) & 0xffffu;
      const uint32_t hi = (in[2 * t + 1][p >> 1] >> sh) & 0xffffu;
      w[t] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4*>(a.hT + (size_t)(k0 + p) * a.Npad + i0) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

__global__ __launch_bounds__(256) void zero_kernel(float* p, size_t n) {
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256)
    p[e] = 0.f;
}

__global__ __launch_bounds__(256) void fill_kernel(float* p, size_t n, float value) {
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256)
    p[e] = value;
}

// ---------------------------------------------------------------- dL/dz from the stored d

// Row m of X holds, for the block's compacted token m, the code c = round(-d 2^9) of every
// entry's d = x - m_col (log2 units, x = z log2 e / T, m_col the maximum of x over the entry's
// 128-entry column, part_max).  With lse in log2 units, log2 p = d + (m_col - lse2), so
//   G[m][v] = (-adv_t / T) (delta(v, y_t) - 2^(-c 2^-9 + m_col - lse2))
// is the dL/dz the dlogits epilogue forms from the recomputed logit, here from the code instead
// (it moves log2 p by at most 2^-10: a relative error of at most 2^-10 ln 2 in p, for every
// entry; the bf16 rounding of G that follows is up to 2^-9).  With an entropy bonus G gains
// (c_t / T) p (ln p + H_t), as in the dlogits epilogue.  Rows of padded token columns
// (Na <= m < the block's 256-token tiles) and the entries past the vocabulary become 0, so the
// GEMMs that read X as dL/dz add nothing for them.  A work-group takes 8192 entries of one row
// (the grid walks (row, segment) pairs): each thread converts four groups of 8 consecutive
// entries, 2048 entries apart, in place, with all four 16-byte loads issued before any result
// is formed.
template <bool kEnt>
__global__ __launch_bounds__(256) void dz_from_d_kernel(DzArgs a) {
  constexpr int kU = 4;                  // 16-byte groups per thread per segment
  constexpr int kSeg = 8 * 256 * kU;     // entries per segment (8192)
  const int Na = *a.n_active;
  const int rows = (Na + kTile - 1) / kTile * kTile;
  const int vr = (a.V + kTile - 1) / kTile * kTile;  // columns the GEMMs may read
  const int nseg = (vr + kSeg - 1) / kSeg;
  const int64_t total = (int64_t)rows * nseg;
  for (int64_t u = blockIdx.x; u < total; u += gridDim.x) {
    const int m = (int)(u / nseg);
    const int s0 = (int)(u - (int64_t)m * nseg) * kSeg + 8 * (int)threadIdx.x;
    uint16_t* row = a.X + (size_t)m * a.pitch;
    if (m >= Na) {  // a padded row of the block's last token tile: zeros
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        const int v0 = s0 + 2048 * k;
        if (v0 < vr) *reinterpret_cast<u32x4*>(row + v0) = u32x4{0u, 0u, 0u, 0u};
      }
      continue;
    }
    const int t = a.idx[m];
    const float gs = -a.adv[t] * a.inv_t;
    const int y = a.targets[t];
    const float lse2 = a.lse[t] * kLog2e;
    const float bs = kEnt ? a.ent_coef[t] * a.inv_t : 0.f;
    const float hn = kEnt ? a.entropy[t] : 0.f;
    // group k: entries v0 .. v0 + 7 (inside one 128-entry column), loaded before any is used
    u32x4 cw[kU];
    float off[kU];
#pragma unroll
    for (int k = 0; k < kU; ++k) {
      const int v0 = s0 + 2048 * k;
      const bool in = v0 < a.V;  // (the quadrant holding v0 was stored: its entries are set)
      cw[k] = in ? *reinterpret_cast<const u32x4*>(row + v0) : u32x4{0u, 0u, 0u, 0u};
      off[k] = in ? a.part_max[(size_t)(v0 / kVocabPartial) * a.pstride + m] - lse2 : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kU; ++k) {
      const int v0 = s0 + 2048 * k;
      if (v0 >= vr) continue;
      float G[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int v = v0 + e;
        const uint32_t c = (cw[k][e >> 1] >> (16 * (e & 1))) & 0xffffu;
        const float xl = __builtin_fmaf((float)c, -1.f / 512.f, off[k]);  // log2 p
        const float pv = __builtin_amdgcn_exp2f(xl);
        float g = gs * ((v == y ? 1.f : 0.f) - pv);
        if constexpr (kEnt) {
          // log p, clamped where p is 0 (underflow) so that 0 * log p = 0
          g = __builtin_fmaf(bs * pv, fmaxf(xl, -126.f) * kLn2 + hn, g);
        }
        G[e] = v < a.V ? g : 0.f;
      }
      u32x4 out;
      out.x = pack_bf16(G[0], G[1]);
      out.y = pack_bf16(G[2], G[3]);
      out.z = pack_bf16(G[4], G[5]);
      out.w = pack_bf16(G[6], G[7]);
      *reinterpret_cast<u32x4*>(row + v0) = out;
    }
  }
}

// ---------------------------------------------------------------- dlogits of one chunk

struct DlogitsCtx {
  int vbase;   // first vocabulary entry of the tile
  int tok[kBlkB];  // compacted token index of each of this lane's four columns
  int tgt[kBlkB];
  float lse2[kBlkB], gs[kBlkB];
  float bs[kBlkB], hn[kBlkB];  // entropy bonus: c_t / T and H_t
};

template <bool kEnt>
__global__ __launch_bounds__(kThreads) void dlogits_kernel(BwdArgs a, int c0) {
  __shared__ RingSmem sm;
  const int Na = *a.n_active;
  const int vc = min(kBwdChunk, a.V - c0);  // vocabulary entries in this chunk
  const int nTokTiles = (Na + kTile - 1) / kTile;
  const int nVocTiles = (vc + kTile - 1) / kTile;
  const int band = nTokTiles <= 12 ? nTokTiles : 8;  // as the forward tile kernel's order
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const size_t row_bytes = (size_t)a.H * 2;
  const int nk = (int)(row_bytes / kKBytes);
  const float c2 = a.inv_t * kLog2e;
  const int wv = wave_a0(wave);
  const int wt = wave_b0(wave);

  auto setup = [&](int u, TileSrc& src, DlogitsCtx& c) {
    int vt, tt;
    tile_coords(u, nVocTiles, nTokTiles, band, vt, tt);
    const int vbase = c0 + vt * kTile;
    const int tbase = tt * kTile;
    src.nk = nk;
    src.a_kstep = src.b_kstep = kKBytes;
    src.a = uniform_ptr(static_cast<const uint8_t*>(a.W) + (size_t)vbase * row_bytes);
    src.b = uniform_ptr(a.h);
    src.a_bytes = operand_bytes((size_t)(a.V - vbase) * row_bytes);
    src.b_bytes = operand_bytes((size_t)a.N * row_bytes);
#pragma unroll
    for (int q = 0; q < kDmaPerWave; ++q) {
      const int r = dma_row(q, wave, lane);
      const int ch = dma_chunk(q, wave, lane);
      const int v = min(vbase + r, a.V - 1);
      const int t = a.idx[min(tbase + r, Na - 1)];
      src.ao[q] = (uint32_t)((size_t)(v - vbase) * row_bytes) + 16 * ch;
      src.bo[q] = (uint32_t)((size_t)t * row_bytes) + 16 * ch;
    }
    c.vbase = vbase;
#pragma unroll
    for (int j = 0; j < kBlkB; ++j) {
      c.tok[j] = tbase + wt + acc_col(j, lane);
      const bool ok = c.tok[j] < Na;
      const int t = ok ? a.idx[c.tok[j]] : 0;
      c.tgt[j] = ok ? a.targets[t] : -1;
      // padded columns: p = 2^(x - inf) = 0 exactly, so G is 0 whatever the logit
      c.lse2[j] = ok ? a.lse[t] * kLog2e : INFINITY;
      c.gs[j] = ok ? -a.adv[t] * a.inv_t : 0.f;
      if constexpr (kEnt) {
        c.bs[j] = ok ? a.ent_coef[t] * a.inv_t : 0.f;
        c.hn[j] = ok ? a.entropy[t] : 0.f;
      }
    }
  };

  // Per block, lane l < 32 holds the rows 8 g + 0..3 of group g and lane l + 32 the rows
  // 8 g + 4..7 (same token).  v_permlane32_swap on the packed groups (2h, 2h + 1) hands lane
  // l the rows 16 h + 0..7 and lane l + 32 the rows 16 h + 8..15, so each store writes 16 B
  // per lane, 32 contiguous bytes per token row.
  //
  // Entry (i, r) of a block sits at row offset ro = 32 i + 8 (r >> 2) + (r & 3) from this
  // lane's first row base.  Every entry takes the non-target form gs (0 - p); the rare
  // blocks that hold some lane's target (a wave-uniform ballot) redo that entry with
  // gs (1 - p), and in the quadrant that reaches past V the entries at ro >= V - base
  // become 0, so the per-entry work is the exponential and one multiply.
  auto epilogue = [&](const DlogitsCtx& c, Acc& acc) {
    const int base = c.vbase + wv + 4 * (lane >> 5);
    const bool tail = __builtin_amdgcn_readfirstlane(c.vbase + wv + kWaveA > a.V ? 1 : 0) != 0;
    const int lim = a.V - base;
#pragma unroll
    for (int j = 0; j < kBlkB; ++j) {
      const int ti = c.tok[j];
      const int dt = c.tgt[j] - base;  // row offset of the target (no entry matches if < 0)
      auto gval = [&](float acc_v, float delta) __attribute__((always_inline)) {
        const float x = acc_v * c2 - c.lse2[j];
        const float p = __builtin_amdgcn_exp2f(x);
        float G = c.gs[j] * (delta - p);
        if constexpr (kEnt) {
          // log p, clamped where p is 0 (underflow, padded columns) so that 0 * log p = 0
          const float lp = fmaxf(x, -126.f) * kLn2;
          G = __builtin_fmaf(c.bs[j] * p, lp + c.hn[j], G);
        }
        return G;
      };
#pragma unroll
      for (int i = 0; i < kBlkA; ++i) {
        const bool hit = __builtin_amdgcn_ballot_w64(dt >= 32 * i && dt < 32 * i + 32) != 0;
        u32x2 pk[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float G[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) G[e] = gval(acc.c[i][j][4 * g + e], 0.f);
          if (hit) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (32 * i + 8 * g + e == dt) G[e] = gval(acc.c[i][j][4 * g + e], 1.f);
          }
          if (tail) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (32 * i + 8 * g + e >= lim) G[e] = 0.f;
          }
          pk[g][0] = pack_bf16(G[0], G[1]);
          pk[g][1] = pack_bf16(G[2], G[3]);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          // lanes 32-63 of x trade places with lanes 0-31 of y:
          // x' = [x lanes 0-31, y lanes 0-31], y' = [x lanes 32-63, y lanes 32-63]
          const auto s0 =
              __builtin_amdgcn_permlane32_swap(pk[2 * h][0], pk[2 * h + 1][0], false, false);
          const auto s1 =
              __builtin_amdgcn_permlane32_swap(pk[2 * h][1], pk[2 * h + 1][1], false, false);
          u32x4 q;
          q.x = s0[0];
          q.y = s1[0];
          q.z = s0[1];
          q.w = s1[1];
          const int vl = c.vbase - c0 + wv + 32 * i + 16 * h + 8 * (lane >> 5);  // first of 8
          *reinterpret_cast<u32x4*>(a.Gv + (size_t)ti * a.gv_pitch + vl) = q;
        }
        // one block at a time: keeps the live ranges short (no spills)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  persistent_tiles<true, DlogitsCtx>(sm, nTokTiles * nVocTiles, setup, epilogue);
}

// ---------------------------------------------------------------- dh += Gv W[chunk]

struct RowColCtx {
  int abase, bbase;  // first A row and first B row of the tile
  int piece;         // dh_chunk: which K piece of the chunk (into dhp[piece])
};

// Exchange of a value with the lane one (dpp_xor1) or two (dpp_xor2) positions away in the
// same group of four lanes (DPP quad permutations [1, 0, 3, 2] and [2, 3, 0, 1]).
__device__ __forceinline__ float dpp_xor1(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
}

// 4 x 4 transpose within each group of four lanes: if lane c of the group holds element e of
// v = M[e][c], it returns M[c][0 .. 3].  Two exchanges: the first swaps the roles of lane
// bit 0 and element bit 0, the second those of lane bit 1 and element bit 1; each lane sends
// the elements it replaces.
__device__ __forceinline__ f32x4 quad_transpose(f32x4 v, int lane) {
  const bool c0 = (lane & 1) != 0;
  const bool c1 = (lane & 2) != 0;
  float s0 = c0 ? v.x : v.y;
  float s1 = c0 ? v.z : v.w;
  s0 = dpp_xor1(s0);
  s1 = dpp_xor1(s1);
  v.x = c0 ? s0 : v.x;
  v.y = c0 ? v.y : s0;
  v.z = c0 ? s1 : v.z;
  v.w = c0 ? v.w : s1;
  float t0 = c1 ? v.x : v.z;
  float t1 = c1 ? v.y : v.w;
  t0 = dpp_xor2(t0);
  t1 = dpp_xor2(t1);
  v.x = c1 ? t0 : v.x;
  v.y = c1 ? t1 : v.y;
  v.z = c1 ? v.z : t0;
  v.w = c1 ? v.w : t1;
  return v;
}

// kFirst: the first chunk, whose tiles store their sums (later chunks add to them).
// kSpread: a last, partial round of tiles is dealt out across the XCDs (for the combined
// launch, whose work-groups go on to claim dL/dW tiles from their XCD's counter).
// kWhole: the whole vocabulary as one chunk (c0 = 0; Gv holds every column), split into the
// pieces whole_dh_split gives; every piece stores its sum.
template <bool kFirst, bool kSpread, bool kWhole = false>
__device__ __forceinline__ void dh_chunk_tiles(RingSmem& sm, const BwdArgs& a, int c0) {
  static_assert(!kWhole || kFirst, "a whole-vocabulary piece is its token's only sum");
  const int Na = *a.n_active;
  const int vc = kWhole ? a.V : min(kBwdChunk, a.V - c0);
  const int kc = (vc + 63) & ~63;  // K extent (zero columns past V)
  const int split = kWhole ? whole_dh_split(a.V) : kDhSplitK;
  const int npiece = (kc + split - 1) / split;
  const int nTokTiles = (Na + kTile - 1) / kTile;
  const int nHTiles = a.H / kTile;
  const int per_piece = nTokTiles * nHTiles;
  const int band = nHTiles < 8 ? nHTiles : 8;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const size_t g_row = (size_t)a.gv_pitch * 2;  // bytes per Gv row (one token)
  const size_t gcol = a.gv_full ? (size_t)c0 : 0;  // the chunk's first column in a Gv row
  const uint32_t w_pitch = (uint32_t)a.H * 2;  // bytes per W row
  const int wa = wave_a0(wave);
  const int wb = wave_b0(wave);

  // A = Gv rows of tokens abase .. (K = the piece's vocabulary entries, contiguous), B =
  // W[c0 + k0 ..][hidden columns bbase ..] read K-strided (a transposing panel, rows past V as
  // zeros).  W is the operand with the transposing reads, so each wave reads it for its 64
  // hidden columns (two 32-column blocks) rather than 128.
  auto setup = [&](int u, TileSrc& src, RowColCtx& c) {
    const int piece = u / per_piece;
    int tt, ht;
    tile_coords(u - piece * per_piece, nTokTiles, nHTiles, band, tt, ht);
    c.abase = tt * kTile;
    c.bbase = ht * kTile;
    c.piece = piece;
    const int k0 = piece * split;  // K entries [k0, k1) of this piece
    const int k1 = min(kc, k0 + split);
    src.nk = (k1 - k0) * 2 / kKBytes;
    src.a_kstep = kKBytes;
    src.b_kstep = 64 * w_pitch;  // 64 W rows per stage
    const size_t v0 = (size_t)c0 + k0;
    src.a = uniform_ptr(reinterpret_cast<const uint8_t*>(a.Gv) + (size_t)c.abase * g_row +
                        2 * (gcol + k0));
    src.b = uniform_ptr(static_cast<const uint8_t*>(a.W) + v0 * w_pitch + 2 * (size_t)c.bbase);
    src.a_bytes = operand_bytes((size_t)(a.Npad - c.abase) * g_row - 2 * (gcol + k0));
    src.b_bytes = operand_bytes(((size_t)a.V - v0) * w_pitch - 2 * (size_t)c.bbase);
#pragma unroll
    for (int q = 0; q < kDmaPerWave; ++q) {
      src.ao[q] = (uint32_t)(dma_row(q, wave, lane) * g_row) + 16 * dma_chunk(q, wave, lane);
      src.bo[q] = (uint32_t)(tdma_row(q, wave, lane) * w_pitch) + 16 * tdma_chunk(q, wave, lane);
    }
  };

  // Accumulator rows are tokens, columns hidden entries.  Register group g of block (i, j)
  // holds four consecutive token rows of the lane's hidden column; a transpose within each
  // group of four lanes gives lane e of the group token row e of that group and the group's
  // four consecutive hidden columns, added into the token's row 16 bytes at a time.  Piece 0
  // accumulates in dh's own row of the token (idx[m]); every later piece in the token's
  // compacted row of dhp[piece].  Every row starts 16-byte aligned: dh and the 256-byte
  // aligned dhp buffers are 16-byte aligned and H % 256 == 0.
  //
  // The piece's buffer is chosen once per tile, in wave-uniform code before the per-lane
  // branch: chosen inside it (a nested select under a divergent mask, with four pieces), this
  // compiler sent piece 3's stores of half the lanes to piece 1's buffer.
  auto epilogue = [&](const RowColCtx& c, Acc& acc) {
    static_assert(kDhPieces >= 1 && kDhPieces <= 4, "piece buffers");
    float* base = a.dh;
#pragma unroll
    for (int q = 1; q < kDhPieces; ++q) base = c.piece == q ? a.dhp[q] : base;
    const bool in_dh = c.piece == 0;
    const int col = c.bbase + wb + 4 * ((lane & 31) >> 2);
#pragma unroll
    for (int i = 0; i < kBlkA; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 t[kBlkB];
#pragma unroll
        for (int j = 0; j < kBlkB; ++j) {
          f32x4 v;
          v.x = acc.c[i][j][4 * g + 0];
          v.y = acc.c[i][j][4 * g + 1];
          v.z = acc.c[i][j][4 * g + 2];
          v.w = acc.c[i][j][4 * g + 3];
          t[j] = quad_transpose(v, lane);
        }
        const int m = c.abase + wa + acc_row(i, 4 * g + (lane & 3), lane);
        if (m < Na) {
          const size_t r = in_dh ? (size_t)a.idx[m] : (size_t)m;
          float* row = base + r * a.H + col;
#pragma unroll
          for (int j = 0; j < kBlkB; ++j) {
            f32x4* p = reinterpret_cast<f32x4*>(row + 32 * j);
            f32x4 v = kFirst ? f32x4{0.f, 0.f, 0.f, 0.f} : *p;
            v.x += t[j].x;
            v.y += t[j].y;
            v.z += t[j].z;
            v.w += t[j].w;
            *p = v;
          }
        }
      }
  };

  persistent_tiles<true, RowColCtx, false, true, kSpread>(sm, per_piece * npiece, setup, epilogue);
}

// dh[idx[m]] = (dh[idx[m]] + dhp[1][m]) + ... + dhp[kP-1][m] over the kP pieces the first
// chunk has (every later chunk has at most as many, and adds to them; the others were never
// written), piece 0 being the sum dh[idx[m]] already holds.  A work-group walks rows
// m = blockIdx.x, blockIdx.x + gridDim.x, ...; its threads take 4 consecutive entries at a time.
template <int kP>
__global__ __launch_bounds__(256) void dh_finish_kernel(BwdArgs a) {
  const int Na = *a.n_active;
  const int h4 = a.H / 4;
  for (int m = blockIdx.x; m < Na; m += gridDim.x) {
    f32x4* out = reinterpret_cast<f32x4*>(a.dh + (size_t)a.idx[m] * a.H);
    for (int k = threadIdx.x; k < h4; k += 256) {
      f32x4 v = out[k];
#pragma unroll
      for (int q = 1; q < kP; ++q) {
        const f32x4 w = reinterpret_cast<const f32x4*>(a.dhp[q] + (size_t)m * a.H)[k];
        v.x += w.x;
        v.y += w.y;
        v.z += w.z;
        v.w += w.w;
      }
      out[k] = v;
    }
  }
}

// ---------------------------------------------------------------- dW rows = Gv^T hT^T

// kClaimed: tiles claimed from the XCD counters in a.sched (claimed_tiles) instead of the fixed
// order.  kAccum: a later token block, whose sums are added to the dL/dW rows the earlier blocks
// stored (the first block stores, so dW is the blocks' sums in ascending block order); an empty
// later block changes nothing and returns at once.
// kWhole: every vocabulary row (c0 = 0; Gv holds every column).
template <bool kClaimed, bool kAccum, bool kWhole = false>
__device__ __forceinline__ void dw_chunk_tiles(RingSmem& sm, const BwdArgs& a, int c0) {
  const int Na = *a.n_active;
  if (kAccum && Na == 0) return;
  const int vc = kWhole ? a.V : min(kBwdChunk, a.V - c0);
  const int nVocTiles = (vc + kTile - 1) / kTile;
  const int nHTiles = a.H / kTile;
  const int band = nVocTiles < 8 ? nVocTiles : 8;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const size_t row_bytes = (size_t)a.Npad * 2;         // hT rows
  const uint32_t g_pitch = (uint32_t)a.gv_pitch * 2;  // Gv rows (one token each)
  const size_t gcol = a.gv_full ? (size_t)c0 : 0;      // the chunk's first column in a Gv row
  const int nk = ((Na + 63) & ~63) * 2 / kKBytes;
  const int wa = wave_a0(wave);
  const int wb = wave_b0(wave);

  // A = hT rows of hidden columns abase .. (K = the block's tokens, contiguous), B = the chunk's
  // dL/dz columns bbase .. read K-strided from the token-major Gv (a transposing panel).
  auto setup = [&](int u, TileSrc& src, RowColCtx& c) {
    int ht, vt;
    tile_coords(u, nHTiles, nVocTiles, band, ht, vt);
    c.abase = ht * kTile;
    c.bbase = vt * kTile;  // within the chunk
    c.piece = 0;
    src.nk = nk;
    src.a_kstep = kKBytes;
    src.b_kstep = 64 * g_pitch;  // 64 token rows of Gv per stage
    src.a = uniform_ptr(reinterpret_cast<const uint8_t*>(a.hT) + (size_t)c.abase * row_bytes);
    src.b = uniform_ptr(reinterpret_cast<const uint8_t*>(a.Gv) + 2 * (gcol + c.bbase));
    src.a_bytes = operand_bytes((size_t)(a.H - c.abase) * row_bytes);
    src.b_bytes = operand_bytes((size_t)a.Npad * g_pitch - 2 * (gcol + c.bbase));
#pragma unroll
    for (int q = 0; q < kDmaPerWave; ++q) {
      src.ao[q] = (uint32_t)((size_t)dma_row(q, wave, lane) * row_bytes) + 16 * dma_chunk(q, wave, lane);
      src.bo[q] = (uint32_t)(tdma_row(q, wave, lane) * g_pitch) + 16 * tdma_chunk(q, wave, lane);
    }
  };

  // Accumulator rows are hidden columns, columns are vocabulary rows: a lane holds 4
  // consecutive hidden columns of its vocabulary row per register group and writes them 16 bytes
  // at a time (dW rows start 16-byte aligned: H % 256 == 0; the whole-row offset keeps dW's own
  // alignment, which is checked).  A later block adds to the stored rows, its old values loaded
  // (per vocabulary column of the wave) before any is added and stored back.
  auto epilogue = [&](const RowColCtx& c, Acc& acc) {
#pragma unroll
    for (int j = 0; j < kBlkB; ++j) {
      const int v = c0 + c.bbase + wb + acc_col(j, lane);
      if (v < a.V) {
        float* row = a.dW + (size_t)v * a.H + c.abase + wa;
        f32x4 old[kBlkA][4];
        if constexpr (kAccum) {
#pragma unroll
          for (int i = 0; i < kBlkA; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g)
              old[i][g] = *reinterpret_cast<const f32x4*>(row + acc_row(i, 4 * g, lane));
        }
#pragma unroll
        for (int i = 0; i < kBlkA; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 x;
            x.x = acc.c[i][j][4 * g + 0];
            x.y = acc.c[i][j][4 * g + 1];
            x.z = acc.c[i][j][4 * g + 2];
            x.w = acc.c[i][j][4 * g + 3];
            if constexpr (kAccum) {
              x.x += old[i][g].x;
              x.y += old[i][g].y;
              x.z += old[i][g].z;
              x.w += old[i][g].w;
            }
            *reinterpret_cast<f32x4*>(row + acc_row(i, 4 * g, lane)) = x;
          }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if constexpr (kClaimed)
    claimed_tiles<true, RowColCtx, false, true>(sm, nVocTiles * nHTiles, a.sched, setup, epilogue);
  else
    persistent_tiles<true, RowColCtx, false, true>(sm, nVocTiles * nHTiles, setup, epilogue);
}

template <bool kFirst>
__global__ __launch_bounds__(kThreads) void dh_chunk_kernel(BwdArgs a, int c0) {
  __shared__ RingSmem sm;
  dh_chunk_tiles<kFirst, false>(sm, a, c0);
}

template <bool kAccum>
__global__ __launch_bounds__(kThreads) void dw_chunk_kernel(BwdArgs a, int c0) {
  __shared__ RingSmem sm;
  dw_chunk_tiles<false, kAccum>(sm, a, c0);
}

// Both GEMMs of a chunk in one launch: each work-group first takes its dL/dh tiles in the
// fixed order (a partial last round spread over the XCDs), then claims dL/dW tiles
// (claim_tile) until none are left, so the work-groups that got one dL/dh tile fewer fill the
// last round of dL/dh with dL/dW tiles.  The two are independent (both read Gv; dL/dh writes
// dhp, dL/dW writes dW), and which work-group computes a tile changes no result: the
// separate launches give the same bits.
template <bool kFirst, bool kAccum>
__global__ __launch_bounds__(kThreads) void grad_chunk_kernel(BwdArgs a, int c0) {
  __shared__ RingSmem sm;
  dh_chunk_tiles<kFirst, true>(sm, a, c0);
  dw_chunk_tiles<true, kAccum>(sm, a, c0);
}

// The same for the whole vocabulary at once, when Gv holds every column (the fused forward +
// backward): the dL/dh tiles of the whole-vocabulary pieces, then claimed dL/dW tiles of every
// vocabulary row.  One launch per token block instead of one per chunk, so a block has one
// partial last round instead of one per chunk.
template <bool kAccum>
__global__ __launch_bounds__(kThreads) void grad_whole_kernel(BwdArgs a) {
  __shared__ RingSmem sm;
  dh_chunk_tiles<true, true, true>(sm, a, 0);
  dw_chunk_tiles<true, kAccum, true>(sm, a, 0);
}

}  // namespace

hipError_t launch_zero(float* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int zb = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  hipLaunchKernelGGL(zero_kernel, dim3(zb), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_fill(float* p, size_t n, float value, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int zb = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  hipLaunchKernelGGL(fill_kernel, dim3(zb), dim3(256), 0, stream, p, n, value);
  return hipGetLastError();
}

hipError_t launch_dz_from_d(const DzArgs& a, hipStream_t stream) {
  if (a.ent_coef)
    hipLaunchKernelGGL(dz_from_d_kernel<true>, dim3(4096), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(dz_from_d_kernel<false>, dim3(4096), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_transpose(const BwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(transpose_h_kernel, dim3(a.Npad / 64, a.H / 256), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// The combined launch for token blocks of at most this many tokens.  There the GEMMs have few tiles per chunk (at 2053 active
// tokens, 576 dL/dh tiles: 2.25 rounds of 256 work-groups) and the combined launch made the
// backward 6% faster; with all of 9831 active tokens in one pass it was ~1% slower than two
// launches: the chip is at its power limit there, and dL/dW tiles started at staggered times
// share fewer L2 panels.  A scheduling choice only: the bits are the same.
constexpr int64_t kCombinedMaxTokens = 4096;

template <bool kFirst, bool kAccum>
static void launch_two(const BwdArgs& a, int c0, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(dh_chunk_kernel<kFirst>, dim3(grid), dim3(kThreads), 0, stream, a, c0);
  hipLaunchKernelGGL(dw_chunk_kernel<kAccum>, dim3(grid), dim3(kThreads), 0, stream, a, c0);
}

static hipError_t launch_grad_chunk(const BwdArgs& a, int c0, int grid, bool accum_dw,
                                    hipStream_t stream) {
  const bool first = c0 == 0;
  // The ragged last chunk (20864 entries of the Qwen3-8B vocabulary) takes the combined launch
  // at any block size: its dL/dh pieces have unequal K (16384 and 4480 entries), and the claimed
  // dL/dW tiles fill the work-groups that drew short pieces (0.3 ms per step at 9831 tokens).
  if (a.Npad <= kCombinedMaxTokens || a.V - c0 < kBwdChunk) {
    hipError_t e = launch_zero(reinterpret_cast<float*>(a.sched), 8, stream);  // claim counters
    if (e != hipSuccess) return e;
    auto k = first ? (accum_dw ? grad_chunk_kernel<true, true> : grad_chunk_kernel<true, false>)
                   : (accum_dw ? grad_chunk_kernel<false, true> : grad_chunk_kernel<false, false>);
    hipLaunchKernelGGL(k, dim3(grid), dim3(kThreads), 0, stream, a, c0);
  } else if (first) {
    if (accum_dw) launch_two<true, true>(a, c0, grid, stream);
    else launch_two<true, false>(a, c0, grid, stream);
  } else {
    if (accum_dw) launch_two<false, true>(a, c0, grid, stream);
    else launch_two<false, false>(a, c0, grid, stream);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_chunk(const BwdArgs& a, int chunk, int grid, bool accum_dw,
                            hipStream_t stream) {
  const int c0 = chunk * kBwdChunk;
  if (a.ent_coef)
    hipLaunchKernelGGL(dlogits_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, a, c0);
  else
    hipLaunchKernelGGL(dlogits_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, a, c0);
  return launch_grad_chunk(a, c0, grid, accum_dw, stream);
}

hipError_t launch_bwd_chunk_gemms(const BwdArgs& a, int chunk, int grid, bool accum_dw,
                                  hipStream_t stream) {
  const int c0 = chunk * kBwdChunk;
  return launch_grad_chunk(a, c0, grid, accum_dw, stream);
}

hipError_t launch_bwd_whole_gemms(const BwdArgs& a, int grid, bool accum_dw, hipStream_t stream) {
  if (!a.gv_full) return hipErrorInvalidValue;
  hipError_t e = launch_zero(reinterpret_cast<float*>(a.sched), 8, stream);  // claim counters
  if (e != hipSuccess) return e;
  if (accum_dw)
    hipLaunchKernelGGL(grad_whole_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(grad_whole_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_finish_whole(const BwdArgs& a, hipStream_t stream) {
  const int kc = (a.V + 63) / 64 * 64;
  const int split = whole_dh_split(a.V);
  if ((kc + split - 1) / split == 2)
    hipLaunchKernelGGL(dh_finish_kernel<2>, dim3(2048), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_finish(const BwdArgs& a, hipStream_t stream) {
  const int kc0 = ((a.V < kBwdChunk ? a.V : kBwdChunk) + 63) / 64 * 64;  // first chunk's K extent
  const int pieces = (kc0 + kDhSplitK - 1) / kDhSplitK;
  // one piece: dh holds the result already
  if (pieces == 2)
    hipLaunchKernelGGL(dh_finish_kernel<2>, dim3(2048), dim3(256), 0, stream, a);
  if constexpr (kDhPieces >= 3) {
    if (pieces == 3) hipLaunchKernelGGL(dh_finish_kernel<3>, dim3(2048), dim3(256), 0, stream, a);
  }
  if constexpr (kDhPieces >= 4) {
    if (pieces >= 4) hipLaunchKernelGGL(dh_finish_kernel<4>, dim3(2048), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace rlk
