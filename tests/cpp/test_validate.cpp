// Host-side argument checks and workspace layouts of the C ABI (csrc/validate.hpp), compiled
// for the CPU alone and run under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_validate_cpp.py.  Every status path of every check, the layouts' alignment and
// disjointness, and the arithmetic at the size limits (N and V at 2^22, H at 2^16, h at
// 2^31 - 1 bytes), where a 32-bit intermediate or a size_t wrap would show.
//
// The checks only compare pointer values (null, alignment); they never dereference them, so
// the pointers below are plain numbers with the wanted alignment.
#include <cmath>
#include <cstdint>
#include <algorithm>
#include <cstdio>
#include <limits>
#include <vector>

#include "validate.hpp"

using namespace rlk;

static int g_fail = 0;
static int g_checks = 0;

#define EXPECT(cond)                                                          \
  do {                                                                        \
    ++g_checks;                                                               \
    if (!(cond)) {                                                            \
      ++g_fail;                                                               \
      std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
    }                                                                         \
  } while (0)

static const void* P(uintptr_t v) { return reinterpret_cast<const void*>(v); }
template <class T>
static T* PT(uintptr_t v) { return reinterpret_cast<T*>(v); }

// 256-byte aligned stand-ins, and one that is only 2-byte aligned
constexpr uintptr_t A = 0x10000;
constexpr uintptr_t ODD = 0x10002;

static void test_shape() {
  EXPECT(check_shape(16, 4096, 151936, RLK_BF16) == RLK_SUCCESS);
  EXPECT(check_shape(0, 64, 1, RLK_FP32) == RLK_SUCCESS);
  EXPECT(check_shape(-1, 64, 10, RLK_BF16) == RLK_ERROR_INVALID_VALUE);
  EXPECT(check_shape(1, 0, 10, RLK_BF16) == RLK_ERROR_INVALID_VALUE);
  EXPECT(check_shape(1, -64, 10, RLK_BF16) == RLK_ERROR_INVALID_VALUE);
  EXPECT(check_shape(1, 64, 0, RLK_BF16) == RLK_ERROR_INVALID_VALUE);
  EXPECT(check_shape(1, 64, 10, 2) == RLK_ERROR_UNSUPPORTED);
  EXPECT(check_shape(1, 64, 10, -1) == RLK_ERROR_UNSUPPORTED);
  EXPECT(check_shape(1, 96, 10, RLK_BF16) == RLK_ERROR_UNSUPPORTED);  // H % 64
  // the size limits, at and one past
  EXPECT(check_shape(1, 64, kMaxVocab, RLK_BF16) == RLK_SUCCESS);
  EXPECT(check_shape(1, 64, kMaxVocab + 1, RLK_BF16) == RLK_ERROR_UNSUPPORTED);
  EXPECT(check_shape(1, kMaxHidden, 10, RLK_BF16) == RLK_SUCCESS);
  EXPECT(check_shape(1, kMaxHidden + 64, 10, RLK_BF16) == RLK_ERROR_UNSUPPORTED);
  EXPECT(check_shape(kMaxTokens + 1, 64, 10, RLK_BF16) == RLK_ERROR_UNSUPPORTED);
  // h at most 2^31 - 1 bytes: 2^22 - 1 tokens x 256 bf16 = 2^31 - 512 bytes fits, 2^22 does not
  EXPECT(check_shape(kMaxTokens - 1, 256, 10, RLK_BF16) == RLK_SUCCESS);
  EXPECT(check_shape(kMaxTokens, 256, 10, RLK_BF16) == RLK_ERROR_UNSUPPORTED);
  EXPECT(check_shape(kMaxTokens - 1, 128, 10, RLK_FP32) == RLK_SUCCESS);
  EXPECT(check_shape(kMaxTokens, 128, 10, RLK_FP32) == RLK_ERROR_UNSUPPORTED);
  // the largest N x H products stay exact in 64 bits
  EXPECT(check_shape(kMaxTokens, kMaxHidden, kMaxVocab, RLK_FP32) == RLK_ERROR_UNSUPPORTED);
  EXPECT(check_shape(int64_t(1) << 40, 64, 10, RLK_BF16) == RLK_ERROR_UNSUPPORTED);
  EXPECT(check_shape(std::numeric_limits<int64_t>::max(), 64, 10, RLK_BF16) ==
         RLK_ERROR_UNSUPPORTED);
}

static void test_shard() {
  EXPECT(check_shard(151936, 0, 151936) == RLK_SUCCESS);
  EXPECT(check_shard(1024, 128, 151936) == RLK_SUCCESS);
  EXPECT(check_shard(128, 151936 - 128, 151936) == RLK_SUCCESS);
  EXPECT(check_shard(100, 151936 - 100, 151936) == RLK_ERROR_UNSUPPORTED);  // start off-column
  EXPECT(check_shard(1000, 151936 - 1000 - 24, 151936) == RLK_ERROR_UNSUPPORTED);
  EXPECT(check_shard(200, 0, 151936) == RLK_ERROR_UNSUPPORTED);  // ends inside a column
  EXPECT(check_shard(200, 0, 200) == RLK_SUCCESS);                // ... unless it is the last
  EXPECT(check_shard(10, -128, 151936) == RLK_ERROR_INVALID_VALUE);
  EXPECT(check_shard(256, 151936 - 128, 151936) == RLK_ERROR_INVALID_VALUE);
  EXPECT(check_shard(10, 0, 0) == RLK_ERROR_INVALID_VALUE);
  EXPECT(check_shard(128, 0, kMaxVocab + 1) == RLK_ERROR_UNSUPPORTED);
}

static void test_temperature() {
  EXPECT(check_temperature(1.0f) == RLK_SUCCESS);
  EXPECT(check_temperature(0.7f) == RLK_SUCCESS);
  EXPECT(check_temperature(std::numeric_limits<float>::max()) == RLK_SUCCESS);
  EXPECT(check_temperature(0.f) == RLK_ERROR_INVALID_VALUE);
  EXPECT(check_temperature(-0.f) == RLK_ERROR_INVALID_VALUE);
  EXPECT(check_temperature(-1.f) == RLK_ERROR_INVALID_VALUE);
  EXPECT(check_temperature(std::nanf("")) == RLK_ERROR_INVALID_VALUE);
  EXPECT(check_temperature(std::numeric_limits<float>::infinity()) == RLK_ERROR_INVALID_VALUE);
  // 1/T overflows fp32 for the smallest positive floats
  EXPECT(check_temperature(std::numeric_limits<float>::denorm_min()) == RLK_ERROR_INVALID_VALUE);
  EXPECT(check_temperature(1e-39f) == RLK_ERROR_INVALID_VALUE);
}

// Offsets of a layout's pieces: each 256-byte aligned, in order, each past the previous piece's
// end, and the total past the last one.
static void expect_layout(const std::vector<size_t>& off, const std::vector<size_t>& size,
                          size_t total) {
  size_t end = 0;
  for (size_t i = 0; i < off.size(); ++i) {
    EXPECT(off[i] % 256 == 0);
    EXPECT(off[i] >= end);
    EXPECT(off[i] + size[i] >= off[i]);  // no wrap
    end = off[i] + size[i];
  }
  EXPECT(total >= end);
  EXPECT(total % 256 == 0);
}

static void test_fwd_layout(int64_t N, int64_t V, bool ent) {
  const FwdLayout L = fwd_layout(N, V, ent);
  const size_t n = (size_t)(N > 0 ? N : 1), j = (size_t)num_partials(V);
  std::vector<size_t> off = {L.idx, L.n_active, L.target_logit, L.part_max, L.part_sum};
  std::vector<size_t> sz = {4 * n, 4, 4 * n, 4 * n * j, 4 * n * j};
  if (ent) {
    off.push_back(L.part_w);
    sz.push_back(4 * n * j);
  }
  expect_layout(off, sz, L.total);
}

static void test_layouts() {
  for (int64_t N : {int64_t(0), int64_t(1), int64_t(255), int64_t(16384), kMaxTokens})
    for (int64_t V : {int64_t(1), int64_t(1000), int64_t(151936), kMaxVocab}) {
      test_fwd_layout(N, V, false);
      test_fwd_layout(N, V, true);
    }
  EXPECT(num_partials(0) == 0 && num_partials(1) == 1 && num_partials(128) == 1 &&
         num_partials(129) == 2 && num_partials(151936) == 1187);
  // at the limits the forward's workspace is 2^40 bytes and more: exact in size_t
  EXPECT(fwd_layout(kMaxTokens, kMaxVocab).part_sum == fwd_layout(kMaxTokens, kMaxVocab).part_max +
                                                            (size_t(4) << 37));
  for (int64_t N : {int64_t(1), int64_t(300), int64_t(4096), int64_t(16384), kMaxTokens})
    for (int64_t H : {int64_t(256), int64_t(4096), int64_t(7168), kMaxHidden}) {
      const BwdLayout L = bwd_layout(N, H);
      const size_t np = (size_t)bwd_npad(N, H);
      const int64_t cap = bwd_token_cap(H);
      std::vector<size_t> off = {L.idx, L.n_active, L.block_desc, L.bidx, L.bn, L.sched, L.hT, L.Gv};
      std::vector<size_t> sz = {4 * (size_t)N, 4, 8 * (size_t)bwd_blocks(N, H), 4 * np, 4, 32,
                                2 * (size_t)H * np, 2 * np * (size_t)(kBwdChunkEntries + 64)};
      for (int q = 1; q < kBwdDhPieces; ++q) {
        off.push_back(L.dhp[q]);
        sz.push_back(4 * np * (size_t)H);
      }
      expect_layout(off, sz, L.total);
      // the block buffers hold min(N, capacity) rows, rounded up to the 256-token tile, and the
      // capacity's buffers fit the budget
      EXPECT(cap % 256 == 0 && cap >= 256);
      EXPECT((size_t)cap * bwd_bytes_per_token(H) <= kBwdBlockBudget || cap == 256);
      EXPECT((size_t)(cap + 256) * bwd_bytes_per_token(H) > kBwdBlockBudget);
      EXPECT(np % 256 == 0 && np >= (size_t)(N < cap ? N : cap) && np <= (size_t)cap);
      EXPECT((int64_t)bwd_blocks(N, H) * cap >= N && (int64_t)(bwd_blocks(N, H) - 1) * cap < N);
      // the compaction writes the block descriptors with one thread each: at most 1024 blocks
      // for every shape the checks accept
      if (check_shape(N, H, 151936, RLK_BF16) == RLK_SUCCESS) EXPECT(bwd_blocks(N, H) <= 1024);
      // the block buffers are all the workspace but for the index and the block descriptors
      EXPECT(L.total - L.hT <= (size_t)kBwdBlockBudget + 8 * 256);
    }
  EXPECT(bwd_token_cap(4096) == 11008 && bwd_token_cap(7168) == 8960);
  EXPECT(kl_fwd_token_cap(151936) == 32512 && kl_fwd_blocks(16384, 151936) == 1);
  // the KL forward's block capacity follows from the workspace: the default workspace gives the
  // default capacity (one block for fewer tokens), a workspace for any multiple of 256 that
  // capacity, and too small a workspace none
  for (int64_t N : {int64_t(1), int64_t(255), int64_t(20000), int64_t(65536), int64_t(1) << 20})
    for (int64_t V : {int64_t(1), int64_t(2000), int64_t(151936)}) {
      const int64_t top = (N + 255) / 256 * 256, cap = kl_fwd_token_cap(V);
      if (bwd_blocks_cap(N, cap) <= 1024)
        EXPECT(kl_fwd_cap_for_workspace(N, V, kl_fwd_layout(N, V).total) == std::min(cap, top));
      for (int64_t b : {int64_t(256), int64_t(3584), int64_t(8192)}) {
        if (b > top || bwd_blocks_cap(N, b) > 1024) continue;
        EXPECT(kl_fwd_cap_for_workspace(N, V, kl_fwd_layout_cap(N, V, b).total) == b);
        EXPECT(kl_fwd_cap_for_workspace(N, V, kl_fwd_layout_cap(N, V, b).total - 1) < b);
      }
      EXPECT(kl_fwd_cap_for_workspace(N, V, kKlScratchBytes) == 0);
      EXPECT(kl_fwd_cap_for_workspace(N, V, (size_t)1 << 40) == top ||
             bwd_blocks_cap(N, top) > 1024);
    }
  EXPECT(kl_fwd_layout(16384, 151936).total <= (size_t)kBwdBlockBudget);
  // the KL backward: the backward's buffers for blocks of its own capacity, then the scratch,
  // within the budget but for the index and the block descriptors
  EXPECT(kl_bwd_token_cap(4096) == 10240);
  for (int64_t N : {int64_t(0), int64_t(1), int64_t(10240), int64_t(10241), int64_t(16384),
                    kMaxTokens})
    for (int64_t H : {int64_t(256), int64_t(4096), int64_t(7168), kMaxHidden}) {
      const BwdLayout K = kl_bwd_layout(N, H);
      const int64_t cap = kl_bwd_token_cap(H);
      EXPECT(cap % 256 == 0 && cap >= 256 && cap <= bwd_token_cap(H));
      EXPECT((size_t)cap * bwd_bytes_per_token(H) + kKlScratchBytes <= kBwdBlockBudget ||
             cap == 256);
      EXPECT(kl_bwd_bytes(N, H) == K.total + kKlScratchBytes && K.total % 256 == 0);
      EXPECT(kl_bwd_bytes(N, H) - K.hT <= (size_t)kBwdBlockBudget + 8 * 256 || cap == 256);
      EXPECT((int64_t)bwd_blocks_cap(N, cap) * cap >= N);
    }
  int max_blocks = 0;
  for (int64_t H = 64; H <= kMaxHidden; H += 64) {
    const int64_t n = std::min<int64_t>(kMaxTokens, kMaxHiddenStateBytes / (2 * H));
    if (check_shape(n, H, 151936, RLK_BF16) == RLK_SUCCESS)
      max_blocks = std::max(max_blocks, bwd_blocks(n, H));
  }
  EXPECT(max_blocks > 1 && max_blocks <= 1024);
  EXPECT(bwd_blocks(0, 4096) == 1 && bwd_blocks(11008, 4096) == 1 &&
         bwd_blocks(11009, 4096) == 2);
  for (int64_t N : {int64_t(0), int64_t(1), int64_t(1023), int64_t(1024), int64_t(1) << 20,
                    kMaxTokens}) {
    const DiagLayout D = diag_layout(N);
    const size_t n = (size_t)(N > 0 ? N : 1), nb = (n + 1023) / 1024;
    expect_layout({D.idx, D.n_active, D.keys, D.part, D.pmax, D.ptok, D.hist, D.sel},
                  {4 * n, 4, 8 * n, 32 * nb, 8 * nb, 4 * nb, 4 * 8 * 6 * 256, 16 * 6}, D.total);
    const LogitsLayout G = logits_layout(N);
    expect_layout({G.idx, G.n_active}, {4 * n, 4}, G.total);
    EXPECT(loss_workspace(N) >= 32 * nb && loss_workspace(N) % 256 == 0);
    for (int64_t V : {int64_t(1), int64_t(151936), kMaxVocab}) {
      const KlLayout K = kl_fwd_layout(N, V);
      const int64_t np = kl_fwd_npad(N, V), cap = kl_fwd_token_cap(V);
      const size_t jn = 4 * (size_t)np * (size_t)num_partials(V);
      expect_layout({K.idx, K.n_active, K.block_count, K.tmax, K.tsum, K.smax, K.ssum, K.wf,
                     K.wr, K.scratch},
                    {4 * n, 4, 4 * (size_t)kl_fwd_blocks(N, V), jn, jn, jn, jn, jn, jn,
                     kKlScratchBytes},
                    K.total);
      // the KL forward's buffers hold one block of its own capacity, within the budget
      EXPECT(cap % 256 == 0 && cap >= 256 && np <= cap && np % 256 == 0);
      EXPECT((size_t)cap * kl_fwd_bytes_per_token(V) + kKlScratchBytes <= kBwdBlockBudget ||
             cap == 256);
      EXPECT(K.total - K.tmax <= (size_t)kBwdBlockBudget + 8 * 256 || cap == 256);
    }
  }
}

// The fused forward + backward: one token block's rows of fp16 d / bf16 dL/dz (every row starts
// 16-byte aligned and holds every column a GEMM reads), its column statistics, hT and the dL/dh
// piece rows within the budget; at most 1024 blocks wherever the checks accept the call.
static void test_fused() {
  EXPECT(fused_token_cap(4096, 151936) == 2816 && fused_token_cap(7168, 129280) == 3072);
  EXPECT(fused_blocks(16384, 4096, 151936) == 6 && fused_blocks(2816, 4096, 151936) == 1 &&
         fused_blocks(2817, 4096, 151936) == 2);
  for (int64_t V : {int64_t(1), int64_t(257), int64_t(1000), int64_t(151936), kMaxVocab}) {
    EXPECT(fused_pitch(V) >= (V + 255) / 256 * 256 && (fused_pitch(V) * 2) % 16 == 0);
    for (int64_t H : {int64_t(256), int64_t(4096), int64_t(7168), kMaxHidden})
      for (int64_t N : {int64_t(1), int64_t(300), int64_t(4096), int64_t(16384), kMaxTokens}) {
        const FusedLayout L = fused_layout(N, H, V);
        const size_t np = (size_t)fused_npad(N, H, V);
        const int64_t cap = fused_token_cap(H, V);
        const size_t jn = 4 * np * (size_t)num_partials(V);
        std::vector<size_t> off = {L.idx, L.n_active, L.block_desc, L.bidx, L.bn, L.sched,
                                   L.target_logit, L.part_max, L.part_sum, L.hT, L.X};
        std::vector<size_t> sz = {4 * (size_t)N, 4, 8 * (size_t)fused_blocks(N, H, V), 4 * np, 4,
                                  32, 4 * np, jn, jn, 2 * (size_t)H * np,
                                  2 * np * (size_t)fused_pitch(V)};
        for (int q = 1; q < kBwdDhPieces; ++q) {
          off.push_back(L.dhp[q]);
          sz.push_back(4 * np * (size_t)H);
        }
        expect_layout(off, sz, L.total);
        EXPECT(cap % 256 == 0 && cap >= 256);
        EXPECT((size_t)cap * fused_bytes_per_token(H, V) <= kBwdBlockBudget || cap == 256 ||
               cap == kMaxTokens);
        EXPECT(np % 256 == 0 && np >= (size_t)(N < cap ? N : cap) && np <= (size_t)cap);
        EXPECT((int64_t)fused_blocks(N, H, V) * cap >= N);
        const rlk_status_t s = check_fused(P(A), P(A), PT<const int32_t>(A), PT<const uint8_t>(A),
                                           N, H, V, RLK_BF16, 1.f, PT<const float>(A),
                                           PT<float>(A), PT<float>(A), PT<float>(A),
                                           PT<float>(A), P(A), L.total);
        if (s == RLK_SUCCESS) EXPECT(fused_blocks(N, H, V) <= 1024);
        if (fused_blocks(N, H, V) > 1024) EXPECT(s == RLK_ERROR_UNSUPPORTED);
      }
  }
  const size_t ws = fused_layout(16384, 4096, 151936).total;
  EXPECT(ws <= (size_t)kBwdBlockBudget);
  // a workspace gives the largest capacity (a multiple of 256, at most one block) whose layout
  // fits it: the budget's size the budget's capacity, a larger one more, a smaller one less,
  // and below the 256-token blocks' size none
  for (int64_t N : {int64_t(300), int64_t(9831), int64_t(16384), int64_t(100000)}) {
    const int64_t c0 = fused_token_cap(4096, 151936), top = (N + 255) / 256 * 256;
    EXPECT(fused_cap_for_workspace(N, 4096, 151936, fused_layout(N, 4096, 151936).total) ==
           std::min(c0, top));
    EXPECT(fused_cap_for_workspace(N, 4096, 151936, size_t(1) << 62) == top);
    for (int64_t c = 256; c <= top && c <= c0 + 256 * 40; c += 256) {
      const size_t t = fused_layout_cap(N, 4096, 151936, c).total;
      EXPECT(fused_cap_for_workspace(N, 4096, 151936, t) == c);
      EXPECT(fused_cap_for_workspace(N, 4096, 151936, t - 1) == c - 256);
    }
  }
  auto call = [&](uintptr_t lp, uintptr_t ls, uintptr_t dh, int dt, int64_t H, size_t bytes) {
    return check_fused(P(A), P(A), PT<const int32_t>(A), PT<const uint8_t>(A), 16384, H, 151936,
                       dt, 0.7f, PT<const float>(A), PT<float>(lp), PT<float>(ls), PT<float>(dh),
                       PT<float>(A), P(A), bytes);
  };
  EXPECT(call(A, A, A, RLK_BF16, 4096, ws) == RLK_SUCCESS);
  EXPECT(call(A, A, A, RLK_BF16, 4096, ws - 1) == RLK_SUCCESS);  // smaller blocks
  EXPECT(call(A, A, A, RLK_BF16, 4096, fused_layout_cap(16384, 4096, 151936, 256).total - 1) ==
         RLK_ERROR_WORKSPACE);
  EXPECT(call(0, A, A, RLK_BF16, 4096, ws) == RLK_ERROR_INVALID_VALUE);
  EXPECT(call(A, 0, A, RLK_BF16, 4096, ws) == RLK_ERROR_INVALID_VALUE);
  EXPECT(call(A, A, 0, RLK_BF16, 4096, ws) == RLK_ERROR_INVALID_VALUE);
  EXPECT(call(A, A, A + 4, RLK_BF16, 4096, ws) == RLK_ERROR_UNSUPPORTED);
  EXPECT(call(A, A, A, RLK_FP32, 4096, ws) == RLK_ERROR_UNSUPPORTED);
  EXPECT(call(A, A, A, RLK_BF16, 4160, ws) == RLK_ERROR_UNSUPPORTED);
}

static void test_fwd() {
  const size_t ws = fwd_layout(1000, 151936).total;
  auto call = [&](const void* h, const void* W, uintptr_t tg, uintptr_t mk, int64_t N, int64_t H,
                  int64_t V, int dt, float T, uintptr_t lp, uintptr_t ls, const void* w,
                  size_t bytes) {
    return check_fwd(h, W, PT<const int32_t>(tg), PT<const uint8_t>(mk), N, H, V, dt, T,
                     PT<const float>(lp), PT<const float>(ls), w, bytes);
  };
  EXPECT(call(P(A), P(A), A, A, 1000, 4096, 151936, RLK_BF16, 1.f, A, A, P(A), ws) ==
         RLK_SUCCESS);
  EXPECT(call(P(A), P(A), A, A, 1000, 4096, 151936, RLK_BF16, 1.f, A, 0, P(A), ws) ==
         RLK_SUCCESS);  // lse may be NULL
  EXPECT(call(P(A), P(A), A, A, 1000, 4096, 151936, RLK_BF16, 1.f, A, A, P(A), ws - 1) ==
         RLK_ERROR_WORKSPACE);
  // N == 0: nothing is read, NULL pointers are fine
  EXPECT(call(nullptr, nullptr, 0, 0, 0, 4096, 151936, RLK_BF16, 1.f, 0, 0, nullptr, 0) ==
         RLK_SUCCESS);
  // shape and temperature errors come before pointer checks
  EXPECT(call(nullptr, nullptr, 0, 0, 0, 4096, 151936, RLK_BF16, 0.f, 0, 0, nullptr, 0) ==
         RLK_ERROR_INVALID_VALUE);
  EXPECT(call(nullptr, nullptr, 0, 0, 5, 100, 151936, RLK_BF16, 1.f, 0, 0, nullptr, 0) ==
         RLK_ERROR_UNSUPPORTED);
  const uintptr_t ptrs[6] = {A, A, A, A, A, A};
  for (int k = 0; k < 6; ++k) {  // each required pointer NULL in turn
    uintptr_t p[6];
    for (int i = 0; i < 6; ++i) p[i] = ptrs[i];
    p[k] = 0;
    EXPECT(call(P(p[0]), P(p[1]), p[2], p[3], 1000, 4096, 151936, RLK_BF16, 1.f, p[4], A,
                P(p[5]), ws) == RLK_ERROR_INVALID_VALUE);
  }
  // misalignment: h, W 16 B; targets, logp, lse 4 B; workspace 256 B (mask: any)
  EXPECT(call(P(ODD), P(A), A, A, 1000, 4096, 151936, RLK_BF16, 1.f, A, A, P(A), ws) ==
         RLK_ERROR_UNSUPPORTED);
  EXPECT(call(P(A), P(A + 8), A, A, 1000, 4096, 151936, RLK_BF16, 1.f, A, A, P(A), ws) ==
         RLK_ERROR_UNSUPPORTED);
  EXPECT(call(P(A), P(A), ODD, A, 1000, 4096, 151936, RLK_BF16, 1.f, A, A, P(A), ws) ==
         RLK_ERROR_UNSUPPORTED);
  EXPECT(call(P(A), P(A), A, ODD + 1, 1000, 4096, 151936, RLK_BF16, 1.f, A, A, P(A), ws) ==
         RLK_SUCCESS);
  EXPECT(call(P(A), P(A), A, A, 1000, 4096, 151936, RLK_BF16, 1.f, ODD, A, P(A), ws) ==
         RLK_ERROR_UNSUPPORTED);
  EXPECT(call(P(A), P(A), A, A, 1000, 4096, 151936, RLK_BF16, 1.f, A, ODD, P(A), ws) ==
         RLK_ERROR_UNSUPPORTED);
  EXPECT(call(P(A), P(A), A, A, 1000, 4096, 151936, RLK_BF16, 1.f, A, A, P(A + 128), ws) ==
         RLK_ERROR_UNSUPPORTED);
  // the entropy forward needs the larger workspace
  EXPECT(check_fwd(P(A), P(A), PT<const int32_t>(A), PT<const uint8_t>(A), 1000, 4096, 151936,
                   RLK_BF16, 1.f, PT<const float>(A), nullptr, P(A), ws, true) ==
         RLK_ERROR_WORKSPACE);
}

static void test_bwd() {
  const size_t ws = bwd_layout(300, 4096).total;
  auto call = [&](int64_t N, int64_t H, int dt, uintptr_t dh, uintptr_t dW, uintptr_t w,
                  size_t bytes, uintptr_t adv = A) {
    return check_bwd(P(A), P(A), PT<const int32_t>(A), PT<const uint8_t>(A), N, H, 151936, dt,
                     1.f, PT<const float>(adv), PT<const float>(A), PT<const float>(dh),
                     PT<const float>(dW), P(w), bytes);
  };
  EXPECT(call(300, 4096, RLK_BF16, A, A, A, ws) == RLK_SUCCESS);
  EXPECT(call(300, 4096, RLK_BF16, A, A, A, ws - 256) == RLK_ERROR_WORKSPACE);
  EXPECT(call(300, 4096, RLK_FP32, A, A, A, ws) == RLK_ERROR_UNSUPPORTED);
  EXPECT(call(300, 4160, RLK_BF16, A, A, A, ws) == RLK_ERROR_UNSUPPORTED);  // H % 256
  EXPECT(call(300, 4096, RLK_BF16, A, 0, A, ws) == RLK_ERROR_INVALID_VALUE);
  EXPECT(call(0, 4096, RLK_BF16, 0, A, 0, 0) == RLK_SUCCESS);  // N == 0 still zeroes dW
  EXPECT(call(0, 4096, RLK_BF16, 0, 0, 0, 0) == RLK_ERROR_INVALID_VALUE);
  EXPECT(call(300, 4096, RLK_BF16, 0, A, A, ws) == RLK_ERROR_INVALID_VALUE);
  EXPECT(call(300, 4096, RLK_BF16, A, A, A, ws, 0) == RLK_ERROR_INVALID_VALUE);
  EXPECT(call(300, 4096, RLK_BF16, ODD, A, A, ws) == RLK_ERROR_UNSUPPORTED);
  EXPECT(call(300, 4096, RLK_BF16, A + 4, A, A, ws) == RLK_ERROR_UNSUPPORTED);  // dh: 16 B
  EXPECT(call(300, 4096, RLK_BF16, A + 16, A + 4, A, ws) == RLK_SUCCESS);     // dW: 4 B
  EXPECT(call(300, 4096, RLK_BF16, A, A, A + 64, ws) == RLK_ERROR_UNSUPPORTED);
}

static void test_logits() {
  const size_t ws = logits_layout(100).total;
  auto call = [&](int64_t N, int64_t V, int64_t ld, int dt, float T, uintptr_t lg, size_t bytes) {
    return check_logits(P(lg), N, V, ld, dt, T, PT<const int32_t>(A), PT<const uint8_t>(A),
                        PT<const float>(A), nullptr, P(A), bytes);
  };
  EXPECT(call(100, 1000, 1000, RLK_FP32, 1.f, A, ws) == RLK_SUCCESS);
  EXPECT(call(100, 1000, 1000, RLK_BF16, 1.f, A, ws) == RLK_SUCCESS);
  EXPECT(call(100, 1000, 1004, RLK_BF16, 1.f, A, ws) == RLK_ERROR_UNSUPPORTED);  // 16 B rows
  EXPECT(call(100, 1000, 999, RLK_FP32, 1.f, A, ws) == RLK_ERROR_INVALID_VALUE);  // ld < V
  EXPECT(call(100, kMaxLogitsVocab + 1, kMaxLogitsVocab + 8, RLK_FP32, 1.f, A, ws) ==
         RLK_ERROR_UNSUPPORTED);
  EXPECT(call(100, 1000, 1000, RLK_FP32, -1.f, A, ws) == RLK_ERROR_INVALID_VALUE);
  EXPECT(call(100, 1000, 1000, RLK_FP32, 1.f, 0, ws) == RLK_ERROR_INVALID_VALUE);
  EXPECT(call(100, 1000, 1000, RLK_FP32, 1.f, A + 4, ws) == RLK_ERROR_UNSUPPORTED);
  EXPECT(call(100, 1000, 1000, RLK_FP32, 1.f, A, ws - 1) == RLK_ERROR_WORKSPACE);
  EXPECT(call(0, 1000, 1000, RLK_FP32, 1.f, 0, 0) == RLK_SUCCESS);
}

static void test_kl() {
  auto call = [&](int64_t Hs, int64_t Ht, uintptr_t ws) {
    return check_kl(P(A), P(A), P(A), P(A), PT<const uint8_t>(A), 64, Hs, Ht, 1000, RLK_BF16,
                    1.f, P(ws));
  };
  EXPECT(call(512, 256, A) == RLK_SUCCESS);
  EXPECT(call(512, 100, A) == RLK_ERROR_UNSUPPORTED);
  EXPECT(call(512, 256, 0) == RLK_ERROR_INVALID_VALUE);
  EXPECT(call(512, 256, A + 16) == RLK_ERROR_UNSUPPORTED);
}

int main() {
  test_shape();
  test_shard();
  test_temperature();
  test_layouts();
  test_fwd();
  test_bwd();
  test_fused();
  test_logits();
  test_kl();
  std::printf("validate: %d checks, %d failed\n", g_checks, g_fail);
  return g_fail == 0 ? 0 : 1;
}
