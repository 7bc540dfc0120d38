// Host-side check of the C ABI (abi.hip) built with AddressSanitizer.
//
// abi.hip is compiled for the host only and linked against this file, which
// stands in for the kernel launchers and workspace-size functions of the
// other sources: each stub counts its calls and returns VEDA_OK.  No GPU and
// no device code is involved.  The checks:
//   - layouts: valid ones derive the expected grids and offsets, invalid ones
//     are refused, and random layouts (also corrupted after derivation) never
//     touch memory out of bounds;
//   - every device entry point refuses invalid arguments before any launch
//     and, given valid ones, launches exactly once;
//   - workspace queries and the static-scratch distillation call.
// AddressSanitizer aborts the program on any out-of-bounds access or
// use-after-free in the host code; the program prints ALL OK on success.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>

#include "veda_internal.hpp"

namespace veda {
int g_launches = 0;
int g_scratch_lookups = 0;
void* g_last_workspace = nullptr;

int launch_permute(const DevLayout&, int, int, const void*, void*, hipStream_t) { return ++g_launches, VEDA_OK; }
int launch_tripool_score(const DevLayout&, int, const void*, const void*, const float*, const float*,
                         const float*, const float*, int, float*, float*, float*, hipStream_t) {
  return ++g_launches, VEDA_OK;
}
int launch_permute_pool(const DevLayout&, int, const void*, void*, float*, hipStream_t) { return ++g_launches, VEDA_OK; }
int launch_project_score(const DevLayout&, const float*, const float*, const float*, const float*,
                         const float*, int, float*, float*, hipStream_t) {
  return ++g_launches, VEDA_OK;
}
int launch_select(const DevLayout&, const float*, const int32_t*, int32_t*, int32_t*, hipStream_t) {
  return ++g_launches, VEDA_OK;
}
int launch_sparse_attn(const DevLayout&, const void*, const void*, const void*, const int32_t*,
                       const int32_t*, float, void*, float*, bool, int* claim, hipStream_t) {
  g_last_workspace = claim;
  return ++g_launches, VEDA_OK;
}
int launch_oracle_map(const DevLayout&, const void*, const void*, float, const int32_t*, int, void* ws,
                      float*, float*, hipStream_t) {
  g_last_workspace = ws;
  return ++g_launches, VEDA_OK;
}
int64_t map_workspace_bytes(const DevLayout& L, int64_t n_sub) {
  return n_sub <= 0 ? 0 : n_sub * L.max_tiles * L.S * 4 + n_sub * 16 * L.S * 8;
}
int64_t distill_workspace_bytes(const DevLayout& L, int64_t n_sub, int d_e) {
  return 4096 + 4 * n_sub * (L.max_tiles + d_e + 2) + 4 * L.tile_off[L.heads] * (int64_t)d_e;
}
int launch_distill(const DevLayout&, const float*, const float*, const int32_t*, int, const float*,
                   const float*, int, void* ws, float*, float*, float*, float*, float*, hipStream_t) {
  g_last_workspace = ws;
  return ++g_launches, VEDA_OK;
}
int distill_static_scratch(void** ptr) {
  ++g_scratch_lookups;
  static unsigned char fake_device_scratch[256];
  *ptr = fake_device_scratch;
  return VEDA_OK;
}
int64_t head_error_workspace_bytes(const DevLayout& L) { return (int64_t)L.heads * 64 * 16; }
int launch_head_choose(const double*, int, int, int32_t*, hipStream_t) { return ++g_launches, VEDA_OK; }
int launch_score_select(const DevLayout&, const float*, int, const int32_t*, int32_t*, int32_t*, hipStream_t) {
  return ++g_launches, VEDA_OK;
}
int score_select_max_cols() { return 2048; }
int launch_head_error(const DevLayout&, const void*, const void*, double*, double*, void*, hipStream_t) {
  return ++g_launches, VEDA_OK;
}
int64_t attn_bwd_workspace_bytes(const DevLayout& L, int64_t nnz) {
  return 8 * L.tile_off[L.heads] * L.S * L.d + 8 * nnz + 4096;
}
int launch_sparse_attn_bwd(const DevLayout&, const void*, const void*, const void*, const void*,
                           const void*, const float*, const int32_t*, const int32_t*, int64_t, float,
                           void*, void*, void*, void*, bool, hipStream_t) {
  return ++g_launches, VEDA_OK;
}
}  // namespace veda

using veda::g_launches;

static int g_fail = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::printf("FAILED line %d: %s\n", __LINE__, #cond);                \
      ++g_fail;                                                            \
    }                                                                      \
  } while (0)

// status and number of launches of one call
#define EXPECT_CALL(expr, status, launches)                                \
  do {                                                                     \
    const int before_ = g_launches;                                        \
    const int st_ = (expr);                                                \
    if (st_ != (status) || g_launches - before_ != (launches)) {           \
      std::printf("FAILED line %d: %s -> %d (%d launches), want %d (%d)\n", \
                  __LINE__, #expr, st_, g_launches - before_, (status),    \
                  (launches));                                             \
      ++g_fail;                                                            \
    }                                                                      \
  } while (0)

static veda_layout make_layout(int T, int H, int W, int d, int S, int heads, const int (*shapes)[3]) {
  veda_layout L;
  std::memset(&L, 0, sizeof(L));
  L.T = T; L.H = H; L.W = W; L.head_dim = d; L.tile_size = S; L.num_heads = heads;
  for (int h = 0; h < heads; ++h)
    for (int a = 0; a < 3; ++a) L.tile_shape[h][a] = shapes[h][a];
  return L;
}

int main() {
  // ---- layouts
  const int mixed[4][3] = {{1, 8, 16}, {2, 8, 8}, {4, 4, 8}, {8, 4, 4}};
  veda_layout L = make_layout(61, 45, 80, 128, 128, 4, mixed);
  CHECK(veda_layout_init(&L) == VEDA_OK);
  CHECK(L.n_tiles[0] == 61 * 6 * 5 && L.n_tiles[1] == 31 * 6 * 10 && L.n_tiles[2] == 16 * 12 * 10);
  CHECK(L.tile_off[4] == (int64_t)L.n_tiles[0] + L.n_tiles[1] + L.n_tiles[2] + L.n_tiles[3]);
  CHECK(L.max_tiles == 1920);
  {
    veda_layout bad = make_layout(0, 45, 80, 128, 128, 4, mixed);
    CHECK(veda_layout_init(&bad) == VEDA_ERR_INVALID_ARG);
    bad = make_layout(61, 45, 80, 128, 96, 4, mixed);   // shape volume != tile size
    CHECK(veda_layout_init(&bad) == VEDA_ERR_INVALID_ARG);
    bad = make_layout(61, 45, 80, 128, 128, 4, mixed);
    bad.num_heads = VEDA_MAX_HEADS + 1;
    CHECK(veda_layout_init(&bad) == VEDA_ERR_INVALID_ARG);
    const int big[1][3] = {{1, 1, 128}};
    bad = make_layout(46341, 1, 128, 128, 128, 1, big);   // n^2 beyond int32 CSR entries
    CHECK(veda_layout_init(&bad) == VEDA_ERR_INVALID_ARG);
    CHECK(veda_layout_init(nullptr) == VEDA_ERR_INVALID_ARG);
  }
  int k = 0;
  CHECK(veda_keep_count(720, 95, &k) == VEDA_OK && k == 36);
  CHECK(veda_keep_count(0, 95, &k) == VEDA_ERR_INVALID_ARG);
  CHECK(veda_keep_count(10, 101, &k) == VEDA_ERR_INVALID_ARG);
  CHECK(veda_keep_count(10, 5, nullptr) == VEDA_ERR_INVALID_ARG);

  // ---- device entry points: fake, aligned, far-apart addresses (never dereferenced)
  auto P = [](uint64_t i) { return reinterpret_cast<void*>((uint64_t)(1) << 40 | (i << 34)); };
  auto F = [&](uint64_t i) { return static_cast<float*>(P(i)); };
  auto I = [&](uint64_t i) { return static_cast<int32_t*>(P(i)); };
  void* odd = reinterpret_cast<void*>(((uint64_t)1 << 40) + 8);
  veda_layout tampered = L;
  tampered.tile_off[2] += 1;

  EXPECT_CALL(veda_tile_permute(&L, VEDA_BF16, VEDA_FWD, P(1), P(2), nullptr), VEDA_OK, 1);
  EXPECT_CALL(veda_tile_permute(&L, VEDA_BF16, VEDA_FWD_T, P(1), P(2), nullptr), VEDA_OK, 1);
  EXPECT_CALL(veda_tile_permute(&tampered, VEDA_BF16, VEDA_FWD, P(1), P(2), nullptr), VEDA_ERR_INVALID_ARG, 0);
  EXPECT_CALL(veda_tile_permute(&L, 7, VEDA_FWD, P(1), P(2), nullptr), VEDA_ERR_INVALID_ARG, 0);
  EXPECT_CALL(veda_tile_permute(&L, VEDA_BF16, 9, P(1), P(2), nullptr), VEDA_ERR_INVALID_ARG, 0);
  EXPECT_CALL(veda_tile_permute(&L, VEDA_BF16, VEDA_FWD, odd, P(2), nullptr), VEDA_ERR_UNSUPPORTED, 0);
  EXPECT_CALL(veda_tile_permute(&L, VEDA_BF16, VEDA_FWD, P(1), P(1), nullptr), VEDA_ERR_INVALID_ARG, 0);

  EXPECT_CALL(veda_tile_permute_pool(&L, VEDA_BF16, P(1), P(2), F(3), nullptr), VEDA_OK, 1);
  EXPECT_CALL(veda_tile_permute_pool(&L, VEDA_BF16, P(1), P(2), nullptr, nullptr), VEDA_ERR_INVALID_ARG, 0);

  EXPECT_CALL(veda_tripool_score(&L, VEDA_BF16, P(1), P(2), F(3), F(3), nullptr, nullptr, 128, F(4),
                                 F(5), F(6), nullptr), VEDA_OK, 1);
  EXPECT_CALL(veda_tripool_score(&L, VEDA_BF16, P(1), P(2), F(3), F(3), nullptr, nullptr, 0, F(4),
                                 F(5), F(6), nullptr), VEDA_ERR_INVALID_ARG, 0);
  EXPECT_CALL(veda_tile_score(&L, F(1), F(2), F(2), nullptr, nullptr, 128, F(3), F(4), nullptr), VEDA_OK, 1);
  EXPECT_CALL(veda_tile_score(&L, F(1), F(2), F(2), nullptr, nullptr, 300, F(3), F(4), nullptr),
              VEDA_ERR_UNSUPPORTED, 0);

  int32_t kh[4] = {92, 93, 96, 96};
  EXPECT_CALL(veda_select_tiles(&L, F(1), kh, I(2), I(3), nullptr), VEDA_OK, 1);
  int32_t kbad[4] = {92, 93, 0, 96};
  EXPECT_CALL(veda_select_tiles(&L, F(1), kbad, I(2), I(3), nullptr), VEDA_ERR_INVALID_ARG, 0);
  kbad[2] = 1921;
  EXPECT_CALL(veda_select_tiles(&L, F(1), kbad, I(2), I(3), nullptr), VEDA_ERR_INVALID_ARG, 0);

  // projection only, then the fused score + selection
  EXPECT_CALL(veda_tile_score(&L, F(1), F(2), F(2), nullptr, nullptr, 128, F(3), nullptr, nullptr), VEDA_OK, 1);
  EXPECT_CALL(veda_score_select(&L, F(3), 128, kh, I(2), I(3), nullptr), VEDA_OK, 1);
  EXPECT_CALL(veda_score_select(&L, F(3), 64, kh, I(2), I(3), nullptr), VEDA_OK, 1);
  EXPECT_CALL(veda_score_select(&L, F(3), 96, kh, I(2), I(3), nullptr), VEDA_ERR_UNSUPPORTED, 0);
  EXPECT_CALL(veda_score_select(&L, reinterpret_cast<float*>(reinterpret_cast<char*>(F(3)) + 4), 128, kh,
                                I(2), I(3), nullptr), VEDA_ERR_UNSUPPORTED, 0);
  EXPECT_CALL(veda_score_select(&L, F(3), 0, kh, I(2), I(3), nullptr), VEDA_ERR_INVALID_ARG, 0);
  EXPECT_CALL(veda_score_select(&L, nullptr, 128, kh, I(2), I(3), nullptr), VEDA_ERR_INVALID_ARG, 0);
  EXPECT_CALL(veda_score_select(&L, F(3), 128, kh, I(2), nullptr, nullptr), VEDA_ERR_INVALID_ARG, 0);
  EXPECT_CALL(veda_score_select(&L, F(3), 128, kbad, I(2), I(3), nullptr), VEDA_ERR_INVALID_ARG, 0);
  {
    const int wide[1][3] = {{1, 8, 16}};
    veda_layout Lw = make_layout(64, 64, 256, 128, 128, 1, wide);   // 8192 tiles in the head
    CHECK(veda_layout_init(&Lw) == VEDA_OK && Lw.max_tiles == 8192);
    int32_t kw[1] = {410};
    EXPECT_CALL(veda_score_select(&Lw, F(3), 128, kw, I(2), I(3), nullptr), VEDA_ERR_UNSUPPORTED, 0);
    EXPECT_CALL(veda_select_tiles(&Lw, F(1), kw, I(2), I(3), nullptr), VEDA_OK, 1);
  }

  EXPECT_CALL(veda_sparse_attn_fwd(&L, P(1), P(2), P(3), I(4), I(5), 0.088f, P(6), F(7), nullptr, 0,
                                   nullptr), VEDA_OK, 1);
  EXPECT_CALL(veda_sparse_attn_fwd_tokens(&L, P(1), P(2), P(3), I(4), I(5), 0.088f, P(6), nullptr,
                                          nullptr, 0, nullptr),
              VEDA_OK, 1);
  {
    // the optional workspace reaches the launch; too small or misaligned is rejected
    int64_t aw = -1;
    CHECK(veda_sparse_attn_fwd_workspace(&L, &aw) == VEDA_OK && aw == 256);
    CHECK(veda_sparse_attn_fwd_workspace(&L, nullptr) == VEDA_ERR_INVALID_ARG);
    EXPECT_CALL(veda_sparse_attn_fwd_tokens(&L, P(1), P(2), P(3), I(4), I(5), 0.088f, P(6), nullptr,
                                            P(8), aw, nullptr),
                VEDA_OK, 1);
    CHECK(veda::g_last_workspace == P(8));
    EXPECT_CALL(veda_sparse_attn_fwd(&L, P(1), P(2), P(3), I(4), I(5), 0.088f, P(6), F(7), P(8),
                                     aw - 1, nullptr),
                VEDA_ERR_INVALID_ARG, 0);
    EXPECT_CALL(veda_sparse_attn_fwd(&L, P(1), P(2), P(3), I(4), I(5), 0.088f, P(6), F(7),
                                     static_cast<char*>(P(8)) + 4, aw, nullptr),
                VEDA_ERR_INVALID_ARG, 0);
  }
  EXPECT_CALL(veda_sparse_attn_fwd(&L, P(1), P(2), P(3), I(4), I(5), -1.f, P(6), F(7), nullptr, 0,
                                   nullptr),
              VEDA_ERR_INVALID_ARG, 0);
  EXPECT_CALL(veda_sparse_attn_fwd(&L, P(1), P(2), nullptr, I(4), I(5), 0.088f, P(6), F(7), nullptr,
                                   0, nullptr),
              VEDA_ERR_INVALID_ARG, 0);
  EXPECT_CALL(veda_sparse_attn_fwd_tokens(&L, P(1), P(2), P(3), I(4), I(5), 0.088f, P(1), nullptr,
                                          nullptr, 0, nullptr),
              VEDA_ERR_INVALID_ARG, 0);

  int64_t ws = -1;
  CHECK(veda_oracle_maxpool_map_workspace(&L, 100, &ws) == VEDA_OK && ws > 0);
  EXPECT_CALL(veda_oracle_maxpool_map(&L, P(1), P(2), 0.088f, I(3), 100, P(4), ws, F(5), F(6), nullptr),
              VEDA_OK, 1);
  EXPECT_CALL(veda_oracle_maxpool_map(&L, P(1), P(2), 0.088f, I(3), 100, P(4), ws - 1, F(5), F(6), nullptr),
              VEDA_ERR_INVALID_ARG, 0);
  EXPECT_CALL(veda_oracle_maxpool_map(&L, P(1), P(2), 0.088f, I(3), VEDA_MAX_SUBSET + 1, P(4), ws, F(5),
                                      F(6), nullptr), VEDA_ERR_UNSUPPORTED, 0);

  CHECK(veda_distill_grad_workspace(&L, 400, 128, &ws) == VEDA_OK && ws > 0);
  EXPECT_CALL(veda_distill_grad(&L, F(1), F(2), I(3), 400, F(4), F(5), 128, P(6), ws, F(7), F(8), F(9),
                                nullptr, nullptr, nullptr), VEDA_OK, 1);
  CHECK(veda::g_last_workspace == P(6));
  EXPECT_CALL(veda_distill_grad(&L, F(1), F(2), I(3), 400, F(4), F(5), 128, P(6), ws - 1, F(7), F(8), F(9),
                                nullptr, nullptr, nullptr), VEDA_ERR_INVALID_ARG, 0);
  // static scratch: looked up, passed to the launch; too large a problem refused first
  const int lookups = veda::g_scratch_lookups;
  EXPECT_CALL(veda_distill_grad_noalloc(&L, F(1), F(2), I(3), 400, F(4), F(5), 128, F(7), F(8), F(9),
                                        nullptr, nullptr, nullptr), VEDA_OK, 1);
  CHECK(veda::g_scratch_lookups == lookups + 1 && veda::g_last_workspace != P(6));
  EXPECT_CALL(veda_distill_grad_noalloc(&L, F(1), F(2), I(3), 1 << 20, F(4), F(5), 128, F(7), F(8), F(9),
                                        nullptr, nullptr, nullptr), VEDA_ERR_UNSUPPORTED, 0);
  CHECK(veda::g_scratch_lookups == lookups + 1);

  const int64_t nnz = (int64_t)L.n_tiles[0] * 92 + (int64_t)L.n_tiles[1] * 93 + (int64_t)L.n_tiles[2] * 96 +
                      (int64_t)L.n_tiles[3] * 96;
  CHECK(veda_sparse_attn_bwd_workspace(&L, nnz, &ws) == VEDA_OK && ws > 0);
  EXPECT_CALL(veda_sparse_attn_bwd(&L, P(1), P(2), P(3), P(4), P(5), F(6), I(7), I(8), nnz, 0.088f, P(9), ws,
                                   P(10), P(11), P(12), nullptr), VEDA_OK, 1);
  EXPECT_CALL(veda_sparse_attn_bwd_tiles(&L, P(1), P(2), P(3), P(4), P(5), F(6), I(7), I(8), nnz, 0.088f, P(9),
                                         ws, P(10), P(11), P(12), nullptr), VEDA_OK, 1);
  EXPECT_CALL(veda_sparse_attn_bwd(&L, P(1), P(2), P(3), P(4), P(5), F(6), I(7), I(8), nnz, 0.088f, P(9),
                                   ws - 1, P(10), P(11), P(12), nullptr), VEDA_ERR_INVALID_ARG, 0);
  EXPECT_CALL(veda_sparse_attn_bwd(&L, P(1), P(2), P(3), P(4), P(5), F(6), I(7), I(8), nnz, 0.088f, P(9), ws,
                                   P(1), P(11), P(12), nullptr), VEDA_ERR_INVALID_ARG, 0);

  CHECK(veda_head_sq_error_workspace(&L, &ws) == VEDA_OK);
  EXPECT_CALL(veda_head_sq_error(&L, P(1), P(2), static_cast<double*>(P(3)), nullptr, P(4), ws, nullptr),
              VEDA_OK, 1);
  EXPECT_CALL(veda_head_sq_error(&L, P(1), P(2), static_cast<double*>(P(3)), nullptr, P(4), ws - 1, nullptr),
              VEDA_ERR_INVALID_ARG, 0);

  double* de = static_cast<double*>(P(3));
  int32_t* dc = I(4);
  EXPECT_CALL(veda_head_choose(de, 4, 24, dc, nullptr), VEDA_OK, 1);
  EXPECT_CALL(veda_head_choose(de, VEDA_MAX_CANDIDATES, VEDA_MAX_HEADS, dc, nullptr), VEDA_OK, 1);
  EXPECT_CALL(veda_head_choose(nullptr, 4, 24, dc, nullptr), VEDA_ERR_INVALID_ARG, 0);
  EXPECT_CALL(veda_head_choose(de, 4, 24, nullptr, nullptr), VEDA_ERR_INVALID_ARG, 0);
  EXPECT_CALL(veda_head_choose(de, 0, 24, dc, nullptr), VEDA_ERR_INVALID_ARG, 0);
  EXPECT_CALL(veda_head_choose(de, VEDA_MAX_CANDIDATES + 1, 24, dc, nullptr), VEDA_ERR_INVALID_ARG, 0);
  EXPECT_CALL(veda_head_choose(de, 4, 0, dc, nullptr), VEDA_ERR_INVALID_ARG, 0);
  EXPECT_CALL(veda_head_choose(de, 4, VEDA_MAX_HEADS + 1, dc, nullptr), VEDA_ERR_INVALID_ARG, 0);
  EXPECT_CALL(veda_head_choose(reinterpret_cast<double*>(reinterpret_cast<char*>(de) + 4), 4, 24, dc, nullptr),
              VEDA_ERR_INVALID_ARG, 0);

  for (int s : {0, -1, -2, -3, -4, 77}) CHECK(std::strlen(veda_status_string(s)) > 0);
  CHECK(veda_layout_sizeof() == (int64_t)sizeof(veda_layout));

  // ---- random layouts, and random corruption of derived ones: no call may
  // read or write out of bounds, whatever the struct holds
  std::mt19937 rng(1234);
  const int shapes128[4][3] = {{1, 8, 16}, {2, 8, 8}, {4, 4, 8}, {8, 4, 4}};
  int derived = 0;
  for (int it = 0; it < 20000; ++it) {
    veda_layout R;
    std::memset(&R, 0, sizeof(R));
    R.T = (int)(rng() % 70) - 2;
    R.H = (int)(rng() % 60) - 2;
    R.W = (int)(rng() % 90) - 2;
    R.num_heads = (int)(rng() % (VEDA_MAX_HEADS + 3)) - 1;
    R.head_dim = rng() % 4 == 0 ? 64 : 128;
    R.tile_size = 128;
    for (int h = 0; h < VEDA_MAX_HEADS; ++h) {
      const int c = (int)(rng() % 4);
      for (int a = 0; a < 3; ++a) R.tile_shape[h][a] = shapes128[c][a];
    }
    if (veda_layout_init(&R) == VEDA_OK) {
      ++derived;
      if (rng() % 2) {   // corrupt one derived field
        const int h = (int)(rng() % VEDA_MAX_HEADS);
        switch (rng() % 4) {
          case 0: R.n_tiles[h] += 1 + (int)(rng() % 5); break;
          case 1: R.tile_off[h + 1] -= 1; break;
          case 2: R.max_tiles = (int)rng(); break;
          default: R.num_heads = VEDA_MAX_HEADS + 5; break;
        }
      }
    }
    int32_t kk[VEDA_MAX_HEADS];
    for (int h = 0; h < VEDA_MAX_HEADS; ++h) kk[h] = 1;
    veda_tile_permute(&R, VEDA_BF16, VEDA_FWD, P(1), P(2), nullptr);
    veda_select_tiles(&R, F(1), kk, I(2), I(3), nullptr);
    veda_sparse_attn_fwd(&R, P(1), P(2), P(3), I(4), I(5), 0.1f, P(6), nullptr, nullptr, 0, nullptr);
    veda_oracle_maxpool_map_workspace(&R, 10, &ws);
    veda_sparse_attn_bwd_workspace(&R, 10, &ws);
  }
  CHECK(derived > 1000);

  if (g_fail == 0) std::printf("ALL OK (%d launches)\n", g_launches);
  return g_fail == 0 ? 0 : 1;
}
