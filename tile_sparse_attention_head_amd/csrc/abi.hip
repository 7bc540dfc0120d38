// C ABI of libveda.so: argument validation, layout derivation and launches.
// Every check runs on the host before anything is enqueued; see veda.h for
// the contract of each call.
#include <cstdlib>
#include <cstring>
#include <vector>

#include "veda_internal.hpp"

namespace veda {

DevLayout make_dev_layout(const veda_layout* L) {
  DevLayout d;
  std::memset(&d, 0, sizeof(d));
  d.T = L->T; d.H = L->H; d.W = L->W;
  d.heads = L->num_heads; d.d = L->head_dim; d.S = L->tile_size;
  d.max_tiles = L->max_tiles;
  for (int h = 0; h < L->num_heads; ++h)
    for (int a = 0; a < 3; ++a) {
      d.shape[h][a] = L->tile_shape[h][a];
      d.grid[h][a] = L->tile_grid[h][a];
    }
  for (int h = 0; h <= L->num_heads; ++h) {
    d.tile_off[h] = L->tile_off[h];
    d.score_off[h] = L->score_off[h];
  }
  return d;
}

namespace {

bool debug_sync() {
  static const bool on = [] {
    const char* e = std::getenv("VEDA_DEBUG_SYNC");
    return e != nullptr && e[0] == '1';
  }();
  return on;
}

int finish(int st, void* stream) {
  if (st != VEDA_OK || !debug_sync()) return st;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return VEDA_ERR_LAUNCH;
  return hipGetLastError() == hipSuccess ? VEDA_OK : VEDA_ERR_LAUNCH;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Derive every field from the inputs into `out`; false if the inputs are bad.
bool derive(const veda_layout* L, veda_layout* out) {
  if (L == nullptr) return false;
  if (L->T < 1 || L->H < 1 || L->W < 1) return false;
  if (L->num_heads < 1 || L->num_heads > VEDA_MAX_HEADS) return false;
  if (L->head_dim < 1 || L->tile_size < 1) return false;
  if ((int64_t)L->T * L->H * L->W > INT32_MAX) return false;
  *out = *L;
  int64_t toff = 0, soff = 0;
  int32_t mx = 0;
  for (int h = 0; h < L->num_heads; ++h) {
    const int32_t* p = L->tile_shape[h];
    if (p[0] < 1 || p[1] < 1 || p[2] < 1) return false;
    if ((int64_t)p[0] * p[1] * p[2] != L->tile_size) return false;
    const int64_t nT = ceil_div(L->T, p[0]), nH = ceil_div(L->H, p[1]), nW = ceil_div(L->W, p[2]);
    const int64_t n = nT * nH * nW;
    if (n > INT32_MAX) return false;
    out->tile_grid[h][0] = (int32_t)nT;
    out->tile_grid[h][1] = (int32_t)nH;
    out->tile_grid[h][2] = (int32_t)nW;
    out->n_tiles[h] = (int32_t)n;
    out->tile_off[h] = toff;
    out->score_off[h] = soff;
    toff += n;
    soff += n * n;
    if (n > mx) mx = (int32_t)n;
  }
  for (int h = L->num_heads; h < VEDA_MAX_HEADS; ++h) {
    out->tile_grid[h][0] = out->tile_grid[h][1] = out->tile_grid[h][2] = 0;
    out->n_tiles[h] = 0;
  }
  out->tile_off[L->num_heads] = toff;
  out->score_off[L->num_heads] = soff;
  for (int h = L->num_heads + 1; h <= VEDA_MAX_HEADS; ++h) {
    out->tile_off[h] = toff;
    out->score_off[h] = soff;
  }
  out->max_tiles = mx;
  out->reserved0 = 0;
  // CSR rows and entries are int32: rows = tiles, entries <= sum n^2.
  if (toff + 1 > INT32_MAX || soff > INT32_MAX) return false;
  return true;
}

// A layout passed to a device call must be exactly what veda_layout_init made.
bool layout_ok(const veda_layout* L) {
  veda_layout d;
  if (!derive(L, &d)) return false;
  for (int h = 0; h < L->num_heads; ++h) {
    if (d.n_tiles[h] != L->n_tiles[h]) return false;
    for (int a = 0; a < 3; ++a)
      if (d.tile_grid[h][a] != L->tile_grid[h][a]) return false;
  }
  for (int h = 0; h <= L->num_heads; ++h)
    if (d.tile_off[h] != L->tile_off[h] || d.score_off[h] != L->score_off[h]) return false;
  return d.max_tiles == L->max_tiles;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool disjoint(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x + na <= y || y + nb <= x;
}

bool attn_shape_ok(const veda_layout* L) {
  return (L->head_dim == 128 && L->tile_size == 128) || (L->head_dim == 64 && L->tile_size == 64);
}

// The K/V tiles of one head are read through a buffer resource whose range
// is a 32-bit byte count, and the forward packs a tile index into 16 bits.
bool tiles_per_head_ok(const veda_layout* L) {
  return L->max_tiles <= VEDA_MAX_TILES_PER_HEAD &&
         (int64_t)L->max_tiles * L->tile_size * L->head_dim * 2 <= INT32_MAX;
}

// Checks shared by the two attention entry points, plus the debug-mode CSR
// validation (synchronous).
int attn_args(const veda_layout* L, const void* q_perm, const void* k_perm, const void* vt_perm,
              const int32_t* row_ptr, const int32_t* col_idx, float sm_scale, const void* o,
              void* stream) {
  if (L == nullptr || !layout_ok(L)) return VEDA_ERR_INVALID_ARG;
  if (q_perm == nullptr || k_perm == nullptr || vt_perm == nullptr || row_ptr == nullptr ||
      col_idx == nullptr || o == nullptr)
    return VEDA_ERR_INVALID_ARG;
  if (!(sm_scale > 0.f) || sm_scale == INFINITY) return VEDA_ERR_INVALID_ARG;
  if (!attn_shape_ok(L) || !tiles_per_head_ok(L)) return VEDA_ERR_UNSUPPORTED;
  if (!aligned16(q_perm) || !aligned16(k_perm) || !aligned16(vt_perm) || !aligned16(o))
    return VEDA_ERR_UNSUPPORTED;
  if (debug_sync()) {
    const int64_t rows = L->tile_off[L->num_heads];
    std::vector<int32_t> rp(rows + 1);
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return VEDA_ERR_LAUNCH;
    if (hipMemcpy(rp.data(), row_ptr, (rows + 1) * sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
      return VEDA_ERR_LAUNCH;
    if (rp[0] < 0) return VEDA_ERR_BAD_CSR;
    for (int64_t r = 0; r < rows; ++r)
      if (rp[r + 1] < rp[r]) return VEDA_ERR_BAD_CSR;
    std::vector<int32_t> ci(rp[rows]);
    if (!ci.empty() && hipMemcpy(ci.data(), col_idx, ci.size() * sizeof(int32_t),
                                 hipMemcpyDeviceToHost) != hipSuccess)
      return VEDA_ERR_LAUNCH;
    for (int h = 0; h < L->num_heads; ++h)
      for (int64_t r = L->tile_off[h]; r < L->tile_off[h + 1]; ++r)
        for (int32_t p = rp[r]; p < rp[r + 1]; ++p)
          if (ci[p] < 0 || ci[p] >= L->n_tiles[h]) return VEDA_ERR_BAD_CSR;
  }
  return VEDA_OK;
}

// Checks shared by the two backward entry points, plus the debug-mode CSR
// validation (synchronous).  qk_bytes: the size of q and k as passed (token
// or tile order).
int bwd_args(const veda_layout* L, const void* q, const void* k, size_t qk_bytes, const void* v,
             const void* o, const void* d_o, const float* lse, const int32_t* row_ptr,
             const int32_t* col_idx, int64_t nnz, float sm_scale, void* workspace,
             int64_t workspace_bytes, void* dq, void* dk, void* dv, void* stream) {
  if (L == nullptr || !layout_ok(L)) return VEDA_ERR_INVALID_ARG;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || d_o == nullptr ||
      lse == nullptr || row_ptr == nullptr || col_idx == nullptr || workspace == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr)
    return VEDA_ERR_INVALID_ARG;
  if (nnz < 0 || nnz > INT32_MAX) return VEDA_ERR_INVALID_ARG;
  if (!(sm_scale > 0.f) || sm_scale == INFINITY) return VEDA_ERR_INVALID_ARG;
  if (!attn_shape_ok(L) || !tiles_per_head_ok(L)) return VEDA_ERR_UNSUPPORTED;
  for (const void* p : {q, k, v, o, d_o, (const void*)dq, (const void*)dk, (const void*)dv,
                        (const void*)workspace})
    if (!aligned16(p)) return VEDA_ERR_UNSUPPORTED;
  const DevLayout dl = make_dev_layout(L);
  if (workspace_bytes < attn_bwd_workspace_bytes(dl, nnz)) return VEDA_ERR_INVALID_ARG;
  const size_t tok = (size_t)L->T * L->H * L->W * L->num_heads * L->head_dim * 2;
  for (const void* out : {(const void*)dq, (const void*)dk, (const void*)dv}) {
    for (const void* in : {v, o, d_o})
      if (!disjoint(out, tok, in, tok)) return VEDA_ERR_INVALID_ARG;
    for (const void* in : {q, k})
      if (!disjoint(out, tok, in, qk_bytes)) return VEDA_ERR_INVALID_ARG;
  }
  if (!disjoint(dq, tok, dk, tok) || !disjoint(dq, tok, dv, tok) || !disjoint(dk, tok, dv, tok))
    return VEDA_ERR_INVALID_ARG;
  if (debug_sync()) {   // host-side CSR validation (synchronous, debug only)
    const int64_t rows = L->tile_off[L->num_heads];
    std::vector<int32_t> rp(rows + 1);
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return VEDA_ERR_LAUNCH;
    if (hipMemcpy(rp.data(), row_ptr, (rows + 1) * sizeof(int32_t), hipMemcpyDeviceToHost) !=
        hipSuccess)
      return VEDA_ERR_LAUNCH;
    if (rp[0] != 0 || rp[rows] != nnz) return VEDA_ERR_BAD_CSR;
    for (int64_t r = 0; r < rows; ++r)
      if (rp[r + 1] < rp[r]) return VEDA_ERR_BAD_CSR;
    std::vector<int32_t> ci(nnz);
    if (nnz > 0 && hipMemcpy(ci.data(), col_idx, nnz * sizeof(int32_t), hipMemcpyDeviceToHost) !=
                       hipSuccess)
      return VEDA_ERR_LAUNCH;
    for (int h = 0; h < L->num_heads; ++h)
      for (int64_t r = L->tile_off[h]; r < L->tile_off[h + 1]; ++r)
        for (int32_t p = rp[r]; p < rp[r + 1]; ++p) {
          if (ci[p] < 0 || ci[p] >= L->n_tiles[h]) return VEDA_ERR_BAD_CSR;
          if (p > rp[r] && ci[p] < ci[p - 1]) return VEDA_ERR_BAD_CSR;
        }
  }
  return VEDA_OK;
}

// Checks shared by the two distillation entry points (all but the workspace).
int distill_args(const veda_layout* L, const float* scores, const float* map,
                 const int32_t* q_tiles, int32_t n_sub, const float* desc, const float* phi,
                 int32_t d_e, const float* loss, const float* grad_w_q, const float* grad_w_k) {
  if (L == nullptr || !layout_ok(L)) return VEDA_ERR_INVALID_ARG;
  if (n_sub < 0 || d_e < 1) return VEDA_ERR_INVALID_ARG;
  if (desc == nullptr || phi == nullptr || loss == nullptr || grad_w_q == nullptr ||
      grad_w_k == nullptr)
    return VEDA_ERR_INVALID_ARG;
  if (n_sub > 0 && (scores == nullptr || map == nullptr || q_tiles == nullptr))
    return VEDA_ERR_INVALID_ARG;
  if (d_e > 256 || n_sub > VEDA_MAX_SUBSET) return VEDA_ERR_UNSUPPORTED;
  if (L->head_dim != 64 && L->head_dim != 128) return VEDA_ERR_UNSUPPORTED;
  return VEDA_OK;
}

}  // namespace
}  // namespace veda

using namespace veda;

extern "C" {

int veda_layout_init(veda_layout* L) {
  veda_layout d;
  if (!derive(L, &d)) return VEDA_ERR_INVALID_ARG;
  *L = d;
  return VEDA_OK;
}

int veda_keep_count(int32_t n_tiles, int32_t sparsity_pct, int32_t* k_out) {
  if (k_out == nullptr || n_tiles < 1 || sparsity_pct < 0 || sparsity_pct > 100)
    return VEDA_ERR_INVALID_ARG;
  const int64_t k = ceil_div((int64_t)n_tiles * (100 - sparsity_pct), 100);
  *k_out = (int32_t)(k < 1 ? 1 : k);
  return VEDA_OK;
}

int veda_tile_permute(const veda_layout* L, int32_t dtype, int32_t dir, const void* x, void* y,
                      void* stream) {
  if (L == nullptr || !layout_ok(L)) return VEDA_ERR_INVALID_ARG;
  if (dtype != VEDA_BF16 && dtype != VEDA_F32) return VEDA_ERR_INVALID_ARG;
  if (dir != VEDA_FWD && dir != VEDA_INV && dir != VEDA_FWD_T) return VEDA_ERR_INVALID_ARG;
  if (x == nullptr || y == nullptr) return VEDA_ERR_INVALID_ARG;
  const int esize = dtype == VEDA_F32 ? 4 : 2;
  if ((L->head_dim * esize) % 16 != 0) return VEDA_ERR_UNSUPPORTED;
  if (L->tile_size > 256) return VEDA_ERR_UNSUPPORTED;   // per-tile row table in LDS
  if (!aligned16(x) || !aligned16(y)) return VEDA_ERR_UNSUPPORTED;
  if (dir == VEDA_FWD_T) {
    if ((L->tile_size * esize) % 16 != 0) return VEDA_ERR_UNSUPPORTED;
    if (esize == 4 && (size_t)L->head_dim * (L->tile_size + 4) * 4 + 2048 > 65536)
      return VEDA_ERR_UNSUPPORTED;
  }
  const size_t tok = (size_t)L->T * L->H * L->W * L->num_heads * L->head_dim * esize;
  const size_t til = (size_t)L->tile_off[L->num_heads] * L->tile_size * L->head_dim * esize;
  if (!disjoint(x, dir == VEDA_INV ? til : tok, y, dir == VEDA_INV ? tok : til))
    return VEDA_ERR_INVALID_ARG;
  const DevLayout dl = make_dev_layout(L);
  return finish(launch_permute(dl, dtype, dir, x, y, (hipStream_t)stream), stream);
}

int veda_tripool_score(const veda_layout* L, int32_t dtype, const void* q_perm,
                       const void* k_perm, const float* w_q, const float* w_k, const float* b_q,
                       const float* b_k, int32_t d_e, float* desc, float* phi, float* scores,
                       void* stream) {
  if (L == nullptr || !layout_ok(L)) return VEDA_ERR_INVALID_ARG;
  if (dtype != VEDA_BF16 && dtype != VEDA_F32) return VEDA_ERR_INVALID_ARG;
  if (q_perm == nullptr || k_perm == nullptr || w_q == nullptr || w_k == nullptr ||
      desc == nullptr || phi == nullptr || scores == nullptr)
    return VEDA_ERR_INVALID_ARG;
  if (d_e < 1) return VEDA_ERR_INVALID_ARG;
  if (d_e > 256) return VEDA_ERR_UNSUPPORTED;
  if (L->head_dim != 64 && L->head_dim != 128) return VEDA_ERR_UNSUPPORTED;
  if (!aligned16(q_perm) || !aligned16(k_perm)) return VEDA_ERR_UNSUPPORTED;
  const DevLayout dl = make_dev_layout(L);
  return finish(launch_tripool_score(dl, dtype, q_perm, k_perm, w_q, w_k, b_q, b_k, d_e, desc, phi,
                                     scores, (hipStream_t)stream),
                stream);
}

int veda_tile_permute_pool(const veda_layout* L, int32_t dtype, const void* x, void* y,
                           float* desc, void* stream) {
  if (L == nullptr || !layout_ok(L)) return VEDA_ERR_INVALID_ARG;
  if (dtype != VEDA_BF16 && dtype != VEDA_F32) return VEDA_ERR_INVALID_ARG;
  if (x == nullptr || y == nullptr || desc == nullptr) return VEDA_ERR_INVALID_ARG;
  if (L->head_dim != 64 && L->head_dim != 128) return VEDA_ERR_UNSUPPORTED;
  if (L->tile_size > 256) return VEDA_ERR_UNSUPPORTED;   // per-tile row table in LDS
  if (!aligned16(x) || !aligned16(y)) return VEDA_ERR_UNSUPPORTED;
  const int esize = dtype == VEDA_F32 ? 4 : 2;
  const size_t tok = (size_t)L->T * L->H * L->W * L->num_heads * L->head_dim * esize;
  const size_t til = (size_t)L->tile_off[L->num_heads] * L->tile_size * L->head_dim * esize;
  const size_t dsc = (size_t)L->tile_off[L->num_heads] * 3 * L->head_dim * 4;
  if (!disjoint(x, tok, y, til) || !disjoint(x, tok, desc, dsc) || !disjoint(y, til, desc, dsc))
    return VEDA_ERR_INVALID_ARG;
  const DevLayout dl = make_dev_layout(L);
  return finish(launch_permute_pool(dl, dtype, x, y, desc, (hipStream_t)stream), stream);
}

int veda_tile_score(const veda_layout* L, const float* desc, const float* w_q, const float* w_k,
                    const float* b_q, const float* b_k, int32_t d_e, float* phi, float* scores,
                    void* stream) {
  if (L == nullptr || !layout_ok(L)) return VEDA_ERR_INVALID_ARG;
  if (desc == nullptr || w_q == nullptr || w_k == nullptr || phi == nullptr)
    return VEDA_ERR_INVALID_ARG;
  if (d_e < 1) return VEDA_ERR_INVALID_ARG;
  if (d_e > 256) return VEDA_ERR_UNSUPPORTED;
  if (L->head_dim != 64 && L->head_dim != 128) return VEDA_ERR_UNSUPPORTED;
  const DevLayout dl = make_dev_layout(L);
  return finish(launch_project_score(dl, desc, w_q, w_k, b_q, b_k, d_e, phi, scores,
                                     (hipStream_t)stream),
                stream);
}

int veda_score_select(const veda_layout* L, const float* phi, int32_t d_e,
                      const int32_t* k_per_head, int32_t* row_ptr, int32_t* col_idx,
                      void* stream) {
  if (L == nullptr || !layout_ok(L)) return VEDA_ERR_INVALID_ARG;
  if (phi == nullptr || k_per_head == nullptr || row_ptr == nullptr || col_idx == nullptr)
    return VEDA_ERR_INVALID_ARG;
  if (d_e < 1) return VEDA_ERR_INVALID_ARG;
  int64_t nnz = 0;
  for (int h = 0; h < L->num_heads; ++h) {
    if (k_per_head[h] < 1 || k_per_head[h] > L->n_tiles[h]) return VEDA_ERR_INVALID_ARG;
    nnz += (int64_t)L->n_tiles[h] * k_per_head[h];
  }
  if (nnz > INT32_MAX) return VEDA_ERR_INVALID_ARG;
  if ((d_e != 64 && d_e != 128) || !aligned16(phi)) return VEDA_ERR_UNSUPPORTED;
  if (L->max_tiles > score_select_max_cols()) return VEDA_ERR_UNSUPPORTED;
  const DevLayout dl = make_dev_layout(L);
  return finish(launch_score_select(dl, phi, d_e, k_per_head, row_ptr, col_idx,
                                    (hipStream_t)stream),
                stream);
}

int veda_select_tiles(const veda_layout* L, const float* scores, const int32_t* k_per_head,
                      int32_t* row_ptr, int32_t* col_idx, void* stream) {
  if (L == nullptr || !layout_ok(L)) return VEDA_ERR_INVALID_ARG;
  if (scores == nullptr || k_per_head == nullptr || row_ptr == nullptr || col_idx == nullptr)
    return VEDA_ERR_INVALID_ARG;
  int64_t nnz = 0;
  for (int h = 0; h < L->num_heads; ++h) {
    if (k_per_head[h] < 1 || k_per_head[h] > L->n_tiles[h]) return VEDA_ERR_INVALID_ARG;
    nnz += (int64_t)L->n_tiles[h] * k_per_head[h];
  }
  if (nnz > INT32_MAX) return VEDA_ERR_INVALID_ARG;
  if (L->max_tiles > 8192) return VEDA_ERR_UNSUPPORTED;
  const DevLayout dl = make_dev_layout(L);
  return finish(launch_select(dl, scores, k_per_head, row_ptr, col_idx, (hipStream_t)stream),
                stream);
}

int veda_sparse_attn_fwd_workspace(const veda_layout* L, int64_t* bytes) {
  if (L == nullptr || bytes == nullptr || !layout_ok(L)) return VEDA_ERR_INVALID_ARG;
  *bytes = kAttnWorkspaceBytes;
  return VEDA_OK;
}

int veda_sparse_attn_fwd(const veda_layout* L, const void* q_perm, const void* k_perm,
                         const void* vt_perm, const int32_t* row_ptr, const int32_t* col_idx,
                         float sm_scale, void* o_perm, float* lse, void* workspace,
                         int64_t workspace_bytes, void* stream) {
  if (workspace != nullptr && (workspace_bytes < kAttnWorkspaceBytes || !aligned16(workspace)))
    return VEDA_ERR_INVALID_ARG;
  const int st = attn_args(L, q_perm, k_perm, vt_perm, row_ptr, col_idx, sm_scale, o_perm, stream);
  if (st != VEDA_OK) return st;
  const DevLayout dl = make_dev_layout(L);
  return finish(launch_sparse_attn(dl, q_perm, k_perm, vt_perm, row_ptr, col_idx, sm_scale, o_perm,
                                   lse, false, static_cast<int*>(workspace), (hipStream_t)stream),
                stream);
}

int veda_sparse_attn_fwd_tokens(const veda_layout* L, const void* q_perm, const void* k_perm,
                                const void* vt_perm, const int32_t* row_ptr,
                                const int32_t* col_idx, float sm_scale, void* o, float* lse,
                                void* workspace, int64_t workspace_bytes, void* stream) {
  if (workspace != nullptr && (workspace_bytes < kAttnWorkspaceBytes || !aligned16(workspace)))
    return VEDA_ERR_INVALID_ARG;
  const int st = attn_args(L, q_perm, k_perm, vt_perm, row_ptr, col_idx, sm_scale, o, stream);
  if (st != VEDA_OK) return st;
  const size_t tok = (size_t)L->T * L->H * L->W * L->num_heads * L->head_dim * 2;
  const size_t til = (size_t)L->tile_off[L->num_heads] * L->tile_size * L->head_dim * 2;
  if (!disjoint(o, tok, q_perm, til) || !disjoint(o, tok, k_perm, til) ||
      !disjoint(o, tok, vt_perm, til))
    return VEDA_ERR_INVALID_ARG;
  const DevLayout dl = make_dev_layout(L);
  return finish(launch_sparse_attn(dl, q_perm, k_perm, vt_perm, row_ptr, col_idx, sm_scale, o, lse,
                                   true, static_cast<int*>(workspace), (hipStream_t)stream),
                stream);
}

int veda_sparse_attn_bwd_workspace(const veda_layout* L, int64_t nnz, int64_t* bytes) {
  if (L == nullptr || bytes == nullptr || !layout_ok(L) || nnz < 0 || nnz > INT32_MAX)
    return VEDA_ERR_INVALID_ARG;
  if (!tiles_per_head_ok(L)) return VEDA_ERR_UNSUPPORTED;
  *bytes = attn_bwd_workspace_bytes(make_dev_layout(L), nnz);
  return VEDA_OK;
}


int veda_sparse_attn_bwd(const veda_layout* L, const void* q, const void* k, const void* v,
                         const void* o, const void* d_o, const float* lse,
                         const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                         float sm_scale, void* workspace, int64_t workspace_bytes, void* dq,
                         void* dk, void* dv, void* stream) {
  const size_t tok = L ? (size_t)L->T * L->H * L->W * L->num_heads * L->head_dim * 2 : 0;
  const int st = bwd_args(L, q, k, tok, v, o, d_o, lse, row_ptr, col_idx, nnz, sm_scale,
                          workspace, workspace_bytes, dq, dk, dv, stream);
  if (st != VEDA_OK) return st;
  return finish(launch_sparse_attn_bwd(make_dev_layout(L), q, k, v, o, d_o, lse, row_ptr,
                                       col_idx, nnz, sm_scale, workspace, dq, dk, dv, false,
                                       (hipStream_t)stream),
                stream);
}

int veda_sparse_attn_bwd_tiles(const veda_layout* L, const void* q_perm, const void* k_perm,
                               const void* v, const void* o, const void* d_o, const float* lse,
                               const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                               float sm_scale, void* workspace, int64_t workspace_bytes,
                               void* dq, void* dk, void* dv, void* stream) {
  const size_t tiles = L && layout_ok(L)
                           ? (size_t)L->tile_off[L->num_heads] * L->tile_size * L->head_dim * 2
                           : 0;
  const int st = bwd_args(L, q_perm, k_perm, tiles, v, o, d_o, lse, row_ptr, col_idx, nnz,
                          sm_scale, workspace, workspace_bytes, dq, dk, dv, stream);
  if (st != VEDA_OK) return st;
  return finish(launch_sparse_attn_bwd(make_dev_layout(L), q_perm, k_perm, v, o, d_o, lse,
                                       row_ptr, col_idx, nnz, sm_scale, workspace, dq, dk, dv,
                                       true, (hipStream_t)stream),
                stream);
}

int veda_oracle_maxpool_map_workspace(const veda_layout* L, int32_t n_sub, int64_t* bytes) {
  if (L == nullptr || bytes == nullptr || !layout_ok(L) || n_sub < 0) return VEDA_ERR_INVALID_ARG;
  if (n_sub > VEDA_MAX_SUBSET || !tiles_per_head_ok(L)) return VEDA_ERR_UNSUPPORTED;
  *bytes = map_workspace_bytes(make_dev_layout(L), n_sub);
  return VEDA_OK;
}

int veda_oracle_maxpool_map(const veda_layout* L, const void* q_perm, const void* k_perm,
                            float sm_scale, const int32_t* q_tiles, int32_t n_sub,
                            void* workspace, int64_t workspace_bytes, float* lse, float* map,
                            void* stream) {
  if (L == nullptr || !layout_ok(L)) return VEDA_ERR_INVALID_ARG;
  if (n_sub < 0) return VEDA_ERR_INVALID_ARG;
  if (n_sub > VEDA_MAX_SUBSET) return VEDA_ERR_UNSUPPORTED;   // keeps both grids in range
  if (n_sub > 0 && (q_perm == nullptr || k_perm == nullptr || q_tiles == nullptr ||
                    lse == nullptr || map == nullptr || workspace == nullptr))
    return VEDA_ERR_INVALID_ARG;
  if (!(sm_scale > 0.f) || sm_scale == INFINITY) return VEDA_ERR_INVALID_ARG;
  if (!attn_shape_ok(L) || !tiles_per_head_ok(L)) return VEDA_ERR_UNSUPPORTED;
  const DevLayout dl = make_dev_layout(L);
  if (n_sub > 0 && workspace_bytes < map_workspace_bytes(dl, n_sub)) return VEDA_ERR_INVALID_ARG;
  if (n_sub > 0 && (!aligned16(q_perm) || !aligned16(k_perm) || !aligned16(workspace)))
    return VEDA_ERR_UNSUPPORTED;
  return finish(launch_oracle_map(dl, q_perm, k_perm, sm_scale, q_tiles, n_sub, workspace, lse,
                                  map, (hipStream_t)stream),
                stream);
}

int veda_distill_grad_workspace(const veda_layout* L, int32_t n_sub, int32_t d_e,
                                int64_t* bytes) {
  if (L == nullptr || bytes == nullptr || !layout_ok(L) || n_sub < 0 || d_e < 1)
    return VEDA_ERR_INVALID_ARG;
  if (n_sub > VEDA_MAX_SUBSET) return VEDA_ERR_UNSUPPORTED;
  *bytes = distill_workspace_bytes(make_dev_layout(L), n_sub, d_e);
  return VEDA_OK;
}

int veda_distill_grad(const veda_layout* L, const float* scores, const float* map,
                      const int32_t* q_tiles, int32_t n_sub, const float* desc, const float* phi,
                      int32_t d_e, void* workspace, int64_t workspace_bytes, float* loss,
                      float* grad_w_q, float* grad_w_k, float* grad_b_q, float* grad_b_k,
                      void* stream) {
  const int st = distill_args(L, scores, map, q_tiles, n_sub, desc, phi, d_e, loss, grad_w_q,
                              grad_w_k);
  if (st != VEDA_OK) return st;
  if (workspace == nullptr) return VEDA_ERR_INVALID_ARG;
  const DevLayout dl = make_dev_layout(L);
  if (workspace_bytes < distill_workspace_bytes(dl, n_sub, d_e)) return VEDA_ERR_INVALID_ARG;
  if (!aligned16(workspace)) return VEDA_ERR_UNSUPPORTED;
  return finish(launch_distill(dl, scores, map, q_tiles, n_sub, desc, phi, d_e, workspace, loss,
                               grad_w_q, grad_w_k, grad_b_q, grad_b_k, (hipStream_t)stream),
                stream);
}

int veda_distill_grad_noalloc(const veda_layout* L, const float* scores, const float* map,
                              const int32_t* q_tiles, int32_t n_sub, const float* desc,
                              const float* phi, int32_t d_e, float* loss, float* grad_w_q,
                              float* grad_w_k, float* grad_b_q, float* grad_b_k, void* stream) {
  const int st = distill_args(L, scores, map, q_tiles, n_sub, desc, phi, d_e, loss, grad_w_q,
                              grad_w_k);
  if (st != VEDA_OK) return st;
  const DevLayout dl = make_dev_layout(L);
  if (distill_workspace_bytes(dl, n_sub, d_e) > VEDA_DISTILL_STATIC_SCRATCH_BYTES)
    return VEDA_ERR_UNSUPPORTED;
  void* scratch_ptr = nullptr;
  const int ss = distill_static_scratch(&scratch_ptr);
  if (ss != VEDA_OK) return ss;
  return finish(launch_distill(dl, scores, map, q_tiles, n_sub, desc, phi, d_e, scratch_ptr, loss,
                               grad_w_q, grad_w_k, grad_b_q, grad_b_k, (hipStream_t)stream),
                stream);
}

int veda_head_sq_error_workspace(const veda_layout* L, int64_t* bytes) {
  if (L == nullptr || bytes == nullptr || !layout_ok(L)) return VEDA_ERR_INVALID_ARG;
  *bytes = head_error_workspace_bytes(make_dev_layout(L));
  return VEDA_OK;
}

int veda_head_sq_error(const veda_layout* L, const void* a, const void* b, double* err,
                       double* ref, void* workspace, int64_t workspace_bytes, void* stream) {
  if (L == nullptr || !layout_ok(L)) return VEDA_ERR_INVALID_ARG;
  if (a == nullptr || b == nullptr || err == nullptr || workspace == nullptr)
    return VEDA_ERR_INVALID_ARG;
  if (L->head_dim % 8 != 0 || 256 % (L->head_dim / 8) != 0) return VEDA_ERR_UNSUPPORTED;
  if (!aligned16(a) || !aligned16(b) || ((uintptr_t)workspace & 7u) != 0)
    return VEDA_ERR_UNSUPPORTED;
  const DevLayout dl = make_dev_layout(L);
  if (workspace_bytes < head_error_workspace_bytes(dl)) return VEDA_ERR_INVALID_ARG;
  return finish(launch_head_error(dl, a, b, err, ref, workspace, (hipStream_t)stream), stream);
}

int veda_head_choose(const double* err, int32_t n_cand, int32_t num_heads, int32_t* choice,
                     void* stream) {
  if (err == nullptr || choice == nullptr) return VEDA_ERR_INVALID_ARG;
  if (n_cand < 1 || n_cand > VEDA_MAX_CANDIDATES || num_heads < 1 || num_heads > VEDA_MAX_HEADS)
    return VEDA_ERR_INVALID_ARG;
  if (((uintptr_t)err & 7u) != 0 || ((uintptr_t)choice & 3u) != 0) return VEDA_ERR_INVALID_ARG;
  return finish(launch_head_choose(err, n_cand, num_heads, choice, (hipStream_t)stream), stream);
}

int64_t veda_layout_sizeof(void) { return (int64_t)sizeof(veda_layout); }

const char* veda_status_string(int status) {
  switch (status) {
    case VEDA_OK: return "VEDA_OK";
    case VEDA_ERR_INVALID_ARG: return "VEDA_ERR_INVALID_ARG: invalid argument";
    case VEDA_ERR_UNSUPPORTED: return "VEDA_ERR_UNSUPPORTED: outside the supported set";
    case VEDA_ERR_LAUNCH: return "VEDA_ERR_LAUNCH: HIP launch or kernel failure";
    case VEDA_ERR_BAD_CSR: return "VEDA_ERR_BAD_CSR: invalid CSR";
    default: return "unknown veda status";
  }
}

}  // extern "C"
