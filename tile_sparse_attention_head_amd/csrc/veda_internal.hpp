// Internal declarations shared by the HIP kernels and the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "veda.h"

namespace veda {

// Geometry handed to kernels by value (kernel-argument memory, scalar loads).
struct DevLayout {
  int32_t T, H, W;
  int32_t heads;
  int32_t d;
  int32_t S;
  int32_t max_tiles;
  int32_t pad0;
  int32_t shape[VEDA_MAX_HEADS][3];   // pt, ph, pw
  int32_t grid[VEDA_MAX_HEADS][3];    // nT, nH, nW
  int64_t tile_off[VEDA_MAX_HEADS + 1];
  int64_t score_off[VEDA_MAX_HEADS + 1];
};

DevLayout make_dev_layout(const veda_layout* L);

// Head owning global tile index g (tile_off[h] <= g < tile_off[h+1]).  The
// value is uniform across a workgroup, so this runs on the scalar unit.
__device__ __forceinline__ int head_of_tile(const DevLayout& L, int64_t g) {
  int h = 0;
  while (h + 1 < L.heads && g >= L.tile_off[h + 1]) ++h;
  return h;
}

// Number of real slots along each axis of tile j of head h, i.e. how much of
// the (pt, ph, pw) box lies inside the T x H x W grid.
// a / b for 0 <= a < 2^20 and b >= 1, given r = small_rcp(b): a multiply and
// two conversions instead of an integer division (about 30 vector
// instructions).  (a + 1/2)/b lies at least 1/(2b) from the integers on either
// side, and r (within 1 ulp of 1/b) and the rounded product move it by less
// than (a + 1/2) 1.6 2^-23 / b < 1/(5b), so the truncation is the quotient.
__device__ __forceinline__ float small_rcp(int b) { return __builtin_amdgcn_rcpf((float)b); }
__device__ __forceinline__ int small_div(int a, float r) {
  return (int)(((float)a + 0.5f) * r);
}

struct TileExtent {
  int it, ih, iw;      // tile coordinates
  int lt, lh, lw;      // real extent along t, h, w (<= pt, ph, pw)
  int pt, ph, pw;
  __device__ __forceinline__ bool full() const { return lt == pt && lh == ph && lw == pw; }
  __device__ __forceinline__ int count() const { return lt * lh * lw; }
  // slot u = (dt*ph + dh)*pw + dw, 0 <= u < 2^20
  __device__ __forceinline__ void slot_coords(int u, int& dt, int& dh, int& dw) const {
    const int r = small_div(u, small_rcp(pw));
    dw = u - r * pw;
    dt = small_div(r, small_rcp(ph));
    dh = r - dt * ph;
  }
  // slot u is real iff dt < lt, dh < lh, dw < lw
  __device__ __forceinline__ bool slot_real(int u) const {
    int dt, dh, dw;
    slot_coords(u, dt, dh, dw);
    return dt < lt && dh < lh && dw < lw;
  }
};

// Tile j (0 <= j < 2^20) of head h: j = (it nH + ih) nW + iw.
__device__ __forceinline__ TileExtent tile_extent(const DevLayout& L, int h, int j) {
  TileExtent e;
  e.pt = L.shape[h][0]; e.ph = L.shape[h][1]; e.pw = L.shape[h][2];
  const int nH = L.grid[h][1], nW = L.grid[h][2];
  const int q = small_div(j, small_rcp(nW));   // j / nW
  e.iw = j - q * nW;
  e.it = small_div(q, small_rcp(nH));          // j / (nW nH)
  e.ih = q - e.it * nH;
  e.lt = min(e.pt, L.T - e.it * e.pt);
  e.lh = min(e.ph, L.H - e.ih * e.ph);
  e.lw = min(e.pw, L.W - e.iw * e.pw);
  return e;
}

// Workgroups of a launch in lockstep XCD order (attn::lockstep_tile): 8 times
// the longest of the 8 per-XCD runs, each the sum over heads of one eighth of
// the head's tiles.
inline int64_t lockstep_grid(const DevLayout& L) {
  int64_t longest = 0;
  for (int x = 0; x < 8; ++x) {
    int64_t run = 0;
    for (int h = 0; h < L.heads; ++h) {
      const int64_t n = L.tile_off[h + 1] - L.tile_off[h];
      run += n * (x + 1) / 8 - n * x / 8;
    }
    if (run > longest) longest = run;
  }
  return 8 * longest;
}

// Launchers (each returns a veda_status; arguments already validated).
int launch_permute(const DevLayout& L, int dtype, int dir, const void* x, void* y,
                   hipStream_t s);
int launch_tripool_score(const DevLayout& L, int dtype, const void* q, const void* k,
                         const float* wq, const float* wk, const float* bq,
                         const float* bk, int d_e, float* desc, float* phi,
                         float* scores, hipStream_t s);
int launch_permute_pool(const DevLayout& L, int dtype, const void* x, void* y, float* desc,
                        hipStream_t s);
int launch_project_score(const DevLayout& L, const float* desc, const float* wq,
                         const float* wk, const float* bq, const float* bk, int d_e,
                         float* phi, float* scores, hipStream_t s);
int launch_select(const DevLayout& L, const float* scores, const int32_t* k_host,
                  int32_t* row_ptr, int32_t* col_idx, hipStream_t s);
// the score product fused with the selection: d_e in {64, 128}, max_tiles
// <= score_select_max_cols()
int launch_score_select(const DevLayout& L, const float* phi, int d_e, const int32_t* k_host,
                        int32_t* row_ptr, int32_t* col_idx, hipStream_t s);
int score_select_max_cols();
// claim: 8 work counters in the caller's workspace, or nullptr (fixed
// XCD shares)
constexpr int64_t kAttnWorkspaceBytes = 256;
int launch_sparse_attn(const DevLayout& L, const void* q, const void* k, const void* vt,
                       const int32_t* row_ptr, const int32_t* col_idx, float sm_scale,
                       void* o, float* lse, bool tokens, int* claim, hipStream_t s);
int launch_oracle_map(const DevLayout& L, const void* q, const void* k, float sm_scale,
                      const int32_t* q_tiles, int n_sub, void* workspace, float* lse,
                      float* map, hipStream_t s);
// Bytes of workspace the map needs (row maxima, then per-chunk partial sums).
int64_t map_workspace_bytes(const DevLayout& L, int64_t n_sub);

// Distillation step: workspace bytes, and the launch.
int64_t distill_workspace_bytes(const DevLayout& L, int64_t n_sub, int d_e);
int launch_distill(const DevLayout& L, const float* scores, const float* map,
                   const int32_t* q_tiles, int n_sub, const float* desc, const float* phi,
                   int d_e, void* workspace, float* loss, float* dwq, float* dwk, float* dbq,
                   float* dbk, hipStream_t s);

// Device address, on the current device, of the library's static scratch for
// veda_distill_grad_noalloc (VEDA_DISTILL_STATIC_SCRATCH_BYTES); looked up on
// the first call per device.  VEDA_OK, or VEDA_ERR_LAUNCH if HIP refuses.
int distill_static_scratch(void** ptr);

// Per-head squared error of two token-order outputs (tiling search).
int64_t head_error_workspace_bytes(const DevLayout& L);
int launch_head_error(const DevLayout& L, const void* a, const void* b, double* err, double* ref,
                      void* workspace, hipStream_t s);
int launch_head_choose(const double* err, int n_cand, int heads, int32_t* choice, hipStream_t s);

// Attention backward: workspace bytes for a CSR of nnz entries, and the launch.
int64_t attn_bwd_workspace_bytes(const DevLayout& L, int64_t nnz);
// qk_tiles: q and k are already in tile order (their gathers are skipped).
int launch_sparse_attn_bwd(const DevLayout& L, const void* q, const void* k, const void* v,
                           const void* o, const void* d_o, const float* lse,
                           const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                           float sm_scale, void* workspace, void* dq, void* dk, void* dv,
                           bool qk_tiles, hipStream_t s);

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? VEDA_OK : VEDA_ERR_LAUNCH;
}

}  // namespace veda
