/*
 * veda.h -- C ABI of the tile-sparse self-attention hot path (libveda.so).
 *
 * The method: "Veda: Scalable Video Diffusion via Distilled Sparse Attention"
 * (technical summary on gist.science; zh/fr/es editions share the section
 * numbers cited here as "Veda §x") and the aikraft.ru news item on Veda
 * ("Veda news").  For one attention layer of a video DiT whose tokens form a
 * T x H x W latent grid, the path is:
 *
 *   veda_tile_permute(FWD)    tokens -> per-head tiles       (Veda §2.2)
 *   veda_tripool_score        TripPool + per-head projection
 *                             + tile-pair scores             (Veda §2.1)
 *   veda_select_tiles         row-wise top-k -> CSR          (Veda lay summary, §5)
 *   veda_sparse_attn_fwd      tile-skipping attention        (Veda §2.3)
 *   veda_tile_permute(INV)    tiles -> tokens
 *   veda_oracle_maxpool_map   two-pass max-pooled attention
 *                             map (distillation target)      (Veda §2.1, §2.3)
 *
 * with fused forms of the same steps (veda_tile_permute_pool: gather +
 * TripPool; veda_tile_score: projection + scores from the descriptors;
 * veda_score_select: scores + top-k without the score matrix;
 * veda_sparse_attn_fwd_tokens: attention + inverse permutation), and the
 * further calls of the method: the distillation step, the tiling search's
 * error and choice, and the attention backward.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked (host).  The caller owns all
 *    memory; the library never allocates, frees or retains a pointer.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Device calls are
 *    enqueued on it asynchronously; the library never synchronises, except
 *    when the environment variable VEDA_DEBUG_SYNC=1 is set (then every call
 *    synchronises and reports kernel failures, and veda_sparse_attn_fwd
 *    validates the CSR on the host first).
 *  - Every argument is validated on the host before anything is enqueued.  An
 *    invalid argument returns a negative veda_status and enqueues nothing.
 *  - Calls keep no state between them and may be made from several threads.
 *    No call enqueues a memset (the kernels clear their own counters), so a
 *    sequence of calls can be captured in a HIP graph and replayed.
 *  - bf16 is the IEEE-754 binary32 high half (bfloat16); f32 is binary32.
 *
 * Token and tile order (the pages leave these open; the readings taken):
 *  - token n of a [N][heads][d] tensor sits at grid point (t, h, w) with
 *    n = (t*H + h)*W + w;
 *  - head `hd` with tile shape (pt, ph, pw), pt*ph*pw = tile_size = S, has
 *    nT*nH*nW tiles, nT = ceil(T/pt) etc.: every grid dimension is padded up
 *    to whole tiles and the slots outside the grid are padding;
 *  - tile j = (it*nH + ih)*nW + iw, slot u = (dt*ph + dh)*pw + dw holds the
 *    token (it*pt + dt, ih*ph + dh, iw*pw + dw) when it lies in the grid;
 *  - "tile order" tensors are [sum_h n_tiles[h]*S][d]: head hd occupies rows
 *    tile_off[hd]*S .. tile_off[hd+1]*S - 1, tile j of that head the S rows
 *    from (tile_off[hd] + j)*S.  Padding rows hold zeros.
 *  - "tile-transposed" tensors hold each tile as a [d][S] block instead of
 *    [S][d] (same per-tile offsets); the attention kernel takes V this way.
 */
#ifndef VEDA_H
#define VEDA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VEDA_MAX_HEADS 64
#define VEDA_MAX_SUBSET (1 << 20) /* most query-tile subset entries of one map or distillation call */
/* Most tiles one head may have in the calls that read K/V tiles through a
 * buffer resource (attention forward and backward, the max-pooled map): a
 * head's tile-order K or V must span at most 2^31 - 1 bytes, and the forward
 * packs a tile index into 16 bits.  Larger: VEDA_ERR_UNSUPPORTED.
 * veda_layout_init already keeps sum_h n_tiles[h]^2 (the CSR entry bound)
 * within int32, so an accepted layout has at most 46340 tiles per head; the
 * calls check this limit anyway. */
#define VEDA_MAX_TILES_PER_HEAD 65535

typedef enum veda_status {
  VEDA_OK = 0,
  VEDA_ERR_INVALID_ARG = -1, /* null pointer, bad size, bad enum, bad layout    */
  VEDA_ERR_UNSUPPORTED = -2, /* valid but outside the built set (see each call) */
  VEDA_ERR_LAUNCH = -3,      /* the HIP runtime refused or failed a launch      */
  VEDA_ERR_BAD_CSR = -4      /* debug validation found an invalid CSR           */
} veda_status;

typedef enum veda_dtype { VEDA_BF16 = 0, VEDA_F32 = 1 } veda_dtype;

typedef enum veda_dir {
  VEDA_FWD = 0,   /* token order -> tile order                    */
  VEDA_INV = 1,   /* tile order -> token order (real slots only)  */
  VEDA_FWD_T = 2  /* token order -> tile-transposed order         */
} veda_dir;

/* Geometry of one attention layer.  The caller fills the inputs and calls
 * veda_layout_init, which checks them and fills the derived fields. */
typedef struct veda_layout {
  /* inputs */
  int32_t T, H, W;                           /* latent grid: frames, height, width */
  int32_t num_heads;                         /* 1 .. VEDA_MAX_HEADS                 */
  int32_t head_dim;                          /* d                                   */
  int32_t tile_size;                         /* S = pt*ph*pw for every head         */
  int32_t tile_shape[VEDA_MAX_HEADS][3];     /* per head (pt, ph, pw)               */
  /* derived by veda_layout_init */
  int32_t tile_grid[VEDA_MAX_HEADS][3];      /* per head (nT, nH, nW)               */
  int32_t n_tiles[VEDA_MAX_HEADS];           /* per head nT*nH*nW                   */
  int32_t max_tiles;                         /* max over heads of n_tiles           */
  int32_t reserved0;
  int64_t tile_off[VEDA_MAX_HEADS + 1];      /* prefix sum of n_tiles               */
  int64_t score_off[VEDA_MAX_HEADS + 1];     /* prefix sum of n_tiles^2             */
} veda_layout;

/* Host only.  Veda §2.2: each head has its own tile shape (pt, ph, pw) whose
 * volume is the hardware tile.  Checks T, H, W >= 1, 1 <= num_heads <=
 * VEDA_MAX_HEADS, head_dim >= 1, tile_size >= 1, every shape positive with
 * pt*ph*pw == tile_size, and that every offset fits int32 row/column indices
 * of the CSR; fills the derived fields.  VEDA_ERR_INVALID_ARG otherwise. */
int veda_layout_init(veda_layout* L);

/* Host only.  Key tiles kept per query tile at `sparsity_pct` percent tile
 * sparsity (Veda: 95 % sparsity keeps about 5 % of the tiles):
 * k = max(1, ceil(n_tiles * (100 - sparsity_pct) / 100)) in integer
 * arithmetic.  Needs n_tiles >= 1 and 0 <= sparsity_pct <= 100 and a non-null
 * (host) k_out; VEDA_ERR_INVALID_ARG otherwise. */
int veda_keep_count(int32_t n_tiles, int32_t sparsity_pct, int32_t* k_out);

/* Veda §2.2 (head-aware tiling); Veda news (head-conditioned tile geometry).
 * FWD:   x [N][num_heads][d] (token order)  -> y tile order   [tile_off*S][d]
 * FWD_T: x [N][num_heads][d]                -> y tile-transposed order
 * INV:   x tile order                       -> y [N][num_heads][d]
 * FWD/FWD_T write zeros to padding slots; INV reads only real slots and
 * writes every element of y.  Pure data movement: bit-exact.
 * dtype VEDA_BF16 or VEDA_F32 (element size 2 or 4 bytes).  Supported:
 * head_dim*element_size a multiple of 16 bytes, tile_size <= 256, pointers
 * 16-byte aligned; FWD_T also needs tile_size*element_size a multiple of 16
 * bytes and, for F32, head_dim*(tile_size+4)*4 + 2048 <= 65536
 * (VEDA_ERR_UNSUPPORTED otherwise).  x and y must not overlap. */
int veda_tile_permute(const veda_layout* L, int32_t dtype, int32_t dir,
                      const void* x, void* y, void* stream);

/* Veda §2.1 (distilled tile scoring): TripPool descriptor per tile, per-head
 * projection, tile-pair scores.  Per head hd and tile j, over the tile's real
 * slots and per channel:
 *   desc[side][tile_off[hd]+j] = [mean | max | min]               (3d floats)
 *   phi[side][tile_off[hd]+j]  = W_side[hd] desc + b_side[hd]     (d_e floats)
 *   scores[score_off[hd] + i*n_tiles[hd] + j] = <phi[0][..i], phi[1][..j]>
 * side 0 uses q_perm/w_q/b_q, side 1 k_perm/w_k/b_k.
 *  q_perm, k_perm  tile order, dtype `dtype` (VEDA_BF16 or VEDA_F32)
 *  w_q, w_k        f32 [num_heads][d_e][3*head_dim] (may be the same pointer)
 *  b_q, b_k        f32 [num_heads][d_e], or NULL for no bias
 *  desc            f32 [2][tile_off[num_heads]][3*head_dim]  (output)
 *  phi             f32 [2][tile_off[num_heads]][d_e]         (output)
 *  scores          f32 [score_off[num_heads]]                (output)
 * Arithmetic in f32.  Supported: head_dim in {64, 128}, 1 <= d_e <= 256,
 * 16-byte aligned q_perm/k_perm. */
int veda_tripool_score(const veda_layout* L, int32_t dtype, const void* q_perm,
                       const void* k_perm, const float* w_q, const float* w_k,
                       const float* b_q, const float* b_k, int32_t d_e,
                       float* desc, float* phi, float* scores, void* stream);

/* The gather of Q or K fused with TripPool (Veda §2.1 TripPool descriptor,
 * §2.2 head-aware tiling): one read of x gives both
 *   y     tile order, exactly as veda_tile_permute FWD writes it
 *   desc  f32 [tile_off[num_heads]][3*head_dim] (output): per tile
 *         [mean | max | min] of each channel over the tile's real slots,
 *         bit-identical to the desc rows veda_tripool_score writes
 * For a layer, call it for Q with desc = D and for K with
 * desc = D + tile_off[num_heads]*3*head_dim, where D is the [2][tiles][3d]
 * buffer veda_tile_score reads.  dtype VEDA_BF16 or VEDA_F32.  Supported:
 * head_dim in {64, 128}, tile_size <= 256, x and y 16-byte aligned
 * (VEDA_ERR_UNSUPPORTED otherwise).  x, y and desc must not overlap. */
int veda_tile_permute_pool(const veda_layout* L, int32_t dtype, const void* x, void* y,
                           float* desc, void* stream);

/* The projection and score half of veda_tripool_score (Veda §2.1), from
 * descriptors already computed (by veda_tile_permute_pool or
 * veda_tripool_score):
 *  desc    f32 [2][tile_off[num_heads]][3*head_dim]: side 0 Q, side 1 K
 *  w_q, w_k, b_q, b_k, d_e, phi  as in veda_tripool_score
 *  scores  as in veda_tripool_score, or NULL: the projection alone (phi for
 *          veda_score_select)
 * Same kernels and results as veda_tripool_score.  Supported: head_dim in
 * {64, 128}, 1 <= d_e <= 256. */
int veda_tile_score(const veda_layout* L, const float* desc, const float* w_q,
                    const float* w_k, const float* b_q, const float* b_k, int32_t d_e,
                    float* phi, float* scores, void* stream);

/* Tile selection (Veda lay summary and §5; Veda news: 95 % sparsity): per
 * query tile row, keep the k_per_head[hd] largest scores; equal scores prefer
 * the lower tile index, -0.0 equals +0.0, NaN ranks below every number.
 *  scores      f32 as written by veda_tripool_score
 *  k_per_head  (host) int32 [num_heads], 1 <= k <= n_tiles[hd]
 *  row_ptr     int32 [tile_off[num_heads] + 1] (output): head-major rows,
 *              row_ptr[tile_off[hd] + i] = sum_{h<hd} n_h*k_h + i*k_hd
 *  col_idx     int32 [row_ptr[last]] (output): head-local tile indices,
 *              ascending within each row
 * Bit-exact and deterministic.  Supported: max_tiles <= 8192. */
int veda_select_tiles(const veda_layout* L, const float* scores,
                      const int32_t* k_per_head, int32_t* row_ptr,
                      int32_t* col_idx, void* stream);

/* The tile-score product fused with the tile selection (Veda §2.1 scores,
 * <phi_Q,i, phi_K,j>; lay summary and §5: keep the top fraction of tiles):
 * the CSR that veda_tile_score followed by veda_select_tiles writes, with the
 * n_tiles x n_tiles score matrix of each head never stored.
 *  phi         f32 [2][tile_off[num_heads]][d_e] as veda_tile_score writes it
 *              (scores may be NULL there), 16-byte aligned
 *  d_e         64 or 128
 *  k_per_head, row_ptr, col_idx  as in veda_select_tiles
 * Each score is the same f32 value veda_tile_score writes (the same product
 * order), so row_ptr and col_idx are bit-identical to the two-call path, and
 * deterministic.  Arguments outside veda_select_tiles' rules:
 * VEDA_ERR_INVALID_ARG.  Supported: d_e in {64, 128}, phi 16-byte aligned,
 * max_tiles <= 2048 (VEDA_ERR_UNSUPPORTED otherwise). */
int veda_score_select(const veda_layout* L, const float* phi, int32_t d_e,
                      const int32_t* k_per_head, int32_t* row_ptr, int32_t* col_idx,
                      void* stream);

/* Tile-skipping attention forward (Veda §2.3).  For every query tile of every
 * head, softmax(sm_scale * Q K^T) V over the real key slots of the key tiles
 * its CSR row lists (any other tile is never read), computed with online
 * softmax, bf16 matrix-core products and f32 accumulation.
 *  q_perm, k_perm  bf16, tile order
 *  vt_perm         bf16, tile-transposed order (veda_tile_permute FWD_T)
 *  row_ptr,col_idx CSR as written by veda_select_tiles (any valid CSR:
 *                  row_ptr non-decreasing, entries in [0, n_tiles[hd]))
 *  o_perm          bf16, tile order (output); padding query rows unspecified
 *  lse             f32 [tile_off[num_heads]*S] natural-log log-sum-exp per
 *                  query slot (padding slots unspecified), or NULL (output)
 *  sm_scale        finite and > 0 (else VEDA_ERR_INVALID_ARG)
 *  workspace       device scratch of at least workspace_bytes >=
 *                  veda_sparse_attn_fwd_workspace(L) bytes, 16-byte aligned,
 *                  owned by the caller, contents on entry and exit
 *                  unspecified; or NULL (workspace_bytes ignored).  With it,
 *                  the query tiles at the end of each XCD's share are handed
 *                  out through counters in it (reset by a small kernel on
 *                  `stream` first), so that XCDs that run faster take them
 *                  over; without it every tile keeps its fixed XCD.  The
 *                  results are the same bits either way.  Calls sharing a
 *                  workspace must be ordered on one stream.  Too small or
 *                  misaligned: VEDA_ERR_INVALID_ARG.
 * A query row whose CSR row is empty gets O = 0 and lse = -inf.  Entries of
 * col_idx outside [0, n_tiles[hd]) are skipped.  Supported: (head_dim,
 * tile_size) in {(64,64), (128,128)}, 16-byte aligned tensors, max_tiles <=
 * VEDA_MAX_TILES_PER_HEAD. */
int veda_sparse_attn_fwd(const veda_layout* L, const void* q_perm, const void* k_perm,
                         const void* vt_perm, const int32_t* row_ptr,
                         const int32_t* col_idx, float sm_scale, void* o_perm,
                         float* lse, void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes veda_sparse_attn_fwd and veda_sparse_attn_fwd_tokens use
 * (the same for any layout: eight counters).  Host-only, no device work.
 *  bytes  (host) output */
int veda_sparse_attn_fwd_workspace(const veda_layout* L, int64_t* bytes);

/* veda_sparse_attn_fwd with the inverse permutation folded into its
 * epilogue (Veda §2.3 tile-skipping kernel, §2.2 tiles): the same O values,
 * written straight to token order.
 *  o       bf16 [N][num_heads][head_dim] (output): every element is written
 *          (each token is a real slot of exactly one tile per head); must not
 *          overlap the inputs
 *  lse     as in veda_sparse_attn_fwd (tile-slot order), or NULL
 * Every other argument, result and limit as veda_sparse_attn_fwd. */
int veda_sparse_attn_fwd_tokens(const veda_layout* L, const void* q_perm, const void* k_perm,
                                const void* vt_perm, const int32_t* row_ptr,
                                const int32_t* col_idx, float sm_scale, void* o,
                                float* lse, void* workspace, int64_t workspace_bytes,
                                void* stream);

/* Backward of the tile-skipping attention (Veda §2.3 kernel; the pages
 * fine-tune with the sparse path in place but give no backward kernel): the
 * gradients of the forward's output with respect to Q, K and V over exactly
 * the kept tiles of the forward's CSR.  With P the forward's softmax of query
 * row r over its kept real keys, D_r = dO_r . O_r:
 *   dV_c = sum_r P_rc dO_r,  dS_rc = P_rc (dO_r . V_c - D_r),
 *   dQ_r = sm_scale sum_c dS_rc K_c,  dK_c = sm_scale sum_r dS_rc Q_r
 * (a tile listed twice in a row contributes twice, as in the forward).
 *  q, k, v     bf16 [N][num_heads][head_dim], token order (the forward's inputs)
 *  o           bf16 token order: the forward's output (veda_sparse_attn_fwd_tokens)
 *  d_o         bf16 token order: gradient of the loss with respect to o
 *  lse         f32 [tile_off[num_heads]*S]: the forward's log-sum-exp (tile-slot order)
 *  row_ptr, col_idx  the forward's CSR, each row's entries ascending (as
 *              veda_select_tiles writes them); entries outside [0, n_tiles[hd])
 *              are skipped.  nnz = row_ptr[tile_off[num_heads]] (host value)
 *  workspace   at least veda_sparse_attn_bwd_workspace(L, nnz) bytes,
 *              16-byte aligned; holds the gathered operands, D and the
 *              accumulator seeds, the transposed CSR and the order the key
 *              tiles are processed in; contents unspecified on entry and exit
 *  dq, dk, dv  bf16 token order (outputs): every element is written; a key
 *              tile no row keeps gets dK = dV = 0, an empty row dQ = 0; must
 *              not overlap the inputs
 * bf16 matrix-core products with f32 accumulation; deterministic.  A row that
 * is not sorted gives wrong gradients (never an out-of-bounds access); with
 * VEDA_DEBUG_SYNC=1 the CSR (monotone rows, in-range and ascending entries,
 * nnz) is checked and VEDA_ERR_BAD_CSR returned.  Supported: (head_dim,
 * tile_size) in {(64,64), (128,128)}, 16-byte aligned tensors, max_tiles <=
 * VEDA_MAX_TILES_PER_HEAD. */
int veda_sparse_attn_bwd(const veda_layout* L, const void* q, const void* k, const void* v,
                         const void* o, const void* d_o, const float* lse,
                         const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                         float sm_scale, void* workspace, int64_t workspace_bytes, void* dq,
                         void* dk, void* dv, void* stream);

/* veda_sparse_attn_bwd with Q and K already in tile order, as the forward's
 * gathers left them (veda_tile_permute_pool / veda_tile_permute FWD): their
 * two gathers are skipped.  Same results, bit for bit, as
 * veda_sparse_attn_bwd on the token-order tensors they were gathered from.
 *  q_perm, k_perm  bf16 [tile_off[num_heads]*S][head_dim], tile order,
 *              zero padding slots
 *  workspace   at least veda_sparse_attn_bwd_workspace(L, nnz) bytes
 * Every other argument, result and limit as veda_sparse_attn_bwd (dq, dk, dv
 * must not overlap q_perm or k_perm either). */
int veda_sparse_attn_bwd_tiles(const veda_layout* L, const void* q_perm, const void* k_perm,
                               const void* v, const void* o, const void* d_o, const float* lse,
                               const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                               float sm_scale, void* workspace, int64_t workspace_bytes,
                               void* dq, void* dk, void* dv, void* stream);

/* Workspace bytes veda_sparse_attn_bwd and veda_sparse_attn_bwd_tiles need
 * for a CSR of nnz entries.  Host-only.  bytes (host) output.  max_tiles
 * above VEDA_MAX_TILES_PER_HEAD: VEDA_ERR_UNSUPPORTED. */
int veda_sparse_attn_bwd_workspace(const veda_layout* L, int64_t nnz, int64_t* bytes);

/* Max-pooled attention map, the distillation target (Veda §2.1 target
 * construction; Veda §2.3: two passes over a random subset of query tiles).
 * For subset entry s, q_tiles[s] = global tile index g (tile_off[hd] <= g <
 * tile_off[hd+1]); pass 1 gives each real query row r of the tile
 *   lse_r = log sum_c exp(sm_scale q_r.k_c)    over every real key of head hd;
 * pass 2 gives, for every key tile j of the head,
 *   map[s][j] = max over real r in the tile, real c in tile j of
 *               exp(sm_scale q_r.k_c - lse_r)
 * and map[s][j] = 0 for n_tiles[hd] <= j < max_tiles.
 *  q_perm, k_perm  bf16, tile order
 *  sm_scale        finite and > 0 (else VEDA_ERR_INVALID_ARG)
 *  q_tiles         int32 [n_sub] global query-tile indices; an entry outside
 *                  [0, tile_off[num_heads]) gets a map row of zeros;
 *                  n_sub <= VEDA_MAX_SUBSET (else VEDA_ERR_UNSUPPORTED)
 *  workspace       device scratch of at least workspace_bytes >=
 *                  veda_oracle_maxpool_map_workspace(L, n_sub) bytes, 16-byte
 *                  aligned (smaller: VEDA_ERR_INVALID_ARG); owned by the
 *                  caller, contents on entry and exit unspecified, must not
 *                  overlap any other argument; calls sharing a workspace
 *                  must be ordered on one stream
 *  lse             f32 [n_sub*S] (output); padding query rows unspecified
 *  map             f32 [n_sub][max_tiles] (output)
 * Pass 1 also records, per query row and key tile, the largest logit, so
 * pass 2 reads n_sub*max_tiles*S floats instead of recomputing Q K^T.  Pass 1
 * hands out its work items (subset tile, chunk of key tiles) through eight
 * counters in the workspace, reset by a small kernel on `stream` first (no
 * memset); which workgroup computes an item does not change the results.
 * Supported: (head_dim, tile_size) in {(64,64), (128,128)}, max_tiles <=
 * VEDA_MAX_TILES_PER_HEAD. */
int veda_oracle_maxpool_map(const veda_layout* L, const void* q_perm, const void* k_perm,
                            float sm_scale, const int32_t* q_tiles, int32_t n_sub,
                            void* workspace, int64_t workspace_bytes, float* lse,
                            float* map, void* stream);

/* Workspace bytes veda_oracle_maxpool_map needs for n_sub subset entries of
 * layout L (0 for n_sub = 0): n_sub*max_tiles*S*4 for the row maxima plus
 * n_sub*16*S*8 for per-chunk partial sums (up to 16 chunks), each rounded up
 * to 256 bytes, plus 256 for pass 1's work counters.  Host-only, no device
 * work.
 * n_sub above VEDA_MAX_SUBSET or max_tiles above VEDA_MAX_TILES_PER_HEAD:
 * VEDA_ERR_UNSUPPORTED.
 *  bytes  (host) output */
int veda_oracle_maxpool_map_workspace(const veda_layout* L, int32_t n_sub, int64_t* bytes);

/* Distillation step of the estimator (Veda §2.1, optimisation: row-wise KL
 * objective, stop-gradient on the backbone features).  For every subset entry
 * s with query tile g = q_tiles[s] (local index i in head hd):
 *   p = softmax over j < n_tiles[hd] of scores[score_off[hd] + i*n + j]
 *   t = map[s][j] / sum_j map[s][j]
 *   loss = (1/R) sum_s KL(t || p)         R = entries with 0 <= g < tiles
 * and the gradients of loss with respect to the projections of
 * veda_tile_score, the TripPool descriptors being constants:
 *   grad_w_q, grad_w_k  f32 [num_heads][d_e][3*head_dim] (output)
 *   grad_b_q, grad_b_k  f32 [num_heads][d_e] (output), or NULL
 * When one weight set serves both sides, its gradient is the sum of the two.
 *  scores    f32 [score_off[num_heads]] as written by veda_tile_score
 *  map       f32 [n_sub][max_tiles]: veda_oracle_maxpool_map over the same
 *            q_tiles (a row whose map sums to 0 contributes nothing)
 *  q_tiles   int32 [n_sub] global query-tile indices; entries outside
 *            [0, tile_off[num_heads]) are ignored (and not counted in R);
 *            n_sub <= VEDA_MAX_SUBSET (else VEDA_ERR_UNSUPPORTED)
 *  desc      f32 [2][tile_off[num_heads]][3*head_dim] TripPool descriptors
 *  phi       f32 [2][tile_off[num_heads]][d_e] projections
 *  workspace device scratch of at least veda_distill_grad_workspace(L, n_sub,
 *            d_e) bytes, 16-byte aligned (smaller: VEDA_ERR_INVALID_ARG);
 *            owned by the caller, contents unspecified on entry and exit
 *  loss      f32 [1] (output)
 * Every output element is written; with R = 0 the loss and gradients are 0.
 * f32 arithmetic, sums in a fixed order (deterministic).  Supported:
 * 1 <= d_e <= 256, head_dim in {64, 128}. */
int veda_distill_grad(const veda_layout* L, const float* scores, const float* map,
                      const int32_t* q_tiles, int32_t n_sub, const float* desc,
                      const float* phi, int32_t d_e, void* workspace, int64_t workspace_bytes,
                      float* loss, float* grad_w_q, float* grad_w_k, float* grad_b_q,
                      float* grad_b_k, void* stream);

/* veda_distill_grad with no workspace argument and no allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight training or serving loops, harnesses that forbid hipMalloc.  The
 * workspace is a static device array inside the library, one per GPU,
 * VEDA_DISTILL_STATIC_SCRATCH_BYTES bytes, held until the process ends; its
 * address on a device is looked up (hipGetSymbolAddress) on the first call
 * made with that device current, and `stream` must belong to the current
 * device.  The call allocates nothing and calls no allocating routine.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind (the kernels write every element they read): calls that overlap in
 * time on one GPU -- on different streams, or from different threads --
 * race, so order them on one stream.  A problem whose
 * veda_distill_grad_workspace(L, n_sub, d_e) exceeds
 * VEDA_DISTILL_STATIC_SCRATCH_BYTES returns VEDA_ERR_UNSUPPORTED before any
 * device work; a failing address lookup returns VEDA_ERR_LAUNCH.  Every other
 * argument, result and limit as veda_distill_grad, bit for bit. */
#define VEDA_DISTILL_STATIC_SCRATCH_BYTES (64ll << 20)
int veda_distill_grad_noalloc(const veda_layout* L, const float* scores, const float* map,
                              const int32_t* q_tiles, int32_t n_sub, const float* desc,
                              const float* phi, int32_t d_e, float* loss, float* grad_w_q,
                              float* grad_w_k, float* grad_b_q, float* grad_b_k, void* stream);

/* Workspace bytes veda_distill_grad needs.  Host-only.  n_sub above
 * VEDA_MAX_SUBSET: VEDA_ERR_UNSUPPORTED.
 *  bytes  (host) output */
int veda_distill_grad_workspace(const veda_layout* L, int32_t n_sub, int32_t d_e,
                                int64_t* bytes);

/* Per-head squared error between two attention outputs, the measure of the
 * head-aware tiling search (Veda §2.2: each head's tile shape is chosen
 * offline by the approximation error between the full-attention output and
 * the sparse-attention output).  a, b: bf16 [N][num_heads][head_dim] in
 * token order (e.g. full attention and veda_sparse_attn_fwd_tokens output).
 *  err   f64 [num_heads] (output): sum over tokens and channels of (a - b)^2
 *  ref   f64 [num_heads] (output): sum of a^2, or NULL
 *  workspace  at least veda_head_sq_error_workspace(L) bytes, 8-byte aligned
 * f64 accumulation in a fixed order (deterministic).  Supported: head_dim a
 * multiple of 8 with head_dim/8 dividing 256, a and b 16-byte aligned. */
int veda_head_sq_error(const veda_layout* L, const void* a, const void* b, double* err,
                       double* ref, void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes veda_head_sq_error needs.  Host-only.
 *  bytes  (host) output */
int veda_head_sq_error_workspace(const veda_layout* L, int64_t* bytes);

/* The decision of the head-aware tiling search (Veda §2.2: per head, the
 * candidate tile shape whose sparse-attention output is closest to the
 * full-attention output on calibration inputs).
 *  err     f64 [n_cand][num_heads] (device, 8-byte aligned): row c holds the
 *          per-head errors of candidate c (e.g. veda_head_sq_error's err)
 *  choice  int32 [num_heads] (device, 4-byte aligned, output): per head the
 *          candidate index picked by the scan best = 0; for c = 1 ..
 *          n_cand - 1: if err[c][h] < err[best][h] then best = c.  Equal
 *          errors keep the earlier candidate; a NaN error never replaces an
 *          earlier candidate, and a NaN error of candidate 0 is never replaced.
 * n_cand in 1..VEDA_MAX_CANDIDATES, num_heads in 1..VEDA_MAX_HEADS, else
 * VEDA_ERR_INVALID_ARG before any device work.  Stream-ordered, no workspace,
 * deterministic. */
#define VEDA_MAX_CANDIDATES 64
int veda_head_choose(const double* err, int32_t n_cand, int32_t num_heads, int32_t* choice,
                     void* stream);

/* Static text for a veda_status value. */
const char* veda_status_string(int status);

/* sizeof(veda_layout) as compiled into the library, so that bindings can
 * check their copy of the struct. */
int64_t veda_layout_sizeof(void);

#ifdef __cplusplus
}
#endif
#endif /* VEDA_H */
