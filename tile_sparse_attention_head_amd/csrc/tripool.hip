// Distilled tile-score estimator (Veda §2.1): TripPool descriptor per tile
// (mean | max | min of the tile's real tokens, per channel), one projection
// per head, and the query-tile x key-tile score product.
//
// Three kernels:
//  1. pool:    one workgroup per (tile, side).  Lanes read the tile's rows as
//              16-byte chunks (coalesced), keep per-lane running sum/max/min of
//              8 (bf16) or 4 (f32) channels, then reduce across row groups in
//              LDS.  HBM-bound: reads the tile once, writes 3d floats.
//  2. project: phi = desc W^T + b, batched over (side, head).
//  3. score:   scores = phi_q phi_k^T, batched over heads.
// 2 and 3 share one LDS-tiled f32 "C = A B^T" tile (the projection 128 x 64
// or 32 x 64, the score product 64 x 64; K steps of 32 fetched one step
// ahead); both operands are read along their contiguous K dimension.
#include "veda_internal.hpp"

namespace veda {
namespace {

constexpr int kPoolThreads = 256;

template <typename E>
struct Vec16;  // 16 bytes of E
template <>
struct Vec16<__bf16> { __bf16 v[8]; };
template <>
struct Vec16<float> { float v[4]; };

template <typename E, int D>
__global__ __launch_bounds__(kPoolThreads) void tripool_pool_kernel(DevLayout L,
                                                                    const E* __restrict__ q,
                                                                    const E* __restrict__ k,
                                                                    float* __restrict__ desc) {
  constexpr int VEC = 16 / sizeof(E);
  constexpr int CH = D / VEC;                 // chunks per row
  constexpr int RG = kPoolThreads / CH;       // row groups
  __shared__ float red[3][RG][D];
  const int side = blockIdx.y;
  const int64_t g = blockIdx.x;
  const int h = head_of_tile(L, g);
  const TileExtent e = tile_extent(L, h, (int)(g - L.tile_off[h]));
  const E* x = (side ? k : q) + g * (int64_t)L.S * D;
  const int ch = threadIdx.x % CH, rg = threadIdx.x / CH;
  float sum[VEC], mx[VEC], mn[VEC];
#pragma unroll
  for (int c = 0; c < VEC; ++c) { sum[c] = 0.f; mx[c] = -INFINITY; mn[c] = INFINITY; }
  const bool full = e.full();
  for (int u = rg; u < L.S; u += RG) {
    if (!full && !e.slot_real(u)) continue;
    const Vec16<E> v = reinterpret_cast<const Vec16<E>*>(x + (int64_t)u * D)[ch];
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
      const float f = (float)v.v[c];
      sum[c] += f;
      mx[c] = fmaxf(mx[c], f);
      mn[c] = fminf(mn[c], f);
    }
  }
#pragma unroll
  for (int c = 0; c < VEC; ++c) {
    red[0][rg][ch * VEC + c] = sum[c];
    red[1][rg][ch * VEC + c] = mx[c];
    red[2][rg][ch * VEC + c] = mn[c];
  }
  __syncthreads();
  const float inv_cnt = 1.0f / (float)e.count();
  float* out = desc + ((int64_t)side * L.tile_off[L.heads] + g) * 3 * D;
  for (int c = threadIdx.x; c < D; c += kPoolThreads) {
    float s = 0.f, a = -INFINITY, b = INFINITY;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      s += red[0][r][c];
      a = fmaxf(a, red[1][r][c]);
      b = fminf(b, red[2][r][c]);
    }
    out[c] = s * inv_cnt;
    out[D + c] = a;
    out[2 * D + c] = b;
  }
}

// ---- batched f32 C[m][n] = sum_k A[m][k] B[n][k] (+ bias[n]) -------------
// A BM x BN output tile per workgroup of 256 lanes, BM = 16 RM, BN = 16 TN.
// Lane (ty, tx) = (t / 16, t % 16) computes RM rows and TN columns: rows
// RM ty + i for RM <= 4, and 4 ty + i, 64 + 4 ty + i (i < 4) for RM = 8;
// columns 4 tx + j (TN = 4) and also 64 + 4 tx + j (TN = 8).  Per k one or two
// LDS reads of A and of B feed RM TN FMAs: at 8 x 8, 64 bytes per 64 FMAs
// (4 x 4: 32 per 16).  Larger tiles serve the long-K projection of large
// layers; small layers keep small tiles so that the grid still fills the chip.  K runs in steps of
// 32; lane t fetches 4 consecutive k of rows t / 8 + 32 u of A and of B, the
// next step's while the current step is multiplied.  Every output is the
// sequential FMA chain over k = 0 .. K-1 from 0, then + bias (or + 0.f),
// whatever the tile: the scores are the same f32 numbers the fused score +
// selection computes.
constexpr int kGemmThreads = 256, GBK = 32;

struct GemmArgs {
  const float* A; const float* B; const float* bias; float* C;
  int M, N, K; int64_t lda, ldb, ldc;
};

// k .. k+3 (k % 4 == 0) of row `row`, 0 outside [0, rows) x [0, K).  The
// address is clamped into the operand, so the load is unconditional and a
// lane's loads are all in flight at once.  VEC: K % 4 == 0 and 16-byte aligned
// rows (then k < K means k + 3 < K).
template <bool VEC>
__device__ __forceinline__ float4 gemm_fetch4(const float* __restrict__ src, int64_t ld, int row,
                                              int rows, int k, int K) {
  const float* p = src + (int64_t)min(row, rows - 1) * ld;
  const bool in_row = row < rows;
  if constexpr (VEC) {
    const float4 v = *reinterpret_cast<const float4*>(p + min(k, K - 4));
    return in_row && k < K ? v : make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
    float e[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float x = p[min(k + c, K - 1)];
      e[c] = in_row && k + c < K ? x : 0.f;
    }
    return make_float4(e[0], e[1], e[2], e[3]);
  }
}

// the i-th of a lane's RM rows (columns alike with RM = TN, i < TN)
template <int RM>
__device__ __forceinline__ int lane_row(int ty, int i) {
  return RM == 8 ? (i < 4 ? 4 * ty + i : 64 + 4 * ty + i - 4) : RM * ty + i;
}

template <int RM, int TN, bool VEC>
__device__ __forceinline__ void gemm_abt_tile(const GemmArgs& a, int m0, int n0) {
  constexpr int BM = 16 * RM, BN = 16 * TN;
  constexpr int AF = BM / 32, BF = BN / 32;   // 16-byte fetches per lane and step
  static_assert(RM == 2 || RM == 4 || RM == 8, "rows per lane");
  static_assert(TN == 4 || TN == 8, "columns per lane");
  __shared__ __attribute__((aligned(16))) float As[GBK][BM + 4];
  __shared__ __attribute__((aligned(16))) float Bs[GBK][BN + 4];
  const int t = threadIdx.x;
  const int ty = t / 16, tx = t % 16;
  const int fr = t / 8, fk = (t % 8) * 4;  // fetched row (+ 32 u) and k offset in the step
  float acc[RM][TN] = {};
  float4 va[AF], vb[BF];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < AF; ++u)
      va[u] = gemm_fetch4<VEC>(a.A, a.lda, m0 + fr + 32 * u, a.M, k0 + fk, a.K);
#pragma unroll
    for (int u = 0; u < BF; ++u)
      vb[u] = gemm_fetch4<VEC>(a.B, a.ldb, n0 + fr + 32 * u, a.N, k0 + fk, a.K);
  };
  fetch(0);
  for (int k0 = 0; k0 < a.K; k0 += GBK) {
#pragma unroll
    for (int u = 0; u < AF; ++u) {
      As[fk + 0][fr + 32 * u] = va[u].x;
      As[fk + 1][fr + 32 * u] = va[u].y;
      As[fk + 2][fr + 32 * u] = va[u].z;
      As[fk + 3][fr + 32 * u] = va[u].w;
    }
#pragma unroll
    for (int u = 0; u < BF; ++u) {
      Bs[fk + 0][fr + 32 * u] = vb[u].x;
      Bs[fk + 1][fr + 32 * u] = vb[u].y;
      Bs[fk + 2][fr + 32 * u] = vb[u].z;
      Bs[fk + 3][fr + 32 * u] = vb[u].w;
    }
    __syncthreads();
    if (k0 + GBK < a.K) fetch(k0 + GBK);   // next step's values, in flight during the products
#pragma unroll
    for (int kk = 0; kk < GBK; ++kk) {
      float am[RM], bn[TN];
      if constexpr (RM == 2) {
        const float2 v = *reinterpret_cast<const float2*>(&As[kk][2 * ty]);
        am[0] = v.x; am[1] = v.y;
      } else {
#pragma unroll
        for (int h = 0; h < RM / 4; ++h) {
          const float4 v = *reinterpret_cast<const float4*>(&As[kk][64 * h + 4 * ty]);
          am[4 * h + 0] = v.x; am[4 * h + 1] = v.y; am[4 * h + 2] = v.z; am[4 * h + 3] = v.w;
        }
      }
#pragma unroll
      for (int h = 0; h < TN / 4; ++h) {
        const float4 v = *reinterpret_cast<const float4*>(&Bs[kk][64 * h + 4 * tx]);
        bn[4 * h + 0] = v.x; bn[4 * h + 1] = v.y; bn[4 * h + 2] = v.z; bn[4 * h + 3] = v.w;
      }
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = fmaf(am[i], bn[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < RM; ++i) {
    const int m = m0 + lane_row<RM>(ty, i);
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int nn = n0 + lane_row<TN>(tx, j);
      if (nn >= a.N) continue;
      a.C[m * a.ldc + nn] = acc[i][j] + (a.bias ? a.bias[nn] : 0.f);
    }
  }
}

// batch = side*heads + h: desc rows of head h -> phi rows of head h.
template <int RM, bool VEC>
__global__ __launch_bounds__(kGemmThreads) void project_kernel(DevLayout L, int d_e,
                                                               const float* __restrict__ desc,
                                                               const float* __restrict__ wq,
                                                               const float* __restrict__ wk,
                                                               const float* bq, const float* bk,
                                                               float* __restrict__ phi) {
  const int side = blockIdx.z / L.heads, h = blockIdx.z % L.heads;
  const int64_t total = L.tile_off[L.heads];
  const int n_h = (int)(L.tile_off[h + 1] - L.tile_off[h]);
  const int m0 = blockIdx.y * 16 * RM, n0 = blockIdx.x * 64;
  if (m0 >= n_h || n0 >= d_e) return;
  const int K = 3 * L.d;
  GemmArgs a;
  a.A = desc + ((int64_t)side * total + L.tile_off[h]) * K;
  a.B = (side ? wk : wq) + (int64_t)h * d_e * K;
  const float* b = side ? bk : bq;
  a.bias = b ? b + (int64_t)h * d_e : nullptr;
  a.C = phi + ((int64_t)side * total + L.tile_off[h]) * d_e;
  a.M = n_h; a.N = d_e; a.K = K; a.lda = K; a.ldb = K; a.ldc = d_e;
  gemm_abt_tile<RM, 4, VEC>(a, m0, n0);
}

template <bool VEC>
__global__ __launch_bounds__(kGemmThreads) void score_kernel(DevLayout L, int d_e,
                                                             const float* __restrict__ phi,
                                                             float* __restrict__ scores) {
  const int h = blockIdx.z;
  const int64_t total = L.tile_off[L.heads];
  const int n_h = (int)(L.tile_off[h + 1] - L.tile_off[h]);
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  if (m0 >= n_h || n0 >= n_h) return;
  GemmArgs a;
  a.A = phi + L.tile_off[h] * d_e;
  a.B = phi + (total + L.tile_off[h]) * d_e;
  a.bias = nullptr;
  a.C = scores + L.score_off[h];
  a.M = n_h; a.N = n_h; a.K = d_e; a.lda = d_e; a.ldb = d_e; a.ldc = n_h;
  gemm_abt_tile<4, 4, VEC>(a, m0, n0);
}

// Compute units of the current device (256 if the query fails).
int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 256;
  return cus;
}

}  // namespace

int launch_tripool_score(const DevLayout& L, int dtype, const void* q, const void* k,
                         const float* wq, const float* wk, const float* bq, const float* bk,
                         int d_e, float* desc, float* phi, float* scores, hipStream_t s) {
  const unsigned tiles = (unsigned)L.tile_off[L.heads];
  if (tiles == 0) return VEDA_OK;
  const dim3 pg(tiles, 2);
  if (dtype == VEDA_F32) {
    if (L.d == 128)
      hipLaunchKernelGGL((tripool_pool_kernel<float, 128>), pg, dim3(kPoolThreads), 0, s, L,
                         (const float*)q, (const float*)k, desc);
    else
      hipLaunchKernelGGL((tripool_pool_kernel<float, 64>), pg, dim3(kPoolThreads), 0, s, L,
                         (const float*)q, (const float*)k, desc);
  } else {
    if (L.d == 128)
      hipLaunchKernelGGL((tripool_pool_kernel<__bf16, 128>), pg, dim3(kPoolThreads), 0, s, L,
                         (const __bf16*)q, (const __bf16*)k, desc);
    else
      hipLaunchKernelGGL((tripool_pool_kernel<__bf16, 64>), pg, dim3(kPoolThreads), 0, s, L,
                         (const __bf16*)q, (const __bf16*)k, desc);
  }
  if (launch_status() != VEDA_OK) return VEDA_ERR_LAUNCH;
  return launch_project_score(L, desc, wq, wk, bq, bk, d_e, phi, scores, s);
}

int launch_project_score(const DevLayout& L, const float* desc, const float* wq, const float* wk,
                         const float* bq, const float* bk, int d_e, float* phi, float* scores,
                         hipStream_t s) {
  if (L.tile_off[L.heads] == 0) return VEDA_OK;
  // 16-byte loads need 16-byte aligned rows: K % 4 == 0 and aligned bases
  auto al = [](const void* p) { return ((uintptr_t)p & 15u) == 0; };
  const bool pvec = al(desc) && al(wq) && al(wk);   // K = 3d is a multiple of 4
  const bool svec = d_e % 4 == 0 && al(phi);
  // projection: 128-row tiles (8 x 4 per lane) when they still give every CU
  // two workgroups, else 32-row tiles (2 x 4) for more workgroups
  const unsigned cus = (unsigned)device_cus();
  auto tiles = [&](int bm) { return (unsigned)((L.max_tiles + bm - 1) / bm); };
  const unsigned n_b = (unsigned)((d_e + 63) / 64), batches = 2u * (unsigned)L.heads;
  const bool pbig = tiles(128) * n_b * batches >= 2 * cus;
  const dim3 pgrid(n_b, tiles(pbig ? 128 : 32), batches);
#define VEDA_PROJ(RM, V)                                                                       \
  hipLaunchKernelGGL((project_kernel<RM, V>), pgrid, dim3(kGemmThreads), 0, s, L, d_e, desc, wq, \
                     wk, bq, bk, phi)
  if (pbig) {
    if (pvec) VEDA_PROJ(8, true); else VEDA_PROJ(8, false);
  } else {
    if (pvec) VEDA_PROJ(2, true); else VEDA_PROJ(2, false);
  }
#undef VEDA_PROJ
  if (launch_status() != VEDA_OK) return VEDA_ERR_LAUNCH;
  if (scores == nullptr) return VEDA_OK;   // projection only
  // the score product keeps 64 x 64 tiles (4 x 4 per lane) at every size: its
  // 8 x 8 tiles (138 registers, 3 waves per SIMD) measured no faster at the
  // 720P layer and slower at the smaller ones
  const dim3 sgrid(tiles(64), tiles(64), L.heads);
  if (svec)
    hipLaunchKernelGGL(score_kernel<true>, sgrid, dim3(kGemmThreads), 0, s, L, d_e, phi, scores);
  else
    hipLaunchKernelGGL(score_kernel<false>, sgrid, dim3(kGemmThreads), 0, s, L, d_e, phi, scores);
  return launch_status();
}

}  // namespace veda
