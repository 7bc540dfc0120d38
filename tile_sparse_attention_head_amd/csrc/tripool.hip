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
// 2 and 3 share one LDS-tiled f32 "C = A B^T" kernel (64x64 tile, 4x4 outputs
// per lane, K steps of 32 fetched one step ahead); both operands are read
// along their contiguous K dimension.
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
// 64x64 output tile per workgroup, 4x4 outputs per lane, K in steps of 64
// (few steps: these products are short and latency-bound).  Each lane
// fetches 16 consecutive k of one A row and one B row per step (four 16-byte
// loads each when VEC: K % 4 == 0 and 16-byte aligned operands), and the next
// step's values are fetched while the current step is multiplied.
constexpr int BN = 64, BK = 64, kGemmThreads = 256;

// projection: few, deep (K = 3d) products -> smaller tiles for more workgroups
constexpr int kProjBM = 32, kScoreBM = 64;

struct GemmArgs {
  const float* A; const float* B; const float* bias; float* C;
  int M, N, K; int64_t lda, ldb, ldc;
};

template <bool VEC>
__device__ __forceinline__ void gemm_fetch(const float* __restrict__ src, int64_t ld, int row,
                                           int rows, int k, int K, float (&v)[8]) {
  if (row >= rows) {
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = 0.f;
    return;
  }
  const float* p = src + row * ld + k;
  if (VEC && k + 8 <= K) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    const float4 y = *reinterpret_cast<const float4*>(p + 4);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = k + c < K ? p[c] : 0.f;
  }
}

// BM x 64 output tile (BM = 64: 4x4 outputs per lane; BM = 32: 2x4).
template <int BM, bool VEC>
__device__ __forceinline__ void gemm_abt_tile(const GemmArgs& a, int m0, int n0) {
  constexpr int RM = BM / 16;              // output rows per lane
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  const int t = threadIdx.x;
  const int tm = (t / 16) * RM, tn = (t % 16) * 4;
  const int r = t / 4, kc = (t % 4) * 16;  // fetched row and k offset within the step
  const bool fa = r < BM;                  // this lane also fetches an A row
  float acc[RM][4] = {};
  float va[16], vb[16];
  auto fetch = [&](int k) {   // 16 consecutive k of one A row and one B row
    if (fa) {
      gemm_fetch<VEC>(a.A, a.lda, m0 + r, a.M, k, a.K, *reinterpret_cast<float(*)[8]>(va));
      gemm_fetch<VEC>(a.A, a.lda, m0 + r, a.M, k + 8, a.K, *reinterpret_cast<float(*)[8]>(va + 8));
    }
    gemm_fetch<VEC>(a.B, a.ldb, n0 + r, a.N, k, a.K, *reinterpret_cast<float(*)[8]>(vb));
    gemm_fetch<VEC>(a.B, a.ldb, n0 + r, a.N, k + 8, a.K, *reinterpret_cast<float(*)[8]>(vb + 8));
  };
  fetch(kc);
  for (int k0 = 0; k0 < a.K; k0 += BK) {
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      if (fa) As[kc + c][r] = va[c];
      Bs[kc + c][r] = vb[c];
    }
    __syncthreads();
    if (k0 + BK < a.K) fetch(k0 + BK + kc);   // next step's values, in flight during the products
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float am[RM];
      if constexpr (RM == 4) {
        const float4 av = *reinterpret_cast<const float4*>(&As[kk][tm]);
        am[0] = av.x; am[1] = av.y; am[2] = av.z; am[3] = av.w;
      } else {
        const float2 av = *reinterpret_cast<const float2*>(&As[kk][tm]);
        am[0] = av.x; am[1] = av.y;
      }
      const float4 bv = *reinterpret_cast<const float4*>(&Bs[kk][tn]);
      const float bn[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(am[i], bn[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < RM; ++i) {
    const int m = m0 + tm + i;
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nn = n0 + tn + j;
      if (nn >= a.N) continue;
      a.C[m * a.ldc + nn] = acc[i][j] + (a.bias ? a.bias[nn] : 0.f);
    }
  }
}

// batch = side*heads + h: desc rows of head h -> phi rows of head h.
template <bool VEC>
__global__ __launch_bounds__(kGemmThreads) void project_kernel(DevLayout L, int d_e,
                                                               const float* __restrict__ desc,
                                                               const float* __restrict__ wq,
                                                               const float* __restrict__ wk,
                                                               const float* bq, const float* bk,
                                                               float* __restrict__ phi) {
  const int side = blockIdx.z / L.heads, h = blockIdx.z % L.heads;
  const int64_t total = L.tile_off[L.heads];
  const int n_h = (int)(L.tile_off[h + 1] - L.tile_off[h]);
  const int m0 = blockIdx.y * kProjBM, n0 = blockIdx.x * BN;
  if (m0 >= n_h || n0 >= d_e) return;
  const int K = 3 * L.d;
  GemmArgs a;
  a.A = desc + ((int64_t)side * total + L.tile_off[h]) * K;
  a.B = (side ? wk : wq) + (int64_t)h * d_e * K;
  const float* b = side ? bk : bq;
  a.bias = b ? b + (int64_t)h * d_e : nullptr;
  a.C = phi + ((int64_t)side * total + L.tile_off[h]) * d_e;
  a.M = n_h; a.N = d_e; a.K = K; a.lda = K; a.ldb = K; a.ldc = d_e;
  gemm_abt_tile<kProjBM, VEC>(a, m0, n0);
}

template <bool VEC>
__global__ __launch_bounds__(kGemmThreads) void score_kernel(DevLayout L, int d_e,
                                                             const float* __restrict__ phi,
                                                             float* __restrict__ scores) {
  const int h = blockIdx.z;
  const int64_t total = L.tile_off[L.heads];
  const int n_h = (int)(L.tile_off[h + 1] - L.tile_off[h]);
  const int m0 = blockIdx.y * kScoreBM, n0 = blockIdx.x * BN;
  if (m0 >= n_h || n0 >= n_h) return;
  GemmArgs a;
  a.A = phi + L.tile_off[h] * d_e;
  a.B = phi + (total + L.tile_off[h]) * d_e;
  a.bias = nullptr;
  a.C = scores + L.score_off[h];
  a.M = n_h; a.N = n_h; a.K = d_e; a.lda = d_e; a.ldb = d_e; a.ldc = n_h;
  gemm_abt_tile<kScoreBM, VEC>(a, m0, n0);
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
  const unsigned mbp = (unsigned)((L.max_tiles + kProjBM - 1) / kProjBM);
  const unsigned mb = (unsigned)((L.max_tiles + kScoreBM - 1) / kScoreBM);
  // 16-byte loads need 16-byte aligned rows: K % 4 == 0 and aligned bases
  auto al = [](const void* p) { return ((uintptr_t)p & 15u) == 0; };
  const bool pvec = al(desc) && al(wq) && al(wk);   // K = 3d is a multiple of 4
  const bool svec = d_e % 4 == 0 && al(phi);
  const dim3 pgrid((d_e + BN - 1) / BN, mbp, 2 * L.heads);
  if (pvec)
    hipLaunchKernelGGL(project_kernel<true>, pgrid, dim3(kGemmThreads), 0, s, L, d_e, desc, wq, wk,
                       bq, bk, phi);
  else
    hipLaunchKernelGGL(project_kernel<false>, pgrid, dim3(kGemmThreads), 0, s, L, d_e, desc, wq,
                       wk, bq, bk, phi);
  if (launch_status() != VEDA_OK) return VEDA_ERR_LAUNCH;
  if (scores == nullptr) return VEDA_OK;   // projection only
  if (svec)
    hipLaunchKernelGGL(score_kernel<true>, dim3(mb, mb, L.heads), dim3(kGemmThreads), 0, s, L,
                       d_e, phi, scores);
  else
    hipLaunchKernelGGL(score_kernel<false>, dim3(mb, mb, L.heads), dim3(kGemmThreads), 0, s, L,
                       d_e, phi, scores);
  return launch_status();
}

}  // namespace veda
