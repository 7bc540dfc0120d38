// Head-aware tile gather / scatter (Veda §2.2 head-aware tiling; Veda news,
// head-conditioned tile geometry): regroup one head's T x H x W tokens into
// its (pt, ph, pw) tiles and back.
//
// One workgroup per tile.  Every row (one token of one head) is d contiguous
// elements in both layouts, moved as 16-byte chunks: consecutive lanes take
// consecutive chunks, so each row is one fully coalesced 16*CPR-byte burst.
// The kernels are pure data movement, bound by HBM bandwidth.
#include "veda_internal.hpp"

namespace veda {
namespace {

constexpr int kThreads = 256;

struct Chunk { uint32_t x, y, z, w; };

__device__ __forceinline__ int64_t token_of_slot(const DevLayout& L, const TileExtent& e, int u) {
  const int dw = u % e.pw;
  const int r = u / e.pw;
  const int dh = r % e.ph;
  const int dt = r / e.ph;
  if (dt >= e.lt || dh >= e.lh || dw >= e.lw) return -1;
  const int64_t t = (int64_t)e.it * e.pt + dt;
  const int64_t h = (int64_t)e.ih * e.ph + dh;
  const int64_t w = (int64_t)e.iw * e.pw + dw;
  return (t * L.H + h) * L.W + w;
}

// x [N][heads][CPR chunks] -> y [tiles*S][CPR chunks]; padding slots = 0.
__global__ __launch_bounds__(kThreads) void permute_fwd_kernel(DevLayout L, int cpr,
                                                               const Chunk* __restrict__ x,
                                                               Chunk* __restrict__ y) {
  const int64_t g = blockIdx.x;
  const int h = head_of_tile(L, g);
  const TileExtent e = tile_extent(L, h, (int)(g - L.tile_off[h]));
  const int total = L.S * cpr;
  Chunk* dst = y + g * (int64_t)total;
  for (int c = threadIdx.x; c < total; c += kThreads) {
    const int u = c / cpr, k = c - u * cpr;
    const int64_t n = token_of_slot(L, e, u);
    Chunk v = {0u, 0u, 0u, 0u};
    if (n >= 0) v = x[(n * L.heads + h) * cpr + k];
    dst[c] = v;
  }
}

// x tile order -> y [N][heads][CPR]; only real slots are read and written.
__global__ __launch_bounds__(kThreads) void permute_inv_kernel(DevLayout L, int cpr,
                                                               const Chunk* __restrict__ x,
                                                               Chunk* __restrict__ y) {
  const int64_t g = blockIdx.x;
  const int h = head_of_tile(L, g);
  const TileExtent e = tile_extent(L, h, (int)(g - L.tile_off[h]));
  const int total = L.S * cpr;
  const Chunk* src = x + g * (int64_t)total;
  for (int c = threadIdx.x; c < total; c += kThreads) {
    const int u = c / cpr, k = c - u * cpr;
    const int64_t n = token_of_slot(L, e, u);
    if (n >= 0) y[(n * L.heads + h) * cpr + k] = src[c];
  }
}

// x [N][heads][d] -> y tile-transposed ([d][S] per tile).  The tile passes
// through LDS: rows are read as coalesced chunks, scattered element-wise into
// a [d][S + pad] LDS image, and written back as coalesced chunks of S.
template <typename E>
__global__ __launch_bounds__(kThreads) void permute_fwd_t_kernel(DevLayout L,
                                                                 const E* __restrict__ x,
                                                                 E* __restrict__ y) {
  constexpr int VEC = 16 / sizeof(E);            // elements per chunk
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  E* lds = reinterpret_cast<E*>(smem_raw);
  const int S = L.S, d = L.d;
  const int ld = S + VEC;                        // padded LDS row (keeps 16-B alignment)
  const int64_t g = blockIdx.x;
  const int h = head_of_tile(L, g);
  const TileExtent e = tile_extent(L, h, (int)(g - L.tile_off[h]));
  const int cpr = d / VEC;                       // chunks per token row
  for (int c = threadIdx.x; c < S * cpr; c += kThreads) {
    const int u = c / cpr, k = c - u * cpr;
    const int64_t n = token_of_slot(L, e, u);
    E v[VEC];
    if (n >= 0) {
      *reinterpret_cast<Chunk*>(v) = reinterpret_cast<const Chunk*>(x + (n * L.heads + h) * (int64_t)d)[k];
    } else {
#pragma unroll
      for (int q = 0; q < VEC; ++q) v[q] = E(0);
    }
#pragma unroll
    for (int q = 0; q < VEC; ++q) lds[(k * VEC + q) * ld + u] = v[q];
  }
  __syncthreads();
  const int cps = S / VEC;                       // chunks per transposed row
  Chunk* dst = reinterpret_cast<Chunk*>(y + g * (int64_t)S * d);
  for (int c = threadIdx.x; c < d * cps; c += kThreads) {
    const int dd = c / cps, k = c - dd * cps;
    dst[c] = *reinterpret_cast<const Chunk*>(lds + dd * ld + k * VEC);
  }
}

}  // namespace

int launch_permute(const DevLayout& L, int dtype, int dir, const void* x, void* y, hipStream_t s) {
  const int esize = dtype == VEDA_F32 ? 4 : 2;
  const int cpr = L.d * esize / 16;
  const unsigned blocks = (unsigned)L.tile_off[L.heads];
  if (blocks == 0) return VEDA_OK;
  if (dir == VEDA_FWD) {
    hipLaunchKernelGGL(permute_fwd_kernel, dim3(blocks), dim3(kThreads), 0, s, L, cpr,
                       (const Chunk*)x, (Chunk*)y);
  } else if (dir == VEDA_INV) {
    hipLaunchKernelGGL(permute_inv_kernel, dim3(blocks), dim3(kThreads), 0, s, L, cpr,
                       (const Chunk*)x, (Chunk*)y);
  } else {
    const size_t lds = (size_t)L.d * (L.S + 16 / esize) * esize;
    if (dtype == VEDA_F32)
      hipLaunchKernelGGL(permute_fwd_t_kernel<float>, dim3(blocks), dim3(kThreads), lds, s, L,
                         (const float*)x, (float*)y);
    else
      hipLaunchKernelGGL(permute_fwd_t_kernel<__bf16>, dim3(blocks), dim3(kThreads), lds, s, L,
                         (const __bf16*)x, (__bf16*)y);
  }
  return launch_status();
}

}  // namespace veda
