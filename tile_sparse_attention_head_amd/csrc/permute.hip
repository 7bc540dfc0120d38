// Head-aware tile gather / scatter (Veda §2.2 head-aware tiling; Veda news,
// head-conditioned tile geometry): regroup one head's T x H x W tokens into
// its (pt, ph, pw) tiles and back.
//
// One workgroup per tile.  The row (token, head) of each of the tile's slots
// is computed once into LDS.  Every row is d contiguous elements in both
// layouts, moved as 16-byte chunks: consecutive lanes take consecutive
// chunks, so each row is one fully coalesced 16*CPR-byte burst, and a lane
// issues several loads before its stores.  Those loads and stores are
// unconditional (a padding slot reads slot 0's row, always a real token, and
// stores zeros; a chunk index past the tile is clamped to its last chunk,
// which is then written twice with the same value): a load or store under a
// branch gets a wait of its own, and then each store waits for the one
// before it.  The kernels are pure data movement, bound by HBM bandwidth.
#include "veda_internal.hpp"

namespace veda {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 8;   // chunks a lane loads before it stores any

struct Chunk { uint32_t x, y, z, w; };

__device__ __forceinline__ int64_t token_of_slot(const DevLayout& L, const TileExtent& e, int u) {
  int dt, dh, dw;
  e.slot_coords(u, dt, dh, dw);
  if (dt >= e.lt || dh >= e.lh || dw >= e.lw) return -1;
  const int64_t t = (int64_t)e.it * e.pt + dt;
  const int64_t h = (int64_t)e.ih * e.ph + dh;
  const int64_t w = (int64_t)e.iw * e.pw + dw;
  return (t * L.H + h) * L.W + w;
}

// Row (token * heads + head) of every slot of tile g in the token-major
// layout, -1 for padding: computed once per workgroup into LDS.
__device__ __forceinline__ int tile_rows(const DevLayout& L, int64_t g, int64_t* rows) {
  const int h = head_of_tile(L, g);
  const TileExtent e = tile_extent(L, h, (int)(g - L.tile_off[h]));
  for (int u = threadIdx.x; u < L.S; u += kThreads) {
    const int64_t n = token_of_slot(L, e, u);
    rows[u] = n >= 0 ? n * L.heads + h : -1;
  }
  __syncthreads();
  return h;
}

// x [N][heads][CPR chunks] -> y [tiles*S][CPR chunks]; padding slots = 0.
__global__ __launch_bounds__(kThreads) void permute_fwd_kernel(DevLayout L, int cpr,
                                                               const Chunk* __restrict__ x,
                                                               Chunk* __restrict__ y) {
  __shared__ int64_t rows[256];
  const int64_t g = blockIdx.x;
  tile_rows(L, g, rows);
  const int total = L.S * cpr;
  Chunk* dst = y + g * (int64_t)total;
  for (int c0 = 0; c0 < total; c0 += kThreads * kBatch) {
    Chunk v[kBatch];
    int cc[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      cc[i] = min(c0 + i * kThreads + (int)threadIdx.x, total - 1);
      const int u = cc[i] / cpr, k = cc[i] - u * cpr;
      const int64_t r = rows[u];
      const Chunk a = x[(r >= 0 ? r : rows[0]) * cpr + k];
      v[i] = r >= 0 ? a : Chunk{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) dst[cc[i]] = v[i];
  }
}

// The gather of Q or K fused with TripPool (Veda §2.1): as permute_fwd_kernel,
// and for each channel the mean, max and min over the tile's real slots,
// written as desc[g] = [mean | max | min] (3 D floats).  Lane t always moves
// channel chunk t % CPR, and walks the slots t / CPR, + RG, + 2 RG, ..., so it
// keeps running statistics of its VEC channels in registers (in the order
// tripool_pool_kernel uses, which makes the two bit-identical); the RG row
// groups are combined through LDS.
template <typename E, int D>
__global__ __launch_bounds__(kThreads) void permute_fwd_pool_kernel(DevLayout L,
                                                                    const Chunk* __restrict__ x,
                                                                    Chunk* __restrict__ y,
                                                                    float* __restrict__ desc) {
  constexpr int VEC = 16 / (int)sizeof(E);
  constexpr int CPR = D / VEC;                 // chunks per row
  constexpr int RG = kThreads / CPR;           // row groups
  static_assert(kThreads % CPR == 0, "every lane keeps one chunk column");
  __shared__ int64_t rows[256];
  __shared__ float red[3][RG][D];
  const int64_t g = blockIdx.x;
  const int h = tile_rows(L, g, rows);
  const int total = L.S * CPR;
  const int ch = threadIdx.x % CPR, rg = threadIdx.x / CPR;
  float sum[VEC], mx[VEC], mn[VEC];
#pragma unroll
  for (int c = 0; c < VEC; ++c) { sum[c] = 0.f; mx[c] = -INFINITY; mn[c] = INFINITY; }
  Chunk* dst = y + g * (int64_t)total;
  for (int c0 = 0; c0 < total; c0 += kThreads * kBatch) {
    Chunk v[kBatch];
    bool real[kBatch];
    int cc[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int c = c0 + i * kThreads + threadIdx.x;
      cc[i] = min(c, total - 1);
      const int64_t r = rows[cc[i] / CPR];
      real[i] = c < total && r >= 0;
      const Chunk a = x[(r >= 0 ? r : rows[0]) * CPR + cc[i] % CPR];
      v[i] = r >= 0 ? a : Chunk{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) dst[cc[i]] = v[i];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (!real[i]) continue;
      E e[VEC];
      __builtin_memcpy(e, &v[i], 16);
#pragma unroll
      for (int c = 0; c < VEC; ++c) {
        const float f = (float)e[c];
        sum[c] += f;
        mx[c] = fmaxf(mx[c], f);
        mn[c] = fminf(mn[c], f);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < VEC; ++c) {
    red[0][rg][ch * VEC + c] = sum[c];
    red[1][rg][ch * VEC + c] = mx[c];
    red[2][rg][ch * VEC + c] = mn[c];
  }
  __syncthreads();
  const TileExtent e = tile_extent(L, h, (int)(g - L.tile_off[h]));
  const float inv_cnt = 1.0f / (float)e.count();
  float* out = desc + g * 3 * D;
  for (int c = threadIdx.x; c < D; c += kThreads) {
    float sm = 0.f, a = -INFINITY, b = INFINITY;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      sm += red[0][r][c];
      a = fmaxf(a, red[1][r][c]);
      b = fminf(b, red[2][r][c]);
    }
    out[c] = sm * inv_cnt;
    out[D + c] = a;
    out[2 * D + c] = b;
  }
}

// x tile order -> y [N][heads][CPR]; only real slots are read and written
// (one chunk per lane per pass: batching the loads slows the scattered
// stores down).
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

// bf16 x [N][heads][d] -> y tile-transposed ([d][S] per tile), in registers:
// each lane moves one block of 8 slots x 8 channels -- eight 16-byte reads
// along token rows, an 8x8 transpose of 16-bit values with byte permutes,
// eight 16-byte writes along channel rows.  Lanes take consecutive channel
// chunks of one slot group, so each read instruction covers whole token rows.
__global__ __launch_bounds__(kThreads) void permute_fwd_t_bf16_kernel(DevLayout L,
                                                                      const Chunk* __restrict__ x,
                                                                      Chunk* __restrict__ y) {
  __shared__ int64_t rows[256];
  const int64_t g = blockIdx.x;
  tile_rows(L, g, rows);
  const int S = L.S, cpr = L.d / 8;             // channel chunks per token row
  Chunk* dst = y + g * (int64_t)S * cpr;        // [d][S] bf16 = d rows of S/8 chunks
  for (int b = threadIdx.x; b < (S / 8) * cpr; b += kThreads) {
    const int k = b % cpr, tg = b / cpr;        // channels 8k..8k+7, slots 8tg..8tg+7
    Chunk r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t row = rows[8 * tg + j];
      r[j] = Chunk{0u, 0u, 0u, 0u};
      if (row >= 0) r[j] = x[row * cpr + k];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      // channel 8k+q of slot j sits in word q/2 of r[j], low half for even q
      const uint32_t sel = (q & 1) ? 0x07060302u : 0x05040100u;
      uint32_t w[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const Chunk& a = r[2 * m];
        const Chunk& c = r[2 * m + 1];
        const uint32_t lo = (q >> 1) == 0 ? a.x : (q >> 1) == 1 ? a.y : (q >> 1) == 2 ? a.z : a.w;
        const uint32_t hi = (q >> 1) == 0 ? c.x : (q >> 1) == 1 ? c.y : (q >> 1) == 2 ? c.z : c.w;
        w[m] = __builtin_amdgcn_perm(hi, lo, sel);
      }
      dst[(int64_t)(8 * k + q) * (S / 8) + tg] = Chunk{w[0], w[1], w[2], w[3]};
    }
  }
}

// f32 x [N][heads][d] -> y tile-transposed ([d][S] per tile).  The tile passes
// through LDS: rows are read as coalesced chunks, scattered element-wise into
// a [d][S + pad] LDS image, and written back as coalesced chunks of S.
__global__ __launch_bounds__(kThreads) void permute_fwd_t_f32_kernel(DevLayout L,
                                                                     const float* __restrict__ x,
                                                                     float* __restrict__ y) {
  constexpr int VEC = 4;                         // elements per chunk
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  float* lds = reinterpret_cast<float*>(smem_raw);
  __shared__ int64_t rows[256];
  const int64_t g = blockIdx.x;
  tile_rows(L, g, rows);
  const int S = L.S, d = L.d;
  const int ld = S + VEC;                        // padded LDS row (keeps 16-B alignment)
  const int cpr = d / VEC;                       // chunks per token row
  for (int c = threadIdx.x; c < S * cpr; c += kThreads) {
    const int u = c / cpr, k = c - u * cpr;
    const int64_t row = rows[u];
    float v[VEC];
    if (row >= 0) {
      *reinterpret_cast<Chunk*>(v) = reinterpret_cast<const Chunk*>(x + row * (int64_t)d)[k];
    } else {
#pragma unroll
      for (int q = 0; q < VEC; ++q) v[q] = 0.f;
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

int launch_permute_pool(const DevLayout& L, int dtype, const void* x, void* y, float* desc,
                        hipStream_t s) {
  const unsigned blocks = (unsigned)L.tile_off[L.heads];
  if (blocks == 0) return VEDA_OK;
  const Chunk* cx = (const Chunk*)x;
  Chunk* cy = (Chunk*)y;
  if (dtype == VEDA_F32) {
    if (L.d == 128)
      hipLaunchKernelGGL((permute_fwd_pool_kernel<float, 128>), dim3(blocks), dim3(kThreads), 0, s,
                         L, cx, cy, desc);
    else
      hipLaunchKernelGGL((permute_fwd_pool_kernel<float, 64>), dim3(blocks), dim3(kThreads), 0, s,
                         L, cx, cy, desc);
  } else {
    if (L.d == 128)
      hipLaunchKernelGGL((permute_fwd_pool_kernel<__bf16, 128>), dim3(blocks), dim3(kThreads), 0,
                         s, L, cx, cy, desc);
    else
      hipLaunchKernelGGL((permute_fwd_pool_kernel<__bf16, 64>), dim3(blocks), dim3(kThreads), 0,
                         s, L, cx, cy, desc);
  }
  return launch_status();
}

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
  } else if (dtype == VEDA_F32) {
    const size_t lds = (size_t)L.d * (L.S + 4) * 4;
    hipLaunchKernelGGL(permute_fwd_t_f32_kernel, dim3(blocks), dim3(kThreads), lds, s, L,
                       (const float*)x, (float*)y);
  } else {
    hipLaunchKernelGGL(permute_fwd_t_bf16_kernel, dim3(blocks), dim3(kThreads), 0, s, L,
                       (const Chunk*)x, (Chunk*)y);
  }
  return launch_status();
}

}  // namespace veda
