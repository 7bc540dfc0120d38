// Row-wise top-k of the tile-score matrix, emitted as CSR (the tile selection
// the Veda pages describe: at 95 % sparsity each query tile keeps about 5 %
// of the key tiles, chosen by the estimator's scores).
//
// One workgroup per query-tile row.  Scores are mapped to order-preserving
// 32-bit keys (NaN -> 0, below every number; -0.0 folded onto +0.0) and kept
// in LDS.  A most-significant-digit-first radix select (four 8-bit rounds,
// LDS histograms) finds the k-th largest key K* and how many of the keys equal
// to K* are needed.  A final pass in index order keeps every key > K* and the
// lowest-index keys == K*, writing them through a block prefix sum, so each
// row comes out ascending and the result does not depend on thread timing.
#include "veda_internal.hpp"

namespace veda {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxCols = 16384;

struct SelectArgs {
  int32_t k[VEDA_MAX_HEADS];
  int64_t nnz_off[VEDA_MAX_HEADS + 1];
};

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (f != f) return 0u;                 // NaN ranks below -inf
  if (b == 0x80000000u) b = 0u;          // -0.0 == +0.0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Exclusive prefix sum of one value per thread over the workgroup.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wave_tot[w];
  __syncthreads();
  return base + incl - v;
}

__global__ __launch_bounds__(kThreads) void select_kernel(DevLayout L, SelectArgs sa,
                                                          const float* __restrict__ scores,
                                                          int32_t* __restrict__ row_ptr,
                                                          int32_t* __restrict__ col_idx) {
  extern __shared__ uint32_t keys[];
  __shared__ int hist[256];
  __shared__ int wave_tot[kThreads / 64];
  __shared__ int sel_digit, sel_above;
  const int64_t r = blockIdx.x;
  const int h = head_of_tile(L, r);
  const int i = (int)(r - L.tile_off[h]);
  const int n = (int)(L.tile_off[h + 1] - L.tile_off[h]);
  const int k = sa.k[h];
  const int64_t start = sa.nnz_off[h] + (int64_t)i * k;
  if (threadIdx.x == 0) {
    row_ptr[r] = (int32_t)start;
    if (r + 1 == L.tile_off[L.heads]) row_ptr[r + 1] = (int32_t)sa.nnz_off[L.heads];
  }
  const float* row = scores + L.score_off[h] + (int64_t)i * n;
  for (int c = threadIdx.x; c < n; c += kThreads) keys[c] = order_key(row[c]);

  uint32_t prefix = 0u, mask = 0u;
  int need = k;                          // still to take among keys matching prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[threadIdx.x] = 0;
    __syncthreads();
    for (int c = threadIdx.x; c < n; c += kThreads) {
      const uint32_t key = keys[c];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    // wave 0: find the digit where the count from the top reaches `need`
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      // lane l owns digits 255-4l-3 .. 255-4l (descending groups of 4)
      int cnt[4], gs = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) { cnt[q] = hist[255 - 4 * lane - q]; gs += cnt[q]; }
      int incl = gs;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      const int excl = incl - gs;
      if (excl < need && incl >= need) {
        int above = excl;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (above + cnt[q] >= need) { sel_digit = 255 - 4 * lane - q; sel_above = above; break; }
          above += cnt[q];
        }
      }
    }
    __syncthreads();
    const uint32_t dg = (uint32_t)sel_digit;
    need -= sel_above;
    prefix |= dg << shift;
    mask |= 255u << shift;
    __syncthreads();
  }
  // prefix is the k-th largest key; `need` (>= 1) keys equal to it are kept.
  const uint32_t kth = prefix;
  const int per = (n + kThreads - 1) / kThreads;
  const int c0 = min(n, (int)threadIdx.x * per), c1 = min(n, c0 + per);
  int n_eq = 0;
  for (int c = c0; c < c1; ++c) n_eq += keys[c] == kth;
  int eq_rank = block_exclusive_scan(n_eq, wave_tot);
  int n_sel = 0;
  {
    int er = eq_rank;
    for (int c = c0; c < c1; ++c) {
      const uint32_t key = keys[c];
      if (key > kth) ++n_sel;
      else if (key == kth) { if (er < need) ++n_sel; ++er; }
    }
  }
  int pos = block_exclusive_scan(n_sel, wave_tot);
  int32_t* out = col_idx + start;
  for (int c = c0; c < c1; ++c) {
    const uint32_t key = keys[c];
    bool take = key > kth;
    if (key == kth) { take = eq_rank < need; ++eq_rank; }
    if (take) out[pos++] = c;
  }
}

}  // namespace

int launch_select(const DevLayout& L, const float* scores, const int32_t* k_host,
                  int32_t* row_ptr, int32_t* col_idx, hipStream_t s) {
  SelectArgs sa;
  sa.nnz_off[0] = 0;
  for (int h = 0; h < L.heads; ++h) {
    sa.k[h] = k_host[h];
    sa.nnz_off[h + 1] = sa.nnz_off[h] + (L.tile_off[h + 1] - L.tile_off[h]) * (int64_t)k_host[h];
  }
  const unsigned rows = (unsigned)L.tile_off[L.heads];
  if (rows == 0) return VEDA_OK;
  hipLaunchKernelGGL(select_kernel, dim3(rows), dim3(kThreads),
                     (size_t)L.max_tiles * sizeof(uint32_t), s, L, sa, scores, row_ptr, col_idx);
  return launch_status();
}

int select_max_cols() { return kMaxCols; }

}  // namespace veda
