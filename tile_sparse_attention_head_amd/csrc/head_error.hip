// Per-head squared error between two token-order attention outputs, the
// measure the head-aware tiling search minimises (Veda §2.2: the tile shape
// of each head is chosen offline by the approximation error between the
// full-attention and the sparse-attention outputs).
//
// err[h] = sum over tokens n and channels c of (a[n][h][c] - b[n][h][c])^2
// ref[h] = sum of a[n][h][c]^2
//
// Pass 1: a (kChunksX x heads) grid; each workgroup walks a strided share of
// the head's token rows in 16-byte chunks (a wave covers whole 2d-byte rows)
// and accumulates in f64, then writes its two partial sums.  Pass 2: one
// workgroup per head adds the kChunksX partials in index order.  Both passes
// have a fixed order, so results are deterministic.  HBM-bound: reads both
// tensors once.
#include "veda_internal.hpp"

namespace veda {
namespace {

constexpr int kThreads = 256;
constexpr int kChunksX = 64;   // workgroups per head in pass 1

struct U4 { uint32_t x, y, z, w; };

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < kThreads / 64; ++w) t += red[w];
  return t;
}

__global__ __launch_bounds__(kThreads) void head_error_partial_kernel(DevLayout L,
                                                                      const U4* __restrict__ a,
                                                                      const U4* __restrict__ b,
                                                                      double* __restrict__ part) {
  __shared__ double red[kThreads / 64];
  const int h = blockIdx.y;
  const int cpr = L.d / 8;                        // 16-byte chunks per row
  const int rows_per_pass = kThreads / cpr;       // token rows a workgroup covers per pass
  const int c = threadIdx.x % cpr;
  const int64_t N = (int64_t)L.T * L.H * L.W;
  double e = 0.0, r = 0.0;
  for (int64_t n = (int64_t)blockIdx.x * rows_per_pass + threadIdx.x / cpr; n < N;
       n += (int64_t)kChunksX * rows_per_pass) {
    const int64_t x = (n * L.heads + h) * cpr + c;
    const U4 va = a[x], vb = b[x];
    const uint32_t wa[4] = {va.x, va.y, va.z, va.w}, wb[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const double a0 = bf_lo(wa[q]), a1 = bf_hi(wa[q]);
      const double d0 = a0 - (double)bf_lo(wb[q]), d1 = a1 - (double)bf_hi(wb[q]);
      e = fma(d0, d0, fma(d1, d1, e));
      r = fma(a0, a0, fma(a1, a1, r));
    }
  }
  e = block_sum_f64(e, red);
  r = block_sum_f64(r, red);
  if (threadIdx.x == 0) {
    part[((int64_t)h * kChunksX + blockIdx.x) * 2] = e;
    part[((int64_t)h * kChunksX + blockIdx.x) * 2 + 1] = r;
  }
}

__global__ __launch_bounds__(64) void head_error_final_kernel(const double* __restrict__ part,
                                                              double* __restrict__ err,
                                                              double* ref) {
  const int h = blockIdx.x;
  if (threadIdx.x != 0) return;
  double e = 0.0, r = 0.0;
  for (int i = 0; i < kChunksX; ++i) {
    e += part[((int64_t)h * kChunksX + i) * 2];
    r += part[((int64_t)h * kChunksX + i) * 2 + 1];
  }
  err[h] = e;
  if (ref != nullptr) ref[h] = r;
}

// The tiling search's choice: one lane per head scans the candidates in
// order and keeps the first strictly smaller error.
__global__ __launch_bounds__(64) void head_choose_kernel(const double* __restrict__ err,
                                                         int n_cand, int heads,
                                                         int32_t* __restrict__ choice) {
  const int h = blockIdx.x * 64 + threadIdx.x;
  if (h >= heads) return;
  int best = 0;
  double be = err[h];
  for (int c = 1; c < n_cand; ++c) {
    const double e = err[(int64_t)c * heads + h];
    if (e < be) {
      be = e;
      best = c;
    }
  }
  choice[h] = best;
}

}  // namespace

int launch_head_choose(const double* err, int n_cand, int heads, int32_t* choice, hipStream_t s) {
  hipLaunchKernelGGL(head_choose_kernel, dim3((heads + 63) / 64), dim3(64), 0, s, err, n_cand, heads,
                     choice);
  return launch_status();
}

int64_t head_error_workspace_bytes(const DevLayout& L) {
  return (int64_t)L.heads * kChunksX * 2 * 8;
}

int launch_head_error(const DevLayout& L, const void* a, const void* b, double* err, double* ref,
                      void* workspace, hipStream_t s) {
  double* part = static_cast<double*>(workspace);
  hipLaunchKernelGGL(head_error_partial_kernel, dim3(kChunksX, L.heads), dim3(kThreads), 0, s, L,
                     (const U4*)a, (const U4*)b, part);
  hipLaunchKernelGGL(head_error_final_kernel, dim3(L.heads), dim3(64), 0, s, part, err, ref);
  return launch_status();
}

}  // namespace veda
