// Distillation step of the tile-score estimator (Veda §2.1, optimisation): the
// row-wise KL divergence between the max-pooled full-attention map (the
// reference, each row normalised to sum 1) and the softmax of the estimator's
// tile scores, averaged over the subset's query-tile rows, and its gradients
// with respect to the per-head projection weights and biases.  The TripPool
// descriptors are constants (the stop-gradient on the backbone features), so
// with S = phi_q phi_k^T and phi = desc W^T + b:
//
//   G[s][j]   = (softmax(S[i_s])[j] - t[s][j]) / R          (dL/dS, row i_s)
//   dphi_q[s] = G[s] phi_k                                   (per subset entry)
//   dphi_k[j] = sum over the head's entries s of G[s][j] phi_q[i_s]
//   dW_side   = dphi_side^T desc_side,   db_side = sum of dphi_side rows
//
// All arithmetic is f32 and every sum runs in a fixed order, so results are
// deterministic.  The work is small next to the map that produces the
// reference (a few matrix products of n_h x d_e x 3d per head), and the
// kernels are plain LDS-tiled vector code.
#include <mutex>

#include "veda_internal.hpp"

namespace veda {
namespace {

constexpr int kThreads = 256;

struct DistillWs {          // carved out of the caller's workspace
  int32_t* count;           // [1]   valid subset entries (R)
  int32_t* head_start;      // [heads + 1] start of each head's entries in `order`
  int32_t* order;           // [n_sub] valid entries grouped by head, ascending s
  float* g;                 // [n_sub][max_tiles]
  float* row_loss;          // [n_sub]
  float* dphi_q;            // [n_sub][d_e]
  float* dphi_k;            // [tiles][d_e]
};

__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w];
  return t;
}

__device__ __forceinline__ float block_max(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t = fmaxf(t, red[w]);
  return t;
}

// Head of subset entry s, or -1 for an entry outside [0, tiles).
__device__ __forceinline__ int entry_head(const DevLayout& L, const int32_t* q_tiles, int s) {
  const int64_t g = q_tiles[s];
  if (g < 0 || g >= L.tile_off[L.heads]) return -1;
  return head_of_tile(L, g);
}

// One workgroup: the valid entries grouped by head, in ascending s within a
// head (a stable compaction per head with a block prefix sum), their count
// R and each head's start.
__global__ __launch_bounds__(kThreads) void distill_group_kernel(DevLayout L,
                                                                 const int32_t* __restrict__ q_tiles,
                                                                 int n_sub, DistillWs ws) {
  __shared__ int wave_tot[kThreads / 64];
  __shared__ int base_s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) base_s = 0;
  __syncthreads();
  for (int h = 0; h < L.heads; ++h) {
    if (threadIdx.x == 0) ws.head_start[h] = base_s;
    for (int c0 = 0; c0 < n_sub; c0 += kThreads) {
      const int s = c0 + threadIdx.x;
      const int mine = s < n_sub && entry_head(L, q_tiles, s) == h;
      const uint64_t bal = __ballot(mine);
      const int below = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) wave_tot[wave] = __popcll(bal);
      __syncthreads();
      int off = base_s;
      for (int w = 0; w < wave; ++w) off += wave_tot[w];
      if (mine) ws.order[off + below] = s;
      __syncthreads();
      if (threadIdx.x == 0)
        for (int w = 0; w < kThreads / 64; ++w) base_s += wave_tot[w];
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) {
    ws.head_start[L.heads] = base_s;
    ws.count[0] = base_s;
  }
}

// One workgroup per subset entry: row KL and G = (p - t) / R.
__global__ __launch_bounds__(kThreads) void distill_rows_kernel(DevLayout L,
                                                                const float* __restrict__ scores,
                                                                const float* __restrict__ map,
                                                                const int32_t* __restrict__ q_tiles,
                                                                DistillWs ws) {
  __shared__ float red[kThreads / 64];
  const int s = blockIdx.x;
  const int mt = L.max_tiles;
  float* grow = ws.g + (int64_t)s * mt;
  const int h = entry_head(L, q_tiles, s);
  const int R = ws.count[0];
  if (h < 0 || R == 0) {
    for (int j = threadIdx.x; j < mt; j += kThreads) grow[j] = 0.f;
    if (threadIdx.x == 0) ws.row_loss[s] = 0.f;
    return;
  }
  const int n = (int)(L.tile_off[h + 1] - L.tile_off[h]);
  const int i = (int)(q_tiles[s] - L.tile_off[h]);
  const float* srow = scores + L.score_off[h] + (int64_t)i * n;
  const float* mrow = map + (int64_t)s * mt;
  float mx = -INFINITY, msum = 0.f;
  for (int j = threadIdx.x; j < n; j += kThreads) {
    mx = fmaxf(mx, srow[j]);
    msum += mrow[j];
  }
  mx = block_max(mx, red);
  msum = block_sum(msum, red);
  if (!(msum > 0.f)) {   // no reference mass: the row contributes nothing
    for (int j = threadIdx.x; j < mt; j += kThreads) grow[j] = 0.f;
    if (threadIdx.x == 0) ws.row_loss[s] = 0.f;
    return;
  }
  float esum = 0.f;
  for (int j = threadIdx.x; j < n; j += kThreads) esum += expf(srow[j] - mx);
  esum = block_sum(esum, red);
  const float log_z = mx + logf(esum);          // log sum_j exp(S_j)
  const float inv_m = 1.0f / msum, inv_r = 1.0f / (float)R;
  float kl = 0.f;
  for (int j = threadIdx.x; j < mt; j += kThreads) {
    float gv = 0.f;
    if (j < n) {
      const float logp = srow[j] - log_z;
      const float t = mrow[j] * inv_m;
      if (t > 0.f) kl += t * (logf(t) - logp);
      gv = (expf(logp) - t) * inv_r;
    }
    grow[j] = gv;
  }
  kl = block_sum(kl, red);
  if (threadIdx.x == 0) ws.row_loss[s] = kl * inv_r;
}

// dphi_q[s][e] = sum_j G[s][j] phi_k[j][e]: one workgroup per subset entry,
// the G row staged through LDS, one output column per thread.
__global__ __launch_bounds__(kThreads) void distill_dphi_q_kernel(DevLayout L, int d_e,
                                                                  const float* __restrict__ phi,
                                                                  const int32_t* __restrict__ q_tiles,
                                                                  DistillWs ws) {
  __shared__ float gs[kThreads];
  const int s = blockIdx.x;
  float* out = ws.dphi_q + (int64_t)s * d_e;
  const int h = entry_head(L, q_tiles, s);
  if (h < 0) {
    for (int e = threadIdx.x; e < d_e; e += kThreads) out[e] = 0.f;
    return;
  }
  const int n = (int)(L.tile_off[h + 1] - L.tile_off[h]);
  const float* grow = ws.g + (int64_t)s * L.max_tiles;
  const float* phik = phi + (L.tile_off[L.heads] + L.tile_off[h]) * (int64_t)d_e;
  const int e = threadIdx.x;
  float acc = 0.f;
  for (int j0 = 0; j0 < n; j0 += kThreads) {
    __syncthreads();
    if (j0 + threadIdx.x < n) gs[threadIdx.x] = grow[j0 + threadIdx.x];
    __syncthreads();
    const int m = min(kThreads, n - j0);
    if (e < d_e)
      for (int jj = 0; jj < m; ++jj) acc = fmaf(gs[jj], phik[(int64_t)(j0 + jj) * d_e + e], acc);
  }
  if (e < d_e) out[e] = acc;
}

// dphi_k[g][e] = sum over head h's entries s (in `order`) of
// G[s][j] phi_q[q_tiles[s]][e], for key tile g = tile_off[h] + j: one
// workgroup per key tile.  Each chunk of entries first has its query tile
// and G value staged in LDS (one parallel round of loads), so the loop over
// entries issues independent row loads.
__global__ __launch_bounds__(kThreads) void distill_dphi_k_kernel(DevLayout L, int d_e,
                                                                  const float* __restrict__ phi,
                                                                  const int32_t* __restrict__ q_tiles,
                                                                  DistillWs ws) {
  __shared__ int qs[kThreads];
  __shared__ float gv[kThreads];
  const int64_t g = blockIdx.x;
  const int h = head_of_tile(L, g);
  const int j = (int)(g - L.tile_off[h]);
  const int a = ws.head_start[h], b = ws.head_start[h + 1];
  const int e = threadIdx.x;
  float acc = 0.f;
  for (int r0 = a; r0 < b; r0 += kThreads) {
    __syncthreads();
    if (r0 + threadIdx.x < b) {
      const int s = ws.order[r0 + threadIdx.x];
      qs[threadIdx.x] = q_tiles[s];
      gv[threadIdx.x] = ws.g[(int64_t)s * L.max_tiles + j];
    }
    __syncthreads();
    const int m = min(kThreads, b - r0);
    if (e < d_e)
      for (int rr = 0; rr < m; ++rr) acc = fmaf(gv[rr], phi[(int64_t)qs[rr] * d_e + e], acc);
  }
  if (e < d_e) ws.dphi_k[g * d_e + e] = acc;
}

// dW_side[h][e][c] = sum over the head's rows r of dphi[r][e] desc[r][c]
// (and, from the c-block 0 workgroups, db_side[h][e] = sum_r dphi[r][e]).
// Side 0 (query): rows are the head's subset entries in `order`; side 1
// (key): the head's key tiles.  A 64 x 64 output block per workgroup, 4 x 4
// per thread, 16 rows at a time through LDS.
constexpr int kWB = 64, kWR = 16;

__global__ __launch_bounds__(kThreads) void distill_dw_kernel(DevLayout L, int d_e,
                                                              const float* __restrict__ desc,
                                                              const int32_t* __restrict__ q_tiles,
                                                              DistillWs ws, float* __restrict__ dwq,
                                                              float* __restrict__ dwk,
                                                              float* dbq, float* dbk) {
  __shared__ float ps[kWR][kWB];   // dphi rows, e
  __shared__ float ds[kWR][kWB];   // desc rows, c
  const int side = blockIdx.z / L.heads, h = blockIdx.z % L.heads;
  const int K3 = 3 * L.d;
  const int c0 = blockIdx.x * kWB, e0 = blockIdx.y * kWB;
  const int64_t tiles = L.tile_off[L.heads];
  int rows;
  if (side == 0) rows = ws.head_start[h + 1] - ws.head_start[h];
  else rows = (int)(L.tile_off[h + 1] - L.tile_off[h]);
  // row r -> (dphi row, desc row)
  auto dphi_row = [&](int r) -> const float* {
    if (side == 0) return ws.dphi_q + (int64_t)ws.order[ws.head_start[h] + r] * d_e;
    return ws.dphi_k + (L.tile_off[h] + r) * (int64_t)d_e;
  };
  auto desc_row = [&](int r) -> const float* {
    if (side == 0) return desc + (int64_t)q_tiles[ws.order[ws.head_start[h] + r]] * K3;
    return desc + (tiles + L.tile_off[h] + r) * (int64_t)K3;
  };
  const int te = (threadIdx.x / 16) * 4, tc = (threadIdx.x % 16) * 4;
  float acc[4][4] = {};
  float bacc = 0.f;   // bias: thread t < 64 of c-block 0 sums column e0 + t
  for (int r0 = 0; r0 < rows; r0 += kWR) {
    // 16 rows x 64 columns of each operand: 1024 values, 4 per thread
    for (int x = threadIdx.x; x < kWR * kWB; x += kThreads) {
      const int rr = x / kWB, cc = x % kWB;
      const bool in = r0 + rr < rows;
      ps[rr][cc] = in && e0 + cc < d_e ? dphi_row(r0 + rr)[e0 + cc] : 0.f;
      ds[rr][cc] = in && c0 + cc < K3 ? desc_row(r0 + rr)[c0 + cc] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < kWR; ++rr) {
      float pv[4], dv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) { pv[a] = ps[rr][te + a]; dv[a] = ds[rr][tc + a]; }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(pv[a], dv[b], acc[a][b]);
    }
    if (blockIdx.x == 0 && threadIdx.x < kWB)
      for (int rr = 0; rr < kWR; ++rr) bacc += ps[rr][threadIdx.x];
    __syncthreads();
  }
  float* dw = (side == 0 ? dwq : dwk) + (int64_t)h * d_e * K3;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int e = e0 + te + a, c = c0 + tc + b;
      if (e < d_e && c < K3) dw[(int64_t)e * K3 + c] = acc[a][b];
    }
  float* db = side == 0 ? dbq : dbk;
  if (db != nullptr && blockIdx.x == 0 && threadIdx.x < kWB && e0 + threadIdx.x < d_e)
    db[(int64_t)h * d_e + e0 + threadIdx.x] = bacc;
}

// loss = sum of the per-entry terms (each already divided by R), in index
// order of fixed-size chunks, one workgroup.
__global__ __launch_bounds__(kThreads) void distill_loss_kernel(int n_sub, DistillWs ws,
                                                                float* __restrict__ loss) {
  __shared__ float red[kThreads / 64];
  float v = 0.f;
  for (int s = threadIdx.x; s < n_sub; s += kThreads) v += ws.row_loss[s];
  v = block_sum(v, red);
  if (threadIdx.x == 0) loss[0] = v;
}

int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }

DistillWs carve(const DevLayout& L, int64_t n_sub, int d_e, void* base, int64_t* total) {
  DistillWs w;
  char* p = static_cast<char*>(base);
  int64_t o = 0;
  auto take = [&](int64_t bytes) {
    char* q = p ? p + o : nullptr;
    o += round256(bytes);
    return q;
  };
  w.count = reinterpret_cast<int32_t*>(take(4));
  w.head_start = reinterpret_cast<int32_t*>(take(4 * (L.heads + 1)));
  w.order = reinterpret_cast<int32_t*>(take(4 * n_sub));
  w.g = reinterpret_cast<float*>(take(4 * n_sub * L.max_tiles));
  w.row_loss = reinterpret_cast<float*>(take(4 * n_sub));
  w.dphi_q = reinterpret_cast<float*>(take(4 * n_sub * (int64_t)d_e));
  w.dphi_k = reinterpret_cast<float*>(take(4 * L.tile_off[L.heads] * (int64_t)d_e));
  *total = o;
  return w;
}

}  // namespace

int64_t distill_workspace_bytes(const DevLayout& L, int64_t n_sub, int d_e) {
  int64_t total = 0;
  carve(L, n_sub, d_e, nullptr, &total);
  return total;
}

// Scratch of veda_distill_grad_noalloc: a device array of the library, one
// copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it names a stand-in, not device
// memory): the address each device holds it at is looked up once per device
// with that device current and kept in `g_scratch`.
static __device__ __align__(256) unsigned char scratch[VEDA_DISTILL_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};
}  // namespace

int distill_static_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return VEDA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return VEDA_ERR_LAUNCH;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return VEDA_OK;
}

int launch_distill(const DevLayout& L, const float* scores, const float* map,
                   const int32_t* q_tiles, int n_sub, const float* desc, const float* phi,
                   int d_e, void* workspace, float* loss, float* dwq, float* dwk, float* dbq,
                   float* dbk, hipStream_t s) {
  int64_t total = 0;
  const DistillWs ws = carve(L, n_sub, d_e, workspace, &total);
  hipLaunchKernelGGL(distill_group_kernel, dim3(1), dim3(kThreads), 0, s, L, q_tiles, n_sub, ws);
  if (n_sub > 0) {
    hipLaunchKernelGGL(distill_rows_kernel, dim3(n_sub), dim3(kThreads), 0, s, L, scores, map,
                       q_tiles, ws);
    hipLaunchKernelGGL(distill_dphi_q_kernel, dim3(n_sub), dim3(kThreads), 0, s, L, d_e, phi,
                       q_tiles, ws);
  }
  const unsigned tiles = (unsigned)L.tile_off[L.heads];
  hipLaunchKernelGGL(distill_dphi_k_kernel, dim3(tiles), dim3(kThreads), 0, s, L, d_e, phi,
                     q_tiles, ws);
  const dim3 wg((3 * L.d + kWB - 1) / kWB, (d_e + kWB - 1) / kWB, 2 * L.heads);
  hipLaunchKernelGGL(distill_dw_kernel, wg, dim3(kThreads), 0, s, L, d_e, desc, q_tiles, ws, dwq,
                     dwk, dbq, dbk);
  hipLaunchKernelGGL(distill_loss_kernel, dim3(1), dim3(kThreads), 0, s, n_sub, ws, loss);
  return launch_status();
}

}  // namespace veda
