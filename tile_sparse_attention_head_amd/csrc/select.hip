// Row-wise top-k of the tile-score matrix, emitted as CSR (the tile selection
// the Veda pages describe: at 95 % sparsity each query tile keeps about 5 %
// of the key tiles, chosen by the estimator's scores).
//
// Rows of up to 2048 columns go to a kernel with one wave per row and the
// keys in registers (see select_wave_kernel); longer rows to one workgroup
// per query-tile row.  Scores are mapped to order-preserving
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

// One wave per row, for rows of at most 64*KPL columns: lane l holds the keys
// of columns l, l + 64, ..., l + 64*(KPL-1) in registers (key 0 past the row's
// end).  The k-th largest key K* is the largest t with at least k keys >= t;
// a threshold is counted over the wave with one compare and a ballot
// population count per register, no barrier.
//
// The search keeps t <= K* with c_lo = count(keys >= t) >= k, and c_hi, the
// count above the range of keys still open (those sharing t's decided upper
// bits), < k:
//   * start: with r = ceil(k / 64) <= 4, every lane's r-th largest key is >=
//     tau0, their minimum over the wave, so at least 64 r >= k keys are >= tau0
//     and K* >= tau0 (tau0 = 0 for larger k); K* <= the row's largest key, so
//     K* has the upper bits tau0 and the largest key share, and t starts there;
//   * while more than 64 keys lie in the open range, the next bit is decided
//     by counting all keys against t | bit;
//   * then those keys (at most 64) are compacted into the wave's LDS, one per
//     lane; the bits they all share are taken at once, and the remaining bits
//     count only them (plus c_hi for the keys above the range).
// On score rows the range holds at most 64 keys after about five full counts.
//
// The final pass walks the columns in index order and writes each kept column
// at the position the ballot prefix gives it: ascending, deterministic, and the
// same result as the workgroup kernel.  When exactly k keys are >= K* (no tie
// at K* beyond the ones needed) it keeps every key >= K*; otherwise every key
// > K* and the lowest-index keys == K*.
constexpr int kWaves = 4;
constexpr int kCand = 64;   // compacted keys per wave (one per lane)

__device__ __forceinline__ uint32_t med3u(uint32_t a, uint32_t b, uint32_t c) {
  return max(min(a, b), min(max(a, b), c));
}
__device__ __forceinline__ uint32_t lane_prefix(uint64_t bal) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}
// bits of x above bit `top` kept, the rest cleared (top < 0: all kept; top =
// 31: none)
__device__ __forceinline__ uint32_t upper_bits(uint32_t x, int top) {
  return top < 0 ? x : top >= 31 ? 0u : (x & ~((2u << top) - 1u));
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

// The selection of one row by one wave, from the row's keys in registers
// (lane l: columns l, l + 64, ..., key 0 past the row's end), 1 <= k <= n:
// writes the k kept columns, ascending, to out.  cl: kCand words of LDS for
// this wave.
template <int KPL>
__device__ __forceinline__ void select_from_keys(const uint32_t (&key)[KPL], int n, int k,
                                                 int lane, uint32_t* cl,
                                                 int32_t* __restrict__ out) {
  // real keys >= v over the wave, for v > 0 (padding keys are 0 and never count)
  auto count_ge = [&](uint32_t v) {
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) cnt += __popcll(__ballot(key[j] >= v));
    return cnt;
  };
  // the lower bound tau0 and the row's largest key
  const int r = (k + 63) / 64;
  uint32_t tau, top_key;
  if (r <= 2) {
    uint32_t m1 = 0u, m2 = 0u;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      m2 = med3u(m1, m2, key[j]);
      m1 = max(m1, key[j]);
    }
    tau = r == 1 ? m1 : m2;
    top_key = m1;
  } else if (r <= 4) {
    uint32_t m1 = 0u, m2 = 0u, m3 = 0u, m4 = 0u;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const uint32_t x = key[j];
      m4 = med3u(m3, m4, x);
      m3 = med3u(m2, m3, x);
      m2 = med3u(m1, m2, x);
      m1 = max(m1, x);
    }
    tau = r == 3 ? m3 : m4;
    top_key = m1;
  } else {
    top_key = 0u;
#pragma unroll
    for (int j = 0; j < KPL; ++j) top_key = max(top_key, key[j]);
    tau = 0u;
  }
  tau = wave_min(tau);
  top_key = wave_max(top_key);

  int b = tau == top_key ? -1 : 31 - __builtin_clz(tau ^ top_key);
  uint32_t t = upper_bits(tau, b);
  int c_lo = t == 0u ? n : count_ge(t);
  int c_hi = 0;
#pragma unroll 1
  for (; b >= 0 && c_lo - c_hi > kCand; --b) {
    const uint32_t cand = t | (1u << b);
    const int cnt = count_ge(cand);
    if (cnt >= k) {
      t = cand;
      c_lo = cnt;
    } else {
      c_hi = cnt;
    }
  }
  if (b >= 0) {
    // the c_lo - c_hi <= 64 real keys in [t, t + 2^(b+1)): one per lane
    const uint32_t span = b >= 31 ? 0xffffffffu : (2u << b) - 1u;
    int base = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const bool is_c = 64 * j + lane < n && key[j] >= t && key[j] - t <= span;
      const uint64_t bal = __ballot(is_c);
      if (is_c) cl[base + lane_prefix(bal)] = key[j];
      base += __popcll(bal);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const bool live = lane < base;
    const uint32_t mine = live ? cl[lane] : 0u;
    // K* is one of them: its bits above where their minimum and maximum differ
    // are decided
    const uint32_t cmin = wave_min(live ? mine : 0xffffffffu);
    const uint32_t cmax = wave_max(live ? mine : 0u);
    const int top2 = cmin == cmax ? -1 : 31 - __builtin_clz(cmin ^ cmax);
    t = upper_bits(cmin, top2);
    c_lo = c_hi + base;
    const int above = c_hi;
#pragma unroll 1
    for (b = top2; b >= 0; --b) {
      const uint32_t cand = t | (1u << b);
      const int cnt = above + __popcll(__ballot(live && mine >= cand));
      if (cnt >= k) {
        t = cand;
        c_lo = cnt;
      }
    }
  }
  // t = K*, c_lo = count(keys >= K*)
  int pos = 0;
  if (c_lo == k) {
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int c = 64 * j + lane;
      const bool take = c < n && key[j] >= t;
      const uint64_t bt = __ballot(take);
      if (take) out[pos + lane_prefix(bt)] = c;
      pos += __popcll(bt);
    }
    return;
  }
  int gt = 0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) gt += __popcll(__ballot(64 * j + lane < n && key[j] > t));
  const int need = k - gt;
  int eq_seen = 0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int c = 64 * j + lane;
    const bool real = c < n;
    const bool eq = real && key[j] == t;
    const uint64_t beq = __ballot(eq);
    const int eq_rank = eq_seen + (int)lane_prefix(beq);
    const bool take = (real && key[j] > t) || (eq && eq_rank < need);
    const uint64_t bt = __ballot(take);
    if (take) out[pos + lane_prefix(bt)] = c;
    pos += __popcll(bt);
    eq_seen += __popcll(beq);
  }
}

template <int KPL>
__global__ __launch_bounds__(64 * kWaves) void select_wave_kernel(DevLayout L, SelectArgs sa,
                                                                  const float* __restrict__ scores,
                                                                  int32_t* __restrict__ row_ptr,
                                                                  int32_t* __restrict__ col_idx) {
  __shared__ uint32_t cand_lds[kWaves][kCand];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t r = (int64_t)blockIdx.x * kWaves + wave;
  if (r >= L.tile_off[L.heads]) return;
  const int h = head_of_tile(L, r);
  const int i = (int)(r - L.tile_off[h]);
  const int n = (int)(L.tile_off[h + 1] - L.tile_off[h]);
  const int k = sa.k[h];
  const int64_t start = sa.nnz_off[h] + (int64_t)i * k;
  if (lane == 0) {
    row_ptr[r] = (int32_t)start;
    if (r + 1 == L.tile_off[L.heads]) row_ptr[r + 1] = (int32_t)sa.nnz_off[L.heads];
  }
  const float* row = scores + L.score_off[h] + (int64_t)i * n;
  // range-checked buffer loads over the row (columns past it read 0): every
  // load is unconditional, so all of them are in flight at once, and the
  // padding keys are masked to 0 after
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), (short)0, n * 4, 0x00020000);
  float v[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j)
    v[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (64 * j + lane) * 4, 0, 0));
  uint32_t key[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j)
    key[j] = order_key(v[j]) & (0u - (uint32_t)(64 * j + lane < n));
  select_from_keys<KPL>(key, n, k, lane, cand_lds[wave], col_idx + start);
}

// ---- the score product fused with the selection ---------------------------
// One workgroup of kSSRows waves per block of kSSRows query-tile rows of one
// head; wave w owns row w.  Phase 1 computes the block's scores
//   s[w][j] = <phi_Q[row w], phi_K[j]>,  j < n:
// key tiles' phi_K rows are staged through LDS 64 at a time (lane c of every
// wave takes column c of the stage), each wave's phi_Q row sits in LDS and is
// read as a broadcast, and every score is the sequential FMA chain over the
// d_e components that the standalone score product uses, so the values are
// the same f32 numbers.  Lane l of wave w computes columns l, l + 64, ... of
// row w, which is the register layout of the wave-per-row selection above, so
// phase 2 runs that selection on the scores where they were computed.  The
// n x n score matrix is never written to memory.
constexpr int kSSRows = 8;          // query rows (and waves) per workgroup
constexpr int kSSCols = 64;         // key rows per stage

struct ScoreSelectArgs {
  int32_t k[VEDA_MAX_HEADS];
  int64_t nnz_off[VEDA_MAX_HEADS + 1];
  int32_t blk_off[VEDA_MAX_HEADS + 1];   // first workgroup of each head
};

template <int KPL, int DE>
__global__ __launch_bounds__(64 * kSSRows) void score_select_kernel(
    DevLayout L, ScoreSelectArgs sa, const float* __restrict__ phi, int32_t* __restrict__ row_ptr,
    int32_t* __restrict__ col_idx) {
  constexpr int CPR = DE / 4;                       // 16-byte chunks per phi row
  static_assert(CPR % 8 == 0, "phi rows of whole 32-float groups");
  // stage of kSSCols phi_K rows, padded by 4 floats (the 16 lanes of a 128-bit
  // read that take one chunk of 16 rows then hit 16 distinct bank groups);
  // after phase 1 it holds the waves' selection candidates
  constexpr int RS = DE + 4;
  __shared__ __attribute__((aligned(16))) float stage[kSSCols * RS];
  __shared__ __attribute__((aligned(16))) float qs[kSSRows][DE];
  static_assert(kSSCols * RS >= kSSRows * kCand, "candidate buffers fit in the stage");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x;
  int h = 0;
  while (h + 1 < L.heads && sa.blk_off[h + 1] <= b) ++h;
  const int n = (int)(L.tile_off[h + 1] - L.tile_off[h]);
  const int i0 = (b - sa.blk_off[h]) * kSSRows;
  const int i = i0 + wave;                          // this wave's row (may lie past n)
  const float* pk = phi + (L.tile_off[L.heads] + L.tile_off[h]) * DE;
  // this wave's phi_Q row (a valid row when i >= n; its scores are unused)
  const float* pq = phi + (L.tile_off[h] + min(i, n - 1)) * DE;
  if (lane < CPR)
    *reinterpret_cast<float4*>(&qs[wave][4 * lane]) = *reinterpret_cast<const float4*>(pq + 4 * lane);

  constexpr int PF = kSSCols * CPR / (64 * kSSRows);   // 16-byte chunks per thread per stage
  static_assert(PF * 64 * kSSRows == kSSCols * CPR, "stage splits evenly");
  typedef float v4f __attribute__((ext_vector_type(4)));
  v4f pf[PF];
  auto fetch = [&](int j0) {
    // the base goes through an empty asm statement here, after the stage's
    // barrier: the loads cannot be hoisted into earlier stages (the
    // unrolled stages would otherwise hold every stage's prefetch at once)
    typedef __attribute__((address_space(1))) const v4f gv4f;
    gv4f* base = (gv4f*)(pk + (int64_t)j0 * DE);
    asm volatile("" : "+s"(base));
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int x = u * 64 * kSSRows + tid;         // chunk of the stage
      const int r = x / CPR, c = x % CPR;
      pf[u] = j0 + r < n ? base[r * CPR + c] : v4f{0.f, 0.f, 0.f, 0.f};
    }
  };
  // Stage jj holds key rows 64 jj .. 64 jj + 63, and lane l of every wave
  // computes column 64 jj + l of its row: exactly the key the selection keeps
  // in register key[jj] of lane l, so the scores go straight to registers.
  uint32_t key[KPL];
  fetch(0);
#pragma unroll
  for (int jj = 0; jj < KPL; ++jj) {
    const int j0 = 64 * jj;
    key[jj] = 0u;
    if (j0 >= n) continue;                          // uniform: no barrier is skipped by some waves only
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int x = u * 64 * kSSRows + tid;
      const int r = x / CPR, c = x % CPR;
      *reinterpret_cast<v4f*>(&stage[r * RS + 4 * c]) = pf[u];
    }
    __syncthreads();
    if (j0 + kSSCols < n) fetch(j0 + kSSCols);     // in flight during the products
    float acc = 0.f;
    const float* krow = &stage[lane * RS];
    // the phi_Q row is read again in every stage: an LDS pointer hidden from
    // the compiler keeps it from holding 4*CPR loop-invariant registers
    typedef __attribute__((address_space(3))) const v4f lds_v4f;
    lds_v4f* qrow = (lds_v4f*)(&qs[wave][0]);
    asm volatile("" : "+v"(qrow));
    // eight chunks at a time, so that few operand reads are in flight
#pragma unroll
    for (int cg = 0; cg < CPR; cg += 8) {
#pragma unroll
      for (int c = cg; c < cg + 8; ++c) {
        const float4 kv = *reinterpret_cast<const float4*>(&krow[4 * c]);
        const v4f qv = qrow[c];
        acc = fmaf(qv.x, kv.x, acc);
        acc = fmaf(qv.y, kv.y, acc);
        acc = fmaf(qv.z, kv.z, acc);
        acc = fmaf(qv.w, kv.w, acc);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the products are done here for every lane (the compiler may not sink
    // them into the masked assignment below and hoist all their reads)
    asm volatile("" : "+v"(acc));
    key[jj] = j0 + lane < n ? order_key(acc + 0.f) : 0u;
    __syncthreads();
  }
  if (i >= n) return;
  const int k = sa.k[h];
  const int64_t start = sa.nnz_off[h] + (int64_t)i * k;
  const int64_t r = L.tile_off[h] + i;
  if (lane == 0) {
    row_ptr[r] = (int32_t)start;
    if (r + 1 == L.tile_off[L.heads]) row_ptr[r + 1] = (int32_t)sa.nnz_off[L.heads];
  }
  select_from_keys<KPL>(key, n, k, lane, reinterpret_cast<uint32_t*>(stage) + wave * kCand,
                        col_idx + start);
}

}  // namespace

int launch_score_select(const DevLayout& L, const float* phi, int d_e, const int32_t* k_host,
                        int32_t* row_ptr, int32_t* col_idx, hipStream_t s) {
  ScoreSelectArgs sa;
  sa.nnz_off[0] = 0;
  sa.blk_off[0] = 0;
  for (int h = 0; h < L.heads; ++h) {
    const int64_t n = L.tile_off[h + 1] - L.tile_off[h];
    sa.k[h] = k_host[h];
    sa.nnz_off[h + 1] = sa.nnz_off[h] + n * (int64_t)k_host[h];
    sa.blk_off[h + 1] = sa.blk_off[h] + (int32_t)((n + kSSRows - 1) / kSSRows);
  }
  const unsigned wgs = (unsigned)sa.blk_off[L.heads];
  if (wgs == 0) return VEDA_OK;
  const dim3 block(64 * kSSRows);
#define VEDA_SS(KPL, DE) \
  hipLaunchKernelGGL((score_select_kernel<KPL, DE>), dim3(wgs), block, 0, s, L, sa, phi, row_ptr, col_idx)
  if (d_e == 128) {
    if (L.max_tiles <= 512) VEDA_SS(8, 128);
    else if (L.max_tiles <= 1024) VEDA_SS(16, 128);
    else VEDA_SS(32, 128);
  } else {
    if (L.max_tiles <= 512) VEDA_SS(8, 64);
    else if (L.max_tiles <= 1024) VEDA_SS(16, 64);
    else VEDA_SS(32, 64);
  }
#undef VEDA_SS
  return launch_status();
}

int score_select_max_cols() { return 64 * 32; }

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
  const unsigned wgs = (rows + kWaves - 1) / kWaves;
  if (L.max_tiles <= 512)
    hipLaunchKernelGGL(select_wave_kernel<8>, dim3(wgs), dim3(64 * kWaves), 0, s, L, sa, scores,
                       row_ptr, col_idx);
  else if (L.max_tiles <= 1024)
    hipLaunchKernelGGL(select_wave_kernel<16>, dim3(wgs), dim3(64 * kWaves), 0, s, L, sa, scores,
                       row_ptr, col_idx);
  else if (L.max_tiles <= 2048)
    hipLaunchKernelGGL(select_wave_kernel<32>, dim3(wgs), dim3(64 * kWaves), 0, s, L, sa, scores,
                       row_ptr, col_idx);
  else
    hipLaunchKernelGGL(select_kernel, dim3(rows), dim3(kThreads),
                       (size_t)L.max_tiles * sizeof(uint32_t), s, L, sa, scores, row_ptr, col_idx);
  return launch_status();
}

int select_max_cols() { return kMaxCols; }

}  // namespace veda
