// Backward of the tile-skipping attention: dQ, dK, dV over the same kept
// tiles as the forward (Veda §2.3 tile-skipping kernel; the pages fine-tune
// with the sparse path in place but give no backward kernel).  With
// P = softmax(sm_scale Q K^T) over a query tile's kept real keys, dO the
// output gradient and D_r = dO_r . O_r (= sum_c P_rc dP_rc):
//
//   dP = dO V^T,  dS = P (dP - D),  dQ = sm_scale dS K,
//   dK = sm_scale dS^T Q,  dV = P^T dO.
//
// Kernels, all on the matrix cores in the forward's transposed forms:
//  * prep: the inputs gathered into tile order (Q, K, V; dO in the pass that
//    computes D); per query slot D and lse*log2(e)
//    (+inf for padding slots, so their probabilities are exactly 0); the CSR
//    transposed (per key tile, the query tiles keeping it, ascending: counts
//    by integer atomics, positions by binary search in each sorted row, so
//    the lists are deterministic); the dK/dV dispatch order.
//  * dQ: one workgroup per query tile, wave w owns 32 queries (Q and dO rows
//    in registers); per 64-key step S^T = K Q^T (seeded with the mask rows),
//    dP^T = V dO^T - D (seeded with -D), dS^T = P^T dP^T, dQ^T += K^T dS^T,
//    with K^T read transposed out of the staged K rows.
//  * dK/dV: one workgroup per key tile, the heaviest key tiles dispatched
//    first; wave w owns 32 keys (K and V rows in registers); per 32-query
//    step of every query tile keeping the key tile:
//    S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS, with dO^T and
//    Q^T read transposed out of the staged rows.  Padding query rows have
//    P = 0; rows of padding keys are computed and never stored.
// Steps stage their operands HBM -> LDS with buffer_load ... lds, two (dQ)
// or four (dK/dV) steps deep, so a step's copies overlap earlier steps'
// products.
// Results are written straight to token order; every output row is written
// once (a tile that no CSR row keeps gets dK = dV = 0, an empty row dQ = 0).
#include "attn_common.hpp"

namespace veda {
namespace {

using namespace attn;

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
// s_waitcnt operand: vmcnt(0) expcnt(7) lgkmcnt(0) (vmcnt bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmLgkm0 = 0x0070;

// Row (token * heads + head) of slot u of a tile with extent e, or -1 for a
// padding slot.
__device__ __forceinline__ int64_t slot_row(const DevLayout& L, const TileExtent& e, int h,
                                            int u) {
  int dt, dh, dw;
  e.slot_coords(u, dt, dh, dw);
  if (dt >= e.lt || dh >= e.lh || dw >= e.lw) return -1;
  const int64_t tok =
      ((int64_t)(e.it * e.pt + dt) * L.H + (e.ih * e.ph + dh)) * L.W + (e.iw * e.pw + dw);
  return tok * L.heads + h;
}

// ---------------------------------------------------------------- prep
// Per query slot, from the slot's token (o and d_o in token order):
//   delta = dO . O,  lse2 = lse * log2(e)           (dQ kernel)
//   seed_s = -lse / sm_scale,  seed_dp = -delta     (dK/dV kernel: the initial
//   values of its S and dP accumulators, so that P = exp2(sm_scale log2(e) S)
//   and dS = P dP with no further per-element work)
// Padding slots: delta = 0, lse2 = +inf, seed_s = -inf (probabilities 0).
// The same pass gathers dO into tile order (dop, zero rows for padding
// slots) and clears the key-tile pair counts of tile g.
__global__ __launch_bounds__(kThreads) void bwd_delta_kernel(DevLayout L,
                                                             const __bf16* __restrict__ o,
                                                             const __bf16* __restrict__ d_o,
                                                             const float* __restrict__ lse,
                                                             float sm_scale,
                                                             float* __restrict__ delta,
                                                             float* __restrict__ lse2,
                                                             float* __restrict__ seed_s,
                                                             float* __restrict__ seed_dp,
                                                             __bf16* __restrict__ dop,
                                                             int32_t* __restrict__ cnt) {
  const int64_t g = blockIdx.x;
  if (threadIdx.x == 0) cnt[g] = 0;
  const int h = head_of_tile(L, g);
  const TileExtent e = tile_extent(L, h, (int)(g - L.tile_off[h]));
  const int cpr = L.d / 8;                  // 16-byte chunks per row (a power of two)
  const int rpp = kThreads / cpr;
  const int c = threadIdx.x % cpr;
  for (int u0 = 0; u0 < L.S; u0 += rpp) {
    const int u = u0 + (int)threadIdx.x / cpr;
    const int64_t row = u < L.S ? slot_row(L, e, h, u) : -1;
    float acc = 0.f;
    bf16x8 b = {};
    if (row >= 0) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(o + row * L.d + 8 * c);
      b = *reinterpret_cast<const bf16x8*>(d_o + row * L.d + 8 * c);
#pragma unroll
      for (int x = 0; x < 8; ++x) acc = fmaf((float)a[x], (float)b[x], acc);
    }
    if (u < L.S) *reinterpret_cast<bf16x8*>(dop + (g * L.S + u) * L.d + 8 * c) = b;
    for (int off = cpr / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (u < L.S && c == 0) {
      const int64_t slot = g * L.S + u;
      delta[slot] = acc;
      lse2[slot] = row >= 0 ? lse[slot] * kLog2e : INFINITY;
      seed_s[slot] = row >= 0 ? -lse[slot] / sm_scale : -INFINITY;
      seed_dp[slot] = -acc;
    }
  }
}

// occurrences of j in the ascending entries [b, e) of col_idx
__device__ __forceinline__ int count_in_row(const int32_t* __restrict__ ci, int b, int e, int j) {
  int lo = b, hi = e;
  while (lo < hi) {                     // first entry >= j
    const int m = (lo + hi) >> 1;
    if (ci[m] < j) lo = m + 1; else hi = m;
  }
  int lo2 = lo, hi2 = e;
  while (lo2 < hi2) {                   // first entry > j
    const int m = (lo2 + hi2) >> 1;
    if (ci[m] <= j) lo2 = m + 1; else hi2 = m;
  }
  return lo2 - lo;
}

__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  __syncthreads();
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < kThreads / 64; ++w) {
    if (w < wave) base += wave_tot[w];
    tot += wave_tot[w];
  }
  *total = tot;
  return base + incl - v;
}

// per key tile: how many (query tile, occurrence) pairs keep it.  One wave
// per CSR row, one lane per entry, adds the row's in-range entries with
// integer atomics (the counts do not depend on the order of the additions);
// cnt starts at zero.  Entries past `cap` (the CSR's entry count) are not
// read.
__global__ __launch_bounds__(64) void csrt_count_kernel(DevLayout L,
                                                        const int32_t* __restrict__ rp,
                                                        const int32_t* __restrict__ ci,
                                                        int32_t cap, int32_t* __restrict__ cnt) {
  const int64_t i = blockIdx.x;
  const int h = head_of_tile(L, i);
  const int64_t off = L.tile_off[h];
  const int n = (int)(L.tile_off[h + 1] - off);
  const int b = max(rp[i], 0), e = min(rp[i + 1], cap);
  for (int p = b + (int)threadIdx.x; p < e; p += 64) {
    const int j = ci[p];
    if (j >= 0 && j < n) atomicAdd(&cnt[off + j], 1);
  }
}

// Dispatch order of the dK/dV workgroups, longest first.  How many query
// tiles keep a key tile varies widely (tiles no row keeps, tiles nearly
// every row keeps), and one workgroup computes one key tile, so the heavy
// tiles must start first or they alone set the kernel's end.  Workgroup b
// takes order[b]: the key tiles by descending pair count, in 64 buckets of
// 2^shift counts (order within a bucket arbitrary), dealt round-robin to the
// XCDs by the hardware.  (Sorting within each XCD's contiguous range
// instead, which keeps neighbouring key tiles on one L2, measured slower.)
// Each key tile's gradients are computed by one workgroup whatever the
// order, so the order changes the time only, never a result.  Run by one
// workgroup; `segs` contiguous ranges are sorted separately (1: the grid).
constexpr int kOrderBuckets = 64;
__device__ void csrt_order(int64_t tiles, int segs, const int32_t* __restrict__ cnt,
                           int32_t* __restrict__ order) {
  __shared__ int hist[kOrderBuckets];
  __shared__ int red[kThreads / 64];
  int m = 0;
  for (int64_t x = threadIdx.x; x < tiles; x += kThreads) m = max(m, cnt[x]);
  for (int o = 32; o > 0; o >>= 1) m = max(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = 0;
  for (int w = 0; w < kThreads / 64; ++w) m = max(m, red[w]);
  int shift = 0;
  while ((m >> shift) >= kOrderBuckets) ++shift;
  auto bucket = [&](int64_t x) { return kOrderBuckets - 1 - (cnt[x] >> shift); };
  const int64_t per = tiles / segs, rem = tiles % segs;
  for (int sg = 0; sg < segs; ++sg) {
    const int64_t lo = sg * per + min<int64_t>(sg, rem), hi = lo + per + (sg < rem ? 1 : 0);
    if (threadIdx.x < kOrderBuckets) hist[threadIdx.x] = 0;
    __syncthreads();
    for (int64_t x = lo + threadIdx.x; x < hi; x += kThreads) atomicAdd(&hist[bucket(x)], 1);
    __syncthreads();
    if (threadIdx.x == 0) {
      int a = 0;
      for (int b = 0; b < kOrderBuckets; ++b) {
        const int t = hist[b];
        hist[b] = a;
        a += t;
      }
    }
    __syncthreads();
    for (int64_t x = lo + threadIdx.x; x < hi; x += kThreads)
      order[lo + atomicAdd(&hist[bucket(x)], 1)] = (int32_t)x;
    __syncthreads();
  }
}

// ptr[g] = sum of cnt[0..g), ptr[tiles] = total, then the dK/dV dispatch
// order (csrt_order): one workgroup, chunks in order
__global__ __launch_bounds__(kThreads) void csrt_scan_kernel(int64_t tiles,
                                                             const int32_t* __restrict__ cnt,
                                                             int32_t* __restrict__ ptr,
                                                             int32_t* __restrict__ order) {
  __shared__ int wave_tot[kThreads / 64];
  int carry = 0;
  for (int64_t x0 = 0; x0 < tiles; x0 += kThreads) {
    const int64_t x = x0 + threadIdx.x;
    const int v = x < tiles ? cnt[x] : 0;
    int tot = 0;
    const int ex = block_exclusive_scan(v, wave_tot, &tot);
    if (x < tiles) ptr[x] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) ptr[tiles] = carry;
  csrt_order(tiles, 1, cnt, order);
}

// rowt[ptr[g] ..] = the head-local query tiles keeping key tile g, ascending
// (a tile kept twice by one row appears twice).  Reads and writes stay below
// `cap` (the CSR's entry count) even for rows that are not sorted.
__global__ __launch_bounds__(kThreads) void csrt_fill_kernel(DevLayout L,
                                                             const int32_t* __restrict__ rp,
                                                             const int32_t* __restrict__ ci,
                                                             const int32_t* __restrict__ ptr,
                                                             int32_t cap,
                                                             int32_t* __restrict__ rowt) {
  __shared__ int wave_tot[kThreads / 64];
  const int64_t g = blockIdx.x;
  const int h = head_of_tile(L, g);
  const int64_t off = L.tile_off[h];
  const int n = (int)(L.tile_off[h + 1] - off), j = (int)(g - off);
  int base = ptr[g];
  for (int i0 = 0; i0 < n; i0 += kThreads) {
    const int i = i0 + threadIdx.x;
    const int c =
        i < n ? count_in_row(ci, max(rp[off + i], 0), min(rp[off + i + 1], cap), j) : 0;
    int tot = 0;
    const int ex = block_exclusive_scan(c, wave_tot, &tot);
    for (int r = 0; r < c; ++r)
      if (base + ex + r < cap) rowt[base + ex + r] = i;
    base += tot;
  }
}

// R rows of one step (Q or dO rows of 32 queries for dK/dV, K or V rows of
// 64 keys for dQ) in LDS, laid out so that both read patterns of the
// backward products are free of bank conflicts (64 banks of 4 bytes; a
// 128-bit read serves 16 lanes a cycle, a 64-bit one 32):
//   [32-dim block b][row r][64 bytes], the four 16-byte chunks of a row's
//   block stored in the order c ^ ((r >> 2) & 3).
// * Row reads (the A operand of S and dP: lane l reads row 32rb + l % 32,
//   chunk 2kk + l / 32): 16 consecutive rows fall on 4 distinct 64-byte
//   windows (r % 4) and, within each, on 4 distinct chunks ((r >> 2) % 4).
// * Transposed reads (ds_read_b64_tr_b16, the A operand of dV, dK and dQ):
//   32 lanes read 4 consecutive rows of one block, 256 contiguous bytes.
// A lane's address for either pattern is one of two per-lane bases plus an
// immediate (block and row group).  Row r holds HBM row swap23(r) of its
// 32-row block of the step, rows GSTRIDE bytes apart.  It is filled by 1 KiB
// copy rounds (64 lanes x 16 bytes of consecutive LDS) shared by NW waves.
template <int R, int D, int GSTRIDE, int NW>
struct TrBuf {
  static constexpr int DB = D / 32;
  static constexpr int BLK = R * 64;                  // bytes of one 32-dim block
  static constexpr int BYTES = DB * BLK;
  static constexpr int ROUNDS = BYTES / 1024;
  static constexpr int PER_WAVE = (ROUNDS + NW - 1) / NW;
  static_assert(R % 32 == 0 && BYTES % 1024 == 0, "32-row blocks, whole copy rounds");
  // round i of wave w fills LDS block w + NW*i; past the last block it fills
  // block w again with the same bytes (every wave issues PER_WAVE rounds)
  static __device__ __forceinline__ int block(int wave, int i) {
    const int q = wave + NW * i;
    return q < ROUNDS ? q : wave;
  }
  static __device__ __forceinline__ void offsets(uint32_t (&off)[PER_WAVE], int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int u = block(wave, i) * 64 + lane;   // 16-byte unit of the buffer
      const int b = u / (R * 4), r = (u / 4) % R;
      const int c = (u & 3) ^ ((r >> 2) & 3);
      off[i] = (uint32_t)(((r & ~31) | swap23(r & 31)) * GSTRIDE + (4 * b + c) * 16);
    }
  }
  static __device__ __forceinline__ void copy(__amdgpu_buffer_rsrc_t rs, uint32_t so,
                                              unsigned char* lds, const uint32_t (&off)[PER_WAVE],
                                              int wave) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + block(wave, i) * 1024), 16,
                                               off[i], so, 0, 0);
  }
  // Row reads: row 32rb + l % 32, chunk 2kk + l / 32.  base[p] is the lane's
  // offset for even (p = 0) and odd (p = 1) kk; block kk / 2 and row block rb
  // are the immediate.
  static __device__ __forceinline__ void row_bases(int (&base)[2], int lane) {
    const int r = lane & 31, y = (lane >> 5) ^ ((r >> 2) & 3);
    base[0] = r * 64 + 16 * y;
    base[1] = r * 64 + 16 * (y ^ 2);
  }
  static __device__ __forceinline__ bf16x8 row(const unsigned char* buf, const int (&base)[2],
                                               int kk, int rb = 0) {
    return *reinterpret_cast<const bf16x8*>(buf + (kk / 2) * BLK + rb * 32 * 64 + base[kk & 1]);
  }
  // Transposed reads: the A operand of a product over the step's rows, 32
  // dims of block db as rows (d = 32db + l%32), 16 step rows (16t + 8(l/32)
  // + 0..7, t < R/16) as the contraction.  Within each group of 16 lanes
  // ds_read_b64_tr_b16 gives lane i, as element e, the (i%4)-th of the four
  // values at the address lane 4e + i/4 supplies; lane 4e+x of group G
  // therefore supplies row 16t + 4(G/2) + e (+8 for the second read) -- step
  // rows 16t + 8(G/2) + e (+4) in swap23 order -- at dims 32db +
  // 16(G%2) + 4x .. +3: chunk 2(G%2) + x/2 of the block, bytes 8(x%2) on.
  // base[s] is the lane's offset for the first (s = 0) and second read.
  static __device__ __forceinline__ void tr_bases(int (&base)[2], int lane) {
    const int G = lane >> 4, j = lane & 15;
    const int c = 2 * (G & 1) + ((j & 3) >> 1);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int r = 4 * (G >> 1) + (j >> 2) + 8 * s;   // row within a 16-row group
      base[s] = r * 64 + 16 * (c ^ ((r >> 2) & 3)) + 8 * (j & 1);
    }
  }
  static __device__ __forceinline__ bf16x8 tr(const unsigned char* buf, const int (&base)[2],
                                              int db, int t) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const unsigned char* p = buf + db * BLK + t * 16 * 64;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + base[0]));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + base[1]));
    typedef short v8s __attribute__((ext_vector_type(8)));
    const v8s both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, both);
  }
};

// ---------------------------------------------------------------- dQ
// One workgroup per query tile, wave w owning queries 32w..32w+31 (Q and dO
// rows in registers).  Per 64-key step of every kept key tile:
// S^T = K Q^T (seeded with the step's mask rows), dP^T = V dO^T - D
// (seeded with -D), dS^T = P^T dP^T, dQ^T += K^T dS^T, the A operand K^T
// read transposed out of the staged K rows.  K and V rows of a step are
// staged in two buffers: step s+1 is copied while step s computes.
template <int D, int S>
__global__ __launch_bounds__(2 * S, 2) void attn_bwd_dq_kernel(
    DevLayout L, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, const __bf16* __restrict__ d_o,
    const float* __restrict__ lse2, const float* __restrict__ delta,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int32_t cap,
    float scale_log2, float sm_scale, __bf16* __restrict__ dq) {
  constexpr int NW = S / 32, SK = 64, SPT = S / SK, KS = D / 16, DB = D / 32, TILE = S * D * 2;
  using KR = TrBuf<SK, D, D * 2, NW>;                 // K or V rows of a step
  __shared__ __attribute__((aligned(1024))) unsigned char k0[KR::BYTES], v0[KR::BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char k1[KR::BYTES], v1[KR::BYTES];
  __shared__ BiasTable<SPT, 9> btab;

  const int64_t g = xcd_remap(blockIdx.x, gridDim.x);
  const int h = head_of_tile(L, g);
  const int64_t head_base = L.tile_off[h];
  const int n_h = (int)(L.tile_off[h + 1] - head_base);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hf = lane >> 5;
  const int64_t qrow = g * S + wave * 32 + n;

  bf16x8 qr[KS], dor[KS];
  load_q_regs<D>(qr, q + qrow * D, hf);
  load_q_regs<D>(dor, d_o + qrow * D, hf);
  const float l2 = lse2[qrow], dl = delta[qrow];

  cint32* rp = (cint32*)row_ptr;
  cint32* cp = (cint32*)col_idx;
  // the row, clamped to the CSR's entries [0, cap)
  const int beg = min(max(rp[g], 0), cap), end = max(beg, min(rp[g + 1], cap));
  const int N = (end - beg) * SPT;
  const auto krs = make_rsrc(reinterpret_cast<const unsigned char*>(k) + head_base * TILE,
                             (int64_t)n_h * TILE);
  const auto vrs = make_rsrc(reinterpret_cast<const unsigned char*>(v) + head_base * TILE,
                             (int64_t)n_h * TILE);
  uint32_t ro[KR::PER_WAVE];
  KR::offsets(ro, wave, lane);
  int rb[2], tb[2];
  KR::row_bases(rb, lane);
  KR::tr_bases(tb, lane);
  build_bias_table<SPT, 9>(btab, L, h, tid, 2 * S);

  // key tile of step s: an entry outside [0, n_h) is a tile whose keys are
  // all masked (cut 8), read from tile 0
  auto tile_of = [&](int s, int& cut) {
    const int c = cp[beg + s / SPT];
    const bool ok = c >= 0 && c < n_h;
    cut = ok ? cut_of(tile_extent(L, h, ok ? c : 0)) : 8;
    return ok ? c : 0;
  };
  // copies of step s; returns its mask cut
  auto stage = [&](int s, unsigned char* kd, unsigned char* vd) {
    int cut;
    const int c = tile_of(s, cut);
    const uint32_t so = (uint32_t)(c * TILE + (s % SPT) * SK * D * 2);
    KR::copy(krs, so, kd, ro, wave);
    KR::copy(vrs, so, vd, ro, wave);
    return cut;
  };

  f32x16 dqa[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqa[db] = f32x16{};

  int cut_next = 0;   // mask cut of the step staged last
  auto step = [&](int s, const unsigned char* ks, const unsigned char* vs, unsigned char* kn,
                  unsigned char* vn) {
    // step s landed in every wave and every wave is past step s-1, whose
    // buffers the copies of step s+1 overwrite.  The wait is the builtin, so
    // that the compiler knows no copy is in flight after it (it would
    // otherwise wait for the next step's copies before this step's reads);
    // the barrier is a bare s_barrier that no memory access crosses.
    __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
    asm volatile("s_barrier" ::: "memory");
    const int cut = cut_next;
    if (s + 1 < N) cut_next = stage(s + 1, kn, vn);
    // S^T starts from the step's mask rows, dP^T from -D (so dS = P dP)
    f32x16 st[2], dpt[2];
    load_bias(st, &btab.v[cut][s % SPT][0][hf][0]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dpt[0][i] = -dl;
      dpt[1][i] = -dl;
    }
    // Products laid out by hand in slots of one MFMA each, with the LDS read
    // of a later slot's operand; the compiler may not move work across
    // slots.  S^T and dP^T alternate (row reads LA1 slots ahead); the first
    // K^T operands are read while P and dS are computed, then the dQ^T
    // products (transposed reads LA2 slots ahead).
    constexpr int LA1 = 2, N1 = 4 * KS, LA2 = 3, N2 = 4 * DB;
    auto op1 = [&](int i) { return KR::row((i & 1) ? vs : ks, rb, i >> 2, (i >> 1) & 1); };
    auto op2 = [&](int i) { return KR::tr(ks, tb, i % DB, i / DB); };
    bf16x8 o1[LA1 + 1], o2[LA2 + 1];
    static_for<0, LA1>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      o1[i] = op1(i);
    });
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, N1>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int kk = i >> 2, b = (i >> 1) & 1;
      if constexpr (i + LA1 < N1) o1[(i + LA1) % (LA1 + 1)] = op1(i + LA1);
      if constexpr (i & 1) dpt[b] = mfma32(o1[i % (LA1 + 1)], dor[kk], dpt[b]);
      else st[b] = mfma32(o1[i % (LA1 + 1)], qr[kk], st[b]);
      __builtin_amdgcn_sched_barrier(0);
    });
    static_for<0, LA2>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      o2[i] = op2(i);
    });
    // element i of block b is key 32b + 16(i/8) + 8hf + i%8 of the step
    bf16x8 ds[4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = exp2_(fmaf(st[b][i], scale_log2, -l2));
        ds[2 * b + i / 8][i % 8] = (__bf16)(p * dpt[b][i]);
      }
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, N2>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i + LA2 < N2) o2[(i + LA2) % (LA2 + 1)] = op2(i + LA2);
      dqa[i % DB] = mfma32(o2[i % (LA2 + 1)], ds[i / DB], dqa[i % DB]);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  if (N > 0) cut_next = stage(0, k0, v0);
  int s = 0;
  for (; s + 1 < N; s += 2) {
    step(s, k0, v0, k1, v1);
    step(s + 1, k1, v1, k0, v0);
  }
  if (s < N) step(s, k0, v0, k1, v1);

  const TileExtent e = tile_extent(L, h, (int)(g - head_base));
  const int64_t row = slot_row(L, e, h, wave * 32 + n);
  if (row >= 0) {
    __bf16* out = dq + row * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 w;
#pragma unroll
        for (int b = 0; b < 4; ++b) w[b] = (__bf16)(dqa[db][4 * a + b] * sm_scale);
        *reinterpret_cast<bf16x4*>(out + db * 32 + 8 * a + 4 * hf) = w;
      }
  }
}

// ---------------------------------------------------------------- dK, dV
// One workgroup per key tile, wave w owning keys 32w..32w+31 (their K and V
// rows in registers).  Per 32-query step of every query tile that keeps the
// key tile:  S = Q K^T (seeded with -lse/sm_scale), dP = dO V^T (seeded with
// -D), P = exp2(sm_scale log2e S), dS = P dP, dV^T += dO^T P, dK^T += Q^T dS.
// The C layout of S (lane = key, 8 consecutive queries per half) is the B
// operand layout of the products over queries, so P and dS feed them as they
// are; their A operands are the step's dO and Q rows read transposed from
// LDS.  Only Q and dO rows are staged (18 KiB a step), four steps deep:
// step s+3 is copied while step s computes.
template <int D, int S>
__global__ __launch_bounds__(2 * S, 2) void attn_bwd_dkv_kernel(
    DevLayout L, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, const __bf16* __restrict__ d_o,
    const float* __restrict__ seed_s, const float* __restrict__ seed_dp,
    const int32_t* __restrict__ colt_ptr, const int32_t* __restrict__ rowt,
    const int32_t* __restrict__ order, int32_t cap, float scale_log2, float sm_scale,
    __bf16* __restrict__ dk, __bf16* __restrict__ dv) {
  constexpr int NW = S / 32, SQ = 32, SPQ = S / SQ, KS = D / 16, DB = D / 32, TILE = S * D * 2;
  constexpr int NB = 4;                                 // steps in flight
  using QR = TrBuf<SQ, D, D * 2, NW>;                 // Q or dO rows of a step, swap23 order
  // per step buffer: Q rows, dO rows, then the 32 + 32 seeds of S and dP
  constexpr int SEEDS = 2 * QR::BYTES, BUF = SEEDS + 256;
  __shared__ __attribute__((aligned(1024))) unsigned char b0[BUF], b1[BUF], b2[BUF], b3[BUF];
  auto buf = [&](auto par) -> unsigned char* {
    constexpr int P = decltype(par)::value;
    return P == 0 ? b0 : P == 1 ? b1 : P == 2 ? b2 : b3;
  };

  const int64_t g = ((cint32*)order)[blockIdx.x];   // key tile, longest first
  const int h = head_of_tile(L, g);
  const int64_t head_base = L.tile_off[h];
  const int n_h = (int)(L.tile_off[h + 1] - head_base);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hf = lane >> 5;
  const int64_t krow = g * S + wave * 32 + n;

  bf16x8 kr[KS], vr[KS];
  load_q_regs<D>(kr, k + krow * D, hf);
  load_q_regs<D>(vr, v + krow * D, hf);

  cint32* cpt = (cint32*)colt_ptr;
  cint32* rt = (cint32*)rowt;
  const int a0 = min(cpt[g], cap), a1 = max(a0, min(cpt[g + 1], cap));
  const int N = (a1 - a0) * SPQ;
  auto rs = [&](const __bf16* base) {
    return make_rsrc(reinterpret_cast<const unsigned char*>(base) + head_base * TILE,
                     (int64_t)n_h * TILE);
  };
  const auto qrs = rs(q), dors = rs(d_o);
  const auto ssrs = make_rsrc(seed_s + head_base * S, (int64_t)n_h * S * 4);
  const auto sdrs = make_rsrc(seed_dp + head_base * S, (int64_t)n_h * S * 4);
  uint32_t ro[QR::PER_WAVE];
  QR::offsets(ro, wave, lane);
  int rb[2], tb[2];
  QR::row_bases(rb, lane);
  QR::tr_bases(tb, lane);

  // copies of step s into buffer PAR.  Every wave issues the same number of
  // copies (each also copies the 256 seed bytes: identical bytes to the same
  // place), so one vmcnt value counts a step's copies in every wave.
  constexpr int CPS = 2 * QR::PER_WAVE + 2;             // copy instructions per step and wave
  auto stage = [&](int s, auto par) {
    unsigned char* bb = buf(par);
    const int i = min(max(rt[a0 + s / SPQ], 0), n_h - 1);   // head-local query tile
    const int qs = s % SPQ;
    const uint32_t rof = (uint32_t)(i * TILE + qs * SQ * D * 2);
    QR::copy(qrs, rof, bb, ro, wave);
    QR::copy(dors, rof, bb + QR::BYTES, ro, wave);
    // the 32 seeds of S, then those of dP: lanes 0-7, 16 bytes each (the
    // descriptor, the LDS place and the step offset are uniform)
    const uint32_t so = (uint32_t)((i * S + qs * SQ) * 4);
    if (lane < 8) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ssrs, (lds_void*)(bb + SEEDS), 16, lane * 16, so,
                                               0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sdrs, (lds_void*)(bb + SEEDS + 128), 16, lane * 16,
                                               so, 0, 0);
    }
  };

  f32x16 dka[DB], dva[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dka[db] = f32x16{};
    dva[db] = f32x16{};
  }

  auto step = [&](int s, auto par) {
    constexpr int PAR = decltype(par)::value;
    const unsigned char* qb = buf(par);
    const unsigned char* dob = qb + QR::BYTES;
    const float* ssb = reinterpret_cast<const float*>(qb + SEEDS);
    const float* sdb = ssb + SQ;
    // step s's copies landed: the copies of the (up to two) later steps
    // already issued may stay in flight; the barrier makes every wave's
    // copies visible and every wave past its reads of step s-1, whose buffer
    // the next copies overwrite
    // (a bare s_barrier: a fenced barrier would also drain those later copies)
    if (s + 2 < N)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(2 * CPS) : "memory");
    else if (s + 1 < N)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(CPS) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (s + 3 < N) stage(s + 3, std::integral_constant<int, (PAR + 3) % NB>{});
    // element x is query 16(x/8) + 8hf + x%8 of the step: S and dP start from
    // their seeds, two runs of 8 consecutive values each
    f32x16 sa, dpa;
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int q0 = 16 * (v4 / 2) + 8 * hf + 4 * (v4 % 2);
      const f32x4 x = *reinterpret_cast<const f32x4*>(ssb + q0);
      const f32x4 y = *reinterpret_cast<const f32x4*>(sdb + q0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sa[4 * v4 + e] = x[e];
        dpa[4 * v4 + e] = y[e];
      }
    }
    // The products are laid out by hand in slots of one MFMA each, with the
    // LDS read of a later slot's operand; the compiler may not move work
    // across slots.  S and dP alternate (operand reads LA1 slots ahead); the
    // first dV/dK operands are read while P and dS are computed, then dV
    // and dK alternate (reads LA2 slots ahead).
    constexpr int LA1 = 2, N1 = 2 * KS, LA2 = 3, N2 = 4 * DB;
    auto op1 = [&](int i) { return QR::row((i & 1) ? dob : qb, rb, i >> 1); };
    auto op2 = [&](int i) { return QR::tr((i & 1) ? qb : dob, tb, (i >> 1) % DB, i / (2 * DB)); };
    bf16x8 o1[LA1 + 1], o2[LA2 + 1];
    static_for<0, LA1>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      o1[i] = op1(i);
    });
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, N1>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i + LA1 < N1) o1[(i + LA1) % (LA1 + 1)] = op1(i + LA1);
      if constexpr (i & 1) dpa = mfma32(o1[i % (LA1 + 1)], vr[i >> 1], dpa);
      else sa = mfma32(o1[i % (LA1 + 1)], kr[i >> 1], sa);
      __builtin_amdgcn_sched_barrier(0);
    });
    static_for<0, LA2>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      o2[i] = op2(i);
    });
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const float p = exp2_(sa[x] * scale_log2);
      pb[x / 8][x % 8] = (__bf16)p;
      dsb[x / 8][x % 8] = (__bf16)(p * dpa[x]);
    }
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, N2>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int db = (i >> 1) % DB, t = i / (2 * DB);
      if constexpr (i + LA2 < N2) o2[(i + LA2) % (LA2 + 1)] = op2(i + LA2);
      if constexpr (i & 1) dka[db] = mfma32(o2[i % (LA2 + 1)], dsb[t], dka[db]);
      else dva[db] = mfma32(o2[i % (LA2 + 1)], pb[t], dva[db]);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  using C3 = std::integral_constant<int, 3>;
  if (N > 0) stage(0, C0{});
  if (N > 1) stage(1, C1{});
  if (N > 2) stage(2, C2{});
  int s = 0;
  for (; s + 3 < N; s += 4) {
    step(s, C0{});
    step(s + 1, C1{});
    step(s + 2, C2{});
    step(s + 3, C3{});
  }
  if (s < N) step(s, C0{});
  if (s + 1 < N) step(s + 1, C1{});
  if (s + 2 < N) step(s + 2, C2{});

  const TileExtent e = tile_extent(L, h, (int)(g - head_base));
  const int64_t row = slot_row(L, e, h, wave * 32 + n);
  if (row >= 0) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 wk, wv;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          wk[b] = (__bf16)(dka[db][4 * a + b] * sm_scale);
          wv[b] = (__bf16)dva[db][4 * a + b];
        }
        *reinterpret_cast<bf16x4*>(dk + row * D + db * 32 + 8 * a + 4 * hf) = wk;
        *reinterpret_cast<bf16x4*>(dv + row * D + db * 32 + 8 * a + 4 * hf) = wv;
      }
  }
}

int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }

struct BwdWs {
  void *qp, *kp, *vp, *dop;
  float *lse2, *delta, *seed_s, *seed_dp;
  int32_t *cnt, *colt_ptr, *rowt, *order;
};

BwdWs carve(const DevLayout& L, int64_t nnz, void* base, int64_t* total) {
  BwdWs w;
  char* p = static_cast<char*>(base);
  int64_t o = 0;
  auto take = [&](int64_t bytes) -> void* {
    void* q = p ? p + o : nullptr;
    o += round256(bytes);
    return q;
  };
  const int64_t tiles = L.tile_off[L.heads];
  const int64_t tb = tiles * L.S * L.d * 2;
  w.qp = take(tb); w.kp = take(tb); w.vp = take(tb); w.dop = take(tb);
  w.lse2 = static_cast<float*>(take(tiles * L.S * 4));
  w.delta = static_cast<float*>(take(tiles * L.S * 4));
  w.seed_s = static_cast<float*>(take(tiles * L.S * 4));
  w.seed_dp = static_cast<float*>(take(tiles * L.S * 4));
  w.cnt = static_cast<int32_t*>(take(tiles * 4));
  w.colt_ptr = static_cast<int32_t*>(take((tiles + 1) * 4));
  w.rowt = static_cast<int32_t*>(take(nnz * 4 + 4));
  w.order = static_cast<int32_t*>(take(tiles * 4));
  *total = o;
  return w;
}

template <int D, int S>
void launch_products(const DevLayout& L, const BwdWs& w, const int32_t* row_ptr,
                     const int32_t* col_idx, int32_t cap, float sm_scale, void* dq, void* dk,
                     void* dv, hipStream_t s) {
  const unsigned G = (unsigned)L.tile_off[L.heads];
  const float sl2 = sm_scale * kLog2e;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, S>), dim3(G), dim3(2 * S), 0, s, L,
                     (const __bf16*)w.qp, (const __bf16*)w.kp, (const __bf16*)w.vp,
                     (const __bf16*)w.dop, w.lse2, w.delta, row_ptr, col_idx, cap, sl2,
                     sm_scale, (__bf16*)dq);
  hipLaunchKernelGGL((attn_bwd_dkv_kernel<D, S>), dim3(G), dim3(2 * S), 0, s, L,
                     (const __bf16*)w.qp, (const __bf16*)w.kp, (const __bf16*)w.vp,
                     (const __bf16*)w.dop, w.seed_s, w.seed_dp, w.colt_ptr, w.rowt, w.order, cap,
                     sl2, sm_scale, (__bf16*)dk, (__bf16*)dv);
}

}  // namespace

int64_t attn_bwd_workspace_bytes(const DevLayout& L, int64_t nnz) {
  int64_t total = 0;
  carve(L, nnz, nullptr, &total);
  return total;
}

int launch_sparse_attn_bwd(const DevLayout& L, const void* q, const void* k, const void* v,
                           const void* o, const void* d_o, const float* lse,
                           const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                           float sm_scale, void* workspace, void* dq, void* dk, void* dv,
                           bool qk_tiles, hipStream_t s) {
  const int64_t tiles = L.tile_off[L.heads];
  if (tiles == 0) return VEDA_OK;
  int64_t total = 0;
  BwdWs w = carve(L, nnz, workspace, &total);
  if (qk_tiles) {   // Q and K come in tile order (the forward's gathers)
    w.qp = const_cast<void*>(q);
    w.kp = const_cast<void*>(k);
  } else {
    if (launch_permute(L, VEDA_BF16, VEDA_FWD, q, w.qp, s) != VEDA_OK ||
        launch_permute(L, VEDA_BF16, VEDA_FWD, k, w.kp, s) != VEDA_OK)
      return VEDA_ERR_LAUNCH;
  }
  if (launch_permute(L, VEDA_BF16, VEDA_FWD, v, w.vp, s) != VEDA_OK) return VEDA_ERR_LAUNCH;
  hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)tiles), dim3(kThreads), 0, s, L,
                     (const __bf16*)o, (const __bf16*)d_o, lse, sm_scale, w.delta, w.lse2,
                     w.seed_s, w.seed_dp, (__bf16*)w.dop, w.cnt);
  hipLaunchKernelGGL(csrt_count_kernel, dim3((unsigned)tiles), dim3(64), 0, s, L, row_ptr,
                     col_idx, (int32_t)nnz, w.cnt);
  hipLaunchKernelGGL(csrt_scan_kernel, dim3(1), dim3(kThreads), 0, s, tiles, w.cnt, w.colt_ptr,
                     w.order);
  hipLaunchKernelGGL(csrt_fill_kernel, dim3((unsigned)tiles), dim3(kThreads), 0, s, L, row_ptr,
                     col_idx, w.colt_ptr, (int32_t)nnz, w.rowt);
  if (L.d == 128)
    launch_products<128, 128>(L, w, row_ptr, col_idx, (int32_t)nnz, sm_scale, dq, dk, dv, s);
  else
    launch_products<64, 64>(L, w, row_ptr, col_idx, (int32_t)nnz, sm_scale, dq, dk, dv, s);
  return launch_status();
}

}  // namespace veda
