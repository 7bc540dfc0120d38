// Building blocks shared by the tile-skipping attention forward and the
// max-pooled map kernels: bf16 matrix-core (MFMA) tile products on gfx950.
//
// Orientation.  Logits are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16: key rows (from LDS) are the A operand and a
// wave's 32 queries (held in registers for the whole kernel) the B operand.
// In the 32x32 accumulator layout lane l holds column l % 32 -- one query --
// and 16 rows, so every softmax row statistic is a reduction inside the lane
// plus one exchange with lane l ^ 32.  The attention output is accumulated
// transposed too, O^T = V^T P^T: V^T rows (from LDS) are the A operand and
// P^T, the probabilities already sitting in the lane that owns the query, the
// B operand, with no data movement.
//
// Key order inside a 32-key block.  Accumulator element i of lane l is row
// m = 8(i/4) + 4(l/32) + i%4.  Key rows are placed in LDS with bits 2 and 3
// of the key index swapped, so A-operand row m is key swap23(m) and element
// i of lane l is key 16(i/8) + 8(l/32) + i%8: each lane holds 8 consecutive
// keys per half block, which are exactly the 8 contraction indices that lane
// supplies to the P V product.  Both operands of each product take their
// contraction indices by the same rule, so the products are exact.
//
// LDS staging.  Tiles are copied HBM -> LDS with buffer_load ... lds (no
// register staging): one instruction moves 64 lanes x 16 bytes into 1 KiB of
// consecutive LDS, and each lane picks the HBM chunk that must land at its
// LDS position.  Rows are padded by 16 bytes (see StepBuf).
//
// Padding key slots of boundary tiles are masked with a row of 0 / -inf per
// key slot (see BiasTable).  Only boundary tiles need it: a full tile's
// products start from an inline zero accumulator and read no mask row, so
// the LDS carries operands alone on most steps.  The map seeds the
// accumulator of a boundary tile with its mask row (no vector instruction);
// the attention kernel adds it to the logits of a boundary step.
#pragma once

#include <type_traits>

#include "veda_internal.hpp"

namespace veda {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
// Read-only, wave-uniform data through the constant address space, so that
// it is fetched with scalar loads (which never wait on the LDS copies).
typedef __attribute__((address_space(4))) const int32_t cint32;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int swap23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// f(integral_constant<int, I>) for I = B .. E-1, expanded at compile time
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Wait for this wave's outstanding memory operations (including LDS copies).
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }

// The wave's 32 query rows as MFMA B operands: qr[s] holds dims
// 16s + 8(l/32) .. +7 of query row (l % 32).
template <int D>
__device__ __forceinline__ void load_q_regs(bf16x8 (&qr)[D / 16], const __bf16* __restrict__ qrow,
                                            int hf) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) qr[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * hf);
}

// Maximum / sum of a value over lanes l and l ^ 32 (v_permlane32_swap).
__device__ __forceinline__ float swap32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// exp2 whose argument is finite or -inf; (-inf) - (-inf) never reaches it.
__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

// Global -> local XCD-aware workgroup order: hardware places workgroup b on
// XCD b % 8; give each XCD a contiguous range of logical work items so that
// neighbouring query tiles (which keep overlapping key tiles) share an L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t G) {
  constexpr int X = 8;
  const int64_t xcd = b % X, per = G / X, rem = G % X;
  return xcd * per + (xcd < rem ? xcd : rem) + b / X;
}

// Lockstep XCD order over the tiles of a layer.  Every head's tiles are cut
// into 8 contiguous chunks, chunk x going to XCD x (the hardware places
// workgroup b on XCD b % 8); XCD x walks chunk x of head 0, then chunk x of
// head 1, and so on.  All XCDs therefore work inside the same head at the
// same time, so the key/value tiles in flight are those of about one head
// (which the memory-side cache holds), while each XCD's query tiles are a
// contiguous, spatially compact run of that head.  Returns the global tile
// of workgroup b, or -1 past the end of its XCD's run (the grid is 8 times
// the longest run; see lockstep_grid).
__device__ __forceinline__ int64_t lockstep_tile(const DevLayout& L, int64_t b) {
  const int x = (int)(b & 7);
  int64_t i = b >> 3;
  for (int h = 0; h < L.heads; ++h) {
    const int64_t n = L.tile_off[h + 1] - L.tile_off[h];
    const int64_t lo = n * x / 8, len = n * (x + 1) / 8 - lo;
    if (i < len) return L.tile_off[h] + lo + i;
    i -= len;
  }
  return -1;
}

// A step buffer in LDS: R rows of CPR 16-byte chunks, each row followed by
// one 16-byte pad, so that 16 lanes reading one chunk column of 16
// consecutive rows hit 16 distinct bank groups (row stride (CPR+1)*16 bytes
// is an odd number of 16-byte units) and a lane's reads along a row are one
// base address plus immediate offsets.  Row r holds HBM row (SWAP ? swap23 :
// id)(r), rows GSTRIDE bytes apart.  It is filled by 1 KiB copy rounds (64
// lanes x 16 bytes of consecutive LDS) shared by NW waves; a lane whose 16
// bytes fall on a pad re-reads chunk 0 of the source.
template <int R, int CPR, bool SWAP, int GSTRIDE, int NW>
struct StepBuf {
  static constexpr int ROWB = (CPR + 1) * 16;
  static constexpr int ROUNDS = (R * (CPR + 1) + 63) / 64;
  static constexpr int BYTES = ROUNDS * 1024;
  static constexpr int PER_WAVE = (ROUNDS + NW - 1) / NW;
  // round i of wave w fills LDS block w + NW*i; past the last block it fills
  // block w again with the same bytes, so that every wave issues PER_WAVE
  // rounds with no branch
  static __device__ __forceinline__ int block(int wave, int i) {
    const int q = wave + NW * i;
    return q < ROUNDS ? q : wave;
  }
  // per-lane byte offsets of this lane's chunks, one per round of the wave
  static __device__ __forceinline__ void offsets(uint32_t (&off)[PER_WAVE], int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int u = block(wave, i) * 64 + lane;   // 16-byte unit of the buffer
      const int r = u / (CPR + 1), c = u % (CPR + 1);
      const int gr = SWAP ? ((r & ~31) | swap23(r & 31)) : r;
      off[i] = (c == CPR || r >= R) ? 0u : (uint32_t)(gr * GSTRIDE + c * 16);
    }
  }
  // issue round i of this wave: buffer `rs` at byte offset `so` (uniform)
  static __device__ __forceinline__ void round(int i, __amdgpu_buffer_rsrc_t rs, uint32_t so,
                                               unsigned char* lds, const uint32_t (&off)[PER_WAVE],
                                               int wave) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + block(wave, i) * 1024), 16,
                                             off[i], so, 0, 0);
  }
  static __device__ __forceinline__ void copy(__amdgpu_buffer_rsrc_t rs, uint32_t so,
                                              unsigned char* lds, const uint32_t (&off)[PER_WAVE],
                                              int wave) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) round(i, rs, so, lds, off, wave);
  }
  static __device__ __forceinline__ bf16x8 read(const unsigned char* buf, int r, int c) {
    return *reinterpret_cast<const bf16x8*>(buf + r * ROWB + c * 16);
  }
};

// Raw buffer resource over `bytes` bytes at `base` (range-checked loads).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Which of the 8 cuts tile e is (0 = whole tile): bit 2/1/0 set = the tile's
// t/h/w extent is the partial one at the far edge of the grid.
__device__ __forceinline__ int cut_of(const TileExtent& e) {
  return (e.lt < e.pt ? 4 : 0) | (e.lh < e.ph ? 2 : 0) | (e.lw < e.pw ? 1 : 0);
}

// Additive key mask of a 64-key step, as the initial value of the S^T
// accumulator: 0 for a real key slot, -inf for padding.  Entry
// [cut][half][b][hf] holds the 16 accumulator elements of 32-key block b of
// step `half` of a tile with that cut, for lanes of half hf (element i is
// key 16(i/8) + 8hf + i%8).  Built once per workgroup.
// NCUT = 9 adds cut 8: every slot masked (a tile that contributes nothing).
template <int SPT, int NCUT = 8>
struct BiasTable {
  f32x4 v[NCUT][SPT][2][2][4];
};

template <int SPT, int NCUT>
__device__ __forceinline__ void build_bias_table(BiasTable<SPT, NCUT>& bt, const DevLayout& L,
                                                 int h, int tid, int nthreads) {
  const int pt = L.shape[h][0], ph = L.shape[h][1], pw = L.shape[h][2];
  const int et = L.T - (L.grid[h][0] - 1) * pt;   // extent of the last tile along t
  const int eh = L.H - (L.grid[h][1] - 1) * ph;
  const int ew = L.W - (L.grid[h][2] - 1) * pw;
  float* flat = reinterpret_cast<float*>(&bt);
  constexpr int ENTRIES = NCUT * SPT * 2 * 2 * 16;
  const float rpw = small_rcp(pw), rph = small_rcp(ph);
  for (int x = tid; x < ENTRIES; x += nthreads) {
    const int i = x & 15, hf = (x >> 4) & 1, b = (x >> 5) & 1, half = (x >> 6) % SPT;
    const int cut = (x >> 6) / SPT;
    const int u = half * 64 + 32 * b + 16 * (i >> 3) + 8 * hf + (i & 7);   // slot in tile
    const int r = small_div(u, rpw), dw = u - r * pw;
    const int dt = small_div(r, rph), dh = r - dt * ph;
    const bool ok = cut < 8 && (!(cut & 4) || dt < et) && (!(cut & 2) || dh < eh) &&
                    (!(cut & 1) || dw < ew);
    flat[x] = ok ? 0.f : -INFINITY;
  }
}

// Seed a step's two S^T accumulators (32-key blocks) from mask rows bp.
__device__ __forceinline__ void load_bias(f32x16 (&acc)[2], const f32x4* bp) {
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 x = bp[b * 8 + c];   // [b][hf][c] with hf fixed: stride 2*4 per b
      acc[b][4 * c + 0] = x[0];
      acc[b][4 * c + 1] = x[1];
      acc[b][4 * c + 2] = x[2];
      acc[b][4 * c + 3] = x[3];
    }
}

// Add the mask rows bp to a step's two S^T accumulators (logits computed
// from a zero start).
__device__ __forceinline__ void add_bias(f32x16 (&acc)[2], const f32x4* bp) {
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 x = bp[b * 8 + c];
      acc[b][4 * c + 0] += x[0];
      acc[b][4 * c + 1] += x[1];
      acc[b][4 * c + 2] += x[2];
      acc[b][4 * c + 3] += x[3];
    }
}

}  // namespace attn
}  // namespace veda
