// Building blocks shared by the tile-skipping attention forward and the
// max-pooled map kernels: bf16 matrix-core (MFMA) tile products on gfx950.
//
// Orientation.  Each wave owns 32 query rows.  Logits are computed transposed,
// S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: the key tile (from LDS) is the
// A operand and the wave's queries (held in registers for the whole kernel)
// are the B operand.  In the 32x32 accumulator layout lane l holds column
// l % 32 -- one query -- and 16 rows, so every row statistic of softmax is a
// reduction inside the lane plus one exchange with lane l ^ 32.  The output
// is accumulated transposed too, O^T = V^T P^T: V^T (from LDS) is the A
// operand and P^T, the probabilities already sitting in the lane that owns
// the query, is the B operand without any data movement.
//
// Key order inside a 32-key block.  Accumulator element i of lane l is row
// m = 8(i/4) + 4(l/32) + i%4.  The key tile is written to LDS with bits 2 and
// 3 of the key index swapped, so row m of the A operand is key swap23(m) and
// element i of lane l is key 16(i/8) + 8(l/32) + i%8: each lane then holds 8
// consecutive keys per half block, exactly the 8 contraction indices the B
// operand of the P V product wants from it (lane half l/32 supplies k-indices
// 8(l/32) .. 8(l/32)+7).  Both operands of each product take their k-indices
// by the same rule, so the products are exact contractions.
#pragma once

#include "veda_internal.hpp"

namespace veda {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct Chunk { uint32_t x, y, z, w; };

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int swap23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Key index (within the tile) of accumulator element i of lane half `hf`
// in key block kb.
__device__ __forceinline__ int key_of(int kb, int i, int hf) {
  return kb * 32 + 16 * (i >> 3) + 8 * hf + (i & 7);
}

template <int D, int S>
struct Cfg {
  static constexpr int NW = S / 32;                // waves per workgroup
  static constexpr int NT = NW * 64;               // threads per workgroup
  static constexpr int KB = S / 32;                // 32-key blocks per tile
  static constexpr int KS = D / 16;                // MFMA k-steps over head_dim
  static constexpr int DB = D / 32;                // 32-row blocks of O^T
  static constexpr int PS = S / 16;                // MFMA k-steps over keys
  static constexpr int KROW = D * 2 + 16;          // LDS bytes per key row (padded)
  static constexpr int VROW = S * 2 + 16;          // LDS bytes per V^T row (padded)
  static constexpr int KBYTES = S * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int CHUNKS = S * D * 2 / 16;    // 16-byte chunks per K (or V) tile
  static constexpr int CPT = CHUNKS / NT;          // chunks per thread
  static_assert(CHUNKS % NT == 0, "tile chunks must split evenly");
};

// Global -> registers: chunk c = tid + q*NT of a contiguous 16-byte-chunked tile.
template <int CPT, int NT>
__device__ __forceinline__ void load_tile_regs(Chunk (&r)[CPT], const Chunk* __restrict__ src,
                                               int tid) {
#pragma unroll
  for (int q = 0; q < CPT; ++q) r[q] = src[tid + q * NT];
}

// Registers -> LDS for a K tile ([S][D] row-major in memory): key rows go to
// LDS row swap23(key) of their 32-key block, padded row pitch KROW.
template <int D, int S>
__device__ __forceinline__ void store_k_lds(unsigned char* lds, const Chunk (&r)[D / 16],
                                            int tid) {
  using C = Cfg<D, S>;
  constexpr int CPR = D / 8;
#pragma unroll
  for (int q = 0; q < C::CPT; ++q) {
    const int c = tid + q * C::NT;
    const int key = c / CPR, col = c % CPR;
    const int row = (key & ~31) | swap23(key & 31);
    *reinterpret_cast<Chunk*>(lds + row * C::KROW + col * 16) = r[q];
  }
}

// Registers -> LDS for a V^T tile ([D][S] in memory), padded pitch VROW.
template <int D, int S>
__device__ __forceinline__ void store_vt_lds(unsigned char* lds, const Chunk (&r)[D / 16],
                                             int tid) {
  using C = Cfg<D, S>;
  constexpr int CPR = S / 8;
#pragma unroll
  for (int q = 0; q < C::CPT; ++q) {
    const int c = tid + q * C::NT;
    const int dd = c / CPR, col = c % CPR;
    *reinterpret_cast<Chunk*>(lds + dd * C::VROW + col * 16) = r[q];
  }
}

// The wave's 32 query rows as MFMA B operands: qr[s] holds dims
// 16s + 8(l/32) .. +7 of query row (l % 32).
template <int D>
__device__ __forceinline__ void load_q_regs(bf16x8 (&qr)[D / 16], const __bf16* __restrict__ qrow,
                                            int hf) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) qr[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * hf);
}

// S^T for one tile: acc[kb] = K[kb block] Q^T (raw dot products, f32).
template <int D, int S>
__device__ __forceinline__ void qk_tile(f32x16 (&acc)[S / 32], const unsigned char* klds,
                                        const bf16x8 (&qr)[D / 16], int n, int hf) {
  using C = Cfg<D, S>;
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
    f32x16 a = {};
    const unsigned char* rowp = klds + (kb * 32 + n) * C::KROW + hf * 16;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const bf16x8 kv = *reinterpret_cast<const bf16x8*>(rowp + s * 32);
      a = mfma32(kv, qr[s], a);
    }
    acc[kb] = a;
  }
}

// Padding keys of a boundary tile -> -inf.
template <int KB>
__device__ __forceinline__ void mask_keys(f32x16 (&acc)[KB], const TileExtent& e, int hf) {
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (!e.slot_real(key_of(kb, i, hf))) acc[kb][i] = -INFINITY;
}

__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, 64); }

// Global -> local XCD-aware workgroup order: hardware places workgroup b on
// XCD b % 8; give each XCD a contiguous range of logical work items so that
// neighbouring query tiles (which keep overlapping key tiles) share an L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t G) {
  constexpr int X = 8;
  const int64_t xcd = b % X, per = G / X, rem = G % X;
  return xcd * per + (xcd < rem ? xcd : rem) + b / X;
}

}  // namespace attn
}  // namespace veda
