// Building blocks shared by the tile-skipping attention forward and the
// max-pooled map kernels: bf16 matrix-core (MFMA) tile products on gfx950.
//
// Orientation.  Logits are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16: key rows (from LDS) are the A operand and a
// wave's 32 queries (held in registers for the whole kernel) the B operand.
// In the 32x32 accumulator layout lane l holds column l % 32 -- one query --
// and 16 rows, so every softmax row statistic is a reduction inside the lane
// plus one exchange with lane l ^ 32.  The output is accumulated transposed
// too, O^T = V^T P^T: V^T rows (from LDS) are the A operand and P^T, the
// probabilities already sitting in the lane that owns the query, the B
// operand, with no data movement.
//
// Key order inside a 32-key block.  Accumulator element i of lane l is row
// m = 8(i/4) + 4(l/32) + i%4.  Key rows are placed in LDS with bits 2 and 3
// of the key index swapped, so A-operand row m is key swap23(m) and element
// i of lane l is key 16(i/8) + 8(l/32) + i%8: each lane holds 8 consecutive
// keys per half block, which are exactly the 8 contraction indices that lane
// supplies to the P V product.  Both operands of each product take their
// contraction indices by the same rule, so the products are exact.
//
// Waves.  A workgroup owns one query tile of S queries with 2*S/32 waves:
// wave w takes query block w % (S/32) and key half w / (S/32) of every key
// tile, so two waves share each SIMD and one's softmax can run while the
// other's matrix products do.  The two halves are merged at the end.
//
// LDS staging.  Tiles are copied global -> LDS with global_load_lds_dwordx4
// (no register staging): one instruction moves 64 lanes x 16 bytes into 1 KiB
// of consecutive LDS, and each lane picks the global 16-byte chunk that must
// land at its LDS position.  Rows are stored unpadded with their 16-byte
// chunks XOR-swizzled by the row index, so the lanes that read one chunk
// column of consecutive rows hit distinct banks.
#pragma once

#include "veda_internal.hpp"

namespace veda {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const unsigned char gbyte;

struct Chunk { uint32_t x, y, z, w; };

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int swap23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Key index (within its 32-key block) of accumulator element i, lane half hf.
__device__ __forceinline__ int key_in_block(int i, int hf) {
  return 16 * (i >> 3) + 8 * hf + (i & 7);
}

template <int D, int S>
struct Cfg {
  static constexpr int QB = S / 32;            // 32-query blocks per tile
  static constexpr int KH = 2;                 // key halves (waves per query block)
  static constexpr int NW = QB * KH;           // waves per workgroup
  static constexpr int NT = NW * 64;           // threads per workgroup
  static constexpr int KPW = S / KH;           // keys per wave per tile
  static constexpr int KBW = KPW / 32;         // 32-key blocks per wave
  static constexpr int KS = D / 16;            // MFMA k-steps over head_dim
  static constexpr int DB = D / 32;            // 32-row blocks of O^T
  static constexpr int PSW = KPW / 16;         // MFMA k-steps over a wave's keys
  static constexpr int CPR_K = D / 8;          // 16-byte chunks per key row
  static constexpr int CPR_V = S / 8;          // 16-byte chunks per V^T row
  static constexpr int TILE_BYTES = S * D * 2; // one bf16 tile
  static constexpr int CHUNKS = TILE_BYTES / 16;
  static constexpr int DMA_PER_WAVE = TILE_BYTES / 1024 / NW;
  static_assert(TILE_BYTES % (1024 * NW) == 0, "tile must split into whole DMA rounds");
  static_assert(KBW >= 1, "a wave needs at least one key block");
};

// Byte offset of logical 16-byte chunk c of row r in a swizzled LDS tile.
template <int CPR>
__device__ __forceinline__ int lds_off(int r, int c) {
  return (r * CPR + (c ^ (r & (CPR - 1)))) * 16;
}

template <int CPR>
__device__ __forceinline__ bf16x8 lds_chunk(const unsigned char* tile, int r, int c) {
  return *reinterpret_cast<const bf16x8*>(tile + lds_off<CPR>(r, c));
}

// Per-lane byte offsets (within a tile in HBM) of the 16-byte chunks this
// lane copies into LDS, one per DMA round of the wave.  LDS block q of the
// tile receives, at lane l, logical chunk (p ^ (r & (CPR-1))) of row r, where
// lc = 64q + l = r*CPR + p; SWAP places key rows at LDS row swap23(row)
// within 32-row blocks.
template <int CPR, int PER_WAVE, bool SWAP>
__device__ __forceinline__ void dma_offsets(uint32_t (&off)[PER_WAVE], int wave, int lane) {
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int q = wave * PER_WAVE + i;
    const int lc = q * 64 + lane;
    const int r = lc / CPR, p = lc % CPR;
    const int c = p ^ (r & (CPR - 1));
    const int gr = SWAP ? ((r & ~31) | swap23(r & 31)) : r;
    off[i] = (uint32_t)((gr * CPR + c) * 16);
  }
}

// Issue this wave's share of the global -> LDS copy of one tile: `g` is the
// tile's address in HBM and `wave` the wave index, both uniform across the
// wave (scalar base + 32-bit lane offset; scalar LDS destination).
template <int PER_WAVE>
__device__ __forceinline__ void dma_tile(const unsigned char* g, unsigned char* lds,
                                         const uint32_t (&off)[PER_WAVE], int wave) {
  gbyte* gg = (gbyte*)g;
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i)
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) const void*)(gg + off[i]),
                                     (lds_void*)(lds + (wave * PER_WAVE + i) * 1024), 16, 0, 0);
}

// Wait for this wave's outstanding memory operations (including LDS DMA).
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }

// The wave's 32 query rows as MFMA B operands: qr[s] holds dims
// 16s + 8(l/32) .. +7 of query row (l % 32).
template <int D>
__device__ __forceinline__ void load_q_regs(bf16x8 (&qr)[D / 16], const __bf16* __restrict__ qrow,
                                            int hf) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) qr[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * hf);
}

// S^T of NKB key blocks starting at block kb0: acc[b] = K[block] Q^T.  The
// blocks are independent accumulation chains, interleaved, and the operands
// of step s+1 are read from LDS while the products of step s run.
template <int D, int NKB>
__device__ __forceinline__ void qk_blocks(f32x16 (&acc)[NKB], const unsigned char* ktile, int kb0,
                                          const bf16x8 (&qr)[D / 16], int n, int hf) {
  constexpr int CPR = D / 8;
  constexpr int KS = D / 16;
#pragma unroll
  for (int b = 0; b < NKB; ++b) acc[b] = f32x16{};
  bf16x8 a[2][NKB];
#pragma unroll
  for (int b = 0; b < NKB; ++b) a[0][b] = lds_chunk<CPR>(ktile, (kb0 + b) * 32 + n, hf);
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (s + 1 < KS) {
#pragma unroll
      for (int b = 0; b < NKB; ++b)
        a[(s + 1) & 1][b] = lds_chunk<CPR>(ktile, (kb0 + b) * 32 + n, 2 * (s + 1) + hf);
    }
#pragma unroll
    for (int b = 0; b < NKB; ++b) acc[b] = mfma32(a[s & 1][b], qr[s], acc[b]);
  }
}

// Validity of the S slots of a tile, as S/32 32-bit words (bit u of word w is
// slot 32w + u), for each of the 8 ways a tile can be cut by the grid:
// combo bit 2/1/0 set = the tile's t/h/w extent is the partial one at the
// far edge of the grid.  Built once per workgroup by S threads.
template <int S>
struct MaskTable {
  uint32_t w[8][S / 32];
};

template <int S>
__device__ __forceinline__ void build_mask_table(MaskTable<S>& mt, const DevLayout& L, int h,
                                                 int tid) {
  const int pt = L.shape[h][0], ph = L.shape[h][1], pw = L.shape[h][2];
  const int et = L.T - (L.grid[h][0] - 1) * pt;   // extent of the last tile along t
  const int eh = L.H - (L.grid[h][1] - 1) * ph;
  const int ew = L.W - (L.grid[h][2] - 1) * pw;
  if (tid < S) {
    const int dw = tid % pw, r = tid / pw, dh = r % ph, dt = r / ph;
    const int lane = tid & 63;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const bool ok = (!(c & 4) || dt < et) && (!(c & 2) || dh < eh) && (!(c & 1) || dw < ew);
      const uint64_t bal = __ballot(ok);
      if (lane == 0) {
        mt.w[c][(tid >> 5)] = (uint32_t)bal;
        if (S >= 64) mt.w[c][(tid >> 5) + 1] = (uint32_t)(bal >> 32);
      }
    }
  }
}

// Which of the 8 cuts tile e is (0 = whole tile).
__device__ __forceinline__ int cut_of(const TileExtent& e) {
  return (e.lt < e.pt ? 4 : 0) | (e.lh < e.ph ? 2 : 0) | (e.lw < e.pw ? 1 : 0);
}

// Padding keys -> -inf for key blocks kb0 .. kb0+NKB-1, given the tile's
// validity words.  Lane half hf holds keys 8hf..8hf+7 and 16+8hf..16+8hf+7 of
// each block, i.e. bytes hf and 2+hf of the block's word.  Per element: a
// sign-extended one-bit extract (all ones or all zeros) selects the logit or
// -inf bitwise.
template <int NKB, int S>
__device__ __forceinline__ void mask_keys(f32x16 (&acc)[NKB], const MaskTable<S>& mt, int cut,
                                          int kb0, int hf) {
#pragma unroll
  for (int b = 0; b < NKB; ++b) {
    const int wbits = (int)(mt.w[cut][kb0 + b] >> (8 * hf));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int keep = __builtin_amdgcn_sbfe(wbits, 16 * (i >> 3) + (i & 7), 1);
      acc[b][i] = __int_as_float((__float_as_int(acc[b][i]) & keep) | (0xff800000 & ~keep));
    }
  }
}

// Maximum of the wave's logits in this lane, as a tree of 3-input maxima.
template <int NKB>
__device__ __forceinline__ float max_of(const f32x16 (&acc)[NKB]) {
  float m[NKB];
#pragma unroll
  for (int b = 0; b < NKB; ++b) {
    float x = fmaxf(fmaxf(acc[b][0], acc[b][1]), acc[b][2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) x = fmaxf(fmaxf(x, acc[b][i]), acc[b][i + 1]);
    m[b] = fmaxf(x, acc[b][15]);
  }
  float r = m[0];
#pragma unroll
  for (int b = 1; b < NKB; ++b) r = fmaxf(r, m[b]);
  return r;
}

__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, 64); }

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

}  // namespace attn
}  // namespace veda
