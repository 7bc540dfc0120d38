// Tile-skipping block-sparse attention forward (Veda §2.3: the kernel visits
// only each query tile's kept, non-contiguous key/value tiles and hides their
// fetch behind dense matrix math).
//
// One workgroup per (head, query tile), S/32 waves: wave w owns queries
// 32w..32w+31, held in registers as MFMA operands, and every key of each kept
// tile.  The workgroup walks its CSR row.  A kept key tile K [S][D] and value
// tile V^T [D][S] are contiguous blocks in HBM that the waves copy straight
// into LDS (global_load_lds, no register staging).  K and V^T have one LDS
// buffer each, so two workgroups fit on a CU and the two waves sharing a SIMD
// come from different, unsynchronised workgroups: one's softmax runs while the
// other's matrix products do.  Within a workgroup the copy of K(t+1) is issued
// as soon as every wave has finished S^T = K(t) Q^T, and that of V(t+1) once
// O^T += V(t)^T P^T is done, so each fetch overlaps half a tile of compute.
//
// Per tile and wave: S^T = K Q^T (MFMA 32x32x16 bf16, f32 accumulate), the
// padding keys of boundary tiles -> -inf, online softmax in base 2 with
// sm_scale*log2(e) folded into one FMA, P rounded to bf16, O^T += V^T P^T.
// The running maximum is raised only when a new logit exceeds it by more than
// 2^8, so the accumulator is rescaled rarely; the result is the same softmax
// (numerator and denominator share one reference).
//
// Workgroups are ordered XCD-aware and head-major, so the query tiles running
// together on one XCD are spatial neighbours whose kept key tiles overlap in
// that XCD's L2.
#include <type_traits>

#include "attn_common.hpp"

namespace veda {
namespace {

using namespace attn;

constexpr float kLazyRescale = 8.0f;   // log2 of the largest unnormalised p

// LDS: K and V^T buffers of S*D*2 bytes each (2 x 32 KiB at S = d = 128) plus
// the mask table.  Per kept tile t:
//   [K(t) ready]  S^T = K Q^T           barrier -> DMA K(t+1) into the K buffer
//   softmax; [V(t) ready]  O^T += V^T P^T  barrier -> DMA V(t+1) into the V buffer
template <int D, int S>
__global__ __launch_bounds__(2 * S, 2) void sparse_attn_fwd_kernel(
    DevLayout L, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ vt, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, float scale_log2, __bf16* __restrict__ o,
    float* __restrict__ lse) {
  constexpr int NW = S / 32;
  constexpr int KB = S / 32, KS = D / 16, DB = D / 32, PS = S / 16;
  constexpr int CPR_K = D / 8, CPR_V = S / 8;
  constexpr int TILE = S * D * 2, DMA_PW = TILE / 1024 / NW;
  static_assert(TILE % (1024 * NW) == 0, "tile must split into whole DMA rounds");
  // separate objects, so that reads of one are not ordered after copies into the other
  __shared__ __attribute__((aligned(1024))) unsigned char kl[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vl[TILE];
  __shared__ MaskTable<S> mtab;

  const int64_t g = xcd_remap(blockIdx.x, gridDim.x);
  const int h = head_of_tile(L, g);
  const int n_h = (int)(L.tile_off[h + 1] - L.tile_off[h]);
  const int64_t head_base = L.tile_off[h];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hf = lane >> 5;

  bf16x8 qr[KS];
  const int64_t qrow = g * S + wave * 32 + n;
  load_q_regs<D>(qr, q + qrow * D, hf);

  int beg = row_ptr[g], end = row_ptr[g + 1];
  if (end < beg) end = beg;
  auto next_valid = [&](int p) {
    while (p < end) {
      const int j = col_idx[p];
      if (j >= 0 && j < n_h) break;
      ++p;
    }
    return p;
  };
  const unsigned char* kg = reinterpret_cast<const unsigned char*>(k) + head_base * TILE;
  const unsigned char* vg = reinterpret_cast<const unsigned char*>(vt) + head_base * TILE;
  uint32_t koff[DMA_PW], voff[DMA_PW];
  dma_offsets<CPR_K, DMA_PW, true>(koff, wave, lane);
  dma_offsets<CPR_V, DMA_PW, false>(voff, wave, lane);

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};

  int p = next_valid(beg);
  int cur_j = p < end ? col_idx[p] : 0;
  if (p < end) {
    dma_tile<DMA_PW>(kg + (int64_t)cur_j * TILE, kl, koff, wave);
    dma_tile<DMA_PW>(vg + (int64_t)cur_j * TILE, vl, voff, wave);
  }
  build_mask_table<S>(mtab, L, h, tid);
  wait_all();
  __syncthreads();

  static_assert(DMA_PW == 8 || DMA_PW == 4, "barrier wait counts below assume 8 or 4 copies");
  while (p < end) {
    const int pn = next_valid(p + 1);
    const int nxt_j = pn < end ? col_idx[pn] : 0;
    f32x16 sacc[KB];
    qk_blocks<D, KB>(sacc, kl, 0, qr, n, hf);
    wait_all();                                        // own share of V(t) landed
    __syncthreads();                                   // K buffer free, V(t) visible
    if (pn < end) dma_tile<DMA_PW>(kg + (int64_t)nxt_j * TILE, kl, koff, wave);

    const int cut = cut_of(tile_extent(L, h, cur_j));
    if (cut != 0) mask_keys<KB, S>(sacc, mtab, cut, 0, hf);
    float mx = max_of<KB>(sacc);
    mx = fmaxf(mx, xor32(mx));
    const float m_cand = fmaxf(m_run, mx * scale_log2);
    if (__any(m_cand > m_run + kLazyRescale)) {
      const float alpha = m_cand == -INFINITY ? 1.f : exp2_(m_run - m_cand);
      m_run = m_cand;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
    const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
    bf16x8 pb[PS];
    float psum = 0.f;
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = exp2_(fmaf(sacc[b][i], scale_log2, neg_m));
        psum += pv;
        pb[2 * b + (i >> 3)][i & 7] = (__bf16)pv;
      }
    l_run += psum;
#pragma unroll
    for (int t = 0; t < PS; ++t)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        oacc[db] = mfma32(lds_chunk<CPR_V>(vl, db * 32 + n, 2 * t + hf), pb[t], oacc[db]);
    // V buffer free: this wave's LDS reads are done (the K(t+1) copy may still fly)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (pn < end) dma_tile<DMA_PW>(vg + (int64_t)nxt_j * TILE, vl, voff, wave);
    // own share of K(t+1) landed (V(t+1) may still be in flight), then barrier
    if constexpr (DMA_PW == 8)
      asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    p = pn;
    cur_j = nxt_j;
  }

  const float l_tot = l_run + xor32(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  __bf16* orow = o + qrow * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      bf16x4 wv;
#pragma unroll
      for (int b = 0; b < 4; ++b) wv[b] = (__bf16)(oacc[db][4 * a + b] * inv);
      *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * a + 4 * hf) = wv;
    }
  if (lse != nullptr && hf == 0)
    lse[qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

int launch_sparse_attn(const DevLayout& L, const void* q, const void* k, const void* vt,
                       const int32_t* row_ptr, const int32_t* col_idx, float sm_scale, void* o,
                       float* lse, hipStream_t s) {
  const unsigned G = (unsigned)L.tile_off[L.heads];
  if (G == 0) return VEDA_OK;
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  if (L.d == 128) {
    hipLaunchKernelGGL((sparse_attn_fwd_kernel<128, 128>), dim3(G), dim3(256), 0, s,
                       L, (const __bf16*)q, (const __bf16*)k, (const __bf16*)vt, row_ptr, col_idx,
                       scale_log2, (__bf16*)o, lse);
  } else {
    hipLaunchKernelGGL((sparse_attn_fwd_kernel<64, 64>), dim3(G), dim3(128), 0, s, L,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)vt, row_ptr, col_idx,
                       scale_log2, (__bf16*)o, lse);
  }
  return launch_status();
}

}  // namespace veda
