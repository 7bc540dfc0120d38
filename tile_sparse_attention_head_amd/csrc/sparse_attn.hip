// Tile-skipping block-sparse attention forward (Veda §2.3: the kernel visits
// only each query tile's kept, non-contiguous key/value tiles and hides their
// fetch behind dense matrix math).
//
// One workgroup per (head, query tile): S/32 waves, each owning 32 queries
// whose bf16 rows stay in registers.  The workgroup walks its CSR row; each
// kept key tile (K [S][D]) and its value tile (V^T [D][S]) are contiguous
// 32 KiB blocks in HBM, fetched by all lanes as 16-byte chunks into registers
// one tile ahead, and written into one of two LDS stages, so the fetch of tile
// t+1 overlaps the matrix products of tile t and one barrier per tile
// suffices.  Per tile: S^T = K Q^T (MFMA), padding keys of boundary tiles set
// to -inf, online softmax in base 2 with sm_scale*log2(e) folded into one FMA,
// P rounded to bf16, O^T += V^T P^T (MFMA), f32 accumulation throughout.
//
// Workgroups are ordered XCD-aware and head-major, so the query tiles running
// together on one XCD are spatial neighbours whose kept key tiles overlap in
// that XCD's L2.
#include "attn_common.hpp"

namespace veda {
namespace {

using namespace attn;

template <int D, int S>
__global__ __launch_bounds__(2 * S, 1) void sparse_attn_fwd_kernel(
    DevLayout L, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ vt, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, float scale_log2, __bf16* __restrict__ o,
    float* __restrict__ lse) {
  using C = Cfg<D, S>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2][C::KBYTES + C::VBYTES];

  const int64_t g = xcd_remap(blockIdx.x, gridDim.x);      // global query tile
  const int h = head_of_tile(L, g);
  const int n_h = (int)(L.tile_off[h + 1] - L.tile_off[h]);
  const int64_t head_base = L.tile_off[h];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, hf = lane >> 5;

  bf16x8 qr[C::KS];
  const int64_t qrow = g * S + wave * 32 + n;
  load_q_regs<D>(qr, q + qrow * D, hf);

  int beg = row_ptr[g], end = row_ptr[g + 1];
  if (end < beg) end = beg;
  // next CSR position >= p holding a valid tile index (uniform scalar loop)
  auto next_valid = [&](int p) {
    while (p < end) {
      const int j = col_idx[p];
      if (j >= 0 && j < n_h) break;
      ++p;
    }
    return p;
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};

  Chunk kreg[C::CPT], vreg[C::CPT];
  int p = next_valid(beg);
  int cur_j = p < end ? col_idx[p] : -1;
  if (p < end) {
    const int64_t tb = (head_base + cur_j) * (int64_t)C::CHUNKS;
    load_tile_regs<C::CPT, C::NT>(kreg, reinterpret_cast<const Chunk*>(k) + tb, tid);
    load_tile_regs<C::CPT, C::NT>(vreg, reinterpret_cast<const Chunk*>(vt) + tb, tid);
    store_k_lds<D, S>(smem[0], kreg, tid);
    store_vt_lds<D, S>(smem[0] + C::KBYTES, vreg, tid);
  }
  __syncthreads();

  int stage = 0;
  while (p < end) {
    const int pn = next_valid(p + 1);
    const int nxt_j = pn < end ? col_idx[pn] : -1;
    if (pn < end) {   // fetch the next kept tile while this one is computed
      const int64_t tb = (head_base + nxt_j) * (int64_t)C::CHUNKS;
      load_tile_regs<C::CPT, C::NT>(kreg, reinterpret_cast<const Chunk*>(k) + tb, tid);
      load_tile_regs<C::CPT, C::NT>(vreg, reinterpret_cast<const Chunk*>(vt) + tb, tid);
    }
    const unsigned char* klds = smem[stage];
    const unsigned char* vlds = smem[stage] + C::KBYTES;

    f32x16 sacc[C::KB];
    qk_tile<D, S>(sacc, klds, qr, n, hf);
    const TileExtent e = tile_extent(L, h, cur_j);
    if (!e.full()) mask_keys<C::KB>(sacc, e, hf);

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;

    bf16x8 pb[C::PS];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], scale_log2, -m_new));
        psum += pv;
        pb[2 * kb + (i >> 3)][i & 7] = (__bf16)pv;
      }
    l_run = fmaf(l_run, alpha, psum);
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;

#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const unsigned char* rowp = vlds + (db * 32 + n) * C::VROW + hf * 16;
#pragma unroll
      for (int t = 0; t < C::PS; ++t) {
        const bf16x8 vv = *reinterpret_cast<const bf16x8*>(rowp + t * 32);
        oacc[db] = mfma32(vv, pb[t], oacc[db]);
      }
    }

    if (pn < end) {
      store_k_lds<D, S>(smem[stage ^ 1], kreg, tid);
      store_vt_lds<D, S>(smem[stage ^ 1] + C::KBYTES, vreg, tid);
    }
    __syncthreads();
    stage ^= 1;
    p = pn;
    cur_j = nxt_j;
  }

  // Epilogue: combine the two half-lanes' partial sums, normalise, store.
  const float l_tot = l_run + xor32(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  __bf16* orow = o + qrow * D;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      bf16x4 w;
#pragma unroll
      for (int b = 0; b < 4; ++b) w[b] = (__bf16)(oacc[db][4 * a + b] * inv);
      *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * a + 4 * hf) = w;
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
    using C = Cfg<128, 128>;
    hipLaunchKernelGGL((sparse_attn_fwd_kernel<128, 128>), dim3(G), dim3(C::NT), 0, s, L,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)vt, row_ptr, col_idx,
                       scale_log2, (__bf16*)o, lse);
  } else {
    using C = Cfg<64, 64>;
    hipLaunchKernelGGL((sparse_attn_fwd_kernel<64, 64>), dim3(G), dim3(C::NT), 0, s, L,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)vt, row_ptr, col_idx,
                       scale_log2, (__bf16*)o, lse);
  }
  return launch_status();
}

}  // namespace veda
