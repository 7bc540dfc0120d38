// Tile-skipping block-sparse attention forward (Veda §2.3: the kernel visits
// only each query tile's kept, non-contiguous key/value tiles and hides their
// fetch behind dense matrix math).
//
// One workgroup per (head, query tile), 2*S/32 waves (see attn_common.hpp):
// wave (qb, kh) owns queries 32qb..32qb+31, held in registers, and key half kh
// of every kept key tile.  The workgroup walks its CSR row; each kept key tile
// K [S][D] and value tile V^T [D][S] are contiguous blocks in HBM that the
// waves copy straight into one of two LDS stages while the other stage is
// being consumed, so the fetch of tile t+1 overlaps the products of tile t
// and one barrier per tile suffices.  Per tile and wave: S^T = K Q^T (MFMA),
// padding keys of boundary tiles -> -inf, online softmax in base 2 with
// sm_scale*log2(e) folded into one FMA, P rounded to bf16, O^T += V^T P^T
// (MFMA), f32 accumulation.  The running maximum is raised only when a new
// logit exceeds it by more than 2^8, so the accumulator is rescaled rarely;
// the result is the same softmax (every term shares one reference).  At the
// end the two key halves of each query block are merged through LDS.
//
// Workgroups are ordered XCD-aware and head-major, so the query tiles running
// together on one XCD are spatial neighbours whose kept key tiles overlap in
// that XCD's L2.
#include "attn_common.hpp"

namespace veda {
namespace {

using namespace attn;

constexpr float kLazyRescale = 8.0f;   // log2 of the largest unnormalised p

template <int D, int S>
__global__ __launch_bounds__(4 * S, S / 64) void sparse_attn_fwd_kernel(
    DevLayout L, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ vt, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, float scale_log2, __bf16* __restrict__ o,
    float* __restrict__ lse) {
  using C = Cfg<D, S>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2][2 * C::TILE_BYTES];
  __shared__ MaskTable<S> mtab;

  const int64_t g = xcd_remap(blockIdx.x, gridDim.x);      // global query tile
  const int h = head_of_tile(L, g);
  const int n_h = (int)(L.tile_off[h + 1] - L.tile_off[h]);
  const int64_t head_base = L.tile_off[h];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, hf = lane >> 5;
  const int qb = wave % C::QB, kh = wave / C::QB;

  bf16x8 qr[C::KS];
  const int64_t qrow = g * S + qb * 32 + n;
  load_q_regs<D>(qr, q + qrow * D, hf);

  int beg = row_ptr[g], end = row_ptr[g + 1];
  if (end < beg) end = beg;
  auto next_valid = [&](int p) {           // next CSR entry naming a tile of this head
    while (p < end) {
      const int j = col_idx[p];
      if (j >= 0 && j < n_h) break;
      ++p;
    }
    return p;
  };
  const Chunk* kc = reinterpret_cast<const Chunk*>(k) + head_base * (int64_t)C::CHUNKS;
  const Chunk* vc = reinterpret_cast<const Chunk*>(vt) + head_base * (int64_t)C::CHUNKS;
  auto fetch = [&](int j, int st) {
    dma_tile<C::CPR_K, C::DMA_PER_WAVE, true>(kc + (int64_t)j * C::CHUNKS, smem[st], wave, lane);
    dma_tile<C::CPR_V, C::DMA_PER_WAVE, false>(vc + (int64_t)j * C::CHUNKS,
                                                smem[st] + C::TILE_BYTES, wave, lane);
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};

  int p = next_valid(beg);
  int cur_j = p < end ? col_idx[p] : -1;
  if (p < end) fetch(cur_j, 0);
  build_mask_table<S>(mtab, L, h, tid);
  wait_all();
  __syncthreads();

  int stage = 0;
  while (p < end) {
    const int pn = next_valid(p + 1);
    const int nxt_j = pn < end ? col_idx[pn] : -1;
    if (pn < end) fetch(nxt_j, stage ^ 1);       // lands while this tile is computed
    const unsigned char* ktile = smem[stage];
    const unsigned char* vtile = smem[stage] + C::TILE_BYTES;

    f32x16 sacc[C::KBW];
    qk_blocks<D, C::KBW>(sacc, ktile, kh * C::KBW, qr, n, hf);
    const int cut = cut_of(tile_extent(L, h, cur_j));
    if (cut != 0) mask_keys<C::KBW, S>(sacc, mtab, cut, kh * C::KBW, hf);

    float mx = max_of<C::KBW>(sacc);
    mx = fmaxf(mx, xor32(mx));
    const float m_cand = fmaxf(m_run, mx * scale_log2);
    if (__any(m_cand > m_run + kLazyRescale)) {
      const float alpha = m_cand == -INFINITY ? 1.f : exp2_(m_run - m_cand);
      m_run = m_cand;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
    }
    const float neg_m = m_run == -INFINITY ? 0.f : -m_run;

    bf16x8 pb[C::PSW];
    float psum = 0.f;
#pragma unroll
    for (int b = 0; b < C::KBW; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = exp2_(fmaf(sacc[b][i], scale_log2, neg_m));
        psum += pv;
        pb[2 * b + (i >> 3)][i & 7] = (__bf16)pv;
      }
    l_run += psum;

    {   // O^T += V^T P^T: DB independent chains, next operands read ahead
      constexpr int C0 = C::KPW / 8;
      bf16x8 va[2][C::DB];
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        va[0][db] = lds_chunk<C::CPR_V>(vtile, db * 32 + n, kh * C0 + hf);
#pragma unroll
      for (int t = 0; t < C::PSW; ++t) {
        if (t + 1 < C::PSW) {
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
            va[(t + 1) & 1][db] = lds_chunk<C::CPR_V>(vtile, db * 32 + n, kh * C0 + 2 * (t + 1) + hf);
        }
#pragma unroll
        for (int db = 0; db < C::DB; ++db) oacc[db] = mfma32(va[t & 1][db], pb[t], oacc[db]);
      }
    }

    wait_all();          // this wave's share of the next tile has landed
    __syncthreads();     // ... everyone's has, and nobody still reads this stage
    stage ^= 1;
    p = pn;
    cur_j = nxt_j;
  }

  // Merge the two key halves of each query block through LDS.
  constexpr int NX = C::DB * 16 + 2;                    // floats per lane exchanged
  float* xch = reinterpret_cast<float*>(&smem[0][0]) + qb * NX * 64;
  if (kh == 1) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) xch[(db * 16 + i) * 64 + lane] = oacc[db][i];
    xch[(NX - 2) * 64 + lane] = m_run;
    xch[(NX - 1) * 64 + lane] = l_run;
  }
  __syncthreads();
  if (kh != 0) return;
  const float m_b = xch[(NX - 2) * 64 + lane], l_b = xch[(NX - 1) * 64 + lane];
  const float mt = fmaxf(m_run, m_b);
  const float ca = m_run == -INFINITY ? 0.f : exp2_(m_run - mt);
  const float cb = m_b == -INFINITY ? 0.f : exp2_(m_b - mt);
  float l_part = l_run * ca + l_b * cb;
  const float l_tot = l_part + xor32(l_part);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  const float wa = ca * inv, wb = cb * inv;
  __bf16* orow = o + qrow * D;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      bf16x4 w;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int i = 4 * a + b;
        w[b] = (__bf16)(oacc[db][i] * wa + xch[(db * 16 + i) * 64 + lane] * wb);
      }
      *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * a + 4 * hf) = w;
    }
  if (lse != nullptr && hf == 0)
    lse[qrow] = l_tot > 0.f ? (mt + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

int launch_sparse_attn(const DevLayout& L, const void* q, const void* k, const void* vt,
                       const int32_t* row_ptr, const int32_t* col_idx, float sm_scale, void* o,
                       float* lse, hipStream_t s) {
  const unsigned G = (unsigned)L.tile_off[L.heads];
  if (G == 0) return VEDA_OK;
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  if (L.d == 128) {
    hipLaunchKernelGGL((sparse_attn_fwd_kernel<128, 128>), dim3(G), dim3(Cfg<128, 128>::NT), 0, s,
                       L, (const __bf16*)q, (const __bf16*)k, (const __bf16*)vt, row_ptr, col_idx,
                       scale_log2, (__bf16*)o, lse);
  } else {
    hipLaunchKernelGGL((sparse_attn_fwd_kernel<64, 64>), dim3(G), dim3(Cfg<64, 64>::NT), 0, s, L,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)vt, row_ptr, col_idx,
                       scale_log2, (__bf16*)o, lse);
  }
  return launch_status();
}

}  // namespace veda
