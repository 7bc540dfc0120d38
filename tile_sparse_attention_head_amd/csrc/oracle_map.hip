// Max-pooled attention map, the distillation target (Veda §2.1 target
// construction: the full attention matrix max-pooled over query-tile x
// key-tile blocks; Veda §2.3: built in two passes over a random subset of
// query tiles).
//
// One workgroup per subset query tile, 2*S/32 waves: wave (qb, kh) holds 32
// queries in registers and takes key half kh of every key tile; key tiles are
// copied straight into two LDS stages one tile ahead.  A
// single loop runs 2*n_h steps over the head's key tiles:
//   pass 1 (steps 0 .. n_h-1): online row maximum and sum of exp2 over the
//     wave's keys; the two key halves are combined through LDS -> lse;
//   pass 2 (steps n_h .. 2n_h-1): per key tile, each query's largest logit,
//     p = exp2(max - lse), then the maximum over the tile's real queries
//     (inside the wave by lane exchanges, across waves through LDS) -> map.
// Pass 2 takes one exp per (query, key tile) rather than one per logit.
#include "attn_common.hpp"

namespace veda {
namespace {

using namespace attn;

template <int D, int S>
__global__ __launch_bounds__(4 * S, S / 64) void oracle_map_kernel(
    DevLayout L, const __bf16* __restrict__ q, const __bf16* __restrict__ k, float scale_log2,
    const int32_t* __restrict__ q_tiles, float* __restrict__ lse_out, float* __restrict__ map) {
  using C = Cfg<D, S>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2][C::TILE_BYTES];
  __shared__ float ml[C::NW][2][64];
  __shared__ float red[2][C::NW];
  __shared__ MaskTable<S> mtab;

  const int64_t sidx = xcd_remap(blockIdx.x, gridDim.x);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, hf = lane >> 5;
  const int qb = wave % C::QB, kh = wave / C::QB;
  float* mrow = map + sidx * (int64_t)L.max_tiles;
  const int64_t g = q_tiles[sidx];
  if (g < 0 || g >= L.tile_off[L.heads]) {           // out-of-range entry: zero row
    for (int j = tid; j < L.max_tiles; j += C::NT) mrow[j] = 0.f;
    return;
  }
  const int h = head_of_tile(L, g);
  const int n_h = (int)(L.tile_off[h + 1] - L.tile_off[h]);
  const int64_t head_base = L.tile_off[h];
  const TileExtent eq = tile_extent(L, h, (int)(g - head_base));
  const bool q_real = eq.slot_real(qb * 32 + n);

  bf16x8 qr[C::KS];
  load_q_regs<D>(qr, q + (g * S + qb * 32 + n) * D, hf);

  const unsigned char* kg = reinterpret_cast<const unsigned char*>(k) + head_base * C::TILE_BYTES;
  uint32_t koff[C::DMA_PER_WAVE];
  dma_offsets<C::CPR_K, C::DMA_PER_WAVE, true>(koff, wave, lane);
  dma_tile<C::DMA_PER_WAVE>(kg, smem[0], koff, wave);
  build_mask_table<S>(mtab, L, h, tid);
  wait_all();
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.f, lse2 = 0.f;
  const int steps = 2 * n_h;
  int stage = 0;
  for (int it = 0; it < steps; ++it) {
    const int j = it < n_h ? it : it - n_h;
    if (it + 1 < steps)
      dma_tile<C::DMA_PER_WAVE>(kg + (int64_t)((it + 1) % n_h) * C::TILE_BYTES, smem[stage ^ 1],
                                koff, wave);
    if (it == n_h) {
      // end of pass 1: combine with the other key half -> base-2 lse per query
      const int partner = (kh ^ 1) * C::QB + qb;
      const float m_a = m_run, l_a = l_run + xor32(l_run);
      const float m_b = ml[partner][0][lane], l_b = ml[partner][1][lane];
      const float mt = fmaxf(m_a, m_b);
      const float lt = (m_a == -INFINITY ? 0.f : l_a * exp2_(m_a - mt)) +
                       (m_b == -INFINITY ? 0.f : l_b * exp2_(m_b - mt));
      lse2 = mt + __log2f(lt);
      if (kh == 0 && hf == 0) lse_out[sidx * S + qb * 32 + n] = lse2 * 0.69314718055994531f;
    }
    if (it > n_h && tid == 0) {   // publish the previous key tile's block maximum
      float v = red[(it - 1) & 1][0];
#pragma unroll
      for (int w = 1; w < C::NW; ++w) v = fmaxf(v, red[(it - 1) & 1][w]);
      mrow[j - 1] = v;
    }

    f32x16 sacc[C::KBW];
    qk_blocks<D, C::KBW>(sacc, smem[stage], kh * C::KBW, qr, n, hf);
    const int cut = cut_of(tile_extent(L, h, j));
    if (cut != 0) mask_keys<C::KBW, S>(sacc, mtab, cut, kh * C::KBW, hf);
    float mx = max_of<C::KBW>(sacc);
    mx = fmaxf(mx, xor32(mx));

    if (it < n_h) {
      const float m_new = fmaxf(m_run, mx * scale_log2);
      const float neg_m = m_new == -INFINITY ? 0.f : -m_new;
      float psum = 0.f;
#pragma unroll
      for (int b = 0; b < C::KBW; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) psum += exp2_(fmaf(sacc[b][i], scale_log2, neg_m));
      l_run = (m_run == -INFINITY ? 0.f : l_run * exp2_(m_run - m_new)) + psum;
      m_run = m_new;
      if (it == n_h - 1) {
        ml[wave][0][lane] = m_run;
        ml[wave][1][lane] = l_run + xor32(l_run);
      }
    } else {
      float pr = (q_real && mx != -INFINITY) ? exp2_(fmaf(mx, scale_log2, -lse2)) : 0.f;
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) pr = fmaxf(pr, __shfl_xor(pr, o, 64));
      if (lane == 0) red[it & 1][wave] = pr;
    }

    wait_all();
    __syncthreads();
    stage ^= 1;
  }
  if (tid == 0) {
    float v = red[(steps - 1) & 1][0];
#pragma unroll
    for (int w = 1; w < C::NW; ++w) v = fmaxf(v, red[(steps - 1) & 1][w]);
    mrow[n_h - 1] = v;
  }
  for (int j = n_h + tid; j < L.max_tiles; j += C::NT) mrow[j] = 0.f;
}

}  // namespace

int launch_oracle_map(const DevLayout& L, const void* q, const void* k, float sm_scale,
                      const int32_t* q_tiles, int n_sub, float* lse, float* map, hipStream_t s) {
  if (n_sub == 0) return VEDA_OK;
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  if (L.d == 128) {
    hipLaunchKernelGGL((oracle_map_kernel<128, 128>), dim3(n_sub), dim3(Cfg<128, 128>::NT), 0, s,
                       L, (const __bf16*)q, (const __bf16*)k, scale_log2, q_tiles, lse, map);
  } else {
    hipLaunchKernelGGL((oracle_map_kernel<64, 64>), dim3(n_sub), dim3(Cfg<64, 64>::NT), 0, s, L,
                       (const __bf16*)q, (const __bf16*)k, scale_log2, q_tiles, lse, map);
  }
  return launch_status();
}

}  // namespace veda
