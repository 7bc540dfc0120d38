// Max-pooled attention map, the distillation target (Veda §2.1 target
// construction: the full attention matrix max-pooled over query-tile x
// key-tile blocks; Veda §2.3: built in two passes over a random subset of
// query tiles).
//
// One workgroup per subset query tile; the wave layout and MFMA products are
// those of the attention kernel (queries in registers, key tiles staged
// through two LDS buffers one tile ahead).  A single loop runs 2*n_h steps over
// the head's key tiles:
//   pass 1 (steps 0 .. n_h-1):   online row maximum and sum of exp2 -> lse;
//   pass 2 (steps n_h .. 2n_h-1): per key tile, each query's largest logit,
//     p = exp2(max - lse), max over the tile's real queries (inside the wave
//     by lane exchanges, across waves through LDS) -> map[s][j].
// Pass 2 takes one exp per (query, key tile) rather than per logit.
#include "attn_common.hpp"

namespace veda {
namespace {

using namespace attn;

template <int D, int S>
__global__ __launch_bounds__(2 * S, 1) void oracle_map_kernel(
    DevLayout L, const __bf16* __restrict__ q, const __bf16* __restrict__ k, float scale_log2,
    const int32_t* __restrict__ q_tiles, float* __restrict__ lse_out, float* __restrict__ map) {
  using C = Cfg<D, S>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2][C::KBYTES];
  __shared__ float red[2][C::NW];

  const int64_t sidx = xcd_remap(blockIdx.x, gridDim.x);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, hf = lane >> 5;
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
  const bool q_real = eq.slot_real(wave * 32 + n);

  bf16x8 qr[C::KS];
  load_q_regs<D>(qr, q + (g * S + wave * 32 + n) * D, hf);

  Chunk kreg[C::CPT];
  const Chunk* kc = reinterpret_cast<const Chunk*>(k) + head_base * (int64_t)C::CHUNKS;
  load_tile_regs<C::CPT, C::NT>(kreg, kc, tid);
  store_k_lds<D, S>(smem[0], kreg, tid);
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.f, lse2 = 0.f;
  const int steps = 2 * n_h;
  int stage = 0;
  for (int it = 0; it < steps; ++it) {
    const int j = it < n_h ? it : it - n_h;
    const bool more = it + 1 < steps;
    if (more) {
      const int jn = (it + 1) % n_h;
      load_tile_regs<C::CPT, C::NT>(kreg, kc + (int64_t)jn * C::CHUNKS, tid);
    }
    if (it == n_h) {
      // end of pass 1: combine the half-lanes' (max, sum) -> base-2 lse
      const float mo = xor32(m_run), lo = xor32(l_run);
      const float mt = fmaxf(m_run, mo);
      const float lt = l_run * __builtin_amdgcn_exp2f(m_run - mt) + lo * __builtin_amdgcn_exp2f(mo - mt);
      lse2 = mt + __log2f(lt);
      if (hf == 0) lse_out[sidx * S + wave * 32 + n] = lse2 * 0.69314718055994531f;
    }
    if (it > n_h && tid == 0) {   // flush the previous key tile's block maximum
      float v = red[(it - 1) & 1][0];
#pragma unroll
      for (int w = 1; w < C::NW; ++w) v = fmaxf(v, red[(it - 1) & 1][w]);
      mrow[j - 1] = v;
    }

    f32x16 sacc[C::KB];
    qk_tile<D, S>(sacc, smem[stage], qr, n, hf);
    const TileExtent e = tile_extent(L, h, j);
    if (!e.full()) mask_keys<C::KB>(sacc, e, hf);
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);

    if (it < n_h) {
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m_run, mx * scale_log2);
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          psum += __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], scale_log2, -m_new));
      l_run = fmaf(l_run, __builtin_amdgcn_exp2f(m_run - m_new), psum);
      m_run = m_new;
    } else {
      mx = fmaxf(mx, xor32(mx));
      float pr = q_real ? __builtin_amdgcn_exp2f(fmaf(mx, scale_log2, -lse2)) : 0.f;
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) pr = fmaxf(pr, __shfl_xor(pr, o, 64));
      if (lane == 0) red[it & 1][wave] = pr;
    }

    if (more) store_k_lds<D, S>(smem[stage ^ 1], kreg, tid);
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
