// Max-pooled attention map, the distillation target (Veda §2.1 target
// construction: the full attention matrix max-pooled over query-tile x
// key-tile blocks; Veda §2.3: built in two passes over a random subset of
// query tiles).
//
// Because exp is monotone, the block maximum of the probabilities of query
// row r over key tile j is exp(sm_scale * max_{c in j} q_r.k_c - lse_r): it
// needs one logit maximum per (row, key tile), not the probabilities
// themselves.  So
//   pass 1 (map_stats_kernel) computes every logit once: per subset query
//     tile and chunk of the head's key tiles, the online row maximum and sum
//     of exp2 (a partial log-sum-exp) and, per key tile, each row's largest
//     logit, written to the workspace;
//   pass 2 (map_reduce_kernel) merges the chunk partials into lse and takes,
//     per key tile, the maximum over the tile's real rows of
//     exp2(largest logit - lse).
// Splitting the key tiles into chunks gives pass 1 enough workgroups to fill
// the chip whatever the subset size; the chunk count is chosen so that the
// last round of workgroups is not nearly empty, and the workgroups are
// ordered chunk-major so that those running together on one XCD share a
// key-tile range in L2.
//
// Pass 1 uses the tile products of the attention kernel: 4 waves of 32
// queries, K copied HBM -> LDS in 64-key steps two steps ahead, and per step
// one hand-laid block interleaving the MFMAs of QK(s+1) with the statistics
// of step s.  Padding keys are masked by seeding the accumulator with -inf.
#include "attn_common.hpp"

namespace veda {
namespace {

using namespace attn;

constexpr float kLazyRescale = 8.0f;   // log2 of the largest unnormalised term

template <int D, int S>
struct MapPipe {
  static constexpr int NW = S / 32;             // waves per workgroup
  static constexpr int SK = 64;                 // keys per step
  static constexpr int SPT = S / SK;            // steps per key tile
  static constexpr int KS = D / 16;             // MFMA k-steps over head_dim
  static constexpr int TILE = S * D * 2;
  static constexpr int KSTEP = SK * D * 2;      // HBM bytes of one K step
  using KBuf = StepBuf<SK, D / 8, true, D * 2, NW>;
};

// Pass 1.  Workgroup (subset entry `sub`, chunk `c`) covers key tiles
// [c n_h / chunks, (c+1) n_h / chunks) of the head.  Writes, per real or
// padding query slot q of the tile:
//   rowmax[sub][j][q] = sm_scale*log2(e) * max over real keys of tile j of q.k
//   ml[sub][c][q]     = (m, l) with sum over the chunk's real keys of
//                       exp2(sm_scale*log2(e) q.k) = l * 2^m  (m = -inf, l = 0
//                       for an empty chunk)
template <int D, int S>
__global__ __launch_bounds__(2 * S, 3) void map_stats_kernel(
    DevLayout L, const __bf16* __restrict__ q, const __bf16* __restrict__ k, float scale_log2,
    const int32_t* __restrict__ q_tiles, int chunks, float* __restrict__ rowmax,
    float2* __restrict__ ml) {
  using P = MapPipe<D, S>;
  using KB = typename P::KBuf;
  constexpr int SPT = P::SPT, KS = P::KS, TILE = P::TILE;
  __shared__ __attribute__((aligned(1024))) unsigned char k0[KB::BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char k1[KB::BYTES];
  __shared__ BiasTable<SPT> btab;

  // chunk-major: the workgroups running together on one XCD take the same
  // key-tile range for consecutive subset tiles, which share it in L2
  const int64_t b = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t n_sub = gridDim.x / chunks;
  const int sub = (int)(b % n_sub), c = (int)(b / n_sub);
  const int64_t g = ((cint32*)q_tiles)[sub];
  if (g < 0 || g >= L.tile_off[L.heads]) return;   // the reduce pass writes a zero row
  const int h = head_of_tile(L, g);
  const int n_h = (int)(L.tile_off[h + 1] - L.tile_off[h]);
  const int64_t head_base = L.tile_off[h];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hf = lane >> 5;
  const int j0 = (int)((int64_t)c * n_h / chunks), j1 = (int)((int64_t)(c + 1) * n_h / chunks);
  const int N = (j1 - j0) * SPT;   // steps

  bf16x8 qr[KS];
  const int qslot = wave * 32 + n;
  load_q_regs<D>(qr, q + (g * S + qslot) * D, hf);

  const auto krs = make_rsrc(reinterpret_cast<const unsigned char*>(k) + head_base * TILE,
                             (int64_t)n_h * TILE);
  uint32_t koff[KB::PER_WAVE];
  KB::offsets(koff, wave, lane);
  auto k_off = [&](int t) { return (uint32_t)((j0 + t / SPT) * TILE + (t % SPT) * P::KSTEP); };
  int qcut = 0;   // cut of the tile whose logits are computed next
  auto bias_of = [&](int t) -> const f32x4* {
    if (t % SPT == 0) qcut = cut_of(tile_extent(L, h, j0 + t / SPT));
    return &btab.v[qcut][t % SPT][0][hf][0];
  };

  float m_run = -INFINITY, l_run = 0.f, tmax = -INFINITY;
  float* rm_row = rowmax + ((int64_t)sub * L.max_tiles + j0) * S + qslot;
  f32x16 sA[2], sB[2];

  // One step s: statistics of step s and, in the same hand-laid block,
  // S^T(s+1) = K(s+1) Q^T, with the copy of K(s+2) spread over the slots.
  auto step = [&](auto has_qk, auto par, int s) {
    constexpr bool QK = decltype(has_qk)::value;
    constexpr int PAR = decltype(par)::value;
    f32x16 (&scur)[2] = PAR ? sB : sA;
    f32x16 (&snext)[2] = PAR ? sA : sB;
    const unsigned char* ksrc = PAR ? k0 : k1;
    unsigned char* kdst = PAR ? k1 : k0;

    if constexpr (QK) load_bias(snext, bias_of(s + 1));
    // K(s+2) over K(s); with no step s+2 the rounds re-copy K(s) into its
    // own, no longer read, slot
    const uint32_t kgs = s + 2 < N ? k_off(s + 2) : k_off(s);
    asm volatile("" :: "s"(kgs));

    constexpr int LA = 3;          // operand reads run LA slots ahead of their MFMA
    constexpr int NSLOT = D / 8;   // QK products of one step
    constexpr int RW = KB::PER_WAVE;
    auto operand = [&](int i) -> bf16x8 {
      return KB::read(ksrc, (i & 1) * 32 + n, 2 * (i >> 1) + hf);
    };
    bf16x8 opnd[LA + 1];
    if constexpr (QK) {
      static_for<0, LA>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        opnd[i % (LA + 1)] = operand(i);
      });
    }
    float pm[4], e[32];
    float mxs = 0.f, m_new = 0.f, neg_m = 0.f, psum0 = 0.f, psum1 = 0.f;
    bool raise = false;
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NSLOT>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      static_for<0, RW>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        if constexpr ((m * (NSLOT - 2)) / RW == i) KB::round(m, krs, kgs, kdst, koff, wave);
      });
      if constexpr (QK) {
        if constexpr (i + LA < NSLOT) opnd[(i + LA) % (LA + 1)] = operand(i + LA);
        snext[i & 1] = mfma32(opnd[i % (LA + 1)], qr[i >> 1], snext[i & 1]);
      }
      // statistics of step s: row maximum in slots 0..4, then the elements
      if constexpr (i < 4) {
        constexpr int bb = i >> 1, o8 = (i & 1) * 8;
        float x = fmaxf(fmaxf(scur[bb][o8], scur[bb][o8 + 1]), scur[bb][o8 + 2]);
        x = fmaxf(fmaxf(x, scur[bb][o8 + 3]), scur[bb][o8 + 4]);
        x = fmaxf(fmaxf(x, scur[bb][o8 + 5]), scur[bb][o8 + 6]);
        pm[i] = fmaxf(x, scur[bb][o8 + 7]);
        asm volatile("" : "+v"(pm[i]));
      }
      if constexpr (i == 3) {
        mxs = fmaxf(fmaxf(pm[0], pm[1]), fmaxf(pm[2], pm[3]));
        mxs = swap32_max(mxs) * scale_log2;
        asm volatile("" : "+v"(mxs));
      }
      if constexpr (i == 4) {
        const float m_cand = fmaxf(m_run, mxs);
        raise = m_cand > m_run + kLazyRescale;
        m_new = raise ? m_cand : m_run;
        neg_m = m_new == -INFINITY ? 0.f : -m_new;
        asm volatile("" : "+v"(neg_m));
      }
      // element pairs: FMA in slot fs(k), exp in fs(k)+1, sum in fs(k)+2
      static_for<0, 16>([&](auto kc_) {
        constexpr int kp = decltype(kc_)::value;
        constexpr int f = 5 + (kp * (NSLOT - 7)) / 16;
        constexpr int el0 = 2 * kp, bb = el0 >> 4, ii = el0 & 15;
        if constexpr (f == i) {
          e[el0] = fmaf(scur[bb][ii], scale_log2, neg_m);
          e[el0 + 1] = fmaf(scur[bb][ii + 1], scale_log2, neg_m);
          asm volatile("" : "+v"(e[el0]), "+v"(e[el0 + 1]));
        }
        if constexpr (f + 1 == i) {
          e[el0] = exp2_(e[el0]);
          e[el0 + 1] = exp2_(e[el0 + 1]);
          asm volatile("" : "+v"(e[el0]), "+v"(e[el0 + 1]));
        }
        if constexpr (f + 2 == i) {
          psum0 += e[el0];
          psum1 += e[el0 + 1];
          asm volatile("" : "+v"(psum0), "+v"(psum1));
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });

    if (raise) l_run *= exp2_(m_run - m_new);
    m_run = m_new;
    l_run += psum0 + psum1;
    // largest logit of the tile, once its last step is in
    tmax = (s % SPT == 0) ? mxs : fmaxf(tmax, mxs);
    if (s % SPT == SPT - 1 && hf == 0) rm_row[(int64_t)(s / SPT) * S] = tmax;
    // own copies landed, and every wave is past its reads of the slot the
    // next step overwrites
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  using T = std::true_type;
  using F = std::false_type;
  using Z = std::integral_constant<int, 0>;
  using O1 = std::integral_constant<int, 1>;
  if (N > 0) {
    KB::copy(krs, k_off(0), k0, koff, wave);
    if (N > 1) KB::copy(krs, k_off(1), k1, koff, wave);
    build_bias_table<SPT>(btab, L, h, tid, 2 * S);
    wait_all();
    __syncthreads();
    load_bias(sA, bias_of(0));
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      sA[0] = mfma32(KB::read(k0, n, 2 * s + hf), qr[s], sA[0]);
      sA[1] = mfma32(KB::read(k0, 32 + n, 2 * s + hf), qr[s], sA[1]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // k0 free
    int s = 0;
    for (; s + 1 <= N - 2; s += 2) {
      step(T{}, Z{}, s);
      step(T{}, O1{}, s + 1);
    }
    if (s <= N - 2) {
      step(T{}, Z{}, s);
      ++s;
    }
    if (s & 1) step(F{}, O1{}, s);
    else step(F{}, Z{}, s);
  }
  const float l_tot = swap32_sum(l_run);
  if (hf == 0) ml[((int64_t)sub * chunks + c) * S + qslot] = make_float2(m_run, l_tot);
}

// Pass 2.  Workgroup (subset entry, block of 32 key tiles), 4 waves.  Lane l
// of every wave holds query slots 2l, 2l+1 (S = 128) or l (S = 64): merges
// the chunk partials into lse2, then wave w takes key tiles jb + w, jb + w +
// 4, ... of the block and reduces max over real slots of exp2(rowmax - lse2)
// across the wave.  Block 0 also writes lse.
constexpr int kReduceTiles = 32;
constexpr int kMaxChunks = 16;   // map_chunks() never returns more

template <int S>
__global__ __launch_bounds__(256) void map_reduce_kernel(
    DevLayout L, const int32_t* __restrict__ q_tiles, int chunks,
    const float* __restrict__ rowmax, const float2* __restrict__ ml, float* __restrict__ lse,
    float* __restrict__ map) {
  constexpr int QPL = S / 64;   // query slots per lane
  const int sub = blockIdx.y;
  const int jb = blockIdx.x * kReduceTiles;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* mrow = map + (int64_t)sub * L.max_tiles;
  const int jend = min(jb + kReduceTiles, (int)L.max_tiles);
  const int64_t g = q_tiles[sub];
  if (g < 0 || g >= L.tile_off[L.heads]) {
    for (int j = jb + tid; j < jend; j += 256) mrow[j] = 0.f;
    return;
  }
  const int h = head_of_tile(L, g);
  const int n_h = (int)(L.tile_off[h + 1] - L.tile_off[h]);
  const TileExtent eq = tile_extent(L, h, (int)(g - L.tile_off[h]));

  // every load of the workgroup goes out first: the chunk partials of this
  // lane's slots and the row maxima of its key tiles
  float2 part[QPL][kMaxChunks];
#pragma unroll
  for (int u = 0; u < QPL; ++u)
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c)
      part[u][c] = c < chunks ? ml[((int64_t)sub * chunks + c) * S + QPL * lane + u]
                              : make_float2(-INFINITY, 0.f);
  const float* rm = rowmax + (int64_t)sub * L.max_tiles * S + QPL * lane;
  constexpr int PER_WAVE = kReduceTiles / 4;
  float x[PER_WAVE][QPL];
#pragma unroll
  for (int t = 0; t < PER_WAVE; ++t) {
    const int j = jb + wave + 4 * t;
#pragma unroll
    for (int u = 0; u < QPL; ++u) x[t][u] = j < n_h ? rm[(int64_t)j * S + u] : 0.f;
  }
  float lse2[QPL];
  bool real[QPL];
#pragma unroll
  for (int u = 0; u < QPL; ++u) {
    const int qs = QPL * lane + u;
    real[u] = eq.slot_real(qs);
    float M = -INFINITY;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) M = fmaxf(M, part[u][c].x);
    float Ls = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c)
        if (part[u][c].y > 0.f) Ls += part[u][c].y * exp2_(part[u][c].x - M);
    }
    lse2[u] = Ls > 0.f ? M + __log2f(Ls) : -INFINITY;
    if (blockIdx.x == 0 && wave == 0) lse[(int64_t)sub * S + qs] = lse2[u] * 0.69314718055994531f;
  }
#pragma unroll
  for (int t = 0; t < PER_WAVE; ++t) {
    const int j = jb + wave + 4 * t;
    float v = 0.f;
#pragma unroll
    for (int u = 0; u < QPL; ++u)
      if (j < n_h && real[u] && lse2[u] != -INFINITY) v = fmaxf(v, exp2_(x[t][u] - lse2[u]));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    if (lane == 0 && j < jend) mrow[j] = v;
  }
}

}  // namespace

// Pass-1 chunks per subset tile.  Pass 1 runs n_sub * c equal workgroups,
// `slots` of them at a time; its time is about rounds(c) * (work of one
// workgroup) with rounds(c) = ceil(n_sub c / slots) and one workgroup's work
// ceil(max_tiles / c) * SPT steps plus a fixed cost of about kChunkFixed
// steps (loading its queries, the first copies, the final partials).  c is
// the smallest minimiser over 1 .. kMaxChunks: a last round that would run
// nearly empty is avoided by cutting the key tiles finer.
constexpr int64_t kChunkFixed = 6;
int64_t map_chunks(int64_t n_sub, int64_t max_tiles, int64_t spt, int64_t slots) {
  if (n_sub <= 0) return 1;
  if (slots < 1) slots = 1;
  int64_t best = 1, best_t = -1;
  for (int64_t c = 1; c <= kMaxChunks && c <= max_tiles; ++c) {
    const int64_t rounds = (n_sub * c + slots - 1) / slots;
    const int64_t t = rounds * ((max_tiles + c - 1) / c * spt + kChunkFixed);
    if (best_t < 0 || t < best_t) {
      best_t = t;
      best = c;
    }
  }
  return best;
}

// Workgroups of pass 1 resident at once on the current device.
template <int D, int S>
int64_t map_slots() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, map_stats_kernel<D, S>, 2 * S, 0) !=
          hipSuccess)
    return 1;
  return (int64_t)cus * (per_cu > 0 ? per_cu : 1);
}

// The workspace holds the partials of kMaxChunks chunks, whatever the
// launch chooses.
int64_t map_workspace_bytes(const DevLayout& L, int64_t n_sub) {
  if (n_sub <= 0) return 0;
  const int64_t S = L.S;
  const int64_t rm = ((n_sub * L.max_tiles * S * 4) + 255) / 256 * 256;
  const int64_t mlb = n_sub * kMaxChunks * S * 8;
  return rm + mlb;
}

int launch_oracle_map(const DevLayout& L, const void* q, const void* k, float sm_scale,
                      const int32_t* q_tiles, int n_sub, void* workspace, float* lse, float* map,
                      hipStream_t s) {
  if (n_sub == 0) return VEDA_OK;
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  const int64_t slots = L.d == 128 ? map_slots<128, 128>() : map_slots<64, 64>();
  const int chunks = (int)map_chunks(n_sub, L.max_tiles, L.S / 64, slots);
  float* rowmax = static_cast<float*>(workspace);
  const int64_t rm = ((n_sub * (int64_t)L.max_tiles * L.S * 4) + 255) / 256 * 256;
  float2* ml = reinterpret_cast<float2*>(static_cast<unsigned char*>(workspace) + rm);
  const unsigned grid1 = (unsigned)(n_sub * chunks);
  const dim3 grid2((unsigned)((L.max_tiles + kReduceTiles - 1) / kReduceTiles), (unsigned)n_sub);
  if (L.d == 128) {
    hipLaunchKernelGGL((map_stats_kernel<128, 128>), dim3(grid1), dim3(256), 0, s, L,
                       (const __bf16*)q, (const __bf16*)k, scale_log2, q_tiles, chunks, rowmax, ml);
    hipLaunchKernelGGL((map_reduce_kernel<128>), grid2, dim3(256), 0, s, L, q_tiles, chunks,
                       rowmax, ml, lse, map);
  } else {
    hipLaunchKernelGGL((map_stats_kernel<64, 64>), dim3(grid1), dim3(128), 0, s, L,
                       (const __bf16*)q, (const __bf16*)k, scale_log2, q_tiles, chunks, rowmax, ml);
    hipLaunchKernelGGL((map_reduce_kernel<64>), grid2, dim3(256), 0, s, L, q_tiles, chunks,
                       rowmax, ml, lse, map);
  }
  return launch_status();
}

}  // namespace veda
