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
#include <type_traits>

#include "attn_common.hpp"

namespace veda {
namespace {

using namespace attn;

constexpr float kLazyRescale = 8.0f;   // log2 of the largest unnormalised term
// Running reference of a row that has seen no real key: finite, so that its
// negation enters the exp2 argument with no test, and far below any logit.
constexpr float kNoRef = -3.0e38f;

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
//                       exp2(sm_scale*log2(e) q.k) = l * 2^m  (l = 0 for a
//                       chunk with no real key)
// Item of pass 1 for a workgroup on XCD x, out of G items in 8 contiguous
// ranges (range y: per + (y < rem) items from y*per + min(y, rem)): the next
// unclaimed item of range x, else of range x+1, x+2, ... (mod 8); -1 when all
// are claimed.  Every item goes to exactly one workgroup: the counters only
// grow, and a range is only given up once its counter has passed its length.
__device__ __forceinline__ int claim_item(int* claim, int x, int G) {
  const int per = G / 8, rem = G % 8;
  for (int o = 0; o < 8; ++o) {
    const int y = (x + o) & 7;
    const int len = per + (y < rem ? 1 : 0);
    if (__hip_atomic_load(&claim[y], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= len) continue;
    const int i = atomicAdd(&claim[y], 1);
    if (i < len) return y * per + min(y, rem) + i;
  }
  return -1;
}

__global__ void map_claim_reset_kernel(int* claim) {
  if (threadIdx.x < 8) claim[threadIdx.x] = 0;
}

template <int D, int S>
__global__ __launch_bounds__(2 * S, 3) void map_stats_kernel(
    DevLayout L, const __bf16* __restrict__ q, const __bf16* __restrict__ k, float scale_log2,
    const int32_t* __restrict__ q_tiles, int n_sub, int chunks, float* __restrict__ rowmax,
    float2* __restrict__ ml, int* __restrict__ claim) {
  using P = MapPipe<D, S>;
  using KB = typename P::KBuf;
  constexpr int SPT = P::SPT, KS = P::KS, TILE = P::TILE;
  __shared__ __attribute__((aligned(1024))) unsigned char k0[KB::BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char k1[KB::BYTES];
  __shared__ BiasTable<SPT> btab;

  // The work items (subset tile, chunk) are numbered chunk-major and cut
  // into 8 contiguous ranges, range x for XCD x: the workgroups running
  // together on one XCD take the same key-tile range for consecutive subset
  // tiles, which share it in L2.  A workgroup claims the next item of its
  // XCD's range (the hardware places workgroup b on XCD b % 8), or, once that
  // range is used up, of the next range that is not: XCDs that run faster
  // take over the end of the slower ones' work.  The grid holds spare
  // workgroups for that; one that finds every range used up exits.
  __shared__ int item_s;
  if (threadIdx.x == 0) item_s = claim_item(claim, (int)(blockIdx.x & 7), n_sub * chunks);
  __syncthreads();
  const int b = item_s;
  if (b < 0) return;
  const int sub = b % n_sub, c = b / n_sub;
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

  // A wave whose 32 query slots are all padding (the cut rows of a boundary
  // subset tile) computes nothing: it issues its share of every copy, joins
  // every barrier, and writes -inf row maxima and an empty partial for its
  // rows, which the reduce pass treats as padding.
  const bool pad_wave =
      !__any(tile_extent(L, h, (int)(g - L.tile_off[h])).slot_real(wave * 32 + n));

  bf16x8 qr[KS];
  const int qslot = wave * 32 + n;
  if (!pad_wave) load_q_regs<D>(qr, q + (g * S + qslot) * D, hf);

  const auto krs = make_rsrc(reinterpret_cast<const unsigned char*>(k) + head_base * TILE,
                             (int64_t)n_h * TILE);
  uint32_t koff[KB::PER_WAVE];
  KB::offsets(koff, wave, lane);
  auto k_off = [&](int t) { return (uint32_t)((j0 + t / SPT) * TILE + (t % SPT) * P::KSTEP); };
  // Grid coordinates and cut of the key tile whose logits are computed next.
  // Steps visit the chunk's tiles in index order, so the coordinates advance
  // one tile at a time (no division per tile); a tile's cut marks the axes
  // along which it is the last, partial tile of the grid.
  const int nH = L.grid[h][1], nW = L.grid[h][2], nT = L.grid[h][0];
  const bool part_t = L.T % L.shape[h][0] != 0, part_h = L.H % L.shape[h][1] != 0,
             part_w = L.W % L.shape[h][2] != 0;
  const TileExtent e0 = tile_extent(L, h, j0);
  int kw = e0.iw, kh = e0.ih, kt = e0.it;
  int qcut = 0;
  // cut of the tile of step t (called once per step, in order)
  auto cut_at = [&](int t) -> int {
    if (t % SPT == 0) {
      if (t > 0 && ++kw == nW) {
        kw = 0;
        if (++kh == nH) { kh = 0; ++kt; }
      }
      qcut = (part_t && kt == nT - 1 ? 4 : 0) | (part_h && kh == nH - 1 ? 2 : 0) |
             (part_w && kw == nW - 1 ? 1 : 0);
    }
    return qcut;
  };
  auto bias_of = [&](int t) -> const f32x4* { return &btab.v[qcut][t % SPT][0][hf][0]; };

  // m_thr = m_run + kLazyRescale, updated with m_run
  float m_run = kNoRef, m_thr = kNoRef + kLazyRescale, l_run = 0.f, tmax = -INFINITY;
  float* rm_row = rowmax + ((int64_t)sub * L.max_tiles + j0) * S + qslot;
  f32x16 sA[2], sB[2];

  // One step s: statistics of step s and, in the same hand-laid block,
  // S^T(s+1) = K(s+1) Q^T, with the copy of K(s+2) spread over the slots.
  // ZS: the tile of step s+1 has no padding key, so its mask rows are all
  // zero; its products then start from an inline zero accumulator instead of
  // reading the rows from LDS.
  auto step = [&](auto has_qk, auto par, auto zero_seed, int s) __attribute__((always_inline)) {
    constexpr bool QK = decltype(has_qk)::value;
    constexpr int PAR = decltype(par)::value;
    constexpr bool ZS = decltype(zero_seed)::value;
    f32x16 (&scur)[2] = PAR ? sB : sA;
    f32x16 (&snext)[2] = PAR ? sA : sB;
    const unsigned char* ksrc = PAR ? k0 : k1;
    unsigned char* kdst = PAR ? k1 : k0;

    if constexpr (QK && !ZS) load_bias(snext, bias_of(s + 1));
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
    float e[32];
    float mx = 0.f, mxs = 0.f, m_new = 0.f, psum0 = 0.f, psum1 = 0.f;
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
        if constexpr (ZS && i < 2)
          snext[i & 1] = mfma32(opnd[i % (LA + 1)], qr[i >> 1], f32x16{});
        else
          snext[i & 1] = mfma32(opnd[i % (LA + 1)], qr[i >> 1], snext[i & 1]);
      }
      // statistics of step s: row maximum in slots 0..4 (one chain of
      // three-operand maxima over the lane's 32 logits), then the elements
      if constexpr (i < 4) {
        constexpr int bb = i >> 1, o8 = (i & 1) * 8;
        float x = i == 0 ? fmaxf(scur[bb][o8], scur[bb][o8 + 1])
                         : fmaxf(fmaxf(mx, scur[bb][o8]), scur[bb][o8 + 1]);
        x = fmaxf(fmaxf(x, scur[bb][o8 + 2]), scur[bb][o8 + 3]);
        x = fmaxf(fmaxf(x, scur[bb][o8 + 4]), scur[bb][o8 + 5]);
        mx = fmaxf(fmaxf(x, scur[bb][o8 + 6]), scur[bb][o8 + 7]);
        asm volatile("" : "+v"(mx));
      }
      if constexpr (i == 3) {
        mxs = swap32_max(mx) * scale_log2;
        asm volatile("" : "+v"(mxs));
      }
      // the reference is held as m_new; its negation is a source modifier of
      // the FMAs below, not an instruction of its own
      if constexpr (i == 4) {
        const float m_cand = fmaxf(m_run, mxs);
        raise = m_cand > m_thr;
        m_new = raise ? m_cand : m_run;
        asm volatile("" : "+v"(m_new));
      }
      // element pairs: FMA in slot fs(k), exp in fs(k)+1, sum in fs(k)+2
      static_for<0, 16>([&](auto kc_) {
        constexpr int kp = decltype(kc_)::value;
        constexpr int f = 5 + (kp * (NSLOT - 7)) / 16;
        constexpr int el0 = 2 * kp, bb = el0 >> 4, ii = el0 & 15;
        if constexpr (f == i) {
          e[el0] = fmaf(scur[bb][ii], scale_log2, -m_new);
          e[el0 + 1] = fmaf(scur[bb][ii + 1], scale_log2, -m_new);
          asm volatile("" : "+v"(e[el0]), "+v"(e[el0 + 1]));
        }
        if constexpr (f + 1 == i) {
          e[el0] = exp2_(e[el0]);
          e[el0 + 1] = exp2_(e[el0 + 1]);
          asm volatile("" : "+v"(e[el0]), "+v"(e[el0 + 1]));
        }
        if constexpr (f + 2 == i) {
          // the first pair starts the two sums (0 + e is e: no add)
          psum0 = kp == 0 ? e[el0] : psum0 + e[el0];
          psum1 = kp == 0 ? e[el0 + 1] : psum1 + e[el0 + 1];
          asm volatile("" : "+v"(psum0), "+v"(psum1));
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });

    // the sum to the new reference: rare after a row's first real key, so
    // the exponential is skipped unless some lane raised
    if (__builtin_expect(__any(raise), 0)) {
      l_run *= raise ? exp2_(m_run - m_new) : 1.f;
      m_thr = m_new + kLazyRescale;
    }
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
  // a padding wave's step: the same copy of K(s+2) (K(s) again when there is
  // no step s+2) into the same slot, the row maxima as -inf, and the same
  // end-of-step wait and barrier
  auto copy_step = [&](int s) {
    const uint32_t kgs = s + 2 < N ? k_off(s + 2) : k_off(s);
    unsigned char* kdst = (s & 1) ? k1 : k0;
    static_for<0, KB::PER_WAVE>([&](auto mc) {
      KB::round(decltype(mc)::value, krs, kgs, kdst, koff, wave);
    });
    if (s % SPT == SPT - 1 && hf == 0) rm_row[(int64_t)(s / SPT) * S] = -INFINITY;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  // a step with products, in the variant its next tile's cut asks for
  auto qk_step = [&](auto par, int s) __attribute__((always_inline)) {
    if (cut_at(s + 1) == 0) step(T{}, par, T{}, s);
    else step(T{}, par, F{}, s);
  };
  if (N > 0) {
    KB::copy(krs, k_off(0), k0, koff, wave);
    if (N > 1) KB::copy(krs, k_off(1), k1, koff, wave);
    build_bias_table<SPT>(btab, L, h, tid, 2 * S);
    wait_all();
    __syncthreads();
    if (pad_wave) {
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      for (int s = 0; s < N; ++s) copy_step(s);
    } else {
    cut_at(0);
    load_bias(sA, bias_of(0));
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      sA[0] = mfma32(KB::read(k0, n, 2 * s + hf), qr[s], sA[0]);
      sA[1] = mfma32(KB::read(k0, 32 + n, 2 * s + hf), qr[s], sA[1]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // k0 free
    int s = 0;
    for (; s + 1 <= N - 2; s += 2) {
      qk_step(Z{}, s);
      qk_step(O1{}, s + 1);
    }
    if (s <= N - 2) {
      qk_step(Z{}, s);
      ++s;
    }
    if (s & 1) step(F{}, O1{}, F{}, s);
    else step(F{}, Z{}, F{}, s);
    }
  }
  const float l_tot = swap32_sum(l_run);
  if (hf == 0) ml[((int64_t)sub * chunks + c) * S + qslot] = make_float2(m_run, l_tot);
}

// Maximum of v over the 64 lanes of the wave, in every lane: within each
// quad and row of 16 by DPP (swap neighbours, swap pairs, rotate by 4 and 8),
// then across rows by exchanging with lane l ^ 16 and l ^ 32.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_max_all(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x124>(v));   // row_ror:4
  v = fmaxf(v, dpp_f32<0x128>(v));   // row_ror:8
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  return swap32_max(v);
}

// Pass 2.  Workgroup (subset entry, block of tb key tiles), 4 waves.  Lane l
// of every wave holds query slots 2l, 2l+1 (S = 128) or l (S = 64): it merges
// the chunk partials of its slots into lse2 once, then wave w takes key tiles
// jb + w, jb + w + 4, ... of the block, kAhead at a time.  Per key tile the
// wave reads the tile's S row maxima (one 4*QPL-byte load per lane), takes
// the largest rowmax - lse2 over the tile's real rows with a wave reduction
// (the kAhead reductions interleaved), and writes exp2 of it: exp2 is
// monotone, so this is the largest probability of the block.  Block 0 also
// writes lse.
constexpr int kAhead = 8;
constexpr int kMaxChunks = 16;   // map_chunks() never returns more

template <int S>
__global__ __launch_bounds__(256) void map_reduce_kernel(
    DevLayout L, const int32_t* __restrict__ q_tiles, int chunks, int tb,
    const float* __restrict__ rowmax, const float2* __restrict__ ml, float* __restrict__ lse,
    float* __restrict__ map) {
  constexpr int QPL = S / 64;   // query slots per lane
  using Vec = typename std::conditional<QPL == 2, float2, float>::type;
  const int sub = blockIdx.y;
  const int jb = blockIdx.x * tb;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  float* mrow = map + (int64_t)sub * L.max_tiles;
  const int jend = min(jb + tb, (int)L.max_tiles);
  const int64_t g = q_tiles[sub];
  if (g < 0 || g >= L.tile_off[L.heads]) {
    for (int j = jb + tid; j < jend; j += 256) mrow[j] = 0.f;
    return;
  }
  const int h = head_of_tile(L, g);
  const int n_h = (int)(L.tile_off[h + 1] - L.tile_off[h]);
  const TileExtent eq = tile_extent(L, h, (int)(g - L.tile_off[h]));
  for (int j = max(jb, n_h) + tid; j < jend; j += 256) mrow[j] = 0.f;   // beyond the head

  // lse2 of this lane's slots; -inf for a padding slot, so that it never
  // wins.  Every partial is loaded first (predicated, all in flight at once).
  float2 part[QPL][kMaxChunks];
#pragma unroll
  for (int u = 0; u < QPL; ++u)
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c)
      part[u][c] = c < chunks ? ml[((int64_t)sub * chunks + c) * S + QPL * lane + u]
                              : make_float2(-INFINITY, 0.f);
  float neg_lse[QPL];
#pragma unroll
  for (int u = 0; u < QPL; ++u) {
    const int qs = QPL * lane + u;
    float M = -INFINITY;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) M = fmaxf(M, part[u][c].x);
    float Ls = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c)
        if (part[u][c].y > 0.f) Ls += part[u][c].y * exp2_(part[u][c].x - M);
    }
    const float lse2 = Ls > 0.f ? M + __log2f(Ls) : -INFINITY;
    if (blockIdx.x == 0 && wave == 0) lse[(int64_t)sub * S + qs] = lse2 * 0.69314718055994531f;
    // a real row always has a real key, so lse2 is finite for it
    neg_lse[u] = eq.slot_real(qs) && lse2 != -INFINITY ? -lse2 : -INFINITY;
  }
  const float* rm = rowmax + (int64_t)sub * L.max_tiles * S + QPL * lane;
  const int jlast = min(jend, n_h);
  // tiles jb + wave + 4t of this block that lie in the head
  const int nt = jlast > jb + wave ? (jlast - (jb + wave) + 3) / 4 : 0;
  for (int t0 = 0; t0 < nt; t0 += kAhead) {
    Vec x[kAhead];
#pragma unroll
    for (int a = 0; a < kAhead; ++a) {
      const int j = jb + wave + 4 * min(t0 + a, nt - 1);   // past the end: re-read the last
      x[a] = *reinterpret_cast<const Vec*>(rm + (int64_t)j * S);
    }
    float v[kAhead];
#pragma unroll
    for (int a = 0; a < kAhead; ++a) {
      if constexpr (QPL == 2) v[a] = fmaxf(x[a].x + neg_lse[0], x[a].y + neg_lse[1]);
      else v[a] = x[a] + neg_lse[0];
    }
#pragma unroll
    for (int a = 0; a < kAhead; ++a) v[a] = wave_max_all(v[a]);
    if (lane < kAhead) {
      float w = v[0];
#pragma unroll
      for (int a = 1; a < kAhead; ++a) w = lane == a ? v[a] : w;
      if (t0 + lane < nt) mrow[jb + wave + 4 * (t0 + lane)] = w == -INFINITY ? 0.f : exp2_(w);
    }
  }
}

}  // namespace

// Pass-1 chunks per subset tile.  Pass 1 runs n_sub * c items of w(c) =
// ceil(max_tiles / c) * SPT steps plus a fixed cost of about kChunkFixed steps
// (loading its queries, the first copies, the final partials), `slots`
// workgroups at a time.  The work claiming keeps every slot busy until the
// items run out, so the time is about the work per slot, n_sub c (w(c) +
// kChunkFixed) / slots, plus the drain at the end, which lasts about one
// item: t(c) = n_sub c (w(c) + fixed) / slots + w(c).  Finer chunks shorten
// the drain and add fixed costs; c is the smallest minimiser over
// 1 .. kMaxChunks.
constexpr int64_t kChunkFixed = 6;
int64_t map_chunks(int64_t n_sub, int64_t max_tiles, int64_t spt, int64_t slots) {
  if (n_sub <= 0) return 1;
  if (slots < 1) slots = 1;
  int64_t best = 1;
  double best_t = -1.0;
  for (int64_t c = 1; c <= kMaxChunks && c <= max_tiles; ++c) {
    const int64_t w = (max_tiles + c - 1) / c * spt;
    const double t = (double)(n_sub * c) * (double)(w + kChunkFixed) / (double)slots + (double)w;
    if (best_t < 0.0 || t < best_t) {
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
  const int64_t mlb = (n_sub * kMaxChunks * S * 8 + 255) / 256 * 256;
  return rm + mlb + 256;   // + the 8 claim counters of pass 1
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
  const int64_t mlb = ((int64_t)n_sub * kMaxChunks * L.S * 8 + 255) / 256 * 256;
  float2* ml = reinterpret_cast<float2*>(static_cast<unsigned char*>(workspace) + rm);
  int* claim = reinterpret_cast<int*>(static_cast<unsigned char*>(workspace) + rm + mlb);
  // items plus a quarter of each XCD's share in spare workgroups
  const int64_t items = (int64_t)n_sub * chunks;
  const unsigned grid1 = (unsigned)(items + 8 * (((items + 7) / 8 + 3) / 4));
  hipLaunchKernelGGL(map_claim_reset_kernel, dim3(1), dim3(64), 0, s, claim);
  // pass 2: blocks of 32..256 key tiles, about 4096 workgroups in all
  int64_t tb = ((int64_t)L.max_tiles * n_sub / 4096 + 31) / 32 * 32;
  tb = tb < 32 ? 32 : (tb > 256 ? 256 : tb);
  const dim3 grid2((unsigned)((L.max_tiles + tb - 1) / tb), (unsigned)n_sub);
  if (L.d == 128) {
    hipLaunchKernelGGL((map_stats_kernel<128, 128>), dim3(grid1), dim3(256), 0, s, L,
                       (const __bf16*)q, (const __bf16*)k, scale_log2, q_tiles, n_sub, chunks,
                       rowmax, ml, claim);
    hipLaunchKernelGGL((map_reduce_kernel<128>), grid2, dim3(256), 0, s, L, q_tiles, chunks,
                       (int)tb, rowmax, ml, lse, map);
  } else {
    hipLaunchKernelGGL((map_stats_kernel<64, 64>), dim3(grid1), dim3(128), 0, s, L,
                       (const __bf16*)q, (const __bf16*)k, scale_log2, q_tiles, n_sub, chunks,
                       rowmax, ml, claim);
    hipLaunchKernelGGL((map_reduce_kernel<64>), grid2, dim3(256), 0, s, L, q_tiles, chunks,
                       (int)tb, rowmax, ml, lse, map);
  }
  return launch_status();
}

}  // namespace veda
