// Tile-skipping block-sparse attention forward (Veda §2.3: the kernel visits
// only each query tile's kept, non-contiguous key/value tiles and hides their
// fetch behind dense matrix math).
//
// One workgroup per (head, query tile), S/32 waves: wave w owns queries
// 32w..32w+31, held in registers as MFMA operands.  The workgroup walks the
// kept key tiles of its CSR row in steps of 64 keys (half a 128-key tile).
// Per step s and wave, one straight-line block holds three independent
// pieces of work, so the matrix cores and the vector ALUs of the wave stay
// busy together:
//   softmax(s)   logits S(s) -> probabilities P(s) (vector ALU),
//   QK(s+1)      S(s+1)^T = K(s+1) Q^T             (MFMA, K from LDS),
//   PV(s-1)      O^T += V(s-1)^T P(s-1)^T           (MFMA, V^T from LDS).
// The block is laid out by hand in slots of one MFMA each, with the LDS read
// of a later slot's operand and a share of the softmax; the compiler may not
// move work across slots.
//
// K and V^T steps are copied HBM -> LDS with buffer_load ... lds (no register
// staging) into two slots each.  The copies of K(s+2) and V(s) are spread
// over the slots of step s and land by its end: one barrier per step.  K and
// V^T slots and the mask table take 74 KiB, so two workgroups share a CU and
// the two waves on a SIMD come from different, unsynchronised workgroups.
//
// Per logit: the products start from zero, and the padding keys of a
// boundary tile (or of an entry outside the head) get -inf added from a
// per-workgroup mask table before the softmax, in a uniform branch that full
// tiles skip; online softmax in base 2 with sm_scale*log2(e) folded into one
// FMA, P rounded to bf16, f32 accumulation.  The running maximum is raised only when a new
// logit exceeds it by more than 2^8, so the accumulator is rescaled rarely;
// the result is the same softmax (numerator and denominator share one
// reference).  The CSR row sits in one register, 64 entries at a time (lane
// l: entry l, with its tile's cut), and each step reads its entries with
// v_readlane: no memory access and no integer division per step.  An entry
// outside [0, n_tiles) becomes a tile whose keys are all masked, which leaves
// the result exactly as if it were skipped.
//
// Workgroups take their query tiles in an XCD-aware order.  With heads of at
// least kLockstepTiles tiles, in lockstep: all XCDs work in the same head at
// once, so the key/value tiles in flight are about one head's, which the
// memory-side cache holds, and the query tiles running together on one XCD
// are a contiguous run of that head (neighbours whose kept key tiles overlap
// in its L2).  With smaller heads, one eighth of a head is shorter than the
// workgroups an XCD runs at once, and each XCD takes a contiguous eighth of
// the layer instead.  Either way XCD x has a run of tiles; with a workspace
// the last tenth of every run is handed out through counters to whichever
// XCD gets there first (see claim_tail_tile).
#include <algorithm>
#include <climits>

#include "attn_common.hpp"

namespace veda {
namespace {

using namespace attn;

constexpr float kLazyRescale = 8.0f;   // log2 of the largest unnormalised p
// Running reference of a row that has seen no real key: finite, so that its
// negation enters the exp2 argument with no test, and far below any logit.
constexpr float kNoRef = -3.0e38f;
// Lockstep XCD order from this many tiles per head on: 8 XCDs x 64 resident
// workgroups (two per CU on 32 CUs).
constexpr int kLockstepTiles = 512;

template <int D, int S>
struct Pipe {
  static constexpr int NW = S / 32;             // waves per workgroup
  static constexpr int SK = 64;                 // keys per step
  static constexpr int SPT = S / SK;            // steps per key tile
  static constexpr int KS = D / 16;             // MFMA k-steps over head_dim
  static constexpr int DB = D / 32;             // 32-row blocks of O^T
  static constexpr int TILE = S * D * 2;
  static constexpr int KSTEP = SK * D * 2;      // HBM bytes of one K step
  using KBuf = StepBuf<SK, D / 8, true, D * 2, NW>;    // K rows (keys), swap23 order
  using VBuf = StepBuf<D, SK / 8, false, S * 2, NW>;   // V^T rows (dims), SK keys
  static_assert(S % SK == 0, "tile must hold whole steps");
};

// TOK: O is written in token order ([N][heads][D], real slots only) instead
// of tile order, which folds the inverse permutation into the epilogue.
// Work claiming at the end of the lockstep order.  XCD x's run has len[x]
// tiles; workgroup b = 8 i + x with i < fixed[x] takes run position i as
// before, and the last len[x] - fixed[x] positions (about a tenth) are handed
// out through counter x of the caller's workspace: a workgroup past fixed[x]
// takes the next unclaimed position of its own XCD's tail, else of the next
// XCD's tail that has one left (x+1, x+2, ... mod 8), else nothing (-1).  The
// counters only grow and a tail is only passed over once its counter has
// reached its length, so every position goes to exactly one workgroup.  The
// XCDs do not all run at the same speed (on one box the odd ones took 2.5 %
// longer per tile); with fixed shares the last of them finished 1.5 ms after
// the first.
struct ClaimPlan {
  int len[8];
  int fixed[8];
};

// Tile at position i of XCD x's run: the lockstep order, or the x-th
// contiguous eighth of the layer's tiles.
__device__ __forceinline__ int64_t run_tile(const DevLayout& L, int lockstep, int x, int i) {
  if (lockstep) return lockstep_tile(L, (int64_t)i * 8 + x);
  const int64_t G = L.tile_off[L.heads];
  return xcd_remap((int64_t)i * 8 + x, G);
}

__device__ __forceinline__ int64_t claim_tail_tile(const DevLayout& L, int lockstep, int* claim,
                                                   const ClaimPlan& plan, int x) {
  for (int o = 0; o < 8; ++o) {
    const int y = (x + o) & 7;
    const int tail = plan.len[y] - plan.fixed[y];
    if (__hip_atomic_load(&claim[y], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= tail) continue;
    const int c = atomicAdd(&claim[y], 1);
    if (c < tail) return run_tile(L, lockstep, y, plan.fixed[y] + c);
  }
  return -1;
}

__global__ void attn_claim_reset_kernel(int* claim) {
  if (threadIdx.x < 8) claim[threadIdx.x] = 0;
}

template <int D, int S, bool TOK>
__global__ __launch_bounds__(2 * S, 2) void sparse_attn_fwd_kernel(
    DevLayout L, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ vt, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, float scale_log2, __bf16* __restrict__ o,
    float* __restrict__ lse, int lockstep, int* __restrict__ claim, ClaimPlan plan) {
  using P = Pipe<D, S>;
  using KB = typename P::KBuf;
  using VB = typename P::VBuf;
  constexpr int SPT = P::SPT, KS = P::KS, DB = P::DB, TILE = P::TILE;
  static_assert(KS == 8 || KS == 4, "head_dim 128 or 64");
  // four separate objects: reads of one slot are never ordered after copies
  // into another
  __shared__ __attribute__((aligned(1024))) unsigned char k0[KB::BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char k1[KB::BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char v0[VB::BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char v1[VB::BYTES];
  __shared__ BiasTable<SPT, 9> btab;

  int64_t g;
  const int x = (int)(blockIdx.x & 7);
  const int i = (int)(blockIdx.x >> 3);
  if (claim == nullptr) {
    g = lockstep ? lockstep_tile(L, blockIdx.x) : xcd_remap(blockIdx.x, gridDim.x);
  } else if (i < plan.fixed[x]) {
    g = run_tile(L, lockstep, x, i);
  } else {
    __shared__ int64_t g_s;
    if (threadIdx.x == 0) g_s = claim_tail_tile(L, lockstep, claim, plan, x);
    __syncthreads();
    g = g_s;
  }
  if (g < 0) return;   // past the end of this XCD's run, or nothing left to claim
  const int h = head_of_tile(L, g);
  const int n_h = (int)(L.tile_off[h + 1] - L.tile_off[h]);
  const int64_t head_base = L.tile_off[h];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hf = lane >> 5;

  // A wave whose 32 query slots are all padding (a boundary tile's cut rows)
  // computes nothing: it issues its share of every copy and joins every
  // barrier, and leaves O = 0 and lse = -inf for its rows.
  const TileExtent eq = tile_extent(L, h, (int)(g - head_base));
  const bool pad_wave = !__any(eq.slot_real(wave * 32 + n));

  bf16x8 qr[KS];
  const int64_t qrow = g * S + wave * 32 + n;
  if (!pad_wave) load_q_regs<D>(qr, q + qrow * D, hf);

  cint32* rp = (cint32*)row_ptr;
  int beg = rp[g], end = rp[g + 1];
  if (end < beg) end = beg;
  // every CSR entry is a tile of SPT steps; an entry outside [0, n_h) is a
  // tile whose keys are all masked, which leaves the result as if skipped
  const int N = (end - beg) * SPT;   // steps

  // the head's K and V^T tiles as buffer resources (raw, bounds = the head)
  const auto krs = make_rsrc(reinterpret_cast<const unsigned char*>(k) + head_base * TILE,
                             (int64_t)n_h * TILE);
  const auto vrs = make_rsrc(reinterpret_cast<const unsigned char*>(vt) + head_base * TILE,
                             (int64_t)n_h * TILE);
  uint32_t koff[KB::PER_WAVE], voff[VB::PER_WAVE];
  KB::offsets(koff, wave, lane);
  VB::offsets(voff, wave, lane);

  // A window of 64 CSR entries in one register: lane l holds entry wbase + l
  // as col | cut << 16 (cut 8 for an entry outside [0, n_h)).  Steps read
  // their tile with v_readlane: no memory access per step.
  int wbase = 0, win = 0;
  auto load_window = [&](int base) {
    const int p = beg + base + lane;
    const int c = p < end ? col_idx[p] : -1;
    const bool ok = c >= 0 && c < n_h;
    const int cut = ok ? cut_of(tile_extent(L, h, ok ? c : 0)) : 8;
    win = (ok ? c : 0) | (cut << 16);
    wbase = base;
  };
  auto entry = [&](int t) { return __builtin_amdgcn_readlane(win, t / SPT - wbase); };
  auto k_off = [&](int e, int t) { return (uint32_t)((e & 0xffff) * TILE + (t % SPT) * P::KSTEP); };
  auto v_off = [&](int e, int t) {
    return (uint32_t)((e & 0xffff) * TILE + (t % SPT) * (P::SK * 2));
  };
  auto bias_of = [&](int e, int t) -> const f32x4* {
    return &btab.v[e >> 16][t % SPT][0][hf][0];
  };

  // m_thr = m_run + kLazyRescale, updated with m_run
  float m_run = kNoRef, m_thr = kNoRef + kLazyRescale, l_run = 0.f;
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  f32x16 sA[2], sB[2];
  bf16x8 pA[4], pB[4];


  // One step s.  PAR = s & 1 picks slots and register sets at compile time.
  // The matrix products, their LDS operand reads and the softmax are laid out
  // by hand in 32 slots of one MFMA each (even: QK(s+1), odd: PV(s-1)); the
  // compiler may not move work across slots.
  auto step = [&](auto has_qk, auto has_pv, auto par, int s) {
    constexpr bool QK = decltype(has_qk)::value, PV = decltype(has_pv)::value;
    constexpr int PAR = decltype(par)::value;
    f32x16 (&scur)[2] = PAR ? sB : sA;
    f32x16 (&snext)[2] = PAR ? sA : sB;
    bf16x8 (&pcur)[4] = PAR ? pB : pA;
    const bf16x8 (&pprev)[4] = PAR ? pA : pB;
    const unsigned char* ksrc = PAR ? k0 : k1;
    const unsigned char* vsrc = PAR ? v0 : v1;

    // K(s+2) over K(s) and V(s) over V(s-2), issued spread over the slots
    // below; with no step s+2 the K rounds re-copy K(s) into its own, no
    // longer read, slot.  The window moves on when step s+2 leaves it (no
    // copy is in flight at this point).
    if ((s + 2) / SPT - wbase >= 64) load_window((s + 2) / SPT - 2);
    const int es = entry(s);
    // step s+2, or s itself when there is none (its K rounds then re-copy K(s)
    // into its own, no longer read, slot); a scalar select, not a branch
    const int t2 = s + 2 < N ? s + 2 : s;
    const int e2 = entry(t2);
    const uint32_t kgs = k_off(e2, t2);
    const uint32_t vgs = v_off(es, s);
    unsigned char* kdst = PAR ? k1 : k0;
    unsigned char* vdst = PAR ? v1 : v0;
    constexpr int RW = KB::PER_WAVE + VB::PER_WAVE;
    // the addresses come from scalar loads: have them land before the slots,
    // whose LDS waits then count the operand reads alone
    asm volatile("" :: "s"(kgs), "s"(vgs));
    // padding keys of step s's tile (rare: boundary tiles and entries outside
    // the head) get their mask rows added to the logits before the softmax
    if (es >> 16) add_bias(scur, bias_of(es, s));

    constexpr int LA = 3;          // operand reads run LA slots ahead of their MFMA
    constexpr int NSLOT = D / 4;   // D/8 QK and D/8 PV products
    auto has_mfma = [](int i) constexpr { return (i & 1) ? PV : QK; };
    auto operand = [&](int i) -> bf16x8 {
      const int j = i >> 1;
      if (i & 1) return VB::read(vsrc, (j % DB) * 32 + n, 2 * (j / DB) + hf);
      return KB::read(ksrc, (j & 1) * 32 + n, 2 * (j >> 1) + hf);
    };
    bf16x8 opnd[LA + 1];
    static_for<0, LA>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (has_mfma(i)) opnd[i % (LA + 1)] = operand(i);
    });

    float e[32];
    float mx = 0.f, mxs = 0.f, m_new = 0.f, psum0 = 0.f, psum1 = 0.f;
    bool raise = false;
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NSLOT>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      static_for<0, RW>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        if constexpr ((m * (NSLOT - 4)) / RW == i) {
          if constexpr (m < KB::PER_WAVE) KB::round(m, krs, kgs, kdst, koff, wave);
          else VB::round(m - KB::PER_WAVE, vrs, vgs, vdst, voff, wave);
        }
      });
      if constexpr (i + LA < NSLOT && has_mfma(i + LA))
        opnd[(i + LA) % (LA + 1)] = operand(i + LA);
      if constexpr (has_mfma(i)) {
        constexpr int j = i >> 1;
        if constexpr (i & 1) oacc[j % DB] = mfma32(opnd[i % (LA + 1)], pprev[j / DB], oacc[j % DB]);
        else snext[j & 1] = mfma32(opnd[i % (LA + 1)], qr[j >> 1], j < 2 ? f32x16{} : snext[j & 1]);
      }
      // softmax(s): row maximum in slots 0..4 (one chain of three-operand
      // maxima over the lane's 32 logits), then the elements
      if constexpr (i < 4) {
        constexpr int b = i >> 1, o8 = (i & 1) * 8;
        float x = i == 0 ? fmaxf(scur[b][o8], scur[b][o8 + 1])
                         : fmaxf(fmaxf(mx, scur[b][o8]), scur[b][o8 + 1]);
        x = fmaxf(fmaxf(x, scur[b][o8 + 2]), scur[b][o8 + 3]);
        x = fmaxf(fmaxf(x, scur[b][o8 + 4]), scur[b][o8 + 5]);
        mx = fmaxf(fmaxf(x, scur[b][o8 + 6]), scur[b][o8 + 7]);
        asm volatile("" : "+v"(mx));
      }
      if constexpr (i == 3) {
        mxs = swap32_max(mx);
        asm volatile("" : "+v"(mxs));
      }
      // the reference is held as m_new; its negation is a source modifier of
      // the FMAs below, not an instruction of its own
      if constexpr (i == 4) {
        const float m_cand = fmaxf(m_run, mxs * scale_log2);
        raise = m_cand > m_thr;
        m_new = raise ? m_cand : m_run;
        asm volatile("" : "+v"(m_new));
      }
      // element pairs get their FMAs in slot fs(k), exps in fs(k)+1, sums and
      // bf16 conversion in fs(k)+2; an empty asm statement pins each value to
      // its slot
      static_for<0, 16>([&](auto kc_) {
        constexpr int kp = decltype(kc_)::value;
        constexpr int f = 5 + (kp * (NSLOT - 7)) / 16;
        constexpr int el0 = 2 * kp, b = el0 >> 4, ii = el0 & 15;
        if constexpr (f == i) {
          e[el0] = fmaf(scur[b][ii], scale_log2, -m_new);
          e[el0 + 1] = fmaf(scur[b][ii + 1], scale_log2, -m_new);
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
          pcur[2 * b + (ii >> 3)][ii & 7] = (__bf16)e[el0];
          pcur[2 * b + (ii >> 3)][(ii & 7) + 1] = (__bf16)e[el0 + 1];
          // the bf16 conversion stays in this slot: left to itself the
          // compiler sinks it to the next step, whose PV reads it, where it
          // runs before the first product with nothing to overlap
          asm volatile("" : "+v"(psum0), "+v"(psum1), "+v"(pcur[2 * b + (ii >> 3)]));
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });

    // O and l to the new reference (rare), after PV(s-1), before PV(s)
    if (__builtin_expect(__any(raise), 0)) {
      const float alpha = raise ? exp2_(m_run - m_new) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      m_thr = m_new + kLazyRescale;
    }
    m_run = m_new;
    l_run += psum0 + psum1;
    // own copies landed, and every wave is past its reads of the slots the
    // next step overwrites
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  // A padding wave's step: the same copies of step s (K(s+2), or K(s) again
  // when there is no step s+2, and V(s)) into the same slots, and the same
  // end-of-step wait and barrier, with no product.
  auto copy_step = [&](int s) {
    if ((s + 2) / SPT - wbase >= 64) load_window((s + 2) / SPT - 2);
    const int es = entry(s);
    const int t2 = s + 2 < N ? s + 2 : s;
    const int e2 = entry(t2);
    const uint32_t kgs = k_off(e2, t2);
    const uint32_t vgs = v_off(es, s);
    unsigned char* kdst = (s & 1) ? k1 : k0;
    unsigned char* vdst = (s & 1) ? v1 : v0;
    static_for<0, KB::PER_WAVE>([&](auto mc) {
      KB::round(decltype(mc)::value, krs, kgs, kdst, koff, wave);
    });
    static_for<0, VB::PER_WAVE>([&](auto mc) {
      VB::round(decltype(mc)::value, vrs, vgs, vdst, voff, wave);
    });
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  using T = std::true_type;
  using F = std::false_type;
  using Z = std::integral_constant<int, 0>;
  using O1 = std::integral_constant<int, 1>;
  if (N > 0) {
    load_window(0);
    KB::copy(krs, k_off(entry(0), 0), k0, koff, wave);
    if (N > 1) KB::copy(krs, k_off(entry(1), 1), k1, koff, wave);
    build_bias_table<SPT, 9>(btab, L, h, tid, 2 * S);
    wait_all();
    __syncthreads();
    if (pad_wave) {
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      for (int s = 0; s < N; ++s) copy_step(s);
    } else {
    // logits of step 0 (its mask rows are added by the step)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      sA[0] = mfma32(KB::read(k0, n, 2 * s + hf), qr[s], s == 0 ? f32x16{} : sA[0]);
      sA[1] = mfma32(KB::read(k0, 32 + n, 2 * s + hf), qr[s], s == 0 ? f32x16{} : sA[1]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // k0 free
    if (N == 1) {
      step(F{}, F{}, Z{}, 0);
    } else {
      step(T{}, F{}, Z{}, 0);
      int s = 1;
      for (; s + 1 <= N - 2; s += 2) {
        step(T{}, T{}, O1{}, s);
        step(T{}, T{}, Z{}, s + 1);
      }
      if (s <= N - 2) {
        step(T{}, T{}, O1{}, s);
        ++s;
      }
      if (s & 1) step(F{}, T{}, O1{}, s);
      else step(F{}, T{}, Z{}, s);
    }
    // PV of the last step
    auto pv_last = [&](const bf16x8 (&pb)[4], const unsigned char* vb) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          oacc[db] = mfma32(VB::read(vb, db * 32 + n, 2 * t + hf), pb[t], oacc[db]);
    };
    if ((N - 1) & 1) pv_last(pB, v1);
    else pv_last(pA, v0);
    }
  }

  const float l_tot = swap32_sum(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  // output row of this lane's query: its slot, or (TOK) its token's row of
  // head h, none for a padding slot
  int64_t orow_i = qrow;
  if constexpr (TOK) {
    const TileExtent& e = eq;
    int dt, dh, dw;
    e.slot_coords(wave * 32 + n, dt, dh, dw);
    const int64_t tok =
        ((int64_t)(e.it * e.pt + dt) * L.H + (e.ih * e.ph + dh)) * L.W + (e.iw * e.pw + dw);
    orow_i = dt < e.lt && dh < e.lh && dw < e.lw ? tok * L.heads + h : -1;
  }
  if (orow_i >= 0) {
    __bf16* orow = o + orow_i * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 wv;
#pragma unroll
        for (int b = 0; b < 4; ++b) wv[b] = (__bf16)(oacc[db][4 * a + b] * inv);
        *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * a + 4 * hf) = wv;
      }
  }
  if (lse != nullptr && hf == 0)
    lse[qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

namespace {
template <bool TOK>
void launch_attn(const DevLayout& L, const void* q, const void* k, const void* vt,
                 const int32_t* row_ptr, const int32_t* col_idx, float scale_log2, void* o,
                 float* lse, int* claim, hipStream_t s) {
  int min_tiles = INT32_MAX;
  for (int h = 0; h < L.heads; ++h)
    min_tiles = std::min<int>(min_tiles, (int)(L.tile_off[h + 1] - L.tile_off[h]));
  const int lockstep = min_tiles >= kLockstepTiles;
  unsigned G = (unsigned)(lockstep ? lockstep_grid(L) : L.tile_off[L.heads]);
  ClaimPlan plan{};
  if (claim != nullptr) {
    // the last tenth of every XCD's run is claimed; each XCD gets spare
    // workgroups for twice its own tail, to take over other XCDs' tails
    int most = 0;
    const int64_t G_all = L.tile_off[L.heads];
    for (int x = 0; x < 8; ++x) {
      int64_t len = G_all / 8 + (x < G_all % 8 ? 1 : 0);
      if (lockstep) {
        len = 0;
        for (int h = 0; h < L.heads; ++h) {
          const int64_t n = L.tile_off[h + 1] - L.tile_off[h];
          len += n * (x + 1) / 8 - n * x / 8;
        }
      }
      plan.len[x] = (int)len;
      plan.fixed[x] = (int)(len - (len + 9) / 10);
      most = std::max(most, plan.fixed[x] + 2 * (plan.len[x] - plan.fixed[x]));
    }
    G = 8u * (unsigned)most;
    hipLaunchKernelGGL(attn_claim_reset_kernel, dim3(1), dim3(64), 0, s, claim);
  }
  if (L.d == 128) {
    hipLaunchKernelGGL((sparse_attn_fwd_kernel<128, 128, TOK>), dim3(G), dim3(256), 0, s,
                       L, (const __bf16*)q, (const __bf16*)k, (const __bf16*)vt, row_ptr, col_idx,
                       scale_log2, (__bf16*)o, lse, lockstep, claim, plan);
  } else {
    hipLaunchKernelGGL((sparse_attn_fwd_kernel<64, 64, TOK>), dim3(G), dim3(128), 0, s, L,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)vt, row_ptr, col_idx,
                       scale_log2, (__bf16*)o, lse, lockstep, claim, plan);
  }
}
}  // namespace

int launch_sparse_attn(const DevLayout& L, const void* q, const void* k, const void* vt,
                       const int32_t* row_ptr, const int32_t* col_idx, float sm_scale, void* o,
                       float* lse, bool tokens, int* claim, hipStream_t s) {
  if (L.tile_off[L.heads] == 0) return VEDA_OK;
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  if (tokens)
    launch_attn<true>(L, q, k, vt, row_ptr, col_idx, scale_log2, o, lse, claim, s);
  else
    launch_attn<false>(L, q, k, vt, row_ptr, col_idx, scale_log2, o, lse, claim, s);
  return launch_status();
}

}  // namespace veda
