// fa2_fwd_4wave.h -- fused exact-attention forward pass for gfx950, four
// wavefronts per workgroup.  Used for head dim 256, whose unnormalised output
// (128 fp32 registers per lane) leaves room for one wavefront per SIMD only.
//
// One workgroup owns kBr = 128 query rows of one (batch, head) and streams the
// key/value tiles of that head through LDS, kBc = 64 keys at a time; the N x N
// score matrix never leaves registers.  From the pages:
//  * query tiles outside, key/value tiles inside; Q loaded once, O written once
//    ("6.2 FlashAttention V2 in depth", section 2.2); the grid runs over
//    (query tile x head x batch) ("FlashAttention-2: Where the Second 2x
//    Actually Comes From", section "Parallelism over sequence length");
//  * split-Q: each wavefront owns 32 whole query rows ("6.2 FlashAttention V2
//    in depth", section 4.2);
//  * online softmax with an unnormalised accumulator divided once at the end,
//    and L = m + log l per row (same page, sections 3.2, 6.1, 7.1);
//  * causal block classes: skip, mask on the diagonal, plain below it (same
//    page, section 5.3).
// gfx950 mapping: S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16, so each
// lane holds 16 keys of one query per 32x32 block (row max and sum are in-lane
// plus one v_permlane32_swap); V^T fragments come from the row-major V tile via
// ds_read_b64_tr_b16; K and V tiles alternate in two single LDS buffers filled
// by global_load_lds (the next K tile streams under softmax and P.V, the next V
// tile under the next S); K is stored in 16-row blocks and V with XOR-swizzled
// chunks, both for conflict-free reads.
#pragma once

#include <type_traits>

#include "fa2_common.h"

namespace fa2 {
namespace w4 {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;  // query rows per workgroup
constexpr int kBc = 64;           // keys per K/V tile

// LDS tile layouts (head dim D = 256: 32 chunks of 16 bytes per row).
//  K: 256-byte blocks, block (row / 16, chunk) at index (row / 16) * CPR + chunk
//     holding one chunk of 16 consecutive rows.  The A-operand read of 16 lanes
//     (16 rows, one chunk) covers one whole block, so it is free of bank
//     conflicts, and each lane reads at one base address plus an immediate.
//  V: row-major, the chunk index of row r XOR-swizzled by 4 * (r % 4): a
//     transposed read touches 4 consecutive rows x 64 bytes per half wave, and
//     the swizzle puts those 4 rows in 4 distinct 64-byte bank windows.
__device__ __forceinline__ int swz_v(int row) { return (row & 3) << 2; }

// Issue the global -> LDS copy of one kBc x D K tile (rows kv0.., clamped to
// N - 1).  Copy instruction t of a wave fills the 1 KB at q = t * kWaves + wave,
// blocks 4q .. 4q + 3: lane i copies row 16 * ((4q + i / 16) / CPR) + i % 16 at
// chunk (4q + i / 16) % CPR.
template <int D>
__device__ __forceinline__ void load_k_tile(const uint16_t* __restrict__ kh, FA2_LDS uint16_t* dst, int kv0, int N,
                                            int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int kPerWave = kBc * CPR / (64 * kWaves);
#pragma unroll
  for (int t = 0; t < kPerWave; ++t) {
    const int q = t * kWaves + wave;
    const int b = 4 * q + (lane >> 4);
    const int row = 16 * (b / CPR) + (lane & 15);
    const int grow = min(kv0 + row, N - 1);
    dma16(kh + (int64_t)grow * D + (b % CPR) * 8, dst + q * 512);
  }
}
// The same for an e4m3 K tile (D bytes per row, CPR = D / 16 chunks).
template <int D>
__device__ __forceinline__ void load_k_tile_fp8(const char* __restrict__ kh, FA2_LDS uint16_t* dst, int kv0, int N,
                                                int wave, int lane) {
  constexpr int CPR = D / 16;
  constexpr int kPerWave = kBc * CPR / (64 * kWaves);
#pragma unroll
  for (int t = 0; t < kPerWave; ++t) {
    const int q = t * kWaves + wave;
    const int b = 4 * q + (lane >> 4);
    const int row = 16 * (b / CPR) + (lane & 15);
    const int grow = min(kv0 + row, N - 1);
    dma16(kh + (int64_t)grow * D + (b % CPR) * 16, dst + q * 512);
  }
}

// The same for a V tile (row-major, swizzled): each instruction of a wave fills
// 64 consecutive 16-byte LDS slots; slot s holds logical chunk
// (s % CPR) ^ swz_v(row) of row s / CPR.
template <int D>
__device__ __forceinline__ void load_v_tile(const uint16_t* __restrict__ vh, FA2_LDS uint16_t* dst, int kv0, int N,
                                            int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int kPerWave = kBc * CPR / (64 * kWaves);
#pragma unroll
  for (int t = 0; t < kPerWave; ++t) {
    const int s0 = (t * kWaves + wave) * 64;
    const int s = s0 + lane;
    const int row = s / CPR;
    const int ch = (s % CPR) ^ swz_v(row);
    const int grow = min(kv0 + row, N - 1);
    dma16(vh + (int64_t)grow * D + ch * 8, dst + s0 * 8);
  }
}

template <int kDType, int D, int kMask>
__global__ __launch_bounds__(kThreads, D == 256 ? 1 : 2) void fa2_fwd_4wave(FwdArgs a) {
  constexpr bool kCausal = kMask == kMaskCausal;
  constexpr bool kGeneral = kMask == kMaskGeneral || kMask == kMaskSegments;
  constexpr bool kSeg = kMask == kMaskSegments;
  // fp8 instances: S = K Q^T on the fp8 MFMA from e4m3 Q and K (one byte per
  // element); V, P and O stay 16-bit.
  constexpr bool kQK8 = kDType == kFp8Fp16 || kDType == kFp8Bf16;
  typedef Elem<kDType & 1> E;
  typedef typename E::V8 V8;
  typedef std::conditional_t<kQK8, i32x8, V8> QF;  // one S operand fragment of Q
  constexpr int kEbK = kQK8 ? 1 : 2;                 // bytes per element of Q and K
  constexpr int CPR = D / 8;                          // 16-byte chunks per V row
  constexpr int CPRK = D * kEbK / 16;                 // 16-byte chunks per K row
  constexpr int KS = kQK8 ? D / 64 : D / 16;          // MFMA k-steps of S = K Q^T
  constexpr int DB = D / 32;  // 32-wide blocks of the output columns
  constexpr int kLoads = kBc * CPR / (64 * kWaves);    // V copies per wave per tile
  constexpr int kLoadsK = kBc * CPRK / (64 * kWaves);  // K copies per wave per tile
  constexpr float kNegInf = -__builtin_huge_valf();
  static_assert(D == 256, "the four-wave kernel serves head dim 256");

  __shared__ __attribute__((aligned(1024))) uint16_t sK_[kBc * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sV_[kBc * D];
  FA2_LDS uint16_t* const sK = (FA2_LDS uint16_t*)sK_;
  FA2_LDS uint16_t* const sV = (FA2_LDS uint16_t*)sV_;
  __shared__ int red_[kSeg ? 2 * kWaves : 2];
  // Segment ids of the keys of the current and of the next K tile.
  __shared__ __attribute__((aligned(16))) int seg_[kSeg ? 2 * kBc : 4];
  FA2_LDS int* const sSeg = (FA2_LDS int*)seg_;
  // Copies in flight per wave for one K tile: its rows, plus under segment ids
  // the keys' ids (copied by every wave, so the counts stay uniform).
  constexpr int kKLoads = kLoadsK + (kSeg ? 1 : 0);

  const int N = a.N;
  int bh, qtile;
  wg_to_tile(a, kCausal || (kGeneral && a.grow), bh, qtile);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hl = lane >> 5;   // which half of the wave
  const int col = lane & 31;  // query column of S^T / O^T held by this lane
  const int q_row0 = qtile * kBr + wave * 32;
  const int my_q = q_row0 + col;
  const int64_t head_off = (int64_t)bh * N * D;
  const uint16_t* __restrict__ kh = a.k + head_off;
  const char* __restrict__ kh8 = (const char*)a.k + head_off;  // e4m3 K of this head
  const uint16_t* __restrict__ vh = a.v + head_off;
  // Score multiplier in log2 units (the fp8 instances fold in the descales).
  float c2 = a.c2;
  if constexpr (kQK8) {
    if (a.descale_q) c2 *= a.descale_q[bh];
    if (a.descale_k) c2 *= a.descale_k[bh];
  }

  // Key tiles: step st of the loop visits tile tile_of(st), st < nt (as in the
  // eight-wave kernel: tiles 0 .. nt-1 without a general mask, the runs of
  // general_runs with one).
  int nt, run_a0 = 0, run_na = 0, run_b0 = 0;
  const int* __restrict__ segb = nullptr;  // this batch's segment ids
  int seg_q = 0;
  if constexpr (kGeneral) {
    const int q0 = qtile * kBr, q1 = min(N, q0 + kBr) - 1;
    int kf = 0, kl = N - 1;
    if constexpr (kSeg) {
      segb = a.seg + (int64_t)(bh / a.H) * N;
      seg_q = segb[min(my_q, N - 1)];
      const TileRuns all = general_runs(a, q0, q1, 0, N - 1, kBc);
      const int lo = all.na > 0 ? 0 : all.b0 * kBc;
      const int hi = min(N - 1, (all.b0 + all.nb) * kBc - 1);
      segment_span<kWaves>(segb, q0, q1, lo, hi, (FA2_LDS int*)red_, kf, kl);
    }
    const TileRuns r = general_runs(a, q0, q1, kf, kl, kBc);
    run_a0 = r.a0;
    run_na = r.na;
    run_b0 = r.b0;
    nt = r.na + r.nb;
  } else {
    const int kv_end = kCausal ? min(N, (qtile + 1) * kBr) : N;
    nt = (kv_end + kBc - 1) / kBc;
  }
  auto tile_of = [&](int step) __attribute__((always_inline)) {
    if constexpr (kGeneral) return step < run_na ? run_a0 + step : run_b0 + (step - run_na);
    else return step;
  };
  // With segment ids: when all 32 rows of this wave share one id (seg_w), a
  // tile's class follows from a comparison of each key's id with it.
  bool rows_one_seg = false;
  int seg_w = 0;
  if constexpr (kSeg) {
    seg_w = __builtin_amdgcn_readfirstlane(seg_q);
    rows_one_seg = __all(seg_q == seg_w);
  }

  auto load_k = [&](int kv0, int st) __attribute__((always_inline)) {
    if constexpr (kQK8) load_k_tile_fp8<D>(kh8, sK, kv0, N, wave, lane);
    else load_k_tile<D>(kh, sK, kv0, N, wave, lane);
    if constexpr (kSeg) dma4(segb + min(kv0 + lane, N - 1), sSeg + (st & 1) * kBc);
  };

  // First K and V tiles start streaming before anything else.
  load_k(tile_of(0) * kBc, 0);
  load_v_tile<D>(vh, sV, tile_of(0) * kBc, N, wave, lane);

  // Q fragments (B operand of S^T = K Q^T), loaded once and kept in registers.
  // They are consumed right here so that the compiler's own wait for them
  // happens once, outside the loop (it also covers the two tile copies above).
  QF qf[KS];
  if constexpr (kQK8) {
    // Lane (hl, col): bytes 64 ks + 32 hl .. + 31 of its query row.
    const char* qp = (const char*)a.q + head_off + (int64_t)min(my_q, N - 1) * D + 32 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 lo = *(const u32x4*)(qp + 64 * ks);
      const u32x4 hi = *(const u32x4*)(qp + 64 * ks + 16);
      // (two 128-bit operands: a 256-bit "v" operand is invalid for the host pass)
      asm volatile("" ::"v"(lo), "v"(hi));
      qf[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  } else {
    const uint16_t* qp = a.q + head_off + (int64_t)min(my_q, N - 1) * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_bit_cast(V8, *(const u32x4*)(qp + 16 * ks));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = kNegInf;  // reference max of this lane's query row (log2 units)
  float l_part = 0.f;     // this lane's share of the row sum

  // Operand reads run as pipelines kPipe fragments ahead of the MFMAs that use
  // them.  The reads of a loop cannot move above it (the wait-and-barrier
  // before it clobbers memory); a scheduling fence after each loop keeps them
  // from sinking into the code that follows, where the compiler would hold
  // every read of a phase at once (a register quad each) and spill.
  // Consecutive MFMAs use different accumulators.
  constexpr int kPipe = 4;
  V8 fr[kPipe];
  // S^T = K Q^T, fragment f: key block kb = f % 2, k-step ks = f / 2; lane
  // (hl, col) reads row 32 kb + col, chunk 2 ks + hl of the K tile.  e4m3: an
  // operand is two 16-byte halves, fragments f = 2 m + h with kb = m % 2,
  // ks = m / 2, chunk 4 ks + 2 hl + h.
  const uint32_t kbase = opaque_vgpr((uint32_t)(size_t)sK +
                                     (uint32_t)(((((col >> 4) * CPRK) + (kQK8 ? 2 * hl : hl)) << 8) + ((col & 15) << 4)));
  auto k_frag = [&](int f) __attribute__((always_inline)) {
    uint32_t ad;
    if constexpr (kQK8) {
      const int m = f >> 1;
      ad = kbase + (uint32_t)(((2 * (m & 1) * CPRK) + 4 * (m >> 1) + (f & 1)) << 8);
    } else {
      ad = kbase + (uint32_t)(((2 * (f & 1) * CPRK) + 2 * (f >> 1)) << 8);
    }
    return __builtin_bit_cast(V8, *(const FA2_LDS u32x4*)(size_t)ad);
  };
  // O^T += V^T P^T, fragment f: key block c = f / DB, output block db = f % DB.
  // Lane (g, L) = (lane / 16, lane % 16) takes keys kr = 16 c + 4 (g / 2) + L / 4
  // and kr + 8, columns 32 db + 16 (g % 2) + 4 (L % 4) .. + 3, from the
  // swizzled V tile: chunk 4 db + y with y = 2 (g % 2) + (L % 4) / 2 lands at
  // 4 (db ^ x) + y, x = kr % 4 = L / 4, so each lane keeps one base address per
  // value of db % 4 and everything else is an immediate.
  uint32_t vbase[4];
  {
    const int g = lane >> 4, L = lane & 15;
    const int x = L >> 2, y = 2 * (g & 1) + ((L & 3) >> 1);
    const uint32_t lane_part = (uint32_t)((4 * (g >> 1) + x) * CPR * 16 + 16 * y + 8 * (L & 1));
#pragma unroll
    for (int j = 0; j < 4; ++j) vbase[j] = opaque_vgpr((uint32_t)(size_t)sV + lane_part + (uint32_t)(64 * (j ^ x)));
  }
  auto v_frag = [&](int f) __attribute__((always_inline)) {
    const int c = f / DB, db = f % DB;
    const uint32_t ad = vbase[db & 3] + (uint32_t)(16 * c * CPR * 16 + 64 * (db & 4));
    const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)(size_t)ad);
    const i16x4 t2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)(size_t)(ad + 8 * CPR * 16));
    const u32x2 w1 = __builtin_bit_cast(u32x2, t1);
    const u32x2 w2 = __builtin_bit_cast(u32x2, t2);
    return __builtin_bit_cast(V8, u32x4{w1[0], w1[1], w2[0], w2[1]});
  };
  constexpr int kNs = kQK8 ? 4 * KS : 2 * KS;  // S fragments
  constexpr int kNpv = (kBc / 16) * DB;   // P.V fragments

  for (int st = 0; st < nt; ++st) {
    const int kv0 = tile_of(st) * kBc;
    // Wave-uniform classification of this tile for this wave's 32 rows.
    bool active = !kCausal || kv0 <= q_row0 + 31;
    bool need_mask = (kv0 + kBc > N) || (kCausal && kv0 + kBc - 1 > q_row0);
    if constexpr (kGeneral) {
      const int k1 = kv0 + kBc - 1, qa = q_row0, qb = q_row0 + 31;
      active = !(kv0 >= a.prefix && ((a.wr >= 0 && kv0 > qb + a.wr) || (a.wl >= 0 && k1 < qa - a.wl)));
      need_mask = !(k1 < N &&
                    (k1 < a.prefix || ((a.wl < 0 || kv0 >= qb - a.wl) && (a.wr < 0 || k1 <= qa + a.wr))));
    }

    wait_vm_barrier<kLoads>();  // K_j has landed (V_j may still be in flight)
    f32x16 s[2];
    if (active) {
      s[0] = f32x16{};
      s[1] = f32x16{};
#pragma unroll
      for (int i = 0; i < kPipe; ++i) fr[i] = k_frag(i);
#pragma unroll
      for (int f = 0; f < kNs; ++f) {
        if constexpr (kQK8) {
          // An fp8 MFMA takes the fragment pair (f - 1, f): issue it on the
          // second half, and reload the pair's slots only then.
          if (f & 1) {
            const int m = f >> 1;
            const u32x4 lo = __builtin_bit_cast(u32x4, fr[(f - 1) % kPipe]);
            const u32x4 hi = __builtin_bit_cast(u32x4, fr[f % kPipe]);
            const i32x8 ka = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                              (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            s[m & 1] = mfma_fp8(ka, qf[m >> 1], s[m & 1]);
            if (f - 1 + kPipe < kNs) fr[(f - 1) % kPipe] = k_frag(f - 1 + kPipe);
            if (f + kPipe < kNs) fr[f % kPipe] = k_frag(f + kPipe);
          }
        } else {
          s[f & 1] = E::mfma(fr[f % kPipe], qf[f >> 1], s[f & 1]);
          if (f + kPipe < kNs) fr[f % kPipe] = k_frag(f + kPipe);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_done_barrier();  // every wave is done with sK
    // The prefetch is issued on every step (the last step re-reads its own
    // tile, which nobody consumes) so that the number of loads in flight is the
    // same on every path through the loop.
    const int kv_next = st + 1 < nt ? tile_of(st + 1) * kBc : kv0;
    load_k(kv_next, st + 1);

    // Under segment ids: no key of the tile shares the rows' one id (nothing
    // survives), or every key does (the ids need no comparison).
    bool seg_all = false;
    const FA2_LDS int* sk = sSeg + (st & 1) * kBc;
    if constexpr (kSeg) {
      if (rows_one_seg) {
        const int seg_k = sk[lane];
        seg_all = __all(seg_k == seg_w);
        active = active && __any(seg_k == seg_w);
      }
      if (!seg_all) need_mask = true;
    }
    const bool generic = need_mask || !(c2 > 0.f);

    uint32_t pk[2][8];  // probabilities, packed pairs, B-operand order
    if (active) {
      float mul = c2;
      if (generic) {
        // Scale first, then mask: t = -inf for keys past N or after the query.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          u32x4 sg[4] = {};
          if (kSeg && !seg_all) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) sg[g4] = *(const FA2_LDS u32x4*)(sk + 32 * kb + 8 * g4 + 4 * hl);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
            bool masked = key >= N || (kCausal && key > my_q);
            if constexpr (kGeneral) {
              masked = key >= N ||
                       !(key < a.prefix || ((a.wl < 0 || key >= my_q - a.wl) && (a.wr < 0 || key <= my_q + a.wr)));
              if (kSeg && !seg_all) masked = masked || (int)sg[r >> 2][r & 3] != seg_q;
            }
            const float t = s[kb][r] * c2;
            s[kb][r] = masked ? kNegInf : t;
          }
        }
        mul = 1.f;
      }
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = max_pair32(mx);
      const float m_tile = mx * mul;
      const bool need = m_tile > m_run + kTau;
      if (__any(need)) {
        const float m_new = need ? m_tile : m_run;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        m_run = m_new;
      }
      const float m_use = m_run == kNegInf ? 0.f : m_run;
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], mul, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 1], mul, -m_use));
          rs[(r >> 1) & 3] += p0 + p1;
          pk[kb][r >> 1] = E::pack2(p0, p1);
        }
      }
      l_part += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    }

    wait_vm_barrier<kKLoads>();  // V_j has landed (K_{j+1} may be in flight)
    if (active) {
#pragma unroll
      for (int i = 0; i < kPipe; ++i) fr[i] = v_frag(i);
#pragma unroll
      for (int f = 0; f < kNpv; ++f) {
        const int c = f / DB;
        const u32x4 bw = {pk[c >> 1][4 * (c & 1) + 0], pk[c >> 1][4 * (c & 1) + 1], pk[c >> 1][4 * (c & 1) + 2],
                          pk[c >> 1][4 * (c & 1) + 3]};
        o[f % DB] = E::mfma(fr[f % kPipe], __builtin_bit_cast(V8, bw), o[f % DB]);
        if (f + kPipe < kNpv) fr[f % kPipe] = v_frag(f + kPipe);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_done_barrier();  // every wave is done with sV
    load_v_tile<D>(vh, sV, kv_next, N, wave, lane);
  }
  // No LDS write may still be in flight when the workgroup retires.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Epilogue: one division per row, logsumexp in natural-log units.
  const float l_row = sum_pair32(l_part);
  const float inv = 1.f / l_row;
  if (my_q < N) {
    uint16_t* op = a.o + head_off + (int64_t)my_q * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dim = 32 * db + 8 * r4 + 4 * hl;
        const u32x2 wv = {E::pack2(o[db][4 * r4 + 0] * inv, o[db][4 * r4 + 1] * inv),
                          E::pack2(o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv)};
        *(u32x2*)(op + dim) = wv;
      }
    }
    if (hl == 0) a.lse[(int64_t)bh * N + my_q] = (m_run + __log2f(l_row)) * kLn2;
  }
}

}  // namespace w4
}  // namespace fa2
