// fa2_fwd_8wave.h -- fused exact-attention forward pass for gfx950 with eight
// wavefronts per workgroup in two alternating groups (head dims 64 and 128).
//
// What the pages fix, and where it lives here:
//  * Query tiles outside, key/value tiles inside; Q is loaded once and O written
//    once per query tile ("6.2 FlashAttention V2 in depth", section 2.2).  The
//    grid covers (query tile x head x batch), so one long sequence at batch 1
//    still fills the chip ("FlashAttention-2: Where the Second 2x Actually Comes
//    From", section "Parallelism over sequence length").
//  * Split-Q: each wavefront owns 32 whole query rows and sees every key of the
//    tile, so row max and row sum never cross wavefronts ("6.2 FlashAttention V2
//    in depth", section 4.2).
//  * Online softmax with an unnormalised output, divided by the row sum once
//    after the key loop, and the per-row statistic L = m + log l (same page,
//    sections 3.2, 6.1 and 7.1).
//  * Causal block classes: tiles past the query tile are never visited, tiles
//    crossing the diagonal are masked element by element (same page, 5.3).
//
// gfx950 design (the pages' A100 kernel is prior art, not the blueprint):
//  * Work split.  A workgroup owns 256 query rows.  Waves 0-3 (group 0) and
//    4-7 (group 1) put one wave of each group on every SIMD.  Each step of the
//    key loop has two phases separated by workgroup barriers; in every phase
//    one group runs its matrix products (P.V of the previous tile, then
//    S = K Q^T of the current one) while the other runs the softmax of its
//    scores, so MFMA and VALU work of the two waves on a SIMD overlap.  The
//    same overlap idea is what the pages credit to the Hopper redesign
//    ("Flash Attention: Memory-Efficient Attention at Scale", section "Flash
//    Attention 3"); here it comes from wave scheduling alone.
//  * Products.  Both run on v_mfma_f32_32x32x16 with fp32 accumulation, scores
//    transposed (S^T = K Q^T): a lane holds 16 keys of one query per 32x32 block,
//    so row max and row sum are in-lane plus one v_permlane32_swap.  O^T += V^T P^T
//    takes the probabilities straight from the score registers as its B operand:
//    the rows of each K tile are stored in LDS with bits 2 and 3 of the row index
//    swapped, which makes the 8 keys a lane holds for one MFMA k-step consecutive.
//  * Data movement.  K and V tiles go global -> LDS with global_load_lds (no
//    register staging), two tiles ahead, into three K and three V slots.  Each V
//    tile is transposed once per workgroup (ds_read_b64_tr_b16 + ds_write_b64,
//    half by each group in its softmax phase) into one of two V^T slots, so the
//    P.V operand reads are full-rate ds_read_b128.  16-byte chunks are
//    XOR-swizzled per row so that every read and write instruction is free of
//    bank conflicts.
//  * Softmax.  exp2 with the multiplier and log2(e) folded into one FMA; the
//    row sum adds the fp32 weights with plain adds (v_dot2 would be cheaper in
//    instructions, but it stalls behind the other wave's MFMAs on the same
//    SIMD).  The reference max of a row moves only when a weight would exceed
//    2^kTau, so the O rescale is rare and the steady state computes no row max
//    at all (the weights' own sum shows that none is too large); the result is
//    the same mathematically, since O and l share the reference.
//  * Scheduling.  Workgroups are remapped so each XCD walks a contiguous range
//    of heads (L2 reuse of K/V); causal query tiles go heaviest first.
#pragma once

#include <type_traits>

#include "fa2_common.h"

namespace fa2 {
namespace w8 {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;  // query rows per workgroup
constexpr int kBc = 64;           // keys per tile
constexpr int kKSlots = 3;        // K tiles resident or in flight
constexpr int kVSlots = 3;        // row-major V tiles resident or in flight
constexpr int kTSlots = 2;        // transposed V tiles

// LDS row i of a K tile holds key sigma(i) of the tile (bits 2 and 3 swapped).
__device__ __forceinline__ int sigma(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

// LDS tile layouts.  Every tile is a sequence of 256-byte blocks; a block holds
// one 16-byte chunk of 16 consecutive rows, and block (row / 16, chunk) sits at
// index (row / 16) * chunks_per_row + chunk.
//  * K (64 rows x D) and V^T (D rows x 64 keys): an operand read of 16 lanes
//    (16 consecutive rows, one chunk) covers one whole block, so every read is
//    free of bank conflicts without any swizzle, and each lane's address is one
//    base register plus an immediate that depends on (block row, chunk) only.
//  * V staging (64 rows x D, read by ds_read_b64_tr_b16): the 16-byte slot of
//    row r within its block is (r % 16) ^ (4 * (chunk % 4)), which spreads the
//    4 rows x 4 chunks read by one half wave over 16 distinct bank groups.
// One copy instruction of a wave fills 1 KB = 4 consecutive blocks, i.e. 16 rows
// x 4 chunks (64 contiguous bytes of each of 16 rows in global memory).
template <int CPR> __device__ __forceinline__ uint32_t k_byte(int row, int chunk) {
  return (uint32_t)((((row >> 4) * CPR + chunk) << 8) + ((row & 15) << 4));
}
template <int CPR> __device__ __forceinline__ uint32_t vs_byte(int row, int chunk) {
  return (uint32_t)((((row >> 4) * CPR + chunk) << 8) + ((((row & 15) ^ (4 * (chunk & 3)))) << 4));
}

template <int kDType, int D, int kMask>
__global__ __launch_bounds__(kThreads, 1) void fa2_fwd_8wave(FwdArgs a) {
  constexpr bool kCausal = kMask == kMaskCausal;
  constexpr bool kGeneral = kMask == kMaskGeneral || kMask == kMaskSegments;
  constexpr bool kSeg = kMask == kMaskSegments;
  // fp8 instances: S = K Q^T on the fp8 MFMA from e4m3 Q and K; V, P and O stay
  // 16-bit, so P.V and everything after the scores are those of the 16-bit
  // instances.
  constexpr bool kQK8 = kDType == kFp8Fp16 || kDType == kFp8Bf16;
  typedef Elem<kDType & 1> E;  // P.V and the output
  typedef typename E::V8 V8;
  typedef std::conditional_t<kQK8, i32x8, V8> QF;  // one S operand fragment of Q
  constexpr int kEbK = kQK8 ? 1 : 2;                 // bytes per element of Q and K
  constexpr int CPR = D / 8;                          // 16-byte chunks per V row
  constexpr int CPRK = D * kEbK / 16;                 // 16-byte chunks per K row
  constexpr int KS = kQK8 ? D / 64 : D / 16;          // k-steps of S = K Q^T
  constexpr int DB = D / 32;                          // 32-wide output column blocks
  constexpr int kTile = kBc * D;                      // elements of one K, V or V^T slot
  constexpr int kLoads = kBc * CPR / (64 * kWaves);   // copy instructions per wave per V tile
  // 1 KB copies per K tile.  With fewer than one per wave (e4m3 K at d = 64:
  // 4 KB per tile) waves w and w + kKCopies copy the same rows (the same bytes
  // to the same place), so every wave still issues one copy per tile and the
  // copy counts the waits rely on stay uniform.
  constexpr int kKCopies = kBc * CPRK / 64;
  constexpr int kLoadsK = kKCopies < kWaves ? 1 : kKCopies / kWaves;  // ... per K tile
  constexpr int kRowStep = 4 * 16 * kWaves / CPR;     // rows covered by one instruction of all waves (V)
  constexpr int kRowStepK = 4 * 16 * kWaves / CPRK;   // ... (K)
  constexpr float kNegInf = -__builtin_huge_valf();
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(kKCopies >= kWaves || kWaves % kKCopies == 0, "duplicated K copies");
  static_assert(kLoads >= 1 && kLoads * 64 * kWaves == kBc * CPR, "tile copy split");
  static_assert(kLoadsK >= 1 && (kKCopies < kWaves || kLoadsK * 64 * kWaves == kBc * CPRK), "tile copy split");
  // Copy instructions per wave per tile: K and V, plus the keys' segment ids
  // under segment ids (issued by every wave, so the counts stay uniform).
  constexpr int kTileLoads = kLoadsK + kLoads + (kSeg ? 1 : 0);
  constexpr int kSegSlots = 4;  // segment ids of tiles st..st+2 stay readable while group 1 reads st-1

  __shared__ __attribute__((aligned(1024))) uint16_t smem_[(kKSlots + kVSlots + kTSlots) * kTile];
  FA2_LDS uint16_t* const sK = (FA2_LDS uint16_t*)smem_;
  FA2_LDS uint16_t* const sVs = sK + kKSlots * kTile;
  FA2_LDS uint16_t* const sVt = sVs + kVSlots * kTile;
  __shared__ __attribute__((aligned(16))) int seg_[kSeg ? kSegSlots * kBc : 4];
  FA2_LDS int* const sSeg = (FA2_LDS int*)seg_;
  __shared__ int red_[kSeg ? 2 * kWaves : 2];

  const int N = a.N;
  int bh, qtile;
  wg_to_tile(a, kCausal || (kGeneral && a.grow), bh, qtile);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: products first in each step, 1: softmax first
  const int lane = tid & 63;
  const int hl = lane >> 5;
  const int col = lane & 31;
  const int q_row0 = qtile * kBr + wave * 32;
  const int my_q = q_row0 + col;
  const int64_t head_off = (int64_t)bh * N * D;
  const char* __restrict__ kh = (const char*)a.k + head_off * kEbK;  // K of this head, bytes
  const uint16_t* __restrict__ vh = a.v + head_off;
  // Score multiplier in log2 units (the fp8 instances fold in the descales).
  float c2 = a.c2;
  if constexpr (kQK8) {
    if (a.descale_q) c2 *= a.descale_q[bh];
    if (a.descale_k) c2 *= a.descale_k[bh];
  }

  // Copy layout: instruction t of this wave fills the 1 KB at q = t*kWaves +
  // wave, i.e. blocks 4q..4q+3: rows 16*(4q / CPR) + 0..15 of chunks
  // (4q % CPR) + 0..3.  Lane i takes block 4q + i/16 and slot i % 16.  From one
  // t to the next only the block row moves (by kRowStep rows), so each lane
  // keeps one global byte offset per tensor and t and the tile move a
  // wave-uniform base.
  const int cch = (4 * wave) % CPR + (lane >> 4);     // chunk this lane copies
  const int crow = 16 * ((4 * wave) / CPR);          // first row of its block (t = 0)
  const int vr = crow + ((lane & 15) ^ (4 * (cch & 3)));  // V: row that lands in slot lane & 15
  const uint32_t voffV = (uint32_t)((vr * D + cch * 8) * 2);
  // The same for K with its own row length (CPRK chunks); LDS row krK holds
  // key sigma(krK).
  const int wk = kKCopies < kWaves ? wave % kKCopies : wave;  // this wave's K copy slot
  const int cchK = (4 * wk) % CPRK + (lane >> 4);
  const int krK = 16 * ((4 * wk) / CPRK) + (lane & 15);
  const uint32_t voffK = (uint32_t)(sigma(krK) * D * kEbK + cchK * 16);

  // Key tiles: step st of the loop visits tile tile_of(st), st < nt.  Without a
  // general mask those are tiles 0 .. nt-1 (under the causal mask up to the
  // rows' last key); a general mask visits the runs of general_runs, cut to the
  // keys whose segment ids can match.
  int nt, run_a0 = 0, run_na = 0, run_b0 = 0;
  const int* __restrict__ segb = nullptr;  // this batch's segment ids
  int seg_q = 0;                           // this lane's query's segment id
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

  // Copy instruction p (0 .. kTileLoads-1) of tile `step` into `slot`: under
  // segment ids first the keys' ids (every wave copies the same 256 bytes),
  // then the K rows, then the V rows.  (Issued one at a time every fourth MFMA
  // instead of together, the copies measured 1-1.5 % slower.)
  auto issue_tile_part = [&](int step, int slot, int p) __attribute__((always_inline)) {
    const int kv0 = tile_of(step) * kBc;
    if (kSeg && p == 0) {
      dma4(segb + min(kv0 + lane, N - 1), sSeg + (step % kSegSlots) * kBc);
      return;
    }
    const int t = p - (kSeg ? 1 : 0);
    if (t < kLoadsK) {
      FA2_LDS uint16_t* dk = sK + slot * kTile + (t * kWaves + wk) * 64 * 8;
      if (kv0 + kBc <= N) {
        dma16_sbase(kh + (int64_t)kv0 * D * kEbK + t * kRowStepK * D * kEbK, voffK, dk);
      } else {
        // Ragged last tile: rows past N re-read row N-1 (their scores are masked).
        const int gk = min(kv0 + sigma(krK + t * kRowStepK), N - 1);
        dma16(kh + (int64_t)gk * D * kEbK + cchK * 16, dk);
      }
    } else {
      const int tv = t - kLoadsK;
      FA2_LDS uint16_t* dv = sVs + slot * kTile + (tv * kWaves + wave) * 64 * 8;
      if (kv0 + kBc <= N) {
        dma16_sbase((const char*)(vh + (int64_t)kv0 * D) + tv * kRowStep * D * 2, voffV, dv);
      } else {
        const int gv = min(kv0 + vr + tv * kRowStep, N - 1);
        dma16(vh + (int64_t)gv * D + cch * 8, dv);
      }
    }
  };
  auto issue_tile = [&](int step, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < kTileLoads; ++p) issue_tile_part(step, slot, p);
  };

  // The V^T slot that the first product phase reads (with all-zero weights)
  // must hold finite values: fill it with zeros.
  {
    FA2_LDS u32x4* z = (FA2_LDS u32x4*)(sVt + ((kTSlots - 1) % kTSlots) * kTile);
#pragma unroll
    for (int i = tid; i < kTile / 8; i += kThreads) z[i] = u32x4{0u, 0u, 0u, 0u};
  }

  // Tile 0 starts streaming first; tile 1 (which repeats tile 0 if there is
  // only one: every step keeps the same number of copies in flight) follows
  // once Q has arrived, so that the wait for Q does not also wait for it.
  issue_tile(0, 0);

  // Q fragments (B operand of S^T = K Q^T), kept in registers for the whole
  // loop.  Consumed here so the compiler's wait for them stays out of the loop.
  QF qf[KS];
  if constexpr (kQK8) {
    // Lane (hl, col): bytes 64 ks + 32 hl .. + 31 of its query row.
    const char* qp = (const char*)a.q + head_off + (int64_t)min(my_q, N - 1) * D + 32 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 lo = *(const u32x4*)(qp + 64 * ks);
      const u32x4 hi = *(const u32x4*)(qp + 64 * ks + 16);
      // (128-bit operands: the host pass checks the constraint against the host
      // target, where a 256-bit "v" operand is not valid.)
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
  issue_tile(min(1, nt - 1), 1);

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = kNegInf;  // reference max of this lane's query row, log2 units
  float l_part = 0.f;     // this lane's share of the row sum
  f32x16 s[2];            // scores of one tile, between its S and softmax phases
  uint32_t pk[2][8];      // probabilities of one tile, between softmax and P.V

  // Tile classes for this wave's 32 rows: does any (row, key) pair survive the
  // mask (wave_active), and does every pair (softmax's need_mask)?  Under
  // segment ids wave_active also records whether every key of the tile shares
  // the rows' one id (seg_all), for softmax on the same step.
  bool seg_all = false;
  auto wave_active = [&](int step) __attribute__((always_inline)) {
    const int k0 = tile_of(step) * kBc;
    if constexpr (kGeneral) {
      const int qa = q_row0, qb = q_row0 + 31;
      bool act = !(k0 >= a.prefix && ((a.wr >= 0 && k0 > qb + a.wr) || (a.wl >= 0 && k0 + kBc - 1 < qa - a.wl)));
      seg_all = false;
      if (kSeg && rows_one_seg) {
        const int sk = sSeg[(step % kSegSlots) * kBc + lane];
        seg_all = __all(sk == seg_w);
        act = act && __any(sk == seg_w);
      }
      return act;
    } else {
      return !kCausal || k0 <= q_row0 + 31;
    }
  };

  // Operand addresses: lane (hl, col) reads row 32*kb + col, chunk 2*ks + hl of
  // K, and column 32*db + col, chunk 2*c + hl of V^T.
  const uint32_t kaddr0 = k_byte<CPRK>(col, kQK8 ? 2 * hl : hl);
  const uint32_t taddr0 = k_byte<kBc / 8>(col, hl);

  // The products of one phase run as one pipeline over their operand
  // fragments: loads run kPipe fragments ahead of the MFMAs that use them,
  // across the boundary between the two products, and the scheduling fences
  // keep the compiler from hoisting every load of the phase (a register quad
  // each).  The copy of a future K/V tile is issued from the middle of the
  // pipeline so that its address work hides under the MFMAs.  Consecutive MFMAs
  // use different accumulators (4 output blocks, 2 score blocks).
  //
  // P.V runs first, over the key blocks of the V^T tile in the order 32-47,
  // 48-63, 0-15, 16-31 (fragment f -> key block c = (f / DB + 2) % 4, output
  // block f % DB).  Keys 32-63 of a V^T tile are written by group 1 before the
  // middle barrier of the step that transposes it, so both groups may load the
  // first kPipe fragments before the barrier that opens their product phase
  // (prefetch): the barrier's wait then covers the load latency.
  constexpr int kPipe = 4;
  constexpr int kNpv = (kBc / 16) * DB;  // P.V fragments
  // S fragments: f -> (ks = f / 2, kb = f % 2); an fp8 S operand is two
  // 16-byte halves, loaded as consecutive fragments 2f and 2f + 1.
  constexpr int kNs = kQK8 ? 4 * KS : 2 * KS;
  static_assert(kPipe <= 2 * DB, "prefetched fragments must lie in keys 32-63");
  auto pv_c = [](int f) constexpr { return (f / DB + 2) % (kBc / 16); };
  V8 fr[kPipe];
  auto load_op = [&](uint32_t tbase, uint32_t kbase, int i) __attribute__((always_inline)) {
    uint32_t ad;
    if (i < kNpv) {
      ad = tbase + (uint32_t)((((i % DB) * 2 * (kBc / 8)) + 2 * pv_c(i)) << 8);
    } else if constexpr (kQK8) {
      const int f = (i - kNpv) >> 1, h = (i - kNpv) & 1;  // lane reads chunk 4 ks + 2 hl + h of row 32 kb + col
      ad = kbase + (uint32_t)((((f & 1) * 2 * CPRK) + 4 * (f >> 1) + h) << 8);
    } else {
      ad = kbase + (uint32_t)(((((i - kNpv) & 1) * 2 * CPRK) + 2 * ((i - kNpv) >> 1)) << 8);
    }
    return __builtin_bit_cast(V8, *(const FA2_LDS u32x4*)(size_t)ad);
  };
  auto tslot_base = [&](int tslot) __attribute__((always_inline)) {
    // One base register per operand; every fragment address is that base plus
    // an immediate offset.
    return opaque_vgpr((uint32_t)(size_t)(sVt + tslot * kTile) + taddr0);
  };
  auto prefetch = [&](int tslot) __attribute__((always_inline)) {
    const uint32_t tbase = tslot_base(tslot);
#pragma unroll
    for (int i = 0; i < kPipe; ++i) fr[i] = load_op(tbase, 0u, i);
  };
  // One product phase: O^T += V^T P^T for the V^T tile in slot tslot, then
  // S^T = K Q^T for the K tile in slot kslot.  Both always run: a step without a
  // P.V term has all-zero probabilities (pk), and scores nobody needs are simply
  // not used, which keeps a single code path (and register allocation) for the
  // loop.
  auto mfma_phase = [&](int tslot, int kslot, int copy_tile, int copy_slot, bool prefetched)
                        __attribute__((always_inline)) {
    const uint32_t tbase = tslot_base(tslot);
    const uint32_t kbase = opaque_vgpr((uint32_t)(size_t)(sK + kslot * kTile) + kaddr0);
    // The wave running products is preferred at instruction issue so that
    // its MFMAs are not held back by the other wave's softmax on the SIMD.
    __builtin_amdgcn_s_setprio(2);
    if (!prefetched) {
#pragma unroll
      for (int i = 0; i < kPipe; ++i) fr[i] = load_op(tbase, kbase, i);
    }
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int i = 0; i < kNpv + kNs; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i < kNpv) {
        const int c = pv_c(i);
        const u32x4 bw = {pk[c >> 1][4 * (c & 1) + 0], pk[c >> 1][4 * (c & 1) + 1], pk[c >> 1][4 * (c & 1) + 2],
                          pk[c >> 1][4 * (c & 1) + 3]};
        o[i % DB] = E::mfma(fr[i % kPipe], __builtin_bit_cast(V8, bw), o[i % DB]);
      } else if constexpr (kQK8) {
        // An fp8 MFMA takes the fragment pair (i - 1, i): issue it on the second
        // half, and reload the pair's slots only then.
        const int k = i - kNpv;
        if (k & 1) {
          const u32x4 lo = __builtin_bit_cast(u32x4, fr[(i - 1) % kPipe]);
          const u32x4 hi = __builtin_bit_cast(u32x4, fr[i % kPipe]);
          const i32x8 ka = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                            (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          s[(k >> 1) & 1] = mfma_fp8(ka, qf[k >> 2], s[(k >> 1) & 1]);
          if (i - 1 + kPipe < kNpv + kNs) fr[(i - 1) % kPipe] = load_op(tbase, kbase, i - 1 + kPipe);
        }
      } else {
        const int k = i - kNpv;
        s[k & 1] = E::mfma(fr[i % kPipe], qf[k >> 1], s[k & 1]);
      }
      if (i + kPipe < kNpv + kNs && !(kQK8 && i >= kNpv && ((i - kNpv) & 1) == 0))
        fr[i % kPipe] = load_op(tbase, kbase, i + kPipe);
      if (i == 6 && copy_tile >= 0) {
        __builtin_amdgcn_sched_barrier(0);
        issue_tile(copy_tile, copy_slot);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };
  auto zero_pk = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 8; ++r) pk[kb][r] = 0u;
  };

  // Half of V tile j (this group's share), staging -> V^T.  Wave w handles keys
  // 8w .. 8w+7 (group 0 the first 32 keys, group 1 the rest).  For each span of
  // 64 columns, two ds_read_b64_tr_b16 give lane (g, L) keys 8w + 0..3 and
  // 8w + 4..7 of column 16g + L, which one ds_write_b128 stores as a whole
  // 16-byte slot (each 16 lanes write 256 contiguous bytes).
  const int tg = lane >> 4;
  const int tl = lane & 15;
  const int tch = 2 * tg + ((tl & 3) >> 1);  // source chunk within a span
  const uint32_t trd0 = vs_byte<CPR>(8 * wave + (tl >> 2), tch) + 8 * (tl & 1);
  const uint32_t trd1 = vs_byte<CPR>(8 * wave + 4 + (tl >> 2), tch) + 8 * (tl & 1);
  const uint32_t twr0 = k_byte<kBc / 8>(16 * tg + tl, wave);
  u32x2 tv[D / 64][2];  // transposed V data between its read and its write
  auto transpose_read = [&](int j) __attribute__((always_inline)) {
    const uint32_t src = (uint32_t)(size_t)(sVs + (j % kVSlots) * kTile);
    const uint32_t a0 = opaque_vgpr(src + trd0), a1 = opaque_vgpr(src + trd1);
#pragma unroll
    for (int dq = 0; dq < D / 64; ++dq) {
      const uint32_t so = (uint32_t)(dq * 8 * 256);  // chunk + 8 per span
      tv[dq][0] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)(size_t)(a0 + so)));
      tv[dq][1] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)(size_t)(a1 + so)));
    }
  };
  auto transpose_write = [&](int j) __attribute__((always_inline)) {
    const uint32_t dst = opaque_vgpr((uint32_t)(size_t)(sVt + (j % kTSlots) * kTile) + twr0);
#pragma unroll
    for (int dq = 0; dq < D / 64; ++dq)
      *(FA2_LDS u32x4*)(size_t)(dst + (uint32_t)(dq * 32 * 256)) = u32x4{tv[dq][0][0], tv[dq][0][1], tv[dq][1][0], tv[dq][1][1]};
  };

  // Softmax of tile j into pk, updating the row statistics.  The reference max
  // m_run moves only when some weight would exceed 2^kTau, and a lane's share of
  // the tile's row sum bounds every weight it holds, so the steady state needs no
  // row max: the weights are formed against the current reference and accepted
  // when every lane's share is at most kSumCap (an overflowed exp fails the test
  // too).  Otherwise (and always on the first tile) the tile's row max decides
  // whether the reference moves, O and l are rescaled by 2^(old - new), and the
  // weights are formed again.
  auto softmax = [&](int step) __attribute__((always_inline)) {
    const int kv0 = tile_of(step) * kBc;
    bool need_mask = (kv0 + kBc > N) || (kCausal && kv0 + kBc - 1 > q_row0);
    if constexpr (kGeneral) {
      const int k1 = kv0 + kBc - 1, qa = q_row0, qb = q_row0 + 31;
      const bool full = k1 < N && (!kSeg || seg_all) &&
                        (k1 < a.prefix || ((a.wl < 0 || kv0 >= qb - a.wl) && (a.wr < 0 || k1 <= qa + a.wr)));
      need_mask = !full;
    }
    float mul = c2;
    if (kGeneral && need_mask) {
      // Key of element (kb, r) = kv0 + 8*hl + off with a constant off.
      const int base = kv0 + 8 * hl;
      const int lim_n = N - base;
      const int lim_p = a.prefix - base;
      const int lo_w = a.wl < 0 ? INT32_MIN / 2 : my_q - a.wl - base;
      const int hi_w = a.wr < 0 ? INT32_MAX / 2 : my_q + a.wr - base;
      const FA2_LDS int* sk = sSeg + (step % kSegSlots) * kBc + 8 * hl;
      const bool pos = c2 > 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
          u32x4 sg[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
          if (kSeg && !seg_all) {
            sg[0] = *(const FA2_LDS u32x4*)(sk + 32 * kb + 16 * h8);
            sg[1] = *(const FA2_LDS u32x4*)(sk + 32 * kb + 16 * h8 + 4);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int r = 8 * h8 + i;
            const int off = 32 * kb + 16 * h8 + i;
            bool ok = off < lim_n && (off < lim_p || (off >= lo_w && off <= hi_w));
            if (kSeg && !seg_all) ok = ok && (int)sg[i >> 2][i & 3] == seg_q;
            const float t = pos ? s[kb][r] : s[kb][r] * c2;
            s[kb][r] = ok ? t : kNegInf;
          }
        }
      }
      if (!pos) mul = 1.f;
    } else if (need_mask) {
      // Key of element (kb, r) = kv0 + 8*hl + off with a constant off; it is
      // allowed iff off < lim (key < N, and key <= query under the causal mask).
      const int base = kv0 + 8 * hl;
      int lim = N - base;
      if (kCausal) lim = min(lim, my_q + 1 - base);
      if (c2 > 0.f) {
        // -inf times a positive multiplier stays -inf: mask the raw scores.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 32 * kb + 16 * (r >> 3) + (r & 7);
            s[kb][r] = off < lim ? s[kb][r] : kNegInf;
          }
      } else {
        // Scale first, then mask.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 32 * kb + 16 * (r >> 3) + (r & 7);
            const float t = s[kb][r] * c2;
            s[kb][r] = off < lim ? t : kNegInf;
          }
        mul = 1.f;
      }
    }
    // Weights 2^(s*mul - m) of this lane's 32 scores, rounded into pk; returns
    // their fp32 sum (the unrounded weights), formed with 31 adds in four
    // independent chains.
    auto weights = [&](float m) __attribute__((always_inline)) {
      float ls[4];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int kb = e >> 3, r = 2 * (e & 7);
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], mul, -m));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 1], mul, -m));
        pk[kb][r >> 1] = E::pack2(p0, p1);
        if (e < 4) ls[e] = p0 + p1;
        else ls[e & 3] += p0 + p1;
      }
      return (ls[0] + ls[1]) + (ls[2] + ls[3]);
    };
    float lsum = 0.f;
    bool accepted = false;
    // The fast path needs a finite reference in every row: a row's reference
    // stays -inf until a tile holds one of its allowed keys.  Without a general
    // mask the first tile always does (key 0 is visible to every row).
    const bool fast = kGeneral ? __all(m_run != kNegInf) : step > 0;
    if (fast) {
      lsum = weights(m_run);
      accepted = __all(lsum <= kSumCap);
    }
    if (!accepted) {
      // Row max of the scaled scores (-inf for a row none of whose keys in this
      // tile is allowed).
      float mx = s[0][0] * mul;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r] * mul);
      const float m_tile = max_pair32(mx);
      const bool need = m_tile > m_run + kTau;
      if (!fast || __any(need)) {
        const float m_new = need ? m_tile : m_run;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        m_run = m_new;
        // A row still without an allowed key has only -inf scores: any finite
        // reference gives it zero weights.
        lsum = weights(kGeneral && m_run == kNegInf ? 0.f : m_run);
      }
    }
    l_part += lsum;
  };

  // Step st: both groups meet at the two barriers; in between, group 0 runs
  // [P.V(st-1), S(st)] then [softmax(st), transpose half of V(st)], and group 1
  // runs [softmax(st-1), transpose half of V(st)] then [P.V(st-1), S(st)].
  // Each wave copies its share of tile st+2 from inside its product phase:
  // tile st+2 goes to slot (st+2) % 3, which held tile st-1 (no longer read);
  // past the last tile the copy repeats tile nt-1 into that free slot, so that
  // every step keeps the same number of copies in flight.  Each group has its
  // own copy of the loop so that the compiler sees which registers stay live
  // across steps (pk for group 0, s for group 1); both copies execute the same
  // barriers in the same order.
  auto copy_tile_of = [&](int st) __attribute__((always_inline)) { return st < nt ? min(st + 2, nt - 1) : -1; };
  zero_pk();
  // The scheduling fences keep each phase's work on its own side of the
  // barriers (register-only arithmetic could otherwise move across them and
  // unbalance the two phases).
  if (grp == 0) {
    for (int st = 0; st <= nt; ++st) {
      // Tile st has landed for every wave (tile st+1 may still be in flight),
      // and every LDS access of the previous step is complete.
      __builtin_amdgcn_sched_barrier(0);
      wait_vm_lds_barrier<kTileLoads>();
      __builtin_amdgcn_sched_barrier(0);
      // The zeroed V^T slot read at st = 0 is visible only after this barrier.
      mfma_phase((st + kTSlots - 1) % kTSlots, st % kKSlots, copy_tile_of(st), (st + 2) % kKSlots, st > 0);
      __builtin_amdgcn_sched_barrier(0);
      lds_done_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (st < nt) {
        transpose_read(st);
        if (wave_active(st)) softmax(st);
        else zero_pk();
        transpose_write(st);
        __builtin_amdgcn_sched_barrier(0);
        prefetch(st % kTSlots);  // keys 32-63 of V^T(st), written by group 1
      } else {
        zero_pk();
      }
    }
  } else {
    for (int st = 0; st <= nt; ++st) {
      __builtin_amdgcn_sched_barrier(0);
      wait_vm_lds_barrier<kTileLoads>();
      __builtin_amdgcn_sched_barrier(0);
      if (st < nt) transpose_read(st);
      if (st >= 1 && wave_active(st - 1)) softmax(st - 1);
      else zero_pk();
      if (st < nt) transpose_write(st);
      __builtin_amdgcn_sched_barrier(0);
      prefetch((st + kTSlots - 1) % kTSlots);  // V^T(st-1): complete since the step's first barrier
      __builtin_amdgcn_sched_barrier(0);
      lds_done_barrier();
      __builtin_amdgcn_sched_barrier(0);
      mfma_phase((st + kTSlots - 1) % kTSlots, st % kKSlots, copy_tile_of(st), (st + 2) % kKSlots, true);
    }
  }
  // No LDS write may still be in flight when the workgroup retires.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Epilogue: one division per row, logsumexp in natural-log units.  A lane
  // holds 4-element pieces of one row, so O goes through LDS (free once every
  // wave has left the loop): each wave writes its 32 rows row-major, reads them
  // back 16 bytes per lane and stores whole rows, D * 2 contiguous bytes per
  // row and 1 KB per store instruction.  The wave's registers are released
  // only once its stores have read them, so the fewer, fuller stores also let
  // the next workgroup start sooner.
  const float l_row = sum_pair32(l_part);
  const float inv = 1.f / l_row;
  if (my_q < N && hl == 0) a.lse[(int64_t)bh * N + my_q] = (m_run + __log2f(l_row)) * kLn2;
  // Staging row stride: 16 bytes more than a row, which keeps the 16-byte reads
  // aligned and conflict-free; the 8-byte writes of a half wave meet 2-way
  // (about 0.05 % of the kernel's time on the long-context workload).
  constexpr int kRowB = D * 2 + 16;
  static_assert(kWaves * 32 * kRowB <= (int)sizeof(smem_), "O staging fits in the tile buffers");
  lds_done_barrier();  // every wave is done with the tile buffers
  FA2_LDS char* const stg = (FA2_LDS char*)smem_ + wave * 32 * kRowB;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int dim = 32 * db + 8 * r4 + 4 * hl;
      const u32x2 wv = {E::pack2(o[db][4 * r4 + 0] * inv, o[db][4 * r4 + 1] * inv),
                        E::pack2(o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv)};
      *(FA2_LDS u32x2*)(stg + col * kRowB + dim * 2) = wv;
    }
  }
  constexpr int kLanesPerRow = D / 8;              // 16 bytes each
  constexpr int kRowsPerStore = 64 / kLanesPerRow;
  const int sr = lane / kLanesPerRow, sc = lane % kLanesPerRow;
#pragma unroll
  for (int i = 0; i < 32 / kRowsPerStore; ++i) {
    const int row = i * kRowsPerStore + sr;
    const u32x4 v = *(const FA2_LDS u32x4*)(stg + row * kRowB + sc * 16);
    if (q_row0 + row < N) *(u32x4*)(a.o + head_off + (int64_t)(q_row0 + row) * D + sc * 8) = v;
  }
}

}  // namespace w8
}  // namespace fa2
