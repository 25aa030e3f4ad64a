// fa2_fwd_pair.h -- fused exact-attention forward pass for gfx950 at head dim
// 256: eight wavefronts per workgroup, the two of a pair sharing query rows.
//
// What the pages fix, and where it lives here (as in the other forward kernels):
//  * Query tiles outside, key/value tiles inside; Q is loaded once and O written
//    once per query tile ("6.2 FlashAttention V2 in depth", section 2.2); the
//    grid covers (query tile x head x batch) ("FlashAttention-2: Where the
//    Second 2x Actually Comes From", section "Parallelism over sequence
//    length").
//  * Online softmax with an unnormalised output divided by the row sum once
//    after the key loop, and the statistic L = m + log l (same page as above,
//    "Method"; "6.2 FlashAttention V2 in depth", sections 3.2, 6.1, 7.1).
//  * Causal block classes: key tiles past the query tile are never visited,
//    tiles crossing the diagonal are masked element by element (section 5.3).
//    General masks (sliding window, a prefix visible to every query, document
//    segment ids: "Flash Attention 2", section "Causal masking") likewise: the
//    key tiles the rows can see come in at most two runs (the prefix, the
//    window), cut to the span of matching segment ids, and the keys a wavefront
//    cannot see are masked element by element.
//  * Head dims up to 256 ("FlashAttention-2: ...", "Limitations & open
//    questions").
//
// gfx950 design.  At head dim 256 the unnormalised output of 32 query rows is
// 128 fp32 registers per lane and their Q operand 64 more, so one wavefront
// owning whole rows leaves no room for a second wavefront on its SIMD, and
// its softmax cannot overlap its products.  Here the two wavefronts of a pair
// own the same 32 query rows and split the work between them:
//  * S = K Q^T: wavefront h of the pair takes keys 32h .. 32h+31 of each 64-key
//    tile over the whole head dim (16 MFMAs of 32x32x16), so it holds 16 scores
//    per lane and forms their softmax weights itself: half the exponentials per
//    MFMA of the head-dim-128 kernel.
//  * O^T += V^T P^T: wavefront h owns output columns 128h .. 128h+127 (64
//    accumulator registers) and needs the weights of all 64 keys; the pair
//    trades its packed fp16/bf16 weights through LDS (2 KB per wavefront and
//    tile) between the softmax phase and the next product phase.
//  * Both wavefronts of a pair must weigh every key against the same reference
//    max.  Each writes the row max of its 32 scores to LDS right after its
//    score products; in the softmax phase both read the other's and take the
//    same decision (the reference moves only when the tile max exceeds it by
//    more than 2^kTau, then O and l are rescaled).  Each keeps its own share of
//    the row sum; the shares are added once at the end.
// About 200 registers per wavefront, so the eight wavefronts run two per SIMD
// in two groups (waves 0-3 and 4-7, pairs (0,1), (2,3), (4,5), (6,7)); each
// step of the key loop has two phases split by workgroup barriers, and in each
// phase one group runs its products while the other runs its softmax, so MFMA
// and VALU work on a SIMD overlap.
//
// Data movement: K and V tiles go global -> LDS with global_load_lds, one tile
// ahead, into two K and two V slots (128 KB; there is no room for a transposed
// copy of V next to them).  K is stored in 256-byte blocks of 16 rows x one
// 16-byte chunk (the A-operand read of 16 lanes covers one block); V is stored
// row-major with its chunks XOR-swizzled per row and read as V^T operands by
// ds_read_b64_tr_b16.
#pragma once

#include <type_traits>

#include "fa2_common.h"

namespace fa2 {
namespace pr {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 128;  // query rows per workgroup: 4 pairs x 32
constexpr int kBc = 64;   // keys per K/V tile
constexpr int D = 256;
constexpr int CPR = D / 8;                              // 16-byte chunks per row
constexpr int kTile = kBc * D;                          // elements of one K or V slot

// V rows keep their 16-byte chunks XOR-swizzled by 4 * (row % 4): a transposed
// read touches 4 consecutive rows x 64 bytes per half wave, which the swizzle
// spreads over 4 distinct 64-byte bank windows.
__device__ __forceinline__ int swz_v(int row) { return (row & 3) << 2; }

template <int kDType, int kMask>
__global__ __launch_bounds__(kThreads, 1) void fa2_fwd_pair(FwdArgs a) {
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
  constexpr int CPRK = D * kEbK / 16;                 // 16-byte chunks per K row
  constexpr int KS = kQK8 ? D / 64 : D / 16;          // k-steps of S
  constexpr int DBH = 4;      // 32-column output blocks per wavefront (half the head dim)
  // S fragments: one per 16-bit MFMA; an fp8 operand is two 16-byte halves,
  // loaded as consecutive fragments 2 ks and 2 ks + 1.
  constexpr int kNs = kQK8 ? 2 * KS : KS;
  constexpr int kNpv = 4 * DBH;  // P.V fragments: 4 key steps x 4 output blocks
  constexpr int kPipe = 4;
  constexpr float kNegInf = -__builtin_huge_valf();

  __shared__ __attribute__((aligned(1024))) uint16_t sK_[2 * kTile];
  __shared__ __attribute__((aligned(1024))) uint16_t sV_[2 * kTile];
  // Packed weights of each wavefront's 32 keys: [wave][quad][lane], 16 bytes.
  __shared__ __attribute__((aligned(16))) uint32_t sP_[kWaves * 2 * 64 * 4];
  // Row max of each wavefront's scores (and at the end its row-sum share).
  __shared__ __attribute__((aligned(16))) float sM_[kWaves * 64];
  FA2_LDS uint16_t* const sK = (FA2_LDS uint16_t*)sK_;
  FA2_LDS uint16_t* const sV = (FA2_LDS uint16_t*)sV_;
  FA2_LDS uint32_t* const sP = (FA2_LDS uint32_t*)sP_;
  FA2_LDS float* const sM = (FA2_LDS float*)sM_;
  // Under segment ids: the keys' ids of the two K slots, and the span reduction.
  __shared__ __attribute__((aligned(16))) int seg_[kSeg ? 2 * kBc : 4];
  __shared__ int red_[kSeg ? 2 * kWaves : 2];
  FA2_LDS int* const sSeg = (FA2_LDS int*)seg_;

  const int N = a.N;
  int bh, qtile;
  wg_to_tile(a, kCausal || (kGeneral && a.grow), bh, qtile);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;   // 0: products first in each step, 1: softmax first
  const int kh = wave & 1;     // key half of S, column half of O
  const int partner = wave ^ 1;
  const int lane = tid & 63;
  const int hl = lane >> 5;
  const int col = lane & 31;   // query column of S^T / O^T held by this lane
  const int q_row0 = qtile * kBr + (wave >> 1) * 32;
  const int my_q = q_row0 + col;
  const int64_t head_off = (int64_t)bh * N * D;
  const uint16_t* __restrict__ kh_ptr = a.k + head_off;             // K of this head (16-bit instances)
  const char* __restrict__ kh_b = (const char*)a.k + head_off * kEbK;  // the same, bytes (e4m3 instances)
  const uint16_t* __restrict__ vh_ptr = a.v + head_off;
  // Score multiplier in log2 units (the fp8 instances fold in the descales).
  float c2 = a.c2;
  if constexpr (kQK8) {
    if (a.descale_q) c2 *= a.descale_q[bh];
    if (a.descale_k) c2 *= a.descale_k[bh];
  }
  const bool pos = c2 > 0.f;  // -inf times the multiplier stays -inf: mask raw scores
  // A pair whose 32 rows all lie past N (the last query tile of a ragged N)
  // skips its products and softmax and only issues its share of the copies.
  const bool live = q_row0 < N;

  // Key tiles: step st visits tile tile_of(st), st < nt.  Without a general
  // mask tiles 0 .. nt-1 (under the causal mask up to the rows' last key); a
  // general mask visits the runs of general_runs, cut to the keys whose segment
  // ids can match.
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
  // Under segment ids: when the pair's 32 rows share one id (seg_w), a block's
  // visibility follows from a comparison of each key's id with it.
  bool rows_one_seg = false;
  int seg_w = 0;
  if constexpr (kSeg) {
    seg_w = __builtin_amdgcn_readfirstlane(seg_q);
    rows_one_seg = __all(seg_q == seg_w);
  }

  // Copies: 64 KB per step through the CU's load path, which takes in the
  // order of 2000 cycles to accept them when they are issued all at once, and
  // a wavefront waits at an issue the path cannot take yet.  So each group
  // issues half, at a point where the wait costs the least: group 1 the V tile
  // st as its softmax phase opens (vector work only), group 0 the K tile st + 1
  // between its P.V products (one copy every second MFMA), which still leaves
  // a phase and a half for the copies to land before the next step.
  // Copy-wave c = wave % 4, instruction t fills 1 KB:
  //  * K (kTPR = CPRK / 16 instructions per 16 rows: 2 for 16-bit K, 1 for
  //    e4m3): blocks 4 (4t + c) .. + 3, i.e. rows 16 (t / kTPR) + lane % 16 of
  //    chunk 16 (t % kTPR) + 4c + lane / 16: one lane offset, the rest in the
  //    scalar base;
  //  * V: 16-byte slots 64 (4t + c) + lane, i.e. row 8t + 2c + lane / 32, stored
  //    chunk lane % 32 holding logical chunk (lane % 32) ^ swz_v(row) (row % 4
  //    does not depend on t).
  constexpr int kCopyWaves = 4;
  constexpr int kLoads = kBc * CPR / (64 * kCopyWaves);    // V copy instructions per copy-wave per tile (8)
  constexpr int kLoadsK = kBc * CPRK / (64 * kCopyWaves);  // K: 8, or 4 for e4m3
  constexpr int kTPR = CPRK / 16;
  static_assert(kLoads * 64 * kCopyWaves == kBc * CPR, "tile copy split");
  static_assert(kLoadsK * 64 * kCopyWaves == kBc * CPRK && kTPR >= 1, "K tile copy split");
  const int cw = wave & 3;
  const int krow = lane & 15, kch = 4 * cw + (lane >> 4);
  const uint32_t voffK = kQK8 ? (uint32_t)(krow * D + kch * 16) : (uint32_t)((krow * D + kch * 8) * 2);
  const int vrow = 2 * cw + (lane >> 5);
  const int vch = (lane & 31) ^ swz_v(vrow);
  const uint32_t voffV = (uint32_t)((vrow * D + vch * 8) * 2);
  // Copy instruction t of K tile `tile` into `slot` (under segment ids, with
  // the first one, wave 0 also copies the keys' ids).
  auto issue_k1 = [&](int tile, int slot, int t) __attribute__((always_inline)) {
    const int kv0 = tile * kBc;
    if (kSeg && t == 0 && wave == 0) dma4(segb + min(kv0 + lane, N - 1), sSeg + slot * kBc);
    FA2_LDS uint16_t* dk = sK + slot * kTile + (t * kCopyWaves + cw) * 512;
    if constexpr (kQK8) {
      if (kv0 + kBc <= N) {
        dma16_sbase(kh_b + (int64_t)kv0 * D + t * 16 * D, voffK, dk);
      } else {
        const int g = min(kv0 + t * 16 + krow, N - 1);
        dma16(kh_b + (int64_t)g * D + kch * 16, dk);
      }
    } else if (kv0 + kBc <= N) {
      dma16_sbase((const char*)(kh_ptr + (int64_t)kv0 * D) + (t >> 1) * 16 * D * 2 + (t & 1) * 256, voffK, dk);
    } else {
      // Ragged last tile: rows past N re-read row N-1 (their scores are masked).
      const int g = min(kv0 + (t >> 1) * 16 + krow, N - 1);
      dma16(kh_ptr + (int64_t)g * D + kch * 8 + (t & 1) * 128, dk);
    }
  };
  auto issue_k = [&](int tile, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < kLoadsK; ++t) issue_k1(tile, slot, t);
  };
  auto issue_v = [&](int tile, int slot) __attribute__((always_inline)) {
    const int kv0 = tile * kBc;
    FA2_LDS uint16_t* dv = sV + slot * kTile;
    if (kv0 + kBc <= N) {
      const char* vb = (const char*)(vh_ptr + (int64_t)kv0 * D);
#pragma unroll
      for (int t = 0; t < kLoads; ++t) dma16_sbase(vb + t * 8 * D * 2, voffV, dv + (t * kCopyWaves + cw) * 512);
    } else {
#pragma unroll
      for (int t = 0; t < kLoads; ++t) {
        const int g = min(kv0 + 8 * t + vrow, N - 1);
        dma16(vh_ptr + (int64_t)g * D + vch * 8, dv + (t * kCopyWaves + cw) * 512);
      }
    }
  };

  // The first K tile streams while Q is loaded.  The first product phase runs
  // P.V with zero weights on V slot 1 and the partners' weights in LDS, so
  // both start as zeros (finite values: a zero weight times garbage could be
  // NaN); they are visible after the first barrier.
  if (grp == 0) issue_k(tile_of(0), 0);
  {
    FA2_LDS u32x4* zv = (FA2_LDS u32x4*)(sV + kTile);
#pragma unroll
    for (int i = tid; i < kTile / 8; i += kThreads) zv[i] = u32x4{0u, 0u, 0u, 0u};
    FA2_LDS u32x4* zp = (FA2_LDS u32x4*)sP;
#pragma unroll
    for (int i = tid; i < kWaves * 2 * 64; i += kThreads) zp[i] = u32x4{0u, 0u, 0u, 0u};
  }

  // Q fragments (B operand of S^T = K Q^T) over the whole head dim, kept in
  // registers; consumed here so that the compiler's wait for them (which also
  // covers the copy above) stays out of the loop.
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

  f32x16 o[DBH];
#pragma unroll
  for (int j = 0; j < DBH; ++j) o[j] = f32x16{};
  float m_run = kNegInf;  // reference max of this lane's query row (log2 units), shared by the pair
  float l_part = 0.f;     // this lane's share of the row sum over this wavefront's keys
  f32x16 s;               // scores of this wavefront's 32 keys, between products and softmax
  float mx = kNegInf;     // their row max (raw units when pos, else log2 units)
  uint32_t pk[8];         // packed weights of this wavefront's 32 keys, B-operand order

  // Operand addresses.  K: lane (hl, col) reads key 32 kh + col, chunk 2 ks + hl
  // (e4m3: chunks 4 ks + 2 hl and + 1).
  // V^T (output block 4 kh + j, key step c of 16 keys): lane (g, L) = (lane / 16,
  // lane % 16) takes keys 16 c + 4 (g / 2) + L / 4 and + 8 of columns 32 (4 kh + j)
  // + 16 (g % 2) + 4 (L % 4) .. + 3, i.e. the key order the score registers hold
  // (stored chunk 4 (4 kh + j) + y XOR-swizzled by 4 x, x = L / 4).  P.V takes the
  // two key steps of this wavefront's own half first (weights in registers),
  // then the partner's two (weights from LDS): one base address per (half, j),
  // everything else an immediate.
  const uint32_t kaddr0 =
      (uint32_t)(((((2 * kh + (col >> 4)) * CPRK) + (kQK8 ? 2 * hl : hl)) << 8) + ((col & 15) << 4));
  uint32_t vaddr0[2][4];
  {
    const int g = lane >> 4, L = lane & 15;
    const int x = L >> 2, y = 2 * (g & 1) + ((L & 3) >> 1);
    const uint32_t lane_part = (uint32_t)((4 * (g >> 1) + x) * CPR * 16 + 16 * y + 8 * (L & 1) + 256 * kh);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vaddr0[0][j] = lane_part + (uint32_t)(64 * (j ^ x)) + (uint32_t)(2 * kh * 16 * CPR * 16);
      vaddr0[1][j] = lane_part + (uint32_t)(64 * (j ^ x)) + (uint32_t)(2 * (1 - kh) * 16 * CPR * 16);
    }
  }
  FA2_LDS uint32_t* const my_p = sP + wave * 512;
  FA2_LDS uint32_t* const partner_p = sP + partner * 512;

  V8 fr[kPipe];
  // Fragment i: S for i < kNs (k-step i), else P.V fragment f = i - kNs: key
  // step c' = f / 4 of this wavefront's order (c' < 2: own half, key step
  // 2 kh + c'; else the partner's, key step 2 (1 - kh) + c' - 2), output block
  // j = f % 4.
  auto load_op = [&](uint32_t kbase, const uint32_t (*vb)[4], int i) __attribute__((always_inline)) {
    if (i < kNs) {
      const int chunk = kQK8 ? 4 * (i >> 1) + (i & 1) : 2 * i;
      return __builtin_bit_cast(V8, *(const FA2_LDS u32x4*)(size_t)(kbase + (uint32_t)(chunk << 8)));
    }
    const int f = i - kNs, cp = f >> 2, j = f & 3;
    const uint32_t ad = vb[cp >> 1][j] + (uint32_t)(16 * (cp & 1) * CPR * 16);
    const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)(size_t)ad);
    const i16x4 t2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)(size_t)(ad + 8 * CPR * 16));
    const u32x2 w1 = __builtin_bit_cast(u32x2, t1);
    const u32x2 w2 = __builtin_bit_cast(u32x2, t2);
    return __builtin_bit_cast(V8, u32x4{w1[0], w1[1], w2[0], w2[1]});
  };

  // One product phase: S^T = K Q^T for key tile st (with the tile's masking and
  // row max, written to LDS for the partner), then O^T += V^T P^T for tile
  // st - 1 with this wavefront's weights (pk) and the partner's (from LDS).
  // Both always run, which keeps one code path (and one register allocation)
  // for the loop: on the first step the weights are all zero and the V slot
  // holds zeros, and the closing step's scores are not used.
  // kCopyK (compile-time, group 0): also issue the copies of K tile st + 1,
  // one after every second P.V product (every fourth for e4m3 K).
  auto products = [&](int st, auto kCopyK) __attribute__((always_inline)) {
    constexpr bool copy_k = decltype(kCopyK)::value;
    const bool k_next = st + 1 < nt;
    const uint32_t kbase = opaque_vgpr((uint32_t)(size_t)(sK + (st & 1) * kTile) + kaddr0);
    uint32_t vb[2][4];
    const uint32_t vslot = (uint32_t)(size_t)(sV + ((st + 1) & 1) * kTile);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) vb[h][j] = opaque_vgpr(vslot + vaddr0[h][j]);
    __builtin_amdgcn_s_setprio(2);
    f32x16 sa = f32x16{};
#pragma unroll
    for (int i = 0; i < kPipe; ++i) fr[i] = load_op(kbase, vb, i);
    uint32_t pp[8];
    constexpr int kCopyStride = kNpv / kLoadsK;
#pragma unroll
    for (int i = 0; i < kNs + kNpv; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i < kNs) {
        if constexpr (kQK8) {
          // An fp8 MFMA takes the fragment pair (i - 1, i): issue it on the
          // second half, and reload the pair's slots only then.
          if (i & 1) {
            const u32x4 lo = __builtin_bit_cast(u32x4, fr[(i - 1) % kPipe]);
            const u32x4 hi = __builtin_bit_cast(u32x4, fr[i % kPipe]);
            const i32x8 ka = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                              (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            sa = mfma_fp8(ka, qf[i >> 1], sa);
            if (i - 1 + kPipe < kNs + kNpv) fr[(i - 1) % kPipe] = load_op(kbase, vb, i - 1 + kPipe);
          }
        } else {
          sa = E::mfma(fr[i % kPipe], qf[i], sa);
        }
      } else {
        const int f = i - kNs, cp = f >> 2, j = f & 3;
        if (f == 8) {  // the partner's weights, needed from here on
          const u32x4 p0 = *(const FA2_LDS u32x4*)(partner_p + 4 * lane);
          const u32x4 p1 = *(const FA2_LDS u32x4*)(partner_p + 256 + 4 * lane);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pp[r] = p0[r];
            pp[4 + r] = p1[r];
          }
        }
        const uint32_t* w = cp < 2 ? pk : pp;
        const u32x4 bw = {w[4 * (cp & 1) + 0], w[4 * (cp & 1) + 1], w[4 * (cp & 1) + 2], w[4 * (cp & 1) + 3]};
        o[j] = E::mfma(fr[i % kPipe], __builtin_bit_cast(V8, bw), o[j]);
      }
      if (i + kPipe < kNs + kNpv && !(kQK8 && i < kNs && (i & 1) == 0)) fr[i % kPipe] = load_op(kbase, vb, i + kPipe);
      if (copy_k && i >= kNs && ((i - kNs) % kCopyStride) == 0 && k_next)
        issue_k1(tile_of(st + 1), (st + 1) & 1, (i - kNs) / kCopyStride);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    s = sa;
    const int k0 = tile_of(st) * kBc + 32 * kh;  // this wavefront's first key
    bool need_mask = k0 + 31 >= N || (kCausal && k0 + 31 > q_row0);
    if constexpr (kGeneral) {
      // (wave-uniform) every pair of the 32 rows x 32 keys visible: all keys
      // below N, the keys all in the prefix or the window satisfied at the
      // block's corners, and under segment ids one id for all of them.
      const int k1 = k0 + 31, qa = q_row0, qb = q_row0 + 31;
      bool full = k1 < N && (k1 < a.prefix || ((a.wl < 0 || k0 >= qb - a.wl) && (a.wr < 0 || k1 <= qa + a.wr)));
      if constexpr (kSeg) {
        if (full) full = rows_one_seg && __all(sSeg[(st & 1) * kBc + 32 * kh + col] == seg_w);
      }
      need_mask = !full;
    }
    // Key of score r of this lane: k0 + 8 (r / 4) + 4 hl + r % 4.
    int lim = N - (k0 + 4 * hl);
    if (kCausal) lim = min(lim, my_q + 1 - (k0 + 4 * hl));
    if (kGeneral && need_mask) {
      // Score r is key base + off, off = 8 (r / 4) + r % 4: visible iff below N
      // and in the prefix or the window (and, under segment ids, of the row's id).
      const int base = k0 + 4 * hl;
      const int lim_p = a.prefix - base;
      const int lo_w = a.wl < 0 ? INT32_MIN / 2 : my_q - a.wl - base;
      const int hi_w = a.wr < 0 ? INT32_MAX / 2 : my_q + a.wr - base;
      u32x4 sg[4] = {};
      if constexpr (kSeg) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) sg[g4] = *(const FA2_LDS u32x4*)(sSeg + (st & 1) * kBc + 32 * kh + 8 * g4 + 4 * hl);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        bool ok = off < lim && (off < lim_p || (off >= lo_w && off <= hi_w));
        if constexpr (kSeg) ok = ok && (int)sg[r >> 2][r & 3] == seg_q;
        const float tt = pos ? s[r] : s[r] * c2;
        s[r] = ok ? tt : kNegInf;
      }
    } else if (pos) {
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = (8 * (r >> 2) + (r & 3)) < lim ? s[r] : kNegInf;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = (!need_mask || (8 * (r >> 2) + (r & 3)) < lim) ? s[r] * c2 : kNegInf;
    }
    float m = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) m = fmaxf(m, s[r]);
    mx = max_pair32(m);
    sM[wave * 64 + lane] = mx;
  };

  // Softmax of this wavefront's scores of tile st into pk, with the reference
  // decided from both halves' row maxima; the weights go to LDS for the
  // partner's next product phase.
  auto softmax = [&]() __attribute__((always_inline)) {
    const float mul = pos ? c2 : 1.f;
    const float m_tile = fmaxf(mx, sM[partner * 64 + lane]) * mul;
    const bool need = m_tile > m_run + kTau;
    if (__any(need)) {
      const float m_new = need ? m_tile : m_run;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      l_part *= alpha;
#pragma unroll
      for (int j = 0; j < DBH; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[j][r] *= alpha;
      m_run = m_new;
    }
    // A row none of whose keys so far is visible has only -inf scores: any
    // finite reference gives it zero weights.
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    float ls[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * e], mul, -m_use));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * e + 1], mul, -m_use));
      pk[e] = E::pack2(p0, p1);
      if (e < 4) ls[e] = p0 + p1;
      else ls[e & 3] += p0 + p1;
    }
    l_part += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    *(FA2_LDS u32x4*)(my_p + 4 * lane) = u32x4{pk[0], pk[1], pk[2], pk[3]};
    *(FA2_LDS u32x4*)(my_p + 256 + 4 * lane) = u32x4{pk[4], pk[5], pk[6], pk[7]};
  };

  // Step st: group 0 runs [products(st) with the copies of K tile st + 1] then
  // [softmax(st)], group 1 runs [copies of V tile st, softmax(st - 1)] then
  // [products(st)]; the copies land by the next step's first barrier.  Both groups execute the same barriers in the same
  // order; each has its own copy of the loop so that the compiler sees which
  // registers stay live across the barriers.

#pragma unroll
  for (int r = 0; r < 8; ++r) pk[r] = 0u;
  if (!live) {
    // No row of this pair exists: its copies and the barriers only.
    for (int st = 0; st <= nt; ++st) {
      __builtin_amdgcn_sched_barrier(0);
      wait_vm_lds_barrier<0>();
      __builtin_amdgcn_sched_barrier(0);
      if (grp == 0) {
        if (st + 1 < nt) issue_k(tile_of(st + 1), (st + 1) & 1);
      } else {
        if (st < nt) issue_v(tile_of(st), st & 1);
      }
      lds_done_barrier();
    }
  } else if (grp == 0) {
    for (int st = 0; st <= nt; ++st) {
      __builtin_amdgcn_sched_barrier(0);
      wait_vm_lds_barrier<0>();
      __builtin_amdgcn_sched_barrier(0);
      products(st, std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
      lds_done_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (st < nt) softmax();
    }
  } else {
    for (int st = 0; st <= nt; ++st) {
      __builtin_amdgcn_sched_barrier(0);
      wait_vm_lds_barrier<0>();
      __builtin_amdgcn_sched_barrier(0);
      if (st < nt) issue_v(tile_of(st), st & 1);
      if (st > 0) softmax();
      __builtin_amdgcn_sched_barrier(0);
      lds_done_barrier();
      __builtin_amdgcn_sched_barrier(0);
      products(st, std::false_type{});
    }
  }

  // Epilogue: the row sum is the pair's two shares; one division per row, the
  // logsumexp in natural-log units.  A lane holds 4-element pieces of one row,
  // so this wavefront's half of O goes through LDS (free after the barriers
  // below): written row-major, read back 16 bytes per lane and stored as whole
  // 256-byte row halves, 1 KB per store instruction.
  const float l_mine = sum_pair32(l_part);
  lds_done_barrier();  // every wavefront is done with the tiles and with sM
  sM[wave * 64 + lane] = l_mine;
  lds_done_barrier();
  const float l_row = l_mine + sM[partner * 64 + lane];
  const float inv = 1.f / l_row;
  if (my_q < N && hl == 0 && kh == 0) a.lse[(int64_t)bh * N + my_q] = (m_run + __log2f(l_row)) * kLn2;
  constexpr int kRowB = 256 + 16;  // staging row stride: aligned, conflict-free 16-byte reads
  static_assert(4 * 32 * kRowB <= 2 * kTile * 2, "a group's staging fits in its tile buffers");
  FA2_LDS char* const stg = (FA2_LDS char*)(grp == 0 ? sK_ : sV_) + (wave & 3) * 32 * kRowB;
#pragma unroll
  for (int j = 0; j < DBH; ++j) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int dim = 32 * j + 8 * r4 + 4 * hl;
      const u32x2 wv = {E::pack2(o[j][4 * r4 + 0] * inv, o[j][4 * r4 + 1] * inv),
                        E::pack2(o[j][4 * r4 + 2] * inv, o[j][4 * r4 + 3] * inv)};
      *(FA2_LDS u32x2*)(stg + col * kRowB + dim * 2) = wv;
    }
  }
  const int sr = lane >> 4, sc = lane & 15;  // 16 lanes per 256-byte row half, 4 rows per store
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 4 * i + sr;
    const u32x4 v = *(const FA2_LDS u32x4*)(stg + row * kRowB + sc * 16);
    if (q_row0 + row < N) *(u32x4*)(a.o + head_off + (int64_t)(q_row0 + row) * D + 128 * kh + sc * 8) = v;
  }
}

}  // namespace pr
}  // namespace fa2
