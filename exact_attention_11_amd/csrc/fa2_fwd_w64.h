// fa2_fwd_w64.h -- fused exact-attention forward pass for gfx950 at head dim 128
// (no mask or the causal mask): one wavefront per SIMD, 64 query rows per
// wavefront, and each wavefront overlapping its own softmax with its matrix
// products.
//
// What the pages fix, and where it lives here:
//  * Query tiles outside, key/value tiles inside; Q is loaded once and O written
//    once per query tile ("6.2 FlashAttention V2 in depth", section 2.2), over a
//    grid of (query tile x head x batch) ("FlashAttention-2: Where the Second 2x
//    Actually Comes From", section "Parallelism over sequence length").
//  * Split-Q: each wavefront owns whole query rows and sees every key of a tile,
//    so row statistics never cross wavefronts ("6.2 FlashAttention V2 in depth",
//    section 4.2).
//  * Online softmax with an unnormalised output, divided by the row sum once
//    after the key loop, and L = m + log l (same page, sections 3.2, 6.1, 7.1).
//  * Causal block classes: tiles past the query tile are never visited, tiles
//    crossing the diagonal are masked element by element (same page, 5.3).
//
// gfx950 design:
//  * Work split.  Four wavefronts, one per SIMD, each owning 64 query rows as
//    two 32-row blocks.  Every K or V^T operand fragment read from LDS feeds two
//    MFMAs (one per row block), which halves the LDS operand traffic per FLOP
//    of 32-row wavefronts, and the 512 registers of a lone wavefront hold O and
//    Q in accumulation registers and two tiles of scores in vector registers.
//  * Overlap inside the wavefront.  Step j issues 64 MFMAs -- O^T += V^T P^T
//    for tile j-1, then S^T = K Q^T for tile j+1 -- and between consecutive
//    MFMAs a slice of the softmax of tile j (whose scores step j-1 produced),
//    so the vector ALU work runs while the matrix core is busy.  Scheduling
//    fences fix that order; the exact same softmax as the pages' (the lazy
//    reference of the other forward kernels) is then checked once per step.
//  * Operands.  Scores are computed transposed, S^T = K Q^T, with the rows of
//    each K tile permuted (bits 2 and 3 of the row index swapped) so that a
//    lane's scores are the B operand of the P.V product as they stand.  The
//    A operand V^T is read straight from the row-major V tile with
//    ds_read_b64_tr_b16 (two per fragment).
//  * Data movement.  K and V tiles go global -> LDS with global_load_lds, K
//    three steps ahead into three slots and V two steps ahead into four (a V
//    tile is read during two steps: prefetched at the end of one, consumed in
//    the next); one workgroup barrier per step.
#pragma once

#include <type_traits>

#include "fa2_fwd_8wave.h"  // K row permutation and LDS tile layouts

namespace fa2 {
namespace w64 {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsW = 64;               // query rows per wavefront
constexpr int kBr = kRowsW * kWaves;     // query rows per workgroup
constexpr int kBc = 32;                  // keys per tile (one step of the key loop)
constexpr int kKSlots = 3;
constexpr int kVSlots = 4;
constexpr int kPipe = 4;                 // operand fragments read ahead of their MFMAs

using w8::k_byte;
using w8::sigma;
using w8::vs_byte;

// S^T = K Q^T blocks on the matrix core with the accumulator in vector
// registers, where the softmax reads it.  Written as inline assembly: the
// compiler gives every builtin MFMA of a kernel that holds accumulators in
// accumulation registers (O, here) the accumulation-register form.  The
// compiler does not see these as MFMAs, so their hazards are covered by
// construction and checked on the built code: the operands come from memory
// loads (no vector ALU write shortly before); the accumulating form rewrites
// its own accumulator in place (same registers and opcode, which needs no wait
// states); and the kernel reads the results no earlier than the next step
// (dozens of instructions later; after the first tile, behind explicit
// s_nops).  Templates, so that the host pass
// (which only emits launch stubs) never checks the gfx950 operands.
template <int kDType, typename V8>
__device__ __forceinline__ void s_mfma_first(f32x16& d, V8 a, V8 b) {
  if constexpr (kDType == kFp16)
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
template <int kDType, typename V8>
__device__ __forceinline__ void s_mfma_acc(f32x16& d, V8 a, V8 b) {
  if constexpr (kDType == kFp16)
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}

template <int kDType, int kMask>
__global__ __launch_bounds__(kThreads, 1) void fa2_fwd_w64(FwdArgs a) {
  constexpr int D = 128;
  constexpr bool kCausal = kMask == kMaskCausal;
  static_assert(kMask == kMaskNone || kMask == kMaskCausal, "no mask or the causal mask");
  static_assert(kDType == kFp16 || kDType == kBf16, "16-bit inputs");
  typedef Elem<kDType> E;
  typedef typename E::V8 V8;
  constexpr int CPR = D / 8;                          // 16-byte chunks per row
  constexpr int KS = D / 16;                          // k-steps of S = K Q^T
  constexpr int DB = D / 32;                          // 32-wide output column blocks
  constexpr int kTile = kBc * D;                      // elements of one K or V slot
  constexpr int kLoads = kBc * CPR / (64 * kWaves);   // copy instructions per wave per tile
  constexpr int kRowStep = 4 * 16 * kWaves / CPR;     // rows covered by one instruction of all waves
  constexpr int kStepLoads = 2 * kLoads;              // copies per wave per step (K and V)
  constexpr int kKB = kBc / 32;                       // 32-key blocks per tile
  constexpr int kNv = (kBc / 16) * DB;                // V^T fragments per tile
  constexpr int kNk = kKB * KS;                       // K fragments per tile
  constexpr int kNe = 2 * kKB * 16;                   // scores per lane per tile
  constexpr int kOps = kNv + kNk;                     // fragments per step, two MFMAs each
  constexpr float kNegInf = -__builtin_huge_valf();
  static_assert(kBc % 32 == 0 && kLoads * 64 * kWaves == kBc * CPR && kRowStep == 16, "tile copy split");
  static_assert(kOps % kPipe == 0 && kPipe <= kNv && kPipe <= kNk, "fragment ring");
  static_assert(2 * kOps == 8 * kStepLoads && (2 * kNk) % kStepLoads == 0, "copy issue slots");
  static_assert(kNe == 2 * kOps, "one pair of scores per two MFMA slots");
  constexpr int kRowB = D * 2 + 16;  // O staging row stride: aligned 16-byte reads, 2-way conflicts on the 8-byte writes
  constexpr int kTileElems = (kKSlots + kVSlots) * kTile;
  constexpr int kStageElems = kWaves * kRowsW * kRowB / 2;

  __shared__ __attribute__((aligned(1024))) uint16_t smem_[kTileElems > kStageElems ? kTileElems : kStageElems];
  FA2_LDS uint16_t* const sK = (FA2_LDS uint16_t*)smem_;
  FA2_LDS uint16_t* const sV = sK + kKSlots * kTile;

  const int N = a.N;
  int bh, qtile;
  wg_to_tile(a, kCausal, bh, qtile);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hl = lane >> 5;
  const int col = lane & 31;
  const int q_row0 = qtile * kBr + wave * kRowsW;
  const int64_t head_off = (int64_t)bh * N * D;
  const char* __restrict__ kh = (const char*)(a.k + head_off);
  const char* __restrict__ vh = (const char*)(a.v + head_off);
  const float c2 = a.c2;

  // Copy layout: instruction t of this wave fills blocks 16t + 4 wave + 0..3,
  // i.e. rows 16t + 0..15 of chunks 4 wave + 0..3; lane i takes chunk
  // 4 wave + i / 16 and the block's slot i % 16 (K: LDS row 16t + i % 16, which
  // holds key sigma of it; V: the row whose swizzled slot is i % 16).
  const int cch = 4 * wave + (lane >> 4);
  const int crow = lane & 15;
  const int vr = crow ^ (4 * (cch & 3));

  const int kv_end = kCausal ? min(N, (qtile + 1) * kBr) : N;
  const int nt = (kv_end + kBc - 1) / kBc;

  // Copy instruction t of a tile: the lane's row within the tile is 16 t + rowK
  // (K, whose LDS row 16 t + crow holds that key) or 16 t + vr (V).  Rows past
  // N (the ragged last tile) re-read row N-1; their scores are masked.  The row
  // is clamped in the lane's offset, so the copies never branch.
  const int rowK = sigma(crow);
  auto copy_k = [&](int tile, int slot, int t) __attribute__((always_inline)) {
    const int kv0 = tile * kBc;
    FA2_LDS uint16_t* dk = sK + slot * kTile + (t * kWaves + wave) * 64 * 8;
    const uint32_t voff = (uint32_t)((min(t * kRowStep + rowK, N - 1 - kv0) * D + cch * 8) * 2);
    dma16_sbase(kh + (int64_t)kv0 * D * 2, voff, dk);
  };
  auto copy_v = [&](int tile, int slot, int t) __attribute__((always_inline)) {
    const int kv0 = tile * kBc;
    FA2_LDS uint16_t* dv = sV + slot * kTile + (t * kWaves + wave) * 64 * 8;
    const uint32_t voff = (uint32_t)((min(t * kRowStep + vr, N - 1 - kv0) * D + cch * 8) * 2);
    dma16_sbase(vh + (int64_t)kv0 * D * 2, voff, dv);
  };
  // Copy instruction i of step st: K of tile st+3, then V of tile st+2 (past the
  // last tile both repeat it, so that every step keeps the same number of copies
  // in flight).  K tile st+3 takes the slot of K tile st (last read in step
  // st-1), V tile st+2 the slot of V tile st-2 (last read in step st-1).
  auto copy_part = [&](int st, int i) __attribute__((always_inline)) {
    if (i < kLoads) copy_k(min(st + 3, nt - 1), (st + 3) % kKSlots, i);
    else copy_v(min(st + 2, nt - 1), (st + 2) % kVSlots, i - kLoads);
  };

  // The V slot that step 0 reads for its (all-zero-weight) P.V term must hold
  // finite values.
  {
    FA2_LDS u32x4* z = (FA2_LDS u32x4*)(sV + (kVSlots - 1) * kTile);
#pragma unroll
    for (int i = tid; i < kTile / 8; i += kThreads) z[i] = u32x4{0u, 0u, 0u, 0u};
  }

  // K of tile 0 streams first; K of tile 1 and V of tile 0 follow once Q has
  // arrived (the compiler's wait for Q also waits for everything issued before).
#pragma unroll
  for (int t = 0; t < kLoads; ++t) copy_k(0, 0, t);

  // Q fragments (B operand of S^T = K Q^T): lane (hl, col) holds elements
  // 16 ks + 8 hl .. + 7 of query row q_row0 + 32 rb + col.
  V8 qf[2][KS];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const uint16_t* qp = a.q + head_off + (int64_t)min(q_row0 + 32 * rb + col, N - 1) * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[rb][ks] = __builtin_bit_cast(V8, *(const u32x4*)(qp + 16 * ks));
  }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[rb][ks]));
#pragma unroll
  for (int t = 0; t < kLoads; ++t) copy_k(min(1, nt - 1), 1, t);
#pragma unroll
  for (int t = 0; t < kLoads; ++t) copy_v(0, 0, t);

  // O^T blocks: lane (hl, col) holds query 32 rb + col, dims 32 db + 8 (r / 4) +
  // 4 hl + r % 4.  They live in accumulation registers for the whole loop (the
  // empty asm statements place them there wherever a vector ALU op produced
  // them).
  f32x16 o[2][DB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      o[rb][db] = f32x16{};
      asm volatile("" : "+a"(o[rb][db]));
    }
  float m_run[2] = {kNegInf, kNegInf};  // reference max of the lane's two rows, log2 units
  float l_part[2] = {0.f, 0.f};         // the lane's share of the two row sums
  // Scores of two tiles (S^T blocks [row block][key block]: lane (hl, col) holds
  // query 32 rb + col and keys 32 kb + 16 (r / 8) + 8 hl + r % 8) and the
  // weights of two tiles (pairs of consecutive keys, 16-bit each).
  // At the start of step st: the scores of tile st in sA, the weights of tile
  // st-1 in pB; the step writes the scores of tile st+1 to sB and the weights of
  // tile st to pA (steps in pairs swap the roles back).
  f32x16 sA[2][kKB], sB[2][kKB];
  uint32_t pA[2][kKB][8], pB[2][kKB][8];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int r = 0; r < 8; ++r) pB[rb][kb][r] = 0u;

  // Operand addresses: K fragment (kb, ks) is row 32 kb + col, chunk 2 ks + hl
  // of the K tile; V^T fragment (c, db) is keys 16 c + 8 hl + 0..7 of column
  // 32 db + col, read as two 4-key transposed reads (rows +0..3 and +4..7; the
  // swizzle makes them two base registers).
  const uint32_t kaddr0 = k_byte<CPR>(col, hl);
  const int tl = lane & 15;
  const int vch = 2 * (col >> 4) + ((tl & 3) >> 1);
  const uint32_t vaddr0 = vs_byte<CPR>(8 * hl + (tl >> 2), vch) + 8 * (tl & 1);
  const uint32_t vaddr1 = vs_byte<CPR>(8 * hl + 4 + (tl >> 2), vch) + 8 * (tl & 1);

  V8 fr[kPipe];  // operand fragments in flight, indexed by fragment number % kPipe
  auto read_v = [&](uint32_t va0, uint32_t va1, int u) __attribute__((always_inline)) {
    const uint32_t off = (uint32_t)((((u / DB) * CPR) + 4 * (u % DB)) << 8);
    const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)(size_t)(va0 + off)));
    const u32x2 y = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)(size_t)(va1 + off)));
    return __builtin_bit_cast(V8, u32x4{x[0], x[1], y[0], y[1]});
  };
  auto read_k = [&](uint32_t kb0, int g) __attribute__((always_inline)) {
    const uint32_t off = (uint32_t)(((2 * (g / KS) * CPR) + 2 * (g % KS)) << 8);
    return __builtin_bit_cast(V8, *(const FA2_LDS u32x4*)(size_t)(kb0 + off));
  };
  auto vbase = [&](int tile, uint32_t addr) __attribute__((always_inline)) {
    return opaque_vgpr((uint32_t)(size_t)(sV + ((tile + kVSlots) % kVSlots) * kTile) + addr);
  };
  auto kbase = [&](int tile) __attribute__((always_inline)) {
    return opaque_vgpr((uint32_t)(size_t)(sK + (tile % kKSlots) * kTile) + kaddr0);
  };

  // Causal and ragged masking of tile st: element (kb, r) of lane hl is key
  // kv0 + 8 hl + key_off(kb, r), allowed iff key < N and, under the causal mask,
  // key <= query; lim[rb] is the bound on key_off for the lane's row of row
  // block rb.  Masked elements get weight 0 (their exponent is set to -inf
  // after the scaling, whatever the sign of the scale).
  auto key_off = [](int kb, int r) constexpr { return 32 * kb + 16 * (r >> 3) + (r & 7); };
  auto limits = [&](int st, int(&lim)[2]) __attribute__((always_inline)) {
    const int base = st * kBc + 8 * hl;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      lim[rb] = N - base;
      if (kCausal) lim[rb] = min(lim[rb], q_row0 + 32 * rb + col + 1 - base);
    }
  };

  // One step's matrix products with interleaved work, as 64 MFMA slots: slot i
  // issues MFMA i, then the operand read kPipe fragments ahead (after the second
  // MFMA of a fragment), then a slice of the softmax of the current tile and at
  // every eighth slot one copy instruction.  Fragments 0..15 are V^T of tile
  // st-1 (P.V), 16..31 K of tile st+1 (S), 32.. the first V^T fragments of
  // tile st (the next step's P.V), read at the end.
  //   kMode 0: the whole step; 1: S only (the first tile, before the loop);
  //   2: P.V only (the last tile, after the loop).
  // Softmax slices: slot 2p + 2 forms the weights of pair p (scores 2p and
  // 2p + 1 of the lane's 2 * kBc / 2 scores, row block first) and slot 2p + 3
  // packs and sums them (four sum chains per row); the last two slices follow
  // the MFMAs.
  // The step's operand base addresses: V^T of tile st-1, K of tile st+1, V^T
  // of tile st.
  struct StepAddr {
    uint32_t va0, va1, kb0, vn0, vn1;
  };
  auto step_addr = [&](int st) __attribute__((always_inline)) {
    return StepAddr{vbase(st - 1, vaddr0), vbase(st - 1, vaddr1), kbase(st + 1), vbase(st, vaddr0),
                    vbase(st, vaddr1)};
  };
  auto products = [&](auto mode, auto masked, int st, const StepAddr& ad, f32x16(&sc)[2][kKB],
                      f32x16(&sn)[2][kKB], uint32_t(&pp)[2][kKB][8], uint32_t(&pc)[2][kKB][8], const int(&lim)[2],
                      float(&lacc)[2][4]) __attribute__((always_inline)) {
    constexpr int kMode = decltype(mode)::value;
    constexpr bool kMasked = decltype(masked)::value;
    const uint32_t va0 = ad.va0, va1 = ad.va1, kb0 = ad.kb0, vn0 = ad.vn0, vn1 = ad.vn1;
    constexpr int i0 = kMode == 1 ? 2 * kNv : 0;
    constexpr int i1 = kMode == 2 ? 2 * kNv : 2 * kOps;
    constexpr int i_end = i1;
    if constexpr (kMode == 1) {
#pragma unroll
      for (int u = kNv; u < kNv + kPipe; ++u) fr[u % kPipe] = read_k(kb0, u - kNv);
    }
    float ex0 = 0.f, ex1 = 0.f;
#pragma unroll
    for (int i = i0; i < i_end; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const int u = i >> 1, rb = i & 1;
      if constexpr (kMode == 0) {
        // Pair p (scores 2p and 2p + 1 of the lane, row block first): weights
        // on slot 2p, packing and row sums on slot 2p + 1.  Each stage's
        // results pass through an empty asm statement on its own slot: ordered
        // with the MFMAs, they keep the stage between them.
        if ((i & 1) == 0) {
          const int p = i >> 1, prb = p / (8 * kKB), pkb = (p / 8) % kKB, r = 2 * (p & 7);
          float t0 = __builtin_fmaf(sc[prb][pkb][r], c2, -m_run[prb]);
          float t1 = __builtin_fmaf(sc[prb][pkb][r + 1], c2, -m_run[prb]);
          if constexpr (kMasked) {
            // The bound passes through an empty asm statement on this slot, so
            // that the comparisons stay here instead of being computed (and
            // held) ahead of the MFMAs.
            int lm = lim[prb];
            asm volatile("" : "+v"(lm));
            t0 = key_off(pkb, r) < lm ? t0 : kNegInf;
            t1 = key_off(pkb, r + 1) < lm ? t1 : kNegInf;
          }
          ex0 = __builtin_amdgcn_exp2f(t0);
          ex1 = __builtin_amdgcn_exp2f(t1);
          asm volatile("" : "+v"(ex0), "+v"(ex1));
        } else {
          const int p = i >> 1, prb = p / (8 * kKB), pkb = (p / 8) % kKB, r = 2 * (p & 7);
          pc[prb][pkb][r >> 1] = E::pack2(ex0, ex1);
          if (p % (8 * kKB) < 4) lacc[prb][p & 3] = ex0 + ex1;
          else lacc[prb][p & 3] += ex0 + ex1;
          asm volatile("" : "+v"(pc[prb][pkb][r >> 1]), "+v"(lacc[prb][p & 3]));
        }
      }
      if (i < i1) {
        if (u < kNv) {
          const int c = u / DB, db = u % DB;
          const u32x4 bw = {pp[rb][c >> 1][4 * (c & 1) + 0], pp[rb][c >> 1][4 * (c & 1) + 1],
                            pp[rb][c >> 1][4 * (c & 1) + 2], pp[rb][c >> 1][4 * (c & 1) + 3]};
          o[rb][db] = E::mfma(fr[u % kPipe], __builtin_bit_cast(V8, bw), o[rb][db]);
        } else {
          const int g = u - kNv, kb = g / KS, ks = g % KS;
          if (ks == 0) s_mfma_first<kDType>(sn[rb][kb], fr[u % kPipe], qf[rb][ks]);
          else s_mfma_acc<kDType>(sn[rb][kb], fr[u % kPipe], qf[rb][ks]);
        }
        if (rb == 1) {
          const int un = u + kPipe;
          if (un < kNv) fr[un % kPipe] = read_v(va0, va1, un);
          else if (un < kOps && kMode != 2) fr[un % kPipe] = read_k(kb0, un - kNv);
          else if (un >= kOps && kMode != 2) fr[un % kPipe] = read_v(vn0, vn1, un - kOps);
        }
      }
      if constexpr (kMode == 0) {
        if ((i & 7) == 4 && i < i1) copy_part(st, i >> 3);
      }
      constexpr int kCopyEvery = 2 * kNk / kStepLoads;
      if (kMode == 1 && (i - i0) % kCopyEvery == 0) copy_part(st, (i - i0) / kCopyEvery);
    }
    __builtin_amdgcn_sched_barrier(0);
    // The first tile's scores are read by the next step after only a few
    // instructions: wait states for the S MFMA results.
    if constexpr (kMode == 1) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  };

  // After the step's weights were formed against the current references: they
  // are accepted when each lane's share of each row sum is at most kSumCap
  // (which bounds every weight by 2^kTau; an overflowed or NaN weight fails the
  // test too).  Otherwise the tile's row maxima decide whether a reference
  // moves; O and l are rescaled by 2^(old - new) and the weights formed again.
  // The first tile always lands here (its references are -inf).
  auto finish_softmax = [&](const f32x16(&sc)[2][kKB], uint32_t(&pc)[2][kKB][8], bool masked, const int(&lim)[2],
                            float(&lacc)[2][4]) __attribute__((always_inline)) {
    float lsum[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) lsum[rb] = (lacc[rb][0] + lacc[rb][1]) + (lacc[rb][2] + lacc[rb][3]);
    if (!__all(lsum[0] <= kSumCap && lsum[1] <= kSumCap)) {
      float m_tile[2];
      bool need[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float t = sc[rb][kb][r] * c2;
            mx = fmaxf(mx, masked && key_off(kb, r) >= lim[rb] ? kNegInf : t);
          }
        m_tile[rb] = max_pair32(mx);
        need[rb] = m_tile[rb] > m_run[rb] + kTau;
      }
      if (__any(need[0] || need[1])) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const float m_new = need[rb] ? m_tile[rb] : m_run[rb];
          const float alpha = need[rb] ? __builtin_amdgcn_exp2f(m_run[rb] - m_new) : 1.f;
          l_part[rb] *= alpha;
          // One O block at a time: the empty asm statements keep the reads of
          // the next block from moving ahead of the write-back of this one.
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            asm volatile("" : "+a"(o[rb][db]));
#pragma unroll
            for (int r = 0; r < 16; ++r) o[rb][db][r] *= alpha;
            asm volatile("" : "+a"(o[rb][db]));
          }
          m_run[rb] = m_new;
          float ls[4];
#pragma unroll
          for (int e = 0; e < 8 * kKB; ++e) {
            const int kb = e >> 3, r = 2 * (e & 7);
            float t0 = __builtin_fmaf(sc[rb][kb][r], c2, -m_new);
            float t1 = __builtin_fmaf(sc[rb][kb][r + 1], c2, -m_new);
            if (masked) {
              t0 = key_off(kb, r) < lim[rb] ? t0 : kNegInf;
              t1 = key_off(kb, r + 1) < lim[rb] ? t1 : kNegInf;
            }
            const float p0 = __builtin_amdgcn_exp2f(t0);
            const float p1 = __builtin_amdgcn_exp2f(t1);
            pc[rb][kb][r >> 1] = E::pack2(p0, p1);
            if (e < 4) ls[e] = p0 + p1;
            else ls[e & 3] += p0 + p1;
          }
          lsum[rb] = (ls[0] + ls[1]) + (ls[2] + ls[3]);
        }
      }
    }
    l_part[0] += lsum[0];
    l_part[1] += lsum[1];
  };

  // One step of the key loop: tile st+1's K and tile st's V have landed for
  // every wave (vmcnt: the copies of the previous step may stay in flight), and
  // every wave has finished the previous step, whose slots this step's copies
  // overwrite.
  auto step = [&](auto masked, int st, f32x16(&sc)[2][kKB], f32x16(&sn)[2][kKB], uint32_t(&pp)[2][kKB][8],
                  uint32_t(&pc)[2][kKB][8]) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    wait_vm_barrier<kStepLoads>();
    __builtin_amdgcn_sched_barrier(0);
    const StepAddr ad = step_addr(st);
    int lim[2];
    limits(st, lim);
    float lacc[2][4];
    products(std::integral_constant<int, 0>{}, masked, st, ad, sc, sn, pp, pc, lim, lacc);
    finish_softmax(sc, pc, decltype(masked)::value, lim, lacc);
  };
  // Back to the step-start layout after a single step (scores to sA, weights
  // to pB).
  auto swap_back = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
        sA[rb][kb] = sB[rb][kb];
#pragma unroll
        for (int r = 0; r < 8; ++r) pB[rb][kb][r] = pA[rb][kb][r];
      }
  };

  float lacc0[2][4];
  const int lim0[2] = {0, 0};
  lds_done_barrier();  // K of tile 0 (waited for with Q) and the zeroed V slot are visible
  products(std::integral_constant<int, 1>{}, std::false_type{}, -1, step_addr(-1), sB, sA, pA, pB, lim0, lacc0);
  // Steps from this wave's first masked tile on (the tile that reaches its
  // first row under the causal mask, and the ragged last tile) run the masked
  // variant.  The unmasked steps run in pairs, which swap the buffer roles
  // back; the few masked ones one at a time.
  int st_mask = nt;
  if (kCausal) st_mask = min(st_mask, q_row0 / kBc);
  if (N % kBc != 0) st_mask = min(st_mask, nt - 1);
  int st = 0;
  for (; st + 2 <= st_mask; st += 2) {
    step(std::false_type{}, st, sA, sB, pB, pA);
    step(std::false_type{}, st + 1, sB, sA, pA, pB);
  }
  if (st < st_mask) {
    step(std::false_type{}, st, sA, sB, pB, pA);
    swap_back();
    ++st;
  }
  for (; st < nt; ++st) {
    step(std::true_type{}, st, sA, sB, pB, pA);
    swap_back();
  }
  products(std::integral_constant<int, 2>{}, std::false_type{}, nt, step_addr(nt), sA, sB, pB, pA, lim0, lacc0);
  // No LDS write may still be in flight when the buffers are reused or the
  // workgroup retires.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Epilogue: one division per row, logsumexp in natural-log units, O staged
  // through LDS and stored as whole rows (D * 2 contiguous bytes per row).
  float inv[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float l_row = sum_pair32(l_part[rb]);
    inv[rb] = 1.f / l_row;
    const int q = q_row0 + 32 * rb + col;
    if (q < N && hl == 0) a.lse[(int64_t)bh * N + q] = (m_run[rb] + __log2f(l_row)) * kLn2;
  }
  static_assert(kWaves * kRowsW * kRowB <= (int)sizeof(smem_), "O staging fits in the tile buffers");
  lds_done_barrier();  // every wave is done with the tile buffers
  FA2_LDS char* const stg = (FA2_LDS char*)smem_ + wave * kRowsW * kRowB;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dim = 32 * db + 8 * r4 + 4 * hl;
        const u32x2 wv = {E::pack2(o[rb][db][4 * r4 + 0] * inv[rb], o[rb][db][4 * r4 + 1] * inv[rb]),
                          E::pack2(o[rb][db][4 * r4 + 2] * inv[rb], o[rb][db][4 * r4 + 3] * inv[rb])};
        *(FA2_LDS u32x2*)(stg + (32 * rb + col) * kRowB + dim * 2) = wv;
      }
  constexpr int kLanesPerRow = D / 8;  // 16 bytes each
  constexpr int kRowsPerStore = 64 / kLanesPerRow;
  const int sr = lane / kLanesPerRow, sc_ = lane % kLanesPerRow;
#pragma unroll
  for (int i = 0; i < kRowsW / kRowsPerStore; ++i) {
    const int row = i * kRowsPerStore + sr;
    const u32x4 v = *(const FA2_LDS u32x4*)(stg + row * kRowB + sc_ * 16);
    if (q_row0 + row < N) *(u32x4*)(a.o + head_off + (int64_t)(q_row0 + row) * D + sc_ * 8) = v;
  }
}

}  // namespace w64
}  // namespace fa2
