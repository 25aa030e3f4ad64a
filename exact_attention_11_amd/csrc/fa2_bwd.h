// fa2_bwd.h -- gradients of exact attention for gfx950 (head dims 64, 128, 256).
//
// What the pages fix, and where it lives here:
//  * The backward pass recomputes the probabilities from the saved row
//    statistic instead of storing them: P = exp(s - L) with L the forward's
//    logsumexp ("6.2 FlashAttention V2 in depth", section 7.1; "Flash
//    Attention: Memory-Efficient Attention at Scale", section "Recomputation
//    in the backward pass").
//  * The softmax gradient is dS = P o (dP - D) with D = rowsum(dO o O), and D
//    is computed once for all rows by a separate preprocess kernel before the
//    main loop ("6.2 FlashAttention V2 in depth", section 7.3): fa2_bwd_delta.
//  * The main backward loop runs over key/value tiles outside and query tiles
//    inside, so the dK and dV of a key tile are accumulated by one workgroup
//    alone; dQ must then be gathered across workgroups, either by atomic adds
//    or by a second pass (same page, section 7.2).  This file takes the second
//    pass: fa2_bwd_dkdv (key tiles outside) writes dK and dV, fa2_bwd_dq (query
//    tiles outside, as in the forward pass) writes dQ.  Both recompute the
//    scores; no atomics, no fp32 dQ buffer, and the result is bitwise
//    reproducible.
//  * The gradients themselves follow from s = scale * q.k, p = softmax(s),
//    o = p.v by the chain rule: dV = P^T dO, dP = dO V^T, dQ = scale dS K,
//    dK = scale dS^T Q.
//
// gfx950 mapping.  Four wavefronts per workgroup, one per SIMD, and two
// workgroups per CU up to d = 128 (64 KB of LDS each), so that two wavefronts
// share every SIMD and one's products overlap the other's elementwise work.
// All products run on v_mfma_f32_32x32x16 with fp32 accumulation.
//  * fa2_bwd_dkdv: wave w owns keys kw0 .. kw0+31 and keeps K and V of those
//    keys in registers as the B operands of S = Q K^T and dP = dO V^T; the Q and
//    dO tiles (64 rows) stream through LDS.  In the accumulator of S a lane
//    holds one key and 16 queries, so P and dS feed dV^T += dO^T P and
//    dK^T += Q^T dS directly as B operands; the A operands (dO^T, Q^T) come
//    from the same LDS tiles through ds_read_b64_tr_b16, reading the query rows
//    in the order the accumulator holds them.
//  * fa2_bwd_dkdv_pair (d = 256): the same product chain over eight
//    wavefronts, two per block of 32 keys: one holds K and forms S, P and dV,
//    the other holds V and forms dP, dS and dK, with P passed between them
//    through LDS, so that neither needs more than 256 registers.
//  * fa2_bwd_dq: the forward's layout: S^T = K Q^T and dP^T = V dO^T with Q and
//    dO of the wave's 32 rows in registers and K, V tiles in LDS; a lane holds
//    one query, so L and D are per-lane scalars; dQ^T += K^T dS^T reads K^T
//    through ds_read_b64_tr_b16.
//  * Every LDS tile is row-major with the 16-byte chunk index XORed by a
//    rotation of the low row bits, which keeps both the row reads (MFMA A
//    operands) and the transposed reads free of bank conflicts.
#pragma once

#include <type_traits>

#include "fa2_common.h"

namespace fa2 {
namespace bwd {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeysPerWg = 32 * kWaves;  // fa2_bwd_dkdv: keys per workgroup
constexpr int kQTile = 64;               // fa2_bwd_dkdv: query rows per streamed tile
constexpr int kRowsPerWg = 32 * kWaves;  // fa2_bwd_dq: query rows per workgroup
constexpr int kKTile = 64;               // fa2_bwd_dq: keys per streamed tile
constexpr int kDeltaRows = 16;           // fa2_bwd_delta: rows per workgroup (16 lanes each)
// fa2_bwd_dkdv and fa2_bwd_dq (d = 64, 128) are compiled for two workgroups
// per CU (two wavefronts per SIMD, at most 256 registers each), so that one
// workgroup's products overlap the other's softmax gradient and memory waits.
// (At d = 128 fa2_bwd_dkdv then needs 255 registers, and fits them only because
// its LDS operand offsets are formed at each use; see the lane values in its
// loop.)  At d = 256 the gradients come from fa2_bwd_dkdv_pair and
// fa2_bwd_dq_pair, which split each block's work between two wavefronts.

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;  // [B, H, N] natural-log logsumexp from the forward pass
  float* delta;      // [B, H, N] D = rowsum(dO o O), written by fa2_bwd_delta
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int N;
  int BH;
  int n_kv_wg;  // ceil(N / kKeysPerWg)
  int n_q_wg;   // ceil(N / kRowsPerWg)
  float scale;  // multiplier of the scores
  float c2;     // scale * log2(e)
  // General mask (the kMaskGeneral and kMaskSegments instances): key c is
  // visible to query r iff c < N, seg[b, c] == seg[b, r] (segment instances),
  // and c < prefix or r - wl <= c <= r + wr (a negative bound is no bound).
  int wl;
  int wr;
  int prefix;
  int H;           // heads per batch: batch b = (b*H + h) / H
  const int* seg;  // [B, N] segment ids, or nullptr
};

constexpr float kLog2e = 1.44269504088896340736f;

// Chunk swizzle of the LDS tiles: chunk c of row r is stored at c ^ swz(r).
// Over any 16 consecutive rows swz takes 16 distinct values in the low 4 bits
// (row reads of 16 lanes hit 16 distinct 16-byte bank groups), and the 4 rows
// of a transposed read (aligned to 4) get XOR values 4 apart, so chunks c and
// c + 1 of those rows land on 8 distinct bank groups.  At d = 64 two rows share
// a 256-byte bank window and the rotation runs on row / 2.
template <int D> __device__ __forceinline__ int swz(int row) {
  if constexpr (D == 64) {
    const int x = (row >> 1) & 7;
    return ((x & 1) << 2) | (x >> 1);
  } else {
    const int x = row & 15;
    return ((x & 3) << 2) | (x >> 2);
  }
}
template <int D> __device__ __forceinline__ uint32_t tile_byte(int row, int chunk) {
  return (uint32_t)(row * D * 2 + ((chunk ^ swz<D>(row)) << 4));
}

// A wave-uniform address that the compiler holds in VGPRs (it came through
// LDS or a local argument block), moved into SGPRs for the scalar base of dma16_sbase: v_readfirstlane of
// each half (the builtin returns int: back to uint32_t before the halves are
// joined, or bit 31 of the low half would sign-extend over the high half),
// then the 5 wait states that a vector memory instruction reading an SGPR needs
// after a VALU instruction wrote it.  The compiler keeps that distance before
// its own memory instructions, but cannot see that the copies (inline asm) read
// SGPRs.  The s_nop reads both halves, so it follows their writes, and as a
// volatile asm statement it stays ahead of the copies (volatile too).  (The
// halves do not pass through the asm as outputs: the compiler would no longer
// know they are uniform.)
__device__ __forceinline__ const void* sgpr_base(const void* p) {
  const uint64_t x = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(x >> 32));
  asm volatile("s_nop 4" ::"s"(lo), "s"(hi));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo);
}

// Copy R rows (r0.., clamped to N - 1) of a [N, D] head into an LDS tile; each
// instruction of a wave fills 64 consecutive 16-byte slots.  Addressed as the
// wave-uniform row r0 plus a 32-bit per-lane offset, so that no per-lane 64-bit
// address stays live across the kernel's loop.  kVBase: r0 is uniform but the
// compiler cannot prove it (the general-mask kernels' tile bounds, which pass
// through an LDS reduction under segment ids and through a local argument
// block otherwise), so the base goes to scalar registers through sgpr_base.
template <int D, int R, bool kVBase = false, int kNW = kWaves>
__device__ __forceinline__ void load_rows(const uint16_t* __restrict__ head, FA2_LDS uint16_t* dst, int r0, int N,
                                          int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int kPer = R * CPR / (64 * kNW);
  constexpr int kStride = 64 * kNW / CPR;  // rows between a wave's consecutive copies
  static_assert(kPer * 64 * kNW == R * CPR, "tile copy split");
  const uint16_t* base = head + (int64_t)r0 * D;
  if constexpr (kVBase) base = (const uint16_t*)sgpr_base(base);
  const int last = N - 1 - r0;  // rows past it re-read row N - 1
  // From d = 128 on, the lane index as a value the compiler cannot see
  // through: the per-copy offsets below are then formed here, at each call,
  // instead of being kept (or spilled) across the caller's loop.  (At d = 64
  // the kernels have registers to spare and keep them.)
  const int ln = D >= 128 ? (int)opaque_vgpr((uint32_t)lane) : lane;
  // Whole tile at d = 128, and at d = 256 over eight wavefronts: copy t reads
  // 16 * t rows further on and the swizzle repeats every 16 rows, so one lane
  // offset serves every copy and the row step goes in the scalar base.
  // (Measured slower at d = 64 and in the four-wavefront kernels at d = 256,
  // which keep the per-copy offsets below.)
  constexpr bool kOneOffset = D == 128 || (D == 256 && kNW == 8);
  if (kOneOffset && last >= R - 1) {
    static_assert(!kOneOffset || kStride == 16, "row step of the whole-tile copies");
    const uint32_t s0 = (uint32_t)(wave * 64 + ln);
    const uint32_t row = s0 / CPR;
    const uint32_t off = row * D * 2 + (((s0 % CPR) ^ (uint32_t)swz<D>((int)row)) << 4);
#pragma unroll
    for (int t = 0; t < kPer; ++t) dma16_sbase(base + t * kStride * D, off, dst + (t * kNW + wave) * 64 * 8);
    return;
  }
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const int s0 = (t * kNW + wave) * 64;
    const uint32_t s = (uint32_t)(s0 + ln);
    const uint32_t row = s / CPR;
    const uint32_t ch = (s % CPR) ^ (uint32_t)swz<D>((int)row);
    dma16_sbase(base, (uint32_t)min((int)row, last) * D * 2 + ch * 16, dst + s0 * 8);
  }
}

template <int kDType> __device__ __forceinline__ float to_f32(uint16_t x) {
  if constexpr (kDType == 0) return (float)__builtin_bit_cast(_Float16, x);
  else return __uint_as_float((uint32_t)x << 16);
}

// ---------------------------------------------------------------------------
// D = rowsum(dO o O) for every row of every head, in fp32.  16 lanes per row.
template <int kDType, int D>
__global__ __launch_bounds__(256) void fa2_bwd_delta(BwdArgs a) {
  constexpr int kPer = D / 16;  // elements per lane: 4, 8 or 16
  const int t = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * kDeltaRows + (t >> 4);
  const int part = t & 15;
  const int64_t rows = (int64_t)a.BH * a.N;
  float acc = 0.f;
  if (row < rows) {
    const uint16_t* op = a.o + row * D + part * kPer;
    const uint16_t* gp = a.dout + row * D + part * kPer;
#pragma unroll
    for (int c = 0; c < kPer; c += 4) {
      const u32x2 ov = *(const u32x2*)(op + c);
      const u32x2 gv = *(const u32x2*)(gp + c);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        acc += to_f32<kDType>((uint16_t)(ov[h] & 0xffffu)) * to_f32<kDType>((uint16_t)(gv[h] & 0xffffu));
        acc += to_f32<kDType>((uint16_t)(ov[h] >> 16)) * to_f32<kDType>((uint16_t)(gv[h] >> 16));
      }
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (part == 0 && row < rows) a.delta[row] = acc;
}

// ---------------------------------------------------------------------------
// dK and dV of kKeysPerWg keys of one head (d = 64, 128); query tiles stream
// through LDS.
template <int kDType, int D, int kMask>
__global__ __launch_bounds__(kThreads, 2) void fa2_bwd_dkdv(BwdArgs a) {
  constexpr bool kCausal = kMask == kMaskCausal;
  constexpr bool kGeneral = kMask == kMaskGeneral || kMask == kMaskSegments;
  constexpr bool kSeg = kMask == kMaskSegments;
  typedef Elem<kDType> E;
  typedef typename E::V8 V8;
  constexpr int KS = D / 16;  // k-steps of S = Q K^T over the head dim
  constexpr int DB = D / 32;  // 32-wide blocks of the head dim
  static_assert(D == 64 || D == 128, "head dim 256: fa2_bwd_dkdv_pair");
  constexpr int QT = kQTile;  // query rows per streamed tile
  constexpr int kTile = QT * D;
  constexpr int kStat = 64;  // floats per L or D row of the stat buffers (one copy of 64 lanes)
  constexpr int kNStat = kSeg ? 3 : 2;  // stat rows per buffer: L, D (and the rows' segment ids)
  // Operand offsets formed at each use from a few lane values (below) at
  // d = 128, where holding all of them across the loop costs spills.
  constexpr bool kXorAddr = D >= 128;

  // [buffer][Q | dO] tiles, then [buffer][L | D] rows.
  __shared__ __attribute__((aligned(1024))) uint16_t smem_[2 * 2 * kTile];
  __shared__ __attribute__((aligned(1024))) float stat_[2][kNStat][kStat];
  __shared__ int red_[2 * kWaves];  // segment span reduction
  FA2_LDS uint16_t* const sT = (FA2_LDS uint16_t*)smem_;
  FA2_LDS float* const sS = (FA2_LDS float*)&stat_[0][0][0];

  const int N = a.N;
  // Key tiles with a low index see the most query tiles under the causal mask:
  // dispatch all heads' first key tiles first.
  const int kt = blockIdx.x / a.BH;
  const int bh = blockIdx.x - kt * a.BH;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hl = lane >> 5;
  const int col = lane & 31;
  const int kw0 = kt * kKeysPerWg + wave * 32;  // this wave's first key
  const int my_k = kw0 + col;                   // the key of this lane's accumulator column
  const int64_t head_off = (int64_t)bh * N * D;
  const uint16_t* __restrict__ qh = a.q + head_off;
  const uint16_t* __restrict__ gh = a.dout + head_off;
  const float* __restrict__ lh = a.lse + (int64_t)bh * N;
  const float* __restrict__ dh = a.delta + (int64_t)bh * N;
  const int* __restrict__ segb = kSeg ? a.seg + (int64_t)(bh / a.H) * N : nullptr;

  // Query tiles that see these keys: under the causal mask those from the
  // keys' own tile on; under a general mask the rows whose window reaches the
  // keys (every row when a key lies in the prefix), narrowed under segment ids
  // to the rows whose ids lie between the keys' least and greatest id.
  int it0 = kCausal ? (kt * kKeysPerWg) / QT : 0;
  int it1 = (N + QT - 1) / QT;
  if constexpr (kGeneral) {
    const int k0 = kt * kKeysPerWg, k1 = min(N - 1, k0 + kKeysPerWg - 1);
    int lo = 0, hi = N - 1;
    if (k0 >= a.prefix) {
      if (a.wr >= 0) lo = max(0, k0 - a.wr);
      if (a.wl >= 0) hi = min(N - 1, k1 + a.wl);
    }
    if constexpr (kSeg) {
      int f, l;
      segment_span<kWaves>(segb, k0, k1, lo, hi, (FA2_LDS int*)red_, f, l);
      lo = max(lo, f);
      hi = min(hi, l);
    }
    it0 = lo / QT;
    it1 = hi / QT + 1;
  }

  auto load_tile = [&](int it, int buf) __attribute__((always_inline)) {
    load_rows<D, QT, kGeneral>(qh, sT + (2 * buf + 0) * kTile, it * QT, N, wave, lane);
    load_rows<D, QT, kGeneral>(gh, sT + (2 * buf + 1) * kTile, it * QT, N, wave, lane);
    if (wave == 0) {
      const int r = min(it * QT + lane, N - 1);
      dma4(lh + r, sS + (kNStat * buf + 0) * kStat);
      dma4(dh + r, sS + (kNStat * buf + 1) * kStat);
      if constexpr (kSeg) dma4(segb + r, sS + (kNStat * buf + 2) * kStat);
    }
  };
  load_tile(it0, 0);

  // The segment id of this lane's key; whether the wave's 32 keys share one id.
  const int seg_k = kSeg ? segb[min(my_k, N - 1)] : 0;
  int seg_w = 0;
  bool keys_one_seg = false;
  if constexpr (kSeg) {
    seg_w = wave_min(seg_k);
    keys_one_seg = seg_w == wave_max(seg_k);
  }
  // K and V of this lane's key (B operands of S = Q K^T and dP = dO V^T).
  V8 kf[KS], vf[KS];
  {
    const int r = min(my_k, N - 1);
    const uint16_t* kp = a.k + head_off + (int64_t)r * D + 8 * hl;
    const uint16_t* vp = a.v + head_off + (int64_t)r * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = __builtin_bit_cast(V8, *(const u32x4*)(kp + 16 * ks));
      vf[ks] = __builtin_bit_cast(V8, *(const u32x4*)(vp + 16 * ks));
    }
  }
  // The compiler waits for these loads here, once: otherwise it waits for them
  // inside the loop, and that wait (a count of outstanding loads) also waits
  // for the next tile's copies, which the hardware counts alike.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(kf[ks]), "v"(vf[ks]));

  f32x16 dkt[DB], dvt[DB];  // dK^T, dV^T: rows = head dim, columns = this wave's keys
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dkt[db] = f32x16{};
    dvt[db] = f32x16{};
  }

  // Transposed-read addresses (rows = queries of a 16-query k-step, in the
  // order the S accumulator holds them; columns = 4 head dims).
  const int tg = lane >> 4;
  const int tl = lane & 15;

  for (int it = it0; it < it1; ++it) {
    const int buf = (it - it0) & 1;
    // Tile it has landed for every wave; every wave is done with the other buffer.
    wait_vm_lds_barrier<0>();
    if (it + 1 < it1) load_tile(it + 1, buf ^ 1);
    const FA2_LDS uint16_t* tq = sT + (2 * buf + 0) * kTile;
    const FA2_LDS uint16_t* tg_ = sT + (2 * buf + 1) * kTile;
    const FA2_LDS float* tL = sS + (kNStat * buf + 0) * kStat;
    const FA2_LDS float* tD = sS + (kNStat * buf + 1) * kStat;
    const FA2_LDS int* tG = (const FA2_LDS int*)(sS + (kNStat * buf + (kSeg ? 2 : 0)) * kStat);
#pragma unroll
    for (int sb = 0; sb < QT / 32; ++sb) {
      const int q0 = it * QT + sb * 32;
      if (q0 >= N) break;
      if (kCausal && q0 + 31 < kw0) continue;  // every query precedes every key of this wave
      // (wave-uniform) no query of these 32 rows sees a key of this wave
      if (kGeneral && kw0 >= a.prefix &&
          ((a.wr >= 0 && kw0 > q0 + 31 + a.wr) || (a.wl >= 0 && kw0 + 31 < q0 - a.wl)))
        continue;
      // LDS byte offsets of this lane's operand reads.  Row reads (row r of a
      // tile, chunk 2 ks + hl): the swizzle depends on r % 16 only, and
      // (2 ks + hl) ^ z = 2 ks ^ (hl ^ z), so chunk ks sits at
      // r * 2D + ((32 ks) ^ hz16).  Transposed reads (rows r1, r1 + 8, 4 head
      // dims from 32 db + ...): likewise 64 db ^ w16.  At d = 128 the offsets
      // are formed at each use from five lane values derived here, in the
      // loop, from an opaque lane index: held across the loop, the distinct
      // offsets would be spilled.
      const int ln = kXorAddr ? (int)opaque_vgpr((uint32_t)lane) : lane;
      const int lcol = ln & 31, lhl = (ln >> 5) & 1, ltg = (ln >> 4) & 3, ltl = ln & 15;
      const uint32_t hz16 = (uint32_t)((lhl ^ swz<D>(lcol)) << 4);
      const int x0 = 2 * (ltg & 1) + ((ltl & 3) >> 1);
      const int x1 = 4 * (ltg >> 1) + (ltl >> 2);
      const uint32_t w1_16 = (uint32_t)((x0 ^ swz<D>(x1)) << 4), w2_16 = (uint32_t)((x0 ^ swz<D>(x1 + 8)) << 4);
      const uint32_t t1 = (uint32_t)(x1 * D * 2 + 8 * (ltl & 1));
      auto qoff = [&](int ks) __attribute__((always_inline)) {
        if constexpr (kXorAddr) return (uint32_t)((sb * 32 + lcol) * D * 2) + ((uint32_t)(32 * ks) ^ hz16);
        else return tile_byte<D>(sb * 32 + col, 2 * ks + hl);
      };
      // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys.
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t off = qoff(ks);
        const V8 aq = __builtin_bit_cast(V8, *(const FA2_LDS u32x4*)((const FA2_LDS char*)tq + off));
        const V8 ag = __builtin_bit_cast(V8, *(const FA2_LDS u32x4*)((const FA2_LDS char*)tg_ + off));
        s = E::mfma(aq, kf[ks], s);
        dp = E::mfma(ag, vf[ks], dp);
      }
      // Element e of the accumulators is query q0 + 8*(e/4) + 4*hl + e%4 of this
      // lane's key; its L and D sit at the same offset in the stat rows.
      bool need_mask = (q0 + 32 > N) || (kCausal && kw0 + 31 > q0);
      if constexpr (kGeneral) {
        // (wave-uniform) every pair of the 32 x 32 block visible: all rows and
        // keys below N, the keys all in the prefix or the window satisfied at
        // the block's corners, and under segment ids one id for all of them.
        bool full = q0 + 31 < N && kw0 + 31 < N &&
                    (kw0 + 31 < a.prefix || ((a.wl < 0 || kw0 >= q0 + 31 - a.wl) && (a.wr < 0 || kw0 + 31 <= q0 + a.wr)));
        if constexpr (kSeg) {
          if (full) full = keys_one_seg && __all(tG[sb * 32 + col] == seg_w);
        }
        need_mask = !full;
      }
      const int lim_n = N - q0 - 4 * hl;          // query < N      <=> qi < lim_n
      const int lim_c = my_k - q0 - 4 * hl;       // key <= query   <=> qi >= lim_c
      uint32_t pp[2][4], pd[2][4];                // P and dS packed, per 16-query k-step
      // The masked and the unmasked variant as separate branches: one variant
      // with the mask behind a select would evaluate the mask on every block.
      auto probs = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x4 lw = *(const FA2_LDS u32x4*)(tL + sb * 32 + 8 * g + 4 * hl);
          const u32x4 dw = *(const FA2_LDS u32x4*)(tD + sb * 32 + 8 * g + 4 * hl);
          u32x4 sq = {0u, 0u, 0u, 0u};
          if constexpr (kSeg && decltype(masked)::value) sq = *(const FA2_LDS u32x4*)(tG + sb * 32 + 8 * g + 4 * hl);
          float p[4], ds[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = 4 * g + i;
            float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], a.c2, -__uint_as_float(lw[i]) * kLog2e));
            if (decltype(masked)::value && (D != 128 || need_mask)) {
              const int qi = 8 * g + i;
              bool ok = qi < lim_n && (!kCausal || qi >= lim_c);
              if constexpr (kGeneral) {
                const int qa = q0 + 4 * hl + qi;  // the query of this element
                ok = ok &&
                     (my_k < a.prefix || ((a.wl < 0 || my_k >= qa - a.wl) && (a.wr < 0 || my_k <= qa + a.wr)));
                if constexpr (kSeg) ok = ok && (int)sq[i] == seg_k;
              }
              x = ok ? x : 0.f;
            }
            p[i] = x;
            ds[i] = x * (dp[e] - __uint_as_float(dw[i]));
          }
          pp[g >> 1][2 * (g & 1) + 0] = E::pack2(p[0], p[1]);
          pp[g >> 1][2 * (g & 1) + 1] = E::pack2(p[2], p[3]);
          pd[g >> 1][2 * (g & 1) + 0] = E::pack2(ds[0], ds[1]);
          pd[g >> 1][2 * (g & 1) + 1] = E::pack2(ds[2], ds[3]);
        }
      };
      if constexpr (D == 128) {
        // At d = 128 the two variants as separate code exceed the registers
        // (spills): the mask stays a select, evaluated on every block.
        probs(std::true_type{});
      } else {
        if (need_mask) probs(std::true_type{});
        else probs(std::false_type{});
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the two 16-query k-steps.
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const V8 bp = __builtin_bit_cast(V8, u32x4{pp[c][0], pp[c][1], pp[c][2], pp[c][3]});
        const V8 bd = __builtin_bit_cast(V8, u32x4{pd[c][0], pd[c][1], pd[c][2], pd[c][3]});
        const int r1 = sb * 32 + 16 * c + 4 * (tg >> 1) + (tl >> 2);
        const int r2 = r1 + 8;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int dim = 32 * db + 16 * (tg & 1) + 4 * (tl & 3);
          uint32_t o1, o2;
          if constexpr (kXorAddr) {
            const uint32_t rb = (uint32_t)((sb * 32 + 16 * c) * D * 2) + t1;
            o1 = rb + ((uint32_t)(64 * db) ^ w1_16);
            o2 = rb + (uint32_t)(8 * D * 2) + ((uint32_t)(64 * db) ^ w2_16);
          } else {
            o1 = tile_byte<D>(r1, dim >> 3) + 8 * ((dim >> 2) & 1);
            o2 = tile_byte<D>(r2, dim >> 3) + 8 * ((dim >> 2) & 1);
          }
          const u32x2 g1 = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)((const FA2_LDS char*)tg_ + o1)));
          const u32x2 g2 = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)((const FA2_LDS char*)tg_ + o2)));
          const u32x2 q1 = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)((const FA2_LDS char*)tq + o1)));
          const u32x2 q2 = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)((const FA2_LDS char*)tq + o2)));
          dvt[db] = E::mfma(__builtin_bit_cast(V8, u32x4{g1[0], g1[1], g2[0], g2[1]}), bp, dvt[db]);
          dkt[db] = E::mfma(__builtin_bit_cast(V8, u32x4{q1[0], q1[1], q2[0], q2[1]}), bd, dkt[db]);
        }
      }
    }
  }
  // No LDS write may still be in flight when the workgroup retires.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Element e of block db is head dim 32*db + 8*(e/4) + 4*hl + e%4 of key my_k.
  if (my_k < N) {
    uint16_t* kp = a.dk + head_off + (int64_t)my_k * D;
    uint16_t* vp = a.dv + head_off + (int64_t)my_k * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dim = 32 * db + 8 * r4 + 4 * hl;
        *(u32x2*)(kp + dim) = u32x2{E::pack2(dkt[db][4 * r4 + 0] * a.scale, dkt[db][4 * r4 + 1] * a.scale),
                                    E::pack2(dkt[db][4 * r4 + 2] * a.scale, dkt[db][4 * r4 + 3] * a.scale)};
        *(u32x2*)(vp + dim) = u32x2{E::pack2(dvt[db][4 * r4 + 0], dvt[db][4 * r4 + 1]),
                                    E::pack2(dvt[db][4 * r4 + 2], dvt[db][4 * r4 + 3])};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dK and dV at head dim 256.  The dK and dV accumulators of 32 keys take 256
// registers, so one wavefront holding both (with K as an operand) spills.
// Here two wavefronts share each block of 32 keys and split the chain rule
// between them:
//  * wave kb (role 0) holds K of the keys, forms S = Q K^T, the probabilities
//    P = exp(s - L) and accumulates dV^T += dO^T P;
//  * wave kb + 4 (role 1) holds V, forms dP = dO V^T, takes P from role 0
//    through LDS (fp32, so dS is formed from the same values as in a single
//    wavefront), forms dS = P o (dP - D) and accumulates dK^T += Q^T dS.
// Each holds 128 accumulators and a 64-register operand, so the eight
// wavefronts run two per SIMD (the two of a pair on one SIMD when waves are
// placed round-robin): one's elementwise work overlaps the other's products.
// Per streamed tile of 32 query rows: the tile barrier, the first products and
// role 0's probabilities, a barrier that publishes P, then role 1's dS and both
// second products.  Every product and every rounding is the one the
// single-wavefront kernel performs, in the same order.
constexpr int kPairWaves = 8;
constexpr int kPairThreads = 64 * kPairWaves;
// LDS operand fragments read ahead of their products (two under segment ids,
// whose mask state leaves fewer registers).
template <int kMask> constexpr int kPairPipe = kMask == kMaskSegments ? 2 : 4;

template <int kDType, int kMask>
__global__ __launch_bounds__(kPairThreads, 1) void fa2_bwd_dkdv_pair(BwdArgs a) {
  constexpr int D = 256;
  constexpr bool kCausal = kMask == kMaskCausal;
  constexpr bool kGeneral = kMask == kMaskGeneral || kMask == kMaskSegments;
  constexpr bool kSeg = kMask == kMaskSegments;
  typedef Elem<kDType> E;
  typedef typename E::V8 V8;
  constexpr int KS = D / 16;  // k-steps of S = Q K^T and dP = dO V^T
  constexpr int DB = D / 32;  // 32-wide blocks of the head dim
  constexpr int QT = 32;      // query rows per streamed tile
  constexpr int kTile = QT * D;
  constexpr int kStat = 64;
  constexpr int kNStat = kSeg ? 3 : 2;  // stat rows per buffer: L, D (and the rows' segment ids)
  static_assert(kKeysPerWg == 4 * 32, "four key blocks per workgroup");

  __shared__ __attribute__((aligned(1024))) uint16_t smem_[2 * 2 * kTile];  // [buffer][Q | dO]
  __shared__ __attribute__((aligned(1024))) float stat_[2][kNStat][kStat];
  __shared__ __attribute__((aligned(1024))) float xch_[4 * 64 * 16];  // P of each key block, per lane
  __shared__ int red_[2 * kPairWaves];                                // segment span reduction
  FA2_LDS uint16_t* const sT = (FA2_LDS uint16_t*)smem_;
  FA2_LDS float* const sS = (FA2_LDS float*)&stat_[0][0][0];

  const int N = a.N;
  const int kt = blockIdx.x / a.BH;
  const int bh = blockIdx.x - kt * a.BH;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = wave & 3;     // key block
  const int role = wave >> 2;  // 0: S, P, dV; 1: dP, dS, dK
  const int lane = tid & 63;
  const int hl = lane >> 5;
  const int col = lane & 31;
  const int kw0 = kt * kKeysPerWg + kb * 32;  // the pair's first key
  const int my_k = kw0 + col;
  const int64_t head_off = (int64_t)bh * N * D;
  const uint16_t* __restrict__ qh = a.q + head_off;
  const uint16_t* __restrict__ gh = a.dout + head_off;
  const float* __restrict__ lh = a.lse + (int64_t)bh * N;
  const float* __restrict__ dh = a.delta + (int64_t)bh * N;
  const int* __restrict__ segb = kSeg ? a.seg + (int64_t)(bh / a.H) * N : nullptr;

  // Query tiles that see the workgroup's keys (as in fa2_bwd_dkdv).
  int it0 = kCausal ? (kt * kKeysPerWg) / QT : 0;
  int it1 = (N + QT - 1) / QT;
  if constexpr (kGeneral) {
    const int k0 = kt * kKeysPerWg, k1 = min(N - 1, k0 + kKeysPerWg - 1);
    int lo = 0, hi = N - 1;
    if (k0 >= a.prefix) {
      if (a.wr >= 0) lo = max(0, k0 - a.wr);
      if (a.wl >= 0) hi = min(N - 1, k1 + a.wl);
    }
    if constexpr (kSeg) {
      int f, l;
      segment_span<kPairWaves>(segb, k0, k1, lo, hi, (FA2_LDS int*)red_, f, l);
      lo = max(lo, f);
      hi = min(hi, l);
    }
    it0 = lo / QT;
    it1 = hi / QT + 1;
  }

  auto load_tile = [&](int it, int buf) __attribute__((always_inline)) {
    load_rows<D, QT, kGeneral, kPairWaves>(qh, sT + (2 * buf + 0) * kTile, it * QT, N, wave, lane);
    load_rows<D, QT, kGeneral, kPairWaves>(gh, sT + (2 * buf + 1) * kTile, it * QT, N, wave, lane);
    if (wave == 0) {
      const int r = min(it * QT + lane, N - 1);
      dma4(lh + r, sS + (kNStat * buf + 0) * kStat);
      dma4(dh + r, sS + (kNStat * buf + 1) * kStat);
      if constexpr (kSeg) dma4(segb + r, sS + (kNStat * buf + 2) * kStat);
    }
  };
  load_tile(it0, 0);

  // Role 0 masks P: the segment id of its lane's key, and whether the pair's
  // 32 keys share one id.
  const int seg_k = kSeg ? segb[min(my_k, N - 1)] : 0;
  int seg_w = 0;
  bool keys_one_seg = false;
  if constexpr (kSeg) {
    seg_w = wave_min(seg_k);
    keys_one_seg = seg_w == wave_max(seg_k);
  }
  // K (role 0) or V (role 1) of this lane's key: the B operand of the first
  // product.
  V8 bop[KS];
  {
    const uint16_t* src = (role == 0 ? a.k : a.v) + head_off + (int64_t)min(my_k, N - 1) * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bop[ks] = __builtin_bit_cast(V8, *(const u32x4*)(src + 16 * ks));
  }
  // The compiler waits for these loads here, once (see fa2_bwd_dkdv).
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(bop[ks]));
  f32x16 acc[DB];  // role 0: dV^T, role 1: dK^T (rows = head dim, columns = the pair's keys)
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  // P of the pair's block: quarter g (4 values per lane) at ((kb * 4 + g) * 64 +
  // lane) * 4 floats, so that each 16-byte store and load of a wave covers
  // 1 KB of consecutive slots (no bank conflicts).
  FA2_LDS float* const xp = (FA2_LDS float*)xch_ + (kb * 4 * 64 + lane) * 4;

  // Each role runs its own copy of the query loop (the same barriers in the
  // same order), so that the compiler sees which registers each keeps live.
  auto run = [&](auto role_c) __attribute__((always_inline)) {
  constexpr int R = decltype(role_c)::value;
  for (int it = it0; it < it1; ++it) {
    const int buf = (it - it0) & 1;
    // Tile it has landed for every wave; every wave is done with the other
    // buffer and has read the previous tile's P.
    wait_vm_lds_barrier<0>();
    if (it + 1 < it1) load_tile(it + 1, buf ^ 1);
    const FA2_LDS uint16_t* tq = sT + (2 * buf + 0) * kTile;
    const FA2_LDS uint16_t* tg_ = sT + (2 * buf + 1) * kTile;
    const FA2_LDS float* tL = sS + (kNStat * buf + 0) * kStat;
    const FA2_LDS float* tD = sS + (kNStat * buf + 1) * kStat;
    const FA2_LDS int* tG = (const FA2_LDS int*)(sS + (kNStat * buf + (kSeg ? 2 : 0)) * kStat);
    const int q0 = it * QT;
    // (pair-uniform) whether any query of the tile sees a key of this block
    // (a block wholly past N, in the ragged last key tile, only copies)
    bool active = kw0 < N && !(kCausal && q0 + 31 < kw0);
    if constexpr (kGeneral)
      active = kw0 < N && !(kw0 >= a.prefix && ((a.wr >= 0 && kw0 > q0 + 31 + a.wr) ||
                                                (a.wl >= 0 && kw0 + 31 < q0 - a.wl)));
    // LDS operand offsets from lane values formed here, from an opaque lane
    // index, so that the compiler does not hold them across the loop.
    const int ln = (int)opaque_vgpr((uint32_t)lane);
    const int lcol = ln & 31, lhl = (ln >> 5) & 1, ltg = (ln >> 4) & 3, ltl = ln & 15;
    const uint32_t hz16 = (uint32_t)((lhl ^ swz<D>(lcol)) << 4);
    f32x16 x = f32x16{};  // role 0: S, role 1: dP (32 queries x 32 keys)
    uint32_t pk[2][4];    // role 0: P, role 1: dS, packed per 16-query k-step
    if (active) {
      const FA2_LDS char* t1 = (const FA2_LDS char*)(R == 0 ? tq : tg_);
      auto row_frag = [&](int ks) __attribute__((always_inline)) {
        const uint32_t off = (uint32_t)(lcol * D * 2) + ((uint32_t)(32 * ks) ^ hz16);
        return __builtin_bit_cast(V8, *(const FA2_LDS u32x4*)(t1 + off));
      };
      // Operand reads kPairPipe fragments ahead of their products.
      V8 fr[kPairPipe<kMask>];
#pragma unroll
      for (int u = 0; u < kPairPipe<kMask>; ++u) fr[u] = row_frag(u);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
        x = E::mfma(fr[ks % kPairPipe<kMask>], bop[ks], x);
        if (ks + kPairPipe<kMask> < KS) fr[ks % kPairPipe<kMask>] = row_frag(ks + kPairPipe<kMask>);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (R == 0) {
        // Element e is query q0 + 8*(e/4) + 4*hl + e%4 of this lane's key.
        bool need_mask = (q0 + 32 > N) || (kCausal && kw0 + 31 > q0);
        if constexpr (kGeneral) {
          bool full = q0 + 31 < N && kw0 + 31 < N &&
                      (kw0 + 31 < a.prefix ||
                       ((a.wl < 0 || kw0 >= q0 + 31 - a.wl) && (a.wr < 0 || kw0 + 31 <= q0 + a.wr)));
          if constexpr (kSeg) {
            if (full) full = keys_one_seg && __all(tG[col] == seg_w);
          }
          need_mask = !full;
        }
        const int lim_n = N - q0 - 4 * hl;     // query < N     <=> qi < lim_n
        const int lim_c = my_k - q0 - 4 * hl;  // key <= query  <=> qi >= lim_c
        // The masked and the unmasked variant as separate branches: one
        // variant with the mask behind a select would evaluate the mask on
        // every tile.
        auto probs = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const u32x4 lw = *(const FA2_LDS u32x4*)(tL + 8 * g + 4 * hl);
            u32x4 sq = {0u, 0u, 0u, 0u};
            if constexpr (kSeg && decltype(masked)::value) sq = *(const FA2_LDS u32x4*)(tG + 8 * g + 4 * hl);
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int e = 4 * g + i;
              float v = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], a.c2, -__uint_as_float(lw[i]) * kLog2e));
              if constexpr (decltype(masked)::value) {
                const int qi = 8 * g + i;
                bool ok = qi < lim_n && (!kCausal || qi >= lim_c);
                if constexpr (kGeneral) {
                  const int qa = q0 + 4 * hl + qi;
                  ok = ok &&
                       (my_k < a.prefix || ((a.wl < 0 || my_k >= qa - a.wl) && (a.wr < 0 || my_k <= qa + a.wr)));
                  if constexpr (kSeg) ok = ok && (int)sq[i] == seg_k;
                }
                v = ok ? v : 0.f;
              }
              p[i] = v;
            }
            *(FA2_LDS u32x4*)(xp + 256 * g) =
                u32x4{__float_as_uint(p[0]), __float_as_uint(p[1]), __float_as_uint(p[2]), __float_as_uint(p[3])};
            pk[g >> 1][2 * (g & 1) + 0] = E::pack2(p[0], p[1]);
            pk[g >> 1][2 * (g & 1) + 1] = E::pack2(p[2], p[3]);
          }
        };
        if (need_mask) probs(std::true_type{});
        else probs(std::false_type{});
      }
    }
    // Role 0's P is visible to role 1.
    lds_done_barrier();
    if (active) {
      if constexpr (R == 1) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x4 p = *(const FA2_LDS u32x4*)(xp + 256 * g);
          const u32x4 dw = *(const FA2_LDS u32x4*)(tD + 8 * g + 4 * hl);
          float ds[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) ds[i] = __uint_as_float(p[i]) * (x[4 * g + i] - __uint_as_float(dw[i]));
          pk[g >> 1][2 * (g & 1) + 0] = E::pack2(ds[0], ds[1]);
          pk[g >> 1][2 * (g & 1) + 1] = E::pack2(ds[2], ds[3]);
        }
      }
      // dV^T += dO^T P (role 0) or dK^T += Q^T dS (role 1) over the two
      // 16-query k-steps; the A operand is read transposed, its query rows in
      // the order the accumulator of the first product holds them.
      const FA2_LDS char* t2 = (const FA2_LDS char*)(R == 0 ? tg_ : tq);
      const int x0 = 2 * (ltg & 1) + ((ltl & 3) >> 1);
      const int x1 = 4 * (ltg >> 1) + (ltl >> 2);
      const uint32_t w1_16 = (uint32_t)((x0 ^ swz<D>(x1)) << 4), w2_16 = (uint32_t)((x0 ^ swz<D>(x1 + 8)) << 4);
      const uint32_t t1o = (uint32_t)(x1 * D * 2 + 8 * (ltl & 1));
      auto tr_frag = [&](int u) __attribute__((always_inline)) {  // fragment u = (c, db)
        const int c = u / DB, db = u % DB;
        const uint32_t rb = (uint32_t)(16 * c * D * 2) + t1o;
        const uint32_t o1 = rb + ((uint32_t)(64 * db) ^ w1_16);
        const uint32_t o2 = rb + (uint32_t)(8 * D * 2) + ((uint32_t)(64 * db) ^ w2_16);
        const u32x2 r1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)(t2 + o1)));
        const u32x2 r2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)(t2 + o2)));
        return __builtin_bit_cast(V8, u32x4{r1[0], r1[1], r2[0], r2[1]});
      };
      V8 fr[kPairPipe<kMask>];
#pragma unroll
      for (int u = 0; u < kPairPipe<kMask>; ++u) fr[u] = tr_frag(u);
#pragma unroll
      for (int u = 0; u < 2 * DB; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        const int c = u / DB, db = u % DB;
        const V8 bp = __builtin_bit_cast(V8, u32x4{pk[c][0], pk[c][1], pk[c][2], pk[c][3]});
        acc[db] = E::mfma(fr[u % kPairPipe<kMask>], bp, acc[db]);
        if (u + kPairPipe<kMask> < 2 * DB) fr[u % kPairPipe<kMask>] = tr_frag(u + kPairPipe<kMask>);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  };
  if (role == 0) run(std::integral_constant<int, 0>{});
  else run(std::integral_constant<int, 1>{});
  // No LDS write may still be in flight when the workgroup retires.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Element e of block db is head dim 32*db + 8*(e/4) + 4*hl + e%4 of key my_k.
  if (my_k < N) {
    uint16_t* dst = (role == 0 ? a.dv : a.dk) + head_off + (int64_t)my_k * D;
    const float mul = role == 0 ? 1.f : a.scale;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dim = 32 * db + 8 * r4 + 4 * hl;
        *(u32x2*)(dst + dim) = u32x2{E::pack2(acc[db][4 * r4 + 0] * mul, acc[db][4 * r4 + 1] * mul),
                                     E::pack2(acc[db][4 * r4 + 2] * mul, acc[db][4 * r4 + 3] * mul)};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ of kRowsPerWg query rows of one head (d = 64, 128); key/value tiles
// stream through LDS.
template <int kDType, int D, int kMask>
__global__ __launch_bounds__(kThreads, 2) void fa2_bwd_dq(BwdArgs a) {
  constexpr bool kCausal = kMask == kMaskCausal;
  constexpr bool kGeneral = kMask == kMaskGeneral || kMask == kMaskSegments;
  constexpr bool kSeg = kMask == kMaskSegments;
  typedef Elem<kDType> E;
  typedef typename E::V8 V8;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  static_assert(D == 64 || D == 128, "head dim 256: fa2_bwd_dq_pair");
  constexpr int KT = kKTile;  // keys per streamed tile
  constexpr int kTile = KT * D;

  __shared__ __attribute__((aligned(1024))) uint16_t smem_[2 * 2 * kTile];  // [buffer][K | V]
  FA2_LDS uint16_t* const sT = (FA2_LDS uint16_t*)smem_;
  __shared__ __attribute__((aligned(16))) int segk_[kSeg ? 2 * 64 : 4];  // [buffer] the keys' segment ids
  __shared__ int red_[2 * kWaves];                                      // segment span reduction

  const int N = a.N;
  // Under the causal mask the last query tiles see the most keys: dispatch
  // all heads' last tiles first.
  const int level = blockIdx.x / a.BH;
  const int bh = blockIdx.x - level * a.BH;
  const int qt = kCausal ? a.n_q_wg - 1 - level : level;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hl = lane >> 5;
  const int col = lane & 31;
  const int q_row0 = qt * kRowsPerWg + wave * 32;
  const int my_q = q_row0 + col;
  const int64_t head_off = (int64_t)bh * N * D;
  const uint16_t* __restrict__ kh = a.k + head_off;
  const uint16_t* __restrict__ vh = a.v + head_off;

  const int* __restrict__ segb = kSeg ? a.seg + (int64_t)(bh / a.H) * N : nullptr;

  // Key tiles: step j visits tile tile_of(j), j < nt.  Without a general mask
  // tiles 0 .. nt-1 (under the causal mask up to the rows' last key); a general
  // mask visits the runs of key tiles the forward pass visits (the prefix, the
  // window), cut under segment ids to the keys whose ids can match.
  int nt, run_a0 = 0, run_na = 0, run_b0 = 0;
  if constexpr (kGeneral) {
    const int q0 = qt * kRowsPerWg, q1 = min(N, q0 + kRowsPerWg) - 1;
    FwdArgs m{};
    m.N = N;
    m.wl = a.wl;
    m.wr = a.wr;
    m.prefix = a.prefix;
    int kf = 0, kl = N - 1;
    if constexpr (kSeg) {
      const TileRuns all = general_runs(m, q0, q1, 0, N - 1, KT);
      const int lo = all.na > 0 ? 0 : all.b0 * KT;
      const int hi = min(N - 1, (all.b0 + all.nb) * KT - 1);
      segment_span<kWaves>(segb, q0, q1, lo, hi, (FA2_LDS int*)red_, kf, kl);
    }
    const TileRuns r = general_runs(m, q0, q1, kf, kl, KT);
    run_a0 = r.a0;
    run_na = r.na;
    run_b0 = r.b0;
    nt = r.na + r.nb;
  } else {
    const int kv_end = kCausal ? min(N, (qt + 1) * kRowsPerWg) : N;
    nt = (kv_end + KT - 1) / KT;
  }
  auto tile_of = [&](int j) __attribute__((always_inline)) {
    if constexpr (kGeneral) return j < run_na ? run_a0 + j : run_b0 + (j - run_na);
    else return j;
  };

  auto load_tile = [&](int j, int buf) __attribute__((always_inline)) {
    const int kv0 = tile_of(j) * KT;
    load_rows<D, KT, kGeneral>(kh, sT + (2 * buf + 0) * kTile, kv0, N, wave, lane);
    load_rows<D, KT, kGeneral>(vh, sT + (2 * buf + 1) * kTile, kv0, N, wave, lane);
    if (kSeg && wave == 0) dma4(segb + min(kv0 + lane, N - 1), (FA2_LDS int*)segk_ + buf * 64);
  };
  load_tile(0, 0);

  // Q and dO of this lane's query row (B operands of S^T = K Q^T, dP^T = V dO^T),
  // and its L (in log2 units) and D.
  V8 qf[KS], gf[KS];
  const int rq = min(my_q, N - 1);
  {
    const uint16_t* qp = a.q + head_off + (int64_t)rq * D + 8 * hl;
    const uint16_t* gp = a.dout + head_off + (int64_t)rq * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = __builtin_bit_cast(V8, *(const u32x4*)(qp + 16 * ks));
      gf[ks] = __builtin_bit_cast(V8, *(const u32x4*)(gp + 16 * ks));
    }
  }
  float l2 = a.lse[(int64_t)bh * N + rq] * kLog2e;
  float dd = a.delta[(int64_t)bh * N + rq];
  const int seg_q = kSeg ? segb[rq] : 0;
  int seg_w = 0;
  bool rows_one_seg = false;  // the wave's 32 rows share one segment id
  if constexpr (kSeg) {
    seg_w = wave_min(seg_q);
    rows_one_seg = seg_w == wave_max(seg_q);
  }
  // The compiler waits for these loads here, once (see fa2_bwd_dkdv).
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]), "v"(gf[ks]));
  asm volatile("" : "+v"(l2), "+v"(dd));

  f32x16 dqt[DB];  // dQ^T: rows = head dim, columns = this wave's queries
#pragma unroll
  for (int db = 0; db < DB; ++db) dqt[db] = f32x16{};

  const int tg = lane >> 4;
  const int tl = lane & 15;

  for (int j = 0; j < nt; ++j) {
    const int buf = j & 1;
    wait_vm_lds_barrier<0>();
    if (j + 1 < nt) load_tile(j + 1, buf ^ 1);
    const int kv0 = tile_of(j) * KT;
    bool active = !kCausal || kv0 <= q_row0 + 31;
    if constexpr (kGeneral)
      active = !(kv0 >= a.prefix && ((a.wr >= 0 && kv0 > q_row0 + 31 + a.wr) ||
                                     (a.wl >= 0 && kv0 + KT - 1 < q_row0 - a.wl)));
    if (!active) continue;  // wave-uniform; the barriers stay in step
    const FA2_LDS uint16_t* tk = sT + (2 * buf + 0) * kTile;
    const FA2_LDS uint16_t* tv = sT + (2 * buf + 1) * kTile;
    // S^T = K Q^T and dP^T = V dO^T for KT keys x this wave's 32 queries.
    f32x16 s[KT / 32], dp[KT / 32];
#pragma unroll
    for (int kb = 0; kb < KT / 32; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t off = tile_byte<D>(32 * kb + col, 2 * ks + hl);
        const V8 ak = __builtin_bit_cast(V8, *(const FA2_LDS u32x4*)((const FA2_LDS char*)tk + off));
        const V8 av = __builtin_bit_cast(V8, *(const FA2_LDS u32x4*)((const FA2_LDS char*)tv + off));
        s[kb] = E::mfma(ak, qf[ks], s[kb]);
        dp[kb] = E::mfma(av, gf[ks], dp[kb]);
      }
    }
    // Element (kb, e) is key kv0 + 32*kb + 8*(e/4) + 4*hl + e%4 of query my_q.
    const FA2_LDS int* tsg = (const FA2_LDS int*)segk_ + buf * 64;
    bool need_mask = (kv0 + KT > N) || (kCausal && kv0 + KT - 1 > q_row0);
    if constexpr (kGeneral) {
      // (wave-uniform) every pair of the 32 rows x KT keys visible: all keys
      // below N (rows past N are not stored), the keys all in the prefix or the
      // window satisfied at the block's corners, and under segment ids one id
      // for all of them.
      bool full = kv0 + KT <= N && (kv0 + KT - 1 < a.prefix || ((a.wl < 0 || kv0 >= q_row0 + 31 - a.wl) &&
                                                                (a.wr < 0 || kv0 + KT - 1 <= q_row0 + a.wr)));
      if constexpr (kSeg) {
        if (full) full = rows_one_seg && __all(tsg[lane % KT] == seg_w);
      }
      need_mask = !full;
    }
    const int base = kv0 + 4 * hl;
    uint32_t pd[KT / 32][8];
    // Masked and unmasked variants as separate branches (see fa2_bwd_dkdv).
    auto probs = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < KT / 32; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          float ds2[2];
          u32x2 sk = {0u, 0u};
          if constexpr (kSeg && decltype(masked)::value)
            sk = *(const FA2_LDS u32x2*)(tsg + 32 * kb + 8 * (e >> 2) + 4 * hl + (e & 3));
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e + i], a.c2, -l2));
            if constexpr (decltype(masked)::value) {
              const int key = base + 32 * kb + 8 * ((e + i) >> 2) + ((e + i) & 3);
              bool ok = key < N && (!kCausal || key <= my_q);
              if constexpr (kGeneral) {
                ok = ok &&
                     (key < a.prefix || ((a.wl < 0 || key >= my_q - a.wl) && (a.wr < 0 || key <= my_q + a.wr)));
                if constexpr (kSeg) ok = ok && (int)sk[i] == seg_q;
              }
              x = ok ? x : 0.f;
            }
            ds2[i] = x * (dp[kb][e + i] - dd);
          }
          pd[kb][e >> 1] = E::pack2(ds2[0], ds2[1]);
        }
      }
    };
    if (need_mask) probs(std::true_type{});
    else probs(std::false_type{});
    // dQ^T += K^T dS^T over the 16-key k-steps.
#pragma unroll
    for (int c = 0; c < KT / 16; ++c) {
      const V8 bd = __builtin_bit_cast(V8, u32x4{pd[c >> 1][4 * (c & 1) + 0], pd[c >> 1][4 * (c & 1) + 1],
                                                 pd[c >> 1][4 * (c & 1) + 2], pd[c >> 1][4 * (c & 1) + 3]});
      const int r1 = 16 * c + 4 * (tg >> 1) + (tl >> 2);
      const int r2 = r1 + 8;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int dim = 32 * db + 16 * (tg & 1) + 4 * (tl & 3);
        const uint32_t o1 = tile_byte<D>(r1, dim >> 3) + 8 * ((dim >> 2) & 1);
        const uint32_t o2 = tile_byte<D>(r2, dim >> 3) + 8 * ((dim >> 2) & 1);
        const u32x2 k1 = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)((const FA2_LDS char*)tk + o1)));
        const u32x2 k2 = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)((const FA2_LDS char*)tk + o2)));
        dqt[db] = E::mfma(__builtin_bit_cast(V8, u32x4{k1[0], k1[1], k2[0], k2[1]}), bd, dqt[db]);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (my_q < N) {
    uint16_t* qp = a.dq + head_off + (int64_t)my_q * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dim = 32 * db + 8 * r4 + 4 * hl;
        *(u32x2*)(qp + dim) = u32x2{E::pack2(dqt[db][4 * r4 + 0] * a.scale, dqt[db][4 * r4 + 1] * a.scale),
                                    E::pack2(dqt[db][4 * r4 + 2] * a.scale, dqt[db][4 * r4 + 3] * a.scale)};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ at head dim 256.  The dQ accumulators of 32 rows (128 registers) and the
// Q and dO operands of those rows (64 each) do not fit one wavefront's share
// of a SIMD shared with a second wavefront, so two wavefronts share each block
// of 32 query rows:
//  * wave rb (role 0) holds Q of the rows, forms S^T = K Q^T and the
//    probabilities P = exp(s - L), and passes P (fp32) through LDS;
//  * wave rb + 4 (role 1) holds dO, forms dP^T = V dO^T, then dS = P o (dP - D)
//    and accumulates dQ^T += K^T dS^T.
// Eight wavefronts, two per SIMD; every product and rounding as in fa2_bwd_dq.
template <int kDType, int kMask>
__global__ __launch_bounds__(kPairThreads, 1) void fa2_bwd_dq_pair(BwdArgs a) {
  constexpr int D = 256;
  constexpr bool kCausal = kMask == kMaskCausal;
  constexpr bool kGeneral = kMask == kMaskGeneral || kMask == kMaskSegments;
  constexpr bool kSeg = kMask == kMaskSegments;
  typedef Elem<kDType> E;
  typedef typename E::V8 V8;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int KT = 32;  // keys per streamed tile
  constexpr int kTile = KT * D;
  static_assert(kRowsPerWg == 4 * 32, "four row blocks per workgroup");

  __shared__ __attribute__((aligned(1024))) uint16_t smem_[2 * 2 * kTile];  // [buffer][K | V]
  __shared__ __attribute__((aligned(1024))) float xch_[4 * 64 * 16];       // P of each row block, per lane
  __shared__ __attribute__((aligned(16))) int segk_[kSeg ? 2 * 64 : 4];    // [buffer] the keys' segment ids
  __shared__ int red_[2 * kPairWaves];                                     // segment span reduction
  FA2_LDS uint16_t* const sT = (FA2_LDS uint16_t*)smem_;

  const int N = a.N;
  const int level = blockIdx.x / a.BH;
  const int bh = blockIdx.x - level * a.BH;
  const int qt = kCausal ? a.n_q_wg - 1 - level : level;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rb = wave & 3;     // row block
  const int role = wave >> 2;  // 0: S, P; 1: dP, dS, dQ
  const int lane = tid & 63;
  const int hl = lane >> 5;
  const int col = lane & 31;
  const int q_row0 = qt * kRowsPerWg + rb * 32;
  const int my_q = q_row0 + col;
  const int64_t head_off = (int64_t)bh * N * D;
  const uint16_t* __restrict__ kh = a.k + head_off;
  const uint16_t* __restrict__ vh = a.v + head_off;
  const int* __restrict__ segb = kSeg ? a.seg + (int64_t)(bh / a.H) * N : nullptr;

  // Key tiles visited (as in fa2_bwd_dq).
  int nt, run_a0 = 0, run_na = 0, run_b0 = 0;
  if constexpr (kGeneral) {
    const int q0 = qt * kRowsPerWg, q1 = min(N, q0 + kRowsPerWg) - 1;
    FwdArgs m{};
    m.N = N;
    m.wl = a.wl;
    m.wr = a.wr;
    m.prefix = a.prefix;
    int kf = 0, kl = N - 1;
    if constexpr (kSeg) {
      const TileRuns all = general_runs(m, q0, q1, 0, N - 1, KT);
      const int lo = all.na > 0 ? 0 : all.b0 * KT;
      const int hi = min(N - 1, (all.b0 + all.nb) * KT - 1);
      segment_span<kPairWaves>(segb, q0, q1, lo, hi, (FA2_LDS int*)red_, kf, kl);
    }
    const TileRuns r = general_runs(m, q0, q1, kf, kl, KT);
    run_a0 = r.a0;
    run_na = r.na;
    run_b0 = r.b0;
    nt = r.na + r.nb;
  } else {
    const int kv_end = kCausal ? min(N, (qt + 1) * kRowsPerWg) : N;
    nt = (kv_end + KT - 1) / KT;
  }
  auto tile_of = [&](int j) __attribute__((always_inline)) {
    if constexpr (kGeneral) return j < run_na ? run_a0 + j : run_b0 + (j - run_na);
    else return j;
  };

  auto load_tile = [&](int j, int buf) __attribute__((always_inline)) {
    const int kv0 = tile_of(j) * KT;
    load_rows<D, KT, kGeneral, kPairWaves>(kh, sT + (2 * buf + 0) * kTile, kv0, N, wave, lane);
    load_rows<D, KT, kGeneral, kPairWaves>(vh, sT + (2 * buf + 1) * kTile, kv0, N, wave, lane);
    if (kSeg && wave == 0) dma4(segb + min(kv0 + lane, N - 1), (FA2_LDS int*)segk_ + buf * 64);
  };
  load_tile(0, 0);

  // Q (role 0) or dO (role 1) of this lane's query row: the B operand of the
  // first product; L (log2 units) and D of the row.
  const int rq = min(my_q, N - 1);
  V8 bop[KS];
  {
    const uint16_t* src = (role == 0 ? a.q : a.dout) + head_off + (int64_t)rq * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bop[ks] = __builtin_bit_cast(V8, *(const u32x4*)(src + 16 * ks));
  }
  float l2 = a.lse[(int64_t)bh * N + rq] * kLog2e;
  float dd = a.delta[(int64_t)bh * N + rq];
  const int seg_q = kSeg ? segb[rq] : 0;
  int seg_w = 0;
  bool rows_one_seg = false;  // the block's 32 rows share one segment id
  if constexpr (kSeg) {
    seg_w = wave_min(seg_q);
    rows_one_seg = seg_w == wave_max(seg_q);
  }
  // The compiler waits for these loads here, once (see fa2_bwd_dkdv).
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(bop[ks]));
  asm volatile("" : "+v"(l2), "+v"(dd));

  // P of the block: quarter g at ((rb * 4 + g) * 64 + lane) * 4 words (each
  // 16-byte store and load of a wave covers 1 KB of consecutive slots).
  FA2_LDS uint32_t* const xp = (FA2_LDS uint32_t*)xch_ + (rb * 4 * 64 + lane) * 4;

  // Each role runs its own copy of the key loop (the same barriers in the same
  // order), so that the compiler sees which registers each keeps live: role 0
  // holds no dQ accumulators.
  auto run = [&](auto role_c) __attribute__((always_inline)) {
  constexpr int R = decltype(role_c)::value;
  constexpr int kDqt = R == 1 ? DB : 1;
  f32x16 dqt[kDqt];  // role 1: dQ^T (rows = head dim, columns = the block's queries)
#pragma unroll
  for (int db = 0; db < kDqt; ++db) dqt[db] = f32x16{};

  for (int j = 0; j < nt; ++j) {
    const int buf = j & 1;
    // Tile j has landed for every wave; every wave is done with the other
    // buffer and has read the previous tile's P.
    wait_vm_lds_barrier<0>();
    if (j + 1 < nt) load_tile(j + 1, buf ^ 1);
    const int kv0 = tile_of(j) * KT;
    // (pair-uniform) whether a row of the block sees a key of the tile (a
    // block wholly past N, in the ragged last query tile, only copies)
    bool active = q_row0 < N && (!kCausal || kv0 <= q_row0 + 31);
    if constexpr (kGeneral)
      active = q_row0 < N && !(kv0 >= a.prefix && ((a.wr >= 0 && kv0 > q_row0 + 31 + a.wr) ||
                                                   (a.wl >= 0 && kv0 + KT - 1 < q_row0 - a.wl)));
    const FA2_LDS uint16_t* tk = sT + (2 * buf + 0) * kTile;
    const FA2_LDS uint16_t* tv = sT + (2 * buf + 1) * kTile;
    // LDS operand offsets from lane values formed here, from an opaque lane
    // index, so that the compiler does not hold them across the loop (as in
    // fa2_bwd_dkdv at d = 128).
    const int ln = (int)opaque_vgpr((uint32_t)lane);
    const int lcol = ln & 31, lhl = (ln >> 5) & 1, ltg = (ln >> 4) & 3, ltl = ln & 15;
    f32x16 x = f32x16{};  // role 0: S^T, role 1: dP^T (KT keys x 32 queries)
    if (active) {
      const FA2_LDS char* t1 = (const FA2_LDS char*)(R == 0 ? tk : tv);
      const uint32_t hz16 = (uint32_t)((lhl ^ swz<D>(lcol)) << 4);
      auto row_frag = [&](int ks) __attribute__((always_inline)) {
        const uint32_t off = (uint32_t)(lcol * D * 2) + ((uint32_t)(32 * ks) ^ hz16);
        return __builtin_bit_cast(V8, *(const FA2_LDS u32x4*)(t1 + off));
      };
      V8 fr[kPairPipe<kMask>];
#pragma unroll
      for (int u = 0; u < kPairPipe<kMask>; ++u) fr[u] = row_frag(u);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
        x = E::mfma(fr[ks % kPairPipe<kMask>], bop[ks], x);
        if (ks + kPairPipe<kMask> < KS) fr[ks % kPairPipe<kMask>] = row_frag(ks + kPairPipe<kMask>);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (R == 0) {
        // Element e is key kv0 + 8*(e/4) + 4*hl + e%4 of query my_q.
        const FA2_LDS int* tsg = (const FA2_LDS int*)segk_ + buf * 64;
        bool need_mask = (kv0 + KT > N) || (kCausal && kv0 + KT - 1 > q_row0);
        if constexpr (kGeneral) {
          bool full = kv0 + KT <= N && (kv0 + KT - 1 < a.prefix || ((a.wl < 0 || kv0 >= q_row0 + 31 - a.wl) &&
                                                                    (a.wr < 0 || kv0 + KT - 1 <= q_row0 + a.wr)));
          if constexpr (kSeg) {
            if (full) full = rows_one_seg && __all(tsg[lane % KT] == seg_w);
          }
          need_mask = !full;
        }
        const int base = kv0 + 4 * hl;
        // Masked and unmasked variants as separate branches (see
        // fa2_bwd_dkdv_pair).
        auto probs = [&](auto masked) __attribute__((always_inline)) {
          float p[16];
#pragma unroll
          for (int e = 0; e < 16; e += 2) {
            u32x2 sk = {0u, 0u};
            if constexpr (kSeg && decltype(masked)::value)
              sk = *(const FA2_LDS u32x2*)(tsg + 8 * (e >> 2) + 4 * hl + (e & 3));
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              float v = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e + i], a.c2, -l2));
              if constexpr (decltype(masked)::value) {
                const int key = base + 8 * ((e + i) >> 2) + ((e + i) & 3);
                bool ok = key < N && (!kCausal || key <= my_q);
                if constexpr (kGeneral) {
                  ok = ok &&
                       (key < a.prefix || ((a.wl < 0 || key >= my_q - a.wl) && (a.wr < 0 || key <= my_q + a.wr)));
                  if constexpr (kSeg) ok = ok && (int)sk[i] == seg_q;
                }
                v = ok ? v : 0.f;
              }
              p[e + i] = v;
            }
          }
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *(FA2_LDS u32x4*)(xp + 256 * g) = u32x4{__float_as_uint(p[4 * g + 0]), __float_as_uint(p[4 * g + 1]),
                                                  __float_as_uint(p[4 * g + 2]), __float_as_uint(p[4 * g + 3])};
        };
        if (need_mask) probs(std::true_type{});
        else probs(std::false_type{});
      }
    }
    // Role 0's P is visible to role 1.
    lds_done_barrier();
    if (R == 1 && active) {
      uint32_t pd[8];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x4 p = *(const FA2_LDS u32x4*)(xp + 256 * g);
        float ds[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ds[i] = __uint_as_float(p[i]) * (x[4 * g + i] - dd);
        pd[2 * g + 0] = E::pack2(ds[0], ds[1]);
        pd[2 * g + 1] = E::pack2(ds[2], ds[3]);
      }
      // dQ^T += K^T dS^T over the two 16-key k-steps; K^T is read transposed,
      // rows 16 c + x1 and + 8 (the swizzle of a row depends on its low 4
      // bits), 4 head dims from 32 db + 4 x0.
      const int x0 = 2 * (ltg & 1) + ((ltl & 3) >> 1);
      const int x1 = 4 * (ltg >> 1) + (ltl >> 2);
      const uint32_t w1_16 = (uint32_t)((x0 ^ swz<D>(x1)) << 4), w2_16 = (uint32_t)((x0 ^ swz<D>(x1 + 8)) << 4);
      const uint32_t t1o = (uint32_t)(x1 * D * 2 + 8 * (ltl & 1));
      auto tr_frag = [&](int u) __attribute__((always_inline)) {  // fragment u = (c, db)
        const int c = u / DB, db = u % DB;
        const uint32_t rbase = (uint32_t)(16 * c * D * 2) + t1o;
        const uint32_t o1 = rbase + ((uint32_t)(64 * db) ^ w1_16);
        const uint32_t o2 = rbase + (uint32_t)(8 * D * 2) + ((uint32_t)(64 * db) ^ w2_16);
        const u32x2 k1 = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)((const FA2_LDS char*)tk + o1)));
        const u32x2 k2 = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)((const FA2_LDS char*)tk + o2)));
        return __builtin_bit_cast(V8, u32x4{k1[0], k1[1], k2[0], k2[1]});
      };
      // Operand reads kPairPipe fragments ahead of their products.
      V8 fr[kPairPipe<kMask>];
#pragma unroll
      for (int u = 0; u < kPairPipe<kMask>; ++u) fr[u] = tr_frag(u);
#pragma unroll
      for (int u = 0; u < (KT / 16) * DB; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        const int c = u / DB, db = u % DB;
        const V8 bd = __builtin_bit_cast(V8, u32x4{pd[4 * c + 0], pd[4 * c + 1], pd[4 * c + 2], pd[4 * c + 3]});
        dqt[db % kDqt] = E::mfma(fr[u % kPairPipe<kMask>], bd, dqt[db % kDqt]);
        if (u + kPairPipe<kMask> < (KT / 16) * DB) fr[u % kPairPipe<kMask>] = tr_frag(u + kPairPipe<kMask>);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (R == 1 && my_q < N) {
    uint16_t* qp = a.dq + head_off + (int64_t)my_q * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dim = 32 * db + 8 * r4 + 4 * hl;
        *(u32x2*)(qp + dim) =
            u32x2{E::pack2(dqt[db % kDqt][4 * r4 + 0] * a.scale, dqt[db % kDqt][4 * r4 + 1] * a.scale),
                  E::pack2(dqt[db % kDqt][4 * r4 + 2] * a.scale, dqt[db % kDqt][4 * r4 + 3] * a.scale)};
      }
    }
  }
  };
  if (role == 0) run(std::integral_constant<int, 0>{});
  else run(std::integral_constant<int, 1>{});
}

}  // namespace bwd
}  // namespace fa2
