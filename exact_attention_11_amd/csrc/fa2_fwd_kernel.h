// fa2_fwd_kernel.h -- fused exact-attention forward pass for gfx950 (CDNA4).
//
// One workgroup owns one tile of kBr = 128 query rows of one (batch, head) and
// streams the key/value tiles of that head through LDS, kBc = 64 keys at a time.
// The N x N score matrix never leaves registers.  What the pages fix, and what
// this kernel does with it:
//
//  * Query tiles outside, key/value tiles inside; each query tile is loaded once
//    and its output written once ("6.2 FlashAttention V2 in depth", section 2.2).
//    The grid runs over (query tile x head x batch), so one long sequence at
//    batch 1 still fills the chip ("FlashAttention-2: Where the Second 2x
//    Actually Comes From", section "Parallelism over sequence length").
//  * Split-Q: each of the 4 wavefronts owns 32 whole query rows and sees the
//    full key tile, so row max and row sum never cross wavefronts
//    ("6.2 FlashAttention V2 in depth", section 4.2).
//  * Online softmax with an unnormalised output accumulator, divided by the row
//    sum once after the key loop, and the logsumexp L = m + log l kept per row
//    ("6.2 FlashAttention V2 in depth", sections 3.2, 6.1 and 7.1).
//  * Causal block classes: key tiles past the query tile are never visited,
//    tiles crossing the diagonal are masked element by element, the rest run
//    unmasked ("6.2 FlashAttention V2 in depth", section 5.3).
//
// gfx950 mapping (prior art adapted, not copied):
//  * Both products run on v_mfma_f32_32x32x16_{f16,bf16} with fp32 accumulation.
//    Scores are formed transposed, S^T = K Q^T, so each lane holds 16 keys of a
//    single query per 32x32 block: a row max or row sum is an in-lane reduction
//    plus one v_permlane32_swap exchange with the partner lane (l ^ 32).
//  * The output is accumulated transposed too, O^T += V^T P^T: the probabilities
//    leave the score accumulator already in the B-operand layout (the key order
//    inside an MFMA k-step is permuted consistently on both operands), and V^T
//    fragments come straight from the row-major V tile in LDS through
//    ds_read_b64_tr_b16.
//  * K and V tiles go global -> LDS with global_load_lds_dwordx4 (no register
//    staging), into two single buffers that alternate: the next K tile streams
//    in under the softmax and P.V of the current tile, the next V tile under the
//    next S = K Q^T.  16-byte chunks are XOR-swizzled per row so that the
//    fragment reads of one instruction fall in distinct LDS banks.
//  * exp2 with the multiplier and log2(e) folded into one FMA.  The running max
//    used as the exponent's reference is only moved when a row's tile max
//    exceeds it by more than kTau (log2 units), so the O rescale runs rarely;
//    the weights then stay below 2^kTau, and the result is the same
//    mathematically (the final division and L use the same reference).
//  * Workgroup ids are remapped so that the round-robin dispatch over the 8 XCDs
//    gives each XCD a contiguous range of heads (its L2 keeps that head's K/V),
//    and causal query tiles are issued heaviest first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa2 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FA2_LDS __attribute__((address_space(3)))

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;  // query rows per workgroup
constexpr int kBc = 64;           // keys per K/V tile
constexpr float kTau = 8.0f;      // lazy-rescale threshold, log2 units

// Element-type specific pieces: the MFMA and the fp32 -> storage conversion.
template <int kDType> struct Elem;
template <> struct Elem<0> {  // fp16
  typedef f16x8 V8;
  __device__ static inline f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float a, float b) {  // round to nearest even
    f16x2 h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
  }
};
template <> struct Elem<1> {  // bf16
  typedef bf16x8 V8;
  __device__ static inline f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float a, float b) {  // round to nearest even
    bf16x2 h = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, h);
  }
};

// XOR swizzles of the 16-byte chunk index inside a tile row.
//  K: the A-operand read of one MFMA touches 32 rows at the same logical chunk;
//     the swizzle spreads every 16 consecutive rows over 16 distinct 16-byte
//     bank groups (rows of 128 bytes pair up, hence the shift for d = 64).
//  V: a transposed read touches 4 consecutive rows x 64 bytes per half wave;
//     the swizzle puts those 4 rows in 4 distinct 64-byte bank windows.
template <int D> __device__ __forceinline__ int swz_k(int row) {
  return D == 64 ? ((row >> 1) & 7) : (row & 15);
}
template <int D> __device__ __forceinline__ int swz_v(int row) {
  return D == 64 ? (((row >> 1) & 1) << 2) : ((row & 3) << 2);
}

// s_waitcnt vmcnt(n) followed by a workgroup barrier.  The explicit count lets
// the other buffer's load stay in flight across the barrier.
template <int N> __device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"(N) : "memory");
}
// All of this wave's LDS reads have returned, then a workgroup barrier: after it
// the buffer may be overwritten.
__device__ __forceinline__ void lds_done_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second.  With x in both, one result holds this lane's own
// value and the other the value of lane l ^ 32 (which one depends on the half),
// so a symmetric combination of the two is the combination across the pair.
__device__ __forceinline__ u32x2 pair32(float x) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false));
}
__device__ __forceinline__ float max_pair32(float x) {
  const u32x2 r = pair32(x);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_pair32(float x) {
  const u32x2 r = pair32(x);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int N;         // sequence length
  int n_qtiles;  // ceil(N / kBr)
  int n_wg;      // B * H * n_qtiles
  float c2;      // scale * log2(e)
};

// One global_load_lds_dwordx4: every lane copies 16 bytes from its own global
// address to lds_base + 16 * lane (lds_base is wave-uniform and goes in M0).
// Written as inline asm so that the compiler does not track it: the compiler
// would otherwise wait for every outstanding LDS copy before any LDS read, while
// the loop below waits with exact counts (s_waitcnt vmcnt) for the tile it needs.
__device__ __forceinline__ void dma16(const void* g, FA2_LDS void* lds_base) {
  const uint32_t m0v = (uint32_t)(size_t)lds_base;
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0v) : "memory");
}

// Issue the global -> LDS copy of one kBc x D tile (rows kv0.., clamped to N-1).
// Each instruction of a wave fills 64 consecutive 16-byte LDS slots; slot s
// holds logical chunk (s % CPR) ^ swz(row) of row s / CPR.
template <int D, bool kIsV>
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ src_head, FA2_LDS uint16_t* dst,
                                          int kv0, int N, int wave, int lane) {
  constexpr int CPR = D / 8;                        // 16-byte chunks per row
  constexpr int kPerWave = kBc * CPR / (64 * kWaves);  // instructions per wave
#pragma unroll
  for (int t = 0; t < kPerWave; ++t) {
    const int s0 = (t * kWaves + wave) * 64;
    const int s = s0 + lane;
    const int row = s / CPR;
    const int chp = s % CPR;
    const int ch = chp ^ (kIsV ? swz_v<D>(row) : swz_k<D>(row));
    const int grow = min(kv0 + row, N - 1);
    const uint16_t* g = src_head + (int64_t)grow * D + ch * 8;
    dma16(g, dst + s0 * 8);
  }
}

template <int kDType, int D, bool kCausal>
__global__ __launch_bounds__(kThreads, D == 256 ? 1 : 2) void fa2_fwd_kernel(FwdArgs a) {
  typedef Elem<kDType> E;
  typedef typename E::V8 V8;
  constexpr int CPR = D / 8;
  constexpr int KS = D / 16;  // MFMA k-steps of S = K Q^T
  constexpr int DB = D / 32;  // 32-wide blocks of the output columns
  constexpr int kLoads = kBc * CPR / (64 * kWaves);
  constexpr float kLn2 = 0.69314718055994530942f;
  constexpr float kNegInf = -__builtin_huge_valf();

  __shared__ __attribute__((aligned(1024))) uint16_t sK_[kBc * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sV_[kBc * D];
  FA2_LDS uint16_t* const sK = (FA2_LDS uint16_t*)sK_;
  FA2_LDS uint16_t* const sV = (FA2_LDS uint16_t*)sV_;

  const int N = a.N;
  // Workgroup -> (head, query tile).  Consecutive dispatch ids go round-robin
  // over the 8 XCDs; regroup so each XCD walks a contiguous range of heads.
  const int w = blockIdx.x;
  int sidx = w;
  if ((a.n_wg & 7) == 0) sidx = (w & 7) * (a.n_wg >> 3) + (w >> 3);
  const int bh = sidx / a.n_qtiles;
  const int it = sidx - bh * a.n_qtiles;
  const int qtile = kCausal ? (a.n_qtiles - 1 - it) : it;  // causal: heaviest first

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hl = lane >> 5;   // which half of the wave
  const int col = lane & 31;  // query column of S^T / O^T held by this lane
  const int q_row0 = qtile * kBr + wave * 32;
  const int my_q = q_row0 + col;
  const int64_t head_off = (int64_t)bh * N * D;
  const uint16_t* __restrict__ kh = a.k + head_off;
  const uint16_t* __restrict__ vh = a.v + head_off;

  const int kv_end = kCausal ? min(N, (qtile + 1) * kBr) : N;
  const int nt = (kv_end + kBc - 1) / kBc;

  // First K and V tiles start streaming before anything else.
  load_tile<D, false>(kh, sK, 0, N, wave, lane);
  load_tile<D, true>(vh, sV, 0, N, wave, lane);

  // Q fragments (B operand of S^T = K Q^T), loaded once and kept in registers.
  // They are consumed right here so that the compiler's own wait for them
  // happens once, outside the loop (it also covers the two tile copies above).
  V8 qf[KS];
  {
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

  for (int j = 0; j < nt; ++j) {
    const int kv0 = j * kBc;
    // Wave-uniform classification of this tile for this wave's 32 rows.
    const bool active = !kCausal || kv0 <= q_row0 + 31;
    const bool need_mask = (kv0 + kBc > N) || (kCausal && kv0 + kBc - 1 > q_row0);
    const bool generic = need_mask || !(a.c2 > 0.f);

    wait_vm_barrier<kLoads>();  // K_j has landed (V_j may still be in flight)
    f32x16 s[2];
    if (active) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const int row = 32 * kb + col;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int ch = (2 * ks + hl) ^ swz_k<D>(row);
          const V8 kf = __builtin_bit_cast(V8, *(const FA2_LDS u32x4*)(sK + (row * CPR + ch) * 8));
          s[kb] = E::mfma(kf, qf[ks], s[kb]);
        }
      }
    }
    lds_done_barrier();  // every wave is done with sK
    // The prefetch is issued on every step (the last step re-reads its own
    // tile, which nobody consumes) so that the number of loads in flight is the
    // same on every path through the loop.
    const int kv_next = j + 1 < nt ? kv0 + kBc : kv0;
    load_tile<D, false>(kh, sK, kv_next, N, wave, lane);

    uint32_t pk[2][8];  // probabilities, packed pairs, B-operand order
    if (active) {
      float mul = a.c2;
      if (generic) {
        // Scale first, then mask: t = -inf for keys past N or after the query.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
            const bool masked = key >= N || (kCausal && key > my_q);
            const float t = s[kb][r] * a.c2;
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

    wait_vm_barrier<kLoads>();  // V_j has landed (K_{j+1} may be in flight)
    if (active) {
      const int g = lane >> 4;
      const int L = lane & 15;
#pragma unroll
      for (int c = 0; c < kBc / 16; ++c) {
        const u32x4 bw = {pk[c >> 1][4 * (c & 1) + 0], pk[c >> 1][4 * (c & 1) + 1],
                          pk[c >> 1][4 * (c & 1) + 2], pk[c >> 1][4 * (c & 1) + 3]};
        const V8 bop = __builtin_bit_cast(V8, bw);
        const int kr1 = 16 * c + 4 * (g >> 1) + (L >> 2);
        const int kr2 = kr1 + 8;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int dim = 32 * db + 16 * (g & 1) + 4 * (L & 3);
          const int ch = dim >> 3;
          const int hv = (dim >> 2) & 1;
          const FA2_LDS uint16_t* p1 = sV + (kr1 * CPR + (ch ^ swz_v<D>(kr1))) * 8 + 4 * hv;
          const FA2_LDS uint16_t* p2 = sV + (kr2 * CPR + (ch ^ swz_v<D>(kr2))) * 8 + 4 * hv;
          const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)p1);
          const i16x4 t2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)p2);
          const u32x2 w1 = __builtin_bit_cast(u32x2, t1);
          const u32x2 w2 = __builtin_bit_cast(u32x2, t2);
          const u32x4 aw = {w1[0], w1[1], w2[0], w2[1]};
          o[db] = E::mfma(__builtin_bit_cast(V8, aw), bop, o[db]);
        }
      }
    }
    lds_done_barrier();  // every wave is done with sV
    load_tile<D, true>(vh, sV, kv_next, N, wave, lane);
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

}  // namespace fa2
