// fa2_common.h -- pieces shared by the gfx950 attention forward kernels:
// vector types, the per-element-type MFMA and conversions, LDS copy and
// barrier primitives, cross-half reductions and the kernel argument block.
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

// Lazy-rescale threshold in log2 units: the reference max of a row only moves
// when a tile's row max exceeds it by more than this, so unnormalised weights
// stay below 2^kTau (far inside the fp16 range).
constexpr float kTau = 8.0f;
// A lane's share of a tile's row sum at most this bounds each of its weights by
// 2^kTau as well (the weights are non-negative).
constexpr float kSumCap = 256.0f;
constexpr float kLn2 = 0.69314718055994530942f;

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int N;         // sequence length
  int n_qtiles;  // ceil(N / query rows per workgroup)
  int n_wg;      // B * H * n_qtiles
  float c2;      // scale * log2(e)
  // General mask (used by the kMaskGeneral instances only): key c is visible
  // to query r iff c < N, seg[b, c] == seg[b, r] (when seg is given), and
  // c < prefix or r - wl <= c <= r + wr (a negative bound is no bound).
  int wl;
  int wr;
  int prefix;
  int H;            // heads per batch: batch b = (b*H + h) / H
  const int* seg;   // [B, N] segment ids, or nullptr
};

// Mask modes of the forward kernels.
constexpr int kMaskNone = 0;
constexpr int kMaskCausal = 1;
constexpr int kMaskGeneral = 2;

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

// One global_load_lds_dwordx4: every lane copies 16 bytes from its own global
// address to lds_base + 16 * lane (lds_base is wave-uniform and goes in M0).
// Written as inline asm so that the compiler does not track it: the compiler
// would otherwise wait for every outstanding LDS copy before any LDS read,
// while the kernels wait with exact counts (s_waitcnt vmcnt) for the tile they
// need.
__device__ __forceinline__ void dma16(const void* g, FA2_LDS void* lds_base) {
  const uint32_t m0v = (uint32_t)(size_t)lds_base;
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0v) : "memory");
}
// The same copy addressed as a wave-uniform base (SGPR pair) plus a per-lane
// 32-bit byte offset.
__device__ __forceinline__ void dma16_sbase(const void* sbase, uint32_t voff, FA2_LDS void* lds_base) {
  const uint32_t m0v = (uint32_t)(size_t)lds_base;
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m0v) : "memory");
}

// One global_load_lds_dword: every lane copies 4 bytes to lds_base + 4 * lane.
__device__ __forceinline__ void dma4(const void* g, FA2_LDS void* lds_base) {
  const uint32_t m0v = (uint32_t)(size_t)lds_base;
  asm volatile("global_load_lds_dword %0, off" ::"v"(g), "{m0}"(m0v) : "memory");
}

// s_waitcnt vmcnt(n) followed by a workgroup barrier.  The explicit count lets
// later copies stay in flight across the barrier.
template <int N> __device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"(N) : "memory");
}
// Same, and also every LDS access of this wave has completed first.
template <int N> __device__ __forceinline__ void wait_vm_lds_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(N) : "memory");
}
// All of this wave's LDS accesses have completed, then a workgroup barrier:
// after it the buffers this wave read may be overwritten and what it wrote is
// visible.
__device__ __forceinline__ void lds_done_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The value itself, computed into a VGPR the compiler cannot see through: the
// addresses derived from it stay "base + immediate offset" instead of being
// re-associated into one register (and one add per step) per access.
__device__ __forceinline__ uint32_t opaque_vgpr(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second.  With x in both, one result holds this lane's own
// value and the other the value of lane l ^ 32 (which one depends on the half),
// so a symmetric combination of the two is the combination across the pair.
__device__ __forceinline__ u32x2 pair32(float x) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                                     false));
}
__device__ __forceinline__ float max_pair32(float x) {
  const u32x2 r = pair32(x);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_pair32(float x) {
  const u32x2 r = pair32(x);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup id -> (head, query tile).  Consecutive dispatch ids go round-robin
// over the 8 XCDs (32 CUs and one L2 each on MI355X), so id w runs on XCD w % 8.
//  * Without a mask every tile costs the same: regroup the ids so that each XCD
//    walks a contiguous range of heads (its L2 then serves that head's K/V to
//    every query tile).
//  * Under a causal mask tile cost grows with the tile index.  When the head
//    count is a multiple of 8, XCD x takes heads x, x + 8, ... in groups of g
//    heads, g = 32 / (query tiles per head) (at least 1): inside a group the
//    query tiles go heaviest first across the group's heads.  A group then
//    fills about one round of the XCD's CUs, which keeps the concurrent
//    workgroups on few heads (L2 reuse) while every CU's queue still runs
//    heaviest first.  Otherwise all heads' heaviest tiles go first.
constexpr int kCusPerXcd = 32;
__device__ __forceinline__ void wg_to_tile(const FwdArgs& a, bool causal, int& bh, int& qtile) {
  const int w = blockIdx.x;
  const int nq = a.n_qtiles;
  const int n_bh = a.n_wg / nq;
  if (causal) {
    if ((n_bh & 7) == 0) {
      const int x = w & 7, it = w >> 3;
      const int hpx = n_bh >> 3;  // heads per XCD
      int g = kCusPerXcd / nq;
      g = g < 1 ? 1 : (g > hpx ? hpx : g);
      const int grp = it / (g * nq);
      const int r = it - grp * g * nq;
      const int gg = min(g, hpx - grp * g);  // the last group may be smaller
      const int level = r / gg;
      bh = (grp * g + (r - level * gg)) * 8 + x;
      qtile = nq - 1 - level;
    } else {
      const int level = w / n_bh;
      bh = w - level * n_bh;
      qtile = nq - 1 - level;
    }
    return;
  }
  int sidx = w;
  if ((a.n_wg & 7) == 0) sidx = (w & 7) * (a.n_wg >> 3) + (w >> 3);
  bh = sidx / nq;
  qtile = sidx - bh * nq;
}

}  // namespace fa2
