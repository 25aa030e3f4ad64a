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
typedef int i32x8 __attribute__((ext_vector_type(8)));

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
  // General mask (used by the kMaskGeneral and kMaskSegments instances only):
  // key c is visible to query r iff c < N, seg[b, c] == seg[b, r] (segment
  // instances), and c < prefix or r - wl <= c <= r + wr (a negative bound is
  // no bound).
  int wl;
  int wr;
  int prefix;
  int H;            // heads per batch: batch b = (b*H + h) / H
  const int* seg;   // [B, N] segment ids, or nullptr
  int grow;         // general mask whose tile cost grows with the query tile (order those heaviest first)
  // fp8 instances: per-(batch, head) factors that turn the stored e4m3 values
  // of Q and K into real ones (nullptr: 1).
  const float* descale_q;
  const float* descale_k;
};

// Element types of the forward kernels: Q, K, V and O in fp16 or bf16, or Q and
// K in fp8 (OCP e4m3) with V and O in fp16 or bf16.
constexpr int kFp16 = 0;
constexpr int kBf16 = 1;
constexpr int kFp8Fp16 = 2;
constexpr int kFp8Bf16 = 3;

// Mask modes of the forward kernels.
constexpr int kMaskNone = 0;
constexpr int kMaskCausal = 1;
constexpr int kMaskGeneral = 2;   // window and prefix
constexpr int kMaskSegments = 3;  // window, prefix and segment ids

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

// S^T = K Q^T over 64 k-elements of fp8 (OCP e4m3) K and Q, fp32 accumulation:
// v_mfma_f32_32x32x64_f8f6f4 with both operand formats e4m3 (format code 0) and
// no block scales.  Lane l holds 32 consecutive k-bytes of row l % 32 of its
// operand; which 32 (the lane half) only has to agree between the two
// operands.  A template, like Elem's products, so that the host pass of the
// kernels that call it (which only emits their launch stubs) never checks the
// gfx950-only builtin.
template <int kFormat = 0> __device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, kFormat, kFormat, 0, 0, 0, 0);
}

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

// Wave-wide minimum and maximum (every lane receives the result).
__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = min(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = max(x, __shfl_xor(x, m));
  return x;
}

// Key tiles (of bc keys) that a general mask leaves to the query rows q0..q1,
// as at most two runs of consecutive tiles: the prefix, then the window around
// the rows (one run when the two meet).  Step s of the key loop visits tile
// a0 + s for s < na, else b0 + s - na.  Both runs are cut to the keys kf..kl
// (the keys whose segment ids can match those of the rows; 0..N-1 without
// segment ids).  Row q0 always sees key q0, so na + nb >= 1.
struct TileRuns {
  int a0, na, b0, nb;
};
__device__ __forceinline__ TileRuns general_runs(const FwdArgs& a, int q0, int q1, int kf, int kl, int bc) {
  const int N = a.N;
  const int w_lo = a.wl < 0 ? 0 : max(0, q0 - a.wl);
  const int w_hi = a.wr < 0 ? N - 1 : min(N - 1, q1 + a.wr);
  int b0 = w_lo / bc, b1 = w_hi / bc + 1;          // window tiles [b0, b1)
  int a0 = 0, a1 = (min(a.prefix, N) + bc - 1) / bc;  // prefix tiles [0, a1)
  if (a1 >= b0) {  // the runs touch: one run
    b0 = 0;
    b1 = max(a1, b1);
    a1 = 0;
  }
  const int f = kf / bc, l = kl / bc + 1;
  a0 = max(a0, f);
  a1 = min(a1, l);
  b0 = max(b0, f);
  b1 = min(b1, l);
  TileRuns r;
  r.a0 = a0;
  r.na = max(0, a1 - a0);
  r.b0 = b0;
  r.nb = max(0, b1 - b0);
  return r;
}

// Under segment ids: the first and last key in lo..hi whose id lies between the
// least and the greatest id of the rows q0..q1 (kf, kl).  Every key that one of
// those rows may see lies in kf..kl (and with ids that never decrease along the
// sequence, documents, the bound is tight).  The rows' own keys match, so only
// lo..q0-1 and q1+1..hi are read (q0..q1 must lie in lo..hi).  All threads of
// the workgroup take part; red holds 2 ints per wave.  The row ids and the first
// batch of key ids are all in flight at once, so a span of up to
// kUnroll * 64 * kWaves keys costs one round trip to L2.
template <int kWaves>
__device__ void segment_span(const int* __restrict__ segb, int q0, int q1, int lo, int hi, FA2_LDS int* red,
                             int& kf, int& kl) {
  constexpr int kThreads = 64 * kWaves;
  constexpr int kRowLoads = (32 * kWaves + 63) / 64;  // rows q0..q1 over the 64 lanes of each wave
  constexpr int kUnroll = 32;                         // key loads in flight per lane
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nl = q0 - lo, n = nl + (hi - q1);  // keys left of the rows, then right of them
  int rv[kRowLoads];
#pragma unroll
  for (int u = 0; u < kRowLoads; ++u) rv[u] = segb[min(q0 + lane + 64 * u, q1)];
  int kv[kUnroll];
  auto load_batch = [&](int base) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = base + u * kThreads + tid;
      const int c = i >= n ? q0 : (i < nl ? lo + i : q1 + 1 + (i - nl));
      kv[u] = segb[c];
    }
  };
  load_batch(0);
  int qmin = rv[0], qmax = rv[0];
#pragma unroll
  for (int u = 1; u < kRowLoads; ++u) {
    qmin = min(qmin, rv[u]);
    qmax = max(qmax, rv[u]);
  }
  qmin = wave_min(qmin);
  qmax = wave_max(qmax);
  int f = q0, l = q1;
  for (int base = 0;;) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = base + u * kThreads + tid;
      const int c = i < nl ? lo + i : q1 + 1 + (i - nl);
      if (i < n && kv[u] >= qmin && kv[u] <= qmax) {
        f = min(f, c);
        l = max(l, c);
      }
    }
    base += kUnroll * kThreads;
    if (base >= n) break;
    load_batch(base);
  }
  f = wave_min(f);
  l = wave_max(l);
  if (lane == 0) {
    red[2 * wave] = f;
    red[2 * wave + 1] = l;
  }
  __syncthreads();
  kf = red[0];
  kl = red[1];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    kf = min(kf, red[2 * w]);
    kl = max(kl, red[2 * w + 1]);
  }
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
//    General masks whose cost grows with the row (a right bound and no left
//    bound) are ordered the same way.
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
