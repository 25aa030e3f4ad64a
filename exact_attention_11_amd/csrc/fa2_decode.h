// fa2_decode.h -- decode for gfx950: a few new query rows per (batch, head)
// against a key/value cache, with the cache split across workgroups and the
// parts merged through their logsumexp.
//
// From the pages: single-token decoding has one query row, so the work per
// (batch, head) is one pass over the cached keys and values and needs kernels
// of its own ("Flash Attention: Memory-Efficient Attention at Scale", section
// "Common misconceptions"); partial results over disjoint key ranges combine
// exactly through their row maximum and sum, the rule the online softmax uses
// between key tiles ("6.2 FlashAttention V2 in depth", sections 3.2 and 6.1).
//
// gfx950 design.  With at most 8 query rows the products are matrix-vector
// work: each cached byte is used for at most 8 multiply-adds, far below what
// an MFMA would need, and the pass is bound by HBM bandwidth.  So:
//  * The cache of each (batch, head) is cut into chunks, one workgroup per
//    (chunk, head, batch), enough of them to keep every CU streaming.
//  * A row of K or V (d halves) is spread over d / 8 lanes, 16 bytes each, so
//    one load instruction reads 64 / (d / 8) whole rows with full 16-byte
//    accesses; each wave keeps kUnroll such loads of K and of V in flight.
//  * Scores are partial dot products reduced across the row's lanes; the
//    online softmax runs per block of rows, every lane of the wave holding the
//    block's running max; P.V accumulates in fp32 registers per lane.
//  * At the end the waves of a workgroup merge through LDS; with one chunk the
//    workgroup writes O and L, otherwise it writes its normalised partial
//    output and logsumexp, and a second kernel merges the chunks.
#pragma once

#include "fa2_common.h"

namespace fa2 {
namespace dec {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxQ = 8;  // new query rows per (batch, head)

struct DecArgs {
  const uint16_t* q;   // [B, H, Mq, d]
  const uint16_t* k;   // [B, H, Nk, d]
  const uint16_t* v;   // [B, H, Nk, d]
  uint16_t* o;         // [B, H, Mq, d]
  float* lse;          // [B, H, Mq]
  const int* seqlens;  // [B] valid cache rows, or nullptr (all Nk)
  float* part_o;       // [n_split, B*H, Mq, d] normalised partial outputs (n_split > 1)
  float* part_lse;     // [n_split, B*H, Mq] partial logsumexp, log2 units (n_split > 1)
  int H, Mq, Nk;
  int n_split;  // chunks per (batch, head)
  int chunk;    // keys per chunk
  int causal;   // query i sees keys c <= len - Mq + i
  int n_bh;     // B * H
  float c2;     // scale * log2(e)
};

// Eight consecutive elements (16 bytes) as fp32.  Each word is copied out of
// the vector before the bit cast: a bit cast of the element expression raw[w]
// itself compiles to a read of element 0 for every w.
template <int kDType> __device__ __forceinline__ void to_f32x8(u32x4 raw, float* out) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t word = raw[w];
    if constexpr (kDType == 0) {
      const f16x2 h = __builtin_bit_cast(f16x2, word);
      out[2 * w] = (float)h[0];
      out[2 * w + 1] = (float)h[1];
    } else {
      out[2 * w] = __uint_as_float(word << 16);
      out[2 * w + 1] = __uint_as_float(word & 0xffff0000u);
    }
  }
}

__device__ __forceinline__ float exp2_or_zero(float x) {
  return x == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(x);
}

// One workgroup: keys [split * chunk, min((split + 1) * chunk, len)) of one
// (batch, head), all of its MQ (>= Mq) query rows.
template <int kDType, int D, int MQ>
__global__ __launch_bounds__(kThreads) void fa2_decode_split(DecArgs a) {
  constexpr int G = D / 8;   // lanes per cache row
  constexpr int R = 64 / G;  // rows per load instruction
  constexpr int kUnroll = MQ >= 8 ? 4 : (MQ >= 4 ? 8 : 16);  // loads in flight per tensor
  constexpr int kBlock = kUnroll * R;                        // rows per wave per block
  constexpr float kNegInf = -__builtin_huge_valf();
  static_assert(MQ >= 1 && MQ <= kMaxQ, "query rows");

  __shared__ float red_m[kWaves][MQ];
  __shared__ float red_l[kWaves][MQ];
  __shared__ float red_o[kWaves][MQ][D];

  const int split = blockIdx.x % a.n_split;
  const int bh = blockIdx.x / a.n_split;
  const int b = bh / a.H;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int grp = lane / G;  // row of a load instruction this lane reads
  const int cl = lane % G;   // its 16-byte chunk of the row

  int len = a.Nk;
  if (a.seqlens) len = min(max(a.seqlens[b], 0), a.Nk);
  const int k_lo = split * a.chunk;
  const int k_hi = min(k_lo + a.chunk, len);
  const int Mq = a.Mq;

  // This lane's 8 dims of every query, multiplier folded in (log2 units).
  float qv[MQ][8];
#pragma unroll
  for (int i = 0; i < MQ; ++i) {
    if (i < Mq) {
      const u32x4 raw = *(const u32x4*)(a.q + ((int64_t)bh * Mq + i) * D + cl * 8);
      to_f32x8<kDType>(raw, qv[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[i][e] *= a.c2;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[i][e] = 0.f;
    }
  }

  float m[MQ], l[MQ], o[MQ][8];
#pragma unroll
  for (int i = 0; i < MQ; ++i) {
    m[i] = kNegInf;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[i][e] = 0.f;
  }

  const uint16_t* kh = a.k + (int64_t)bh * a.Nk * D + cl * 8;
  const uint16_t* vh = a.v + (int64_t)bh * a.Nk * D + cl * 8;
  const int last_q = len - Mq;  // query i sees keys <= last_q + i under the causal flag

  for (int kb = k_lo + wave * kBlock; kb < k_hi; kb += kWaves * kBlock) {
    u32x4 kr[kUnroll], vr[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int key = kb + u * R + grp;
      const int row = key < k_hi ? key : k_lo;  // rows past the chunk re-read its first row (masked)
      kr[u] = *(const u32x4*)(kh + (int64_t)row * D);
      vr[u] = *(const u32x4*)(vh + (int64_t)row * D);
    }
    float s[kUnroll][MQ];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float kf[8];
      to_f32x8<kDType>(kr[u], kf);
#pragma unroll
      for (int i = 0; i < MQ; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(qv[i][e], kf[e], acc);
        s[u][i] = acc;
      }
    }
    // Sum the partial dot products over the G lanes of each row.
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1)
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int i = 0; i < MQ; ++i) s[u][i] += __shfl_xor(s[u][i], off);
    // Mask, then the block's row max over every lane of the wave.
    float mb[MQ];
#pragma unroll
    for (int i = 0; i < MQ; ++i) {
      mb[i] = kNegInf;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int key = kb + u * R + grp;
        const bool ok = key < k_hi && (!a.causal || key <= last_q + i);
        s[u][i] = ok ? s[u][i] : kNegInf;
        mb[i] = fmaxf(mb[i], s[u][i]);
      }
    }
#pragma unroll
    for (int off = G; off < 64; off <<= 1)
#pragma unroll
      for (int i = 0; i < MQ; ++i) mb[i] = fmaxf(mb[i], __shfl_xor(mb[i], off));
    float p[kUnroll][MQ];
#pragma unroll
    for (int i = 0; i < MQ; ++i) {
      const float m_new = fmaxf(m[i], mb[i]);
      const float ref = m_new == kNegInf ? 0.f : m_new;  // rows with no visible key yet keep zero weights
      const float alpha = exp2_or_zero(m[i] - ref);
      m[i] = m_new;
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        p[u][i] = exp2_or_zero(s[u][i] - ref);
        ps += p[u][i];
      }
      l[i] = l[i] * alpha + ps;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[i][e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float vf[8];
      to_f32x8<kDType>(vr[u], vf);
#pragma unroll
      for (int i = 0; i < MQ; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[i][e] = __builtin_fmaf(p[u][i], vf[e], o[i][e]);
    }
  }

  // Rows of the wave: lanes with the same chunk hold different keys' sums.
#pragma unroll
  for (int off = G; off < 64; off <<= 1)
#pragma unroll
    for (int i = 0; i < MQ; ++i) {
      l[i] += __shfl_xor(l[i], off);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[i][e] += __shfl_xor(o[i][e], off);
    }
  // Every lane of a row group holds the same weights, so the sum over the
  // groups is the wave's row sum.
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < MQ; ++i) {
      red_m[wave][i] = m[i];
      red_l[wave][i] = l[i];
    }
  }
  if (grp == 0) {
#pragma unroll
    for (int i = 0; i < MQ; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) red_o[wave][i][cl * 8 + e] = o[i][e];
  }
  __syncthreads();

  // Merge the waves: thread t takes (query, dim) pairs t, t + kThreads, ...
  for (int idx = tid; idx < Mq * D; idx += kThreads) {
    const int i = idx / D, e = idx % D;
    float M = red_m[0][i];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, red_m[w][i]);
    const float ref = M == kNegInf ? 0.f : M;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = exp2_or_zero(red_m[w][i] - ref);
      L += red_l[w][i] * f;
      O += red_o[w][i][e] * f;
    }
    const float out = L > 0.f ? O / L : 0.f;
    const float lse2 = L > 0.f ? M + __log2f(L) : kNegInf;
    const int64_t row = (int64_t)bh * Mq + i;
    if (a.n_split == 1) {
      typedef Elem<kDType> E;
      const uint32_t packed = E::pack2(out, 0.f);
      a.o[row * D + e] = (uint16_t)(packed & 0xffffu);
      if (e == 0) a.lse[row] = lse2 * kLn2;
    } else {
      const int64_t prow = (int64_t)split * a.n_bh * Mq + row;
      a.part_o[prow * D + e] = out;
      if (e == 0) a.part_lse[prow] = lse2;
    }
  }
}

// Merge the chunks of one (batch, head, query row): L = log2 sum_s 2^L_s and
// O = sum_s 2^(L_s - L) O_s.  One workgroup of D threads per row.
template <int kDType, int D>
__global__ __launch_bounds__(D) void fa2_decode_combine(DecArgs a) {
  constexpr float kNegInf = -__builtin_huge_valf();
  const int64_t row = blockIdx.x;  // (b * H + h) * Mq + i
  const int e = threadIdx.x;
  const int64_t stride = (int64_t)a.n_bh * a.Mq;  // between chunks
  float M = kNegInf;
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, a.part_lse[s * stride + row]);
  const float ref = M == kNegInf ? 0.f : M;
  float L = 0.f, O = 0.f;
  for (int s = 0; s < a.n_split; ++s) {
    const float f = exp2_or_zero(a.part_lse[s * stride + row] - ref);
    L += f;
    O += f * a.part_o[(s * stride + row) * D + e];
  }
  const float out = L > 0.f ? O / L : 0.f;
  typedef Elem<kDType> E;
  a.o[row * D + e] = (uint16_t)(E::pack2(out, 0.f) & 0xffffu);
  if (e == 0) a.lse[row] = L > 0.f ? (M + __log2f(L)) * kLn2 : kNegInf;
}

}  // namespace dec
}  // namespace fa2
