/*
 * fa2.h -- C ABI of fused exact attention for AMD Instinct MI355X (gfx950):
 * the forward pass and its gradients.
 *
 * The operation.  For every batch b < B, head h < H and query row r < N:
 *
 *   s_rc  = scale * sum_t Q[b,h,r,t] * K[b,h,c,t]       for allowed keys c
 *   O[b,h,r,:] = sum_c softmax_c(s_r.) * V[b,h,c,:]
 *   lse[b,h,r] = log(sum_c exp(s_rc))                   (natural log)
 *
 * where the allowed keys are c < N, and with a causal mask only c <= r.
 *  - Standard attention (scores, row softmax, P.V): "Flash Attention:
 *    Memory-Efficient Attention at Scale" (Lesson 6.6), section "A quick recap
 *    of standard attention"; "Flash Attention 2", section "Standard Attention".
 *  - The causal mask (0 for key <= query, -inf otherwise, so masked keys carry
 *    no weight): "6.2 FlashAttention V2 in depth", section 5.1, and "Flash
 *    Attention 2", section "Causal masking".
 *  - The per-row statistic L = m + log(l), i.e. the logsumexp of the scaled,
 *    masked scores, returned next to O: "6.2 FlashAttention V2 in depth",
 *    sections 6.1 and 7.1.
 *  - The result is exact attention, computed tile by tile without ever storing
 *    the N x N score matrix: "6.2 FlashAttention V2 in depth", sections 2-6.
 *
 * Everything here is plain C: pointers, sizes and an opaque stream handle.
 */
#ifndef FA2_H
#define FA2_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V and O. */
typedef enum {
  FA2_DTYPE_FP16 = 0, /* IEEE binary16 */
  FA2_DTYPE_BF16 = 1  /* bfloat16 */
} fa2_dtype;

/* Return codes.  Every failure is reported before anything is launched, except
 * FA2_ERR_LAUNCH. */
typedef enum {
  FA2_OK = 0,
  FA2_ERR_NULLPTR = 1, /* a pointer argument is NULL while the problem is not empty */
  FA2_ERR_SHAPE = 2,   /* B, H or N is negative, or the problem is too large to index */
  FA2_ERR_HEADDIM = 3, /* d is not 64, 128 or 256 */
  FA2_ERR_DTYPE = 4,   /* dtype is not a fa2_dtype value */
  FA2_ERR_SCALE = 5,   /* scale is NaN, infinite, or so large that scale*log2(e) overflows */
  FA2_ERR_ALIGN = 6,   /* a pointer is not 16-byte aligned */
  FA2_ERR_ALIAS = 7,   /* an output overlaps an input or another output */
  FA2_ERR_DEVICE = 8,  /* no current HIP device, or it is not a gfx950 */
  FA2_ERR_LAUNCH = 9,  /* the HIP launch itself reported an error */
  FA2_ERR_MASK = 10,   /* fa2_fwd_masked: a window bound below -1, a negative
                          prefix, or segment ids not 4-byte aligned */
  FA2_ERR_WORKSPACE = 11, /* fa2_decode: the workspace it needs is missing, smaller
                            than fa2_decode_workspace_bytes, or not 16-byte aligned */
  FA2_ERR_SCRATCH = 12    /* fa2_decode_static: the problem needs more than
                             FA2_DECODE_STATIC_SCRATCH_BYTES of chunk scratch */
} fa2_status;

/*
 * A general attention mask for fa2_fwd_masked.  Key c is visible to query r
 * (both in [0, N)) iff
 *   segment_ids == NULL or segment_ids[b*N + c] == segment_ids[b*N + r], and
 *   c < prefix, or
 *   (window_left  < 0 or c >= r - window_left) and
 *   (window_right < 0 or c <= r + window_right)  [causal: window_right = 0].
 * Every query sees at least itself, so no row is ever empty.
 *  - A mask is a 0 / -inf term added to the scores before the softmax, and the
 *    same block-skipping scheme as the causal mask covers sliding windows,
 *    document boundaries and prefix language models: "Flash Attention 2",
 *    section "Causal masking" (its option A).  Tiles no pair of which is
 *    visible are not visited (window bounds), tiles only partly visible are
 *    masked element by element.
 */
typedef struct {
  int causal;                 /* nonzero: key <= query (sets window_right to 0) */
  int64_t window_left;        /* -1: no left bound; else key >= query - window_left */
  int64_t window_right;       /* -1: no right bound; else key <= query + window_right */
  int64_t prefix;             /* keys < prefix are visible to every query of the same segment */
  const int32_t* segment_ids; /* NULL, or a [B, N] device array of int32 document ids shared
                                 by all heads (4-byte aligned); read only */
} fa2_mask;

/*
 * fa2_fwd -- enqueue the forward pass on `stream` and return without waiting.
 *
 * q, k, v : device pointers to [B, H, N, d] arrays of `dtype`, contiguous and
 *           row-major (d innermost; strides d, N*d, H*N*d elements).  Read only.
 * o       : device pointer to a [B, H, N, d] array of `dtype`; written.
 * lse     : device pointer to a [B, H, N] float32 array; written with the
 *           natural-log logsumexp of each row's scaled, masked scores.
 * B, H, N : batch, heads, sequence length.  Any N >= 1 (no multiple of a tile
 *           is required).  If B*H*N == 0 the call does nothing and returns
 *           FA2_OK; pointers are then not inspected.
 * d       : head dimension, 64, 128 or 256.
 * causal  : nonzero applies the causal mask (key index <= query index).
 * scale   : multiplier of the scores; any finite value, including 0 and
 *           negative values.  The library never substitutes 1/sqrt(d).
 * dtype   : a fa2_dtype value.
 * stream  : a hipStream_t of the current device (NULL = the null stream).
 *
 * Ownership: the caller allocates and owns every buffer.  The library keeps no
 * state between calls beyond a per-device cache of the device check, allocates
 * no memory and needs no workspace.  All pointers must be 16-byte aligned and
 * reside on the current device; o and lse must not overlap each other or q, k, v.
 *
 * Errors: argument checks run before any HIP call; on a failed check nothing is
 * written or launched.  FA2_ERR_DEVICE is returned when the current device
 * cannot be queried or is not gfx950.  FA2_ERR_LAUNCH carries a launch error;
 * faults during execution surface at the caller's next synchronisation, as for
 * any HIP kernel.  No C++ exception crosses this boundary.
 */
int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
            int64_t B, int64_t H, int64_t N, int64_t d,
            int causal, float scale, int dtype, void* stream);

/*
 * fa2_fwd_masked -- fa2_fwd under a general mask (NULL: no mask).  Arguments,
 * layout, ownership and errors as for fa2_fwd, plus FA2_ERR_MASK; segment_ids
 * must not overlap o or lse.  fa2_fwd(..., causal, ...) is this call with
 * {causal, -1, -1, 0, NULL}.
 */
int fa2_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t B, int64_t H, int64_t N, int64_t d,
                   const fa2_mask* mask, float scale, int dtype, void* stream);

/*
 * fa2_bwd -- enqueue the gradients of fa2_fwd on `stream` and return without
 * waiting.  For a scalar loss with gradient dO = dL/dO, with P the softmax
 * weights of the forward pass (masked pairs have P = 0) and s = scale * q.k:
 *
 *   D[b,h,r]  = sum_t dO[b,h,r,t] * O[b,h,r,t]
 *   dS        = P o (dO V^T - D)              (row by row)
 *   dQ = scale * dS K,   dK = scale * dS^T Q,   dV = P^T dO
 *
 *  - P is recomputed from the forward's logsumexp, P = exp(s - lse): "6.2
 *    FlashAttention V2 in depth", section 7.1; "Flash Attention: Memory-
 *    Efficient Attention at Scale", section "Recomputation in the backward pass".
 *  - dS = P o (dP - D) with D = rowsum(dO o O), D computed by a preprocess step
 *    for all rows first: "6.2 FlashAttention V2 in depth", section 7.3.
 *  - Key/value tiles outside, query tiles inside, so dK and dV need no atomic
 *    adds; dQ is gathered by a second pass instead of atomics (same page,
 *    section 7.2).
 *
 * q, k, v     : the forward's inputs ([B, H, N, d], `dtype`).  Read only.
 * o, lse      : the forward's outputs for the same q, k, v, causal, scale
 *               (o: [B, H, N, d] `dtype`; lse: [B, H, N] float32).  Read only.
 * dout        : dO, [B, H, N, d] `dtype`.  Read only.
 * delta       : [B, H, N] float32 work array owned by the caller; overwritten
 *               with D (its contents on return are D).
 * dq, dk, dv  : [B, H, N, d] `dtype`; written.
 * B, H, N, d, causal, scale, dtype, stream: as for fa2_fwd.
 *
 * Layout, alignment (16 bytes, every pointer), ownership, error reporting and
 * the empty-problem rule are those of fa2_fwd; delta, dq, dk, dv must not
 * overlap each other or any input.  The three kernels (D, then dK/dV, then dQ)
 * run in order on `stream`; results are bitwise reproducible (no atomics).
 */
int fa2_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
            const float* lse, float* delta, void* dq, void* dk, void* dv,
            int64_t B, int64_t H, int64_t N, int64_t d,
            int causal, float scale, int dtype, void* stream);

/*
 * fa2_bwd_masked -- fa2_bwd under a general mask (NULL: no mask): the
 * gradients of fa2_fwd_masked for the same mask, which must be the one the
 * forward pass that produced o and lse used.  Masked pairs have P = 0 and so
 * contribute to no gradient (the mask is a 0 / -inf term added to the scores:
 * "Flash Attention 2", section "Causal masking").  Arguments, layout,
 * ownership and errors as for fa2_bwd, plus FA2_ERR_MASK (as for
 * fa2_fwd_masked); segment_ids must not overlap delta, dq, dk or dv.
 * fa2_bwd(..., causal, ...) is this call with {causal, -1, -1, 0, NULL}.
 *  - The key/value tiles a workgroup visits are cut to those some pair of which
 *    is visible (the window's reach, the prefix, and under segment ids the span
 *    of matching ids), as in the forward pass; pairs inside a visited tile are
 *    masked element by element.
 */
int fa2_bwd_masked(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, float* delta, void* dq, void* dk, void* dv,
                   int64_t B, int64_t H, int64_t N, int64_t d,
                   const fa2_mask* mask, float scale, int dtype, void* stream);

/*
 * fa2_decode -- enqueue decode against a key/value cache on `stream` and return
 * without waiting: Mq new query rows per (batch, head) attend to the first
 * len_b rows of the cache of their (batch, head), len_b = seqlens[b] (clamped
 * to [0, Nk]) or Nk when seqlens is NULL.  The new rows are the last Mq
 * positions of a sequence of len_b tokens; with causal != 0 query i (0-based)
 * sees keys c <= len_b - Mq + i, otherwise every key c < len_b:
 *
 *   O[b,h,i,:] = sum_c softmax_c(scale * q_i . k_c) v_c,   L[b,h,i] = log sum_c exp(scale * q_i . k_c)
 *
 * over the visible keys (natural log; a query with no visible key gets O = 0
 * and L = -inf).
 *  - One query row against the cached keys and values is the single-token
 *    decoding regime that "Flash Attention: Memory-Efficient Attention at
 *    Scale", section "Common misconceptions", sets apart (Flash-Decoding).
 *  - The cache is split into chunks processed in parallel; each chunk's
 *    normalised output and logsumexp merge exactly through the row max and sum,
 *    the online-softmax rule of "6.2 FlashAttention V2 in depth", sections 3.2
 *    and 6.1.
 *
 * q         : [B, H, Mq, d] `dtype`, device, read only; 1 <= Mq <= 8.
 * k, v      : [B, H, Nk, d] `dtype`, device, read only (the cache; rows past a
 *             batch's length are never used).
 * seqlens   : [B] int32, device, read only, 4-byte aligned; or NULL.
 * o, lse    : [B, H, Mq, d] `dtype` and [B, H, Mq] float32, device, written.
 * workspace : device memory of at least fa2_decode_workspace_bytes(B, H, Mq,
 *             Nk, d) bytes, 16-byte aligned, owned by the caller, overwritten;
 *             NULL is allowed when that size is 0.  Its contents between
 *             calls do not matter.
 * B, H, Nk, d, causal, scale, dtype, stream: as for fa2_fwd (d in {64, 128,
 *             256}); Nk = 0 is allowed (every row then has no visible key).
 *
 * Returns FA2_OK, or FA2_ERR_SHAPE (Mq outside [0, 8], negative or too large
 * sizes), FA2_ERR_HEADDIM, FA2_ERR_DTYPE, FA2_ERR_SCALE, FA2_ERR_NULLPTR,
 * FA2_ERR_ALIGN (q, k, v, o, lse not 16-byte aligned; seqlens not 4-byte
 * aligned), FA2_ERR_WORKSPACE, FA2_ERR_ALIAS (o, lse or the workspace overlap
 * an input or each other), FA2_ERR_DEVICE, FA2_ERR_LAUNCH.  B*H*Mq = 0 is a
 * no-op.  One or two kernels run in order on `stream`; results are bitwise
 * reproducible.
 */
int fa2_decode(const void* q, const void* k, const void* v, const int32_t* seqlens,
               void* o, float* lse, int64_t B, int64_t H, int64_t Mq, int64_t Nk, int64_t d,
               int causal, float scale, int dtype, void* workspace, int64_t workspace_bytes,
               void* stream);

/*
 * fa2_decode_static -- fa2_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same operation, arguments (minus the workspace), plan,
 * kernels and results, with the chunk partials kept in a fixed device array of
 * FA2_DECODE_STATIC_SCRATCH_BYTES that the library holds on every device it
 * runs on until the process ends.  The call allocates nothing and calls no
 * allocating routine; its first call on a device looks the array's address up
 * (hipGetSymbolAddress) with that device current.
 *
 * Returns FA2_ERR_SCRATCH, before any HIP call, when fa2_decode_workspace_bytes
 * for these sizes exceeds FA2_DECODE_STATIC_SCRATCH_BYTES; otherwise the
 * statuses of fa2_decode (FA2_ERR_DEVICE also when the address lookup fails).
 * Nothing in the array has to start at zero: every chunk writes its partial.
 * All calls on one device share the array, so calls that can overlap on one
 * device (on different streams, or from different threads) race and must be
 * ordered by the caller; calls in order on one stream are safe.
 */
#define FA2_DECODE_STATIC_SCRATCH_BYTES (4 << 20)
int fa2_decode_static(const void* q, const void* k, const void* v, const int32_t* seqlens,
                      void* o, float* lse, int64_t B, int64_t H, int64_t Mq, int64_t Nk, int64_t d,
                      int causal, float scale, int dtype, void* stream);

/*
 * fa2_fwd_fp8 -- fa2_fwd with Q and K stored in fp8 (OCP e4m3, one byte per
 * element) and V, O in fp16 or bf16 (`dtype`): enqueue on `stream` and return
 * without waiting.  The real inputs are q_real = descale_q[b*H + h] * q and
 * k_real = descale_k[b*H + h] * k, and the result is fa2_fwd's on them:
 *
 *   O = softmax(scale * q_real k_real^T [+ causal mask]) V,   L = log sum exp(...)
 *
 *  - Lower-precision inputs for speed, with the extra rounding error kept small,
 *    is the FP8 idea of "Flash Attention: Memory-Efficient Attention at Scale",
 *    section "Flash Attention 3".  Here the products q.k run on the fp8 MFMA,
 *    which sums the 64 products of one instruction with an error of up to
 *    about 2^-11 of the largest of them (measured); the weights P and the P.V
 *    product stay 16-bit.  Beyond fa2_fwd's rounding there is thus the
 *    caller's own quantisation of Q and K and that summation error.
 *
 * q, k       : [B, H, N, d] e4m3 bytes, device, read only.
 * v          : [B, H, N, d] `dtype`, device, read only.
 * o, lse     : as for fa2_fwd.
 * descale_q, descale_k : [B*H] float32 device arrays (read only, 4-byte
 *              aligned), or NULL for all ones.
 * Other arguments, layout rules, errors and the empty-problem rule as for
 * fa2_fwd; d must be 64, 128 or 256 (FA2_ERR_HEADDIM otherwise).
 */
int fa2_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                const float* descale_q, const float* descale_k, int dtype, void* stream);

/*
 * fa2_fwd_fp8_masked -- fa2_fwd_fp8 under a general mask (NULL: no mask):
 *
 *   O = softmax(scale * q_real k_real^T + M) V,   L = log sum exp(...)
 *
 * with M the mask of fa2_fwd_masked (sliding window, prefix, segment ids; the
 * mask as a 0 / -inf score term: "Flash Attention 2", section "Causal
 * masking").  Arguments, layout, ownership and errors as for fa2_fwd_fp8, plus
 * FA2_ERR_MASK (as for fa2_fwd_masked); segment_ids must not overlap o or lse.
 * fa2_fwd_fp8(..., causal, ...) is this call with {causal, -1, -1, 0, NULL}.
 */
int fa2_fwd_fp8_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t B, int64_t H, int64_t N, int64_t d, const fa2_mask* mask, float scale,
                       const float* descale_q, const float* descale_k, int dtype, void* stream);

/* Bytes of workspace fa2_decode needs for these sizes (0: none), or minus a
 * fa2_status code for sizes fa2_decode would reject.  Host only; no HIP call. */
int64_t fa2_decode_workspace_bytes(int64_t B, int64_t H, int64_t Mq, int64_t Nk, int64_t d);

/*
 * fa2_clock_sample -- measurement aid, not part of the attention computation:
 * enqueue on `stream` one small kernel of FA2_CLOCK_BLOCKS workgroups (enough
 * for every CU of the chip to run some), each of which writes four uint64
 * values to out[4*i .. 4*i+3] (i = its workgroup index): the id of the XCD it
 * ran on, its HW_ID register (bits 8-15 name the CU, shader array and shader
 * engine), that CU's shader-clock counter (s_memtime) and the 100 MHz
 * real-time counter (s_memrealtime).  Each CU has its own shader-clock
 * counter, which advances at the engine clock while the CU is busy and almost
 * stops while it idles; so two samples taken around a run of launches on the
 * same stream, matched CU by CU, give each CU's average engine clock over the
 * run: (counter difference) / (real-time difference) x 100 MHz.  Utilisation
 * is a ratio to a peak that assumes one clock ("6.2 FlashAttention V2 in
 * depth", sections 1.1 and 8.1); the measured clock turns it into the ratio to
 * the peak at the clock the chip actually ran.
 *
 * out    : device pointer to 4 * FA2_CLOCK_BLOCKS uint64 values, 16-byte
 *          aligned; written.
 * stream : as for fa2_fwd.
 * Returns FA2_OK, FA2_ERR_NULLPTR, FA2_ERR_ALIGN, FA2_ERR_DEVICE or
 * FA2_ERR_LAUNCH; checks run before any launch.
 */
#define FA2_CLOCK_BLOCKS 2048
int fa2_clock_sample(uint64_t* out, void* stream);

/* Static, NUL-terminated description of a return code (never NULL). */
const char* fa2_status_str(int status);

/* Last HIP error code seen by a failing fa2_fwd, fa2_fwd_masked, fa2_fwd_fp8,
 * fa2_bwd, fa2_decode, fa2_decode_static or fa2_clock_sample call on this
 * thread (0 if none); useful after FA2_ERR_DEVICE or FA2_ERR_LAUNCH. */
int fa2_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H */
