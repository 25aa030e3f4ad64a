// fa2_api.hip -- C ABI of the fused attention forward pass, of its gradients
// and of decode against a key/value cache (declared in include/fa2.h): argument
// checks, device check, instance dispatch and launch.
//
// Forward instances: element type {fp16, bf16} x head dim {64, 128, 256} x mask
// {none, causal, window/prefix, window/prefix/segment ids}.  The head-dim limit of 256 follows "FlashAttention-2: Where the Second
// 2x Actually Comes From" (section "Limitations & open questions").
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "fa2.h"
#include "fa2_bwd.h"
#include "fa2_decode.h"
#include "fa2_fwd_8wave.h"
#include "fa2_fwd_pair.h"
#include "fa2_fwd_w64.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture
int g_dev_arch[kMaxDevices] = {0};

int check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    g_last_hip_error = (int)e;
    (void)hipGetLastError();
    return FA2_ERR_DEVICE;
  }
  if (dev < kMaxDevices && g_dev_arch[dev] != 0) return g_dev_arch[dev] == 1 ? FA2_OK : FA2_ERR_DEVICE;
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    (void)hipGetLastError();
    return FA2_ERR_DEVICE;
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                  (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':');
  if (dev < kMaxDevices) g_dev_arch[dev] = ok ? 1 : 2;
  return ok ? FA2_OK : FA2_ERR_DEVICE;
}

bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// The caller's mask (NULL: none) after its checks: FA2_OK or FA2_ERR_MASK.
int read_mask(const fa2_mask* mask, fa2_mask& m) {
  m = {0, -1, -1, 0, nullptr};
  if (mask) m = *mask;
  if (m.window_left < -1 || m.window_right < -1 || m.prefix < 0) return FA2_ERR_MASK;
  if (((uintptr_t)m.segment_ids) & 3) return FA2_ERR_MASK;
  return FA2_OK;
}

// A mask as the kernels take it: the causal flag folded into the right bound,
// bounds that cannot bite dropped, and the instance's mask mode.
struct FoldedMask {
  int64_t wl, wr, prefix;
  int mode;
};
FoldedMask fold_mask(const fa2_mask& m, int64_t N) {
  FoldedMask f = {m.window_left, m.window_right, m.prefix, fa2::kMaskGeneral};
  if (m.causal) f.wr = 0;       // key <= query, whatever right bound was given
  if (f.wl >= N - 1) f.wl = -1;  // r - wl <= 0 for every row
  if (f.wr >= N - 1) f.wr = -1;
  if (f.prefix >= N) {  // every key is in the prefix: the window no longer matters
    f.wl = -1;
    f.wr = -1;
    f.prefix = 0;
  }
  if (f.wl < 0 && f.wr < 0) f.prefix = 0;  // the window admits every key already
  if (m.segment_ids) {
    f.mode = fa2::kMaskSegments;
  } else if (f.prefix == 0 && f.wl < 0) {
    if (f.wr < 0) f.mode = fa2::kMaskNone;
    else if (f.wr == 0) f.mode = fa2::kMaskCausal;
  }
  return f;
}

// The mask fields of the forward kernels' argument block.
void set_mask_args(fa2::FwdArgs& args, const FoldedMask& f, const fa2_mask& m, int64_t H) {
  args.wl = (int)f.wl;
  args.wr = (int)f.wr;
  args.prefix = (int)f.prefix;
  args.H = (int)H;
  args.seg = m.segment_ids;
  // general masks whose tile cost grows with the query tile: heaviest first
  args.grow = f.mode == fa2::kMaskGeneral && f.wl < 0 && f.wr >= 0;
}

// Query rows per workgroup of the kernel that serves head dim d.
int64_t rows_per_workgroup(int64_t d) { return d == 256 ? fa2::pr::kBr : fa2::w8::kBr; }

// One workgroup's sample for fa2_clock_sample: its XCD, its HW_ID (which CU),
// that CU's shader-clock counter and the real-time counter.  Thread 0 writes
// with vector stores.
__global__ void fa2_clock_kernel(uint64_t* out) {
  uint32_t xcc, hw;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
  const uint64_t t = __builtin_amdgcn_s_memtime();
  const uint64_t r = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    uint64_t* o = out + 4 * blockIdx.x;
    o[0] = xcc & 15u;
    o[1] = hw;
    o[2] = t;
    o[3] = r;
  }
}

template <int kDType, int D, int kMask>
hipError_t launch(const fa2::FwdArgs& args, hipStream_t stream) {
  if constexpr (D == 256) {
    hipLaunchKernelGGL((fa2::pr::fa2_fwd_pair<kDType, kMask>), dim3(args.n_wg), dim3(fa2::pr::kThreads), 0, stream,
                       args);
  } else if constexpr (D == 128 && (kDType == fa2::kFp16 || kDType == fa2::kBf16) &&
                       (kMask == fa2::kMaskNone || kMask == fa2::kMaskCausal)) {
    static_assert(fa2::w64::kBr == fa2::w8::kBr, "both head-dim-128 kernels take the same query tiles");
    hipLaunchKernelGGL((fa2::w64::fa2_fwd_w64<kDType, kMask>), dim3(args.n_wg), dim3(fa2::w64::kThreads), 0, stream,
                       args);
  } else {
    hipLaunchKernelGGL((fa2::w8::fa2_fwd_8wave<kDType, D, kMask>), dim3(args.n_wg), dim3(fa2::w8::kThreads), 0,
                       stream, args);
  }
  return hipGetLastError();
}

template <int kDType, int D>
hipError_t launch_m(const fa2::FwdArgs& args, int mask_mode, hipStream_t stream) {
  switch (mask_mode) {
    case fa2::kMaskNone: return launch<kDType, D, fa2::kMaskNone>(args, stream);
    case fa2::kMaskCausal: return launch<kDType, D, fa2::kMaskCausal>(args, stream);
    case fa2::kMaskGeneral: return launch<kDType, D, fa2::kMaskGeneral>(args, stream);
    default: return launch<kDType, D, fa2::kMaskSegments>(args, stream);
  }
}

template <int kDType>
hipError_t launch_d(const fa2::FwdArgs& args, int64_t d, int mask_mode, hipStream_t stream) {
  switch (d) {
    case 64: return launch_m<kDType, 64>(args, mask_mode, stream);
    case 128: return launch_m<kDType, 128>(args, mask_mode, stream);
    default: return launch_m<kDType, 256>(args, mask_mode, stream);
  }
}

template <int kDType, int D, int kMask>
hipError_t launch_bwd(const fa2::bwd::BwdArgs& args, hipStream_t stream) {
  using namespace fa2::bwd;
  const int64_t rows = (int64_t)args.BH * args.N;
  hipLaunchKernelGGL((fa2_bwd_delta<kDType, D>), dim3((unsigned)((rows + kDeltaRows - 1) / kDeltaRows)), dim3(256),
                     0, stream, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (D == 256)
    hipLaunchKernelGGL((fa2_bwd_dkdv_pair<kDType, kMask>), dim3((unsigned)(args.n_kv_wg * args.BH)),
                       dim3(kPairThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((fa2_bwd_dkdv<kDType, D, kMask>), dim3((unsigned)(args.n_kv_wg * args.BH)), dim3(kThreads), 0,
                       stream, args);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (D == 256)
    hipLaunchKernelGGL((fa2_bwd_dq_pair<kDType, kMask>), dim3((unsigned)(args.n_q_wg * args.BH)),
                       dim3(kPairThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((fa2_bwd_dq<kDType, D, kMask>), dim3((unsigned)(args.n_q_wg * args.BH)), dim3(kThreads), 0,
                       stream, args);
  return hipGetLastError();
}

template <int kDType, int D>
hipError_t launch_bwd_m(const fa2::bwd::BwdArgs& args, int mask_mode, hipStream_t stream) {
  switch (mask_mode) {
    case fa2::kMaskNone: return launch_bwd<kDType, D, fa2::kMaskNone>(args, stream);
    case fa2::kMaskCausal: return launch_bwd<kDType, D, fa2::kMaskCausal>(args, stream);
    case fa2::kMaskGeneral: return launch_bwd<kDType, D, fa2::kMaskGeneral>(args, stream);
    default: return launch_bwd<kDType, D, fa2::kMaskSegments>(args, stream);
  }
}

template <int kDType>
hipError_t launch_bwd_d(const fa2::bwd::BwdArgs& args, int64_t d, int mask_mode, hipStream_t stream) {
  switch (d) {
    case 64: return launch_bwd_m<kDType, 64>(args, mask_mode, stream);
    case 128: return launch_bwd_m<kDType, 128>(args, mask_mode, stream);
    default: return launch_bwd_m<kDType, 256>(args, mask_mode, stream);
  }
}

// Decode plan: chunks per (batch, head) so that about kDecodeWgTarget
// workgroups stream the cache (2 per CU, each wave with 2 x 16 row loads in
// flight; 1024 or 2048 workgroups measured slower on short and ragged caches),
// chunks of at least kDecodeMinChunk keys, a multiple of 64.
constexpr int64_t kDecodeWgTarget = 512;
constexpr int64_t kDecodeMinChunk = 256;
struct DecodePlan {
  int64_t n_split, chunk;
};
DecodePlan decode_plan(int64_t bh, int64_t Nk) {
  int64_t n = (kDecodeWgTarget + bh - 1) / bh;
  const int64_t most = (Nk + kDecodeMinChunk - 1) / kDecodeMinChunk;
  if (n > most) n = most;
  if (n < 1) n = 1;
  int64_t chunk = (Nk + n - 1) / n;
  chunk = (chunk + 63) / 64 * 64;
  if (chunk < 64) chunk = 64;
  n = (Nk + chunk - 1) / chunk;
  if (n < 1) n = 1;
  return {n, chunk};
}

// Shape checks shared by fa2_decode and fa2_decode_workspace_bytes; FA2_OK or
// an error status.
int decode_shape_status(int64_t B, int64_t H, int64_t Mq, int64_t Nk, int64_t d) {
  if (B < 0 || H < 0 || Mq < 0 || Nk < 0) return FA2_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return FA2_ERR_HEADDIM;
  if (Mq > fa2::dec::kMaxQ) return FA2_ERR_SHAPE;
  if (B > INT32_MAX || H > INT32_MAX || Nk > (int64_t)INT32_MAX - 65536) return FA2_ERR_SHAPE;
  const int64_t bh = B * H;
  if (bh == 0 || Mq == 0) return FA2_OK;
  if (bh > (int64_t)INT32_MAX / 64) return FA2_ERR_SHAPE;
  const DecodePlan p = decode_plan(bh, Nk);
  if (p.n_split * bh > (int64_t)INT32_MAX || bh * Mq > (int64_t)INT32_MAX) return FA2_ERR_SHAPE;
  if (Nk > 0 && bh > (INT64_MAX / 4) / (Nk * d)) return FA2_ERR_SHAPE;
  return FA2_OK;
}

int64_t decode_workspace(int64_t B, int64_t H, int64_t Mq, int64_t Nk, int64_t d) {
  const int64_t bh = B * H;
  if (bh == 0 || Mq == 0) return 0;
  const DecodePlan p = decode_plan(bh, Nk);
  if (p.n_split == 1) return 0;
  return p.n_split * bh * Mq * (d + 1) * 4;  // partial outputs, then partial logsumexp
}

template <int kDType, int D, int MQ>
hipError_t launch_decode(const fa2::dec::DecArgs& args, hipStream_t stream) {
  using namespace fa2::dec;
  hipLaunchKernelGGL((fa2_decode_split<kDType, D, MQ>), dim3((unsigned)(args.n_split * args.n_bh)), dim3(kThreads),
                     0, stream, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || args.n_split == 1) return e;
  hipLaunchKernelGGL((fa2_decode_combine<kDType, D>), dim3((unsigned)(args.n_bh * args.Mq)), dim3(D), 0, stream,
                     args);
  return hipGetLastError();
}

template <int kDType, int D>
hipError_t launch_decode_q(const fa2::dec::DecArgs& args, hipStream_t stream) {
  if (args.Mq <= 1) return launch_decode<kDType, D, 1>(args, stream);
  if (args.Mq <= 2) return launch_decode<kDType, D, 2>(args, stream);
  if (args.Mq <= 4) return launch_decode<kDType, D, 4>(args, stream);
  return launch_decode<kDType, D, 8>(args, stream);
}

template <int kDType>
hipError_t launch_decode_d(const fa2::dec::DecArgs& args, int64_t d, hipStream_t stream) {
  switch (d) {
    case 64: return launch_decode_q<kDType, 64>(args, stream);
    case 128: return launch_decode_q<kDType, 128>(args, stream);
    default: return launch_decode_q<kDType, 256>(args, stream);
  }
}

// fa2_decode_static's scratch: the chunk partials of one call (normalised
// outputs, then log2-sum-exps), at most kScratchBytes.  Each device holds its
// own copy for the life of the process; calls on one device share it.  In host
// code `scratch` names a host-side stand-in: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed on.
constexpr int64_t kScratchBytes = FA2_DECODE_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
void* g_scratch_dev[kMaxDevices] = {nullptr};
std::mutex g_scratch_mu;

// The current device's address of `scratch` (looked up on first use), or an
// error status.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    g_last_hip_error = (int)e;
    (void)hipGetLastError();
    return FA2_ERR_DEVICE;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      g_last_hip_error = (int)e;
      (void)hipGetLastError();
      return FA2_ERR_DEVICE;
    }
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return FA2_OK;
}

// fa2_decode (caller's workspace) and fa2_decode_static (the device scratch
// above): the same checks, plan and kernels.
int decode_entry(const void* q, const void* k, const void* v, const int32_t* seqlens, void* o, float* lse,
                 int64_t B, int64_t H, int64_t Mq, int64_t Nk, int64_t d, int causal, float scale, int dtype,
                 void* workspace, int64_t workspace_bytes, bool use_scratch, void* stream) {
  g_last_hip_error = 0;
  // ---- argument checks: no HIP call before they all pass -------------------
  const int st = decode_shape_status(B, H, Mq, Nk, d);
  if (st != FA2_OK) return st;
  if (dtype != FA2_DTYPE_FP16 && dtype != FA2_DTYPE_BF16) return FA2_ERR_DTYPE;
  const float c2 = (float)((double)scale * 1.4426950408889634074);
  if (!std::isfinite(scale) || !std::isfinite(c2)) return FA2_ERR_SCALE;
  const int64_t bh = B * H;
  if (bh == 0 || Mq == 0) return FA2_OK;
  if (!q || !o || !lse || (Nk > 0 && (!k || !v))) return FA2_ERR_NULLPTR;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse) & 15) return FA2_ERR_ALIGN;
  if (((uintptr_t)seqlens) & 3) return FA2_ERR_ALIGN;
  const int64_t need = decode_workspace(B, H, Mq, Nk, d);
  if (use_scratch) {
    if (need > kScratchBytes) return FA2_ERR_SCRATCH;
  } else if (need > 0 && (!workspace || workspace_bytes < need || (((uintptr_t)workspace) & 15))) {
    return FA2_ERR_WORKSPACE;
  }
  const uint64_t qb = (uint64_t)(bh * Mq * d) * 2, kb = (uint64_t)(bh * Nk * d) * 2;
  const uint64_t lb = (uint64_t)(bh * Mq) * 4, sb = seqlens ? (uint64_t)B * 4 : 0;
  const uint64_t wb = use_scratch ? 0 : (uint64_t)need;
  const void* in[4] = {q, k, v, seqlens};
  const uint64_t in_n[4] = {qb, kb, kb, sb};
  const void* out[3] = {o, lse, workspace};
  const uint64_t out_n[3] = {qb, lb, wb};
  for (int i = 0; i < 3; ++i) {
    if (out_n[i] == 0) continue;
    for (int j = 0; j < 4; ++j)
      if (in_n[j] > 0 && overlaps(out[i], out_n[i], in[j], in_n[j])) return FA2_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (out_n[j] > 0 && overlaps(out[i], out_n[i], out[j], out_n[j])) return FA2_ERR_ALIAS;
  }

  // ---- device ---------------------------------------------------------------
  const int dev_status = check_device();
  if (dev_status != FA2_OK) return dev_status;
  if (use_scratch && need > 0) {
    const int sc = scratch_address(&workspace);
    if (sc != FA2_OK) return sc;
  }

  const DecodePlan plan = decode_plan(bh, Nk);
  fa2::dec::DecArgs args;
  args.q = (const uint16_t*)q;
  args.k = (const uint16_t*)k;
  args.v = (const uint16_t*)v;
  args.o = (uint16_t*)o;
  args.lse = lse;
  args.seqlens = seqlens;
  args.part_o = need > 0 ? (float*)workspace : nullptr;
  args.part_lse = need > 0 ? (float*)workspace + plan.n_split * bh * Mq * d : nullptr;
  args.H = (int)H;
  args.Mq = (int)Mq;
  args.Nk = (int)Nk;
  args.n_split = (int)plan.n_split;
  args.chunk = (int)plan.chunk;
  args.causal = causal != 0;
  args.n_bh = (int)bh;
  args.c2 = c2;

  hipStream_t s = (hipStream_t)stream;
  hipError_t e = dtype == FA2_DTYPE_FP16 ? launch_decode_d<0>(args, d, s) : launch_decode_d<1>(args, d, s);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return FA2_ERR_LAUNCH;
  }
  return FA2_OK;
}

}  // namespace

extern "C" {

const char* fa2_status_str(int status) {
  switch (status) {
    case FA2_OK: return "ok";
    case FA2_ERR_NULLPTR: return "null pointer for a non-empty problem";
    case FA2_ERR_SHAPE: return "negative or too large B, H or N";
    case FA2_ERR_HEADDIM: return "head dim must be 64, 128 or 256";
    case FA2_ERR_DTYPE: return "dtype must be FA2_DTYPE_FP16 or FA2_DTYPE_BF16";
    case FA2_ERR_SCALE: return "scale must be finite";
    case FA2_ERR_ALIGN: return "pointers must be 16-byte aligned";
    case FA2_ERR_ALIAS: return "an output overlaps an input or another output";
    case FA2_ERR_DEVICE: return "no usable gfx950 device";
    case FA2_ERR_LAUNCH: return "kernel launch failed";
    case FA2_ERR_MASK: return "mask: window bound below -1, negative prefix or misaligned segment ids";
    case FA2_ERR_WORKSPACE: return "workspace missing, too small or not 16-byte aligned";
    case FA2_ERR_SCRATCH: return "problem needs more chunk scratch than fa2_decode_static holds (FA2_DECODE_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int fa2_last_hip_error(void) { return g_last_hip_error; }

int fa2_clock_sample(uint64_t* out, void* stream) {
  g_last_hip_error = 0;
  if (!out) return FA2_ERR_NULLPTR;
  if (((uintptr_t)out) & 15) return FA2_ERR_ALIGN;
  const int dev_status = check_device();
  if (dev_status != FA2_OK) return dev_status;
  hipLaunchKernelGGL(fa2_clock_kernel, dim3(FA2_CLOCK_BLOCKS), dim3(64), 0, (hipStream_t)stream, out);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return FA2_ERR_LAUNCH;
  }
  return FA2_OK;
}

int fa2_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                   int64_t N, int64_t d, const fa2_mask* mask, float scale, int dtype, void* stream) {
  g_last_hip_error = 0;
  // ---- argument checks: no HIP call before they all pass -------------------
  if (B < 0 || H < 0 || N < 0) return FA2_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return FA2_ERR_HEADDIM;
  if (dtype != FA2_DTYPE_FP16 && dtype != FA2_DTYPE_BF16) return FA2_ERR_DTYPE;
  const float c2 = (float)((double)scale * 1.4426950408889634074);  // scale * log2(e)
  if (!std::isfinite(scale) || !std::isfinite(c2)) return FA2_ERR_SCALE;
  fa2_mask m;
  const int mask_status = read_mask(mask, m);
  if (mask_status != FA2_OK) return mask_status;
  if (B == 0 || H == 0 || N == 0) return FA2_OK;  // empty problem: nothing to do
  // Index limits: rows (plus the span of one pass of the segment-id scan) fit
  // in int32 inside the kernel, the grid in 2^31 - 1 workgroups, byte sizes in
  // 63 bits.
  if (N > (int64_t)INT32_MAX - 65536) return FA2_ERR_SHAPE;
  if (B > INT32_MAX || H > INT32_MAX) return FA2_ERR_SHAPE;
  const int64_t bh = B * H;  // both < 2^31: no overflow
  const int64_t br = rows_per_workgroup(d);
  const int64_t n_qtiles = (N + br - 1) / br;
  if (bh > (int64_t)INT32_MAX / n_qtiles) return FA2_ERR_SHAPE;
  if (bh > (INT64_MAX / 4) / (N * d)) return FA2_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse) return FA2_ERR_NULLPTR;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse) & 15) return FA2_ERR_ALIGN;
  const uint64_t tensor_bytes = (uint64_t)(bh * N * d) * 2;
  const uint64_t lse_bytes = (uint64_t)(bh * N) * 4;
  if (overlaps(o, tensor_bytes, q, tensor_bytes) || overlaps(o, tensor_bytes, k, tensor_bytes) ||
      overlaps(o, tensor_bytes, v, tensor_bytes) || overlaps(lse, lse_bytes, q, tensor_bytes) ||
      overlaps(lse, lse_bytes, k, tensor_bytes) || overlaps(lse, lse_bytes, v, tensor_bytes) ||
      overlaps(o, tensor_bytes, lse, lse_bytes))
    return FA2_ERR_ALIAS;
  if (m.segment_ids) {
    const uint64_t seg_bytes = (uint64_t)(B * N) * 4;
    if (overlaps(m.segment_ids, seg_bytes, o, tensor_bytes) || overlaps(m.segment_ids, seg_bytes, lse, lse_bytes))
      return FA2_ERR_ALIAS;
  }

  const FoldedMask f = fold_mask(m, N);

  // ---- device ---------------------------------------------------------------
  const int dev_status = check_device();
  if (dev_status != FA2_OK) return dev_status;

  fa2::FwdArgs args;
  args.q = (const uint16_t*)q;
  args.k = (const uint16_t*)k;
  args.v = (const uint16_t*)v;
  args.o = (uint16_t*)o;
  args.lse = lse;
  args.N = (int)N;
  args.n_qtiles = (int)n_qtiles;
  args.n_wg = (int)(bh * n_qtiles);
  args.c2 = c2;
  set_mask_args(args, f, m, H);
  args.descale_q = nullptr;
  args.descale_k = nullptr;

  hipStream_t s = (hipStream_t)stream;
  hipError_t e = dtype == FA2_DTYPE_FP16 ? launch_d<0>(args, d, f.mode, s) : launch_d<1>(args, d, f.mode, s);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return FA2_ERR_LAUNCH;
  }
  return FA2_OK;
}

int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t N,
            int64_t d, int causal, float scale, int dtype, void* stream) {
  const fa2_mask m = {causal != 0, -1, -1, 0, nullptr};
  return fa2_fwd_masked(q, k, v, o, lse, B, H, N, d, &m, scale, dtype, stream);
}

int fa2_bwd_masked(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   float* delta, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d,
                   const fa2_mask* mask, float scale, int dtype, void* stream) {
  g_last_hip_error = 0;
  // ---- argument checks: no HIP call before they all pass -------------------
  if (B < 0 || H < 0 || N < 0) return FA2_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return FA2_ERR_HEADDIM;
  if (dtype != FA2_DTYPE_FP16 && dtype != FA2_DTYPE_BF16) return FA2_ERR_DTYPE;
  const float c2 = (float)((double)scale * 1.4426950408889634074);
  if (!std::isfinite(scale) || !std::isfinite(c2)) return FA2_ERR_SCALE;
  fa2_mask m;
  const int mask_status = read_mask(mask, m);
  if (mask_status != FA2_OK) return mask_status;
  if (B == 0 || H == 0 || N == 0) return FA2_OK;
  if (N > (int64_t)INT32_MAX - 65536) return FA2_ERR_SHAPE;
  if (B > INT32_MAX || H > INT32_MAX) return FA2_ERR_SHAPE;
  const int64_t bh = B * H;
  const int64_t n_kv = (N + fa2::bwd::kKeysPerWg - 1) / fa2::bwd::kKeysPerWg;
  const int64_t n_q = (N + fa2::bwd::kRowsPerWg - 1) / fa2::bwd::kRowsPerWg;
  if (bh > (int64_t)INT32_MAX / (n_kv > n_q ? n_kv : n_q)) return FA2_ERR_SHAPE;
  if (bh > (INT64_MAX / 4) / (N * d)) return FA2_ERR_SHAPE;
  if ((bh * N + fa2::bwd::kDeltaRows - 1) / fa2::bwd::kDeltaRows > (int64_t)INT32_MAX) return FA2_ERR_SHAPE;
  if (!q || !k || !v || !o || !dout || !lse || !delta || !dq || !dk || !dv) return FA2_ERR_NULLPTR;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)lse |
       (uintptr_t)delta | (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv) & 15)
    return FA2_ERR_ALIGN;
  const uint64_t tb = (uint64_t)(bh * N * d) * 2;
  const uint64_t sb = (uint64_t)(bh * N) * 4;
  const void* in[6] = {q, k, v, o, dout, lse};
  const uint64_t in_n[6] = {tb, tb, tb, tb, tb, sb};
  const void* out[4] = {delta, dq, dk, dv};
  const uint64_t out_n[4] = {sb, tb, tb, tb};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(out[i], out_n[i], in[j], in_n[j])) return FA2_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(out[i], out_n[i], out[j], out_n[j])) return FA2_ERR_ALIAS;
    if (m.segment_ids && overlaps(out[i], out_n[i], m.segment_ids, (uint64_t)(B * N) * 4)) return FA2_ERR_ALIAS;
  }

  // ---- mask: folded as in fa2_fwd_masked (the forward that produced lse must
  // have used the same mask) ----------------------------------------------------
  const FoldedMask f = fold_mask(m, N);

  // ---- device ---------------------------------------------------------------
  const int dev_status = check_device();
  if (dev_status != FA2_OK) return dev_status;

  fa2::bwd::BwdArgs args;
  args.q = (const uint16_t*)q;
  args.k = (const uint16_t*)k;
  args.v = (const uint16_t*)v;
  args.o = (const uint16_t*)o;
  args.dout = (const uint16_t*)dout;
  args.lse = lse;
  args.delta = delta;
  args.dq = (uint16_t*)dq;
  args.dk = (uint16_t*)dk;
  args.dv = (uint16_t*)dv;
  args.N = (int)N;
  args.BH = (int)bh;
  args.n_kv_wg = (int)n_kv;
  args.n_q_wg = (int)n_q;
  args.scale = scale;
  args.c2 = c2;
  args.wl = (int)f.wl;
  args.wr = (int)f.wr;
  args.prefix = (int)f.prefix;
  args.H = (int)H;
  args.seg = m.segment_ids;

  hipStream_t s = (hipStream_t)stream;
  hipError_t e =
      dtype == FA2_DTYPE_FP16 ? launch_bwd_d<0>(args, d, f.mode, s) : launch_bwd_d<1>(args, d, f.mode, s);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return FA2_ERR_LAUNCH;
  }
  return FA2_OK;
}

int fa2_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
            float* delta, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d, int causal,
            float scale, int dtype, void* stream) {
  const fa2_mask m = {causal, -1, -1, 0, nullptr};
  return fa2_bwd_masked(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, N, d, &m, scale, dtype, stream);
}

int64_t fa2_decode_workspace_bytes(int64_t B, int64_t H, int64_t Mq, int64_t Nk, int64_t d) {
  const int st = decode_shape_status(B, H, Mq, Nk, d);
  if (st != FA2_OK) return -(int64_t)st;
  return decode_workspace(B, H, Mq, Nk, d);
}

int fa2_decode(const void* q, const void* k, const void* v, const int32_t* seqlens, void* o, float* lse, int64_t B,
               int64_t H, int64_t Mq, int64_t Nk, int64_t d, int causal, float scale, int dtype, void* workspace,
               int64_t workspace_bytes, void* stream) {
  return decode_entry(q, k, v, seqlens, o, lse, B, H, Mq, Nk, d, causal, scale, dtype, workspace, workspace_bytes,
                      false, stream);
}

int fa2_decode_static(const void* q, const void* k, const void* v, const int32_t* seqlens, void* o, float* lse,
                      int64_t B, int64_t H, int64_t Mq, int64_t Nk, int64_t d, int causal, float scale, int dtype,
                      void* stream) {
  return decode_entry(q, k, v, seqlens, o, lse, B, H, Mq, Nk, d, causal, scale, dtype, nullptr, 0, true, stream);
}

int fa2_fwd_fp8_masked(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                       int64_t N, int64_t d, const fa2_mask* mask, float scale, const float* descale_q,
                       const float* descale_k, int dtype, void* stream) {
  g_last_hip_error = 0;
  // ---- argument checks: no HIP call before they all pass -------------------
  if (B < 0 || H < 0 || N < 0) return FA2_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return FA2_ERR_HEADDIM;
  if (dtype != FA2_DTYPE_FP16 && dtype != FA2_DTYPE_BF16) return FA2_ERR_DTYPE;
  const float c2 = (float)((double)scale * 1.4426950408889634074);
  if (!std::isfinite(scale) || !std::isfinite(c2)) return FA2_ERR_SCALE;
  fa2_mask m;
  const int mask_status = read_mask(mask, m);
  if (mask_status != FA2_OK) return mask_status;
  if (B == 0 || H == 0 || N == 0) return FA2_OK;
  if (N > (int64_t)INT32_MAX - 65536) return FA2_ERR_SHAPE;
  if (B > INT32_MAX || H > INT32_MAX) return FA2_ERR_SHAPE;
  const int64_t bh = B * H;
  const int64_t br = rows_per_workgroup(d);
  const int64_t n_qtiles = (N + br - 1) / br;
  if (bh > (int64_t)INT32_MAX / n_qtiles) return FA2_ERR_SHAPE;
  if (bh > (INT64_MAX / 4) / (N * d)) return FA2_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse) return FA2_ERR_NULLPTR;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse) & 15) return FA2_ERR_ALIGN;
  if (((uintptr_t)descale_q | (uintptr_t)descale_k) & 3) return FA2_ERR_ALIGN;
  const uint64_t b8 = (uint64_t)(bh * N * d), b16 = 2 * b8, lb = (uint64_t)(bh * N) * 4, sb = (uint64_t)bh * 4;
  const void* in[5] = {q, k, v, descale_q, descale_k};
  const uint64_t in_n[5] = {b8, b8, b16, descale_q ? sb : 0, descale_k ? sb : 0};
  for (int j = 0; j < 5; ++j) {
    if (in_n[j] == 0) continue;
    if (overlaps(o, b16, in[j], in_n[j]) || overlaps(lse, lb, in[j], in_n[j])) return FA2_ERR_ALIAS;
  }
  if (overlaps(o, b16, lse, lb)) return FA2_ERR_ALIAS;
  if (m.segment_ids) {
    const uint64_t seg_bytes = (uint64_t)(B * N) * 4;
    if (overlaps(m.segment_ids, seg_bytes, o, b16) || overlaps(m.segment_ids, seg_bytes, lse, lb))
      return FA2_ERR_ALIAS;
  }
  const FoldedMask f = fold_mask(m, N);

  // ---- device ---------------------------------------------------------------
  const int dev_status = check_device();
  if (dev_status != FA2_OK) return dev_status;

  fa2::FwdArgs args;
  args.q = (const uint16_t*)q;  // e4m3 bytes, addressed as such by the fp8 instances
  args.k = (const uint16_t*)k;
  args.v = (const uint16_t*)v;
  args.o = (uint16_t*)o;
  args.lse = lse;
  args.N = (int)N;
  args.n_qtiles = (int)n_qtiles;
  args.n_wg = (int)(bh * n_qtiles);
  args.c2 = c2;
  set_mask_args(args, f, m, H);
  args.descale_q = descale_q;
  args.descale_k = descale_k;

  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (d == 64) {
    e = dtype == FA2_DTYPE_FP16 ? launch_m<fa2::kFp8Fp16, 64>(args, f.mode, s)
                                : launch_m<fa2::kFp8Bf16, 64>(args, f.mode, s);
  } else if (d == 128) {
    e = dtype == FA2_DTYPE_FP16 ? launch_m<fa2::kFp8Fp16, 128>(args, f.mode, s)
                                : launch_m<fa2::kFp8Bf16, 128>(args, f.mode, s);
  } else {
    e = dtype == FA2_DTYPE_FP16 ? launch_m<fa2::kFp8Fp16, 256>(args, f.mode, s)
                                : launch_m<fa2::kFp8Bf16, 256>(args, f.mode, s);
  }
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return FA2_ERR_LAUNCH;
  }
  return FA2_OK;
}

int fa2_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t N,
                int64_t d, int causal, float scale, const float* descale_q, const float* descale_k, int dtype,
                void* stream) {
  const fa2_mask m = {causal != 0, -1, -1, 0, nullptr};
  return fa2_fwd_fp8_masked(q, k, v, o, lse, B, H, N, d, &m, scale, descale_q, descale_k, dtype, stream);
}

}  // extern "C"
