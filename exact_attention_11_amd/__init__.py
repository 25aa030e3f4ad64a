"""Fused exact attention for AMD Instinct MI355X (gfx950): forward pass,
gradients, and decode against a key/value cache.

Thin Python binding of the C ABI declared in ``include/fa2.h``; every step of
the computation runs in the HIP kernels of ``libfa2.so``.  torch supplies device
memory and streams only.

    o, lse = exact_attention_11_amd.forward(q, k, v, causal=True)
    dq, dk, dv = exact_attention_11_amd.backward(q, k, v, o, do, lse, causal=True)
    o1, lse1 = exact_attention_11_amd.decode(q1, k_cache, v_cache, seqlens=lens)

``q, k, v``: [B, H, N, d] fp16 or bf16 CUDA (HIP) tensors, contiguous.
``forward`` returns ``o`` (same shape and dtype) and ``lse`` ([B, H, N] float32,
the natural-log logsumexp of each row's scaled, masked scores); ``backward``
takes those and the gradient ``do`` of a loss with respect to ``o``.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa2.so")

FA2_DTYPE_FP16 = 0
FA2_DTYPE_BF16 = 1

FA2_OK = 0
FA2_ERR_NULLPTR = 1
FA2_ERR_SHAPE = 2
FA2_ERR_HEADDIM = 3
FA2_ERR_DTYPE = 4
FA2_ERR_SCALE = 5
FA2_ERR_ALIGN = 6
FA2_ERR_ALIAS = 7
FA2_ERR_DEVICE = 8
FA2_ERR_LAUNCH = 9
FA2_ERR_MASK = 10
FA2_ERR_WORKSPACE = 11
FA2_ERR_SCRATCH = 12

# Every symbol include/fa2.h declares.
EXPORTED_SYMBOLS = ("fa2_fwd", "fa2_fwd_masked", "fa2_fwd_fp8", "fa2_fwd_fp8_masked", "fa2_bwd", "fa2_bwd_masked",
                    "fa2_decode", "fa2_decode_static",
                    "fa2_decode_workspace_bytes", "fa2_clock_sample", "fa2_status_str", "fa2_last_hip_error")
DECODE_STATIC_SCRATCH_BYTES = 4 << 20  # FA2_DECODE_STATIC_SCRATCH_BYTES
CLOCK_BLOCKS = 2048  # FA2_CLOCK_BLOCKS
DECODE_MAX_QUERIES = 8


class Fa2Mask(ctypes.Structure):
    """The C struct fa2_mask of include/fa2.h."""
    _fields_ = [("causal", ctypes.c_int), ("window_left", ctypes.c_int64), ("window_right", ctypes.c_int64),
                ("prefix", ctypes.c_int64), ("segment_ids", ctypes.c_void_p)]

HEAD_DIMS = (64, 128, 256)


class Fa2Error(RuntimeError):
    def __init__(self, status: int, msg: str, entry: str = "fa2_fwd"):
        super().__init__(f"{entry} failed: {msg} (status {status})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa2.so.  Raises ImportError when it has not been built.

    torch is imported first so that its HIP runtime is the one the library binds
    to (both carry the SONAME libamdhip64.so.7).
    """
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    import torch  # noqa: F401  (binds the HIP runtime before the library loads)

    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m exact_attention_11_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.fa2_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                            ctypes.c_int, vp]
    lib.fa2_fwd.restype = ctypes.c_int
    lib.fa2_fwd_masked.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.POINTER(Fa2Mask),
                                   ctypes.c_float, ctypes.c_int, vp]
    lib.fa2_fwd_masked.restype = ctypes.c_int
    lib.fa2_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                            ctypes.c_float, ctypes.c_int, vp]
    lib.fa2_bwd.restype = ctypes.c_int
    lib.fa2_bwd_masked.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                   ctypes.POINTER(Fa2Mask), ctypes.c_float, ctypes.c_int, vp]
    lib.fa2_bwd_masked.restype = ctypes.c_int
    lib.fa2_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float, vp, vp,
                                ctypes.c_int, vp]
    lib.fa2_fwd_fp8.restype = ctypes.c_int
    lib.fa2_fwd_fp8_masked.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.POINTER(Fa2Mask), ctypes.c_float,
                                       vp, vp, ctypes.c_int, vp]
    lib.fa2_fwd_fp8_masked.restype = ctypes.c_int
    lib.fa2_decode.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                               ctypes.c_int, vp, i64, vp]
    lib.fa2_decode.restype = ctypes.c_int
    lib.fa2_decode_static.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                                      ctypes.c_int, vp]
    lib.fa2_decode_static.restype = ctypes.c_int
    lib.fa2_decode_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
    lib.fa2_decode_workspace_bytes.restype = i64
    lib.fa2_clock_sample.argtypes = [vp, vp]
    lib.fa2_clock_sample.restype = ctypes.c_int
    lib.fa2_status_str.argtypes = [ctypes.c_int]
    lib.fa2_status_str.restype = ctypes.c_char_p
    lib.fa2_last_hip_error.argtypes = []
    lib.fa2_last_hip_error.restype = ctypes.c_int
    if path == LIB_PATH:
        _lib = lib
    return lib


def fa2_fwd(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, d: int,
            causal: int, scale: float, dtype: int, stream: int) -> int:
    """Direct call of the C entry point with raw device addresses; returns the status."""
    return load_library().fa2_fwd(q, k, v, o, lse, B, H, N, d, int(causal), float(scale), int(dtype),
                                  stream)


def fa2_fwd_masked(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, d: int, mask,
                   scale: float, dtype: int, stream: int) -> int:
    """Direct call of the masked forward entry point (mask: a Fa2Mask or None)."""
    ptr = ctypes.byref(mask) if mask is not None else None
    return load_library().fa2_fwd_masked(q, k, v, o, lse, B, H, N, d, ptr, float(scale), int(dtype), stream)


def fa2_bwd(q: int, k: int, v: int, o: int, dout: int, lse: int, delta: int, dq: int, dk: int, dv: int,
            B: int, H: int, N: int, d: int, causal: int, scale: float, dtype: int, stream: int) -> int:
    """Direct call of the gradient entry point with raw device addresses; returns the status."""
    return load_library().fa2_bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, N, d, int(causal),
                                  float(scale), int(dtype), stream)


def fa2_bwd_masked(q: int, k: int, v: int, o: int, dout: int, lse: int, delta: int, dq: int, dk: int, dv: int,
                   B: int, H: int, N: int, d: int, mask, scale: float, dtype: int, stream: int) -> int:
    """Direct call of the masked gradient entry point (mask: a Fa2Mask or None)."""
    ptr = ctypes.byref(mask) if mask is not None else None
    return load_library().fa2_bwd_masked(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, N, d, ptr, float(scale),
                                         int(dtype), stream)


def _general_mask(causal, window, prefix, segment_ids, B, N, device):
    """A Fa2Mask for a general mask, or None when there is none."""
    import torch

    if window is None and not prefix and segment_ids is None:
        return None
    wl, wr = (-1, -1) if window is None else (int(window[0]), int(window[1]))
    seg_ptr = None
    if segment_ids is not None:
        if (segment_ids.shape != (B, N) or segment_ids.dtype != torch.int32 or not segment_ids.is_contiguous()
                or segment_ids.device != device):
            raise ValueError("segment_ids must be a contiguous int32 [B, N] tensor on q's device")
        seg_ptr = segment_ids.data_ptr()
    return Fa2Mask(int(bool(causal)), wl, wr, int(prefix), seg_ptr)


def fa2_fwd_fp8_masked(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, d: int, mask,
                       scale: float, descale_q: int | None, descale_k: int | None, dtype: int, stream: int) -> int:
    """Direct call of the masked fp8 forward entry point (mask: a Fa2Mask or None)."""
    ptr = ctypes.byref(mask) if mask is not None else None
    return load_library().fa2_fwd_fp8_masked(q, k, v, o, lse, B, H, N, d, ptr, float(scale), descale_q, descale_k,
                                             int(dtype), stream)


def fa2_fwd_fp8(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, d: int, causal: int,
                scale: float, descale_q: int | None, descale_k: int | None, dtype: int, stream: int) -> int:
    """Direct call of the fp8 forward entry point with raw device addresses; returns the status."""
    return load_library().fa2_fwd_fp8(q, k, v, o, lse, B, H, N, d, int(causal), float(scale), descale_q, descale_k,
                                      int(dtype), stream)


def fa2_decode(q: int, k: int, v: int, seqlens: int | None, o: int, lse: int, B: int, H: int, Mq: int, Nk: int,
               d: int, causal: int, scale: float, dtype: int, workspace: int | None, workspace_bytes: int,
               stream: int) -> int:
    """Direct call of the decode entry point with raw device addresses; returns the status."""
    return load_library().fa2_decode(q, k, v, seqlens, o, lse, B, H, Mq, Nk, d, int(causal), float(scale),
                                     int(dtype), workspace, int(workspace_bytes), stream)


def fa2_decode_static(q: int, k: int, v: int, seqlens: int | None, o: int, lse: int, B: int, H: int, Mq: int,
                      Nk: int, d: int, causal: int, scale: float, dtype: int, stream: int) -> int:
    """Direct call of the allocation-free decode entry point (chunk partials in
    the library's fixed device scratch); returns the status."""
    return load_library().fa2_decode_static(q, k, v, seqlens, o, lse, B, H, Mq, Nk, d, int(causal), float(scale),
                                            int(dtype), stream)


def fa2_decode_workspace_bytes(B: int, H: int, Mq: int, Nk: int, d: int) -> int:
    """Workspace bytes fa2_decode needs (0: none), or minus a status code."""
    return load_library().fa2_decode_workspace_bytes(B, H, Mq, Nk, d)


def fa2_clock_sample(out: int, stream: int) -> int:
    """Direct call of the clock-sample entry point (out: device address of
    4 * CLOCK_BLOCKS uint64 values); returns the status."""
    return load_library().fa2_clock_sample(out, stream)


def clock_sample(out, stream=None):
    """Enqueue fa2_clock_sample into ``out`` (an int64 device tensor of
    4 * CLOCK_BLOCKS elements) on ``stream`` (default: the current stream)."""
    import torch

    if out.dtype != torch.int64 or out.numel() != 4 * CLOCK_BLOCKS or not out.is_cuda or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous int64 device tensor of {4 * CLOCK_BLOCKS} elements")
    with torch.cuda.device(out.device):
        s = stream if stream is not None else torch.cuda.current_stream(out.device)
        rc = fa2_clock_sample(out.data_ptr(), s.cuda_stream)
    if rc != FA2_OK:
        raise Fa2Error(rc, fa2_status_str(rc), "fa2_clock_sample")
    return out


def clock_ghz(before, after):
    """Average engine clock (GHz) between two clock samples (host sequences of
    4 * CLOCK_BLOCKS integers from fa2_clock_sample), per CU: each CU's own
    shader-clock counter difference over the real-time difference (100 MHz
    ticks), from the first record of that CU in each sample.  Returns
    {(xcd, cu key): GHz} for the CUs seen in both samples."""
    def first(sample):
        seen = {}
        for i in range(len(sample) // 4):
            xcc, hw, t, r = (int(x) for x in sample[4 * i:4 * i + 4])
            seen.setdefault((xcc, (hw >> 8) & 0xFF), (t, r))
        return seen

    b, a = first(list(before)), first(list(after))
    out = {}
    for cu in sorted(set(b) & set(a)):
        dt, dr = a[cu][0] - b[cu][0], a[cu][1] - b[cu][1]
        if dr > 0 and dt > 0:
            out[cu] = dt / dr * 0.1
    return out


def xcd_clocks(per_cu: dict) -> dict:
    """Per XCD, the clock of its busiest CU (the largest per-CU average: a CU's
    counter almost stops while it idles, so less busy CUs read low)."""
    out = {}
    for (xcc, _), ghz in per_cu.items():
        out[xcc] = max(out.get(xcc, 0.0), ghz)
    return out


def fa2_status_str(status: int) -> str:
    return load_library().fa2_status_str(int(status)).decode()


def fa2_last_hip_error() -> int:
    return load_library().fa2_last_hip_error()


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float16:
        return FA2_DTYPE_FP16
    if t.dtype == torch.bfloat16:
        return FA2_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float16 or bfloat16")


def forward(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None, stream=None,
            window=None, prefix: int = 0, segment_ids=None):
    """Attention forward on the GPU.  Returns ``(o, lse)``.

    ``scale`` defaults to 1/sqrt(d) (computed here, not in the library).  ``out``
    and ``lse`` may be given preallocated; ``stream`` defaults to torch's current
    stream of the tensors' device.  A general mask: ``window=(left, right)``
    (-1 for no bound), ``prefix`` (keys below it visible to every query of the
    same segment) and ``segment_ids`` (an int32 [B, N] tensor on the device).
    """
    import torch

    if not (q.shape == k.shape == v.shape) or q.dim() != 4:
        raise ValueError(f"q, k, v must share one [B, H, N, d] shape, got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    code = _dtype_code(q)
    if not (q.is_cuda and k.is_cuda and v.is_cuda) or not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one GPU")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous [B, H, N, d]")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    mask = _general_mask(causal, window, prefix, segment_ids, B, N, q.device)
    general = mask is not None
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        if general:
            rc = fa2_fwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                B, H, N, d, mask, float(scale), code, s.cuda_stream)
        else:
            rc = fa2_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                         B, H, N, d, int(bool(causal)), float(scale), code, s.cuda_stream)
    if rc != FA2_OK:
        raise Fa2Error(rc, fa2_status_str(rc))
    return out, lse


def backward(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None, stream=None,
             delta=None, dq=None, dk=None, dv=None, window=None, prefix: int = 0, segment_ids=None):
    """Gradients of attention on the GPU.  Returns ``(dq, dk, dv)``.

    ``o`` and ``lse`` are the forward pass's outputs for the same ``q, k, v``,
    ``causal``, ``scale`` and mask (``window``, ``prefix``, ``segment_ids``, as
    for ``forward``); ``dout`` is the gradient of the loss with respect to
    ``o``.  ``delta`` ([B, H, N] float32) receives the row statistic
    D = rowsum(dout * o); it and the outputs are allocated here unless given.
    """
    import torch

    ts = (q, k, v, o, dout)
    if q.dim() != 4 or any(t.shape != q.shape for t in ts):
        raise ValueError("q, k, v, o, dout must share one [B, H, N, d] shape")
    if any(t.dtype != q.dtype for t in ts):
        raise TypeError("q, k, v, o, dout must share one dtype")
    code = _dtype_code(q)
    if any(not t.is_cuda or t.device != q.device for t in ts + (lse,)):
        raise ValueError("all tensors must be on one GPU")
    if any(not t.is_contiguous() for t in ts + (lse,)):
        raise ValueError("all tensors must be contiguous")
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, N]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    own_delta = delta is None
    delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if own_delta else delta
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t in (dq, dk, dv):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device:
            raise ValueError("dq, dk, dv must be contiguous tensors like q")
    if (delta.shape != (B, H, N) or delta.dtype != torch.float32 or not delta.is_contiguous()
            or not delta.is_cuda or delta.device != q.device):
        raise ValueError("delta must be a contiguous float32 [B, H, N] tensor on q's device")
    mask = _general_mask(causal, window, prefix, segment_ids, B, N, q.device)
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        if own_delta:
            # delta is dropped on return while the kernels may still use it on s:
            # the caching allocator must not hand its block to other streams first.
            delta.record_stream(s)
        if mask is not None:
            rc = fa2_bwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                lse.data_ptr(), delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H,
                                N, d, mask, float(scale), code, s.cuda_stream)
        else:
            rc = fa2_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                         delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d,
                         int(bool(causal)), float(scale), code, s.cuda_stream)
    if rc != FA2_OK:
        raise Fa2Error(rc, fa2_status_str(rc), "fa2_bwd_masked" if mask is not None else "fa2_bwd")
    return dq, dk, dv


def _decode_args(q, k, v, seqlens, out, lse):
    """Checks shared by decode() and decode_static(); returns (B, H, Mq, Nk, d,
    dtype code, seqlens address, out, lse)."""
    import torch

    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError(f"expected q [B, H, Mq, d] and k, v [B, H, Nk, d], got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    code = _dtype_code(q)
    if not (q.is_cuda and k.is_cuda and v.is_cuda) or not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one GPU")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, Mq, d = q.shape
    Nk = k.shape[2]
    len_ptr = None
    if seqlens is not None:
        if (seqlens.shape != (B,) or seqlens.dtype != torch.int32 or not seqlens.is_contiguous()
                or seqlens.device != q.device):
            raise ValueError("seqlens must be a contiguous int32 [B] tensor on q's device")
        len_ptr = seqlens.data_ptr()
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Mq), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (B, H, Mq) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, Mq] tensor on q's device")
    return B, H, Mq, Nk, d, code, len_ptr, out, lse


def decode(q, k, v, seqlens=None, causal: bool = False, scale: float | None = None, out=None, lse=None,
           stream=None, workspace=None):
    """Decode on the GPU: ``q`` [B, H, Mq, d] (1 <= Mq <= 8 new rows) against the
    cache ``k, v`` [B, H, Nk, d], of which the first ``seqlens[b]`` rows are
    valid (``seqlens``: int32 [B] on the device, or None for all Nk).  The new
    rows are the last Mq positions of each sequence; under ``causal`` query i
    sees keys c <= seqlens[b] - Mq + i.  Returns ``(o, lse)``; a query with no
    visible key gets o = 0 and lse = -inf.  ``workspace`` (a uint8 device
    tensor of at least ``fa2_decode_workspace_bytes`` bytes) is allocated here
    when needed and not given.
    """
    import torch

    B, H, Mq, Nk, d, code, len_ptr, out, lse = _decode_args(q, k, v, seqlens, out, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa2_decode_workspace_bytes(B, H, Mq, Nk, d)
    if need < 0:
        raise Fa2Error(-need, fa2_status_str(-need), "fa2_decode")
    own_ws = workspace is None and need > 0
    if own_ws:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif workspace is not None and (not workspace.is_cuda or workspace.device != q.device
                                    or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        if own_ws:
            # The workspace is dropped on return while the kernels may still use
            # it on s: keep its block from other streams until they are done.
            workspace.record_stream(s)
        rc = fa2_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), len_ptr, out.data_ptr(), lse.data_ptr(),
                        B, H, Mq, Nk, d, int(bool(causal)), float(scale), code, ws_ptr, ws_bytes, s.cuda_stream)
    if rc != FA2_OK:
        raise Fa2Error(rc, fa2_status_str(rc), "fa2_decode")
    return out, lse


def decode_static(q, k, v, seqlens=None, causal: bool = False, scale: float | None = None, out=None, lse=None,
                  stream=None):
    """decode() through fa2_decode_static: no workspace, the chunk partials go
    to the library's fixed device scratch (at most DECODE_STATIC_SCRATCH_BYTES;
    calls that may overlap on one device race on it).  With ``out`` and
    ``lse`` given, this call allocates no device memory."""
    import torch

    B, H, Mq, Nk, d, code, len_ptr, out, lse = _decode_args(q, k, v, seqlens, out, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        rc = fa2_decode_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), len_ptr, out.data_ptr(), lse.data_ptr(),
                               B, H, Mq, Nk, d, int(bool(causal)), float(scale), code, s.cuda_stream)
    if rc != FA2_OK:
        raise Fa2Error(rc, fa2_status_str(rc), "fa2_decode_static")
    return out, lse


def forward_fp8(q8, k8, v, descale_q=None, descale_k=None, causal: bool = False, scale: float | None = None,
                out=None, lse=None, stream=None, window=None, prefix: int = 0, segment_ids=None):
    """Attention forward with Q and K in fp8 (``torch.float8_e4m3fn``, [B, H, N,
    d], d = 64, 128 or 256) and V in fp16 or bf16.  The real inputs are ``q8 * descale_q[b*H + h]``
    and ``k8 * descale_k[b*H + h]`` (``descale_*``: float32 [B*H] device tensors,
    or None for ones).  ``window``, ``prefix`` and ``segment_ids`` give a general
    mask, as for ``forward``.  Returns ``(o, lse)`` with ``o`` in V's dtype."""
    import torch

    if not (q8.shape == k8.shape == v.shape) or q8.dim() != 4:
        raise ValueError("q8, k8, v must share one [B, H, N, d] shape")
    if q8.dtype != torch.float8_e4m3fn or k8.dtype != torch.float8_e4m3fn:
        raise TypeError("q8 and k8 must be torch.float8_e4m3fn")
    code = _dtype_code(v)
    ts = (q8, k8, v)
    if any(not t.is_cuda or t.device != v.device for t in ts) or any(not t.is_contiguous() for t in ts):
        raise ValueError("q8, k8, v must be contiguous tensors on one GPU")
    B, H, N, d = v.shape
    ptrs = []
    for ds in (descale_q, descale_k):
        if ds is None:
            ptrs.append(None)
            continue
        if ds.shape != (B * H,) or ds.dtype != torch.float32 or not ds.is_contiguous() or ds.device != v.device:
            raise ValueError("descales must be contiguous float32 [B*H] tensors on the inputs' device")
        ptrs.append(ds.data_ptr())
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(v) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=v.device) if lse is None else lse
    if out.shape != v.shape or out.dtype != v.dtype or not out.is_contiguous() or out.device != v.device:
        raise ValueError("out must be a contiguous tensor like v")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != v.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on the inputs' device")
    mask = _general_mask(causal, window, prefix, segment_ids, B, N, v.device)
    with torch.cuda.device(v.device):
        s = stream if stream is not None else torch.cuda.current_stream(v.device)
        if mask is not None:
            rc = fa2_fwd_fp8_masked(q8.data_ptr(), k8.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H,
                                    N, d, mask, float(scale), ptrs[0], ptrs[1], code, s.cuda_stream)
        else:
            rc = fa2_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
                             int(bool(causal)), float(scale), ptrs[0], ptrs[1], code, s.cuda_stream)
    if rc != FA2_OK:
        raise Fa2Error(rc, fa2_status_str(rc), "fa2_fwd_fp8_masked" if mask is not None else "fa2_fwd_fp8")
    return out, lse

