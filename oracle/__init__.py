"""CPU oracle for exact attention -- TEST INFRASTRUCTURE, not the product.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the GPU library
and never imports it.

Contents
--------
``attention_f64`` / ``attention_rows_f64``
    The plain definition of attention (scores, row softmax, P.V, plus the
    natural-log logsumexp per row) in fp64, implemented in ``attention_ref.c``
    and loaded through ctypes.  See that file's header for the passages of the
    pages it follows.
``attention_masked_f64``
    The same definition under a general mask (sliding window, a prefix visible
    to every query, document segment ids), implemented in
    ``attention_mask_ref.c``.
``attention_bwd_f64``
    The gradients dQ, dK, dV of that definition for a given dO (and the row
    statistic D), by the chain rule in fp64, implemented in
    ``attention_bwd_ref.c``.
``attention_bwd_masked_f64``
    The same gradients under a general mask (the mask of
    ``attention_masked_f64``), implemented in ``attention_bwd_mask_ref.c``.
``attention_decode_f64``
    A few new query rows against a key/value cache with per-batch valid
    lengths (the last Mq positions of each sequence; causal or not),
    implemented in ``attention_decode_ref.c``.
``tiled``
    A numpy model of the tiled forward recurrence the pages describe (online
    softmax, delayed normalisation, block-level causal skip).  It is used only to
    check that the recurrence reaches the definition and to reproduce the pages'
    printed intermediate values.

Inputs are exact fp64 upcasts of the fp16/bf16 values the GPU receives, and the
multiplier is the float32 value the GPU receives, widened to double.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attention_ref.c")
_BWD_SRC = os.path.join(_HERE, "attention_bwd_ref.c")
_MASK_SRC = os.path.join(_HERE, "attention_mask_ref.c")
_DECODE_SRC = os.path.join(_HERE, "attention_decode_ref.c")
_BWD_MASK_SRC = os.path.join(_HERE, "attention_bwd_mask_ref.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib_cache: dict[str, ctypes.CDLL] = {}


def build(src: str = _SRC, out: str = LIB_PATH, bwd_src: str = _BWD_SRC, mask_src: str = _MASK_SRC,
          decode_src: str = _DECODE_SRC, bwd_mask_src: str = _BWD_MASK_SRC) -> str:
    """Compile the C oracle (forward, gradient, general-mask, decode and
    masked-gradient sources) with gcc (no fast-math: IEEE fp64 throughout)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-pthread", src, bwd_src, mask_src, decode_src, bwd_mask_src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (building first if absent) the oracle library at ``path``."""
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path):
        if path != LIB_PATH:
            raise FileNotFoundError(path)
        build()
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lp = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.oracle_attention_f64.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64,
                                         ctypes.c_int, ctypes.c_double, ctypes.c_int]
    lib.oracle_attention_f64.restype = ctypes.c_int
    lib.oracle_attention_rows_f64.argtypes = [dp, dp, dp, lp, i64, dp, dp, i64, i64,
                                              ctypes.c_int, ctypes.c_double, ctypes.c_int]
    lib.oracle_attention_rows_f64.restype = ctypes.c_int
    lib.oracle_attention_bwd_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, i64, i64, i64, i64,
                                             ctypes.c_int, ctypes.c_double, ctypes.c_int]
    lib.oracle_attention_bwd_f64.restype = ctypes.c_int
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.oracle_attention_masked_f64.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64, i64, i64, i64, ip,
                                                ctypes.c_double, ctypes.c_int]
    lib.oracle_attention_masked_f64.restype = ctypes.c_int
    lib.oracle_attention_decode_f64.argtypes = [dp, dp, dp, ip, dp, dp, i64, i64, i64, i64, i64,
                                                ctypes.c_int, ctypes.c_double, ctypes.c_int]
    lib.oracle_attention_decode_f64.restype = ctypes.c_int
    lib.oracle_attention_bwd_masked_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, i64, i64, i64, i64, i64, i64,
                                                    i64, ip, ctypes.c_double, ctypes.c_int]
    lib.oracle_attention_bwd_masked_f64.restype = ctypes.c_int
    _lib_cache[path] = lib
    return lib


def _threads(nthreads: int | None) -> int:
    """Explicit count, else OMP_NUM_THREADS when set, else the affinity mask."""
    if nthreads is not None:
        return max(1, int(nthreads))
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def attention_f64(q, k, v, causal: bool, scale: float, nthreads: int | None = None,
                  lib_path: str = LIB_PATH):
    """Exact attention over [B, H, N, d] (or [N, d]) fp64 arrays.

    Returns ``(o, lse)`` with ``o`` shaped like ``q`` and ``lse`` shaped like
    ``q.shape[:-1]``.  ``scale`` is used as given (pass the float32 value the
    GPU sees, widened to double).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"shape mismatch {q.shape} {k.shape} {v.shape}")
    squeeze = q.ndim == 2
    if squeeze:
        q, k, v = q[None, None], k[None, None], v[None, None]
    if q.ndim != 4:
        raise ValueError("expected [B, H, N, d] or [N, d]")
    B, H, N, d = q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, N), dtype=np.float64)
    lib = load(lib_path)
    rc = lib.oracle_attention_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                  int(bool(causal)), float(scale), _threads(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_f64 failed with code {rc}")
    if squeeze:
        return o[0, 0], lse[0, 0]
    return o, lse


def attention_rows_f64(q, k, v, rows, causal: bool, scale: float, nthreads: int | None = None,
                       lib_path: str = LIB_PATH):
    """Exact attention for selected query ``rows`` of one head ([N, d] inputs).

    Returns ``(o_rows [R, d], lse_rows [R])``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 2 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("expected three [N, d] arrays of equal shape")
    N, d = q.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    R = rows.shape[0]
    o = np.empty((R, d), dtype=np.float64)
    lse = np.empty((R,), dtype=np.float64)
    lib = load(lib_path)
    rc = lib.oracle_attention_rows_f64(_ptr(q), _ptr(k), _ptr(v),
                                       rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), R,
                                       _ptr(o), _ptr(lse), N, d, int(bool(causal)), float(scale),
                                       _threads(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_rows_f64 failed with code {rc}")
    return o, lse



def attention_bwd_f64(q, k, v, dout, causal: bool, scale: float, nthreads: int | None = None,
                      lib_path: str = LIB_PATH):
    """Gradients of exact attention over [B, H, N, d] (or [N, d]) fp64 arrays.

    ``dout`` is the gradient with respect to the output O.  Returns
    ``(dq, dk, dv, delta)``: three arrays shaped like ``q`` and the row
    statistic D = rowsum(P o dP), shaped like ``q.shape[:-1]``.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    if not (q.shape == k.shape == v.shape == dout.shape):
        raise ValueError(f"shape mismatch {q.shape} {k.shape} {v.shape} {dout.shape}")
    squeeze = q.ndim == 2
    if squeeze:
        q, k, v, dout = q[None, None], k[None, None], v[None, None], dout[None, None]
    if q.ndim != 4:
        raise ValueError("expected [B, H, N, d] or [N, d]")
    B, H, N, d = q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    delta = np.empty((B, H, N), dtype=np.float64)
    lib = load(lib_path)
    rc = lib.oracle_attention_bwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                      _ptr(delta), B, H, N, d, int(bool(causal)), float(scale),
                                      _threads(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_bwd_f64 failed with code {rc}")
    if squeeze:
        return dq[0, 0], dk[0, 0], dv[0, 0], delta[0, 0]
    return dq, dk, dv, delta


def attention_masked_f64(q, k, v, scale: float, window_left: int = -1, window_right: int = -1,
                         prefix: int = 0, segment_ids=None, causal: bool = False,
                         nthreads: int | None = None, lib_path: str = LIB_PATH):
    """Exact attention over [B, H, N, d] fp64 arrays under a general mask.

    Key c is allowed for query r when c < N, ``segment_ids[b, c] ==
    segment_ids[b, r]`` (if given, an int array [B, N]), and either c < prefix
    or r - window_left <= c <= r + window_right (a negative bound is
    unbounded).  ``causal`` is window_right = 0 (combined with a given
    window_right by taking the smaller bound).  Returns ``(o, lse)``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if not (q.shape == k.shape == v.shape) or q.ndim != 4:
        raise ValueError("expected three [B, H, N, d] arrays of equal shape")
    B, H, N, d = q.shape
    wr = int(window_right)
    if causal:
        wr = 0 if wr < 0 else min(wr, 0)
    seg_ptr = None
    if segment_ids is not None:
        seg = np.ascontiguousarray(np.asarray(segment_ids, dtype=np.int32))
        if seg.shape != (B, N):
            raise ValueError("segment_ids must be [B, N]")
        seg_ptr = seg.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    o = np.empty_like(q)
    lse = np.empty((B, H, N), dtype=np.float64)
    lib = load(lib_path)
    rc = lib.oracle_attention_masked_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                         int(window_left), wr, int(prefix), seg_ptr, float(scale),
                                         _threads(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_masked_f64 failed with code {rc}")
    return o, lse


def attention_bwd_masked_f64(q, k, v, dout, scale: float, window_left: int = -1, window_right: int = -1,
                             prefix: int = 0, segment_ids=None, causal: bool = False,
                             nthreads: int | None = None, lib_path: str = LIB_PATH):
    """Gradients of exact attention over [B, H, N, d] fp64 arrays under the
    general mask of ``attention_masked_f64`` (same arguments).  Returns
    ``(dq, dk, dv, delta)`` as ``attention_bwd_f64`` does.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    if not (q.shape == k.shape == v.shape == dout.shape) or q.ndim != 4:
        raise ValueError("expected four [B, H, N, d] arrays of equal shape")
    B, H, N, d = q.shape
    wr = int(window_right)
    if causal:
        wr = 0 if wr < 0 else min(wr, 0)
    seg_ptr = None
    if segment_ids is not None:
        seg = np.ascontiguousarray(np.asarray(segment_ids, dtype=np.int32))
        if seg.shape != (B, N):
            raise ValueError("segment_ids must be [B, N]")
        seg_ptr = seg.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    delta = np.empty((B, H, N), dtype=np.float64)
    lib = load(lib_path)
    rc = lib.oracle_attention_bwd_masked_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                             _ptr(delta), B, H, N, d, int(window_left), wr, int(prefix), seg_ptr,
                                             float(scale), _threads(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_bwd_masked_f64 failed with code {rc}")
    return dq, dk, dv, delta


def attention_decode_f64(q, k, v, scale: float, seqlens=None, causal: bool = False,
                         nthreads: int | None = None, lib_path: str = LIB_PATH):
    """Exact attention of new query rows q [B, H, Mq, d] against a cache
    k, v [B, H, Nk, d] whose first ``seqlens[b]`` rows are valid (all Nk when
    None).  The new rows are the last Mq positions of each sequence: under
    ``causal`` query i sees keys c <= seqlens[b] - Mq + i.  A query with no
    visible key gets O = 0 and L = -inf.  Returns ``(o, lse)``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("expected q [B, H, Mq, d] and k, v [B, H, Nk, d]")
    B, H, Mq, d = q.shape
    Nk = k.shape[2]
    len_ptr = None
    if seqlens is not None:
        lens = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
        if lens.shape != (B,):
            raise ValueError("seqlens must be [B]")
        len_ptr = lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    o = np.empty_like(q)
    lse = np.empty((B, H, Mq), dtype=np.float64)
    lib = load(lib_path)
    rc = lib.oracle_attention_decode_f64(_ptr(q), _ptr(k), _ptr(v), len_ptr, _ptr(o), _ptr(lse), B, H, Mq, Nk, d,
                                         int(bool(causal)), float(scale), _threads(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_decode_f64 failed with code {rc}")
    return o, lse
