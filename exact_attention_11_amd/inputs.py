"""Seeded synthetic inputs and the named workloads.

This module only draws random numbers and describes shapes; it holds none of
the attention arithmetic, so both the GPU path and the CPU oracle can take their
inputs from it.

The pages measure on synthetic attention shapes (sequence lengths 512-16k,
head dims 64 and 128, batch 8 at length 4096), and the one value distribution
they show is i.i.d. standard normal from a fixed seed ("Flash Attention: Memory-
Efficient Attention at Scale", section "Online softmax", the tiled example).
The workloads below stand in for those sweeps.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str     # "fp16" or "bf16"
    causal: bool
    dist: str      # "normal": Q, K, V ~ N(0, 1); "peaky": Q, K ~ 3 N(0, 1), V ~ U(-1, 1)
    what: str

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "fp16" else torch.bfloat16


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_d64", 1, 1, 128, 64, "fp16", False, "normal",
                 "single head, 128 tokens, head dim 64, no mask"),
        Workload("b8h16_n2048_d64", 8, 16, 2048, 64, "fp16", False, "normal",
                 "batch 8 x 16 heads, 2048 tokens, head dim 64, no mask (16k tokens)"),
        Workload("b8h16_n2048_d128_causal", 8, 16, 2048, 128, "bf16", True, "normal",
                 "batch 8 x 16 heads, 2048 tokens, head dim 128, causal"),
        Workload("b1h32_n16384_d128_causal", 1, 32, 16384, 128, "fp16", True, "normal",
                 "batch 1 x 32 heads, 16384 tokens, head dim 128, causal (long context)"),
        Workload("b4h8_n4099_d256_peaky", 4, 8, 4099, 256, "bf16", False, "peaky",
                 "batch 4 x 8 heads, 4099 tokens (ragged), head dim 256, peaky scores, no mask"),
    ]
}


def make_qkv(B: int, H: int, N: int, d: int, dtype, dist: str = "normal", seed: int = 0):
    """Host tensors q, k, v of shape [B, H, N, d] in ``dtype`` (fp16/bf16).

    Drawn in fp32 from ``torch.Generator('cpu').manual_seed(seed)`` in the order
    Q, K, V, then rounded once to ``dtype`` (round to nearest even).
    """
    if isinstance(dtype, str):
        dtype = torch.float16 if dtype == "fp16" else torch.bfloat16
    g = torch.Generator("cpu").manual_seed(seed)
    shape = (B, H, N, d)
    if dist == "normal":
        q = torch.randn(shape, generator=g, dtype=torch.float32)
        k = torch.randn(shape, generator=g, dtype=torch.float32)
        v = torch.randn(shape, generator=g, dtype=torch.float32)
    elif dist == "peaky":
        q = torch.randn(shape, generator=g, dtype=torch.float32) * 3.0
        k = torch.randn(shape, generator=g, dtype=torch.float32) * 3.0
        v = torch.rand(shape, generator=g, dtype=torch.float32) * 2.0 - 1.0
    else:
        raise ValueError(dist)
    return q.to(dtype), k.to(dtype), v.to(dtype)


def workload_inputs(w: Workload, seed: int = 0):
    return make_qkv(w.B, w.H, w.N, w.d, w.torch_dtype, w.dist, seed)


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    H: int
    Mq: int        # new query rows per (batch, head)
    Nk: int        # cache capacity
    d: int
    dtype: str     # "fp16" or "bf16"
    causal: bool
    lengths: str   # "full": every cache row valid; "ragged": lengths drawn uniformly from [1, Nk]
    what: str

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "fp16" else torch.bfloat16


# Decode against a cache as long as the longest forward workload (16384 tokens,
# head dim 128): a batch of 8 sequences x 32 heads, one new token each.
DECODE_WORKLOADS = {
    w.name: w for w in [
        DecodeWorkload("decode_b8h32_m1_n16384_d128", 8, 32, 1, 16384, 128, "fp16", True, "full",
                       "batch 8 x 32 heads, 1 new token against a 16384-token cache, head dim 128"),
        DecodeWorkload("decode_b8h32_m1_n16384_d128_ragged", 8, 32, 1, 16384, 128, "fp16", True, "ragged",
                       "batch 8 x 32 heads, 1 new token against caches of 1-16384 valid tokens, head dim 128"),
        DecodeWorkload("decode_b1h32_m4_n16384_d128", 1, 32, 4, 16384, 128, "bf16", True, "full",
                       "batch 1 x 32 heads, 4 new tokens (causal) against a 16384-token cache, head dim 128"),
    ]
}


def make_decode_inputs(B: int, H: int, Mq: int, Nk: int, d: int, dtype, seed: int = 0):
    """Host tensors q [B, H, Mq, d] and k, v [B, H, Nk, d] in ``dtype``: i.i.d.
    N(0, 1) drawn in fp32 from ``torch.Generator('cpu').manual_seed(seed)`` in
    the order Q, K, V, rounded once to ``dtype``."""
    if isinstance(dtype, str):
        dtype = torch.float16 if dtype == "fp16" else torch.bfloat16
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((B, H, Mq, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, H, Nk, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, H, Nk, d), generator=g, dtype=torch.float32)
    return q.to(dtype), k.to(dtype), v.to(dtype)


def decode_lengths(B: int, Nk: int, kind: str, seed: int = 0):
    """int32 host tensor [B] of valid cache lengths: "full" (all Nk) or
    "ragged" (uniform on [1, Nk], seeded)."""
    if kind == "full":
        return torch.full((B,), Nk, dtype=torch.int32)
    if kind == "ragged":
        g = torch.Generator("cpu").manual_seed(10_000 + seed)
        return torch.randint(1, max(Nk, 1) + 1, (B,), generator=g, dtype=torch.int32)
    raise ValueError(kind)


def decode_workload_inputs(w: DecodeWorkload, seed: int = 0):
    q, k, v = make_decode_inputs(w.B, w.H, w.Mq, w.Nk, w.d, w.torch_dtype, seed)
    return q, k, v, decode_lengths(w.B, w.Nk, w.lengths, seed)


FP8_E4M3_MAX = 448.0  # largest finite OCP e4m3 value


def make_qkv_fp8(B: int, H: int, N: int, d: int, v_dtype, dist: str = "normal", seed: int = 0):
    """Q and K quantised to OCP e4m3 with one scale per (batch, head), V in
    ``v_dtype``: the values of ``make_qkv(B, H, N, d, float32-like, dist, seed)``
    (drawn in fp32 in the order Q, K, V), with Q[b, h] divided by
    descale_q[b*H + h] = max |Q[b, h]| / 448 and cast to e4m3 by torch (round
    to nearest even), likewise K.  Returns host tensors
    ``(q8, k8, v, descale_q, descale_k)``; q8 * descale_q and k8 * descale_k are
    the real inputs."""
    if isinstance(v_dtype, str):
        v_dtype = torch.float16 if v_dtype == "fp16" else torch.bfloat16
    g = torch.Generator("cpu").manual_seed(seed)
    shape = (B, H, N, d)
    if dist == "normal":
        q = torch.randn(shape, generator=g, dtype=torch.float32)
        k = torch.randn(shape, generator=g, dtype=torch.float32)
        v = torch.randn(shape, generator=g, dtype=torch.float32)
    elif dist == "peaky":
        q = torch.randn(shape, generator=g, dtype=torch.float32) * 3.0
        k = torch.randn(shape, generator=g, dtype=torch.float32) * 3.0
        v = torch.rand(shape, generator=g, dtype=torch.float32) * 2.0 - 1.0
    else:
        raise ValueError(dist)

    def quant(x):
        amax = x.abs().amax(dim=(2, 3)).clamp_min(1e-30)           # [B, H]
        ds = (amax / FP8_E4M3_MAX).to(torch.float32)
        x8 = (x / ds[:, :, None, None]).clamp(-FP8_E4M3_MAX, FP8_E4M3_MAX).to(torch.float8_e4m3fn)
        return x8, ds.reshape(-1).contiguous()

    q8, dq = quant(q)
    k8, dk = quant(k)
    return q8, k8, v.to(v_dtype), dq, dk

