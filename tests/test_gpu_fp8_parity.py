"""GPU parity of the fp8 forward pass (fa2_fwd_fp8 through the C ABI: Q and K in
OCP e4m3 with per-head descales, V and O in fp16/bf16) against the fp64 oracle
(oracle/attention_ref.c) run on the real inputs q8 * descale_q, k8 * descale_k
and V.

The products q.k of the stored e4m3 values are exact in the fp8 MFMA's fp32
accumulation; the weights and P.V are those of the 16-bit forward pass.  The
tolerances are therefore the 16-bit ones, by V's type: max |dO| <= 2e-3
(fp16) / 1e-2 (bf16), max |dL| <= 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_11_amd as fa
import oracle
from exact_attention_11_amd.inputs import make_qkv_fp8

pytestmark = pytest.mark.gpu

TOL_O = {torch.float16: 2e-3, torch.bfloat16: 1e-2}
TOL_L = 1e-3


def _log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()


def _real(x8, ds, B, H):
    return (x8.to(torch.float64) * ds.to(torch.float64).reshape(B, H, 1, 1)).numpy()


def _case(B, H, N, v_dtype, causal, dist="normal", seed=0, descales=True, scale=None):
    d = 128
    q8, k8, v, dq, dk = make_qkv_fp8(B, H, N, d, v_dtype, dist, seed)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    what = f"B={B} H={H} N={N} {v_dtype} causal={causal} {dist} descales={descales} scale={scale}"
    _log(f"case {what}")
    if not descales:
        dq = torch.ones_like(dq)
        dk = torch.ones_like(dk)
    o, lse = fa.forward_fp8(q8.cuda(), k8.cuda(), v.cuda(), dq.cuda() if descales else None,
                            dk.cuda() if descales else None, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_f64(_real(q8, dq, B, H), _real(k8, dk, B, H), v.double().numpy(), causal,
                                        float(np.float32(scale)))
    do = np.abs(o.cpu().double().numpy() - o_ref)
    dl = np.abs(lse.cpu().double().numpy() - l_ref)
    _log(f"  max|dO|={do.max():.3e} max|dL|={dl.max():.3e}")
    assert np.all(np.isfinite(o.cpu().double().numpy()))
    assert do.max() <= TOL_O[v_dtype], (what, float(do.max()), np.unravel_index(np.argmax(do), do.shape))
    assert dl.max() <= TOL_L, (what, float(dl.max()), np.unravel_index(np.argmax(dl), dl.shape))


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 255, 256, 257, 600, 1000])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("v_dtype", [torch.float16, torch.bfloat16], ids=["fp16", "bf16"])
def test_fp8_parity_ragged_sweep(v_dtype, causal, N):
    _case(1, 2, N, v_dtype, causal, seed=1)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_parity_batch_heads(causal):
    _case(2, 3, 700, torch.float16, causal, seed=2)


def test_fp8_parity_without_descales_and_peaky():
    """Descales of one (the e4m3 values themselves are the inputs, |q|, |k| up to
    448) and peaky scores.  The multiplier 2^-17 brings the scores back to the
    size the other cases have: the fp32 accumulation of q.k rounds relative to
    the size of the products, and a multiplier of 2^-12 would leave scores of
    ~30 in which that rounding alone moves weights by a percent."""
    _case(1, 2, 500, torch.float16, True, seed=3, descales=False, scale=2.0 ** -17)
    _case(1, 2, 900, torch.bfloat16, False, dist="peaky", seed=4)


@pytest.mark.parametrize("scale", [0.0, -0.05])
def test_fp8_parity_unusual_scales(scale):
    _case(1, 2, 300, torch.float16, True, seed=5, scale=scale)


def test_fp8_full_size_sampled():
    """The long-context causal workload's shape (1 x 32 heads x 16384 x 128) in
    fp8, checked on strided rows of three heads."""
    B, H, N, d = 1, 32, 16384, 128
    q8, k8, v, dq, dk = make_qkv_fp8(B, H, N, d, torch.float16, "normal", 0)
    _log(f"case full size B={B} H={H} N={N}")
    o, lse = fa.forward_fp8(q8.cuda(), k8.cuda(), v.cuda(), dq.cuda(), dk.cuda(), causal=True)
    torch.cuda.synchronize()
    scale = float(np.float32(1.0 / math.sqrt(d)))
    rows = np.concatenate([np.arange(0, 300), np.arange(300, N, 997), np.arange(N - 300, N)]).astype(np.int64)
    for h in (0, 13, 31):
        qq = (q8[0, h].to(torch.float64) * float(dq[h])).numpy()
        kk = (k8[0, h].to(torch.float64) * float(dk[h])).numpy()
        o_ref, l_ref = oracle.attention_rows_f64(qq, kk, v[0, h].double().numpy(), rows, True, scale)
        do = np.abs(o[0, h].cpu().double().numpy()[rows] - o_ref)
        dl = np.abs(lse[0, h].cpu().double().numpy()[rows] - l_ref)
        _log(f"  head {h}: max|dO|={do.max():.3e} max|dL|={dl.max():.3e}")
        assert do.max() <= TOL_O[torch.float16] and dl.max() <= TOL_L, (h, do.max(), dl.max())


# --- general masks (fa2_fwd_fp8_masked) ---------------------------------------------

def _segments(kind, B, N, seed):
    """[B, N] int32 segment ids: 'docs' contiguous documents of random lengths,
    'blocks' ids that repeat after other ids."""
    rng = np.random.default_rng(500 + seed)
    ids = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        if kind == "docs":
            cuts = np.sort(rng.choice(np.arange(1, N), size=min(4, N - 1), replace=False)) if N > 1 else []
            for i, c in enumerate(cuts):
                ids[b, c:] = i + 1
        else:
            ids[b] = (np.arange(N) // 41) % 3
    return ids


FP8_MASKS = {
    "window": dict(window=(37, 20)),
    "causal_window": dict(window=(100, -1), causal=True),
    "prefix_causal_window": dict(window=(64, -1), causal=True, prefix=50),
    "prefix_two_sided": dict(window=(30, 30), prefix=70),
    "docs_causal": dict(segments="docs", causal=True),
    "blocks": dict(segments="blocks"),
    "docs_prefix_window": dict(segments="docs", prefix=20, window=(150, 10)),
}


def _masked_case(B, H, N, v_dtype, mask_name, seed=0):
    m = FP8_MASKS[mask_name]
    d = 128
    q8, k8, v, dq, dk = make_qkv_fp8(B, H, N, d, v_dtype, "normal", seed)
    scale = 1.0 / math.sqrt(d)
    seg = _segments(m["segments"], B, N, seed) if "segments" in m else None
    window = m.get("window")
    causal = bool(m.get("causal", False))
    prefix = int(m.get("prefix", 0))
    what = f"B={B} H={H} N={N} {v_dtype} mask={mask_name}"
    _log(f"case {what}")
    segc = torch.from_numpy(seg).cuda() if seg is not None else None
    o, lse = fa.forward_fp8(q8.cuda(), k8.cuda(), v.cuda(), dq.cuda(), dk.cuda(), causal=causal, scale=scale,
                            window=window, prefix=prefix, segment_ids=segc)
    torch.cuda.synchronize()
    wl, wr = (-1, -1) if window is None else window
    o_ref, l_ref = oracle.attention_masked_f64(_real(q8, dq, B, H), _real(k8, dk, B, H), v.double().numpy(),
                                               float(np.float32(scale)), window_left=wl, window_right=wr,
                                               prefix=prefix, segment_ids=seg, causal=causal)
    do = np.abs(o.cpu().double().numpy() - o_ref)
    dl = np.abs(lse.cpu().double().numpy() - l_ref)
    _log(f"  max|dO|={do.max():.3e} max|dL|={dl.max():.3e}")
    assert np.all(np.isfinite(o.cpu().double().numpy()))
    assert do.max() <= TOL_O[v_dtype], (what, float(do.max()), np.unravel_index(np.argmax(do), do.shape))
    assert dl.max() <= TOL_L, (what, float(dl.max()), np.unravel_index(np.argmax(dl), dl.shape))


@pytest.mark.parametrize("mask_name", sorted(FP8_MASKS))
@pytest.mark.parametrize("v_dtype", [torch.float16, torch.bfloat16], ids=["fp16", "bf16"])
def test_fp8_masked_parity(v_dtype, mask_name):
    """700 rows: three query tiles per head, two runs of key tiles under a
    prefix, a ragged last tile."""
    _masked_case(2, 2, 700, v_dtype, mask_name, seed=6)


@pytest.mark.parametrize("mask_name", ["prefix_causal_window", "docs_prefix_window"])
@pytest.mark.parametrize("N", [1, 2, 65, 257])
def test_fp8_masked_parity_short(N, mask_name):
    _masked_case(1, 2, N, torch.float16, mask_name, seed=7)


def test_fp8_masked_reductions_match_plain_entry():
    """Masks that reduce to none or causal take the plain fp8 instances: bitwise
    the same as fa2_fwd_fp8."""
    B, H, N, d = 1, 2, 300, 128
    q8, k8, v, dq, dk = make_qkv_fp8(B, H, N, d, torch.float16, "normal", 8)
    args = (q8.cuda(), k8.cuda(), v.cuda(), dq.cuda(), dk.cuda())
    for causal, kw in ((True, dict(causal=True, window=(-1, -1))), (True, dict(window=(-1, 0))),
                       (False, dict(window=(400, 400))), (False, dict(prefix=N, window=(3, 3)))):
        a = fa.forward_fp8(*args, causal=causal, scale=0.1)
        b = fa.forward_fp8(*args, scale=0.1, **kw)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y), kw
