"""GPU parity of the forward pass under general masks (fa2_fwd_masked through
the C ABI) against the fp64 general-mask oracle (oracle/attention_mask_ref.c).

Tolerances as for the plain forward pass: max |dO| <= 2e-3 (fp16) / 1e-2
(bf16), max |dL| <= 1e-3 over every element.  Under narrow windows and at the
start of documents a row averages a handful of values, so |O| approaches |v|
(about 3 for normal inputs), where rounding O to bf16 alone costs up to 8e-3:
V is scaled by 1/4 (exact) so that |O| stays near 1, where the absolute
tolerances apply.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_11_amd as fa
import oracle
from exact_attention_11_amd.inputs import make_qkv

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


def _segments(B, N, kind, seed, n_docs=4):
    rng = np.random.default_rng(seed)
    seg = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        cuts = np.sort(rng.choice(np.arange(1, N), size=min(N - 1, n_docs), replace=False)) if N > 1 else []
        runs = np.searchsorted(cuts, np.arange(N), side="right")
        if kind == "documents":  # contiguous documents of random lengths, ids increasing
            seg[b] = runs
        elif kind == "shuffled":  # contiguous runs whose ids go up and down and repeat
            seg[b] = rng.integers(0, max(2, n_docs // 2), size=runs.max() + 1)[runs]
        else:  # interleaved ids
            seg[b] = rng.integers(0, 3, size=N)
    return seg


def _case(B, H, N, d, dtype, window=None, prefix=0, seg_kind=None, causal=False, seed=0, n_docs=4):
    q, k, v = make_qkv(B, H, N, d, dtype, "normal", seed)
    v = v * 0.25
    scale = 1.0 / math.sqrt(d)
    seg = _segments(B, N, seg_kind, seed, n_docs) if seg_kind else None
    what = f"B={B} H={H} N={N} d={d} {dtype} window={window} prefix={prefix} seg={seg_kind} causal={causal}"
    _log(f"case {what}")
    seg_t = torch.from_numpy(seg).cuda() if seg is not None else None
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, window=window, prefix=prefix,
                        segment_ids=seg_t)
    torch.cuda.synchronize()
    wl, wr = window if window is not None else (-1, -1)
    o_ref, l_ref = oracle.attention_masked_f64(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                               float(np.float32(scale)), window_left=wl, window_right=wr,
                                               prefix=prefix, segment_ids=seg, causal=causal)
    do = np.abs(o.cpu().double().numpy() - o_ref)
    dl = np.abs(lse.cpu().double().numpy() - l_ref)
    _log(f"  max|dO|={do.max():.3e} max|dL|={dl.max():.3e}")
    assert np.all(np.isfinite(o.cpu().double().numpy()))
    assert do.max() <= TOL_O[dtype], (what, float(do.max()), np.unravel_index(np.argmax(do), do.shape))
    assert dl.max() <= TOL_L, (what, float(dl.max()), np.unravel_index(np.argmax(dl), dl.shape))


WINDOWS = [(0, 0), (5, 0), (63, 0), (64, 0), (100, 0), (17, 23), (-1, 40), (128, 128), (300, -1)]


@pytest.mark.parametrize("window", WINDOWS, ids=[f"w{a}_{b}" for a, b in WINDOWS])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["fp16", "bf16"])
def test_mask_sliding_window(dtype, d, window):
    _case(1, 2, 521, d, dtype, window=window, seed=1)


@pytest.mark.parametrize("prefix", [1, 7, 100, 255, 256, 300, 399])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_mask_prefix_causal(d, prefix):
    _case(1, 2, 400, d, torch.float16, prefix=prefix, causal=True, seed=2)


@pytest.mark.parametrize("seg_kind", ["documents", "interleaved"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_mask_segments(d, causal, seg_kind):
    _case(2, 2, 333, d, torch.bfloat16, seg_kind=seg_kind, causal=causal, seed=3)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_mask_combined(d):
    """Documents, a prefix and a left window at once."""
    _case(2, 2, 450, d, torch.float16, window=(90, 0), prefix=20, seg_kind="documents", seed=4)


@pytest.mark.parametrize("N", [1, 2, 65, 129])
def test_mask_small_and_ragged(N):
    _case(1, 1, N, 128, torch.float16, window=(3, 1), prefix=1, seed=5)
    _case(1, 1, N, 64, torch.bfloat16, seg_kind="interleaved", causal=True, seed=5)


def test_mask_bounds_that_cannot_bite():
    """Windows at least N - 1 wide and a prefix covering every key reduce to the
    unmasked (or causal) problem."""
    _case(1, 2, 200, 128, torch.float16, window=(199, 500), seed=6)
    _case(1, 2, 200, 128, torch.float16, prefix=200, causal=True, seed=6)
    _case(1, 2, 200, 64, torch.float16, window=(400, -1), causal=True, seed=6)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_mask_many_documents(d, causal):
    """Long sequences of many documents: each query tile visits only the key
    tiles of the documents its rows belong to (first with ids that increase
    along the sequence, then with runs whose ids repeat out of order)."""
    _case(2, 2, 1500, d, torch.float16, seg_kind="documents", causal=causal, seed=10, n_docs=12)
    _case(1, 2, 1500, d, torch.bfloat16, seg_kind="shuffled", causal=causal, seed=11, n_docs=12)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_mask_documents_with_window_and_prefix(d):
    """Documents under a causal sliding window plus a prefix: the key tiles come
    in two runs (prefix, then window) cut to the rows' documents."""
    _case(2, 2, 1800, d, torch.float16, window=(200, 0), prefix=70, seg_kind="documents", seed=12, n_docs=6)
    _case(1, 2, 1800, d, torch.float16, window=(150, 40), prefix=130, seg_kind="shuffled", seed=13, n_docs=8)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_mask_prefix_far_from_window(d):
    """A prefix and a window far apart: most key tiles between them are never
    visited."""
    _case(1, 2, 2500, d, torch.float16, window=(300, 0), prefix=100, seed=14)
    _case(1, 2, 2500, d, torch.bfloat16, window=(64, 64), prefix=1, seed=15)


def test_mask_long_sliding_window():
    """Many key tiles skipped on both sides of a window (d = 128, 2000 rows)."""
    _case(1, 2, 2000, 128, torch.bfloat16, window=(256, 64), seed=7)
    _case(1, 2, 2000, 128, torch.float16, window=(700, 0), seed=8)


def test_mask_matches_plain_causal_bitwise():
    """The masked entry with causal=True and no other bound takes the causal
    kernel: results equal fa2_fwd's bit for bit."""
    q, k, v = make_qkv(1, 2, 300, 128, torch.float16, "normal", 9)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    a = fa.forward(q, k, v, causal=True, scale=0.1)
    b = fa.forward(q, k, v, causal=True, scale=0.1, window=(-1, -1))
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_mask_argument_errors():
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float16, device="cuda")
    with pytest.raises(fa.Fa2Error):
        fa.forward(q, q, q, window=(-2, 0))
    with pytest.raises(fa.Fa2Error):
        fa.forward(q, q, q, prefix=-1)
    with pytest.raises(ValueError):
        fa.forward(q, q, q, segment_ids=torch.zeros(1, 8, dtype=torch.int64, device="cuda"))


@pytest.mark.parametrize("mask_name", ["window4096", "documents8"])
def test_mask_workload_full_size(mask_name):
    """The long-context causal workload (1 x 32 x 16384 x 128 fp16, inputs as
    the benchmark draws them) at full size under the two masks the benchmark
    times: a causal window of 4096 keys (the last head, whole, against the
    masked oracle) and 8 contiguous documents of 2048 rows (each document an
    independent causal sequence: the first and the last document of the first
    and the last head against the plain causal oracle); every output finite."""
    from exact_attention_11_amd.inputs import WORKLOADS, workload_inputs

    w = WORKLOADS["b1h32_n16384_d128_causal"]
    q, k, v = workload_inputs(w, seed=0)
    if mask_name == "window4096":
        kw = dict(window=(4096, -1))
    else:
        seg = np.repeat(np.arange(8, dtype=np.int32), w.N // 8)[None].repeat(w.B, 0)
        kw = dict(segment_ids=torch.from_numpy(np.ascontiguousarray(seg)).cuda())
    _log(f"workload b1h32_n16384_d128_causal under {mask_name}")
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=w.causal, scale=w.scale, **kw)
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    s32 = float(np.float32(w.scale))
    if mask_name == "window4096":
        sl = (slice(0, 1), slice(w.H - 1, w.H))
        refs = [(sl,) + tuple(oracle.attention_masked_f64(q[sl].double().numpy(), k[sl].double().numpy(),
                                                          v[sl].double().numpy(), s32, window_left=4096,
                                                          window_right=-1, causal=True))]
    else:
        n = w.N // 8
        refs = []
        for h in (0, w.H - 1):
            for doc in (0, 7):
                sl = (0, h, slice(n * doc, n * (doc + 1)))
                refs.append((sl,) + tuple(oracle.attention_f64(q[sl].double().numpy(), k[sl].double().numpy(),
                                                               v[sl].double().numpy(), True, s32)))
    for sl, o_ref, l_ref in refs:
        do = float(np.max(np.abs(o[sl] - o_ref)))
        dl = float(np.max(np.abs(lse[sl] - l_ref)))
        _log(f"  {mask_name} {sl}: max|dO|={do:.3e} max|dL|={dl:.3e}")
        assert do <= TOL_O[torch.float16] and dl <= TOL_L, (mask_name, sl, do, dl)
