"""GPU parity of decode (fa2_decode through the C ABI) against the fp64 decode
oracle (oracle/attention_decode_ref.c).

Tolerances as for the forward pass: max |dO| <= 2e-3 (fp16) / 1e-2 (bf16),
max |dL| <= 1e-3 over every element; rows with no visible key must give O = 0
and L = -inf exactly.  Short caches leave a row averaging a handful of values,
where |O| approaches |v| and rounding O to bf16 alone would cost up to 1.6e-2
for |v| in [4, 8): V is scaled by 1/4 (exact), which keeps |O| within the range
where the absolute tolerances apply.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_11_amd as fa
import oracle
from exact_attention_11_amd.inputs import decode_lengths, make_decode_inputs

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


def _check(o, lse, o_ref, l_ref, dtype, what):
    o = o.cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lse), empty), (what, "rows without a visible key differ")
    assert np.all(o[empty] == 0.0), (what, "O of a row without a visible key")
    assert np.all(np.isfinite(o)), (what, "non-finite O")
    do = np.abs(o - o_ref)
    dl = np.abs(np.where(empty, 0.0, lse - np.where(empty, 0.0, l_ref)))
    _log(f"  max|dO|={do.max():.3e} max|dL|={dl.max():.3e}")
    assert do.max() <= TOL_O[dtype], (what, float(do.max()), np.unravel_index(np.argmax(do), do.shape))
    assert dl.max() <= TOL_L, (what, float(dl.max()), np.unravel_index(np.argmax(dl), dl.shape))


def _case(B, H, Mq, Nk, d, dtype, causal, lens=None, seed=0, workspace=None):
    q, k, v = make_decode_inputs(B, H, Mq, Nk, d, dtype, seed)
    v = v * 0.25
    scale = 1.0 / math.sqrt(d)
    ws = fa.fa2_decode_workspace_bytes(B, H, Mq, Nk, d)
    what = (f"B={B} H={H} Mq={Mq} Nk={Nk} d={d} {dtype} causal={causal} lens={None if lens is None else list(lens)}"
            f" workspace={ws}")
    _log(f"case {what}")
    lens_t = None if lens is None else torch.tensor(lens, dtype=torch.int32).cuda()
    o, lse = fa.decode(q.cuda(), k.cuda(), v.cuda(), seqlens=lens_t, causal=causal, scale=scale,
                       workspace=workspace)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_decode_f64(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                               float(np.float32(scale)), seqlens=lens, causal=causal)
    _check(o, lse, o_ref, l_ref, dtype, what)
    return o, lse


@pytest.mark.parametrize("Mq", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["fp16", "bf16"])
def test_decode_one_chunk(dtype, d, causal, Mq):
    """Short caches: one workgroup per (batch, head) writes O and L itself."""
    _case(3, 2, Mq, 200, d, dtype, causal, lens=[200, 1, 77], seed=1)


@pytest.mark.parametrize("Mq", [1, 4, 8])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["fp16", "bf16"])
def test_decode_split_cache(dtype, d, causal, Mq):
    """Long caches of few heads: chunks merged through their logsumexp, some of
    them past a batch's length (empty)."""
    _case(2, 2, Mq, 5000, d, dtype, causal, lens=[5000, 1234], seed=2)


@pytest.mark.parametrize("Nk", [1, 63, 64, 65, 255, 256, 257, 1000, 4097])
def test_decode_ragged_capacities(Nk):
    _case(1, 3, 2, Nk, 128, torch.float16, True, lens=None, seed=3)
    _case(2, 1, 1, Nk, 64, torch.bfloat16, False, lens=[Nk, max(0, Nk // 3)], seed=4)


def test_decode_rows_without_visible_keys():
    """Length 0, and causal lengths shorter than the new rows."""
    _case(4, 2, 5, 300, 128, torch.float16, True, lens=[0, 1, 3, 300], seed=5)
    _case(3, 2, 3, 3000, 64, torch.float16, False, lens=[0, 2999, 0], seed=6)
    _case(1, 1, 1, 0, 64, torch.float16, False, lens=None, seed=7)


def test_decode_random_lengths():
    lens = decode_lengths(6, 2500, "ragged", seed=8).tolist()
    _case(6, 4, 1, 2500, 128, torch.bfloat16, True, lens=lens, seed=8)


def test_decode_dirty_workspace_and_bitwise_repeat():
    """The workspace's previous contents do not matter; results repeat bit for bit."""
    B, H, Mq, Nk, d = 1, 4, 2, 6000, 128
    need = fa.fa2_decode_workspace_bytes(B, H, Mq, Nk, d)
    assert need > 0
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda").view(torch.uint8)
    a = _case(B, H, Mq, Nk, d, torch.float16, True, lens=[4321], seed=9, workspace=ws)
    b = _case(B, H, Mq, Nk, d, torch.float16, True, lens=[4321], seed=9)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_matches_forward_last_rows():
    """Decode of the last rows of a causal sequence equals those rows of the
    GPU forward pass within the tolerances (two different kernels)."""
    from exact_attention_11_amd.inputs import make_qkv
    B, H, N, d, Mq = 1, 2, 700, 128, 4
    q, k, v = make_qkv(B, H, N, d, torch.float16, "normal", 10)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    o_f, l_f = fa.forward(q, k, v, causal=True)
    o_d, l_d = fa.decode(q[:, :, N - Mq:].contiguous(), k, v, causal=True)
    torch.cuda.synchronize()
    assert (o_f[:, :, N - Mq:].float() - o_d.float()).abs().max().item() <= 2 * TOL_O[torch.float16]
    assert (l_f[:, :, N - Mq:] - l_d).abs().max().item() <= 2 * TOL_L


def test_decode_full_size_workload_sampled():
    """The benchmark's decode workload (8 x 32 heads, one token, 16384-token
    cache, d = 128) in its launch configuration, checked on sampled heads."""
    from exact_attention_11_amd.inputs import DECODE_WORKLOADS, decode_workload_inputs
    for name in ("decode_b8h32_m1_n16384_d128", "decode_b8h32_m1_n16384_d128_ragged"):
        w = DECODE_WORKLOADS[name]
        q, k, v, lens = decode_workload_inputs(w, seed=0)
        _log(f"case {name} lens={lens.tolist()}")
        o, lse = fa.decode(q.cuda(), k.cuda(), v.cuda(), seqlens=lens.cuda(), causal=w.causal, scale=w.scale)
        torch.cuda.synchronize()
        for b, h in ((0, 0), (3, 17), (7, 31)):
            o_ref, l_ref = oracle.attention_decode_f64(q[b:b + 1, h:h + 1].double().numpy(),
                                                       k[b:b + 1, h:h + 1].double().numpy(),
                                                       v[b:b + 1, h:h + 1].double().numpy(),
                                                       float(np.float32(w.scale)), seqlens=[int(lens[b])],
                                                       causal=w.causal)
            _check(o[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], o_ref, l_ref, w.torch_dtype, f"{name} b={b} h={h}")


def test_decode_on_a_side_stream():
    """Decode launched on a stream other than the current one with the workspace
    allocated by decode() itself equals the same call on the current stream,
    while the current stream keeps allocating and writing."""
    B, H, Mq, Nk, d = 2, 4, 3, 6000, 128
    q, k, v = make_decode_inputs(B, H, Mq, Nk, d, torch.float16, 23)
    assert fa.fa2_decode_workspace_bytes(B, H, Mq, Nk, d) > 0
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    ref_o, ref_l = fa.decode(qc, kc, vc, causal=True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        outs.append(fa.decode(qc, kc, vc, causal=True, stream=s))
        junk = torch.full((fa.fa2_decode_workspace_bytes(B, H, Mq, Nk, d) // 4,), 3.0, device="cuda")
        del junk
    s.synchronize()
    for o, l in outs:
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
