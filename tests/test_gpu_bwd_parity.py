"""GPU parity of the gradients: fa2_bwd through the C ABI against the fp64
gradient oracle (oracle/attention_bwd_ref.c), on the GPU forward pass's own O
and L (the way the two calls are used together).

Tolerance (relative to the largest magnitude of each reference gradient, plus a
small absolute floor): the GPU rounds P and dS to the input type before their
products (unit roundoff u = 2^-11 fp16, 2^-8 bf16), reads O rounded to the input
type for D and rounds the outputs once; each of those contributes at most about
u * max|gradient| to an element, so the bound is 4u relative.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_11_amd as fa
import oracle
from exact_attention_11_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu

UNIT = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}
REL = 4.0


def _log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()


def _dout(shape, dtype, seed):
    g = torch.Generator().manual_seed(1000 + seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype)


def _run(q, k, v, do, causal, scale):
    qc, kc, vc, gc = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.forward(qc, kc, vc, causal=causal, scale=scale)
    delta = torch.empty_like(lse)
    dq, dk, dv = fa.backward(qc, kc, vc, o, gc, lse, causal=causal, scale=scale, delta=delta)
    torch.cuda.synchronize()
    return o.cpu(), dq.cpu(), dk.cpu(), dv.cpu(), delta.cpu()


def _check(name, got, ref, dtype, what):
    got = got.double().numpy()
    assert np.all(np.isfinite(got)), (what, name, "non-finite")
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    tol = REL * UNIT[dtype] * scale + 1e-6
    _log(f"  {what} {name}: max|d|={err:.3e} max|ref|={scale:.3e} rel={err / max(scale, 1e-30):.2e} tol={tol:.2e}")
    assert err <= tol, (what, name, err, tol)


def _parity(B, H, N, d, dtype, causal, scale=None, seed=0, dist="normal"):
    q, k, v = make_qkv(B, H, N, d, dtype, dist, seed)
    do = _dout((B, H, N, d), dtype, seed)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    what = f"B={B} H={H} N={N} d={d} {dtype} causal={causal} scale={scale}"
    _log(f"case {what}")
    o, dq, dk, dv, delta = _run(q, k, v, do, causal, scale)
    s32 = float(np.float32(scale))
    rq, rk, rv, _ = oracle.attention_bwd_f64(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                             do.double().numpy(), causal, s32)
    _check("dQ", dq, rq, dtype, what)
    _check("dK", dk, rk, dtype, what)
    _check("dV", dv, rv, dtype, what)
    # D is the row sum of dO o O over the GPU's own O, accumulated in fp32.
    want = (do.double() * o.double()).sum(-1).numpy()
    err = float(np.max(np.abs(delta.double().numpy() - want)))
    assert err <= 1e-5 * max(1.0, float(np.max(np.abs(want)))), (what, "D", err)


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 127, 128, 129, 200, 257])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["fp16", "bf16"])
def test_bwd_parity_ragged_sweep(dtype, d, causal, N):
    _parity(1, 2, N, d, dtype, causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["fp16", "bf16"])
def test_bwd_parity_medium(dtype, d, causal):
    """700 rows: several key and query workgroups and streamed tiles per head,
    ending in a ragged one."""
    _parity(2, 3, 700, d, dtype, causal, seed=4)


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.5])
def test_bwd_parity_unusual_scales(scale):
    _parity(1, 2, 300, 64, torch.float16, True, scale=scale, seed=6)


def test_bwd_zero_scale_closed_form():
    """Multiplier 0: dQ and dK vanish exactly."""
    q, k, v = make_qkv(1, 1, 130, 64, torch.float16, "normal", 2)
    do = _dout(q.shape, torch.float16, 2)
    _, dq, dk, _, _ = _run(q, k, v, do, True, 0.0)
    assert torch.all(dq == 0) and torch.all(dk == 0)


def test_bwd_deterministic_bitwise():
    q, k, v = make_qkv(2, 2, 333, 128, torch.bfloat16, "normal", 3)
    do = _dout(q.shape, torch.bfloat16, 3)
    a = _run(q, k, v, do, True, 0.1)
    b = _run(q, k, v, do, True, 0.1)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_rejects_host_delta_before_launch():
    """A delta on the host (or another device) with device q, k, v is refused in
    Python, before fa2_bwd could write through a host address."""
    q, k, v = (t.cuda() for t in make_qkv(1, 2, 130, 64, torch.float16, "normal", 21))
    o, lse = fa.forward(q, k, v, causal=True)
    do = torch.randn_like(q)
    with pytest.raises(ValueError):
        fa.backward(q, k, v, o, do, lse, causal=True, delta=torch.empty(lse.shape, dtype=torch.float32))
    torch.cuda.synchronize()


def test_bwd_on_a_side_stream():
    """Gradients launched on a stream other than the current one, with delta
    allocated by backward() itself, equal the same call on the current stream
    while the current stream keeps allocating (the dropped delta must not be
    reused before the side stream's kernels finish)."""
    q, k, v = make_qkv(2, 4, 1000, 128, torch.bfloat16, "normal", 22)
    do = _dout(q.shape, torch.bfloat16, 22)
    qc, kc, vc, gc = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.forward(qc, kc, vc, causal=True)
    ref = fa.backward(qc, kc, vc, o, gc, lse, causal=True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        got = fa.backward(qc, kc, vc, o, gc, lse, causal=True, stream=s)
        # work on the current stream that would reuse a freed delta block
        junk = torch.full((2, 4, 1000), 7.0, device="cuda")
        outs.append(got)
        del junk
    s.synchronize()
    for got in outs:
        for a, b in zip(got, ref):
            assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["b8h16_n2048_d64", "b8h16_n2048_d128_causal", "b4h8_n4099_d256_peaky",
                                  "b1h32_n16384_d128_causal"])
def test_bwd_parity_workload_full_size(name):
    """A named workload at its full size, in the launch configuration that
    bench.py's gradient pass times: whole (batch, head) slices against the
    gradient oracle (the first and the last slice; the last only at 16384
    rows, where one slice costs the oracle about half a minute), and every
    output finite."""
    from exact_attention_11_amd.inputs import WORKLOADS, workload_inputs

    w = WORKLOADS[name]
    dtype = w.torch_dtype
    q, k, v = workload_inputs(w, seed=0)
    do = _dout(q.shape, dtype, 0)
    _log(f"workload {name}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} causal={w.causal}")
    o, dq, dk, dv, delta = _run(q, k, v, do, w.causal, w.scale)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all(), name
    s32 = float(np.float32(w.scale))
    slices = [(w.B - 1, w.H - 1)] if w.N > 8192 else [(0, 0), (w.B - 1, w.H - 1)]
    for (b, h) in slices:
        rq, rk, rv, _ = oracle.attention_bwd_f64(q[b, h].double().numpy(), k[b, h].double().numpy(),
                                                 v[b, h].double().numpy(), do[b, h].double().numpy(), w.causal, s32)
        what = f"{name} (b={b},h={h})"
        _check("dQ", dq[b, h], rq, dtype, what)
        _check("dK", dk[b, h], rk, dtype, what)
        _check("dV", dv[b, h], rv, dtype, what)
    want = (do.double() * o.double()).sum(-1).numpy()
    err = float(np.max(np.abs(delta.double().numpy() - want)))
    assert err <= 1e-5 * max(1.0, float(np.max(np.abs(want)))), (name, "D", err)


@pytest.mark.parametrize("causal,dtype", [(False, torch.bfloat16), (True, torch.float16)], ids=["bf16", "fp16-causal"])
def test_bwd_parity_long_d128(causal, dtype):
    """Head dim 128 on a long sequence with a ragged last tile (8195 rows =
    64 * 128 + 3): 65 key and query workgroups per head."""
    _parity(1, 1, 8195, 128, dtype, causal, seed=4)
