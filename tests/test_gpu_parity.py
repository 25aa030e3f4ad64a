"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Tolerances: max |dO| <= 2e-3 for fp16 and <= 1e-2 for bf16, max |dL| <= 1e-3,
taken over every compared element.  Small problems (several tiles and a ragged
tail) are compared in full; the named workloads run at full size in the same
launch configuration the benchmark times and are compared on whole (batch,
head) slices plus sampled rows that the oracle computes one by one.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_11_amd as fa
import oracle
from exact_attention_11_amd.inputs import WORKLOADS, make_qkv, workload_inputs
from golden_io import exp_terms, matrix, read_kv, vector

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


def _gpu_run(q, k, v, causal, scale, stream=None):
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, stream=stream)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _f32(scale):
    return float(np.float32(scale))


def _compare(o, lse, o_ref, l_ref, dtype, what):
    do = np.abs(o.double().numpy() - o_ref)
    dl = np.abs(lse.double().numpy() - l_ref)
    eo, el = float(do.max()), float(dl.max())
    _log(f"  {what}: max|dO|={eo:.3e} (mean {do.mean():.2e}) max|dL|={el:.3e}")
    assert np.all(np.isfinite(o.double().numpy())) and np.all(np.isfinite(lse.double().numpy()))
    assert eo <= TOL_O[dtype], (what, eo, np.unravel_index(np.argmax(do), do.shape))
    assert el <= TOL_L, (what, el, np.unravel_index(np.argmax(dl), dl.shape))


def _full_parity(B, H, N, d, dtype, causal, scale=None, dist="normal", seed=0):
    q, k, v = make_qkv(B, H, N, d, dtype, dist, seed)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _log(f"case B={B} H={H} N={N} d={d} {dtype} causal={causal} scale={scale} dist={dist} seed={seed}")
    o, lse = _gpu_run(q, k, v, causal, scale)
    o_ref, l_ref = oracle.attention_f64(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal,
                                        _f32(scale))
    _compare(o, lse, o_ref, l_ref, dtype, "full")
    return q, k, v, o, lse


# --- small problems, compared in full ---------------------------------------------

@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 127, 128, 129, 200, 257, 383])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["fp16", "bf16"])
def test_parity_ragged_sweep(dtype, d, causal, N):
    _full_parity(1, 2, N, d, dtype, causal, seed=N)


def test_parity_tiny_workload():
    w = WORKLOADS["tiny_d64"]
    _full_parity(w.B, w.H, w.N, w.d, w.torch_dtype, w.causal, dist=w.dist)


@pytest.mark.parametrize("name", ["b8h16_n2048_d64", "b8h16_n2048_d128_causal", "b4h8_n4099_d256_peaky"])
def test_parity_workload_shapes_reduced_batch(name):
    """The named workloads at full sequence length with one (batch, head) pair
    per batch entry reduced to B=1, H=2, compared in full."""
    w = WORKLOADS[name]
    _full_parity(1, 2, w.N, w.d, w.torch_dtype, w.causal, dist=w.dist, seed=1)


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("scale", [0.0, -0.09, 1e-3, 0.5])
@pytest.mark.parametrize("causal", [False, True])
def test_parity_unusual_scales(scale, causal, d):
    """Multipliers 0 (uniform weights), negative, tiny and large.  V is scaled by
    1/4 (exact): at multiplier 0.5 and head dim 256 the scores have a standard
    deviation of 8, rows are close to one-hot and |O| would reach |v| (about 4),
    where the absolute tolerance no longer applies (the relative bound of
    test_lazy_reference_rounding_bound_unscaled_v covers such rows)."""
    q, k, v = make_qkv(1, 2, 300, d, torch.float16, "normal", 7)
    v = v * 0.25
    _log(f"case unusual scale {scale} d={d} causal={causal}")
    o, lse = _gpu_run(q, k, v, causal, scale)
    o_ref, l_ref = oracle.attention_f64(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal,
                                        _f32(scale))
    _compare(o, lse, o_ref, l_ref, torch.float16, "full")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["fp16", "bf16"])
def test_parity_far_max_growth(dtype, d):
    """Scores whose row max climbs tile after tile (keys sorted by score), which
    forces the running-max rescale on many tiles."""
    N = 700
    q, k, v = make_qkv(1, 1, N, d, dtype, "normal", 3)
    q = torch.zeros_like(q)
    q[..., 0] = 1.0
    k = torch.zeros_like(k)
    k[0, 0, :, 0] = torch.linspace(-30.0, 30.0, N).to(dtype)
    for causal in (False, True):
        _log(f"case max growth {dtype} d={d} causal={causal}")
        o, lse = _gpu_run(q, k, v, causal, 1.0)
        o_ref, l_ref = oracle.attention_f64(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal,
                                            1.0)
        _compare(o, lse, o_ref, l_ref, dtype, f"max growth causal={causal}")


@pytest.mark.parametrize("pattern", ["overflow_jump", "finite_jump", "plateau", "late_dip"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["fp16", "bf16"])
def test_parity_reference_moves(dtype, d, pattern):
    """Score layouts aimed at each way a key tile can meet the row's reference
    max: a later score so far above it that its weight overflows fp32
    (overflow_jump), one far above it but finite (finite_jump), a whole tile of
    scores just under the rescale threshold, whose weights add up past any
    small bound while none is large (plateau), and tiles far below the first
    one (late_dip).  Every row sees the same scores (q = e0, scale 1), so the
    layout is exact for all rows; the causal runs cut it at each row.

    V is scaled by 1/4 (exact) so that |O| stays near 1, where the absolute
    tolerances apply: a single dominant weight can sit anywhere in (1, 2^8] and
    keeps its rounding to the input type (2^-8 relative in bf16), so the error
    of O grows with |v| on such rows."""
    N = 320
    q, k, v = make_qkv(1, 1, N, d, dtype, "normal", 11)
    v = v * 0.25
    q = torch.zeros_like(q)
    q[..., 0] = 1.0
    k = torch.zeros_like(k)
    sc = torch.zeros(N)
    if pattern == "overflow_jump":
        sc[100] = 120.0      # 2^(120 log2 e) overflows fp32
        sc[250] = 240.0
    elif pattern == "finite_jump":
        sc[70] = 40.0
        sc[200] = 60.0
        sc[201] = 61.0
    elif pattern == "plateau":
        sc[64:192] = 5.0     # 7.2 log2 units over the first tile's max
        sc[250:] = 10.0
    else:
        sc[:64] = 20.0
        sc[64:] = -20.0
    k[0, 0, :, 0] = sc.to(dtype)
    for causal in (False, True):
        _log(f"case reference moves {pattern} {dtype} d={d} causal={causal}")
        o, lse = _gpu_run(q, k, v, causal, 1.0)
        o_ref, l_ref = oracle.attention_f64(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal,
                                            1.0)
        _compare(o, lse, o_ref, l_ref, dtype, f"{pattern} causal={causal}")


@pytest.mark.parametrize("pattern", ["peaky", "overflow_jump", "plateau"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["fp16", "bf16"])
def test_lazy_reference_rounding_bound_unscaled_v(dtype, d, pattern):
    """Values as large as they come (V ~ 4 N(0, 1), not scaled down), on rows
    where a few keys carry most of the weight.  The weights are formed against a
    reference max that may lag the row max by up to 2^8, rounded to the input
    type (unit roundoff u = 2^-11 fp16, 2^-8 bf16) for P.V, and divided by a row
    sum of the unrounded weights; O is rounded once at the end.  So every
    element obeys |O - O_ref| <= u (A + |O_ref|) + 2 e A, where A = sum_c p_c |v_c|
    is the oracle's output for |V| and e bounds the relative error of a weight
    from fp32 arithmetic: the score sum in fp32 (at most (n - 1) 2^-24 |scale|
    sum_t |q_t k_t| in the exponent for n nonzero products; none for the
    constructed patterns, whose scores have one nonzero product), the fp32
    multiplier scale * log2(e) and the fused multiply-add that applies it (2 u
    |scale s| more), and a few fp32 ulps for the exponential.  The bound is relative: it holds at any |v|, where the
    absolute tolerances of the other tests assume |O| near 1."""
    N = 333
    u = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}[dtype]
    q, k, v = make_qkv(1, 2, N, d, dtype, "peaky", 31)
    v = (torch.randn(v.shape, generator=torch.Generator().manual_seed(32)) * 4.0).to(dtype)
    scale = 1.0 / math.sqrt(d)
    if pattern != "peaky":
        q = torch.zeros_like(q)
        q[..., 0] = 1.0
        k = torch.zeros_like(k)
        sc = torch.zeros(N)
        if pattern == "overflow_jump":
            sc[100], sc[250] = 120.0, 240.0
        else:
            sc[64:192], sc[250:] = 5.0, 10.0
        k[:, :, :, 0] = sc.to(dtype)
        scale = 1.0
    for causal in (False, True):
        _log(f"case lazy reference bound {pattern} {dtype} d={d} causal={causal} max|v|={float(v.float().abs().max()):.2f}")
        o, lse = _gpu_run(q, k, v, causal, scale)
        qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
        o_ref, l_ref = oracle.attention_f64(qd, kd, vd, causal, _f32(scale))
        a_ref, _ = oracle.attention_f64(qd, kd, np.abs(vd), causal, _f32(scale))
        err = np.abs(o.double().numpy() - o_ref)
        kt = kd.transpose(0, 1, 3, 2)
        dots = np.abs(qd) @ np.abs(kt)                                   # sum_t |q_t k_t| per (row, key)
        adds = np.maximum((qd != 0).astype(np.float64) @ (kt != 0).astype(np.float64) - 1.0, 0.0)
        e_w = 2.0 ** -24 * abs(_f32(scale)) * ((adds + 2.0) * dots).max(axis=-1) + 2.0 ** -21
        bound = u * (a_ref + np.abs(o_ref)) + 2.0 * e_w[..., None] * a_ref + 1e-6
        ratio = float(np.max(err / bound))
        _log(f"  max|dO|={float(err.max()):.3e} worst err/bound={ratio:.3f} max|dL|="
             f"{float(np.max(np.abs(lse.double().numpy() - l_ref))):.3e}")
        assert ratio <= 1.0, (ratio, np.unravel_index(np.argmax(err / bound), err.shape))
        assert float(np.max(np.abs(lse.double().numpy() - l_ref))) <= TOL_L


@pytest.mark.parametrize("B,H,N,d", [(1, 24, 4000, 64), (2, 8, 600, 128), (1, 16, 2500, 128), (2, 8, 1100, 256)])
def test_parity_causal_head_groups(B, H, N, d):
    """Causal launches whose head count is a multiple of 8 order their query
    tiles in groups of heads per XCD, a smaller last group included (24 heads
    of 16 query tiles: each XCD takes 3 heads, as a group of 2 and then 1);
    every (batch, head, query tile) must still be computed exactly once."""
    _full_parity(B, H, N, d, torch.float16, True, seed=5)


# --- named workloads at full size ------------------------------------------------------

def _sample_rows(N, rng, n_random=40):
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, N // 2, N - 129, N - 128, N - 65, N - 64, N - 2, N - 1]
    rows = set(r for r in fixed if 0 <= r < N)
    rows.update(int(x) for x in rng.integers(0, N, size=n_random))
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("name", [n for n in WORKLOADS if n != "tiny_d64"])
def test_parity_workload_full_size(name):
    """Full-size workload in the benchmark's launch configuration: the first and
    the last (batch, head) slices are compared on every row, two more slices on
    sampled rows the oracle computes one by one."""
    w = WORKLOADS[name]
    q, k, v = workload_inputs(w, seed=0)
    _log(f"workload {name}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} causal={w.causal}")
    o, lse = _gpu_run(q, k, v, w.causal, w.scale)
    for (b, h) in [(0, 0), (w.B - 1, w.H - 1)]:
        o_ref, l_ref = oracle.attention_f64(q[b, h].double().numpy(), k[b, h].double().numpy(),
                                            v[b, h].double().numpy(), w.causal, _f32(w.scale))
        _compare(o[b, h], lse[b, h], o_ref, l_ref, w.torch_dtype, f"(b={b},h={h}) all {w.N} rows")
    rng = np.random.default_rng(0)
    for _ in range(2):
        b, h = int(rng.integers(w.B)), int(rng.integers(w.H))
        rows = _sample_rows(w.N, rng)
        o_ref, l_ref = oracle.attention_rows_f64(q[b, h].double().numpy(), k[b, h].double().numpy(),
                                                 v[b, h].double().numpy(), rows, w.causal, _f32(w.scale))
        _compare(o[b, h, rows], lse[b, h, rows], o_ref, l_ref, w.torch_dtype, f"(b={b},h={h}) {len(rows)} rows")
    # properties that hold at any size, over every row
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    assert float(o.float().abs().max()) <= float(v.float().abs().max()) * (1 + 1e-2)
    # every query tile of every (batch, head): two rows of each 128-row block (a
    # workgroup covers one or two such blocks), one from each half, and the
    # last row, so that every workgroup of the launch is compared
    worst_o, worst_l, n_rows = 0.0, 0.0, 0
    for b in range(w.B):
        for h in range(w.H):
            rows = _rows_per_block(w.N, rng)
            o_ref, l_ref = oracle.attention_rows_f64(q[b, h].double().numpy(), k[b, h].double().numpy(),
                                                     v[b, h].double().numpy(), rows, w.causal, _f32(w.scale))
            eo = float(np.max(np.abs(o[b, h, rows].double().numpy() - o_ref)))
            el = float(np.max(np.abs(lse[b, h, rows].double().numpy() - l_ref)))
            assert eo <= TOL_O[w.torch_dtype] and el <= TOL_L, ((b, h), eo, el)
            worst_o, worst_l, n_rows = max(worst_o, eo), max(worst_l, el), n_rows + len(rows)
    _log(f"  every query tile, {n_rows} rows over {w.B * w.H} heads: max|dO|={worst_o:.3e} max|dL|={worst_l:.3e}")


def _rows_per_block(N, rng, block=128):
    """Two rows of every block of ``block`` query rows (one in each half,
    clipped to N) and the last row."""
    rows = set()
    for t in range(0, N, block):
        half = block // 2
        rows.add(min(N - 1, t + int(rng.integers(half))))
        rows.add(min(N - 1, t + half + int(rng.integers(half))))
    rows.add(N - 1)
    return np.array(sorted(rows), dtype=np.int64)


# --- the pages' worked examples, embedded at d = 64 ------------------------------------

def _embed(mat, d=64):
    out = np.zeros((mat.shape[0], d))
    out[:, :mat.shape[1]] = mat
    return torch.from_numpy(out)[None, None]


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["fp16", "bf16"])
def test_lesson_practice_row(dtype):
    g = read_kv("lesson_practice_online_softmax.txt")
    s, vals = vector(g["scores"]), vector(g["values"])
    n = len(s)
    q = _embed(np.ones((n, 1))).to(dtype)
    k = _embed(s[:, None]).to(dtype)
    v = _embed(vals[:, None] / 64.0).to(dtype)  # exact power-of-two scaling keeps |O| <= 1
    o, lse = _gpu_run(q, k, v, False, 1.0)
    final = float(g["final"]) / 64.0
    assert np.max(np.abs(o[0, 0, :, 0].double().numpy() - final)) <= TOL_O[dtype]
    assert np.max(np.abs(o[0, 0, :, 1:].double().numpy())) == 0.0
    m_last, l_last = float(g["_steps"][-1][1]), float(g["_steps"][-1][3])
    assert np.max(np.abs(lse[0, 0].double().numpy() - (m_last + math.log(l_last)))) <= TOL_L
    o, lse = _gpu_run(q, k, v, True, 1.0)
    for st in g["_steps"]:
        r = 2 * int(st[0]) + 1
        assert abs(float(o[0, 0, r, 0]) - float(st[4]) / 64.0) <= TOL_O[dtype]
        assert abs(float(lse[0, 0, r]) - (float(st[1]) + math.log(float(st[3])))) <= TOL_L
    assert float(o[0, 0, 0, 0]) == float(v[0, 0, 0, 0])


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["fp16", "bf16"])
def test_fa2_page_worked_example(dtype):
    g = read_kv("fa2_page_worked_example.txt")
    Q, K, V = matrix(g["Q"]), matrix(g["KT"]).T, matrix(g["V"])
    q, k, v = _embed(Q).to(dtype), _embed(K).to(dtype), _embed(V / 8.0).to(dtype)
    o, lse = _gpu_run(q, k, v, False, 1.0)
    l = np.array([exp_terms(g["l_row0_terms"]), exp_terms(g["l_row1_terms"])])
    acc = np.array([[exp_terms(g["acc_r0c0_terms"]), exp_terms(g["acc_r0c1_terms"])],
                    [exp_terms(g["acc_r1c0_terms"]), exp_terms(g["acc_r1c1_terms"])]])
    want_o = acc / l[:, None] / 8.0
    want_l = vector(g["m_step3"]) + np.log(l)
    assert np.max(np.abs(o[0, 0, :2, :2].double().numpy() - want_o)) <= TOL_O[dtype]
    assert np.max(np.abs(lse[0, 0, :2].double().numpy() - want_l)) <= TOL_L
    o_ref, l_ref = oracle.attention_f64(q.double().numpy(), k.double().numpy(), v.double().numpy(), False, 1.0)
    _compare(o, lse, o_ref, l_ref, dtype, "worked example all rows")


def test_closed_form_4x4():
    Q = np.zeros((4, 64))
    Q[:, :4] = np.eye(4)
    V = np.zeros((4, 64))
    V[:, :4] = np.arange(1, 17, dtype=np.float64).reshape(4, 4) / 16.0
    q = torch.from_numpy(Q)[None, None].half()
    v = torch.from_numpy(V)[None, None].half()
    e = math.e
    o, lse = _gpu_run(q, q, v, False, 1.0)
    for r in range(4):
        want = (e * V[r] + V.sum(axis=0) - V[r]) / (e + 3)
        assert np.max(np.abs(o[0, 0, r].double().numpy() - want)) <= 2e-3
        assert abs(float(lse[0, 0, r]) - math.log(e + 3)) <= TOL_L
    o, lse = _gpu_run(q, q, v, True, 1.0)
    for r in range(4):
        want = (e * V[r] + V[:r].sum(axis=0)) / (e + r)
        assert np.max(np.abs(o[0, 0, r].double().numpy() - want)) <= 2e-3
        assert abs(float(lse[0, 0, r]) - math.log(e + r)) <= TOL_L


# --- invariants and execution properties ---------------------------------------------

def test_identical_value_rows_and_row_sums():
    q, k, _ = make_qkv(2, 3, 333, 128, torch.float16, "normal", 5)
    v = torch.zeros_like(q)
    v[..., 0] = 1.0                                        # weights sum to one
    v[..., 1:] = torch.randn(128 - 1, generator=torch.Generator().manual_seed(1)).half()  # same row everywhere
    for causal in (False, True):
        o, _ = _gpu_run(q, k, v, causal, 1.0 / math.sqrt(128))
        assert float((o.float() - v.float()).abs().max()) <= 2e-3


def test_key_permutation_invariance():
    q, k, v = make_qkv(1, 2, 517, 64, torch.float16, "normal", 6)
    o, lse = _gpu_run(q, k, v, False, 0.125)
    perm = torch.randperm(517, generator=torch.Generator().manual_seed(2))
    o2, lse2 = _gpu_run(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), False, 0.125)
    assert float((o.float() - o2.float()).abs().max()) <= 2e-3
    assert float((lse - lse2).abs().max()) <= TOL_L


def test_causal_future_independence_bitwise():
    q, k, v = make_qkv(1, 2, 400, 128, torch.bfloat16, "normal", 8)
    o, lse = _gpu_run(q, k, v, True, 0.088)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, 150:] = -k2[:, :, 150:] * 3
    v2[:, :, 150:] = v2[:, :, 150:] * -2
    o2, lse2 = _gpu_run(q, k2, v2, True, 0.088)
    assert torch.equal(o[:, :, :150], o2[:, :, :150])
    assert torch.equal(lse[:, :, :150], lse2[:, :, :150])
    assert not torch.equal(o[:, :, 150:], o2[:, :, 150:])


def test_causal_row0_is_v0():
    q, k, v = make_qkv(2, 2, 260, 256, torch.float16, "normal", 9)
    o, lse = _gpu_run(q, k, v, True, 0.0625)
    assert torch.equal(o[:, :, 0], v[:, :, 0])
    want = 0.0625 * (q[:, :, 0].double() * k[:, :, 0].double()).sum(-1)
    assert float((lse[:, :, 0].double() - want).abs().max()) <= TOL_L


def test_batch_head_slices_are_independent_bitwise():
    q, k, v = make_qkv(2, 3, 190, 64, torch.bfloat16, "normal", 10)
    o, lse = _gpu_run(q, k, v, True, 0.125)
    for b in range(2):
        for h in range(3):
            sl = (slice(b, b + 1), slice(h, h + 1))
            o1, l1 = _gpu_run(q[sl].contiguous(), k[sl].contiguous(), v[sl].contiguous(), True, 0.125)
            assert torch.equal(o1, o[sl]) and torch.equal(l1, lse[sl])


def test_deterministic_bitwise():
    w = WORKLOADS["b8h16_n2048_d128_causal"]
    q, k, v = (t.cuda() for t in workload_inputs(w, seed=4))
    o1, l1 = fa.forward(q, k, v, causal=True)
    o2, l2 = fa.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_non_default_stream():
    q, k, v = (t.cuda() for t in make_qkv(2, 4, 1000, 128, torch.float16, "normal", 11))
    ref_o, ref_l = fa.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        q2 = q * 1  # produced on the side stream
        o, lse = fa.forward(q2, k, v, causal=True)
    s.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)


def test_preallocated_outputs_and_empty_problem():
    q, k, v = (t.cuda() for t in make_qkv(1, 1, 70, 64, torch.float16, "normal", 12))
    out = torch.full_like(q, float("nan"))
    lse = torch.full((1, 1, 70), float("nan"), device="cuda")
    fa.forward(q, k, v, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    e = torch.empty(0, 2, 5, 64, dtype=torch.float16, device="cuda")
    o, l = fa.forward(e, e, e)
    assert o.shape == e.shape and l.shape == (0, 2, 5)
