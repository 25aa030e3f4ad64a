"""fa2_decode_static, the decode entry point that allocates nothing, against
fa2_decode with a caller-owned workspace: same kernels, so the results must be
identical, and both within the oracle's tolerances.  Two calls in a row, the
second with a smaller problem, so the second runs on scratch the first has
left its partials in."""
import numpy as np
import pytest
import torch

import exact_attention_11_amd as fa
import oracle
from exact_attention_11_amd.inputs import decode_lengths, make_decode_inputs

pytestmark = pytest.mark.gpu

TOL_O = {torch.float16: 2e-3, torch.bfloat16: 1e-2}
TOL_L = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()


def _run_both(B, H, Mq, Nk, d, dtype, causal, lengths, seed):
    print(f"case static decode B={B} H={H} Mq={Mq} Nk={Nk} d={d} {dtype} causal={causal} lengths={lengths}",
          flush=True)
    need = fa.fa2_decode_workspace_bytes(B, H, Mq, Nk, d)
    assert 0 < need <= fa.DECODE_STATIC_SCRATCH_BYTES  # the case really uses the scratch
    q, k, v = make_decode_inputs(B, H, Mq, Nk, d, dtype, seed)
    lens = decode_lengths(B, Nk, lengths, seed)
    dq, dk, dv, dl = q.cuda(), k.cuda(), v.cuda(), lens.cuda()
    scale = float(np.float32(d ** -0.5))
    code = fa.FA2_DTYPE_FP16 if dtype == torch.float16 else fa.FA2_DTYPE_BF16
    stream = torch.cuda.current_stream().cuda_stream
    # fa2_decode with its own workspace, through the C ABI
    o_ws = torch.full_like(dq, float("nan"))
    l_ws = torch.full((B, H, Mq), float("nan"), device="cuda")
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    rc = fa.fa2_decode(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dl.data_ptr(), o_ws.data_ptr(), l_ws.data_ptr(),
                       B, H, Mq, Nk, d, int(causal), scale, code, ws.data_ptr(), need, stream)
    assert rc == fa.FA2_OK, fa.fa2_status_str(rc)
    # fa2_decode_static, through the C ABI, into outputs allocated beforehand
    o_st = torch.full_like(dq, float("nan"))
    l_st = torch.full((B, H, Mq), float("nan"), device="cuda")
    torch.cuda.synchronize()
    rc = fa.fa2_decode_static(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dl.data_ptr(), o_st.data_ptr(),
                              l_st.data_ptr(), B, H, Mq, Nk, d, int(causal), scale, code, stream)
    assert rc == fa.FA2_OK, fa.fa2_status_str(rc)
    torch.cuda.synchronize()
    assert torch.equal(o_st, o_ws), float((o_st.float() - o_ws.float()).abs().max())
    assert torch.equal(l_st, l_ws)
    o_ref, l_ref = oracle.attention_decode_f64(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale,
                                               seqlens=lens.tolist(), causal=causal)
    eo = float(np.max(np.abs(o_st.cpu().double().numpy() - o_ref)))
    el = float(np.max(np.abs(l_st.cpu().double().numpy() - l_ref)))
    print(f"  max|dO|={eo:.3e} max|dL|={el:.3e}", flush=True)
    assert eo <= TOL_O[dtype] and el <= TOL_L, (eo, el)


def test_static_decode_matches_workspace_decode_twice():
    _run_both(2, 4, 4, 5000, 128, torch.float16, True, "ragged", 1)
    _run_both(1, 2, 2, 1500, 64, torch.bfloat16, False, "full", 2)


def test_static_decode_rejects_problems_beyond_its_scratch():
    # 8 rows of head dim 256 for 64 heads split into 8 chunks: 4.2 MB of partials
    B, H, Mq, Nk, d = 1, 64, 8, 16384, 256
    assert fa.fa2_decode_workspace_bytes(B, H, Mq, Nk, d) > fa.DECODE_STATIC_SCRATCH_BYTES
    q = torch.zeros((B, H, Mq, d), dtype=torch.float16, device="cuda")
    kv = torch.zeros((B, H, Nk, d), dtype=torch.float16, device="cuda")
    with pytest.raises(fa.Fa2Error) as e:
        fa.decode_static(q, kv, kv)
    assert e.value.status == fa.FA2_ERR_SCRATCH
