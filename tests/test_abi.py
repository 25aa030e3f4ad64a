"""The C ABI library: it loads, exports every symbol include/fa2.h declares, and
its argument checks return their codes without touching a device (CPU only)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import exact_attention_11_amd as fa
from exact_attention_11_amd import build as hip_build

HEADER = os.path.join(hip_build.INCLUDE, "fa2.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        hip_build.build()
    return fa.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa2_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_symbols():
    assert _declared_functions() == sorted(fa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings(lib):
    for code in range(0, 13):
        s = fa.fa2_status_str(code)
        assert s and s != "unknown status"
    assert fa.fa2_status_str(123) == "unknown status"
    assert fa.fa2_status_str(-1) == "unknown status"


# Fake but aligned, distinct, non-overlapping addresses: every call below must be
# rejected by the host-side checks before any HIP call is made.
Q, K, V, O, L = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def _call(B=1, H=1, N=16, d=64, causal=0, scale=0.125, dtype=0, q=Q, k=K, v=V, o=O, lse=L):
    return fa.fa2_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(B=-1), fa.FA2_ERR_SHAPE), (dict(H=-2), fa.FA2_ERR_SHAPE), (dict(N=-1), fa.FA2_ERR_SHAPE),
    (dict(N=2 ** 31), fa.FA2_ERR_SHAPE), (dict(B=2 ** 20, H=2 ** 20, N=1024), fa.FA2_ERR_SHAPE),
    (dict(d=32), fa.FA2_ERR_HEADDIM), (dict(d=96), fa.FA2_ERR_HEADDIM), (dict(d=512), fa.FA2_ERR_HEADDIM),
    (dict(dtype=2), fa.FA2_ERR_DTYPE), (dict(dtype=-1), fa.FA2_ERR_DTYPE),
    (dict(scale=math.nan), fa.FA2_ERR_SCALE), (dict(scale=math.inf), fa.FA2_ERR_SCALE),
    (dict(scale=-math.inf), fa.FA2_ERR_SCALE), (dict(scale=3.0e38), fa.FA2_ERR_SCALE),
    (dict(q=0), fa.FA2_ERR_NULLPTR), (dict(k=0), fa.FA2_ERR_NULLPTR), (dict(v=0), fa.FA2_ERR_NULLPTR),
    (dict(o=0), fa.FA2_ERR_NULLPTR), (dict(lse=0), fa.FA2_ERR_NULLPTR),
    (dict(q=Q + 8), fa.FA2_ERR_ALIGN), (dict(o=O + 2), fa.FA2_ERR_ALIGN), (dict(lse=L + 4), fa.FA2_ERR_ALIGN),
    (dict(o=Q), fa.FA2_ERR_ALIAS), (dict(o=K + 1024), fa.FA2_ERR_ALIAS), (dict(lse=V + 16), fa.FA2_ERR_ALIAS),
    (dict(lse=O + 512), fa.FA2_ERR_ALIAS),
])
def test_argument_checks(lib, kwargs, code):
    assert _call(**kwargs) == code


@pytest.mark.parametrize("kwargs", [dict(B=0), dict(H=0), dict(N=0), dict(B=0, q=0, k=0, v=0, o=0, lse=0)])
def test_empty_problem_is_a_no_op(lib, kwargs):
    assert _call(**kwargs) == fa.FA2_OK


def test_inputs_may_alias_each_other_when_no_device(lib):
    # q, k, v may share memory (they are only read); with no GPU the call gets
    # past every argument check and stops at the device check.
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this call would launch on fake pointers")
    assert _call(q=Q, k=Q, v=Q) == fa.FA2_ERR_DEVICE


def test_valid_call_without_device_reports_device_error(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this call would launch on fake pointers")
    for d in (64, 128, 256):
        for dtype in (0, 1):
            assert _call(d=d, dtype=dtype, causal=1, N=4099) == fa.FA2_ERR_DEVICE
    assert fa.fa2_last_hip_error() != 0


def test_single_hip_runtime_in_process(lib):
    import torch  # noqa: F401
    maps = open("/proc/self/maps").read()
    paths = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(paths) == 1, paths


def test_python_forward_rejects_bad_tensors(lib):
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)  # host tensors
    with pytest.raises(ValueError):
        fa.forward(q, q, q[:, :, :4])
    with pytest.raises(TypeError):
        fa.forward(q.float(), q.float(), q.float())


# --- fa2_bwd ----------------------------------------------------------------------

DO, DL, DQ, DK, DV = 0x60000000, 0x70000000, 0x80000000, 0x90000000, 0xA0000000


def _bwd(B=1, H=1, N=16, d=64, causal=0, scale=0.125, dtype=0, q=Q, k=K, v=V, o=O, dout=DO, lse=L,
         delta=DL, dq=DQ, dk=DK, dv=DV):
    return fa.fa2_bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, N, d, causal, scale, dtype, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(B=-1), fa.FA2_ERR_SHAPE), (dict(N=-3), fa.FA2_ERR_SHAPE), (dict(N=2 ** 31), fa.FA2_ERR_SHAPE),
    (dict(B=2 ** 20, H=2 ** 20, N=1024), fa.FA2_ERR_SHAPE),
    (dict(d=32), fa.FA2_ERR_HEADDIM), (dict(d=512), fa.FA2_ERR_HEADDIM),
    (dict(dtype=3), fa.FA2_ERR_DTYPE),
    (dict(scale=math.nan), fa.FA2_ERR_SCALE), (dict(scale=3.0e38), fa.FA2_ERR_SCALE),
    (dict(q=0), fa.FA2_ERR_NULLPTR), (dict(o=0), fa.FA2_ERR_NULLPTR), (dict(dout=0), fa.FA2_ERR_NULLPTR),
    (dict(lse=0), fa.FA2_ERR_NULLPTR), (dict(delta=0), fa.FA2_ERR_NULLPTR), (dict(dq=0), fa.FA2_ERR_NULLPTR),
    (dict(dk=0), fa.FA2_ERR_NULLPTR), (dict(dv=0), fa.FA2_ERR_NULLPTR),
    (dict(dout=DO + 8), fa.FA2_ERR_ALIGN), (dict(delta=DL + 4), fa.FA2_ERR_ALIGN), (dict(dv=DV + 2), fa.FA2_ERR_ALIGN),
    (dict(dq=Q), fa.FA2_ERR_ALIAS), (dict(dk=O + 512), fa.FA2_ERR_ALIAS), (dict(dv=DO + 16), fa.FA2_ERR_ALIAS),
    (dict(delta=L), fa.FA2_ERR_ALIAS), (dict(dq=DK), fa.FA2_ERR_ALIAS), (dict(delta=DV + 1024), fa.FA2_ERR_ALIAS),
])
def test_bwd_argument_checks(lib, kwargs, code):
    assert _bwd(**kwargs) == code


@pytest.mark.parametrize("kwargs", [dict(B=0), dict(N=0), dict(H=0, q=0, dq=0, delta=0)])
def test_bwd_empty_problem_is_a_no_op(lib, kwargs):
    assert _bwd(**kwargs) == fa.FA2_OK


def test_bwd_valid_call_without_device_reports_device_error(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this call would launch on fake pointers")
    for d in (64, 128, 256):
        assert _bwd(d=d, dtype=1, causal=1, N=333) == fa.FA2_ERR_DEVICE


def test_python_backward_rejects_bad_tensors(lib):
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    lse = torch.zeros(1, 1, 8)
    with pytest.raises(ValueError):
        fa.backward(q, q, q, q, q, lse)  # host tensors
    with pytest.raises(ValueError):
        fa.backward(q, q, q, q, q[:, :, :4], lse)
    with pytest.raises(TypeError):
        fa.backward(q, q, q, q, q.float(), lse)


# --- fa2_bwd_masked ---------------------------------------------------------------

def _bwd_masked(mask, B=1, H=1, N=16, d=64, scale=0.125, dtype=0, delta=DL, dq=DQ, dk=DK, dv=DV):
    return fa.fa2_bwd_masked(Q, K, V, O, DO, L, delta, dq, dk, dv, B, H, N, d, mask, scale, dtype, None)


@pytest.mark.parametrize("fields,code", [
    (dict(window_left=-2), fa.FA2_ERR_MASK), (dict(window_right=-5), fa.FA2_ERR_MASK),
    (dict(prefix=-1), fa.FA2_ERR_MASK), (dict(segment_ids=0x60000002), fa.FA2_ERR_MASK),
    (dict(segment_ids=DQ + 64), fa.FA2_ERR_ALIAS), (dict(segment_ids=DL), fa.FA2_ERR_ALIAS),
    (dict(segment_ids=DV + 1024), fa.FA2_ERR_ALIAS),
])
def test_bwd_masked_argument_checks(lib, fields, code):
    m = fa.Fa2Mask(0, -1, -1, 0, None)
    for k_, v_ in fields.items():
        setattr(m, k_, v_)
    assert _bwd_masked(m) == code


def test_bwd_masked_shared_checks(lib):
    # the checks fa2_bwd makes apply to the masked entry as well
    m = fa.Fa2Mask(1, 4, 0, 2, None)
    assert _bwd_masked(m, d=32) == fa.FA2_ERR_HEADDIM
    assert _bwd_masked(m, dtype=2) == fa.FA2_ERR_DTYPE
    assert _bwd_masked(m, dq=Q) == fa.FA2_ERR_ALIAS
    assert _bwd_masked(m, delta=DL + 4) == fa.FA2_ERR_ALIGN


def test_bwd_masked_empty_problem_and_null_mask(lib):
    assert _bwd_masked(fa.Fa2Mask(1, 3, 0, 2, None), B=0) == fa.FA2_OK
    assert _bwd_masked(None, N=0) == fa.FA2_OK


def test_bwd_masked_valid_call_without_device_reports_device_error(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this call would launch on fake pointers")
    for mask in (None, fa.Fa2Mask(1, 5, 0, 3, 0xB0000000), fa.Fa2Mask(0, 7, 2, 0, None)):
        for d in (64, 128, 256):
            assert _bwd_masked(mask, d=d, N=333) == fa.FA2_ERR_DEVICE


# --- fa2_fwd_masked ----------------------------------------------------------------

def _masked(mask, B=1, H=1, N=16, d=64, scale=0.125, dtype=0, o=O, lse=L):
    return fa.fa2_fwd_masked(Q, K, V, o, lse, B, H, N, d, mask, scale, dtype, None)


@pytest.mark.parametrize("fields,code", [
    (dict(window_left=-2), fa.FA2_ERR_MASK), (dict(window_right=-5), fa.FA2_ERR_MASK),
    (dict(prefix=-1), fa.FA2_ERR_MASK), (dict(segment_ids=0x60000002), fa.FA2_ERR_MASK),
    (dict(segment_ids=O + 64), fa.FA2_ERR_ALIAS), (dict(segment_ids=L), fa.FA2_ERR_ALIAS),
])
def test_masked_argument_checks(lib, fields, code):
    m = fa.Fa2Mask(0, -1, -1, 0, None)
    for k_, v_ in fields.items():
        setattr(m, k_, v_)
    assert _masked(m) == code


def test_masked_empty_problem_and_null_mask(lib):
    assert _masked(fa.Fa2Mask(1, 3, 0, 2, None), B=0) == fa.FA2_OK
    assert _masked(None, N=0) == fa.FA2_OK


def test_masked_valid_call_without_device_reports_device_error(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this call would launch on fake pointers")
    for mask in (None, fa.Fa2Mask(1, 5, 0, 3, 0x60000000), fa.Fa2Mask(0, -1, -1, 0, None)):
        for d in (64, 128, 256):
            assert _masked(mask, d=d, N=333) == fa.FA2_ERR_DEVICE


# --- fa2_decode --------------------------------------------------------------------

SL, WS = 0xB0000000, 0xC0000000


def _dec(B=1, H=1, Mq=1, Nk=16, d=64, causal=0, scale=0.125, dtype=0, q=Q, k=K, v=V, seqlens=SL, o=O, lse=L,
         ws=WS, ws_bytes=1 << 20):
    return fa.fa2_decode(q, k, v, seqlens, o, lse, B, H, Mq, Nk, d, causal, scale, dtype, ws, ws_bytes, None)


def test_decode_workspace_sizes(lib):
    # small caches need no split; a long cache of one head splits into chunks
    # of at least 256 keys, each with d + 1 floats per query row
    assert fa.fa2_decode_workspace_bytes(1, 1, 1, 16, 64) == 0
    assert fa.fa2_decode_workspace_bytes(1, 1, 1, 4096, 64) == 16 * 1 * 1 * 65 * 4
    assert fa.fa2_decode_workspace_bytes(2, 4, 3, 4096, 128) == 16 * 8 * 3 * 129 * 4
    assert fa.fa2_decode_workspace_bytes(8, 32, 1, 16384, 128) == 2 * 256 * 129 * 4
    assert fa.fa2_decode_workspace_bytes(64, 64, 1, 16384, 128) == 0  # 4096 heads fill the chip alone
    assert fa.fa2_decode_workspace_bytes(0, 4, 1, 4096, 128) == 0
    assert fa.fa2_decode_workspace_bytes(1, 1, 9, 16, 64) == -fa.FA2_ERR_SHAPE
    assert fa.fa2_decode_workspace_bytes(1, 1, 1, 16, 96) == -fa.FA2_ERR_HEADDIM
    assert fa.fa2_decode_workspace_bytes(-1, 1, 1, 16, 64) == -fa.FA2_ERR_SHAPE


@pytest.mark.parametrize("kwargs,code", [
    (dict(B=-1), fa.FA2_ERR_SHAPE), (dict(Mq=-1), fa.FA2_ERR_SHAPE), (dict(Mq=9), fa.FA2_ERR_SHAPE),
    (dict(Nk=-1), fa.FA2_ERR_SHAPE), (dict(Nk=2 ** 31), fa.FA2_ERR_SHAPE),
    (dict(d=32), fa.FA2_ERR_HEADDIM), (dict(dtype=2), fa.FA2_ERR_DTYPE), (dict(scale=math.nan), fa.FA2_ERR_SCALE),
    (dict(q=0), fa.FA2_ERR_NULLPTR), (dict(k=0), fa.FA2_ERR_NULLPTR), (dict(o=0), fa.FA2_ERR_NULLPTR),
    (dict(lse=0), fa.FA2_ERR_NULLPTR),
    (dict(q=Q + 8), fa.FA2_ERR_ALIGN), (dict(lse=L + 4), fa.FA2_ERR_ALIGN), (dict(seqlens=SL + 2), fa.FA2_ERR_ALIGN),
    (dict(Nk=4096, ws=0), fa.FA2_ERR_WORKSPACE), (dict(Nk=4096, ws_bytes=4159), fa.FA2_ERR_WORKSPACE),
    (dict(Nk=4096, ws=WS + 8), fa.FA2_ERR_WORKSPACE),
    (dict(o=Q), fa.FA2_ERR_ALIAS), (dict(o=K + 64), fa.FA2_ERR_ALIAS), (dict(lse=SL), fa.FA2_ERR_ALIAS),
    (dict(lse=O + 64), fa.FA2_ERR_ALIAS), (dict(Nk=4096, ws=V + 1024), fa.FA2_ERR_ALIAS),
    (dict(Nk=4096, ws=O), fa.FA2_ERR_ALIAS),
])
def test_decode_argument_checks(lib, kwargs, code):
    assert _dec(**kwargs) == code


@pytest.mark.parametrize("kwargs", [dict(B=0), dict(H=0), dict(Mq=0), dict(Mq=0, q=0, k=0, o=0, lse=0)])
def test_decode_empty_problem_is_a_no_op(lib, kwargs):
    assert _dec(**kwargs) == fa.FA2_OK


def test_decode_valid_call_without_device_reports_device_error(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this call would launch on fake pointers")
    for d in (64, 128, 256):
        for Mq in (1, 3, 8):
            assert _dec(d=d, Mq=Mq, Nk=5000, causal=1, dtype=1) == fa.FA2_ERR_DEVICE
    # no workspace is needed without a split, and none without a cache
    assert _dec(ws=0, ws_bytes=0) == fa.FA2_ERR_DEVICE
    assert _dec(Nk=0, k=0, v=0, ws=0, ws_bytes=0) == fa.FA2_ERR_DEVICE
    assert _dec(seqlens=0) == fa.FA2_ERR_DEVICE


def test_python_decode_rejects_bad_tensors(lib):
    import torch
    q = torch.zeros(1, 2, 1, 64, dtype=torch.float16)
    kv = torch.zeros(1, 2, 16, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.decode(q, kv, kv)  # host tensors
    with pytest.raises(ValueError):
        fa.decode(q, kv[:, :1], kv)
    with pytest.raises(TypeError):
        fa.decode(q.float(), kv.float(), kv.float())


# --- fa2_fwd_fp8 -------------------------------------------------------------------

DQS, DKS = 0xD0000000, 0xE0000000


def _fp8(B=1, H=1, N=16, d=128, causal=0, scale=0.125, dtype=0, q=Q, k=K, v=V, o=O, lse=L, dq=DQS, dk=DKS):
    return fa.fa2_fwd_fp8(q, k, v, o, lse, B, H, N, d, causal, scale, dq, dk, dtype, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(B=-1), fa.FA2_ERR_SHAPE), (dict(N=2 ** 31), fa.FA2_ERR_SHAPE),
    (dict(d=32), fa.FA2_ERR_HEADDIM), (dict(d=192), fa.FA2_ERR_HEADDIM),
    (dict(dtype=2), fa.FA2_ERR_DTYPE), (dict(scale=math.inf), fa.FA2_ERR_SCALE),
    (dict(q=0), fa.FA2_ERR_NULLPTR), (dict(v=0), fa.FA2_ERR_NULLPTR), (dict(lse=0), fa.FA2_ERR_NULLPTR),
    (dict(k=K + 8), fa.FA2_ERR_ALIGN), (dict(dq=DQS + 2), fa.FA2_ERR_ALIGN),
    (dict(o=Q), fa.FA2_ERR_ALIAS), (dict(o=V + 256), fa.FA2_ERR_ALIAS), (dict(lse=DKS), fa.FA2_ERR_ALIAS),
    (dict(lse=O + 16), fa.FA2_ERR_ALIAS),
])
def test_fp8_argument_checks(lib, kwargs, code):
    assert _fp8(**kwargs) == code


def test_fp8_empty_problem_is_a_no_op(lib):
    assert _fp8(B=0) == fa.FA2_OK
    assert _fp8(N=0, q=0, k=0) == fa.FA2_OK


def test_fp8_valid_call_without_device_reports_device_error(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this call would launch on fake pointers")
    for dtype in (0, 1):
        for causal in (0, 1):
            for d in (64, 128, 256):
                assert _fp8(dtype=dtype, causal=causal, N=4099, d=d) == fa.FA2_ERR_DEVICE
    assert _fp8(dq=0, dk=0) == fa.FA2_ERR_DEVICE


def _fp8_masked(mask, B=1, H=1, N=16, d=128, scale=0.125, dtype=0, o=O, lse=L, dq=DQS, dk=DKS):
    return fa.fa2_fwd_fp8_masked(Q, K, V, o, lse, B, H, N, d, mask, scale, dq, dk, dtype, None)


@pytest.mark.parametrize("fields,code", [
    (dict(window_left=-2), fa.FA2_ERR_MASK), (dict(window_right=-5), fa.FA2_ERR_MASK),
    (dict(prefix=-1), fa.FA2_ERR_MASK), (dict(segment_ids=0x60000002), fa.FA2_ERR_MASK),
    (dict(segment_ids=O + 64), fa.FA2_ERR_ALIAS), (dict(segment_ids=L), fa.FA2_ERR_ALIAS),
])
def test_fp8_masked_argument_checks(lib, fields, code):
    m = fa.Fa2Mask(0, -1, -1, 0, None)
    for k_, v_ in fields.items():
        setattr(m, k_, v_)
    assert _fp8_masked(m) == code


def test_fp8_masked_shared_checks(lib):
    # the checks fa2_fwd_fp8 makes apply to the masked entry as well
    m = fa.Fa2Mask(1, 4, 0, 2, None)
    assert _fp8_masked(m, d=512) == fa.FA2_ERR_HEADDIM
    assert _fp8_masked(m, dtype=2) == fa.FA2_ERR_DTYPE
    assert _fp8_masked(m, o=Q) == fa.FA2_ERR_ALIAS
    assert _fp8_masked(m, dq=DQS + 2) == fa.FA2_ERR_ALIGN
    assert _fp8_masked(m, B=0) == fa.FA2_OK
    assert _fp8_masked(None, N=0) == fa.FA2_OK


def test_fp8_masked_valid_call_without_device_reports_device_error(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this call would launch on fake pointers")
    for mask in (None, fa.Fa2Mask(1, 5, 0, 3, 0xB0000000), fa.Fa2Mask(0, 7, 2, 0, None)):
        for dtype in (0, 1):
            assert _fp8_masked(mask, dtype=dtype, N=333) == fa.FA2_ERR_DEVICE
    for mask in (None, fa.Fa2Mask(1, -1, -1, 0, None), fa.Fa2Mask(1, 5, 0, 3, 0xB0000000),
                 fa.Fa2Mask(0, 7, 2, 0, None)):
        for d in (64, 256):
            assert _fp8_masked(mask, d=d, N=333) == fa.FA2_ERR_DEVICE


def test_python_fp8_forward_rejects_bad_tensors(lib):
    import torch
    q8 = torch.zeros(1, 1, 8, 128, dtype=torch.float8_e4m3fn)
    v = torch.zeros(1, 1, 8, 128, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.forward_fp8(q8, q8, v)  # host tensors
    with pytest.raises(TypeError):
        fa.forward_fp8(v, v, v)



# --- fa2_decode_static ---------------------------------------------------------------

def _dec_static(B=1, H=1, Mq=1, Nk=16, d=64, causal=0, scale=0.125, dtype=0, q=Q, k=K, v=V, seqlens=SL, o=O,
                lse=L):
    return fa.fa2_decode_static(q, k, v, seqlens, o, lse, B, H, Mq, Nk, d, causal, scale, dtype, None)


def test_decode_static_scratch_limit(lib):
    # the largest chunk partials the fixed scratch holds, and the first shapes past it
    assert fa.fa2_decode_workspace_bytes(8, 32, 1, 16384, 128) <= fa.DECODE_STATIC_SCRATCH_BYTES
    assert fa.fa2_decode_workspace_bytes(1, 64, 8, 16384, 256) > fa.DECODE_STATIC_SCRATCH_BYTES
    assert _dec_static(B=1, H=64, Mq=8, Nk=16384, d=256) == fa.FA2_ERR_SCRATCH
    assert _dec_static(B=2, H=100, Mq=8, Nk=16384, d=256) == fa.FA2_ERR_SCRATCH


@pytest.mark.parametrize("kwargs,code", [
    (dict(B=-1), fa.FA2_ERR_SHAPE), (dict(Mq=9), fa.FA2_ERR_SHAPE), (dict(d=32), fa.FA2_ERR_HEADDIM),
    (dict(dtype=2), fa.FA2_ERR_DTYPE), (dict(scale=math.inf), fa.FA2_ERR_SCALE), (dict(q=0), fa.FA2_ERR_NULLPTR),
    (dict(o=O + 8), fa.FA2_ERR_ALIGN), (dict(seqlens=SL + 2), fa.FA2_ERR_ALIGN), (dict(o=Q), fa.FA2_ERR_ALIAS),
    (dict(lse=SL), fa.FA2_ERR_ALIAS),
])
def test_decode_static_argument_checks(lib, kwargs, code):
    assert _dec_static(**kwargs) == code


def test_decode_static_empty_and_no_device(lib):
    assert _dec_static(B=0) == fa.FA2_OK
    assert _dec_static(Mq=0, q=0, o=0, lse=0) == fa.FA2_OK
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this call would launch on fake pointers")
    assert _dec_static(Nk=5000, Mq=3, causal=1) == fa.FA2_ERR_DEVICE  # needs the scratch
    assert _dec_static() == fa.FA2_ERR_DEVICE                        # one chunk: no scratch


# --- fa2_clock_sample ----------------------------------------------------------------

def test_clock_sample_argument_checks(lib):
    assert fa.fa2_clock_sample(0, None) == fa.FA2_ERR_NULLPTR
    assert fa.fa2_clock_sample(O + 8, None) == fa.FA2_ERR_ALIGN
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this call would launch on a fake pointer")
    assert fa.fa2_clock_sample(O, None) == fa.FA2_ERR_DEVICE


def test_clock_ghz_from_samples():
    # two samples 1 ms apart in real time (100 000 ticks): on XCD 0 two CUs whose
    # counters advanced 2.0e6 and 1.8e6 cycles (the second idled part of the
    # time), on XCD 1 one CU that advanced 1.9e6: 2.0, 1.8 and 1.9 GHz per CU,
    # 2.0 and 1.9 GHz per XCD
    n = fa.CLOCK_BLOCKS
    cus = [(0, 0x100, 2_000_000), (0, 0x200, 1_800_000), (1, 0x100, 1_900_000)]
    before, after = [0] * (4 * n), [0] * (4 * n)
    for i in range(n):
        x, hw, adv = cus[i % 3]
        before[4 * i:4 * i + 4] = [x, hw | (i & 0xff), 1000 * (hw >> 8) + x, 50]
        after[4 * i:4 * i + 4] = [x, hw, 1000 * (hw >> 8) + x + adv, 100_050]
    per_cu = fa.clock_ghz(before, after)
    assert sorted(per_cu) == [(0, 1), (0, 2), (1, 1)]
    assert abs(per_cu[(0, 1)] - 2.0) < 1e-12 and abs(per_cu[(0, 2)] - 1.8) < 1e-12
    assert abs(per_cu[(1, 1)] - 1.9) < 1e-12
    assert fa.xcd_clocks(per_cu) == {0: per_cu[(0, 1)], 1: per_cu[(1, 1)]}


def test_profile_digest_ignores_comments_only():
    # The digest that ties a recorded profile to the kernel sources changes with
    # the code and not with its comments; string literals (inline assembly) are
    # code, even when they hold comment markers.
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "bench_mod", os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    a = 'int f(int x) {  // scale\n  return 2 * x; /* twice\n */ }\nconst char* s = "a // b";\n'
    b = 'int f(int x) {\n  // new note\n  return 2 * x; }\nconst char* s = "a // b";  /* kept */\n'
    c = 'int f(int x) { return 3 * x; }\nconst char* s = "a // b";\n'
    d = 'int f(int x) { return 2 * x; }\nconst char* s = "a /* b";\n'
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(c)
    assert bench.code_text(a) != bench.code_text(d)
    assert '"a // b"' in bench.code_text(a)
