"""The fp8 parity tests hand the oracle the real inputs q8 * descale: the e4m3
bytes decoded by torch (float8_e4m3fn -> float64), times the float32 descale.
This pins that decoding to the OCP e4m3 definition for every one of the 256
codes (sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is
subnormal, m/8 * 2^-6; the all-ones code S.1111.111 is NaN and there is no
infinity), so the oracle's inputs rest on the format's definition, not on the
library alone."""
import math

import numpy as np
import torch


def _ocp_e4m3(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def test_e4m3_decoding_matches_the_format_definition():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    got = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    want = np.array([_ocp_e4m3(c) for c in range(256)])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.nanmax(want) == 448.0 and np.nanmin(want[want > 0]) == 2.0 ** -9


def test_descaled_inputs_are_exact_in_fp64():
    """fp8 value (4 significant bits) times a float32 descale (24 bits) needs 28
    bits: the fp64 product the oracle receives is exact."""
    from exact_attention_11_amd.inputs import make_qkv_fp8
    q8, _, _, dq, _ = make_qkv_fp8(1, 2, 64, 128, "fp16", "normal", 3)
    a = q8.to(torch.float64) * dq.to(torch.float64).reshape(1, 2, 1, 1)
    # exact: dividing back by the descale recovers the e4m3 values bit for bit
    assert torch.equal(a / dq.to(torch.float64).reshape(1, 2, 1, 1), q8.to(torch.float64))
