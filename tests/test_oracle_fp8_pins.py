"""Pins for the oracle's fp8 (OCP e4m3) score-operand quantisation: the encoder against torch's
float8_e4m3fn conversion (a library routine rounding to nearest even), codes worked out by hand
from the format, a round trip over every finite code, and the absmax scale's defining
properties ("softmax can't say zero, so it subtracts", section "Outliers, and the low-bit claim":
dynamic absmax quantisation of the attention logits)."""
import numpy as np
import pytest
import torch

import oracle


def test_encoder_matches_torch_float8_e4m3fn():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * 60, rng.standard_normal(50000) * 0.02,
                        np.arange(-4000, 4000) * 2.0 ** -12,             # the subnormal range and ties
                        np.arange(-448, 449, 0.5)]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x), ref)


@pytest.mark.parametrize("value,code", [
    (1.0, 0x38), (448.0, 0x7E), (-448.0, 0xFE), (2.0 ** -6, 0x08), (2.0 ** -9, 0x01), (7 * 2.0 ** -9, 0x07),
    (2.0 ** -10, 0x00),            # half the smallest subnormal: ties to the even code 0
    (3 * 2.0 ** -10, 0x02),        # 1.5 smallest subnormals: ties to 2
    (1.0625, 0x38),                # halfway between 1 and 1.125: ties to the even mantissa 0
    (1.1875, 0x3A),                # halfway between 1.125 and 1.25: ties to mantissa 2
    (-2.5, 0xC2), (0.0, 0x00), (460.0, 0x7E), (464.0, 0x7F),
])
def test_hand_codes(value, code):
    assert int(oracle.e4m3_encode(np.array([value], np.float32))[0]) == code


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    vals = oracle.e4m3_decode(codes)
    assert np.all(np.isfinite(vals))
    assert np.array_equal(oracle.e4m3_encode(vals.astype(np.float32)), codes)
    assert np.max(vals) == 448.0 and np.min(np.abs(vals[vals != 0])) == 2.0 ** -9


def test_absmax_scale_properties():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((2, 50, 3, 64)) * rng.uniform(0.01, 30, (2, 1, 3, 1))).astype(np.float32)
    x[1, :, 2] = 0.0                                                       # an all-zero slice
    codes, s = oracle.quantize_fp8(x)
    for b in range(2):
        for h in range(3):
            sl = codes[b, :, h]
            if b == 1 and h == 2:
                assert s[b, h] == 1.0 and np.all(sl == 0)
                continue
            # the slice's largest magnitude lands on the largest code, and nothing exceeds it
            assert np.max(sl & 0x7F) == 0x7E
            assert s[b, h] == np.float32(np.max(np.abs(x[b, :, h]))) / np.float32(448.0)
    # dequantised values are within half a step (1/16 relative, or half a subnormal step) of x
    dq = oracle.dequantize_fp8(codes, s)
    step = np.maximum(np.abs(x) / 16.0, 2.0 ** -10 * s[:, None, :, None])
    assert np.all(np.abs(dq - x) <= step * (1 + 1e-6))


def _bf16(bits):
    """The float32 value of a bf16 bit pattern (exact)."""
    return np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]


def test_rounding_of_the_scaled_value(golden_dir):
    """The reading of the quantiser's arithmetic, pinned by hand-worked slices
    (tests/golden/fp8_rounding_cases.json): r = fl32(448 / amax) once per slice, then
    e4m3(fl32(x * r)). Each x lands exactly on an e4m3 tie in exact arithmetic; the rounded
    reciprocal puts the reading's product one fp32 ulp above it, and the division rule
    x / fl32(amax / 448) exactly on it, so the two rules give different codes here."""
    import json
    import os
    with open(os.path.join(golden_dir, "fp8_rounding_cases.json")) as f:
        fix = json.load(f)
    assert len(fix["cases"]) == 4
    x = np.zeros((2, 8, 2, 64), dtype=np.float32)
    x[0, 0, 0, 0] = _bf16(0x4050)          # 13/4, the slice maximum
    x[0, 3, 0, 5] = _bf16(0x3C1C)          # 39/4096
    x[0, 6, 0, 9] = _bf16(0xBC1C)          # -39/4096
    x[0, 2, 1, 7] = _bf16(0xC0D0)          # -13/2: the maximum magnitude is negative here
    x[0, 5, 1, 1] = _bf16(0x3D1C)          # 39/1024
    x[1, 7, 0, 63] = _bf16(0x4150)         # 13
    x[1, 1, 0, 0] = _bf16(0x3C1C)          # 39/4096
    x[1, :, 1, :] = 0.0                    # an empty slice: scale 1, codes 0
    assert x[0, 3, 0, 5] == 39 / 4096 and x[0, 5, 1, 1] == 39 / 1024 and x[0, 2, 1, 7] == -6.5
    codes, s = oracle.quantize_fp8(x)
    want = {(0, 0, 0, 0): 0x7E, (0, 3, 0, 5): 0x3B, (0, 6, 0, 9): 0xBB, (0, 2, 1, 7): 0xFE,
            (0, 5, 1, 1): 0x43, (1, 7, 0, 63): 0x7E, (1, 1, 0, 0): 0x2B}
    for idx, c in want.items():
        assert int(codes[idx]) == c, (idx, hex(int(codes[idx])), hex(c))
    mask = np.zeros(codes.shape, bool)
    for idx in want:
        mask[idx] = True
    assert np.all(codes[~mask] == 0)
    # the hand-worked fp32 products and scales
    assert np.float32(448.0) / np.float32(3.25) == np.float32(9033886 * 2.0 ** -16)
    assert np.float32(39 / 4096) * np.float32(9033886 * 2.0 ** -16) == np.float32(11010049 * 2.0 ** -23)
    assert s[0, 0] == np.float32(15578843 * 2.0 ** -31) and s[1, 1] == 1.0
    # the division rule gives the tie, and so the even code, on the same slices
    div = oracle.e4m3_encode(np.float32(39 / 4096) / s[0, 0])
    assert np.float32(39 / 4096) / s[0, 0] == np.float32(1.3125) and int(div) == 0x3A
    assert int(oracle.e4m3_encode(np.float32(39 / 1024) / s[0, 1])) == 0x42
    assert int(oracle.e4m3_encode(np.float32(39 / 4096) / s[1, 0])) == 0x2A
