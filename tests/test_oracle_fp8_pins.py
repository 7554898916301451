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
