"""Pins of the oracle's storage decoding against library routines and format definitions.

bf16 / fp8 decoding is what turns stored expert bytes into the values the
expert FFN multiplies (the fp8 DeepSeek-V3-shaped layer uses one fp32 scale
per 128x128 block).  The references here are torch's own dtype conversions,
which the oracle does not call, and fixed points of the OCP E4M3FN format.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def test_fp8_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_fp8_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan_ours, nan_ref = np.isnan(ours), np.isnan(ref)
    assert np.array_equal(nan_ours, nan_ref)
    assert nan_ours.sum() == 2  # 0x7F and 0xFF only: E4M3FN has no infinities
    assert np.array_equal(ours[~nan_ours], ref[~nan_ref])
    assert np.array_equal(np.signbit(ours[~nan_ours]), np.signbit(ref[~nan_ref]))


@pytest.mark.parametrize("code,value", [
    (0x7E, 448.0),          # largest finite
    (0xFE, -448.0),
    (0x08, 2.0 ** -6),      # smallest normal
    (0x01, 2.0 ** -9),      # smallest subnormal
    (0x07, 7 * 2.0 ** -9),  # largest subnormal
    (0x38, 1.0),            # exponent field 7 = bias
    (0x3C, 1.5),
    (0x00, 0.0),
])
def test_fp8_fixed_points(code, value):
    assert oracle.decode_fp8_e4m3fn(np.array([code], dtype=np.uint8))[0] == value


def test_fp8_negative_zero_and_nan():
    v = oracle.decode_fp8_e4m3fn(np.array([0x80, 0x7F, 0xFF], dtype=np.uint8))
    assert v[0] == 0.0 and math.copysign(1.0, v[0]) == -1.0
    assert math.isnan(v[1]) and math.isnan(v[2])


def test_bf16_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan_ours, nan_ref = np.isnan(ours), np.isnan(ref)
    assert np.array_equal(nan_ours, nan_ref)
    assert np.array_equal(ours[~nan_ours], ref[~nan_ref])


def test_fp8_block_scales_index_rows_then_columns():
    # rectangular, so a transposed scale index would not line up
    rows, cols = 256, 384
    codes = np.full((rows, cols), 0x38, dtype=np.uint8)  # every code = 1.0
    scales = (np.arange(2 * 3, dtype=np.float32).reshape(2, 3) + 1.0) * np.float32(0.5)
    v = oracle.decode_matrix(codes, "fp8_e4m3", scales)
    for bi in range(2):
        for bj in range(3):
            blk = v[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            assert np.all(blk == scales[bi, bj])


def test_fp8_block_decode_is_code_times_scale():
    g = np.random.default_rng(7)
    codes = g.integers(0, 256, (128, 256)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10      # avoid NaN codes
    scales = g.random((1, 2)).astype(np.float32) + np.float32(0.1)
    v = oracle.decode_matrix(codes, "fp8_e4m3", scales)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    ref[:, :128] *= float(scales[0, 0])
    ref[:, 128:] *= float(scales[0, 1])
    assert np.array_equal(v, ref)


def test_f32_decode_is_exact_widening():
    a = np.random.default_rng(1).standard_normal(1000).astype(np.float32)
    assert np.array_equal(oracle.decode_x(a, "f32"), a.astype(np.float64))
