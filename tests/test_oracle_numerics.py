"""Pins of the oracle's number-format decoders against independent library decoders."""

import numpy as np
import pytest
import torch

import oracle


def test_bf16_round_matches_torch_on_float32_inputs():
    # torch's float32 -> bfloat16 cast rounds to nearest even; on float32
    # inputs there is no double rounding, so both must agree bit for bit.
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),      # subnormal range
        (rng.standard_normal(20000) * 1e38).astype(np.float32),       # near overflow
        rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    ours = oracle.bf16_bits(oracle.bf16_round(x.astype(np.float64)))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_bf16_round_is_single_rounding_from_float64():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties go to the even mantissa (1.0).
    assert oracle.bf16_round([1 + 2.0**-8])[0] == 1.0
    # 1 + 3 * 2^-8 ties between 1 + 2^-7 (odd) and 1 + 2^-6 (even).
    assert oracle.bf16_round([1 + 3 * 2.0**-8])[0] == 1 + 2.0**-6
    # Just above a tie: rounding through float32 first would land on the tie
    # and then go to even (1.0); one rounding from float64 must go up.
    assert oracle.bf16_round([1 + 2.0**-8 + 2.0**-30])[0] == 1 + 2.0**-7
    assert oracle.bf16_round([-(1 + 2.0**-8 + 2.0**-30)])[0] == -(1 + 2.0**-7)
    # Overflow to infinity and zero stay special.
    assert np.isinf(oracle.bf16_round([3.5e38])[0])
    assert oracle.bf16_round([0.0])[0] == 0.0


def test_bf16_value_and_bits_roundtrip_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_value(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    finite = np.isfinite(ref)
    np.testing.assert_array_equal(vals[finite], ref[finite])
    back = oracle.bf16_bits(vals[finite])
    np.testing.assert_array_equal(back, codes[finite])


def test_fp16_value_matches_numpy_for_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.fp16_value(codes)
    ref = codes.view(np.float16).astype(np.float64)
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])


def test_e4m3fn_value_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3fn_value(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])
    assert np.nanmax(ours) == 448.0 and np.nanmin(ours) == -448.0


def test_e8m0_scale_matches_torch_on_normal_bytes():
    codes = np.arange(1, 255, dtype=np.uint8)
    ours = oracle.e8m0_scale(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)
    # The vLLM page's exponent-field placement gives 0.0 for byte 0 and inf for 255.
    assert oracle.e8m0_scale([0])[0] == 0.0
    assert np.isinf(oracle.e8m0_scale([255])[0])


@pytest.mark.parametrize("b", [119, 123, 127])
def test_fp8_products_in_config_range_are_exact_in_bf16(b):
    # Reading A12: for scale bytes 119..127 every finite e4m3 code times the
    # scale is a bf16 value, so the rows stage has a unique correct answer.
    vals = oracle.e4m3fn_value(np.arange(256, dtype=np.uint8))
    vals = vals[np.isfinite(vals)] * oracle.e8m0_scale([b])[0]
    np.testing.assert_array_equal(oracle.bf16_round(vals), vals)
