"""Pins for the MXFP8 projection oracle (oracle/mx.py), CPU only.

* e8m0_mx_scale against torch's float8_e8m0fnu decoder, every byte.
* _e4m3_rne against torch's float8_e4m3fn conversion (round to nearest even)
  on values inside the format's range, and on every E4M3 value (identity).
* quantize_mxfp8: a hand-worked block; the scale rule 2**8 <= amax / scale <
  2**9; blocks of E4M3 values round-trip exactly; saturation at 448; the
  zero block; the error bound of half a quantum.
* rows_fp8_mx: the gathered bytes are the table's; dequantised they equal the
  bf16 row path (rows_fp8) bit for bit on scale bytes 1..254.
* project_mxfp8: the exact rational sum on small cases (fractions), and the
  bf16 projection of the dequantised operands (which are bf16-exact).
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import mx


def test_e8m0_against_torch_every_byte():
    b = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = oracle.e8m0_mx_scale(b)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


def test_e4m3_rne_against_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.uniform(-1, 1, 20000) * 2.0 ** rng.integers(-12, 9, 20000),
        np.array([0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11,
                  1.0625, 1.1875, 464.0 - 1e-9, 2.0 ** -6 - 2.0 ** -12]),
    ])
    x = np.clip(x.astype(np.float32).astype(np.float64), -448, 448)
    want = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = mx._e4m3_rne(x)
    # +-0 compare by value (both encodings of zero are fine for a zero input)
    vw, vg = oracle.e4m3fn_value(want), oracle.e4m3fn_value(got)
    assert np.array_equal(vw, vg)
    assert np.array_equal(got[x != 0], want[x != 0])


def test_e4m3_rne_identity_on_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    v = oracle.e4m3fn_value(codes)
    back = mx._e4m3_rne(v)
    assert np.array_equal(oracle.e4m3fn_value(back), v)


def _bf16(x):
    return oracle.bf16_bits(oracle.bf16_round(np.asarray(x, dtype=np.float64)))


def test_quantize_hand_worked_block():
    # amax = 3 -> floor(log2 3) = 1 -> shared exponent 1 - 8 = -7 -> byte 120;
    # elements are w * 2**7: 1 -> 128, 0.5 -> 64, 3 -> 384, -0.75 -> -96,
    # 0.01171875 (3/256) -> 1.5.
    w = np.zeros((1, 32))
    w[0, :5] = [1.0, 0.5, 3.0, -0.75, 3.0 / 256]
    codes, scales = oracle.quantize_mxfp8(_bf16(w))
    assert scales.tolist() == [[120]]
    # E4M3: 128 = 2**7 -> exp field 14 -> 0x70; 64 -> 0x68; 384 = 1.5 * 2**8 -> 0x7C;
    # -96 = -1.5 * 2**6 -> 0x80 | 0x6C = 0xEC; 1.5 -> exp 7, mant 4 -> 0x3C.
    assert codes[0, :5].tolist() == [0x70, 0x68, 0x7C, 0xEC, 0x3C]
    assert (codes[0, 5:] == 0).all()


def test_quantize_scale_rule_roundtrip_saturation_zero():
    rng = np.random.default_rng(5)
    N, K = 64, 256
    w = rng.standard_normal((N, K)) * 2.0 ** rng.integers(-20, 10, (N, 1))
    wb = _bf16(w)
    codes, scales = oracle.quantize_mxfp8(wb)
    wv = oracle.bf16_value(wb).reshape(N, K // 32, 32)
    amax = np.abs(wv).max(axis=2)
    s = oracle.e8m0_mx_scale(scales)
    ratio = amax / s
    assert ((ratio >= 256) & (ratio < 512)).all()
    # error of each element is at most half an E4M3 quantum at its magnitude (times the
    # scale), or the saturation gap above 448
    deq = oracle.mx_values(codes, scales).reshape(N, K // 32, 32)
    x = wv / s[:, :, None]
    xs = np.clip(np.abs(x), 0, 448)
    _, e = np.frexp(np.maximum(xs, 2.0 ** -12))
    quantum = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)
    err = np.abs(np.abs(deq / s[:, :, None]) - xs)
    assert (err <= quantum / 2 + 1e-12).all()
    # E4M3-exact blocks scaled by a power of two round-trip exactly (one element in 256..448)
    v = oracle.e4m3fn_value(rng.integers(0, 0x7E, (8, 256)).astype(np.uint8))
    v[:, ::32] = 448.0
    v = v * 2.0 ** rng.integers(-30, 20, (8, 1))
    c2, s2 = oracle.quantize_mxfp8(_bf16(v))
    assert np.array_equal(oracle.mx_values(c2, s2), v)
    # saturation: 3.90625 * 2**7 = 500 > 448 -> 448
    w3 = np.zeros((1, 32))
    w3[0, 0], w3[0, 1] = 3.90625, 1.0
    c3, s3 = oracle.quantize_mxfp8(_bf16(w3))
    assert s3[0, 0] == 120 and c3[0, 0] == 0x7E
    # all-zero block: scale byte 127, zero codes
    c4, s4 = oracle.quantize_mxfp8(np.zeros((2, 64), dtype=np.uint16))
    assert (s4 == 127).all() and (c4 == 0).all()


def test_rows_fp8_mx_against_table_and_bf16_rows():
    rng = np.random.default_rng(9)
    R = 40
    table = rng.integers(0, 256, (R, 256)).astype(np.uint8)
    table[(table & 0x7F) == 0x7F] = 0x11            # no NaN codes
    scales = rng.integers(1, 255, (R, 8)).astype(np.uint8)
    scales[0, 0] = 1
    scales[1, 0] = 254
    ids = np.array([[3, 0, 39], [1, -1, 40]], dtype=np.int64)
    codes, scl = oracle.rows_fp8_mx(table, scales, ids)
    assert np.array_equal(codes[0].reshape(3, 256), table[[3, 0, 39]])
    assert np.array_equal(scl[0].reshape(3, 8), scales[[3, 0, 39]])
    assert (codes[1, 256:] == 0).all() and (scl[1, 8:] == 127).all()
    bf = oracle.rows_fp8(table, scales, ids)
    assert np.array_equal(_bf16(oracle.mx_values(codes, scl)), bf)


def _bf16_of_fraction(x: Fraction) -> int:
    """bf16 bits of an exact rational, rounded to nearest even in one step."""
    if x == 0:
        return 0
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = Fraction(2) ** (e - 7)               # 8 significant bits
    n = a / q
    r = int(n)
    rem = n - r
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and r % 2 == 1):
        r += 1
    v = float(r * q)                         # exact: r has at most 9 bits
    return sign | int(np.array([v], dtype=np.float32).view(np.uint32)[0] >> 16)


def test_project_mxfp8_exact_small_and_reduction():
    rng = np.random.default_rng(11)
    T, N, K = 3, 4, 64
    a_codes = rng.integers(0, 0x7E, (T, K)).astype(np.uint8) | (rng.integers(0, 2, (T, K)) << 7).astype(np.uint8)
    w_codes = rng.integers(0, 0x7E, (N, K)).astype(np.uint8)
    a_sc = rng.integers(120, 135, (T, K // 32)).astype(np.uint8)
    w_sc = rng.integers(120, 135, (N, K // 32)).astype(np.uint8)
    got = oracle.project_mxfp8(a_codes, a_sc, w_codes, w_sc)
    av = oracle.mx_values(a_codes, a_sc)
    wv = oracle.mx_values(w_codes, w_sc)
    for t in range(T):
        for n in range(N):
            exact = sum(Fraction(float(av[t, k])) * Fraction(float(wv[n, k])) for k in range(K))
            assert got[t, n] == _bf16_of_fraction(exact)
    # the dequantised operands are bf16-exact, so the bf16 projection gives the same bits
    assert np.array_equal(got, oracle.project(_bf16(av), _bf16(wv)))
