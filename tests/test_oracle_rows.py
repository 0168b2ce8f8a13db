"""Pins of the oracle's row gather + dequant (Q2_K and FP8)."""

import json
import os

import numpy as np
import torch

import oracle
from oracle.engram import _q2k_dequant_blocks


def _block(qs, d_bits, dmin_bits):
    b = np.zeros(84, dtype=np.uint8)
    for g in range(16):
        b[g] = ((g % 4) << 4) | (g % 15 + 1)
    b[16:80] = qs
    b[80], b[81] = d_bits & 0xFF, d_bits >> 8
    b[82], b[83] = dmin_bits & 0xFF, dmin_bits >> 8
    return b


def _golden_blocks(golden_dir):
    with open(os.path.join(golden_dir, "q2k_handworked.json")) as f:
        g = json.load(f)
    out = []
    for blk in g["blocks"]:
        k = np.arange(64)
        qs = k if blk["qs"] == "k" else 255 - k
        out.append((_block(qs.astype(np.uint8), int(blk["d_bits"], 16),
                           int(blk["dmin_bits"], 16)), blk))
    return out


def test_row_sizes():
    # spark page: one Q2_K super-block of 84 bytes per 256-value row:
    # 16 scale/min bytes + 256 * 2 bits + fp16 d + fp16 dmin.
    assert oracle.Q2K_ROW_BYTES == 84 == 16 + 256 * 2 // 8 + 2 + 2
    # vLLM page: FP8 rows carry 256 e4m3 bytes plus one e8m0 byte per 32 values.
    assert oracle.FP8_ROW_BYTES + oracle.FP8_ROW_BYTES // 32 == 264


def test_q2k_handworked_values(golden_dir):
    for block, blk in _golden_blocks(golden_dir):
        table = np.stack([np.zeros(84, np.uint8), block])
        rows = oracle.bf16_value(oracle.rows_q2k(table, np.array([[1]])))[0]
        for i, v in blk["values"].items():
            assert rows[int(i)] == v, (blk["name"], i, rows[int(i)], v)


def test_q2k_unit_scale_block_reproduces_the_quants():
    # scale 1, min 0, d = 1.0: every value is its 2-bit quant.  Pack chosen
    # quants by the stated interleave and read them back.
    rng = np.random.default_rng(1)
    q = rng.integers(0, 4, 256)
    qs = np.zeros(64, dtype=np.uint8)
    for i in range(256):
        qs[32 * (i // 128) + i % 32] |= q[i] << (2 * ((i % 128) // 32))
    b = np.zeros(84, dtype=np.uint8)
    b[:16] = 1
    b[16:80] = qs
    b[81] = 0x3C                      # d = 1.0 (fp16 0x3C00), dmin = 0
    rows = oracle.bf16_value(oracle.rows_q2k(b[None], np.array([[0]])))[0]
    np.testing.assert_array_equal(rows, q.astype(np.float64))


def test_q2k_zero_quants_give_minus_dmin_times_min():
    b = np.zeros(84, dtype=np.uint8)
    mins = np.arange(16)
    b[:16] = (mins << 4) | 7
    b[83] = 0x38                      # dmin = 0.5; d = 0
    rows = oracle.bf16_value(oracle.rows_q2k(b[None], np.array([[0]])))[0]
    np.testing.assert_array_equal(rows, np.repeat(-0.5 * mins, 16))


def test_q2k_values_are_exact_multiples_of_2_pow_minus_24():
    # Reading A11: every value d*scale*q - dmin*min is computed without
    # rounding in float64 (checked against integer arithmetic), so the oracle
    # rounds the exact real value to bf16 exactly once.
    rng = np.random.default_rng(2)
    for _ in range(200):
        blk = rng.integers(0, 256, 84).astype(np.uint8)
        blk[80:84] = rng.uniform(1e-3, 1e-2, 2).astype("<f2").view(np.uint8)
        y = _q2k_dequant_blocks(blk[None])[0]
        d = oracle.fp16_value(blk[80] | (blk[81].astype(np.uint16) << 8))
        dm = oracle.fp16_value(blk[82] | (blk[83].astype(np.uint16) << 8))
        di, dmi = int(d * 2**24), int(dm * 2**24)      # fp16 values are multiples of 2^-24
        assert di == d * 2**24 and dmi == dm * 2**24
        for i in range(256):
            byte = int(blk[16 + 32 * (i // 128) + i % 32])
            q = (byte >> (2 * ((i % 128) // 32))) & 3
            sc, mn = int(blk[i // 16]) & 15, int(blk[i // 16]) >> 4
            assert y[i] * 2**24 == di * sc * q - dmi * mn


def test_q2k_float32_evaluation_is_exact_in_the_workload_range():
    # For d, dmin in [1e-3, 1e-2] (the workloads' range) every float32
    # product and the difference are exact, in either evaluation order and
    # with or without a fused multiply-add, so a float32 kernel reproduces
    # the exact value and its bf16 rounding bit for bit.
    rng = np.random.default_rng(3)
    blk = rng.integers(0, 256, (4096, 84)).astype(np.uint8)
    blk[:, 80:84] = rng.uniform(1e-3, 1e-2, (4096, 2)).astype("<f2").view(np.uint8).reshape(4096, 4)
    exact = _q2k_dequant_blocks(blk)
    d = oracle.fp16_value(blk[:, 80] | (blk[:, 81].astype(np.uint16) << 8)).astype(np.float32)
    dm = oracle.fp16_value(blk[:, 82] | (blk[:, 83].astype(np.uint16) << 8)).astype(np.float32)
    for i in range(0, 256, 7):
        byte = blk[:, 16 + 32 * (i // 128) + i % 32]
        q = ((byte >> (2 * ((i % 128) // 32))) & 3).astype(np.float32)
        sc = (blk[:, i // 16] & 15).astype(np.float32)
        mn = (blk[:, i // 16] >> 4).astype(np.float32)
        a = (d * sc) * q - dm * mn
        b = d * (sc * q) - mn * dm
        np.testing.assert_array_equal(a.astype(np.float64), exact[:, i])
        np.testing.assert_array_equal(b.astype(np.float64), exact[:, i])


def test_out_of_range_ids_read_zero_rows():
    table = np.full((4, 84), 0x55, dtype=np.uint8)
    table[:, 83] = 0x30                       # dmin = 0.125 != d, so rows are non-zero
    ids = np.array([[-1, 4, 2**31 - 1, 3]])
    rows = oracle.rows_q2k(table, ids).reshape(4, 256)
    assert (rows[:3] == 0).all() and (rows[3] != 0).any()
    t8 = np.full((4, 256), 0x38, dtype=np.uint8)
    s8 = np.full((4, 8), 127, dtype=np.uint8)
    rows = oracle.rows_fp8(t8, s8, ids).reshape(4, 256)
    assert (rows[:3] == 0).all() and (rows[3] != 0).all()


def test_fp8_rows_match_torch_decoders():
    # Independent decode: torch's float8_e4m3fn and float8_e8m0fnu casts.
    rng = np.random.default_rng(3)
    R = 64
    vals = np.clip(rng.standard_normal((R, 256)).astype(np.float32), -448, 448)
    codes = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    scales = rng.integers(119, 128, (R, 8)).astype(np.uint8)
    ids = rng.integers(0, R, (5, 3))
    got = oracle.rows_fp8(codes, scales, ids)
    tv = torch.from_numpy(codes).view(torch.float8_e4m3fn).float()
    ts = torch.from_numpy(scales).view(torch.float8_e8m0fnu).float()
    ref = (tv.view(R, 8, 32) * ts.view(R, 8, 1)).view(R, 256)
    ref = ref[torch.from_numpy(ids.reshape(-1))].reshape(5, 3 * 256)
    ref_bits = ref.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref_bits)


def test_rows_layout_is_token_major_then_column():
    # spark page: rows land as [tokens * cols, head_dim], i.e. rows[t, c*256 + i].
    rng = np.random.default_rng(4)
    table = rng.integers(0, 256, (10, 84)).astype(np.uint8)
    ids = np.array([[3, 7], [1, 3]])
    rows = oracle.rows_q2k(table, ids)
    single = lambda r: oracle.rows_q2k(table, np.array([[r]]))[0]
    np.testing.assert_array_equal(rows[0, :256], single(3))
    np.testing.assert_array_equal(rows[0, 256:], single(7))
    np.testing.assert_array_equal(rows[1, :256], single(1))
    np.testing.assert_array_equal(rows[1, 256:], single(3))


# ----------------------------------------------- crafted blocks: one rounding for every fp16

def _bf16_of_fraction(x):
    """Round an exact rational to the nearest bf16 value, ties to even (from the definition)."""
    from fractions import Fraction
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()     # 2^e <= a < 2^(e+2)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, -126) - 7)                    # 8 significant bits
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(fl * quantum)


def _crafted_q2k_blocks():
    """Blocks whose d and dmin lie far apart or at the ends of fp16, where a
    float32 evaluation of d*scale*q - dmin*min is no longer exact."""
    rng = np.random.default_rng(8)
    pairs = [(0x6C00, 0x0001),   # d = 4096, dmin = 2^-24 (smallest subnormal): ratio 2^36
             (0x5BFF, 0x1C01),   # ratio ~2^12
             (0x4000, 0x0C00),   # d = 2, dmin = 2^-12: ratio 2^13
             (0x0200, 0x7BFF),   # d subnormal, dmin = 65504
             (0x0000, 0x3555),   # d = 0
             (0x3C00, 0x0000),   # dmin = 0
             (0xBC00, 0x2000),   # negative d
             (0x7BFF, 0x83FF),   # largest d, negative subnormal dmin
             (0x1400, 0x6400)]   # dmin 2^20 times d
    blocks = []
    for d_bits, m_bits in pairs:
        b = rng.integers(0, 256, 84).astype(np.uint8)
        b[80], b[81] = d_bits & 0xFF, d_bits >> 8
        b[82], b[83] = m_bits & 0xFF, m_bits >> 8
        blocks.append(b)
    for _ in range(40):                       # random finite d, dmin over the whole fp16 range
        b = rng.integers(0, 256, 84).astype(np.uint8)
        for k in (80, 82):
            bits = int(rng.integers(0, 0x7C00)) | (int(rng.integers(0, 2)) << 15)
            b[k], b[k + 1] = bits & 0xFF, bits >> 8
        blocks.append(b)
    return np.stack(blocks)


def test_q2k_crafted_blocks_round_once_from_the_exact_value():
    # The oracle's value for any finite fp16 d, dmin is the exact rational
    # d*scale*q - dmin*min rounded to bf16 once -- including blocks where d
    # and dmin are 2^12 .. 2^36 apart, subnormal, zero or negative.
    from fractions import Fraction
    blocks = _crafted_q2k_blocks()
    rows = oracle.bf16_value(oracle.rows_q2k(blocks, np.arange(len(blocks))[:, None]))
    for r, blk in enumerate(blocks):
        d = Fraction(float(np.frombuffer(blk[80:82].tobytes(), "<f2")[0]))
        dm = Fraction(float(np.frombuffer(blk[82:84].tobytes(), "<f2")[0]))
        for i in range(0, 256, 3):
            byte = int(blk[16 + 32 * (i // 128) + i % 32])
            q = (byte >> (2 * ((i % 128) // 32))) & 3
            sc, mn = int(blk[i // 16]) & 15, int(blk[i // 16]) >> 4
            assert rows[r, i] == _bf16_of_fraction(d * sc * q - dm * mn), (r, i)
