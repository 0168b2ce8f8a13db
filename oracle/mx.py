"""MXFP8 projection for FP8 layers -- oracle side, test infrastructure only.

[vLLM engram page, EngramBatch / wkv_input]: the FP8 rows of a table (E4M3
codes with one E8M0 scale per 32 values of a row) are already MXFP8 blocks,
and the vLLM path hands them, unchanged, to a block-scaled WKV GEMM whose
weight is held in MXFP8 too.  This module defines that projection:

* rows_fp8_mx: the raw row bytes gathered by id (no dequant);
* quantize_mxfp8: an MXFP8 copy of a bf16 wkv [N, K], one E8M0 scale per 32
  consecutive k of a row (reading A22: the OCP MX v1.0 scale rule, shared
  exponent floor(log2(amax)) - 8 for E4M3, elements rounded to nearest even
  and saturated at +-448);
* project_mxfp8: kv = bf16(sum_k a[t, k] * w[n, k]) over the dequantised MX
  operands, the sum taken in float64 and rounded to bf16 once.

E8M0 here follows the OCP MX definition, byte b meaning 2**(b - 127) and 0xFF
NaN (reading A22).  The bf16 row path (rows_fp8) keeps the vLLM lookup's
exponent-field placement (byte 0 -> 0, 0xFF -> inf).  The two agree on bytes
1..254, the only ones the workloads draw.
"""

from __future__ import annotations

import numpy as np

from .numerics import bf16_round, bf16_bits, bf16_value, e4m3fn_value

MX_BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8            # 448 = 1.75 * 2**8


def e8m0_mx_scale(codes) -> np.ndarray:
    """float64 value of OCP E8M0 scale bytes: 2**(b - 127), NaN for 0xFF."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    out = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, out)


def _e4m3_rne(x) -> np.ndarray:
    """E4M3 codes of float64 values already inside [-448, 448], round to nearest even.

    Written from the format: normal binades 2**-6 .. 2**8 keep 3 fraction
    bits, so the quantum is 2**(e - 3) there; below 2**-6 the quantum is the
    subnormal step 2**-9.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = (np.signbit(x)).astype(np.uint8) << 7
    a = np.abs(x)
    _, e = np.frexp(a)                       # a = m * 2**e, 0.5 <= m < 1, so binade e - 1
    binade = np.maximum(e - 1, -6)
    quantum = np.ldexp(1.0, binade - 3)
    q = np.rint(a / quantum) * quantum       # ties to even
    # q may have rounded up into the next binade; re-derive its fields from q
    _, e2 = np.frexp(q)
    b2 = e2 - 1
    normal = (q >= 2.0 ** -6)
    exp_field = np.where(normal, b2 + 7, 0)
    mant = np.where(normal, np.rint((q / np.ldexp(1.0, b2) - 1.0) * 8.0), np.rint(q / 2.0 ** -9))
    code = (exp_field.astype(np.int64) << 3) | mant.astype(np.int64)
    code = np.where(q == 0.0, 0, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def quantize_mxfp8(wkv_bits) -> tuple[np.ndarray, np.ndarray]:
    """MXFP8 copy of bf16 wkv [N, K] (K % 32 == 0): (codes [N, K], scales [N, K/32]).

    Per block of 32 consecutive k: amax = max |w|; the scale byte is
    floor(log2(amax)) - 8 + 127 clamped to 0..254 (127 for an all-zero
    block); each element is w / 2**(byte - 127), saturated to +-448 and
    rounded to the nearest E4M3 value, ties to even.
    """
    w = bf16_value(wkv_bits)
    N, K = w.shape
    assert K % MX_BLOCK == 0
    blocks = w.reshape(N, K // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(blocks), axis=2)
    with np.errstate(divide="ignore"):
        _, e = np.frexp(amax)                # amax = m * 2**e -> floor(log2(amax)) = e - 1
    shared = np.where(amax > 0, e - 1 - E4M3_EMAX, 0)
    byte = np.clip(shared + 127, 0, 254).astype(np.int64)
    x = blocks / np.ldexp(1.0, byte - 127)[:, :, None]
    x = np.clip(x, -E4M3_MAX, E4M3_MAX)
    codes = _e4m3_rne(x).reshape(N, K)
    return codes, byte.astype(np.uint8)


def mx_values(codes, scales) -> np.ndarray:
    """float64 values of MXFP8 data: codes [R, K] times the scale of their 32-block."""
    v = e4m3fn_value(codes)
    s = np.repeat(e8m0_mx_scale(scales), MX_BLOCK, axis=1)
    return v * s


def rows_fp8_mx(table, scales, ids) -> tuple[np.ndarray, np.ndarray]:
    """Raw FP8 rows by id: codes [T, cols*256] and scales [T, cols*8] (uint8).

    An id outside the table gives zero codes and scale byte 127 (value 1), so
    the row contributes exactly zero.
    """
    table = np.asarray(table, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    ids = np.asarray(ids, dtype=np.int64)
    T, cols = ids.shape
    flat = ids.reshape(-1)
    ok = (flat >= 0) & (flat < table.shape[0])
    safe = np.where(ok, flat, 0)
    codes = np.where(ok[:, None], table[safe], 0).astype(np.uint8)
    scl = np.where(ok[:, None], scales[safe], 127).astype(np.uint8)
    return codes.reshape(T, -1), scl.reshape(T, -1)


def project_mxfp8(a_codes, a_scales, w_codes, w_scales) -> np.ndarray:
    """kv = bf16(A @ W^T) over MXFP8 operands, bf16 bits [T, N]; float64 sum, one rounding."""
    a = mx_values(a_codes, a_scales)
    w = mx_values(w_codes, w_scales)
    return bf16_bits(bf16_round(a @ w.T))
