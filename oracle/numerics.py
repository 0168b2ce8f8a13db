"""Number formats used by the Engram forward, decoded from their definitions.

Oracle side; test infrastructure.  Every decoder here is written from the
format's bit layout, so a test can check it against an independent library
decoder (numpy float16, torch float8_e4m3fn / float8_e8m0fnu / bfloat16).

* bf16: the upper 16 bits of an IEEE binary32 (1 sign, 8 exponent, 7 fraction bits).
* fp16: IEEE binary16 (1 sign, 5 exponent bits biased by 15, 10 fraction bits).
* e4m3fn: OCP FP8 E4M3 (1 sign, 4 exponent bits biased by 7, 3 fraction bits;
  no infinities, only S.1111.111 is NaN; largest finite 448).
* e8m0: an unsigned power-of-two scale.  [vLLM engram page,
  _engram_lookup_kernel] turns the byte into a float by placing it in the
  binary32 exponent field (byte << 23, reinterpreted), so byte b means
  2**(b - 127) for b in 1..254.  That placement also fixes the two edge bytes:
  0 gives +0.0 and 255 gives +inf; this oracle follows the page there.
"""

from __future__ import annotations

import numpy as np


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even, in one step.

    Rounds directly from float64 (no intermediate float32 rounding, so no
    double rounding).  Returns float64 arrays holding bf16-representable values.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    finite = np.isfinite(x)
    xf = x[finite]
    _, e = np.frexp(xf)                    # |x| = m * 2**e, 0.5 <= m < 1
    e = np.maximum(e, -125)                # below 2**-126 spacing is fixed (subnormals)
    quantum = np.ldexp(1.0, e - 8)         # 8 significant bits per binade
    r = np.rint(xf / quantum) * quantum    # np.rint rounds half to even
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, xf), r)
    out[finite] = r
    return out


def bf16_bits(x) -> np.ndarray:
    """uint16 storage bits of bf16-representable float64 values (NaN -> 0x7FC0)."""
    x = np.asarray(x, dtype=np.float64)
    f32 = x.astype(np.float32)             # exact for bf16-representable values
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """float64 value of bf16 storage bits."""
    bits = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):     # NaN payloads convert quietly
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def fp16_value(bits) -> np.ndarray:
    """float64 value of IEEE binary16 bits, decoded field by field."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    exp = (b >> 10) & 0x1F
    frac = (b & 0x3FF).astype(np.float64)
    normal = sign * (1.0 + frac / 1024.0) * np.ldexp(1.0, exp - 15)
    subnormal = sign * frac * np.ldexp(1.0, -24)
    special = np.where(frac == 0, sign * np.inf, np.nan)
    return np.where(exp == 0, subnormal, np.where(exp == 31, special, normal))


def e4m3fn_value(codes) -> np.ndarray:
    """float64 value of OCP FP8 E4M3 (fn variant) codes, decoded field by field."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    exp = (b >> 3) & 0xF
    frac = (b & 0x7).astype(np.float64)
    normal = sign * (1.0 + frac / 8.0) * np.ldexp(1.0, exp - 7)
    subnormal = sign * frac * np.ldexp(1.0, -9)
    val = np.where(exp == 0, subnormal, normal)
    return np.where((exp == 15) & (frac == 7), np.nan, val)


def e8m0_scale(codes) -> np.ndarray:
    """float64 scale of e8m0 bytes: the byte placed in the binary32 exponent field."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    val = np.ldexp(1.0, b - 127)
    val = np.where(b == 0, 0.0, val)
    return np.where(b == 255, np.inf, val)
