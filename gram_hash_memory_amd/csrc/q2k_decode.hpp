// Q2_K dequant straight into bf16 MFMA operands, shared by the fused
// projections (gemm_q2k.hip, gemm_skinny.hip), and the exact value rule
// shared with engram_rows (rows.hip).
//
// Every value is y = d*scale*q - dmin*min rounded to bf16 once, for every
// finite fp16 d and dmin.  d*scale (<= 15 significant bits), q*d*scale (<= 17)
// and dmin*min (<= 15) are exact in fp32.  When the fp16 exponents of d and
// dmin (subnormals counted as exponent field 1) differ by -9 .. 7, or one of
// them is zero, y is 2^min(E) times an integer below 2^24, so one fp32 fma
// gives y exactly and the bf16 rounding is the only one (q2k_fp32_exact).
// Other blocks take q2k_exact_odd: the fp32 difference and its exact
// rounding error (Knuth's TwoSum), the difference rounded to odd with that
// error, then rounded to bf16 to nearest even -- one rounding of y (rounding
// to odd at 24 bits then to nearest at 8 <= 24 - 2 bits; Boldo and Melquiond).
//
// [spark engram_v41 page, ENGRAM_ROW_BYTES]: a Q2_K row is one 84-byte
// block; within a 16-value group the scale and min are fixed, so a value
// takes one of only four bf16 results, bf16(q * d * scale - dmin * min) for
// q = 0..3.  They are computed once per group, in fp32 with the same fma and
// rounding as engram_rows, and kept as two byte planes (lo = the four low
// bytes, hi = the four high bytes).  Every output pair is then one v_perm_b32
// of (hi, lo) whose selector bytes are q_a, q_a + 4, q_b, q_b + 4, and the
// selectors of four values are two more v_perm_b32 of (m | 0x04040404, m), m
// being their four 2-bit quants, one per byte: 7 VALU ops per 4 values.
#pragma once

#include "common.hpp"

namespace engram {

struct Q2kPlanes {
  uint32_t lo, hi;
};

// dd = fp16 d | fp16 dmin << 16.  True when one fp32 fma per value is exact
// for the whole block (see above); non-finite d or dmin also take that path
// (their values are inf or NaN either way).
__device__ __forceinline__ bool q2k_fp32_exact(uint32_t dd) {
  const uint32_t ed = (dd >> 10) & 31u, em = (dd >> 26) & 31u;
  const int gap = int(ed > 1u ? ed : 1u) - int(em > 1u ? em : 1u);
  return (dd & 0x7FFFu) == 0 || (dd & 0x7FFF0000u) == 0 || ed == 31u || em == 31u ||
         (gap >= -9 && gap <= 7);
}

// a - b rounded to odd at fp32 precision, for exact fp32 a and b: rounding
// the result to bf16 to nearest even rounds a - b once.
__device__ __forceinline__ float q2k_exact_odd(float a, float b) {
  const float s = __fsub_rn(a, b);
  const float bv = __fsub_rn(s, a);                 // TwoSum of a and -b
  const float av = __fsub_rn(s, bv);
  const float e = __fadd_rn(__fsub_rn(a, av), __fsub_rn(-b, bv));
  uint32_t t = __float_as_uint(s);
  if (e != 0.0f && (t & 1u) == 0u) t += ((__float_as_uint(e) ^ t) >> 31) ? 0xFFFFFFFFu : 1u;
  return __uint_as_float(t);
}

// The group's planes from its scale/min byte sm (low nibble scale, high
// nibble min) and dd = fp16 d | fp16 dmin << 16.
__device__ __forceinline__ Q2kPlanes q2k_group_planes(uint32_t dd, uint32_t sm) {
  const float d = float(__builtin_bit_cast(_Float16, uint16_t(dd & 0xFFFFu)));
  const float dmin = float(__builtin_bit_cast(_Float16, uint16_t(dd >> 16)));
  const float dl = d * float(sm & 0xFu), ml = dmin * float(sm >> 4);
  const uint32_t p01 = pack_bf16x2(fmaf(0.0f, dl, -ml), fmaf(1.0f, dl, -ml));
  const uint32_t p23 = pack_bf16x2(fmaf(2.0f, dl, -ml), fmaf(3.0f, dl, -ml));
  return {__builtin_amdgcn_perm(p23, p01, 0x06040200u), __builtin_amdgcn_perm(p23, p01, 0x07050301u)};
}

// q2k_group_planes for any finite d, dmin: each of the four values rounded once.
__device__ __forceinline__ Q2kPlanes q2k_group_planes_exact(uint32_t dd, uint32_t sm) {
  const float d = float(__builtin_bit_cast(_Float16, uint16_t(dd & 0xFFFFu)));
  const float dmin = float(__builtin_bit_cast(_Float16, uint16_t(dd >> 16)));
  const float dl = d * float(sm & 0xFu), ml = dmin * float(sm >> 4);
  const uint32_t p01 = pack_bf16x2(-ml, q2k_exact_odd(dl, ml));
  const uint32_t p23 = pack_bf16x2(q2k_exact_odd(2.0f * dl, ml), q2k_exact_odd(3.0f * dl, ml));
  return {__builtin_amdgcn_perm(p23, p01, 0x06040200u), __builtin_amdgcn_perm(p23, p01, 0x07050301u)};
}

// Eight consecutive values of the group as four bf16 pairs: their quants are
// the 2-bit fields at bit `shift` of the bytes of q0 (values 0..3) and q1
// (values 4..7).
__device__ __forceinline__ u32x4 q2k_expand8(Q2kPlanes p, uint32_t q0, uint32_t q1, int shift) {
  u32x4 v;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t m = ((w ? q1 : q0) >> shift) & 0x03030303u;
    const uint32_t m4 = m | 0x04040404u;
    v[2 * w] = __builtin_amdgcn_perm(p.hi, p.lo, __builtin_amdgcn_perm(m4, m, 0x05010400u));
    v[2 * w + 1] = __builtin_amdgcn_perm(p.hi, p.lo, __builtin_amdgcn_perm(m4, m, 0x07030602u));
  }
  return v;
}

}  // namespace engram
