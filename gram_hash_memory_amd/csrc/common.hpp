// Internal declarations shared by the HIP sources of libengram.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "engram.h"

namespace engram {

// ---------------------------------------------------------------- bf16 / vectors

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even (gfx950: v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair (low half = a), both rounded to nearest even
// by one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// OCP FP8 E4M3 (fn) code -> fp32, from the format's fields (code 0x7F / 0xFF:
// the quiet NaN of that sign).
__device__ __forceinline__ float e4m3fn_to_float(uint32_t b) {
  const uint32_t sign = (b & 0x80u) << 24;
  const uint32_t e = (b >> 3) & 0xFu, m = b & 0x7u;
  if (e == 0) return __uint_as_float(sign | __float_as_uint(float(m) * 0x1p-9f));
  if (e == 15 && m == 7) return __uint_as_float(0x7FC00000u | sign);
  return __uint_as_float(sign | ((e + 120u) << 23) | (m << 20));
}

// An E8M0 scale byte as fp32: the byte in the binary32 exponent field (0 gives
// 0, 255 gives inf).
__device__ __forceinline__ float e8m0_to_float(uint32_t b) { return __uint_as_float(b << 23); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------- hash params

// Hash tables as kernel arguments (copied from the host arrays at each call).
struct HashTables {
  uint64_t mult[ENGRAM_MAX_LAYERS][ENGRAM_MAX_NGRAM];
  uint32_t prime[ENGRAM_MAX_LAYERS][ENGRAM_MAX_COLS];
  uint32_t offset[ENGRAM_MAX_LAYERS][ENGRAM_MAX_COLS];
  int32_t n_layers, max_ngram, n_heads, pad_id;
};

// ---------------------------------------------------------------- launchers
// Each returns hipGetLastError() after queuing its kernel(s); arguments are
// validated by the caller (api.cpp).

hipError_t launch_hash(const HashTables &tab, const engram_tokens &tok, int32_t *ids,
                       hipStream_t stream);

hipError_t launch_history_update(const engram_tokens &tok, int32_t depth, int32_t *history,
                                 uint8_t *history_live, hipStream_t stream);

hipError_t launch_rows(engram_row_format fmt, const uint8_t *table, const uint8_t *scales,
                       int64_t num_rows, const int32_t *ids, int64_t ids_token_stride,
                       int32_t cols, int32_t T, uint16_t *rows, int32_t *bad_ids,
                       hipStream_t stream);

// Picks the weight-streaming kernel of gemm_skinny.hip for few tokens.
hipError_t launch_project(const uint16_t *a, const uint16_t *w, uint16_t *c, int32_t M,
                          int32_t K, int32_t N, hipStream_t stream);
bool project_uses_skinny(int32_t M);
hipError_t launch_project_skinny(const uint16_t *a, const uint16_t *w, uint16_t *c, int32_t M,
                                 int32_t K, int32_t N, hipStream_t stream);

// Rows + projection fused for Q2_K tables (kv bit-identical to rows -> project).
// launch_project_q2k runs the weight-streaming form (gemm_skinny.hip) where
// project_q2k_skinny_supported holds, the 256 x 256 tiles otherwise.
bool project_q2k_supported(int64_t num_rows, int32_t cols);
bool project_q2k_skinny_supported(int32_t M, int32_t cols);
hipError_t launch_project_q2k_skinny(const uint8_t *table, int64_t num_rows, const int32_t *ids,
                                     int64_t ids_token_stride, int32_t cols, const uint16_t *w,
                                     uint16_t *c, int32_t M, int32_t N, int32_t *bad_ids,
                                     hipStream_t stream);
hipError_t launch_project_q2k(const uint8_t *table, int64_t num_rows, const int32_t *ids,
                              int64_t ids_token_stride, int32_t cols, const uint16_t *w,
                              uint16_t *c, int32_t M, int32_t N, int32_t *bad_ids,
                              hipStream_t stream);

// Rows + bf16 projection fused for FP8 tables (gemm_fp8.hip; kv bit-identical
// to rows -> project), for more than 128 tokens.
hipError_t launch_project_fp8(const uint8_t *table, const uint8_t *scales, int64_t num_rows,
                              const int32_t *ids, int64_t ids_token_stride, int32_t cols,
                              const uint16_t *w, uint16_t *c, int32_t M, int32_t N,
                              int32_t *bad_ids, hipStream_t stream);

// MXFP8 projection for FP8 tables (gemm_mx.hip) and its weight prep (mx_quant.hip).
// launch_project_mx runs the weight-streaming form (gemm_skinny.hip) where
// project_mx_skinny_supported holds (up to 64 tokens), the 256 x 256 tiles
// otherwise.
bool project_mx_supported(int32_t N, int32_t K);
bool project_mx_skinny_supported(int32_t M, int32_t cols);
hipError_t launch_project_mx_skinny(const uint8_t *table, const uint8_t *scales, int64_t num_rows,
                                    const int32_t *ids, int64_t ids_token_stride, int32_t cols,
                                    const uint8_t *w_codes, const uint8_t *w_scales, uint16_t *c,
                                    int32_t M, int32_t N, int32_t *bad_ids, hipStream_t stream);
hipError_t launch_project_mx(const uint8_t *table, const uint8_t *scales, int64_t num_rows,
                             const int32_t *ids, int64_t ids_token_stride, int32_t cols,
                             const uint8_t *w_codes, const uint8_t *w_scales, uint16_t *c,
                             int32_t M, int32_t N, int32_t *bad_ids, hipStream_t stream);
// The MXFP8 activation of FP8 rows (codes [M][cols*256], scales [M][cols*8])
// and the 256 x 256 MXFP8 tiles on it (gemm_mx.hip); for cols >= 2, the same
// kv bits as launch_project_mx's tile form.
hipError_t launch_stage_mx(const uint8_t *table, const uint8_t *scales, int64_t num_rows,
                           const int32_t *ids, int64_t ids_token_stride, int32_t cols, int32_t M,
                           uint8_t *a_codes, uint8_t *a_scales, int32_t *bad_ids,
                           hipStream_t stream);
hipError_t launch_project_mx_staged(const uint8_t *a_codes, const uint8_t *a_scales,
                                    int32_t cols, const uint8_t *w_codes,
                                    const uint8_t *w_scales, uint16_t *c, int32_t M, int32_t N,
                                    hipStream_t stream);
hipError_t launch_quantize_mx(const uint16_t *w, int32_t N, int32_t K, uint8_t *codes,
                              uint8_t *scales, hipStream_t stream);

// The gate of several layers in one pass over h (layer order 0..n-1).
struct GateLayers {
  const uint16_t *kv[ENGRAM_MAX_LAYERS];
  const uint16_t *qw[ENGRAM_MAX_LAYERS];
  const uint16_t *kw[ENGRAM_MAX_LAYERS];
  int32_t n;
};
hipError_t launch_gate_layers(float *h, const GateLayers &ly, const uint8_t *mask, int32_t T,
                              int32_t hc, int32_t dim, float eps, float clamp, float dot_scale,
                              hipStream_t stream);

hipError_t launch_gate(float *h, const uint16_t *kv, const uint16_t *qw, const uint16_t *kw,
                       const uint8_t *mask, int32_t T, int32_t hc, int32_t dim, float eps,
                       float clamp, float dot_scale, hipStream_t stream);

}  // namespace engram
