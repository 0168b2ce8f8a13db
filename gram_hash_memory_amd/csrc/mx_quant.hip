// MXFP8 copy of a bf16 weight [N][K] for the block-scaled projection.
//
// [vLLM engram page, EngramBatch]: the WKV GEMM there runs on MXFP8
// operands, the weight included.  The scale rule is the OCP MX v1.0 one for
// E4M3: per block of 32 consecutive k of a row, the shared exponent is
// floor(log2(amax)) - 8 (8 = E4M3's largest exponent), stored as the E8M0
// byte exponent + 127 clamped to 0..254, 127 for an all-zero block; every
// element is divided by the scale, saturated to +-448 and rounded to the
// nearest E4M3 value, ties to even.
//
// One thread per block: it reads its 64 bytes of bf16 and writes 32 codes and
// one scale byte.  This runs once per weight, off the forward path.
#include "common.hpp"

namespace engram {
namespace {

constexpr int kThreads = 256;

// E4M3 (OCP e4m3fn) code of x, |x| <= 448 after saturation, round to nearest
// even.  Normal binades 2^-6 .. 2^8 keep 3 fraction bits: the fp32 fraction is
// rounded at bit 20 and the exponent rebased from 127 to 7 (a carry out of
// the fraction moves to the next binade by itself).  Below 2^-6 the step is
// the subnormal quantum 2^-9, and the rounded multiple of it is the code
// (8 multiples reach the smallest normal, whose code is also 8).
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {
    code = uint32_t(rintf(a * 512.0f));
  } else {
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    code = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
  }
  return code | sign;
}

__global__ __launch_bounds__(kThreads) void quantize_mx_kernel(const uint16_t *__restrict__ w,
                                                               int64_t blocks,
                                                               uint8_t *__restrict__ codes,
                                                               uint8_t *__restrict__ scales) {
  const int64_t b = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (b >= blocks) return;
  const u32x4 *src = reinterpret_cast<const u32x4 *>(w + b * 32);
  uint32_t v[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 q = src[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * i + e] = q[e];
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[i])), fabsf(bf16_hi(v[i]))));
  int byte = 127;
  if (amax > 0.0f) {
    int e;
    frexpf(amax, &e);                       // amax = m * 2^e, 0.5 <= m < 1
    byte = min(max(e - 1 - 8 + 127, 0), 254);
  }
  const int shift = 127 - byte;             // x = w * 2^shift, exact
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t c0 = e4m3_rne(ldexpf(bf16_lo(v[2 * i]), shift));
    const uint32_t c1 = e4m3_rne(ldexpf(bf16_hi(v[2 * i]), shift));
    const uint32_t c2 = e4m3_rne(ldexpf(bf16_lo(v[2 * i + 1]), shift));
    const uint32_t c3 = e4m3_rne(ldexpf(bf16_hi(v[2 * i + 1]), shift));
    out[i] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
  }
  u32x4 *dst = reinterpret_cast<u32x4 *>(codes + b * 32);
  dst[0] = u32x4{out[0], out[1], out[2], out[3]};
  dst[1] = u32x4{out[4], out[5], out[6], out[7]};
  scales[b] = uint8_t(byte);
}

}  // namespace

hipError_t launch_quantize_mx(const uint16_t *w, int32_t N, int32_t K, uint8_t *codes,
                              uint8_t *scales, hipStream_t stream) {
  const int64_t blocks = int64_t(N) * (K / 32);
  const int64_t grid = (blocks + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(quantize_mx_kernel, dim3(unsigned(grid)), dim3(kThreads), 0, stream, w,
                     blocks, codes, scales);
  return hipGetLastError();
}

}  // namespace engram
