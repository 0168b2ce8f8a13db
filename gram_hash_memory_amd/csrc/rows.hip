// Stage 2: gather quantised table rows by id and dequantise them to bf16.
//
// [spark engram_v41 page, overview stage 2; ENGRAM_ROW_BYTES]: one Q2_K
// super-block of 84 bytes per 256-value row.  [vLLM engram page,
// _engram_lookup_kernel]: FP8 e4m3 rows with one e8m0 scale per 32 values,
// whose byte is the binary32 exponent field; ids outside the table read as
// zero rows.
//
// Work split: the output is [T * cols] rows of 256 bf16 (512 B each), and
// flat row g lands at byte 512 * g.  A 32-lane half-wave produces one row:
// lane l owns values 8l .. 8l+7 and writes them as one 16-byte store, so each
// row is a single contiguous 512 B write.  For Q2_K, those 8 values share one
// scale/min byte and one bit shift, and their quants are 8 consecutive qs
// bytes; so a lane needs only 4 dword loads, all within the block's 84 bytes
// (which are 4-byte aligned).  Every half-wave keeps kRowsPerHalf rows in
// flight: it issues all their loads before it dequantises any of them.
// The random reads are latency-bound; the bf16 write is the bandwidth term.
#include "common.hpp"
#include "q2k_decode.hpp"

namespace engram {
namespace {

constexpr int kThreads = 256;
constexpr int kHalvesPerBlock = kThreads / 32;
constexpr int kRowsPerHalf = 4;
constexpr int kRowsPerBlock = kHalvesPerBlock * kRowsPerHalf;

__device__ __forceinline__ float half_to_float(uint32_t h16) {
  return float(__builtin_bit_cast(_Float16, uint16_t(h16)));
}

__device__ __forceinline__ void count_bad(int32_t *bad_ids, bool bad, int lane32) {
  if (bad && bad_ids && lane32 == 0) atomicAdd(bad_ids, 1);
}

__global__ __launch_bounds__(kThreads) void rows_q2k_kernel(
    const uint8_t *__restrict__ table, int64_t num_rows, const int32_t *__restrict__ ids,
    int64_t ids_stride, int32_t cols, int64_t total_rows, uint16_t *__restrict__ out,
    int32_t *__restrict__ bad_ids) {
  const int lane = threadIdx.x & 31;
  const int half = threadIdx.x >> 5;
  const int64_t g0 = int64_t(blockIdx.x) * kRowsPerBlock + half * kRowsPerHalf;

  // Per-lane byte offsets inside a block: 8 quants, their scale dword, d/dmin.
  const uint32_t qs_off = 16 + 32 * (lane >> 4) + 8 * (lane & 3);
  const uint32_t sc_off = 4 * (lane >> 3);
  const uint32_t sc_shift = 8 * ((lane >> 1) & 3);
  const uint32_t q_shift = 2 * ((lane & 15) >> 2);

  uint32_t q0[kRowsPerHalf], q1[kRowsPerHalf], scw[kRowsPerHalf], dd[kRowsPerHalf];
  bool ok[kRowsPerHalf];
#pragma unroll
  for (int k = 0; k < kRowsPerHalf; ++k) {
    const int64_t g = g0 + k;
    int64_t id = -1;
    if (g < total_rows) {
      const int64_t t = g / cols, r = g - t * cols;
      id = ids[t * ids_stride + r];
    }
    ok[k] = id >= 0 && id < num_rows;
    const uint8_t *blk = table + (ok[k] ? id : 0) * ENGRAM_Q2K_ROW_BYTES;
    const uint32_t *w = reinterpret_cast<const uint32_t *>(blk);
    q0[k] = w[qs_off / 4];
    q1[k] = w[qs_off / 4 + 1];
    scw[k] = w[sc_off / 4];
    dd[k] = w[80 / 4];
  }
#pragma unroll
  for (int k = 0; k < kRowsPerHalf; ++k) {
    const int64_t g = g0 + k;
    if (g >= total_rows) break;
    const uint32_t sm = (scw[k] >> sc_shift) & 0xFFu;
    const float dl = half_to_float(dd[k] & 0xFFFFu) * float(sm & 0xFu);
    const float ml = half_to_float(dd[k] >> 16) * float(sm >> 4);
    float y[8];
    // One fma per value is exact for most blocks; the others (d and dmin
    // far apart) round their difference to odd first (q2k_decode.hpp).
    float q[8];
#pragma unroll
    for (int b = 0; b < 8; ++b)
      q[b] = float(((((b < 4 ? q0[k] : q1[k]) >> (8 * (b & 3))) & 0xFFu) >> q_shift) & 3u);
    if (q2k_fp32_exact(dd[k])) {
#pragma unroll
      for (int b = 0; b < 8; ++b) y[b] = fmaf(q[b], dl, -ml);
    } else {
#pragma unroll
      for (int b = 0; b < 8; ++b) y[b] = q2k_exact_odd(q[b] * dl, ml);
    }
    u32x4 v;
    v[0] = pack_bf16x2(y[0], y[1]);
    v[1] = pack_bf16x2(y[2], y[3]);
    v[2] = pack_bf16x2(y[4], y[5]);
    v[3] = pack_bf16x2(y[6], y[7]);
    if (!ok[k]) v = u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4 *>(out + g * ENGRAM_HEAD_DIM + 8 * lane) = v;
    count_bad(bad_ids, !ok[k], lane);
  }
}

__global__ __launch_bounds__(kThreads) void rows_fp8_kernel(
    const uint8_t *__restrict__ table, const uint8_t *__restrict__ scales, int64_t num_rows,
    const int32_t *__restrict__ ids, int64_t ids_stride, int32_t cols, int64_t total_rows,
    uint16_t *__restrict__ out, int32_t *__restrict__ bad_ids) {
  const int lane = threadIdx.x & 31;
  const int half = threadIdx.x >> 5;
  const int64_t g0 = int64_t(blockIdx.x) * kRowsPerBlock + half * kRowsPerHalf;

  u32x2 code[kRowsPerHalf];
  uint32_t sbyte[kRowsPerHalf];
  bool ok[kRowsPerHalf];
#pragma unroll
  for (int k = 0; k < kRowsPerHalf; ++k) {
    const int64_t g = g0 + k;
    int64_t id = -1;
    if (g < total_rows) {
      const int64_t t = g / cols, r = g - t * cols;
      id = ids[t * ids_stride + r];
    }
    ok[k] = id >= 0 && id < num_rows;
    const int64_t row = ok[k] ? id : 0;
    code[k] = *reinterpret_cast<const u32x2 *>(table + row * ENGRAM_FP8_ROW_BYTES + 8 * lane);
    sbyte[k] = scales[row * ENGRAM_FP8_SCALE_BYTES + (lane >> 2)];
  }
#pragma unroll
  for (int k = 0; k < kRowsPerHalf; ++k) {
    const int64_t g = g0 + k;
    if (g >= total_rows) break;
    const float scale = __uint_as_float(sbyte[k] << 23);
    float y[8];
#pragma unroll
    for (int b = 0; b < 8; ++b)
      y[b] = e4m3fn_to_float((code[k][b >> 2] >> (8 * (b & 3))) & 0xFFu) * scale;
    u32x4 v;
    v[0] = pack_bf16x2(y[0], y[1]);
    v[1] = pack_bf16x2(y[2], y[3]);
    v[2] = pack_bf16x2(y[4], y[5]);
    v[3] = pack_bf16x2(y[6], y[7]);
    if (!ok[k]) v = u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4 *>(out + g * ENGRAM_HEAD_DIM + 8 * lane) = v;
    count_bad(bad_ids, !ok[k], lane);
  }
}

}  // namespace

hipError_t launch_rows(engram_row_format fmt, const uint8_t *table, const uint8_t *scales,
                       int64_t num_rows, const int32_t *ids, int64_t ids_token_stride,
                       int32_t cols, int32_t T, uint16_t *rows, int32_t *bad_ids,
                       hipStream_t stream) {
  const int64_t total = int64_t(T) * cols;
  const int64_t blocks = (total + kRowsPerBlock - 1) / kRowsPerBlock;
  if (fmt == ENGRAM_ROWS_Q2K)
    hipLaunchKernelGGL(rows_q2k_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                       table, num_rows, ids, ids_token_stride, cols, total, rows, bad_ids);
  else
    hipLaunchKernelGGL(rows_fp8_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                       table, scales, num_rows, ids, ids_token_stride, cols, total, rows,
                       bad_ids);
  return hipGetLastError();
}

}  // namespace engram
