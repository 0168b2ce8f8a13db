// Pieces shared by the projection kernels (gemm.hip, gemm_q2k.hip): the
// 256 x 256 tiling constants, the bank-conflict-free LDS swizzle, the
// XCD-aware tile order, buffer resources and the pipeline barrier.
#pragma once

#include <atomic>

#include "common.hpp"

namespace engram {
namespace gemm {

constexpr int BM = 256, BN = 256;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kGroupM = 8;
constexpr int kNumXcd = 8;
// sched_group_barrier instruction classes.
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedDsWrite = 0x200;

// s_waitcnt immediate (gfx9 encoding): vmcnt in bits 3:0 and 15:14,
// expcnt 6:4 (left at max), lgkmcnt 11:8.
constexpr int waitcnt(int vm, int lgkm) {
  return (vm & 15) | (((vm >> 4) & 3) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

// LDS layout of one operand tile: BM rows of BK bf16, in 16-byte chunks.
// gfx950's LDS serves a ds_read_b128 16 lanes per cycle across 64 banks.
// Our fragment reads hit 16 consecutive rows at one logical chunk.  The
// chunk is stored at (logical chunk) ^ key(row), and the key makes those 16
// rows land on 16 distinct 16-byte bank groups:
//   BK = 64 (8 chunks, 128 B rows): the bank group is (row % 2, chunk), so key
//     = (row & 7) ^ ((row >> 3) & 1) is a bijection on the 8 even and on the
//     8 odd rows;
//   BK = 32 (4 chunks, 64 B rows): the bank group is (row % 4, chunk), so key
//     = (row >> 2) & 3 is a bijection on each residue class mod 4.
template <int BK>
__device__ __forceinline__ int swz_key(int row) {
  if constexpr (BK == 64) return (row & 7) ^ ((row >> 3) & 1);
  else return (row >> 2) & 3;
}
// Workgroup barrier for the K pipeline.  __syncthreads() carries a release
// fence, which makes the compiler wait for ALL outstanding loads (vmcnt(0)),
// the LDS-DMA loads of later stages included, and that would serialise the
// prefetch.  Instead: wait explicitly for what this stage needs (the
// s_waitcnt immediate kImm), then a bare s_barrier.  LDS has no cache, so a DMA write
// is visible to every wave once it has been counted down.  The empty asm
// statements stop the compiler from moving LDS accesses across the barrier.
template <int kImm>
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(kImm);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int BK>
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ swz_key<BK>(row)) << 3);
}

__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int &tm,
                                            int &tn) {
  const int total = tiles_m * tiles_n;
  const int xcd = bid % kNumXcd, pos = bid / kNumXcd;
  const int base = total / kNumXcd, extra = total % kNumXcd;
  const int lid = xcd * base + min(xcd, extra) + pos;
  const int per_group = kGroupM * tiles_n;
  const int group = lid / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_group = lid - group * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const int32_t n = int32_t(bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : (bytes < 0 ? 0 : bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, 0x00020000);
}

// Epilogue of a 256 x 256 tile whose waves hold NI x NJ blocks of 32 x 32
// from v_mfma_f32_32x32x16_bf16 (accumulator r of a block is row
// 8 * (r / 4) + 4 * (lane / 32) + r % 4, column lane % 32), the wave's blocks
// starting at tile row row0 and column col0.  The bf16 results go through LDS
// (row-major, 512 B per row) so that global memory sees 16-byte stores of
// whole row segments instead of 2-byte stores scattered over rows.  `smem`
// needs 128 KB that no wave reads any more; the caller's barrier before this
// call guarantees that.  kNThreads: the workgroup's thread count; kCols: the
// tile columns stored (those of the blocks, col0 = 0).
template <int NI, int NJ, int kNThreads = kThreads, int kCols = BN>
__device__ __forceinline__ void store_tile_blocks(const f32x16 (&acc)[NI][NJ], uint16_t *smem,
                                                  uint16_t *__restrict__ C, int M, int N,
                                                  int m0, int n0, int row0, int col0, int lane,
                                                  int tid) {
  const int frow = lane & 31, fhalf = lane >> 5;
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + i * 32 + 8 * (r >> 2) + 4 * fhalf + (r & 3);
        smem[row * BN + col0 + j * 32 + frow] = f32_to_bf16(acc[i][j][r]);
      }
  __syncthreads();
  const bool vec = (N % 8) == 0;
  for (int idx = tid; idx < BM * kCols / 8; idx += kNThreads) {
    const int row = idx / (kCols / 8), c8 = (idx % (kCols / 8)) * 8;
    const int grow = m0 + row, gcol = n0 + c8;
    if (grow >= M || gcol >= N) continue;
    uint16_t *dst = C + int64_t(grow) * N + gcol;
    const uint16_t *src = smem + row * BN + c8;
    if (vec) {
      *reinterpret_cast<u32x4 *>(dst) = *reinterpret_cast<const u32x4 *>(src);
    } else {
      for (int e = 0; e < 8 && gcol + e < N; ++e) dst[e] = src[e];
    }
  }
}

// Epilogue of one wave whose MFMAs took the weight as first operand, so that
// each 32 x 32 block comes out transposed: register r of lane (t, h) in
// acc[i][j] is row row0 + 32 i + t, column col0 + 32 j + 8 (r / 4) + 4 h +
// r % 4.  The wave packs a lane's 4 consecutive columns into 8 bytes of its
// own LDS staging area `stg` (32 kCI rows of kStgStride bf16), a chunk of kCI
// row blocks x 2 column blocks at a time, then reads back 16-byte row pieces
// and stores 128-byte row segments.  A wave's LDS accesses complete in order,
// so no barrier is needed; no other wave touches `stg`.
constexpr int kStgStride = 72;   // 144-byte rows: 16-byte aligned, rows 16 apart on other banks
template <int NI, int NJ, int kCI>
__device__ __forceinline__ void store_wave_transposed(const f32x16 (&acc)[NI][NJ], uint16_t *stg,
                                                      uint16_t *__restrict__ C, int M, int N,
                                                      int row0, int col0, int lane) {
  static_assert(NI % kCI == 0 && NJ % 2 == 0, "whole chunks");
  const int frow = lane & 31, fhalf = lane >> 5;
  const bool vec = (N % 8) == 0;
#pragma unroll
  for (int ci = 0; ci < NI / kCI; ++ci)
#pragma unroll
    for (int cj = 0; cj < NJ / 2; ++cj) {
#pragma unroll
      for (int ii = 0; ii < kCI; ++ii)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x16 &a = acc[ci * kCI + ii][2 * cj + jj];
            const u32x2 v = {pack_bf16x2(a[4 * g], a[4 * g + 1]),
                             pack_bf16x2(a[4 * g + 2], a[4 * g + 3])};
            *reinterpret_cast<u32x2 *>(stg + (ii * 32 + frow) * kStgStride + jj * 32 + 8 * g +
                                       4 * fhalf) = v;
          }
#pragma unroll
      for (int r8 = 0; r8 < 4 * kCI; ++r8) {
        const int row = r8 * 8 + (lane >> 3), c8 = (lane & 7) * 8;
        const int grow = row0 + ci * kCI * 32 + row, gcol = col0 + cj * 64 + c8;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(stg + row * kStgStride + c8);
        if (grow < M && gcol < N) {
          uint16_t *dst = C + int64_t(grow) * N + gcol;
          if (vec) {
            *reinterpret_cast<u32x4 *>(dst) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (gcol + e < N) dst[e] = uint16_t(v[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
    }
}

// The 2 x 2 wave layout of 128 x 128 per wave (wave (wm, wn)).
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[4][4], uint16_t *smem,
                                           uint16_t *__restrict__ C, int M, int N, int m0,
                                           int n0, int wm, int wn, int lane, int tid) {
  store_tile_blocks<4, 4>(acc, smem, C, M, N, m0, n0, wm * 128, wn * 128, lane, tid);
}

// The fused projections' layout (gemm_q2k.hip, gemm_fp8.hip): 4 x 1 waves,
// each wave 64 tile rows x all 256 columns (2 x 8 blocks of 32 x 32), K in
// stages of 64, only B (bf16) in shared LDS stages.
namespace wide {

constexpr int kRowsPerLane = 2;            // tile rows w * 64 + 32 i + (lane % 32), i = 0, 1
constexpr int kNJ = BN / 32;               // 8 column blocks per wave
constexpr int BK = 64;
constexpr int kStageElems = BN * BK;                 // one B stage: 32 KB
constexpr int kSegs = BN * BK * 2 / 1024 / kWaves;   // 1 KB B segments per wave per stage: 8

// ---- B: global -> LDS by LDS-DMA.  One instruction fills a 1 KB segment (8
// tile rows); lane L lands at byte 16 L, i.e. row L / 8 of the segment,
// physical chunk L % 8, and fetches the logical chunk the swizzle keeps
// there.  For segment s the swizzle key of that row is (L / 8) ^ (s & 1).
// Rows past N read as zeros (the resource starts at the tile's first row, and
// the row is part of the VGPR offset, the range-checked part; the SGPR offset
// only carries the K position).
struct BSegs {
  uint32_t voff_even, voff_odd, seg_stride;
};
__device__ __forceinline__ BSegs b_segs(int lane, int K) {
  const int seg_row = lane >> 3;
  return {uint32_t(seg_row * K + ((lane & 7) ^ seg_row) * 8) * 2,
          uint32_t(seg_row * K + ((lane & 7) ^ seg_row ^ 1) * 8) * 2, uint32_t(8 * K) * 2};
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t b_rsrc(const uint16_t *B, int N, int K, int tn) {
  const int n0 = tn * BN;
  return make_rsrc(B + int64_t(n0) * K, int64_t(N - n0) * K * 2);
}
// B slice `slice` (K positions 64 slice ..) of the tile into LDS stage sb.
__device__ __forceinline__ void dma_b_slice(__amdgpu_buffer_rsrc_t rb, uint16_t *sb,
                                            const BSegs &g, int wave, int slice) {
#pragma unroll
  for (int i = 0; i < kSegs; ++i) {
    const int seg = wave * kSegs + i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, sb + seg * 512, 16,
                                             ((i & 1) ? g.voff_odd : g.voff_even) +
                                                 seg * g.seg_stride,
                                             slice * BK * 2, 0, 0);
  }
}
// The 8 B fragments of k-step ks of an LDS stage (block j: columns 32 j ..).
__device__ __forceinline__ void load_b_frags(const uint16_t *sb, int frow, int fhalf, int ks,
                                             bf16x8 (&fb)[kNJ]) {
  const int chunk = 2 * ks + fhalf;
#pragma unroll
  for (int j = 0; j < kNJ; ++j)
    fb[j] = *reinterpret_cast<const bf16x8 *>(sb + swz<BK>(j * 32 + frow, chunk));
}

}  // namespace wide

// Compute units of the stream's device (the grid of the persistent kernels),
// read once per device.
inline int num_cus(hipStream_t stream) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= 64) {
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  }
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Grid of a persistent kernel over `tiles` tiles: one workgroup per CU, and,
// when a workgroup gets several tiles, a multiple of 8 so that tile ids b,
// b + grid, ... all lie in workgroup b's XCD run of tile_coords.
inline int persistent_grid(int tiles, hipStream_t stream) {
  const int cus = num_cus(stream);
  return tiles <= cus ? tiles : (cus / 8 * 8 > 8 ? cus / 8 * 8 : 8);
}

}  // namespace gemm
}  // namespace engram
