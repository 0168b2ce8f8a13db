// Pieces shared by the projection kernels (gemm.hip, gemm_q2k.hip): the
// 256 x 256 tiling constants, the bank-conflict-free LDS swizzle, the
// XCD-aware tile order, buffer resources and the pipeline barrier.
#pragma once

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
// call guarantees that.
template <int NI, int NJ>
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
  for (int idx = tid; idx < BM * BN / 8; idx += kThreads) {
    const int row = idx / (BN / 8), c8 = (idx % (BN / 8)) * 8;
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

// The 2 x 2 wave layout of 128 x 128 per wave (wave (wm, wn)).
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[4][4], uint16_t *smem,
                                           uint16_t *__restrict__ C, int M, int N, int m0,
                                           int n0, int wm, int wn, int lane, int tid) {
  store_tile_blocks<4, 4>(acc, smem, C, M, N, m0, n0, wm * 128, wn * 128, lane, tid);
}

}  // namespace gemm
}  // namespace engram
