// Stage 3: the projection kv = rows x wkv^T, bf16 in, fp32 accumulate, bf16 out.
//
// [spark engram_v41 page, overview stage 3]: the dense bf16 GEMM
// [tokens, cols * head_dim] x wkv^T -> [tokens, dim * (hc + 1)].  [vLLM
// engram page, Engram]: wkv is a bias-free linear.
//
// Both operands are K-contiguous ("NT"), which is the layout the matrix
// cores read directly: v_mfma_f32_32x32x16_bf16 takes, per lane, 8
// consecutive k of one row of A and 8 consecutive k of one row of B.
//
// Tiling (gfx950: 160 KB LDS per CU, 4 SIMDs): a 256 x 256 output tile per
// workgroup of 4 waves in a 2 x 2 grid.  Each wave owns 128 x 128 = 4 x 4
// MFMA tiles, whose 256 fp32 accumulators live in AGPRs.  K advances 64 at a
// time through two LDS stages of 64 KB each (A and B tiles, 256 rows x 128 B).
// The next stage's global loads are in flight while the current stage is
// multiplied.  Inside a row, each 16-byte chunk sits at position
// chunk ^ (row & 7), so the 8 lanes of a ds_read_b128 phase hit 8 distinct
// chunks and never the same banks.
//
// Tile order: the hardware deals workgroups round-robin to the 8 XCDs, each of
// which has its own L2.  The block id is remapped so that every XCD gets a
// contiguous run of tiles, and that run walks 8 M-tiles before it moves along N.
// The ~32 tiles an XCD has in flight then share their A and B panels in its L2.
#include "common.hpp"

namespace engram {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;
constexpr int kNumXcd = 8;
constexpr int kChunks = BK / 8;                         // 16-byte chunks per tile row
constexpr int kLoadsPerThread = BM * kChunks / kThreads;  // per operand, per stage
constexpr int kStageElems = (BM + BN) * BK;             // bf16 elements per stage

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ (row & 7)) << 3);
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

__global__ __launch_bounds__(kThreads, 1) void gemm_nt_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, uint16_t *__restrict__ C,
    int M, int N, int K, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Global -> LDS mapping: thread owns chunk (tid % 8) of rows tid/8 + 32 i.
  const int lchunk = tid & (kChunks - 1);
  const int lrow = tid / kChunks;
  const uint16_t *a_src[kLoadsPerThread];
  const uint16_t *b_src[kLoadsPerThread];
#pragma unroll
  for (int i = 0; i < kLoadsPerThread; ++i) {
    const int r = lrow + i * (kThreads / kChunks);
    const int ar = min(m0 + r, M - 1), br = min(n0 + r, N - 1);   // ragged edges: clamp
    a_src[i] = A + int64_t(ar) * K + lchunk * 8;
    b_src[i] = B + int64_t(br) * K + lchunk * 8;
  }

  u32x4 ra[kLoadsPerThread], rb[kLoadsPerThread];
  auto load_global = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
      ra[i] = *reinterpret_cast<const u32x4 *>(a_src[i] + k0);
      rb[i] = *reinterpret_cast<const u32x4 *>(b_src[i] + k0);
    }
  };
  auto store_lds = [&](int stage) {
    uint16_t *sa = smem + stage * kStageElems;
    uint16_t *sb = sa + BM * BK;
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
      const int r = lrow + i * (kThreads / kChunks);
      *reinterpret_cast<u32x4 *>(sa + swz(r, lchunk)) = ra[i];
      *reinterpret_cast<u32x4 *>(sb + swz(r, lchunk)) = rb[i];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // Fragment reads: lane holds row (lane % 32) of a 32-row slab, k-chunk
  // 2*ks + lane/32 (8 consecutive k) for k sub-step ks of the stage.
  const int frow = lane & 31, fhalf = lane >> 5;
  bf16x8 fa[2][4], fb[2][4];
  auto load_frags = [&](int stage, int ks, int slot) {
    const uint16_t *sa = smem + stage * kStageElems;
    const uint16_t *sb = sa + BM * BK;
    const int chunk = 2 * ks + fhalf;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      fa[slot][i] = *reinterpret_cast<const bf16x8 *>(sa + swz(wm * 128 + i * 32 + frow, chunk));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[slot][j] = *reinterpret_cast<const bf16x8 *>(sb + swz(wn * 128 + j * 32 + frow, chunk));
  };

  const int nk = K / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < nk) load_global((kt + 1) * BK);
    load_frags(stage, 0, 0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < BK / 16) load_frags(stage, ks + 1, cur ^ 1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j],
                                                              acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_lds(stage ^ 1);
    __syncthreads();
  }

  // Epilogue: accumulator r of a 32x32 tile is row 8*(r/4) + 4*(lane/32) + r%4,
  // column lane % 32.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + j * 32 + frow;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * fhalf + (r & 3);
        if (row < M && col < N) C[int64_t(row) * N + col] = f32_to_bf16(acc[i][j][r]);
      }
    }
  }
}

}  // namespace

hipError_t launch_project(const uint16_t *a, const uint16_t *w, uint16_t *c, int32_t M,
                          int32_t K, int32_t N, hipStream_t stream) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const size_t lds = 2 * kStageElems * sizeof(uint16_t);
  // Set on every call: the attribute is per device, and the call is cheap.
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_nt_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemm_nt_kernel, dim3(tiles_m * tiles_n), dim3(kThreads), lds, stream,
                     a, w, c, M, N, K, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace engram
