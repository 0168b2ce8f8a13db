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
// workgroup; A and B tiles stream through two LDS stages of 64 k, and the
// chunk swizzle keeps the fragment reads free of bank conflicts.  Two forms:
//  - gemm_nt_persistent_kernel (K a multiple of 128, the usual case): one
//    workgroup of 8 waves (2 x 4, 128 x 64 each, two waves per SIMD) per CU
//    walks its tiles; the stages are filled by LDS-DMA a whole stage ahead,
//    and the next tile's first slices are fetched during the current tile's
//    last iterations;
//  - gemm_nt_kernel (one tile per workgroup, any K % 64 == 0): 4 waves in a
//    2 x 2 grid, 128 x 128 each with its 256 fp32 accumulators in AGPRs;
//    each stage is filled from global memory through VGPRs (raw buffer
//    loads, then ds_write_b128), its loads issued two iterations ahead of
//    the matrix cores, and fragment reads interleaved one-for-two with the
//    MFMAs.
//
// Tile order: the hardware deals workgroups round-robin to the 8 XCDs, each of
// which has its own L2.  The block id is remapped so that every XCD gets a
// contiguous run of tiles, and that run walks 8 M-tiles before it moves along N.
// The ~32 tiles an XCD has in flight then share their A and B panels in its L2.
#include "gemm_common.hpp"

namespace engram {
namespace {

using namespace gemm;

// One 256 x 256 output tile per workgroup.  K streams through two LDS stages
// (BK = 64 each) fed from two register stages: slice s is requested from
// global memory (raw buffer loads into VGPRs) two iterations before it is
// multiplied, written to LDS one iteration before, and read back as MFMA
// fragments while it is multiplied.  Plain loads plus ds_write move about a
// third more data into LDS per unit time than gfx950's LDS-DMA loads do
// here, and the VGPRs they need are free: the accumulators sit in AGPRs.
__global__ __launch_bounds__(kThreads, 1) void gemm_nt_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, uint16_t *__restrict__ C,
    int M, int N, int K, int tiles_m, int tiles_n) {
  constexpr int BK = 64;
  constexpr int kStageElems = (BM + BN) * BK;      // bf16 elements per LDS stage
  constexpr int kChunks = BK / 8;                  // 16-byte chunks per tile row
  constexpr int kRowStep = kThreads / kChunks;     // rows covered per load round
  constexpr int kLoads = BM / kRowStep;            // loads per operand per thread
  constexpr int kKsub = BK / 16;                   // MFMA k sub-steps per stage
  extern __shared__ __attribute__((aligned(1024))) uint16_t smem[];

  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // Global -> VGPR: thread owns logical chunk (tid % 8) of rows tid/8 + 32 i.
  // The buffer resources start at the tile's first row, so rows past M (or N)
  // read as zeros.
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + int64_t(m0) * K, int64_t(M - m0) * K * 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + int64_t(n0) * K, int64_t(N - n0) * K * 2);
  const int lrow = tid / kChunks, lchunk = tid % kChunks;
  const uint32_t voff = uint32_t(lrow * K + lchunk * 8) * 2;
  const uint32_t row_step = uint32_t(kRowStep * K) * 2;

  u32x4 ga[2][kLoads], gb[2][kLoads];
  auto load_global = [&](int set, int k0) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      // The row goes into the VGPR offset: only that part is range-checked.
      const uint32_t v = voff + i * row_step;
      ga[set][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, v, k0 * 2, 0));
      gb[set][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, v, k0 * 2, 0));
    }
  };
  auto store_lds = [&](int set, int stage) {
    uint16_t *sa = smem + stage * kStageElems;
    uint16_t *sb = sa + BM * BK;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int r = lrow + i * kRowStep;
      *reinterpret_cast<u32x4 *>(sa + swz<BK>(r, lchunk)) = ga[set][i];
      *reinterpret_cast<u32x4 *>(sb + swz<BK>(r, lchunk)) = gb[set][i];
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
      fa[slot][i] =
          *reinterpret_cast<const bf16x8 *>(sa + swz<BK>(wm * 128 + i * 32 + frow, chunk));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[slot][j] =
          *reinterpret_cast<const bf16x8 *>(sb + swz<BK>(wn * 128 + j * 32 + frow, chunk));
  };
  auto mfma_block = [&](int slot) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j],
                                                            acc[i][j], 0, 0, 0);
  };
  // Scheduling patterns for one sub-step (16 MFMAs, 8 fragment reads), with
  // the global loads (16) or the LDS writes (16) of the pipeline spread over it.
  auto sched_reads = [&]() {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
    }
  };
  auto sched_reads_vmem = [&]() {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
    }
  };
  auto sched_reads_dswrite = [&]() {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
    }
  };

  // One iteration multiplies slice kt from LDS stage kt % 2 and
  //  - requests slice kt + 2 into register set kt % 2 (sub-step 0),
  //  - waits for slice kt + 1 (issued one iteration earlier, so vmcnt may
  //    keep the 2 * kLoads newer loads in flight) and writes it to LDS stage
  //    (kt + 1) % 2 (sub-step 2).  That stage was last read in iteration
  //    kt - 1, and every wave passed the barrier after it,
  //  - waits for its LDS traffic and meets the other waves at the barrier,
  //    after which stage (kt + 1) % 2 is complete,
  //  - reads the first fragments of slice kt + 1 while the last sub-step of
  //    slice kt multiplies.
  // Requests past the end re-read the final K slice (in bounds, never used).
  const int nk = K / BK;
  auto iteration = [&](int kt, const int set) {
    const int stage = set;                          // kt % 2, as a compile-time value
    load_global(set, min(kt + 2, nk - 1) * BK);
    load_frags(stage, 1, 1);
    mfma_block(0);
    sched_reads_vmem();
    load_frags(stage, 2, 0);
    mfma_block(1);
    sched_reads();
    __builtin_amdgcn_s_waitcnt(waitcnt(2 * kLoads, 15));
    store_lds(set ^ 1, stage ^ 1);
    load_frags(stage, 3, 1);
    mfma_block(0);
    sched_reads_dswrite();
    stage_barrier<waitcnt(2 * kLoads, 0)>();
    load_frags(stage ^ 1, 0, 0);
    mfma_block(1);
    sched_reads();
  };

  load_global(0, 0);
  load_global(1, min(1, nk - 1) * BK);
  __builtin_amdgcn_s_waitcnt(waitcnt(2 * kLoads, 15));
  store_lds(0, 0);
  stage_barrier<waitcnt(2 * kLoads, 0)>();
  load_frags(0, 0, 0);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    iteration(kt, 0);
    iteration(kt + 1, 1);
  }
  if (kt < nk) iteration(kt, 0);
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
  __syncthreads();                                 // every wave is done with the stages
  store_tile(acc, smem, C, M, N, m0, n0, wm, wn, lane, tid);
}

// The persistent form (K a multiple of 128), one workgroup of 8 waves (two
// per SIMD) per CU, walking the tiles b, b + G, b + 2 G, ... of the
// XCD-aware order.  The waves form a 2 x 4 grid: wave (wm, wn) owns tile rows
// 128 wm .. 128 wm + 127 and columns 64 wn .. 64 wn + 63 (4 x 2 blocks of
// 32 x 32, 128 fp32 accumulators).  With two waves on each SIMD, one wave's
// MFMAs go on while the other waits on its fragment reads, DMA issue or the
// barrier; a wave tile of 128 x 64 reads 1.5 times the LDS bytes per MFMA of
// the 128 x 128 one, well inside what gfx950's LDS serves.  Both operands
// come into LDS by LDS-DMA (buffer_load ... lds, 16 bytes per lane), in the
// same swizzled layout as above.  Iteration kt multiplies stage kt % 2; its
// barrier waits for stage (kt + 1) % 2, and right after it stage kt % 2,
// which no wave reads any more, gets slice kt + 2 (in the tile's last two
// iterations, the next tile's slices 0 and 1), the 8 DMA instructions of a
// wave spread over the MFMAs of the k-step that follows.  The MFMAs take the
// weight as their first operand, so each output block comes out transposed;
// the epilogue is wave-private, through a 4 KB staging area per wave.  The
// same products are summed in the same order, so C is bit-identical to
// gemm_nt_kernel's.
constexpr int kPersThreads = 512;
constexpr int kPersWaves = kPersThreads / 64;
constexpr int kPersStg = 64;          // staging row stride (bf16): 32 x 64 per wave

__global__ __launch_bounds__(kPersThreads, 1) void gemm_nt_persistent_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, uint16_t *__restrict__ C,
    int M, int N, int K, int tiles_m, int tiles_n) {
  constexpr int BK = 64;
  constexpr int kOpElems = BM * BK;
  constexpr int kStageElems = 2 * kOpElems;                // A + B: 64 KB
  constexpr int kSegs = kOpElems * 2 / 1024 / kPersWaves;  // 1 KB segments per wave per operand
  extern __shared__ __attribute__((aligned(1024))) uint16_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int nk = K / BK;
  const int tiles = tiles_m * tiles_n;
  int lid = blockIdx.x;
  if (lid >= tiles) return;
  uint16_t *const stg = smem + 2 * kStageElems + wave * 32 * kPersStg;

  // One DMA instruction fills a 1 KB segment (8 tile rows): lane L lands at
  // byte 16 L (row L / 8, physical chunk L % 8) and fetches the logical chunk
  // the swizzle keeps there; for segment s the row's key is (L / 8) ^ (s & 1).
  // The row goes into the VGPR offset (the range-checked part), so rows past
  // M or N read as zeros; the SGPR offset carries the K position.
  const int seg_row = lane >> 3;
  const uint32_t voff_even = uint32_t(seg_row * K + ((lane & 7) ^ seg_row) * 8) * 2;
  const uint32_t voff_odd = uint32_t(seg_row * K + ((lane & 7) ^ seg_row ^ 1) * 8) * 2;
  const uint32_t seg_stride = uint32_t(8 * K) * 2;
  auto rsrc_a = [&](int tm_) {
    const int m0_ = tm_ * BM;
    return make_rsrc(A + int64_t(m0_) * K, int64_t(M - m0_) * K * 2);
  };
  auto rsrc_b = [&](int tn_) {
    const int n0_ = tn_ * BN;
    return make_rsrc(B + int64_t(n0_) * K, int64_t(N - n0_) * K * 2);
  };
  auto dma = [&](__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, int stage, int slice) {
    uint16_t *sa = smem + stage * kStageElems;
    uint16_t *sb = sa + kOpElems;
#pragma unroll
    for (int i = 0; i < kSegs; ++i) {
      const int seg = wave * kSegs + i;
      const uint32_t v = ((i & 1) ? voff_odd : voff_even) + seg * seg_stride;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, sa + seg * 512, 16, v, slice * BK * 2, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, sb + seg * 512, 16, v, slice * BK * 2, 0, 0);
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int frow = lane & 31, fhalf = lane >> 5;
  bf16x8 fa[2][4], fb[2][2];
  auto load_frags = [&](int stage, int ks, int slot) {
    const uint16_t *sa = smem + stage * kStageElems;
    const uint16_t *sb = sa + kOpElems;
    const int chunk = 2 * ks + fhalf;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      fa[slot][i] =
          *reinterpret_cast<const bf16x8 *>(sa + swz<BK>(wm * 128 + i * 32 + frow, chunk));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      fb[slot][j] =
          *reinterpret_cast<const bf16x8 *>(sb + swz<BK>(wn * 64 + j * 32 + frow, chunk));
  };
  // acc[i][j] holds the transposed 32 x 32 block: accumulator r of lane
  // (t, h) is row 128 wm + 32 i + t, column 64 wn + 32 j + 8 (r / 4) + 4 h + r % 4.
  auto mfma_block = [&](int slot) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[slot][j], fa[slot][i],
                                                            acc[i][j], 0, 0, 0);
  };
  // One k-step: 8 MFMAs with the next step's 6 fragment reads between them
  // (and, after the barrier, the wave's 8 DMA instructions).
  auto sched_reads = [&]() {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (r < 6) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
  };
  auto sched_reads_dma = [&]() {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (r < 6) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
    }
  };
  // The first three k-steps run at raised wave priority, so that the SIMD's
  // arbiter prefers the wave that is issuing MFMAs over the one that has
  // reached the barrier's side of its iteration.
  auto iteration = [&](const int stage, __amdgpu_buffer_rsrc_t ra_f, __amdgpu_buffer_rsrc_t rb_f,
                       int fill_slice) {
    __builtin_amdgcn_sched_barrier(0);
    load_frags(stage, 1, 1);
    __builtin_amdgcn_s_setprio(1);
    mfma_block(0);
    sched_reads();
    load_frags(stage, 2, 0);
    mfma_block(1);
    sched_reads();
    load_frags(stage, 3, 1);
    mfma_block(0);
    sched_reads();
    __builtin_amdgcn_s_setprio(0);
    stage_barrier<waitcnt(0, 0)>();
    __builtin_amdgcn_sched_barrier(0);
    load_frags(stage ^ 1, 0, 0);
    dma(ra_f, rb_f, stage, fill_slice);
    mfma_block(1);
    sched_reads_dma();
  };

  int tm, tn;
  tile_coords(lid, tiles_m, tiles_n, tm, tn);
  __amdgpu_buffer_rsrc_t ra = rsrc_a(tm), rb = rsrc_b(tn);
  dma(ra, rb, 0, 0);
  stage_barrier<waitcnt(0, 0)>();
  dma(ra, rb, 1, 1);
  load_frags(0, 0, 0);

  const bool vec = (N % 8) == 0;
  for (;;) {
    const int next = lid + int(gridDim.x);
    const bool has_next = next < tiles;
    int tm2 = tm, tn2 = tn;
    if (has_next) tile_coords(next, tiles_m, tiles_n, tm2, tn2);
    const __amdgpu_buffer_rsrc_t ra2 = rsrc_a(tm2), rb2 = rsrc_b(tn2);
    const int m0 = tm * BM + wm * 128, n0 = tn * BN + wn * 64;
    // After the last tile, the final iterations reload slice nk - 1, which
    // nothing reads.
    for (int kt = 0; kt < nk; kt += 2) {
      const bool last = kt + 2 == nk;
      iteration(0, last ? ra2 : ra, last ? rb2 : rb, last ? (has_next ? 0 : nk - 1) : kt + 2);
      iteration(1, last ? ra2 : ra, last ? rb2 : rb, last ? (has_next ? 1 : nk - 1) : kt + 3);
    }
    // Epilogue, per wave: 4 chunks of 32 rows x 64 columns.  A lane writes its
    // 4 consecutive columns as 8 bytes; 16-byte chunk c of staging row r sits
    // at chunk c ^ (r % 8), so the writes of 8 rows and the 16-byte reads of
    // one row spread over the banks.  A wave's LDS accesses complete in
    // order, so no barrier is needed.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16 &a = acc[i][j];
          const u32x2 v = {pack_bf16x2(a[4 * g], a[4 * g + 1]),
                           pack_bf16x2(a[4 * g + 2], a[4 * g + 3])};
          const int c = (4 * j + g) ^ (frow & 7);
          *reinterpret_cast<u32x2 *>(stg + frow * kPersStg + c * 8 + 4 * fhalf) = v;
        }
#pragma unroll
      for (int r8 = 0; r8 < 4; ++r8) {
        const int row = r8 * 8 + (lane >> 3), c = lane & 7;
        const int grow = m0 + i * 32 + row, gcol = n0 + c * 8;
        const u32x4 v =
            *reinterpret_cast<const u32x4 *>(stg + row * kPersStg + ((c ^ (row & 7)) * 8));
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
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    if (!has_next) break;
    lid = next;
    tm = tm2;
    tn = tn2;
    ra = ra2;
    rb = rb2;
  }
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));       // the last, unread reloads
}

}  // namespace

hipError_t launch_project(const uint16_t *a, const uint16_t *w, uint16_t *c, int32_t M,
                          int32_t K, int32_t N, hipStream_t stream) {
  if (project_uses_skinny(M)) return launch_project_skinny(a, w, c, M, K, N, stream);
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int tiles = tiles_m * tiles_n;
  const size_t lds_stages = size_t(2) * (BM + BN) * 64 * sizeof(uint16_t);
  // K % 128 == 0: the persistent form (two stages per unrolled step, so the
  // stage of a tile's first slice is always 0); else one tile per workgroup.
  if (K % 128 == 0) {
    const size_t lds = lds_stages + size_t(kPersWaves) * 32 * kPersStg * sizeof(uint16_t);
    const void *fn = reinterpret_cast<const void *>(&gemm_nt_persistent_kernel);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_nt_persistent_kernel, dim3(persistent_grid(tiles, stream)),
                       dim3(kPersThreads), lds, stream, a, w, c, M, N, K, tiles_m, tiles_n);
    return hipGetLastError();
  }
  const void *fn = reinterpret_cast<const void *>(&gemm_nt_kernel);
  // Set on every call: the attribute is per device, and the call is cheap.
  hipError_t e =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds_stages));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemm_nt_kernel, dim3(tiles), dim3(kThreads), lds_stages, stream, a, w, c, M,
                     N, K, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace engram
