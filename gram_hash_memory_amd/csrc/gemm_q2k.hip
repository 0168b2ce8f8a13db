// Stages 2 + 3 fused for Q2_K tables: kv = bf16(dequant(table[ids])) x wkv^T.
//
// [spark engram_v41 page, overview stages 2-3]: rows are Q2_K blocks of 84
// bytes per 256 values (ENGRAM_ROW_BYTES), dequantised to bf16 and
// multiplied by wkv.  Instead of writing the bf16 rows to HBM and reading
// them back, the projection reads the blocks themselves.  A is then 84 bytes
// per 256 values instead of 512, which cuts the bytes each workgroup pulls
// through L2 by about a third; the bf16 values it multiplies are the same
// ones engram_rows produces, so kv is bit-identical to rows -> project.
//
// Same tiling as gemm.hip (256 x 256 tile, 4 waves of 128 x 128, two LDS
// stages of BK = 64).  B goes straight from global memory into its LDS stage
// (buffer_load ... lds, one stage ahead): that drops the VGPR staging, its LDS
// stores and their waits, which in this kernel cost more than the LDS-DMA
// path's lower raw rate.  For A, thread t owns tile row t.  The 84-byte block of row t for table column c (K range
// 256c .. 256c + 255) sits in 21 VGPRs: it is loaded when column c - 1
// starts, and its id one column earlier still.  Every stage, each thread
// decodes its row's 64 values straight into the LDS A tile.  A stage spans
// values 64q .. 64q + 63 of the block; they need the block's 32 quant bytes of
// half q / 2 at two bit shifts, its 4 scale/min bytes q * 4 .. q * 4 + 3, and d/dmin.
#include "gemm_common.hpp"

namespace engram {
namespace {

using namespace gemm;

constexpr int kBlockDwords = ENGRAM_Q2K_ROW_BYTES / 4;   // 21
constexpr uint32_t kNoRow = 0x7FFFFFF0u;   // block offset past the table: loads read 0

__device__ __forceinline__ float half_bits_to_float(uint32_t h16) {
  return float(__builtin_bit_cast(_Float16, uint16_t(h16)));
}

__global__ __launch_bounds__(kThreads, 1) void gemm_q2k_kernel(
    const uint8_t *__restrict__ table, int64_t num_rows, const int32_t *__restrict__ ids,
    int64_t ids_stride, const uint16_t *__restrict__ B, uint16_t *__restrict__ C,
    int M, int N, int K, int tiles_m, int tiles_n, int32_t *__restrict__ bad_ids) {
  constexpr int BK = 64;
  constexpr int kStageElems = (BM + BN) * BK;
  constexpr int kChunks = BK / 8;
  constexpr int kSegs = BN * BK * 2 / 1024 / kWaves;   // 1 KB B segments per wave per stage: 8
  extern __shared__ __attribute__((aligned(1024))) uint16_t smem[];

  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int cols = K / ENGRAM_HEAD_DIM;
  const int nk = K / BK;

  // ---- B: global -> LDS by LDS-DMA.  One instruction fills a 1 KB segment
  // (8 tile rows); lane L lands at byte 16 L, i.e. row L / 8 of the segment,
  // physical chunk L % 8, and fetches the logical chunk the swizzle keeps
  // there.  For segment s the swizzle key of that row is (L / 8) ^ (s & 1).
  // Rows past N read as zeros (the resource starts at the tile's first row,
  // and the row is part of the VGPR offset, the range-checked part; the
  // SGPR offset only carries the K position).
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + int64_t(n0) * K, int64_t(N - n0) * K * 2);
  const int seg_row = lane >> 3;
  const uint32_t voff_even = uint32_t(seg_row * K + ((lane & 7) ^ seg_row) * 8) * 2;
  const uint32_t voff_odd = uint32_t(seg_row * K + ((lane & 7) ^ seg_row ^ 1) * 8) * 2;
  const uint32_t seg_stride = uint32_t(8 * K) * 2;
  auto dma_b = [&](int stage, int slice) {
    const int k0 = min(slice, nk - 1) * BK;
    uint16_t *sb = smem + stage * kStageElems + BM * BK;
#pragma unroll
    for (int i = 0; i < kSegs; ++i) {
      const int seg = wave * kSegs + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, sb + seg * 512, 16,
                                               ((i & 1) ? voff_odd : voff_even) + seg * seg_stride,
                                               k0 * 2, 0, 0);
    }
  };

  // ---- A: the Q2_K block of tile row `tid`, one table column at a time.
  // The byte offset of every (row, column) block is resolved once, before the
  // K loop, into LDS behind the two stages (cols <= ENGRAM_Q2K_FUSED_MAX_COLS):
  // the loop then reads an offset from LDS instead of an id from global
  // memory, and ids outside the table are counted here, once.
  const int arow = m0 + tid;
  const bool row_ok = arow < M;
  const __amdgpu_buffer_rsrc_t rt = make_rsrc(table, num_rows * ENGRAM_Q2K_ROW_BYTES);
  uint32_t *const offs = reinterpret_cast<uint32_t *>(smem + 2 * kStageElems);
  {
    const int32_t *id_ptr = ids + int64_t(row_ok ? arow : M - 1) * ids_stride;
    int32_t idv[ENGRAM_Q2K_FUSED_MAX_COLS];
#pragma unroll
    for (int c = 0; c < ENGRAM_Q2K_FUSED_MAX_COLS; ++c) idv[c] = c < cols ? id_ptr[c] : 0;
    int bad = 0;
#pragma unroll
    for (int c = 0; c < ENGRAM_Q2K_FUSED_MAX_COLS; ++c) {
      if (c < cols) {
        const bool ok = idv[c] >= 0 && idv[c] < num_rows;
        bad += row_ok && !ok;
        offs[c * kThreads + tid] =
            row_ok && ok ? uint32_t(idv[c]) * ENGRAM_Q2K_ROW_BYTES : kNoRow;
      }
    }
    if (bad && tn == 0 && bad_ids) atomicAdd(bad_ids, bad);
  }
  uint32_t blk[2][kBlockDwords];
  auto load_block = [&](int set, int col) {
    const uint32_t off = offs[min(col, cols - 1) * kThreads + tid];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const u32x4 v = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rt, off + 16 * i, 0, 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) blk[set][4 * i + e] = v[e];
    }
    blk[set][20] = __builtin_amdgcn_raw_buffer_load_b32(rt, off + 80, 0, 0);
  };
  // Values 64q .. 64q + 63 of the block in register set `set` -> LDS A tile of `stage`.
  //
  // Inside a 16-value group the scale and min are fixed, so a value takes one
  // of only four bf16 results, bf16(q * dl - ml) for q = 0..3.  They are
  // computed once per group (in fp32, with the same fma and rounding as
  // engram_rows) and kept as two byte planes, lo = the four low bytes and
  // hi = the four high bytes.  Every output pair is then one v_perm_b32 of
  // (hi, lo) whose selector bytes are q_a, q_a + 4, q_b, q_b + 4, and the
  // selectors of four values are two more v_perm_b32 of (m | 0x04040404, m),
  // m being their four 2-bit quants, one per byte.
  // Groups g0 .. g1 - 1 of the four 16-value groups of the stage.
  auto decode_a = [&](int set, const int q, int stage, const int g0, const int g1) {
    uint16_t *sa = smem + stage * kStageElems;
    const uint32_t scw = blk[set][q];                    // scale/min bytes 4q .. 4q + 3
    const float d = half_bits_to_float(blk[set][20] & 0xFFFFu);
    const float dmin = half_bits_to_float(blk[set][20] >> 16);
    const int h = q >> 1, s0 = 4 * (q & 1);
#pragma unroll
    for (int g = g0; g < g1; ++g) {                      // 16-value group inside the stage
      const uint32_t sm = (scw >> (8 * g)) & 0xFFu;
      const float dl = d * float(sm & 0xFu), ml = dmin * float(sm >> 4);
      const uint32_t p01 = pack_bf16x2(fmaf(0.0f, dl, -ml), fmaf(1.0f, dl, -ml));
      const uint32_t p23 = pack_bf16x2(fmaf(2.0f, dl, -ml), fmaf(3.0f, dl, -ml));
      const uint32_t lo = __builtin_amdgcn_perm(p23, p01, 0x06040200u);
      const uint32_t hi = __builtin_amdgcn_perm(p23, p01, 0x07050301u);
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {                   // 8-value chunk c of the stage
        const int c = 2 * g + cc;
        const int shift = s0 + 2 * (c >> 2);
        u32x4 v;
#pragma unroll
        for (int w = 0; w < 2; ++w) {                    // 4 quants per dword
          const uint32_t m = (blk[set][4 + 8 * h + 2 * (c & 3) + w] >> shift) & 0x03030303u;
          const uint32_t m4 = m | 0x04040404u;
          v[2 * w] = __builtin_amdgcn_perm(hi, lo, __builtin_amdgcn_perm(m4, m, 0x05010400u));
          v[2 * w + 1] = __builtin_amdgcn_perm(hi, lo, __builtin_amdgcn_perm(m4, m, 0x07030602u));
        }
        *reinterpret_cast<u32x4 *>(sa + swz<BK>(tid, c)) = v;
      }
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

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
  auto sched_reads = [&]() {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
    }
  };
  // A sub-step that also decodes half a stage of A (about 85 VALU ops and 4
  // LDS writes): a wave issues one instruction per cycle, so the VALU work is
  // spread between the MFMAs, each of which keeps the matrix core busy for
  // 32 cycles while the next few VALU ops issue.  Bunched up, it would leave
  // the matrix core idle for the whole burst.
  auto sched_reads_decode = [&]() {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (r % 2 == 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, 6, 0);
      if (r % 4 == 3) __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
    }
  };

  // Iteration kt multiplies stage kt % 2 and fills stage (kt + 1) % 2, which
  // every wave finished reading before the previous barrier; j = kt % 8 fixes
  // the register sets at compile time:
  //  - B slice kt + 1 is requested into its LDS stage first thing;
  //  - A stage kt + 1 is column (kt + 1) / 4, quarter (kt + 1) % 4, decoded
  //    from block set ((kt + 1) / 4) % 2;
  //  - when kt % 4 == 0 (column m = kt / 4 starts), the block of column m + 1
  //    is requested, after the B segments (6 loads);
  //  - before the barrier, vmcnt lets only those 6 block loads stay in
  //    flight: the B segments (older) have then landed in LDS.
  // Scheduling fences around the loads keep them at the top of the iteration
  // (the compiler would otherwise sink them towards their first use, which
  // shortens the prefetch distance), and keep work of a later iteration (such
  // as the fp16 d of a block still in flight) from being hoisted into this
  // one, where it would wait for the load.
  auto iteration = [&](int kt, const int j) {
    const int stage = j & 1;                         // kt % 2
    __builtin_amdgcn_sched_barrier(0);
    dma_b(stage ^ 1, kt + 1);
    if (j % 4 == 0) load_block(((j / 4) + 1) & 1, kt / 4 + 1);
    __builtin_amdgcn_sched_barrier(0);
    load_frags(stage, 1, 1);
    mfma_block(0);
    decode_a(((j + 1) / 4) & 1, (j + 1) % 4, stage ^ 1, 0, 2);
    sched_reads_decode();
    load_frags(stage, 2, 0);
    mfma_block(1);
    decode_a(((j + 1) / 4) & 1, (j + 1) % 4, stage ^ 1, 2, 4);
    sched_reads_decode();
    load_frags(stage, 3, 1);
    mfma_block(0);
    sched_reads();
    if (j % 4 == 0) stage_barrier<waitcnt(6, 0)>();
    else stage_barrier<waitcnt(0, 0)>();
    load_frags(stage ^ 1, 0, 0);
    mfma_block(1);
    sched_reads();
  };

  // Prologue: stage 0 gets B slice 0 and A quarter 0 of column 0.  (Iteration
  // 0 then requests B slice 1 and the block of column 1.)
  load_block(0, 0);
  dma_b(0, 0);
  decode_a(0, 0, 0, 0, 4);
  stage_barrier<waitcnt(0, 0)>();
  load_frags(0, 0, 0);

  int kt = 0;
  for (; kt + 7 < nk; kt += 8) {
    iteration(kt + 0, 0);
    iteration(kt + 1, 1);
    iteration(kt + 2, 2);
    iteration(kt + 3, 3);
    iteration(kt + 4, 4);
    iteration(kt + 5, 5);
    iteration(kt + 6, 6);
    iteration(kt + 7, 7);
  }
  if (kt < nk) {                                   // nk % 8 == 4 (K is a multiple of 256)
    iteration(kt + 0, 0);
    iteration(kt + 1, 1);
    iteration(kt + 2, 2);
    iteration(kt + 3, 3);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
  __syncthreads();                                 // every wave is done with the stages
  store_tile(acc, smem, C, M, N, m0, n0, wm, wn, lane, tid);
}

}  // namespace

static_assert(ENGRAM_Q2K_FUSED_MAX_BYTES + 128 <= int64_t(kNoRow),
              "a missing row's offset must stay past every table byte");

bool project_q2k_supported(int64_t num_rows, int32_t cols) {
  return num_rows * ENGRAM_Q2K_ROW_BYTES <= ENGRAM_Q2K_FUSED_MAX_BYTES &&
         cols <= ENGRAM_Q2K_FUSED_MAX_COLS;
}

hipError_t launch_project_q2k(const uint8_t *table, int64_t num_rows, const int32_t *ids,
                              int64_t ids_token_stride, int32_t cols, const uint16_t *w,
                              uint16_t *c, int32_t M, int32_t N, int32_t *bad_ids,
                              hipStream_t stream) {
  const int K = cols * ENGRAM_HEAD_DIM;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const size_t lds = size_t(2) * (BM + BN) * 64 * sizeof(uint16_t) +
                    size_t(cols) * kThreads * sizeof(uint32_t);
  const void *fn = reinterpret_cast<const void *>(&gemm_q2k_kernel);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemm_q2k_kernel, dim3(tiles_m * tiles_n), dim3(kThreads), lds, stream,
                     table, num_rows, ids, ids_token_stride, w, c, M, N, K, tiles_m, tiles_n,
                     bad_ids);
  return hipGetLastError();
}

}  // namespace engram
