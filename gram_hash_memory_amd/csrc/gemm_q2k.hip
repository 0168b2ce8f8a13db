// Stages 2 + 3 fused for Q2_K tables: kv = bf16(dequant(table[ids])) x wkv^T.
//
// [spark engram_v41 page, overview stages 2-3]: rows are Q2_K blocks of 84
// bytes per 256 values (ENGRAM_ROW_BYTES), dequantised to bf16 and
// multiplied by wkv.  Instead of writing the bf16 rows to HBM and reading
// them back, the projection reads the blocks themselves: A is 84 bytes per
// 256 values instead of 512.  The bf16 values it multiplies are the ones
// engram_rows produces, and every output sums the same MFMAs in the same K
// order as gemm.hip, so kv is bit-identical to rows -> project.
//
// Tile 256 x 256, each wave a band of tile rows x all 256 columns (blocks of
// v_mfma_f32_32x32x16_bf16), K in stages of BK = 64.
//  - B goes straight from global memory into its LDS stage (buffer_load ...
//    lds); every wave reads the whole B stage as fragments.
//  - A never touches LDS.  Each tile row is needed by exactly one wave, and
//    every lane decodes its own A fragments from the Q2_K block in
//    registers: lane (r, h) of the 32 x 16 fragment holds row r, values
//    8h .. 8h + 7 of the 16-value k-step.  Decoding into LDS instead would
//    add a 32 KB LDS write per stage next to the fragment reads.
//  - The persistent form runs 8 waves of 32 rows (two waves per SIMD, 128
//    accumulators each); the one-tile form 4 waves of 64 rows (256
//    accumulators in AGPRs).
// Per lane and table column (256 values = 4 stages) a row needs the block's
// 16 scale/min bytes, d/dmin, and 32 of its 64 quant bytes: value v's quant
// is byte 32 (v / 128) + v % 32 at bit 2 ((v % 128) / 32), and the lane's
// values (v % 16 in 8h .. 8h + 7) fall in the four 8-byte pieces at quant
// bytes 16 p + 8 h, p = 0..3.  The blocks of a column are loaded one column
// ahead.
// Two forms of the same K loop:
//  - gemm_q2k_persistent_kernel (even column counts): one workgroup of 8
//    waves per CU walks its share of the tiles.  The next tile's ids, its
//    first blocks and its first two B slices are fetched during the current
//    tile's last column, so the K loop runs on from tile to tile; each B
//    slice is requested in the k-step after the barrier that frees its
//    stage, a whole stage ahead of its use.  The MFMAs take wkv as their
//    first operand, so a lane ends with 4 consecutive output columns per
//    block row and writes them to a wave-private LDS staging area as 8
//    bytes; the wave then stores whole 128-byte row segments.  No workgroup
//    barrier sits in the epilogue.
//  - q2k_tile (one tile per workgroup): odd column counts, and the exact
//    recompute below.
// Both give every output the same MFMAs in the same K order as gemm.hip
// (swapping the two operands of an MFMA transposes its output block and
// leaves each dot product as it is), so kv is bit-identical to rows ->
// project.
// Values are rounded once for every finite d, dmin (q2k_decode.hpp).  The
// tiles decode with one fma per value, which is exact unless a block's d and
// dmin lie far apart; a second, small launch then checks every M-tile's
// blocks, counts the ids outside the table, and recomputes, with the exact
// group decode, the tiles of any M-tile that has such a block
// (gemm_q2k_exact_kernel).
#include <algorithm>

#include "gemm_common.hpp"
#include "q2k_decode.hpp"

namespace engram {
namespace {

using namespace gemm;
using namespace gemm::wide;

constexpr uint32_t kNoRow = 0x7FFFFFF0u;   // block offset past the table: loads read 0

// The register copy of the block parts one lane needs for one row.
struct Q2kPart {
  u32x4 sc;          // scale/min bytes 0..15 (low nibble scale, high nibble min)
  u32x2 q[4];        // quant bytes 16 p + 8 h .. + 7 of the 64
  uint32_t dd;       // fp16 d | fp16 dmin << 16
};

// A lane's parts of the block at byte offset `off` of the table.
__device__ __forceinline__ void load_part(__amdgpu_buffer_rsrc_t rt, uint32_t off, int fhalf,
                                          Q2kPart &p) {
  p.sc = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rt, off, 0, 0));
#pragma unroll
  for (int q = 0; q < 4; ++q)
    p.q[q] = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(rt, off + 16 + 16 * q + 8 * fhalf, 0, 0));
  p.dd = __builtin_amdgcn_raw_buffer_load_b32(rt, off + 80, 0, 0);
}
// The lane's A fragment of k-step ks of stage qs (values 64 qs + 16 ks .. + 15
// of the block: 16-value group 4 qs + ks), q2k_decode.hpp.
template <bool kExact>
__device__ __forceinline__ bf16x8 decode_frag(const Q2kPart &b, const int qs, const int ks) {
  const int p = 2 * (qs >> 1) + (ks & 1);
  const int shift = 4 * (qs & 1) + 2 * (ks >> 1);
  const uint32_t sm = (b.sc[qs] >> (8 * ks)) & 0xFFu;
  const Q2kPlanes pl = kExact ? q2k_group_planes_exact(b.dd, sm) : q2k_group_planes(b.dd, sm);
  return __builtin_bit_cast(bf16x8, q2k_expand8(pl, b.q[p][0], b.q[p][1], shift));
}

// One k-step of a wave with 2 x kJ blocks: 2 kJ MFMAs, the next step's kJ
// B fragment reads and 4 VALU ops (the A decode) after each MFMA.
template <int kJ>
__device__ __forceinline__ void sched_step_cols() {
#pragma unroll
  for (int r = 0; r < 2 * kJ; ++r) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if (r % 2 == 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedValu, 4, 0);
  }
}

// Columns 32 kJ part .. 32 kJ part + 32 kJ - 1 of the 256 x 256 output tile
// (tm, tn), by 4 waves of 64 rows, each with 2 x kJ blocks of accumulators
// (kJ = 8: the whole tile, 256 accumulators in AGPRs; kJ = 4: half of it,
// which leaves the registers the exact decode needs).  kExact picks the
// group decode.  Returns at once if the part lies past N.
template <bool kExact, int kJ>
__device__ __forceinline__ void q2k_tile(
    const uint8_t *__restrict__ table, int64_t num_rows, const int32_t *__restrict__ ids,
    int64_t ids_stride, const uint16_t *__restrict__ B, uint16_t *__restrict__ C,
    int M, int N, int K, int tm, int tn, int part, uint16_t *smem) {
  constexpr int kR = kRowsPerLane;                 // 32-row blocks per wave
  constexpr int kSegW = kJ * 4 / kWaves;           // B segments (8 rows) per wave per stage
  const int m0 = tm * BM, n0 = tn * BN + part * 32 * kJ;
  if (n0 >= N) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int frow = lane & 31, fhalf = lane >> 5;
  const int cols = K / ENGRAM_HEAD_DIM;
  const int nk = K / BK;

  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + int64_t(n0) * K, int64_t(N - n0) * K * 2);
  const BSegs segs = b_segs(lane, K);
  auto dma_b = [&](int stage, int slice) {
    uint16_t *sb = smem + stage * kStageElems;
#pragma unroll
    for (int i = 0; i < kSegW; ++i) {
      const int seg = wave * kSegW + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, sb + seg * 512, 16, ((i & 1) ? segs.voff_odd : segs.voff_even) + seg * segs.seg_stride,
          min(slice, nk - 1) * BK * 2, 0, 0);
    }
  };

  // ---- A: byte offsets of every (row, column) block, in LDS behind the two
  // B stages (cols <= ENGRAM_Q2K_FUSED_MAX_COLS).  Thread t resolves tile row t.
  const __amdgpu_buffer_rsrc_t rt = make_rsrc(table, num_rows * ENGRAM_Q2K_ROW_BYTES);
  uint32_t *const offs = reinterpret_cast<uint32_t *>(smem + 2 * kStageElems);
  {
    const int arow = m0 + tid;
    const bool row_ok = arow < M;
    const int32_t *id_ptr = ids + int64_t(row_ok ? arow : M - 1) * ids_stride;
    int32_t idv[ENGRAM_Q2K_FUSED_MAX_COLS];
#pragma unroll
    for (int c = 0; c < ENGRAM_Q2K_FUSED_MAX_COLS; ++c) idv[c] = c < cols ? id_ptr[c] : 0;
#pragma unroll
    for (int c = 0; c < ENGRAM_Q2K_FUSED_MAX_COLS; ++c) {
      if (c < cols) {
        const bool ok = idv[c] >= 0 && idv[c] < num_rows;
        offs[c * BM + tid] = row_ok && ok ? uint32_t(idv[c]) * ENGRAM_Q2K_ROW_BYTES : kNoRow;
      }
    }
  }
  __syncthreads();                                  // offsets of other lanes' rows

  Q2kPart blk[2][kR];
  auto load_block = [&](int set, int col) {
#pragma unroll
    for (int i = 0; i < kR; ++i)
      load_part(rt, offs[min(col, cols - 1) * BM + wave * 32 * kR + 32 * i + frow], fhalf,
                blk[set][i]);
  };

  bf16x8 fa[2][kR], fb[2][kJ];
  auto decode_a = [&](int set, const int qs, const int ks, int slot) {
#pragma unroll
    for (int i = 0; i < kR; ++i) fa[slot][i] = decode_frag<kExact>(blk[set][i], qs, ks);
  };

  f32x16 acc[kR][kJ];
#pragma unroll
  for (int i = 0; i < kR; ++i)
#pragma unroll
    for (int j = 0; j < kJ; ++j) acc[i][j] = f32x16{};

  auto load_b = [&](int stage, int ks, int slot) {
    const uint16_t *sb = smem + stage * kStageElems;
    const int chunk = 2 * ks + fhalf;
#pragma unroll
    for (int j = 0; j < kJ; ++j)
      fb[slot][j] = *reinterpret_cast<const bf16x8 *>(sb + swz<BK>(j * 32 + frow, chunk));
  };
  // Column-block-major: B fragment j, read during the previous k-step in
  // order j, is first used 2 j MFMAs into this one, so every read gets the
  // same 16-MFMA lead (row-major order would give fragment 7 only 9).
  auto mfma_block = [&](int slot) {
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
      for (int i = 0; i < kR; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j],
                                                            acc[i][j], 0, 0, 0);
  };

  // Iteration kt multiplies stage kt % 2 and fills stage (kt + 1) % 2, which
  // every wave finished reading before the previous barrier; j = kt % 8 fixes
  // the register sets at compile time:
  //  - B slice kt + 1 is requested into its LDS stage first thing;
  //  - the MFMAs of stage kt are column kt / 4, quarter kt % 4, from block set
  //    (kt / 4) % 2;
  //  - when kt % 4 == 0 (column kt / 4 starts), the blocks of column kt / 4 + 1
  //    are requested into the other set, after the B segments (12 loads);
  //  - before the barrier, vmcnt lets only those 12 block loads stay in
  //    flight: the B segments (older) have then landed in LDS.
  // `prefetch` is false for the last column: nothing would use those blocks,
  // the compiler drops loads whose results are dead, and a vmcnt that counts
  // them would then let the B segments stay in flight, so that iteration
  // waits for everything.
  // Scheduling fences around the loads keep them at the top of the iteration
  // (the compiler would otherwise sink them towards their first use, which
  // shortens the prefetch distance), and keep work of a later iteration (such
  // as the fp16 d of a block still in flight) from being hoisted into this
  // one, where it would wait for the load.
  auto iteration = [&](int kt, const int j, const bool prefetch) {
    const int stage = j & 1;                         // kt % 2
    const int set = (j >> 2) & 1, qs = j & 3;
    __builtin_amdgcn_sched_barrier(0);
    dma_b(stage ^ 1, kt + 1);
    __builtin_amdgcn_sched_barrier(0);               // the counted wait needs the DMA first
    if (qs == 0 && prefetch) load_block(set ^ 1, kt / 4 + 1);
    __builtin_amdgcn_sched_barrier(0);
    load_b(stage, 1, 1);
    decode_a(set, qs, 1, 1);
    mfma_block(0);
    sched_step_cols<kJ>();
    load_b(stage, 2, 0);
    decode_a(set, qs, 2, 0);
    mfma_block(1);
    sched_step_cols<kJ>();
    load_b(stage, 3, 1);
    decode_a(set, qs, 3, 1);
    mfma_block(0);
    sched_step_cols<kJ>();
    if (qs == 0 && prefetch) stage_barrier<waitcnt(6 * kR, 0)>();
    else stage_barrier<waitcnt(0, 0)>();
    load_b(stage ^ 1, 0, 0);
    decode_a(((j + 1) >> 2) & 1, (j + 1) & 3, 0, 0);
    mfma_block(1);
    sched_step_cols<kJ>();
  };

  // Prologue: stage 0 gets B slice 0, the lanes the blocks of column 0 and
  // the fragments of k-step 0.  (Iteration 0 then requests B slice 1 and the
  // blocks of column 1.)
  load_block(0, 0);
  dma_b(0, 0);
  stage_barrier<waitcnt(0, 0)>();
  load_b(0, 0, 0);
  decode_a(0, 0, 0, 0);

  int kt = 0;
  for (; kt + 7 < nk; kt += 8) {
    iteration(kt + 0, 0, true);
    iteration(kt + 1, 1, true);
    iteration(kt + 2, 2, true);
    iteration(kt + 3, 3, true);
    iteration(kt + 4, 4, true);
    iteration(kt + 5, 5, true);
    iteration(kt + 6, 6, true);
    iteration(kt + 7, 7, true);
  }
  if (kt < nk) {              // nk % 8 == 4 (K is a multiple of 256): the last column
    iteration(kt + 0, 0, false);
    iteration(kt + 1, 1, false);
    iteration(kt + 2, 2, false);
    iteration(kt + 3, 3, false);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
  __syncthreads();                                 // every wave is done with the stages
  store_tile_blocks<kR, kJ, kThreads, 32 * kJ>(acc, smem, C, M, N, m0, n0, wave * 64, 0, lane,
                                              tid);
}

__global__ __launch_bounds__(kThreads, 1) void gemm_q2k_kernel(
    const uint8_t *__restrict__ table, int64_t num_rows, const int32_t *__restrict__ ids,
    int64_t ids_stride, const uint16_t *__restrict__ B, uint16_t *__restrict__ C,
    int M, int N, int K, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(1024))) uint16_t smem[];
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  q2k_tile<false, kNJ>(table, num_rows, ids, ids_stride, B, C, M, N, K, tm, tn, 0, smem);
}

// The persistent form (cols even): one workgroup of 8 waves (two per SIMD)
// per CU.  Workgroup b runs the tiles whose ids in the XCD-aware order
// (tile_coords) are b, b + G, b + 2 G, ... (G = grid size, a multiple of 8
// when a workgroup has more than one tile, so all of them lie in its XCD's
// run).  Wave w owns tile rows 32 w .. 32 w + 31 and all 256 columns: it
// decodes one A fragment per k-step (the same VALU work per MFMA as the
// 4-wave form) and reads all 8 B fragments, and while one wave of a SIMD
// waits on its reads, its DMA issue or the barrier, the other's MFMAs go on.
// LDS: the two B stages (64 KB), the current tile's ids (cols x 256 int32,
// brought in by waves 0-3 and read by every wave after the next barrier), and
// a 4.5 KB staging area per wave.
constexpr int kPersThreads = 512;
constexpr int kPersWaves = kPersThreads / 64;
constexpr int kPersSegs = kStageElems * 2 / 1024 / kPersWaves;   // B segments per wave: 4

__global__ __launch_bounds__(kPersThreads, 1) void gemm_q2k_persistent_kernel(
    const uint8_t *__restrict__ table, int64_t num_rows, const int32_t *__restrict__ ids,
    int64_t ids_stride, const uint16_t *__restrict__ B, uint16_t *__restrict__ C,
    int M, int N, int K, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(1024))) uint16_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int frow = lane & 31, fhalf = lane >> 5;
  const int cols = K / ENGRAM_HEAD_DIM;
  const int nk = K / BK;
  const int tiles = tiles_m * tiles_n;
  int lid = blockIdx.x;
  if (lid >= tiles) return;

  int32_t *const ids_lds = reinterpret_cast<int32_t *>(smem + 2 * kStageElems);
  uint16_t *const stg = smem + 2 * kStageElems + cols * BM * 2 + wave * 32 * kStgStride;
  // B slice `slice` into stage `stage`: this wave's 4 segments of 1 KB (8
  // rows each; segment 4 w + i, whose swizzle key parity is i & 1).
  const BSegs segs = b_segs(lane, K);
  auto dma_b = [&](__amdgpu_buffer_rsrc_t rb, int stage, int slice) {
    uint16_t *sb = smem + stage * kStageElems;
#pragma unroll
    for (int i = 0; i < kPersSegs; ++i) {
      const int seg = wave * kPersSegs + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, sb + seg * 512, 16, ((i & 1) ? segs.voff_odd : segs.voff_even) + seg * segs.seg_stride,
          slice * BK * 2, 0, 0);
    }
  };
  // The ids of tile rows 64 w + lane, all columns, into ids_lds (waves 0-3,
  // one LDS-DMA instruction per column; rows past M read 0 and are never
  // stored).  The other waves see them after the issuing waves' next
  // barrier with vmcnt 0.
  auto dma_ids = [&](int tm_) {
    if (wave >= 4) return;
    const int m0_ = tm_ * BM;
    const __amdgpu_buffer_rsrc_t ri =
        make_rsrc(ids + int64_t(m0_) * ids_stride, int64_t(min(BM, M - m0_)) * ids_stride * 4);
    const uint32_t voff = uint32_t((wave * 64 + lane) * ids_stride) * 4;
    for (int c = 0; c < cols; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ri, ids_lds + c * BM + wave * 64, 4,
                                               voff + uint32_t(c) * 4, 0, 0, 0);
  };

  const __amdgpu_buffer_rsrc_t rt = make_rsrc(table, num_rows * ENGRAM_Q2K_ROW_BYTES);
  Q2kPart blk[2];
  // An id outside the table reads the bytes past it: zeros.
  auto load_block = [&](int set, int col) {
    const int32_t id = ids_lds[col * BM + wave * 32 + frow];
    const uint32_t off =
        (id >= 0 && id < num_rows) ? uint32_t(id) * ENGRAM_Q2K_ROW_BYTES : kNoRow;
    load_part(rt, off, fhalf, blk[set]);
  };

  bf16x8 fa[2], fb[2][kNJ];
  auto decode_a = [&](int set, const int qs, const int ks, int slot) {
    fa[slot] = decode_frag<false>(blk[set], qs, ks);
  };

  // acc[0][j] holds the transposed 32 x 32 output block: accumulator r of
  // lane (t, h) is tile row 32 w + t, column 32 j + 8 (r / 4) + 4 h + r % 4.
  f32x16 acc[1][kNJ];
#pragma unroll
  for (int j = 0; j < kNJ; ++j) acc[0][j] = f32x16{};

  auto load_b = [&](int stage, int ks, int slot) {
    load_b_frags(smem + stage * kStageElems, frow, fhalf, ks, fb[slot]);
  };
  auto mfma_block = [&](int slot) {
#pragma unroll
    for (int j = 0; j < kNJ; ++j)
      acc[0][j] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[slot][j], fa[slot], acc[0][j], 0, 0, 0);
  };
  // One k-step: 8 MFMAs, each followed by one of the next step's 8 B
  // fragment reads and 4 VALU ops of its A decode (about 28).
  auto sched_step = [&]() {
#pragma unroll
    for (int r = 0; r < kNJ; ++r) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, 4, 0);
    }
  };

  // Iteration kt of the current tile multiplies stage kt % 2 (j = kt % 8
  // fixes the register sets at compile time, as in q2k_tile):
  //  - at kt % 4 == 0 the block of column (kt / 4 + 1) % cols is requested
  //    (6 loads); after a tile's last column that is column 0 of the next
  //    tile, whose ids are in ids_lds by then;
  //  - the barrier waits for the B slice of this stage (requested one
  //    iteration earlier) and lets only those 6 block loads stay in flight;
  //  - after it, stage kt % 2, which no wave reads any more, gets the slice
  //    `fill_slice` of resource rb_fill (slice kt + 2, or one of the next
  //    tile's first two slices), its 4 DMA instructions spread over the last
  //    k-step.
  auto iteration = [&](int kt, const int j, __amdgpu_buffer_rsrc_t rb_fill, int fill_slice) {
    const int stage = j & 1;
    const int set = (j >> 2) & 1, qs = j & 3;
    __builtin_amdgcn_sched_barrier(0);
    if (qs == 0) {
      const int col = kt / 4 + 1;
      load_block(set ^ 1, col == cols ? 0 : col);
    }
    __builtin_amdgcn_sched_barrier(0);
    load_b(stage, 1, 1);
    decode_a(set, qs, 1, 1);
    mfma_block(0);
    sched_step();
    load_b(stage, 2, 0);
    decode_a(set, qs, 2, 0);
    mfma_block(1);
    sched_step();
    load_b(stage, 3, 1);
    decode_a(set, qs, 3, 1);
    mfma_block(0);
    sched_step();
    if (qs == 0) stage_barrier<waitcnt(6, 0)>();
    else stage_barrier<waitcnt(0, 0)>();
    __builtin_amdgcn_sched_barrier(0);
    load_b(stage ^ 1, 0, 0);
    decode_a(((j + 1) >> 2) & 1, (j + 1) & 3, 0, 0);
    dma_b(rb_fill, stage, fill_slice);
    mfma_block(1);
#pragma unroll
    for (int r = 0; r < kNJ; ++r) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (r < kPersSegs) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, 4, 0);
    }
  };

  // Prologue of the first tile: its ids, the blocks of column 0 and B
  // slice 0, then slice 1 in flight.
  int tm, tn;
  tile_coords(lid, tiles_m, tiles_n, tm, tn);
  __amdgpu_buffer_rsrc_t rb = b_rsrc(B, N, K, tn);
  dma_ids(tm);
  stage_barrier<waitcnt(0, 0)>();
  load_block(0, 0);
  dma_b(rb, 0, 0);
  stage_barrier<waitcnt(0, 0)>();
  dma_b(rb, 1, 1);
  load_b(0, 0, 0);
  decode_a(0, 0, 0, 0);

  for (;;) {
    const int next = lid + int(gridDim.x);
    const bool has_next = next < tiles;
    int tm2 = tm, tn2 = tn;
    if (has_next) tile_coords(next, tiles_m, tiles_n, tm2, tn2);
    const __amdgpu_buffer_rsrc_t rb2 = b_rsrc(B, N, K, tn2);
    const int m0 = tm * BM, n0 = tn * BN;

    // Two columns per trip (cols is even).  In the last trip, iterations 6
    // and 7 fill the stages with the next tile's slices 0 and 1 (or, after
    // the last tile, reload slice nk - 1, which nothing reads).
    for (int kt = 0; kt < nk; kt += 8) {
      const bool last = kt + 8 == nk;
      iteration(kt + 0, 0, rb, kt + 2);
      // Every wave read this tile's ids for the last time before the barrier
      // just passed (the blocks of column cols - 1); the next tile's replace
      // them and are visible after the next barrier, whose vmcnt is 0.
      if (last && has_next) dma_ids(tm2);
      iteration(kt + 1, 1, rb, kt + 3);
      iteration(kt + 2, 2, rb, kt + 4);
      iteration(kt + 3, 3, rb, kt + 5);
      iteration(kt + 4, 4, rb, kt + 6);
      iteration(kt + 5, 5, rb, kt + 7);
      iteration(kt + 6, 6, last ? rb2 : rb, last ? (has_next ? 0 : nk - 1) : kt + 8);
      iteration(kt + 7, 7, last ? rb2 : rb, last ? (has_next ? 1 : nk - 1) : kt + 9);
    }

    // Epilogue, per wave: its 32 rows in 4 chunks of 64 columns.
    store_wave_transposed<1, kNJ, 1>(acc, stg, C, M, N, m0 + wave * 32, n0, lane);
#pragma unroll
    for (int j = 0; j < kNJ; ++j) acc[0][j] = f32x16{};
    if (!has_next) break;
    lid = next;
    tm = tm2;
    tn = tn2;
    rb = rb2;
  }
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));       // the last, unread B reload
}

// Runs after the tiles on the same stream.  Workgroup (tm, g) checks the
// d/dmin of every block of M-tile tm (the g == 0 workgroups also count the
// ids outside the table, once per (token, column)); if any block lies
// outside the one-fma range (q2k_fp32_exact), it recomputes tiles (tm, g),
// (tm, g + split), ... with the exact group decode, overwriting what the
// first launch stored, one half of the tile's columns at a time (the exact
// decode needs more registers than the one-fma decode; 128 accumulators per
// wave leave room for them).  Otherwise it exits after the check.
__global__ __launch_bounds__(kThreads, 1) void gemm_q2k_exact_kernel(
    const uint8_t *__restrict__ table, int64_t num_rows, const int32_t *__restrict__ ids,
    int64_t ids_stride, const uint16_t *__restrict__ B, uint16_t *__restrict__ C,
    int M, int N, int K, int tiles_n, int split, int32_t *__restrict__ bad_ids) {
  extern __shared__ __attribute__((aligned(1024))) uint16_t smem[];
  // Workgroups are dealt round-robin to the 8 XCDs: with tm = id % tiles_m,
  // the `split` workgroups of an M-tile share an XCD (when tiles_m % 8 == 0)
  // and so its L2, and fetch the M-tile's d/dmin words from HBM once.
  const int tiles_m = int(gridDim.x) / split;
  const int tm = int(blockIdx.x) % tiles_m, g = int(blockIdx.x) / tiles_m;
  const int cols = K / ENGRAM_HEAD_DIM;
  // The tile's (row, column) pairs in row-major order, thread t taking pairs
  // t, t + 256, ... (so a wave's id loads are contiguous runs): all the ids,
  // then all their blocks' d/dmin words, each batch in flight at once (an id
  // outside the table, or a row past M, reads the word past the table: 0).
  const __amdgpu_buffer_rsrc_t rt = make_rsrc(table, num_rows * ENGRAM_Q2K_ROW_BYTES);
  int32_t idv[ENGRAM_Q2K_FUSED_MAX_COLS];
  bool pair_ok[ENGRAM_Q2K_FUSED_MAX_COLS];
#pragma unroll
  for (int i = 0; i < ENGRAM_Q2K_FUSED_MAX_COLS; ++i) {
    const int pair = i * kThreads + int(threadIdx.x);
    const int row = tm * BM + pair / max(cols, 1), c = pair % max(cols, 1);
    pair_ok[i] = i < cols && row < M;
    idv[i] = pair_ok[i] ? ids[int64_t(row) * ids_stride + c] : -1;
  }
  uint32_t ddv[ENGRAM_Q2K_FUSED_MAX_COLS];
  int bad = 0;
#pragma unroll
  for (int i = 0; i < ENGRAM_Q2K_FUSED_MAX_COLS; ++i) {
    const bool ok = idv[i] >= 0 && idv[i] < num_rows;
    bad += pair_ok[i] && !ok;
    ddv[i] = __builtin_amdgcn_raw_buffer_load_b32(
        rt, (ok ? uint32_t(idv[i]) * ENGRAM_Q2K_ROW_BYTES : kNoRow) + 80, 0, 0);
  }
  if (bad && g == 0 && bad_ids) atomicAdd(bad_ids, bad);
  bool fast = true;
#pragma unroll
  for (int c = 0; c < ENGRAM_Q2K_FUSED_MAX_COLS; ++c) fast &= q2k_fp32_exact(ddv[c]);
  if (__syncthreads_and(fast)) return;
  for (int tn = g; tn < tiles_n; tn += split)
    for (int part = 0; part < 2; ++part) {
      __syncthreads();                             // the previous part is done with the LDS
      q2k_tile<true, kNJ / 2>(table, num_rows, ids, ids_stride, B, C, M, N, K, tm, tn, part,
                              smem);
    }
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
  if (project_q2k_skinny_supported(M, cols))
    return launch_project_q2k_skinny(table, num_rows, ids, ids_token_stride, cols, w, c, M, N,
                                     bad_ids, stream);
  const int K = cols * ENGRAM_HEAD_DIM;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  // Per-tile kernels (odd column counts, the exact recompute): the two B
  // stages and the block offsets, or the output tile in the epilogue.
  const size_t lds_loop = size_t(2) * kStageElems * sizeof(uint16_t) +
                         size_t(cols) * kThreads * sizeof(uint32_t);
  const size_t lds_epilogue = size_t(BM) * BN * sizeof(uint16_t);
  const size_t lds = lds_loop > lds_epilogue ? lds_loop : lds_epilogue;
  // Persistent kernel: the two B stages, the ids and 8 staging areas.
  const size_t lds_pers = size_t(2) * kStageElems * sizeof(uint16_t) +
                          size_t(cols) * BM * sizeof(int32_t) +
                          size_t(kPersWaves) * 32 * kStgStride * sizeof(uint16_t);
  const bool persistent = cols % 2 == 0;
  const void *tile_fn = persistent ? reinterpret_cast<const void *>(&gemm_q2k_persistent_kernel)
                                   : reinterpret_cast<const void *>(&gemm_q2k_kernel);
  hipError_t e = hipFuncSetAttribute(tile_fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     int(persistent ? lds_pers : lds));
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_q2k_exact_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  const int tiles = tiles_m * tiles_n;
  if (persistent) {
    hipLaunchKernelGGL(gemm_q2k_persistent_kernel, dim3(persistent_grid(tiles, stream)),
                       dim3(kPersThreads), lds_pers, stream, table, num_rows, ids, ids_token_stride, w,
                       c, M, N, K, tiles_m, tiles_n);
  } else {
    hipLaunchKernelGGL(gemm_q2k_kernel, dim3(tiles), dim3(kThreads), lds, stream, table,
                       num_rows, ids, ids_token_stride, w, c, M, N, K, tiles_m, tiles_n);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // About one checking workgroup per CU; each recomputes every split-th tile
  // of its M-tile when that M-tile needs the exact decode.
  const int split = std::max(1, std::min(tiles_n, (256 + tiles_m - 1) / tiles_m));
  hipLaunchKernelGGL(gemm_q2k_exact_kernel, dim3(tiles_m * split), dim3(kThreads), lds, stream,
                     table, num_rows, ids, ids_token_stride, w, c, M, N, K, tiles_n, split,
                     bad_ids);
  return hipGetLastError();
}

}  // namespace engram
