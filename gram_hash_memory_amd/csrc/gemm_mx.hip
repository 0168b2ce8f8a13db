// Stages 2 + 3 for FP8 tables as one MXFP8 projection:
//   kv = bf16( sum_k a[t, k] * w[n, k] ),
// a = the raw FP8 rows of the table (E4M3 codes, one E8M0 scale per 32
// values), w = an MXFP8 copy of wkv (engram_quantize_mxfp8).
//
// [vLLM engram page, EngramBatch / wkv_input]: an FP8 table row already is a
// run of MX blocks, so the block-scaled matrix cores can take it as it is
// stored; the vLLM path feeds the same blocks to an MXFP8 WKV GEMM.  On
// gfx950 that is v_mfma_scale_f32_32x32x64_f8f6f4: 32 x 32 outputs, 64 k per
// instruction, each lane's operand bytes scaled by one E8M0 byte of its own.
//
// Tiling: 256 x 256 output tile per workgroup, 4 waves of 128 x 128, K in
// stages of 128 values (128 bytes per operand row, the same LDS footprint per
// stage as the bf16 kernels' 64).  Every operand byte reaches LDS by DMA:
//  - A rows are gathered straight from the table: each lane owns one 16-byte
//    chunk of a tile row and loads it with global_load_lds through a 64-bit
//    address (tables may exceed the 4 GB a buffer descriptor can span); an id
//    outside the table, or a row past T, points at a zero row;
//  - B and both scale vectors come by buffer_load ... lds.
// A stage's LDS is free again once every wave has read its fragments into
// registers, which is before the middle barrier of the iteration that
// multiplies it; the DMA for the stage after next starts right there, one
// full stage ahead of its use.
//
// MFMA operand layout (32x32x64, 8-bit formats): lane l = 32 g + i holds row
// (A) or column (B) i, bytes 0..15 = k 16 g .. 16 g + 15 and bytes 16..31 =
// k 32 + 16 g .. 32 + 16 g + 15 of the instruction's 64; its scale byte is
// the one of MX block g (k 32 g .. 32 g + 31).  A lane keeps its row's four
// scale bytes of a stage in one dword shifted right by 8 g, so byte 0 is the
// block of sub-step 0 and byte 2 that of sub-step 1, picked by op_sel.
#include <utility>

#include "gemm_common.hpp"

namespace engram {
namespace {

using namespace gemm;

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr int kBK = 128;                            // fp8 values per stage
constexpr int kTileBytes = BM * kBK;                // 32 KB per operand per stage
constexpr int kScaleBytes = BM * (kBK / 32);        // 1 KB: 4 scale bytes per row
constexpr int kStageBytes = 2 * kTileBytes + 2 * kScaleBytes;
constexpr int kSegs = kTileBytes / 1024 / kWaves;   // 1 KB segments per wave per operand: 8
constexpr int kIdsPerLane = kSegs + 1;              // A code rows + the A scale row

static_assert(2 * kStageBytes >= BM * BN * 2, "the epilogue reuses the stages");

// Stand-in row for ids outside the table and rows past T: zero codes (so the
// product is exactly 0 whatever the scale) and zero scale bytes (2^-127,
// finite).
__device__ __attribute__((aligned(256))) const uint8_t kZeroRow[ENGRAM_HEAD_DIM] = {};

template <typename T>
__device__ __forceinline__ __attribute__((address_space(3))) void *lds_ptr(T *p) {
  return (__attribute__((address_space(3))) void *)(p);
}

// Scheduling of one sub-step: its 16 MFMAs with kReads LDS reads spread over
// the first 12 of them (the reads feed the next sub-step, so the last MFMAs
// cover their latency); the fence keeps later work out of the group.
template <int kReads, int kPer, int R>
__device__ __forceinline__ void sched_one() {
  constexpr int lo = R * kPer < kReads ? R * kPer : kReads;
  constexpr int hi = (R + 1) * kPer < kReads ? (R + 1) * kPer : kReads;
  if constexpr (hi > lo) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, hi - lo, 0);
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
}
template <int kReads, int kPer, int... R>
__device__ __forceinline__ void sched_each(std::integer_sequence<int, R...>) {
  (sched_one<kReads, kPer, R>(), ...);
}
template <int kReads>
__device__ __forceinline__ void sched_substep() {
  sched_each<kReads, (kReads + 11) / 12>(std::make_integer_sequence<int, 16>{});
  __builtin_amdgcn_sched_barrier(0);
}

__global__ __launch_bounds__(kThreads, 1) void gemm_mx_kernel(
    const uint8_t *__restrict__ table, const uint8_t *__restrict__ tscales, int64_t num_rows,
    const int32_t *__restrict__ ids, int64_t ids_stride, const uint8_t *__restrict__ W,
    const uint8_t *__restrict__ WS, uint16_t *__restrict__ C, int M, int N, int K,
    int tiles_m, int tiles_n, int32_t *__restrict__ bad_ids) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int cols = K / ENGRAM_HEAD_DIM;
  const int nk = K / kBK;                            // 2 stages per table column
  const int ks = K / 32;                             // scale bytes per row

  // Ids outside the table, counted once per (row, column) by the first
  // column of tiles.
  if (tn == 0 && bad_ids && m0 + tid < M) {
    const int32_t *id_row = ids + int64_t(m0 + tid) * ids_stride;
    int bad = 0;
    for (int c = 0; c < cols; ++c) {
      const int32_t v = id_row[c];
      bad += v < 0 || v >= num_rows;
    }
    if (bad) atomicAdd(bad_ids, bad);
  }

  // ---- B codes: one buffer_load ... lds fills a 1 KB segment (8 tile rows);
  // lane L lands at byte 16 L (row L / 8, physical chunk L % 8) and fetches
  // the logical chunk the swizzle keeps there; for segment s the row's key is
  // (L / 8) ^ (s & 1).  Rows past N read as zeros: a buffer load range-checks
  // its VGPR offset only, so every row offset goes there and the SGPR offset
  // carries just the position along K.
  const int seg_row = lane >> 3;
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(W + int64_t(n0) * K, int64_t(N - n0) * K);
  const uint32_t voff_even = uint32_t(seg_row * K + ((lane & 7) ^ seg_row) * 16);
  const uint32_t voff_odd = uint32_t(seg_row * K + ((lane & 7) ^ seg_row ^ 1) * 16);
  // ---- B scales: lane L of wave w brings the stage's 4 bytes of row 64 w + L.
  const __amdgpu_buffer_rsrc_t rbs = make_rsrc(WS + int64_t(n0) * ks, int64_t(N - n0) * ks);
  const uint32_t voff_bs = uint32_t((wave * 64 + lane) * ks);

  // ---- A: per table column, the lane's 8 code rows 64 w + 8 k + L / 8
  // (chunk as for B) and its scale row 64 w + L, resolved from the ids into
  // 64-bit addresses.  The ids come through a buffer descriptor (rows past T
  // read as 0 and are replaced below), loaded two columns ahead of their use.
  const __amdgpu_buffer_rsrc_t rid = make_rsrc(ids, int64_t(M) * ids_stride * 4);
  const int row0 = m0 + wave * 64;
  const uint32_t voff_id = uint32_t((row0 + seg_row) * ids_stride * 4);
  const uint32_t voff_ids = uint32_t((row0 + lane) * ids_stride * 4);
  const int chunk_even = ((lane & 7) ^ seg_row) * 16, chunk_odd = chunk_even ^ 16;
  int32_t idn[kIdsPerLane];
  const uint8_t *a_src[kSegs];
  const uint8_t *as_src;
  auto load_ids = [&](int c) {
    c = min(c, cols - 1);
#pragma unroll
    for (int k = 0; k < kSegs; ++k)
      idn[k] = __builtin_amdgcn_raw_buffer_load_b32(
          rid, voff_id + uint32_t(8 * k * ids_stride * 4), c * 4, 0);
    idn[kSegs] = __builtin_amdgcn_raw_buffer_load_b32(rid, voff_ids, c * 4, 0);
  };
  auto resolve = [&]() {
#pragma unroll
    for (int k = 0; k < kSegs; ++k) {
      const bool ok = row0 + 8 * k + seg_row < M && idn[k] >= 0 && idn[k] < num_rows;
      a_src[k] = (ok ? table + int64_t(idn[k]) * ENGRAM_HEAD_DIM : kZeroRow) +
                 ((k & 1) ? chunk_odd : chunk_even);
    }
    const bool ok = row0 + lane < M && idn[kSegs] >= 0 && idn[kSegs] < num_rows;
    as_src = ok ? tscales + int64_t(idn[kSegs]) * (ENGRAM_HEAD_DIM / 32) : kZeroRow;
  };
  // Stage kt (values 128 kt .. 128 kt + 127: half kt % 2 of column kt / 2)
  // into LDS buffer `buf`; a_src/as_src must hold column kt / 2 (clamped to
  // the last column).  The half's offset goes into the address itself: the
  // immediate offset of an LDS-DMA load moves its LDS destination as well.
  auto dma = [&](int buf, int kt, const int half) {
    uint8_t *st = smem + buf * kStageBytes;
    const int kb = min(kt, nk - 1);
#pragma unroll
    for (int i = 0; i < kSegs; ++i) {
      const int seg = wave * kSegs + i;
      __builtin_amdgcn_global_load_lds(a_src[i] + half * kBK, lds_ptr(st + seg * 1024), 16, 0,
                                       0);
    }
#pragma unroll
    for (int i = 0; i < kSegs; ++i) {
      const int seg = wave * kSegs + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, lds_ptr(st + kTileBytes + seg * 1024), 16,
                                               ((i & 1) ? voff_odd : voff_even) + seg * 8 * K,
                                               kb * kBK, 0, 0);
    }
    __builtin_amdgcn_global_load_lds(as_src + half * 4,
                                     lds_ptr(st + 2 * kTileBytes + wave * 256), 4, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rbs, lds_ptr(st + 2 * kTileBytes + kScaleBytes + wave * 256), 4, voff_bs, kb * 4, 0, 0);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // Fragments: a sub-step's 4 A and 4 B fragments (8 VGPRs each), double
  // buffered: those of the next sub-step are read while this one multiplies.
  // Fragment f of sub-step s is chunks 4 s + g and 4 s + 2 + g of row
  // f * 32 + frow of the wave's operand rows; the swizzle key of those rows is
  // that of frow, so a lane's chunk offsets are the same for all four.
  const int frow = lane & 31, fhalf = lane >> 5;
  const int fkey = swz_key<64>(frow);
  const int a_frag = (wm * 128 + frow) * kBK, b_frag = kTileBytes + (wn * 128 + frow) * kBK;
  i32x8 fa[2][4], fb[2][4];
  uint32_t sca[2][4], scb[2][4];
  auto read_frag = [&](int buf, int base, int f, const int s) {
    const uint8_t *p = smem + buf * kStageBytes + base + f * 32 * kBK;
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(p + (((4 * s + fhalf) ^ fkey) << 4));
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(p + (((4 * s + 2 + fhalf) ^ fkey) << 4));
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto load_scales = [&](int buf, const int set) {
    const uint32_t *ss = reinterpret_cast<const uint32_t *>(smem + buf * kStageBytes +
                                                            2 * kTileBytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) sca[set][i] = ss[wm * 128 + i * 32 + frow] >> (8 * fhalf);
#pragma unroll
    for (int j = 0; j < 4; ++j) scb[set][j] = ss[BM + wn * 128 + j * 32 + frow] >> (8 * fhalf);
  };
  auto load_frags = [&](int buf, const int s, const int slot) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      fa[slot][f] = read_frag(buf, a_frag, f, s);
      fb[slot][f] = read_frag(buf, b_frag, f, s);
    }
  };
  // Sub-step s of a stage: 4 x 4 MFMAs of fragment slot `slot` with the
  // scales of set `set` (op_sel 0 picks sub-step 0's block, 2 sub-step 1's).
  auto mfma_block = [&](const int slot, const int set, const int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (s == 0)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa[slot][i], fb[slot][j], acc[i][j], 0, 0, 0, sca[set][i], 0, scb[set][j]);
        else
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa[slot][i], fb[slot][j], acc[i][j], 0, 0, 2, sca[set][i], 2, scb[set][j]);
      }
  };

  // Iteration kt multiplies the stage in buffer j = kt % 2; on entry fragment
  // slot 0 holds its sub-step 0 and sca/scb[j] its scales.
  //  - at even kt, the ids of column kt / 2 + 2 are requested (9 loads);
  //  - sub-step 1's fragments are read while sub-step 0 multiplies: after
  //    that, buffer j is no longer read;
  //  - the barrier waits for stage kt + 1's DMA (issued one iteration ago;
  //    at even kt only the 9 younger id loads may stay in flight) and for
  //    every wave's reads of buffer j;
  //  - buffer j then takes stage kt + 2 (column kt / 2 + 1, half j), and at
  //    odd kt the addresses of column kt / 2 + 2 are resolved for the next
  //    two DMAs;
  //  - stage kt + 1's sub-step 0 fragments and scales are read while
  //    sub-step 1 of stage kt multiplies.
  auto iteration = [&](int kt, const int j) {
    const int b = j;
    __builtin_amdgcn_sched_barrier(0);
    if (j == 0) load_ids(kt / 2 + 2);
    __builtin_amdgcn_sched_barrier(0);
    load_frags(b, 1, 1);
    mfma_block(0, j, 0);
    sched_substep<16>();
    if (j == 0) stage_barrier<waitcnt(kIdsPerLane, 0)>();
    else stage_barrier<waitcnt(0, 0)>();
    dma(b, kt + 2, j);
    if (j == 1) resolve();
    __builtin_amdgcn_sched_barrier(0);
    load_frags(b ^ 1, 0, 0);
    load_scales(b ^ 1, j ^ 1);
    mfma_block(1, j, 1);
    sched_substep<24>();
  };

  // Prologue: stages 0 and 1 (column 0) in flight, then column 1's addresses.
  load_ids(0);
  resolve();
  dma(0, 0, 0);
  dma(1, 1, 1);
  load_ids(1);
  resolve();
  stage_barrier<waitcnt(0, 0)>();
  load_frags(0, 0, 0);
  load_scales(0, 0);

  for (int kt = 0; kt < nk; kt += 2) {               // nk = 2 * cols is even
    iteration(kt, 0);
    iteration(kt + 1, 1);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
  __syncthreads();                                   // every wave is done with the stages
  store_tile(acc, reinterpret_cast<uint16_t *>(smem), C, M, N, m0, n0, wm, wn, lane, tid);
}

// The persistent form (cols >= 2): one workgroup per CU walks the tiles b,
// b + G, b + 2 G, ... of the XCD-aware order with the K loop above, which
// runs on from tile to tile: the ids two columns ahead, the resolved A
// addresses and the DMA of the stage after next simply continue into the
// next tile's first columns (with its rows, its B resources), so the next
// tile's first stages are in LDS when the current tile ends.  The MFMAs take
// the weight as their first operand, so each output block comes out
// transposed and the epilogue is wave-private (store_wave_transposed).  Ids
// outside the table are counted as their column's addresses are resolved,
// for the tiles of the first column of tiles.
// kStaged: A is an MXFP8 activation staged by stage_mx_kernel (`table` =
// codes [M][K], `tscales` = scales [M][K/32], row-major like W and WS), read
// exactly like B; ids, num_rows and bad_ids are unused.  The MFMAs and their
// order are the same, so kv is bit-identical to the gather form's.
template <bool kStaged>
__global__ __launch_bounds__(kThreads, 1) void gemm_mx_persistent_kernel(
    const uint8_t *__restrict__ table, const uint8_t *__restrict__ tscales, int64_t num_rows,
    const int32_t *__restrict__ ids, int64_t ids_stride, const uint8_t *__restrict__ W,
    const uint8_t *__restrict__ WS, uint16_t *__restrict__ C, int M, int N, int K,
    int tiles_m, int tiles_n, int32_t *__restrict__ bad_ids) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int cols = K / ENGRAM_HEAD_DIM;
  const int nk = K / kBK;                            // 2 stages per table column
  const int ks = K / 32;                             // scale bytes per row
  const int tiles = tiles_m * tiles_n;
  int lid = blockIdx.x;
  if (lid >= tiles) return;
  uint16_t *const stg =
      reinterpret_cast<uint16_t *>(smem + 2 * kStageBytes) + wave * 32 * kStgStride;

  // B codes and scales as in gemm_mx_kernel, per tile column tn.
  const int seg_row = lane >> 3;
  const uint32_t voff_even = uint32_t(seg_row * K + ((lane & 7) ^ seg_row) * 16);
  const uint32_t voff_odd = uint32_t(seg_row * K + ((lane & 7) ^ seg_row ^ 1) * 16);
  const uint32_t voff_bs = uint32_t((wave * 64 + lane) * ks);
  auto rsrc_b = [&](int tn_) {
    const int n0_ = tn_ * BN;
    return make_rsrc(W + int64_t(n0_) * K, int64_t(N - n0_) * K);
  };
  auto rsrc_bs = [&](int tn_) {
    const int n0_ = tn_ * BN;
    return make_rsrc(WS + int64_t(n0_) * ks, int64_t(N - n0_) * ks);
  };
  // Staged A: the same addressing as B, over M rows.
  auto rsrc_a = [&](int tm_) {
    const int m0_ = tm_ * BM;
    return make_rsrc(table + int64_t(m0_) * K, kStaged ? int64_t(M - m0_) * K : 0);
  };
  auto rsrc_as = [&](int tm_) {
    const int m0_ = tm_ * BM;
    return make_rsrc(tscales + int64_t(m0_) * ks, kStaged ? int64_t(M - m0_) * ks : 0);
  };

  // A: the ids of one column of one tile (rows row0 .. row0 + 63 of this
  // wave) and their resolved addresses, as in gemm_mx_kernel.
  const __amdgpu_buffer_rsrc_t rid = make_rsrc(ids, int64_t(M) * ids_stride * 4);
  const int chunk_even = ((lane & 7) ^ seg_row) * 16, chunk_odd = chunk_even ^ 16;
  int32_t idn[kIdsPerLane];
  int idn_row0 = 0;
  bool idn_count = false;
  int bad = 0;
  const uint8_t *a_src[kSegs];
  const uint8_t *as_src;
  auto load_ids = [&](int tm_, int c, bool count) {
    if constexpr (kStaged) return;
    const int row0 = tm_ * BM + wave * 64;
    const uint32_t voff_id = uint32_t((row0 + seg_row) * ids_stride * 4);
    const uint32_t voff_ids = uint32_t((row0 + lane) * ids_stride * 4);
#pragma unroll
    for (int k = 0; k < kSegs; ++k)
      idn[k] = __builtin_amdgcn_raw_buffer_load_b32(
          rid, voff_id + uint32_t(8 * k * ids_stride * 4), c * 4, 0);
    idn[kSegs] = __builtin_amdgcn_raw_buffer_load_b32(rid, voff_ids, c * 4, 0);
    idn_row0 = row0;
    idn_count = count;
  };
  auto resolve = [&]() {
    if constexpr (kStaged) return;
#pragma unroll
    for (int k = 0; k < kSegs; ++k) {
      const bool ok = idn_row0 + 8 * k + seg_row < M && idn[k] >= 0 && idn[k] < num_rows;
      a_src[k] = (ok ? table + int64_t(idn[k]) * ENGRAM_HEAD_DIM : kZeroRow) +
                 ((k & 1) ? chunk_odd : chunk_even);
    }
    const bool row_ok = idn_row0 + lane < M;
    const bool ok = row_ok && idn[kSegs] >= 0 && idn[kSegs] < num_rows;
    as_src = ok ? tscales + int64_t(idn[kSegs]) * (ENGRAM_HEAD_DIM / 32) : kZeroRow;
    bad += idn_count && row_ok && !ok;
  };
  // Stage of B slice kb (K positions 128 kb ..) and A half `half` of the
  // resolved column (staged: A slice kb of resource ra) into LDS buffer `buf`.
  auto dma = [&](int buf, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t ras,
                 __amdgpu_buffer_rsrc_t rb, __amdgpu_buffer_rsrc_t rbs, int kb, const int half) {
    uint8_t *st = smem + buf * kStageBytes;
#pragma unroll
    for (int i = 0; i < kSegs; ++i) {
      const int seg = wave * kSegs + i;
      if constexpr (kStaged)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, lds_ptr(st + seg * 1024), 16,
                                                 ((i & 1) ? voff_odd : voff_even) + seg * 8 * K,
                                                 kb * kBK, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(a_src[i] + half * kBK, lds_ptr(st + seg * 1024), 16, 0,
                                         0);
    }
#pragma unroll
    for (int i = 0; i < kSegs; ++i) {
      const int seg = wave * kSegs + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, lds_ptr(st + kTileBytes + seg * 1024), 16,
                                               ((i & 1) ? voff_odd : voff_even) + seg * 8 * K,
                                               kb * kBK, 0, 0);
    }
    if constexpr (kStaged)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ras, lds_ptr(st + 2 * kTileBytes + wave * 256), 4,
                                               voff_bs, kb * 4, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(as_src + half * 4,
                                       lds_ptr(st + 2 * kTileBytes + wave * 256), 4, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rbs, lds_ptr(st + 2 * kTileBytes + kScaleBytes + wave * 256), 4, voff_bs, kb * 4, 0, 0);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int frow = lane & 31, fhalf = lane >> 5;
  const int fkey = swz_key<64>(frow);
  const int a_frag = (wm * 128 + frow) * kBK, b_frag = kTileBytes + (wn * 128 + frow) * kBK;
  i32x8 fa[2][4], fb[2][4];
  uint32_t sca[2][4], scb[2][4];
  auto read_frag = [&](int buf, int base, int f, const int s) {
    const uint8_t *p = smem + buf * kStageBytes + base + f * 32 * kBK;
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(p + (((4 * s + fhalf) ^ fkey) << 4));
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(p + (((4 * s + 2 + fhalf) ^ fkey) << 4));
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto load_scales = [&](int buf, const int set) {
    const uint32_t *ss = reinterpret_cast<const uint32_t *>(smem + buf * kStageBytes +
                                                            2 * kTileBytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) sca[set][i] = ss[wm * 128 + i * 32 + frow] >> (8 * fhalf);
#pragma unroll
    for (int j = 0; j < 4; ++j) scb[set][j] = ss[BM + wn * 128 + j * 32 + frow] >> (8 * fhalf);
  };
  auto load_frags = [&](int buf, const int s, const int slot) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      fa[slot][f] = read_frag(buf, a_frag, f, s);
      fb[slot][f] = read_frag(buf, b_frag, f, s);
    }
  };
  auto mfma_block = [&](const int slot, const int set, const int s) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (s == 0)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fb[slot][j], fa[slot][i], acc[i][j], 0, 0, 0, scb[set][j], 0, sca[set][i]);
        else
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fb[slot][j], fa[slot][i], acc[i][j], 0, 0, 2, scb[set][j], 2, sca[set][i]);
      }
  };

  // Iteration kt (j = kt % 2) as in gemm_mx_kernel; the ids requested at
  // even kt are those of sequence column kt / 2 + 2 (the next tile's column
  // kt / 2 + 2 - cols past this tile's last), and the stage filled after the
  // middle barrier is the sequence's stage kt + 2.
  auto iteration = [&](const int j, int ids_tm, int ids_col, bool ids_count,
                       __amdgpu_buffer_rsrc_t ra_f, __amdgpu_buffer_rsrc_t ras_f,
                       __amdgpu_buffer_rsrc_t rb_f, __amdgpu_buffer_rsrc_t rbs_f, int fill_kb) {
    const int b = j;
    __builtin_amdgcn_sched_barrier(0);
    if (j == 0) load_ids(ids_tm, ids_col, ids_count);
    __builtin_amdgcn_sched_barrier(0);
    load_frags(b, 1, 1);
    mfma_block(0, j, 0);
    sched_substep<16>();
    // The ids requested at j == 0 may stay in flight (the gather form).
    if (j == 0 && !kStaged) stage_barrier<waitcnt(kIdsPerLane, 0)>();
    else stage_barrier<waitcnt(0, 0)>();
    dma(b, ra_f, ras_f, rb_f, rbs_f, fill_kb, j);
    if (j == 1) resolve();
    __builtin_amdgcn_sched_barrier(0);
    load_frags(b ^ 1, 0, 0);
    load_scales(b ^ 1, j ^ 1);
    mfma_block(1, j, 1);
    sched_substep<24>();
  };

  // Prologue: the first tile's stages 0 and 1 (column 0) in flight, then
  // column 1's addresses.
  int tm, tn;
  tile_coords(lid, tiles_m, tiles_n, tm, tn);
  __amdgpu_buffer_rsrc_t ra = rsrc_a(tm), ras = rsrc_as(tm), rb = rsrc_b(tn), rbs = rsrc_bs(tn);
  const bool counting = !kStaged && bad_ids != nullptr;
  load_ids(tm, 0, counting && tn == 0);
  resolve();
  dma(0, ra, ras, rb, rbs, 0, 0);
  dma(1, ra, ras, rb, rbs, 1, 1);
  load_ids(tm, 1, counting && tn == 0);
  resolve();
  stage_barrier<waitcnt(0, 0)>();
  load_frags(0, 0, 0);
  load_scales(0, 0);

  for (;;) {
    const int next = lid + int(gridDim.x);
    const bool has_next = next < tiles;
    int tm2 = tm, tn2 = tn;
    if (has_next) tile_coords(next, tiles_m, tiles_n, tm2, tn2);
    const __amdgpu_buffer_rsrc_t ra2 = rsrc_a(tm2), ras2 = rsrc_as(tm2);
    const __amdgpu_buffer_rsrc_t rb2 = rsrc_b(tn2), rbs2 = rsrc_bs(tn2);
    for (int kt = 0; kt < nk; kt += 2) {
      // Sequence column c + 2 for the ids, stages kt + 2 and kt + 3 for the
      // DMA; after the last tile they repeat this tile's last column and
      // stage, which nothing reads.
      const int c2 = kt / 2 + 2;
      const bool nxt = c2 >= cols;
      const int ids_tm = nxt && has_next ? tm2 : tm;
      const int ids_col = nxt ? (has_next ? c2 - cols : cols - 1) : c2;
      const bool ids_count = counting && (nxt ? has_next && tn2 == 0 : tn == 0);
      const bool fill_next = kt + 2 >= nk;
      const __amdgpu_buffer_rsrc_t raf = fill_next && has_next ? ra2 : ra;
      const __amdgpu_buffer_rsrc_t rasf = fill_next && has_next ? ras2 : ras;
      const __amdgpu_buffer_rsrc_t rbf = fill_next && has_next ? rb2 : rb;
      const __amdgpu_buffer_rsrc_t rbsf = fill_next && has_next ? rbs2 : rbs;
      const int kb0 = fill_next ? (has_next ? kt + 2 - nk : nk - 1) : kt + 2;
      const int kb1 = fill_next ? (has_next ? kt + 3 - nk : nk - 1) : kt + 3;
      iteration(0, ids_tm, ids_col, ids_count, raf, rasf, rbf, rbsf, kb0);
      iteration(1, ids_tm, ids_col, ids_count, raf, rasf, rbf, rbsf, kb1);
    }
    store_wave_transposed<4, 4, 1>(acc, stg, C, M, N, tm * BM + wm * 128, tn * BN + wn * 128,
                                   lane);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    if (!has_next) break;
    lid = next;
    tm = tm2;
    tn = tn2;
    ra = ra2;
    ras = ras2;
    rb = rb2;
    rbs = rbs2;
  }
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));        // the last, unread reloads
  if (bad) atomicAdd(bad_ids, bad);
}

// The MXFP8 activation of FP8 rows: row (t, r) of the flattened [M * cols]
// goes to codes[t][256 r ..] and scales[t][8 r ..].  16 lanes per row, each
// a 16-byte piece of the codes (lane 0 also the 8 scale bytes, as two words:
// the scale arrays are 4-byte aligned); each group of 16 lanes takes
// kStageRows rows, whose ids and then codes are all requested before the
// first store.  An id outside the table writes zero codes and scale bytes
// 127 (2^0: the row is exactly zero) and is counted.
constexpr int kStageRows = 4;
constexpr int kStageRowsPerBlock = kThreads / 16 * kStageRows;

__global__ __launch_bounds__(kThreads) void stage_mx_kernel(
    const uint8_t *__restrict__ table, const uint8_t *__restrict__ tscales, int64_t num_rows,
    const int32_t *__restrict__ ids, int64_t ids_stride, int cols, int M,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, int32_t *__restrict__ bad_ids) {
  const int piece = threadIdx.x & 15;
  const int64_t total = int64_t(M) * cols;
  const int64_t first = int64_t(blockIdx.x) * kStageRowsPerBlock + (threadIdx.x >> 4);
  int32_t id[kStageRows];
  bool ok[kStageRows];
#pragma unroll
  for (int k = 0; k < kStageRows; ++k) {
    const int64_t row = first + int64_t(k) * (kThreads / 16);
    id[k] = -1;
    if (row < total) {
      const int64_t t = row / cols, r = row - t * cols;
      id[k] = ids[t * ids_stride + r];
    }
    ok[k] = row < total && id[k] >= 0 && id[k] < num_rows;
  }
  u32x4 v[kStageRows];
#pragma unroll
  for (int k = 0; k < kStageRows; ++k) {
    v[k] = u32x4{0, 0, 0, 0};
    if (ok[k])
      v[k] = *reinterpret_cast<const u32x4 *>(table + int64_t(id[k]) * ENGRAM_HEAD_DIM +
                                              16 * piece);
  }
  int bad = 0;
#pragma unroll
  for (int k = 0; k < kStageRows; ++k) {
    const int64_t row = first + int64_t(k) * (kThreads / 16);
    if (row >= total) continue;
    *reinterpret_cast<u32x4 *>(codes + row * ENGRAM_HEAD_DIM + 16 * piece) = v[k];
    if (piece == 0) {
      uint32_t s0 = 0x7F7F7F7Fu, s1 = 0x7F7F7F7Fu;
      if (ok[k]) {
        const uint32_t *src = reinterpret_cast<const uint32_t *>(tscales + int64_t(id[k]) * 8);
        s0 = src[0];
        s1 = src[1];
      }
      uint32_t *dst = reinterpret_cast<uint32_t *>(scales + row * 8);
      dst[0] = s0;
      dst[1] = s1;
      bad += !ok[k];
    }
  }
  __shared__ int n_bad;
  if (threadIdx.x == 0) n_bad = 0;
  __syncthreads();
  if (bad) atomicAdd(&n_bad, bad);
  __syncthreads();
  if (threadIdx.x == 0 && n_bad && bad_ids) atomicAdd(bad_ids, n_bad);
}
}  // namespace

bool project_mx_supported(int32_t N, int32_t K) {
  return int64_t(N) * K <= 0x7FFFFFF0LL;
}

hipError_t launch_project_mx(const uint8_t *table, const uint8_t *scales, int64_t num_rows,
                             const int32_t *ids, int64_t ids_token_stride, int32_t cols,
                             const uint8_t *w_codes, const uint8_t *w_scales, uint16_t *c,
                             int32_t M, int32_t N, int32_t *bad_ids, hipStream_t stream) {
  if (project_mx_skinny_supported(M, cols))
    return launch_project_mx_skinny(table, scales, num_rows, ids, ids_token_stride, cols,
                                    w_codes, w_scales, c, M, N, bad_ids, stream);
  const int K = cols * ENGRAM_HEAD_DIM;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  if (cols >= 2) {
    const size_t lds = size_t(2) * kStageBytes + size_t(kWaves) * 32 * kStgStride * 2;
    const void *fn = reinterpret_cast<const void *>(&gemm_mx_persistent_kernel<false>);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_mx_persistent_kernel<false>,
                       dim3(persistent_grid(tiles_m * tiles_n, stream)), dim3(kThreads), lds,
                       stream, table, scales, num_rows, ids, ids_token_stride, w_codes, w_scales,
                       c, M, N, K, tiles_m, tiles_n, bad_ids);
    return hipGetLastError();
  }
  const size_t lds = size_t(2) * kStageBytes;
  const void *fn = reinterpret_cast<const void *>(&gemm_mx_kernel);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemm_mx_kernel, dim3(tiles_m * tiles_n), dim3(kThreads), lds, stream,
                     table, scales, num_rows, ids, ids_token_stride, w_codes, w_scales, c, M, N,
                     K, tiles_m, tiles_n, bad_ids);
  return hipGetLastError();
}

hipError_t launch_stage_mx(const uint8_t *table, const uint8_t *scales, int64_t num_rows,
                           const int32_t *ids, int64_t ids_token_stride, int32_t cols, int32_t M,
                           uint8_t *a_codes, uint8_t *a_scales, int32_t *bad_ids,
                           hipStream_t stream) {
  const int64_t rows = int64_t(M) * cols;
  const int64_t blocks = (rows + kStageRowsPerBlock - 1) / kStageRowsPerBlock;
  hipLaunchKernelGGL(stage_mx_kernel, dim3(uint32_t(blocks)), dim3(kThreads), 0, stream, table,
                     scales, num_rows, ids, ids_token_stride, cols, M, a_codes, a_scales,
                     bad_ids);
  return hipGetLastError();
}

hipError_t launch_project_mx_staged(const uint8_t *a_codes, const uint8_t *a_scales,
                                    int32_t cols, const uint8_t *w_codes,
                                    const uint8_t *w_scales, uint16_t *c, int32_t M, int32_t N,
                                    hipStream_t stream) {
  const int K = cols * ENGRAM_HEAD_DIM;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const size_t lds = size_t(2) * kStageBytes + size_t(kWaves) * 32 * kStgStride * 2;
  const void *fn = reinterpret_cast<const void *>(&gemm_mx_persistent_kernel<true>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemm_mx_persistent_kernel<true>,
                     dim3(persistent_grid(tiles_m * tiles_n, stream)), dim3(kThreads), lds,
                     stream, a_codes, a_scales, int64_t(0), (const int32_t *)nullptr, int64_t(0),
                     w_codes, w_scales, c, M, N, K, tiles_m, tiles_n, (int32_t *)nullptr);
  return hipGetLastError();
}

}  // namespace engram
