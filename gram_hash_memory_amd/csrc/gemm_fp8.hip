// Stages 2 + 3 fused for FP8 tables with the bf16 weight:
//   kv = bf16(dequant(table[ids])) x wkv^T.
//
// [vLLM engram page, _engram_lookup_kernel, bf16 mode]: an FP8 row value is
// its e4m3fn code times 2^(scale byte - 127), rounded to bf16, and the bf16
// rows go through the dense projection ([spark engram_v41 page, overview
// stage 3]).  Here the projection reads the raw rows (256 code bytes + 8
// scale bytes per 256 values) instead of 512-byte bf16 rows, and every
// output sums the same bf16 products in the same K order as rows ->
// engram_project, so kv is bit-identical to that pair.
//
// Structure: the persistent form of gemm_q2k.hip (4 x 1 waves, each 64 tile
// rows x 256 columns, K in stages of 64, transposed MFMA output,
// wave-private epilogue), with A in LDS next to B:
//  - two B stages (bf16, 32 KB each) and two A buffers, each holding half a
//    table column of the tile's 256 rows: 128 codes per row (16-byte chunk q
//    of row r at chunk q ^ ((r >> 1) & 7), so the 8-byte fragment reads of 16
//    consecutive rows fall on distinct banks) and the row's scale word;
//  - A comes by global_load_lds through 64-bit row addresses (tables may pass
//    the 4 GB a buffer descriptor spans): per wave and half column, 8
//    instructions of 8 rows x 128 bytes (whole 128-byte lines) and one of the
//    64 rows' scale words; an id outside the table, or a row past T, reads a
//    zero row.  A half column is requested right after the barrier that frees
//    its buffer, two stages before its use;
//  - the ids of the next table column (of the next tile after the last) are
//    loaded at a column's first stage and resolved into addresses at its
//    second, before the DMA of the next column's first half;
//  - a lane reads its 8 codes of a k-step (ds_read_b64) and converts them
//    with v_cvt_scalef32_pk_bf16_fp8, which equals the rows kernel's
//    arithmetic for every finite code and scale bytes 1..254 (probed over all
//    codes); a fragment with a NaN code or scale byte 0 or 255 is recomputed
//    the rows kernel's way, behind a wave-uniform branch that the workloads
//    never take.
// Measured at the FP8 workload (16384 tokens) it is about 4 % slower than
// engram_rows + engram_project: gathering 128-byte pieces of random rows for
// every column of tiles costs more than one streaming gather of whole rows
// plus dense bf16 reads.  It needs no rows buffer.
#include "gemm_common.hpp"

namespace engram {
namespace {

using namespace gemm;
using namespace gemm::wide;

constexpr int kBBytes = kStageElems * 2;             // one B stage: 32 KB
constexpr int kAOff = 2 * kBBytes;                   // the two A buffers after the B stages
constexpr int kACodes = BM * 2 * BK;                 // 256 rows x 128 codes: 32 KB
constexpr int kABufBytes = kACodes + BM * 4;         // + one scale word per row: 33 KB
constexpr int kLdsLoop = kAOff + 2 * kABufBytes;     // 130 KB
constexpr int kCodeRows = 8;                         // A code rows per lane and column
constexpr int kIdsPerLane = kCodeRows + 1;           // + the lane's scale row

// Zero codes and zero scale bytes: what an id outside the table reads.
__device__ __attribute__((aligned(256))) const uint8_t kZeroFp8Row[ENGRAM_FP8_ROW_BYTES] = {};

template <typename T>
__device__ __forceinline__ __attribute__((address_space(3))) void *lds_ptr(T *p) {
  return (__attribute__((address_space(3))) void *)(p);
}

// Eight e4m3 codes (c.x bytes 0..3, c.y bytes 0..3) times `scale`, as four
// bf16 pairs, the rows kernel's way.
__device__ __forceinline__ u32x4 fp8x8_exact(u32x2 c, float scale) {
  u32x4 v;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t w = c[p >> 1] >> (16 * (p & 1));
    v[p] = pack_bf16x2(e4m3fn_to_float(w & 0xFFu) * scale,
                       e4m3fn_to_float((w >> 8) & 0xFFu) * scale);
  }
  return v;
}

// Two e4m3 codes of w (bytes 0, 1 with false_type, 2, 3 with true_type)
// times sc as a bf16 pair (v_cvt_scalef32_pk_bf16_fp8).
struct false_type {};
struct true_type {};
__device__ __forceinline__ uint32_t cvt_pk(uint32_t w, float sc, false_type) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, sc, false));
}
__device__ __forceinline__ uint32_t cvt_pk(uint32_t w, float sc, true_type) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, sc, true));
}

// Nonzero if a byte of c is 0x7F or 0xFF (an e4m3fn NaN).
__device__ __forceinline__ uint32_t has_nan_code(u32x2 c) {
  return (((c[0] & 0x7F7F7F7Fu) + 0x01010101u) | ((c[1] & 0x7F7F7F7Fu) + 0x01010101u)) &
         0x80808080u;
}

__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_persistent_kernel(
    const uint8_t *__restrict__ table, const uint8_t *__restrict__ tscales, int64_t num_rows,
    const int32_t *__restrict__ ids, int64_t ids_stride, const uint16_t *__restrict__ B,
    uint16_t *__restrict__ C, int M, int N, int K, int tiles_m, int tiles_n,
    int32_t *__restrict__ bad_ids) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int frow = lane & 31, fhalf = lane >> 5;
  const int cols = K / ENGRAM_HEAD_DIM;
  const int nk = K / BK;
  const int tiles = tiles_m * tiles_n;
  int lid = blockIdx.x;
  if (lid >= tiles) return;
  uint16_t *const stg = reinterpret_cast<uint16_t *>(smem + kLdsLoop) + wave * 32 * kStgStride;
  auto stage_b = [&](int stage) { return reinterpret_cast<uint16_t *>(smem + stage * kBBytes); };
  auto abuf = [&](int b) { return smem + kAOff + b * kABufBytes; };

  const BSegs segs = b_segs(lane, K);

  // ---- A addresses.  Code row i of lane L (of its wave's 64) is 8 i + L / 8,
  // its 16-byte chunk L % 8 (holding logical chunk (L % 8) ^ key(row), key(r)
  // = (r >> 1) & 7); the scale row is L.
  const __amdgpu_buffer_rsrc_t rid = make_rsrc(ids, int64_t(M) * ids_stride * 4);
  auto code_chunk = [&](int i) { return 16 * ((lane & 7) ^ ((4 * i + (lane >> 4)) & 7)); };
  int32_t idn[kIdsPerLane];
  int idn_row0 = 0;
  bool idn_count = false;
  int bad = 0;
  const uint8_t *a_src[kCodeRows];
  const uint8_t *as_src;
  auto load_ids = [&](int tm_, int c, bool count) {
    const int row0 = tm_ * BM + wave * 64;
#pragma unroll
    for (int i = 0; i < kCodeRows; ++i)
      idn[i] = __builtin_amdgcn_raw_buffer_load_b32(
          rid, uint32_t((row0 + 8 * i + (lane >> 3)) * ids_stride * 4), c * 4, 0);
    idn[kCodeRows] = __builtin_amdgcn_raw_buffer_load_b32(
        rid, uint32_t((row0 + lane) * ids_stride * 4), c * 4, 0);
    idn_row0 = row0;
    idn_count = count;
  };
  auto resolve = [&]() {
#pragma unroll
    for (int i = 0; i < kCodeRows; ++i) {
      const bool ok = idn_row0 + 8 * i + (lane >> 3) < M && idn[i] >= 0 && idn[i] < num_rows;
      a_src[i] =
          (ok ? table + int64_t(idn[i]) * ENGRAM_FP8_ROW_BYTES : kZeroFp8Row) + code_chunk(i);
    }
    const bool row_ok = idn_row0 + lane < M;
    const bool ok = row_ok && idn[kCodeRows] >= 0 && idn[kCodeRows] < num_rows;
    as_src = ok ? tscales + int64_t(idn[kCodeRows]) * ENGRAM_FP8_SCALE_BYTES : kZeroFp8Row;
    bad += idn_count && row_ok && !ok;
  };
  auto dma_b = [&](__amdgpu_buffer_rsrc_t rb, int stage, int slice) {
    dma_b_slice(rb, stage_b(stage), segs, wave, slice);
  };
  // A buffer b gets half `half` of the resolved column (codes 128 half ..,
  // scale word `half`).
  auto dma_a = [&](int b, const int half) {
    uint8_t *ab = abuf(b);
#pragma unroll
    for (int i = 0; i < kCodeRows; ++i)
      __builtin_amdgcn_global_load_lds(a_src[i] + 128 * half,
                                       lds_ptr(ab + (wave * 64 + 8 * i) * 128), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(as_src + 4 * half, lds_ptr(ab + kACodes + wave * 256), 4, 0,
                                     0);
  };

  // ---- A fragments: lane (r, h) of row block i takes codes 16 ks + 8 h ..
  // + 7 of tile row 64 wave + 32 i + r, with the scale byte of its 32-value
  // block.
  const int a_key = (frow >> 1) & 7;
  u32x2 ra[kRowsPerLane];
  uint32_t sw[2][kRowsPerLane];
  uint32_t sbyte[kRowsPerLane];
  bf16x8 fa[2][kRowsPerLane], fb[2][kNJ];
  // k-step ks of quarter qs: chunk 4 (qs % 2) + ks of A buffer qs / 2.
  auto read_a = [&](const int qs, const int ks) {
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i)
      ra[i] = *reinterpret_cast<const u32x2 *>(abuf(qs >> 1) + (wave * 64 + 32 * i + frow) * 128 +
                                               16 * ((4 * (qs & 1) + ks) ^ a_key) + 8 * fhalf);
  };
  auto read_scales = [&](int b) {
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i)
      sw[b][i] = *reinterpret_cast<const uint32_t *>(abuf(b) + kACodes +
                                                     (wave * 64 + 32 * i + frow) * 4);
  };
  // Fast conversion of ra into fragment slot `slot`; returns the rows whose
  // fragment needs the exact conversion (bit i for row block i).
  auto conv_a = [&](const int qs, const int ks, int slot) {
    uint32_t need = 0;
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) {
      sbyte[i] = (sw[qs >> 1][i] >> (8 * (2 * (qs & 1) + (ks >> 1)))) & 0xFFu;
      const float sc = e8m0_to_float(sbyte[i]);
      u32x4 v;
      v[0] = cvt_pk(ra[i][0], sc, false_type{});
      v[1] = cvt_pk(ra[i][0], sc, true_type{});
      v[2] = cvt_pk(ra[i][1], sc, false_type{});
      v[3] = cvt_pk(ra[i][1], sc, true_type{});
      fa[slot][i] = __builtin_bit_cast(bf16x8, v);
      const bool exact = has_nan_code(ra[i]) != 0u || ((sbyte[i] + 1u) & 0xFEu) == 0u;
      need |= (exact ? 1u : 0u) << i;
    }
    return need;
  };
  auto fixup_a = [&](uint32_t need, int slot) {
    __builtin_amdgcn_sched_barrier(0);
    if (__builtin_amdgcn_ballot_w64(need != 0u) != 0u) {
#pragma unroll
      for (int i = 0; i < kRowsPerLane; ++i)
        if (need & (1u << i))
          fa[slot][i] = __builtin_bit_cast(bf16x8, fp8x8_exact(ra[i], e8m0_to_float(sbyte[i])));
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  f32x16 acc[kRowsPerLane][kNJ];
#pragma unroll
  for (int i = 0; i < kRowsPerLane; ++i)
#pragma unroll
    for (int j = 0; j < kNJ; ++j) acc[i][j] = f32x16{};

  auto load_b = [&](int stage, int ks, int slot) {
    load_b_frags(stage_b(stage), frow, fhalf, ks, fb[slot]);
  };
  auto mfma_block = [&](int slot) {
#pragma unroll
    for (int j = 0; j < kNJ; ++j)
#pragma unroll
      for (int i = 0; i < kRowsPerLane; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[slot][j], fa[slot][i],
                                                            acc[i][j], 0, 0, 0);
  };
  // A k-step: its 16 MFMAs with the next step's fragment reads in the first
  // slots and the conversion (about 24 VALU ops) in the later ones.
  auto sched_k = [&]() {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (r < 12) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      if (r >= 8) __builtin_amdgcn_sched_group_barrier(kSchedValu, 4, 0);
    }
  };
  auto sched_k_dma = [&]() {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (r == 0) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 2, 0);
      else __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
      if (r < 14) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      if (r >= 8) __builtin_amdgcn_sched_group_barrier(kSchedValu, 4, 0);
    }
  };

  // Iteration kt (j = kt % 4: quarter qs = j of table column kt / 4, stage
  // j % 2) multiplies its stage.  On entry slot 0 holds the fragments of
  // k-step 0 and sw[stage] the stage's scale words.
  //  - at qs == 0 the ids of the next column are requested (5 loads), and at
  //    qs == 2 they are resolved, after the barrier;
  //  - the barrier waits for this iteration's other stage (its DMA was issued
  //    one iteration earlier; at qs == 0 only the 5 id loads may stay in
  //    flight);
  //  - after it the stage just multiplied, which no wave reads any more, gets
  //    stage kt + 2 (B slice fill_slice of rb_f, A quarter (qs + 2) % 4 of the
  //    resolved column), its DMA spread over the last k-step's MFMAs.
  auto iteration = [&](const int j, int ids_tm, int ids_col, bool ids_count,
                       __amdgpu_buffer_rsrc_t rb_f, int fill_slice) {
    const int stage = j & 1, qs = j;
    __builtin_amdgcn_sched_barrier(0);
    if (qs == 0) load_ids(ids_tm, ids_col, ids_count);
    __builtin_amdgcn_sched_barrier(0);
    const int nqs = (qs + 1) & 3;                    // the next iteration's quarter
    uint32_t need;
    load_b(stage, 1, 1);
    read_a(qs, 1);
    need = conv_a(qs, 1, 1);
    mfma_block(0);
    sched_k();
    fixup_a(need, 1);
    load_b(stage, 2, 0);
    read_a(qs, 2);
    need = conv_a(qs, 2, 0);
    mfma_block(1);
    sched_k();
    fixup_a(need, 0);
    load_b(stage, 3, 1);
    read_a(qs, 3);
    need = conv_a(qs, 3, 1);
    mfma_block(0);
    sched_k();
    fixup_a(need, 1);
    if (qs == 0) stage_barrier<waitcnt(kIdsPerLane, 0)>();
    else stage_barrier<waitcnt(0, 0)>();
    if (qs == 1) resolve();
    __builtin_amdgcn_sched_barrier(0);
    load_b(stage ^ 1, 0, 0);
    if (qs & 1) read_scales(nqs >> 1);
    read_a(nqs, 0);
    dma_b(rb_f, stage, fill_slice);
    if (qs & 1) dma_a(qs >> 1, qs >> 1);
    need = conv_a(nqs, 0, 0);
    mfma_block(1);
    sched_k_dma();
    fixup_a(need, 0);
  };

  // Prologue: the first tile's column 0 addresses, stage 0 in LDS, stage 1
  // in flight, the fragments of k-step 0.
  int tm, tn;
  tile_coords(lid, tiles_m, tiles_n, tm, tn);
  __amdgpu_buffer_rsrc_t rb = b_rsrc(B, N, K, tn);
  const bool counting = bad_ids != nullptr;
  load_ids(tm, 0, counting && tn == 0);
  resolve();
  dma_b(rb, 0, 0);
  dma_a(0, 0);
  stage_barrier<waitcnt(0, 0)>();
  dma_b(rb, 1, 1);
  dma_a(1, 1);
  load_b(0, 0, 0);
  read_scales(0);
  read_a(0, 0);
  fixup_a(conv_a(0, 0, 0), 0);

  for (;;) {
    const int next = lid + int(gridDim.x);
    const bool has_next = next < tiles;
    int tm2 = tm, tn2 = tn;
    if (has_next) tile_coords(next, tiles_m, tiles_n, tm2, tn2);
    const __amdgpu_buffer_rsrc_t rb2 = b_rsrc(B, N, K, tn2);
    // One table column per trip.  The ids requested are those of the next
    // column (the next tile's column 0 after the last; after the last tile,
    // this tile's last column again), and in the last column the stages get
    // the next tile's slices 0 and 1 (after the last tile, slice nk - 1 again:
    // nothing reads them).
    for (int c = 0; c < cols; ++c) {
      const int kt = 4 * c;
      const bool last = c + 1 == cols;
      const int ids_tm = last && has_next ? tm2 : tm;
      const int ids_col = last ? (has_next ? 0 : cols - 1) : c + 1;
      const bool ids_count = counting && (last ? has_next && tn2 == 0 : tn == 0);
      iteration(0, ids_tm, ids_col, ids_count, rb, kt + 2);
      iteration(1, ids_tm, ids_col, ids_count, rb, kt + 3);
      iteration(2, ids_tm, ids_col, ids_count, last && has_next ? rb2 : rb,
                last ? (has_next ? 0 : nk - 1) : kt + 4);
      iteration(3, ids_tm, ids_col, ids_count, last && has_next ? rb2 : rb,
                last ? (has_next ? 1 : nk - 1) : kt + 5);
    }
    store_wave_transposed<kRowsPerLane, kNJ, 1>(acc, stg, C, M, N,
                                                           tm * BM + wave * 64, tn * BN, lane);
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i)
#pragma unroll
      for (int j = 0; j < kNJ; ++j) acc[i][j] = f32x16{};
    if (!has_next) break;
    lid = next;
    tm = tm2;
    tn = tn2;
    rb = rb2;
  }
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));        // the last, unread reloads
  if (bad) atomicAdd(bad_ids, bad);
}

}  // namespace

hipError_t launch_project_fp8(const uint8_t *table, const uint8_t *scales, int64_t num_rows,
                              const int32_t *ids, int64_t ids_token_stride, int32_t cols,
                              const uint16_t *w, uint16_t *c, int32_t M, int32_t N,
                              int32_t *bad_ids, hipStream_t stream) {
  const int K = cols * ENGRAM_HEAD_DIM;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const size_t lds = size_t(kLdsLoop) + size_t(kWaves) * 32 * kStgStride * 2;
  const void *fn = reinterpret_cast<const void *>(&gemm_fp8_persistent_kernel);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemm_fp8_persistent_kernel,
                     dim3(persistent_grid(tiles_m * tiles_n, stream)), dim3(kThreads), lds, stream,
                     table, scales, num_rows, ids, ids_token_stride, w, c, M, N, K, tiles_m,
                     tiles_n, bad_ids);
  return hipGetLastError();
}

}  // namespace engram
