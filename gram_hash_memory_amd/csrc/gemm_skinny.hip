// Stage 3 for few tokens (decode): kv = rows x wkv^T when T is small.
//
// [spark engram_v41 page, overview stage 3]: the same bf16 projection as
// gemm.hip.  With a few dozen tokens the 256 x 256 tiles of gemm.hip leave
// most of the chip idle and most of each tile empty, while the work itself
// is bound by streaming wkv ((hc + 1) * dim rows of cols * 256 bf16, 252 MB
// in the DeepSeek-V4.1 shape) from HBM once.  This kernel is built for that:
//
//  - one workgroup per NT = 16 * NSUB output columns and per 16 * MI tokens
//    (MI = 4 up to 64 tokens, else 8), with NSUB chosen so that the column
//    tiles about fill the 256 CUs: up to 128 tokens, every CU pulls its
//    share of wkv once;
//  - its 4 waves split K in four and each streams its quarter of the NT wkv
//    rows straight from HBM into MFMA B fragments (v_mfma_f32_16x16x32_bf16:
//    lane l holds 8 consecutive k of row l % 16, starting at k = 8 * (l / 16)),
//    with P steps of 32 k in flight per wave;
//  - the A fragments (the tokens' rows, a few hundred KB shared by every
//    workgroup) come from L2 the same way;
//  - the four partial sums are added in LDS in a fixed order, so results do
//    not depend on timing, and rounded to bf16 once.  Each output's sum runs
//    over the same k in the same order whatever the token tile.
#include <algorithm>

#include "gemm_common.hpp"
#include "q2k_decode.hpp"

namespace engram {
namespace {

using namespace gemm;

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kSkinnyM = 64;             // tokens per workgroup of the Q2_K kernel; reduction pass
constexpr int kSkinnyWaves = 4;
constexpr int kSkinnyMaxTokens = 128;    // above this the 256 x 256 tiles of gemm.hip win

template <int NSUB>
constexpr int red_stride() { return 16 * NSUB + 4; }   // LDS row pitch (floats), bank spread

// Workgroup -> (column tile, token tile).  The dispatcher hands workgroups to
// the 8 XCDs in turn (id % 8), each XCD taking its share in id order, so ids
// L and L + 8 start on one XCD at about the same time.  The token tiles of a
// column tile get ids 8 apart: after the first, they find most of the tile's
// wkv rows in that XCD's L2 rather than in HBM.  The grid covers the column
// tiles rounded up to a multiple of 8; ids past the last tile have nothing
// to do.
struct SkinnyTile {
  int n, m;
};
__device__ __forceinline__ SkinnyTile skinny_tile(int tiles_m) {
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  return {(slot / tiles_m) * 8 + xcd, slot % tiles_m};
}

inline dim3 skinny_grid(int32_t M, int32_t N, int nt, int tm) {
  const int tiles_n = (N + nt - 1) / nt, tiles_m = (M + tm - 1) / tm;
  return dim3(((tiles_n + 7) / 8) * 8 * tiles_m);
}

// 16-token fragments per workgroup of the bf16 kernel.
inline int skinny_mi(int32_t M) { return M <= 64 ? 4 : 8; }

// The waves' partial sums -> LDS [wave][64][RS], then added in wave order
// and rounded to bf16 once, 64 tokens at a time.  D of a 16 x 16 block: lane
// l holds column l % 16 of rows 4 * (l / 16) .. + 3.  Starts with a barrier,
// so the LDS may still be in use by the K loop.
template <int MI, int NSUB>
__device__ __forceinline__ void reduce_store(const f32x4v (&acc)[MI][NSUB], float *red,
                                             uint16_t *__restrict__ C, int N, int m0, int mrows,
                                             int n0, int wave, int tid) {
  constexpr int NT = 16 * NSUB;
  constexpr int RS = red_stride<NSUB>();
  const int lane = tid & 63, r = lane & 15, kg = lane >> 4;
  float *mine = red + wave * kSkinnyM * RS;
#pragma unroll
  for (int h = 0; h < MI / 4; ++h) {
    if (kSkinnyM * h >= mrows) break;                // uniform: no token left
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NSUB; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          mine[(16 * i + 4 * kg + e) * RS + 16 * j + r] = acc[4 * h + i][j][e];
    __syncthreads();
    for (int idx = tid; idx < kSkinnyM * NT; idx += kSkinnyWaves * 64) {
      const int m = idx / NT, n = idx % NT;
      float sum = red[m * RS + n];
#pragma unroll
      for (int w = 1; w < kSkinnyWaves; ++w) sum += red[(w * kSkinnyM + m) * RS + n];
      const int mm = kSkinnyM * h + m;
      if (mm < mrows && n0 + n < N) C[int64_t(m0 + mm) * N + n0 + n] = f32_to_bf16(sum);
    }
  }
}

template <int MI, int NSUB, int P>
__global__ __launch_bounds__(kSkinnyWaves * 64, 1) void gemm_skinny_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, uint16_t *__restrict__ C,
    int M, int N, int K) {
  constexpr int NT = 16 * NSUB;
  constexpr int TM = 16 * MI;
  extern __shared__ __attribute__((aligned(16))) float red[];   // [waves][64][RS]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SkinnyTile tile = skinny_tile((M + TM - 1) / TM);
  const int n0 = tile.n * NT;
  if (n0 >= N) return;                               // whole workgroup: grid rounding
  const int m0 = tile.m * TM;
  const int mrows = min(TM, M - m0);

  // K quarter of this wave, in whole steps of 32 (K % 64 == 0).
  const int kq = ((K / kSkinnyWaves + 31) / 32) * 32;
  const int kbeg = min(K, wave * kq);
  const int kend = min(K, kbeg + kq);
  const int nsteps = (kend - kbeg) / 32;

  // Rows past the token count or past N read as zeros (buffer range check).
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + int64_t(m0) * K, int64_t(mrows) * K * 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + int64_t(n0) * K, int64_t(N - n0) * K * 2);
  const int r = lane & 15, kg = lane >> 4;
  const uint32_t voff = uint32_t(r * K + 8 * kg) * 2;
  const uint32_t sub_step = uint32_t(16 * K) * 2;       // 16 rows further

  u32x4 fa[P][MI], fb[P][NSUB];
  auto load = [&](const int slot, int step) {
    const int k0 = kbeg + min(step, nsteps - 1) * 32;
#pragma unroll
    for (int j = 0; j < NSUB; ++j)
      fb[slot][j] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, voff + j * sub_step, k0 * 2, 0));
#pragma unroll
    for (int i = 0; i < MI; ++i)
      fa[slot][i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, voff + i * sub_step, k0 * 2, 0));
  };
  f32x4v acc[MI][NSUB];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NSUB; ++j) acc[i][j] = f32x4v{};
  auto mma = [&](const int slot) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NSUB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, fa[slot][i]), __builtin_bit_cast(bf16x8, fb[slot][j]),
            acc[i][j], 0, 0, 0);
  };

  if (nsteps > 0) {
#pragma unroll
    for (int p = 0; p < P - 1; ++p) load(p, p);
    int s = 0;
    // Full groups of P steps: step s + q is multiplied from slot q while the
    // load of step s + q + P - 1 goes into the slot freed one step earlier.
    for (; s + P <= nsteps; s += P) {
#pragma unroll
      for (int q = 0; q < P; ++q) {
        load((q + P - 1) % P, s + q + P - 1);
        // Keep the loads ahead of the MFMAs: the compiler would otherwise sink
        // them towards their use and shorten the prefetch distance.
        __builtin_amdgcn_sched_barrier(0);
        mma(q);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Tail (nsteps % P steps): their loads are already in slots 0 .. nsteps % P - 1.
#pragma unroll
    for (int q = 0; q < P - 1; ++q)
      if (s + q < nsteps) mma(q);
  }

  reduce_store<MI, NSUB>(acc, red, C, N, m0, mrows, n0, wave, tid);
}

template <int MI, int NSUB>
hipError_t launch_nsub(const uint16_t *a, const uint16_t *w, uint16_t *c, int32_t M, int32_t K,
                       int32_t N, hipStream_t stream) {
  constexpr int P = 4;
  const size_t lds = size_t(kSkinnyWaves) * kSkinnyM * red_stride<NSUB>() * sizeof(float);
  const void *fn = reinterpret_cast<const void *>(&gemm_skinny_kernel<MI, NSUB, P>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  const dim3 grid = skinny_grid(M, N, 16 * NSUB, 16 * MI);
  hipLaunchKernelGGL((gemm_skinny_kernel<MI, NSUB, P>), grid, dim3(kSkinnyWaves * 64), lds,
                     stream, a, w, c, M, N, K);
  return hipGetLastError();
}

template <int NSUB>
hipError_t launch_mi(const uint16_t *a, const uint16_t *w, uint16_t *c, int32_t M, int32_t K,
                     int32_t N, hipStream_t stream) {
  return skinny_mi(M) == 4 ? launch_nsub<4, NSUB>(a, w, c, M, K, N, stream)
                           : launch_nsub<8, NSUB>(a, w, c, M, K, N, stream);
}

// Stages 2 + 3 fused for few tokens and a Q2_K table ([spark engram_v41
// page, overview stages 2-3]): the kernel above with A decoded on chip from
// the tokens' 84-byte blocks instead of read as bf16 rows.  A workgroup then
// pulls 64 * cols * 84 bytes of blocks from L2 instead of 64 * cols * 512
// bytes of rows, and the rows never go to memory.  Same K quarters, same
// MFMAs in the same order, same reduction: kv is bit-identical to
// engram_rows followed by the kernel above.  The quarters must be whole
// table columns (cols % 4 == 0).
//
// Lane (r, g) of a 16 x 32 A fragment holds token 16 i + r, values
// 32 s + 8 g .. + 7 of the column (s = step in the column, 0..7).  Those sit
// in 16-value group 2 s + g / 2 (scale/min byte of that index) and their
// quants in bytes 32 (s / 4) + 8 g .. + 7 of the 64 at bit 2 (s % 4).  So per
// token and column a lane keeps 16 quant bytes, the 16 scale/min bytes and
// d/dmin (9 dwords).  The byte offsets of all the workgroup's blocks are
// resolved into LDS first; a column's blocks are then brought into the
// wave's own LDS area by LDS-DMA one column ahead (whole 84-byte blocks: a
// fraction of the memory requests of per-lane loads, which would compete with
// the wkv stream), and each lane reads its 9 dwords per token from there.
//
// Its token tile stays at 64 (a 128-token tile needs more than the 512
// registers of a lane at the widest column tiles); 65-128 tokens run two
// token tiles per column tile, paired on one XCD by skinny_tile.
constexpr uint32_t kQ2kNoRow = 0x7FFFFFF0u;   // block offset past the table: loads read 0

struct Q2kLaneBlock {
  u32x4 sc;          // scale/min bytes 0..15
  u32x2 q[2];        // quant bytes 8 g .. 8 g + 7 and 32 + 8 g .. 32 + 8 g + 7
  uint32_t dd;       // fp16 d | fp16 dmin << 16
};

template <int NSUB, int P>
__global__ __launch_bounds__(kSkinnyWaves * 64, 1) void gemm_skinny_q2k_kernel(
    const uint8_t *__restrict__ table, int64_t num_rows, const int32_t *__restrict__ ids,
    int64_t ids_stride, const uint16_t *__restrict__ B, uint16_t *__restrict__ C, int M, int N,
    int K, int32_t *__restrict__ bad_ids) {
  constexpr int NT = 16 * NSUB;
  constexpr int RS = red_stride<NSUB>();
  // [waves][64][RS] partial sums, then the block offsets [cols][64]
  extern __shared__ __attribute__((aligned(16))) float red[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SkinnyTile tile = skinny_tile((M + kSkinnyM - 1) / kSkinnyM);
  const int n0 = tile.n * NT;
  if (n0 >= N) return;                               // whole workgroup: grid rounding
  const int m0 = tile.m * kSkinnyM;
  const int mrows = min(kSkinnyM, M - m0);
  const int cols = K / ENGRAM_HEAD_DIM;
  const int wcols = cols / kSkinnyWaves;             // table columns of this wave's quarter
  const int c0 = wave * wcols;
  const int kbeg = c0 * ENGRAM_HEAD_DIM;
  const int nsteps = wcols * (ENGRAM_HEAD_DIM / 32);

  // Block offsets; ids outside the table are counted once per (token,
  // column), by the first column tile.
  uint32_t *const offs = reinterpret_cast<uint32_t *>(red + kSkinnyWaves * kSkinnyM * RS);
  {
    const int t = tid & 63;
    const bool row_ok = t < mrows;
    int bad = 0;
    for (int c = tid >> 6; c < cols; c += kSkinnyWaves) {
      const int32_t id = row_ok ? ids[int64_t(m0 + t) * ids_stride + c] : 0;
      const bool ok = id >= 0 && id < num_rows;
      bad += row_ok && !ok;
      offs[c * kSkinnyM + t] = row_ok && ok ? uint32_t(id) * ENGRAM_Q2K_ROW_BYTES : kQ2kNoRow;
    }
    if (bad && tile.n == 0 && bad_ids) atomicAdd(bad_ids, bad);
  }
  __syncthreads();

  const __amdgpu_buffer_rsrc_t rt = make_rsrc(table, num_rows * ENGRAM_Q2K_ROW_BYTES);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + int64_t(n0) * K, int64_t(N - n0) * K * 2);
  const int r = lane & 15, kg = lane >> 4;
  const uint32_t voff = uint32_t(r * K + 8 * kg) * 2;
  const uint32_t sub_step = uint32_t(16 * K) * 2;       // 16 rows further

  u32x4 fb[P][NSUB];
  auto load_b = [&](const int slot, int step) {
    const int k0 = kbeg + min(step, nsteps - 1) * 32;
#pragma unroll
    for (int j = 0; j < NSUB; ++j)
      fb[slot][j] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, voff + j * sub_step, k0 * 2, 0));
  };
  Q2kLaneBlock blk[2][4];
  // A column's 64 blocks go into this wave's LDS area by LDS-DMA, 3 blocks
  // of 21 dwords per instruction (lane L: block L / 21, dword L % 21; lane 63
  // reads past the table, i.e. nothing), then each lane reads the 9 dwords
  // per token it keeps.  The area is the wave's own, so no barrier.
  constexpr int kDmaPerCol = (kSkinnyM + 2) / 3;           // 22
  uint32_t *const stage_lds = offs + cols * kSkinnyM + wave * 2 * kDmaPerCol * 64;
  const int dl_tok = lane / 21, dl_dw = lane % 21;
  auto dma_blocks = [&](const int buf, int c) {            // wave-local column c (clamped)
    const uint32_t *o = offs + (c0 + min(c, wcols - 1)) * kSkinnyM;
#pragma unroll
    for (int k = 0; k < kDmaPerCol; ++k) {
      const int t = 3 * k + dl_tok;
      const uint32_t off = (lane < 63 && t < kSkinnyM) ? o[t] + 4 * dl_dw : kQ2kNoRow;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, stage_lds + (buf * kDmaPerCol + k) * 64, 4,
                                               off, 0, 0, 0);
    }
  };
  auto read_blocks = [&](const int set, const int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * i + r;
      const uint32_t *b = stage_lds + (buf * kDmaPerCol + t / 3) * 64 + 21 * (t % 3);
      blk[set][i].sc = u32x4{b[0], b[1], b[2], b[3]};
#pragma unroll
      for (int h = 0; h < 2; ++h) blk[set][i].q[h] = u32x2{b[4 + 8 * h + 2 * kg], b[5 + 8 * h + 2 * kg]};
      blk[set][i].dd = b[20];
    }
  };
  // A fragments of step s of the column from register set `set`: 16-value
  // group 2 s + g / 2 (q2k_decode.hpp).
  const int sc_shift = 8 * (kg >> 1);
  auto decode = [&](const int set, const int s, u32x4 (&fa)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const Q2kLaneBlock &b = blk[set][i];
      const Q2kPlanes pl =
          q2k_group_planes(b.dd, (b.sc[s >> 1] >> (16 * (s & 1) + sc_shift)) & 0xFFu);
      fa[i] = q2k_expand8(pl, b.q[s >> 2][0], b.q[s >> 2][1], 2 * (s & 3));
    }
  };
  f32x4v acc[4][NSUB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NSUB; ++j) acc[i][j] = f32x4v{};
  // One table column: its 8 steps, B of step t + P - 1 requested while step t
  // multiplies (step t's B sits in slot t % P), and the blocks of the next
  // column requested at its start.
  auto column = [&](int c, const int set) {
    // Column c's blocks landed: only the 8 steps' B loads issued since their
    // DMA (one column ago) may still be in flight.
    __builtin_amdgcn_s_waitcnt(waitcnt(8 * NSUB, 15));
    asm volatile("" ::: "memory");
    read_blocks(set, set);
    dma_blocks(set ^ 1, c + 1);
#pragma unroll
    for (int s = 0; s < ENGRAM_HEAD_DIM / 32; ++s) {
      const int t = c * (ENGRAM_HEAD_DIM / 32) + s;
      load_b((s + P - 1) % P, t + P - 1);
      __builtin_amdgcn_sched_barrier(0);
      u32x4 fa[4];
      decode(set, s, fa);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NSUB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, fa[i]), __builtin_bit_cast(bf16x8, fb[s % P][j]),
              acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  dma_blocks(0, 0);
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
  asm volatile("" ::: "memory");
#pragma unroll
  for (int p = 0; p < P - 1; ++p) load_b(p, p);
  for (int c = 0; c < wcols; c += 2) {
    column(c, 0);
    if (c + 1 < wcols) column(c + 1, 1);
  }

  reduce_store<4, NSUB>(acc, red, C, N, m0, mrows, n0, wave, tid);
}

template <int NSUB>
hipError_t launch_q2k_nsub(const uint8_t *table, int64_t num_rows, const int32_t *ids,
                           int64_t ids_stride, const uint16_t *w, uint16_t *c, int32_t M,
                           int32_t K, int32_t N, int32_t *bad_ids, hipStream_t stream) {
  constexpr int P = 4;
  const int cols = K / ENGRAM_HEAD_DIM;
  const size_t lds = size_t(kSkinnyWaves) * kSkinnyM * red_stride<NSUB>() * sizeof(float) +
                     size_t(cols) * kSkinnyM * sizeof(uint32_t) +
                     size_t(kSkinnyWaves) * 2 * ((kSkinnyM + 2) / 3) * 64 * sizeof(uint32_t);
  const void *fn = reinterpret_cast<const void *>(&gemm_skinny_q2k_kernel<NSUB, P>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  const dim3 grid = skinny_grid(M, N, 16 * NSUB, kSkinnyM);
  hipLaunchKernelGGL((gemm_skinny_q2k_kernel<NSUB, P>), grid, dim3(kSkinnyWaves * 64), lds,
                     stream, table, num_rows, ids, ids_stride, w, c, M, N, K, bad_ids);
  return hipGetLastError();
}

int skinny_nsub(int32_t N) {
  // Column tiles of 16 * NSUB, NSUB as small as lets about one tile per CU
  // cover N (the wkv stream is what bounds the kernel).
  const int64_t per_cu = (int64_t(N) + 255) / 256;
  return int(std::min<int64_t>(5, std::max<int64_t>(1, (per_cu + 15) / 16)));
}

}  // namespace

bool project_uses_skinny(int32_t M) { return M <= kSkinnyMaxTokens; }

hipError_t launch_project_skinny(const uint16_t *a, const uint16_t *w, uint16_t *c, int32_t M,
                                 int32_t K, int32_t N, hipStream_t stream) {
  switch (skinny_nsub(N)) {
    case 1: return launch_mi<1>(a, w, c, M, K, N, stream);
    case 2: return launch_mi<2>(a, w, c, M, K, N, stream);
    case 3: return launch_mi<3>(a, w, c, M, K, N, stream);
    case 4: return launch_mi<4>(a, w, c, M, K, N, stream);
    default: return launch_mi<5>(a, w, c, M, K, N, stream);
  }
}

}  // namespace engram

namespace engram {

bool project_q2k_skinny_supported(int32_t M, int32_t cols) {
  return project_uses_skinny(M) && cols % kSkinnyWaves == 0;
}

hipError_t launch_project_q2k_skinny(const uint8_t *table, int64_t num_rows, const int32_t *ids,
                                     int64_t ids_token_stride, int32_t cols, const uint16_t *w,
                                     uint16_t *c, int32_t M, int32_t N, int32_t *bad_ids,
                                     hipStream_t stream) {
  const int32_t K = cols * ENGRAM_HEAD_DIM;
  switch (skinny_nsub(N)) {
    case 1: return launch_q2k_nsub<1>(table, num_rows, ids, ids_token_stride, w, c, M, K, N, bad_ids, stream);
    case 2: return launch_q2k_nsub<2>(table, num_rows, ids, ids_token_stride, w, c, M, K, N, bad_ids, stream);
    case 3: return launch_q2k_nsub<3>(table, num_rows, ids, ids_token_stride, w, c, M, K, N, bad_ids, stream);
    case 4: return launch_q2k_nsub<4>(table, num_rows, ids, ids_token_stride, w, c, M, K, N, bad_ids, stream);
    default: return launch_q2k_nsub<5>(table, num_rows, ids, ids_token_stride, w, c, M, K, N, bad_ids, stream);
  }
}

}  // namespace engram
