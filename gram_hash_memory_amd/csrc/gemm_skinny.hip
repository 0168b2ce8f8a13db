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

constexpr int kSkinnyM = 64;             // tokens per pass of the reduction through LDS
constexpr int kSkinnyWaves = 4;
constexpr int kSkinnyMaxTokens = 128;    // above this the 256 x 256 tiles of gemm.hip win

template <int NSUB>
constexpr int red_stride() { return 16 * NSUB + 4; }   // LDS row pitch (floats), bank spread

// Workgroup -> (column tile, token tile).  Up to 128 tokens there is one
// token tile; should a column tile have several, their ids are 8 apart: the
// dispatcher hands workgroups to the 8 XCDs in turn (id % 8), each XCD taking
// its share in id order, so they start together on one XCD and all but the
// first find most of the tile's wkv rows in that XCD's L2.  The grid covers
// the column tiles rounded up to a multiple of 8; ids past the last tile
// have nothing to do.
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

// 16-token fragments per workgroup.
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
// pulls TM * cols * 84 bytes of blocks from L2 instead of TM * cols * 512
// bytes of rows, and the rows never go to memory.  Same token tiles, K
// quarters, MFMAs in the same order and reduction: kv is bit-identical to
// engram_rows followed by the kernel above.  The quarters must be whole
// table columns (cols % 4 == 0).
//
// Lane (r, g) of a 16 x 32 A fragment holds token 16 i + r, values
// 32 s + 8 g .. + 7 of the column (s = step in the column, 0..7).  Those sit
// in 16-value group 2 s + g / 2 (scale/min byte of that index) and their
// quants in bytes 32 (s / 4) + 8 g .. + 7 of the 64 at bit 2 (s % 4).  The
// byte offsets of all the workgroup's blocks are resolved into LDS first; a
// column's blocks are then brought into the wave's own LDS area by LDS-DMA
// one column ahead (whole 84-byte blocks: a fraction of the memory requests
// of per-lane loads, which would compete with the wkv stream).  They stay
// there: each step reads, per token, the scale/min dword and the two quant
// dwords it decodes (d/dmin once per column), a step ahead.  Holding a
// column's 9 dwords per token in registers instead does not fit a 128-token
// tile at the widest column tiles.
constexpr uint32_t kQ2kNoRow = 0x7FFFFFF0u;   // block offset past the table: loads read 0

template <int MI>
constexpr int q2k_dma_per_col() { return (16 * MI + 2) / 3; }   // 3 blocks per instruction

template <int MI>
size_t q2k_skinny_loop_lds(int cols) {
  return (size_t(cols) * 16 * MI + size_t(kSkinnyWaves) * 2 * q2k_dma_per_col<MI>() * 64) *
         sizeof(uint32_t);
}

// How a weight-streaming Q2_K kernel decodes (q2k_decode.hpp): kQ2kVote
// votes per column and wave between the one-fma and the exact group decode;
// kQ2kFast always takes the one-fma decode, and kQ2kExactFixup, launched
// after it, checks its tile's blocks and, only if one needs it, recomputes
// the tile with the exact decode (for the 128-token tiles, which have no
// registers to spare for both decodes in one kernel).
enum Q2kDecode { kQ2kVote, kQ2kFast, kQ2kExactFixup };

template <int MI, int NSUB, int P, Q2kDecode kMode>
__global__ __launch_bounds__(kSkinnyWaves * 64, 1) void gemm_skinny_q2k_kernel(
    const uint8_t *__restrict__ table, int64_t num_rows, const int32_t *__restrict__ ids,
    int64_t ids_stride, const uint16_t *__restrict__ B, uint16_t *__restrict__ C, int M, int N,
    int K, int32_t *__restrict__ bad_ids) {
  constexpr int TM = 16 * MI;
  constexpr int NT = 16 * NSUB;
  // K loop: the block offsets [cols][TM], then each wave's two staging
  // areas; afterwards the [waves][64][RS] partial sums.
  extern __shared__ __attribute__((aligned(16))) float red[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SkinnyTile tile = skinny_tile((M + TM - 1) / TM);
  const int n0 = tile.n * NT;
  if (n0 >= N) return;                               // whole workgroup: grid rounding
  const int m0 = tile.m * TM;
  const int mrows = min(TM, M - m0);
  const int cols = K / ENGRAM_HEAD_DIM;
  const int wcols = cols / kSkinnyWaves;             // table columns of this wave's quarter
  const int c0 = wave * wcols;
  const int kbeg = c0 * ENGRAM_HEAD_DIM;
  const int nsteps = wcols * (ENGRAM_HEAD_DIM / 32);

  // Block offsets; ids outside the table are counted once per (token,
  // column), by the first column tile.
  uint32_t *const offs = reinterpret_cast<uint32_t *>(red);
  {
    int bad = 0;
    for (int idx = tid; idx < cols * TM; idx += kSkinnyWaves * 64) {
      const int c = idx / TM, t = idx % TM;
      const bool row_ok = t < mrows;
      const int32_t id = row_ok ? ids[int64_t(m0 + t) * ids_stride + c] : 0;
      const bool ok = id >= 0 && id < num_rows;
      bad += row_ok && !ok;
      offs[c * TM + t] = row_ok && ok ? uint32_t(id) * ENGRAM_Q2K_ROW_BYTES : kQ2kNoRow;
    }
    if (bad && tile.n == 0 && bad_ids) atomicAdd(bad_ids, bad);
  }
  __syncthreads();

  const __amdgpu_buffer_rsrc_t rt = make_rsrc(table, num_rows * ENGRAM_Q2K_ROW_BYTES);
  if constexpr (kMode == kQ2kExactFixup) {
    // The d/dmin word of every block of the tile, 8 requests in flight per
    // thread (missing rows point past the table and read 0); nothing to
    // redo unless one lies outside the one-fma range.
    bool fast = true;
    for (int base = 0; base < cols * TM; base += 8 * kSkinnyWaves * 64) {
      uint32_t d[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int idx = base + j * kSkinnyWaves * 64 + tid;
        d[j] = __builtin_amdgcn_raw_buffer_load_b32(
            rt, (idx < cols * TM ? offs[idx] : kQ2kNoRow) + 80, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) fast &= q2k_fp32_exact(d[j]);
    }
    if (__syncthreads_and(fast)) return;           // the first launch was exact already
  }

  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + int64_t(n0) * K, int64_t(N - n0) * K * 2);
  const int r = lane & 15, kg = lane >> 4;
  const uint32_t voff = uint32_t(r * K + 8 * kg) * 2;
  const uint32_t sub_step = uint32_t(16 * K) * 2;       // 16 rows further

  u32x4 fb[P][NSUB];
  auto load_b = [&](const int slot, int step) __attribute__((always_inline)) {
    const int k0 = kbeg + min(step, nsteps - 1) * 32;
#pragma unroll
    for (int j = 0; j < NSUB; ++j)
      fb[slot][j] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, voff + j * sub_step, k0 * 2, 0));
  };
  // A column's TM blocks go into this wave's LDS area by LDS-DMA, 3 blocks
  // of 21 dwords per instruction (lane L: block L / 21, dword L % 21; lane 63
  // and blocks past TM read past the table, i.e. nothing), spread over the
  // column's first kDmaSteps steps.  The area is the wave's own, so no
  // barrier.
  constexpr int kDmaPerCol = q2k_dma_per_col<MI>();        // 22 or 43
  constexpr int kDmaSteps = MI == 8 ? 4 : 1;
  constexpr int kDmaChunk = (kDmaPerCol + kDmaSteps - 1) / kDmaSteps;
  uint32_t *const stage_lds = offs + cols * TM + wave * 2 * kDmaPerCol * 64;
  const int dl_tok = lane / 21, dl_dw = lane % 21;
  auto dma_blocks = [&](const int buf, int c, const int kb, const int ke) __attribute__((always_inline)) {
    const uint32_t *o = offs + (c0 + min(c, wcols - 1)) * TM;   // wave-local column c, clamped
#pragma unroll
    for (int k = kb; k < ke; ++k) {
      const int t = 3 * k + dl_tok;
      const uint32_t ot = o[min(t, TM - 1)];
      const uint32_t off = (lane < 63 && t < TM) ? ot + 4 * dl_dw : kQ2kNoRow;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, stage_lds + (buf * kDmaPerCol + k) * 64, 4,
                                               off, 0, 0, 0);
    }
  };
  // The blocks stay in LDS; a step reads per token the scale/min dword and
  // the two quant dwords it decodes, one step ahead.  Token 16 i + r's block
  // of buffer `buf` starts at tok[i] + buf * kDmaPerCol * 64.
  const uint32_t *tok[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int t = 16 * i + r;
    tok[i] = stage_lds + (t / 3) * 64 + 21 * (t % 3);
  }
  uint32_t sc[2][MI], dd[MI];
  u32x2 qq[2][MI];
  auto read_step = [&](const int buf, const int s) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const uint32_t *b = tok[i] + buf * kDmaPerCol * 64;
      sc[s & 1][i] = b[s >> 1];
      qq[s & 1][i] = u32x2{b[4 + 8 * (s >> 2) + 2 * kg], b[5 + 8 * (s >> 2) + 2 * kg]};
    }
  };
  // A fragments of step s of the column: 16-value group 2 s + g / 2
  // (q2k_decode.hpp).  When any block of the column on this wave has d and
  // dmin too far apart for one fma per value (col_fast false, a wave-uniform
  // vote at the column start), the whole column takes the exact group decode.
  const int sc_shift = 8 * (kg >> 1);
  bool col_fast = kMode == kQ2kFast;
  auto decode = [&](const int s, u32x4 (&fa)[MI]) __attribute__((always_inline)) {
    if (kMode == kQ2kFast || (kMode == kQ2kVote && col_fast)) {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const uint32_t sm = (sc[s & 1][i] >> (16 * (s & 1) + sc_shift)) & 0xFFu;
        fa[i] = q2k_expand8(q2k_group_planes(dd[i], sm), qq[s & 1][i][0], qq[s & 1][i][1],
                            2 * (s & 3));
      }
    } else {
#pragma unroll
      for (int i = 0; i < MI; ++i) {      // one token at a time: few extra registers
        const uint32_t sm = (sc[s & 1][i] >> (16 * (s & 1) + sc_shift)) & 0xFFu;
        fa[i] = q2k_expand8(q2k_group_planes_exact(dd[i], sm), qq[s & 1][i][0],
                            qq[s & 1][i][1], 2 * (s & 3));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  f32x4v acc[MI][NSUB];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NSUB; ++j) acc[i][j] = f32x4v{};
  // One table column: its 8 steps, B of step t + P - 1 requested while step t
  // multiplies (step t's B sits in slot t % P), and the blocks of the next
  // column requested over its first kDmaSteps steps.
  auto column = [&](int c, const int set) __attribute__((always_inline)) {
    // Column c's blocks landed: only the B loads issued after the last of
    // their DMA instructions (9 - kDmaSteps steps' worth) may be in flight.
    __builtin_amdgcn_s_waitcnt(waitcnt((9 - kDmaSteps) * NSUB, 15));
    asm volatile("" ::: "memory");
    bool col_ok = true;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      dd[i] = tok[i][set * kDmaPerCol * 64 + 20];
      col_ok &= q2k_fp32_exact(dd[i]);
    }
    if (kMode == kQ2kVote) col_fast = __builtin_amdgcn_ballot_w64(!col_ok) == 0;
    read_step(set, 0);
#pragma unroll
    for (int s = 0; s < ENGRAM_HEAD_DIM / 32; ++s) {
      const int t = c * (ENGRAM_HEAD_DIM / 32) + s;
      if (s < kDmaSteps) {
        dma_blocks(set ^ 1, c + 1, s * kDmaChunk, min((s + 1) * kDmaChunk, kDmaPerCol));
        __builtin_amdgcn_sched_barrier(0);   // the wait above counts the B loads after these
      }
      load_b((s + P - 1) % P, t + P - 1);
      if (s + 1 < ENGRAM_HEAD_DIM / 32) read_step(set, s + 1);
      __builtin_amdgcn_sched_barrier(0);
      u32x4 fa[MI];
      decode(s, fa);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NSUB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, fa[i]), __builtin_bit_cast(bf16x8, fb[s % P][j]),
              acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  dma_blocks(0, 0, 0, kDmaPerCol);
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
  asm volatile("" ::: "memory");
#pragma unroll
  for (int p = 0; p < P - 1; ++p) load_b(p, p);
  for (int c = 0; c < wcols; c += 2) {
    column(c, 0);
    if (c + 1 < wcols) column(c + 1, 1);
  }

  // The last column still requested a (clamped) next column: its LDS-DMA
  // writes must land before the partial sums reuse the staging areas.
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
  asm volatile("" ::: "memory");
  reduce_store<MI, NSUB>(acc, red, C, N, m0, mrows, n0, wave, tid);
}

template <int MI, int NSUB, Q2kDecode kMode>
hipError_t launch_q2k_mode(const uint8_t *table, int64_t num_rows, const int32_t *ids,
                           int64_t ids_stride, const uint16_t *w, uint16_t *c, int32_t M,
                           int32_t K, int32_t N, int32_t *bad_ids, hipStream_t stream) {
  constexpr int P = 4;
  const int cols = K / ENGRAM_HEAD_DIM;
  const size_t lds = std::max(size_t(kSkinnyWaves) * kSkinnyM * red_stride<NSUB>() * sizeof(float),
                              q2k_skinny_loop_lds<MI>(cols));
  const void *fn = reinterpret_cast<const void *>(&gemm_skinny_q2k_kernel<MI, NSUB, P, kMode>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  const dim3 grid = skinny_grid(M, N, 16 * NSUB, 16 * MI);
  hipLaunchKernelGGL((gemm_skinny_q2k_kernel<MI, NSUB, P, kMode>), grid,
                     dim3(kSkinnyWaves * 64), lds, stream, table, num_rows, ids, ids_stride, w,
                     c, M, N, K, bad_ids);
  return hipGetLastError();
}

template <int MI, int NSUB>
hipError_t launch_q2k_nsub(const uint8_t *table, int64_t num_rows, const int32_t *ids,
                           int64_t ids_stride, const uint16_t *w, uint16_t *c, int32_t M,
                           int32_t K, int32_t N, int32_t *bad_ids, hipStream_t stream) {
  if constexpr (MI == 4) {
    return launch_q2k_mode<MI, NSUB, kQ2kVote>(table, num_rows, ids, ids_stride, w, c, M, K, N,
                                               bad_ids, stream);
  } else {
    hipError_t e = launch_q2k_mode<MI, NSUB, kQ2kFast>(table, num_rows, ids, ids_stride, w, c,
                                                       M, K, N, bad_ids, stream);
    if (e != hipSuccess) return e;
    return launch_q2k_mode<MI, NSUB, kQ2kExactFixup>(table, num_rows, ids, ids_stride, w, c, M,
                                                     K, N, nullptr, stream);
  }
}

template <int NSUB>
hipError_t launch_q2k_mi(const uint8_t *table, int64_t num_rows, const int32_t *ids,
                         int64_t ids_stride, const uint16_t *w, uint16_t *c, int32_t M,
                         int32_t K, int32_t N, int32_t *bad_ids, hipStream_t stream) {
  return skinny_mi(M) == 4
             ? launch_q2k_nsub<4, NSUB>(table, num_rows, ids, ids_stride, w, c, M, K, N, bad_ids, stream)
             : launch_q2k_nsub<8, NSUB>(table, num_rows, ids, ids_stride, w, c, M, K, N, bad_ids, stream);
}

// Stages 2 + 3 for few tokens, an FP8 table and an MXFP8 weight ([vLLM
// engram page, EngramBatch / wkv_input]): the MXFP8 projection of
// gemm_mx.hip in the weight-streaming form of the kernels above.  Each wave
// streams its K quarter of the tile's weight rows (1 byte per value plus one
// E8M0 byte per 32) from HBM into the operands of
// v_mfma_scale_f32_16x16x128_f8f6f4; the tokens' FP8 rows are multiplied as
// they are stored: E4M3 codes with one E8M0 scale per 32 values.
//
// Operand layout (16x16x128, 8-bit formats): lane 16 g + r holds row (A:
// token) or column (B: weight row) r, bytes 0..15 = k 16 g .. 16 g + 15 and
// bytes 16..31 = k 64 + 16 g .. 64 + 16 g + 15 of the instruction's 128; the
// scale of MX block q (k 32 q .. 32 q + 31) comes from lane group q, byte 0
// of its scale register (op_sel 0).  A 128-k step is half a table column, so
// a lane's scale dword for a step holds the step's four blocks and is
// shifted right by 8 g.
//
// The weight goes straight into registers, P steps ahead.  A column's 64 FP8
// rows (and their scale dwords) come into the wave's own LDS stage by
// LDS-DMA one column ahead, through 64-bit addresses (tables may exceed the
// 4 GB a buffer descriptor spans): 18 requests per column instead of two
// 16-byte loads per token and step beside the weight stream.  An id outside
// the table, or a token past T, reads a zero row (zero codes, so the product
// is exactly 0 whatever the scale, and zero scale bytes, 2^-127, finite).
// Token tiles of 64: two 64-token tiles, which pull the weight twice per CU,
// lose to the 256 x 256 tiles of gemm_mx.hip, so this form runs up to 64
// tokens, and up to kMxSkinnyMaxCols columns (its LDS).
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

__device__ __attribute__((aligned(256))) const uint8_t kMxZeroRow[ENGRAM_HEAD_DIM] = {};
constexpr uint32_t kMxNoRow = 0xFFFFFFFFu;

template <typename T>
__device__ __forceinline__ __attribute__((address_space(3))) void *lds_addr(T *p) {
  return (__attribute__((address_space(3))) void *)(p);
}

constexpr int kMxStageBytes = 64 * ENGRAM_HEAD_DIM + 64 * 8;   // a column: 64 rows + their scales
constexpr int kMxSkinnyMaxCols = 64;   // LDS: row indices + 4 waves x 2 stages <= 160 KB

template <int NSUB, int P>
__global__ __launch_bounds__(kSkinnyWaves * 64, 1) void gemm_skinny_mx_kernel(
    const uint8_t *__restrict__ table, const uint8_t *__restrict__ tscales, int64_t num_rows,
    const int32_t *__restrict__ ids, int64_t ids_stride, const uint8_t *__restrict__ W,
    const uint8_t *__restrict__ WS, uint16_t *__restrict__ C, int M, int N, int K,
    int32_t *__restrict__ bad_ids) {
  constexpr int MI = 4, TM = 16 * MI;
  constexpr int NT = 16 * NSUB;
  constexpr int kStep = 128;                          // k per instruction and step
  constexpr int kRowDma = TM * ENGRAM_HEAD_DIM / 1024; // 16-byte LDS-DMA instructions per column: 16
  // K loop: the row indices [cols][TM], then each wave's two column stages;
  // afterwards the [waves][64][RS] partial sums.
  extern __shared__ __attribute__((aligned(1024))) float red[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SkinnyTile tile = skinny_tile((M + TM - 1) / TM);
  const int n0 = tile.n * NT;
  if (n0 >= N) return;                               // whole workgroup: grid rounding
  const int m0 = tile.m * TM;
  const int mrows = min(TM, M - m0);
  const int cols = K / ENGRAM_HEAD_DIM;              // <= kMxSkinnyMaxCols
  const int wcols = cols / kSkinnyWaves;             // table columns of this wave's quarter
  const int c0 = wave * wcols;
  const int kbeg = c0 * ENGRAM_HEAD_DIM;
  const int nsteps = wcols * (ENGRAM_HEAD_DIM / kStep);
  const int ks = K / 32;                             // scale bytes per weight row

  // Row indices; ids outside the table are counted once per (token,
  // column), by the first column tile.
  uint32_t *const rowidx = reinterpret_cast<uint32_t *>(red);
  {
    int bad = 0;
    for (int idx = tid; idx < cols * TM; idx += kSkinnyWaves * 64) {
      const int c = idx / TM, t = idx % TM;
      const bool row_ok = t < mrows;
      const int32_t id = row_ok ? ids[int64_t(m0 + t) * ids_stride + c] : 0;
      const bool ok = id >= 0 && id < num_rows;
      bad += row_ok && !ok;
      rowidx[c * TM + t] = row_ok && ok ? uint32_t(id) : kMxNoRow;
    }
    if (bad && tile.n == 0 && bad_ids) atomicAdd(bad_ids, bad);
  }
  __syncthreads();

  // Weight rows n0 + 16 j + r; rows past N read as zeros (the row is part of
  // the range-checked VGPR offset, the SGPR offset carries the K position).
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(W + int64_t(n0) * K, int64_t(N - n0) * K);
  const __amdgpu_buffer_rsrc_t rbs = make_rsrc(WS + int64_t(n0) * ks, int64_t(N - n0) * ks);
  const int r = lane & 15, g = lane >> 4;
  const uint32_t voff_b = uint32_t(r * K + 16 * g);
  const uint32_t voff_bs = uint32_t(r * ks);

  i32x8 fb[P][NSUB];
  uint32_t sb[P][NSUB];
  auto cat = [](u32x4 lo, u32x4 hi) {
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // Weight operands of step u (clamped to the last) into slot `slot`.
  auto load_b = [&](const int slot, int u) {
    u = min(u, nsteps - 1);
    const int k0 = kbeg + u * kStep;
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      const uint32_t vo = voff_b + uint32_t(j * 16 * K);
      fb[slot][j] = cat(__builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, vo, k0, 0)),
                        __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, vo + 64, k0, 0)));
      sb[slot][j] = __builtin_amdgcn_raw_buffer_load_b32(rbs, voff_bs + uint32_t(j * 16 * ks),
                                                         k0 / 32, 0);
    }
  };
  // A column's 64 FP8 rows and their scale bytes go into this wave's LDS
  // stage by LDS-DMA, one column ahead: instruction k brings rows 4 k ..
  // 4 k + 3 (lane L: row 4 k + L / 16, physical 16-byte chunk L % 16), then
  // two bring the scale dwords ([2][64]).  Chunk q of row t is stored at
  // q ^ (t % 16), so the 16 rows a fragment read touches at one logical
  // chunk sit in 16 different bank groups.  The stage is the wave's own, so
  // no barrier.
  uint8_t *const stage = reinterpret_cast<uint8_t *>(rowidx + cols * TM) +
                         wave * 2 * kMxStageBytes;
  auto dma_rows = [&](const int buf, int c) {        // wave-local column c (clamped)
    const uint32_t *ri = rowidx + (c0 + min(c, wcols - 1)) * TM;
    uint8_t *st = stage + buf * kMxStageBytes;
    uint32_t ix[kRowDma];                            // all index reads first: one LDS wait
#pragma unroll
    for (int k = 0; k < kRowDma; ++k) ix[k] = ri[4 * k + (lane >> 4)];
#pragma unroll
    for (int k = 0; k < kRowDma; ++k) {
      const int t = 4 * k + (lane >> 4);
      const uint32_t idx = ix[k];
      const uint8_t *src = (idx != kMxNoRow ? table + int64_t(idx) * ENGRAM_HEAD_DIM : kMxZeroRow) +
                           16 * ((lane & 15) ^ (t & 15));
      __builtin_amdgcn_global_load_lds(src, lds_addr(st + k * 1024), 16, 0, 0);
    }
    const uint32_t idx = ri[lane];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const uint8_t *src = idx != kMxNoRow ? tscales + int64_t(idx) * (ENGRAM_HEAD_DIM / 32) + 4 * d
                                           : kMxZeroRow;
      __builtin_amdgcn_global_load_lds(src, lds_addr(st + 64 * ENGRAM_HEAD_DIM + d * 256), 4, 0, 0);
    }
  };
  // A operands of half h of the column in stage `buf`.
  i32x8 fa[MI];
  uint32_t sa[MI];
  auto read_a = [&](const int buf, const int h) {
    const uint8_t *st = stage + buf * kMxStageBytes;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const uint8_t *row = st + (16 * i + r) * ENGRAM_HEAD_DIM;
      fa[i] = cat(*reinterpret_cast<const u32x4 *>(row + 16 * ((8 * h + g) ^ r)),
                  *reinterpret_cast<const u32x4 *>(row + 16 * ((8 * h + 4 + g) ^ r)));
      sa[i] = *reinterpret_cast<const uint32_t *>(st + 64 * ENGRAM_HEAD_DIM + h * 256 +
                                                  4 * (16 * i + r));
    }
  };
  f32x4v acc[MI][NSUB];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NSUB; ++j) acc[i][j] = f32x4v{};
  auto mma = [&](const int slot) {
    uint32_t xa[MI], xb[NSUB];
#pragma unroll
    for (int i = 0; i < MI; ++i) xa[i] = sa[i] >> (8 * g);
#pragma unroll
    for (int j = 0; j < NSUB; ++j) xb[j] = sb[slot][j] >> (8 * g);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NSUB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            fa[i], fb[slot][j], acc[i][j], 0, 0, 0, xa[i], 0, xb[j]);
  };
  // Step u = 2 c + h of the wave's quarter: h = 0 waits for column c's rows
  // (only the weight loads of the two steps issued since their DMA may
  // still be in flight) and requests column c + 1's; then the weight of
  // step u + P - 1 is requested and step u multiplies.
  auto step = [&](int u, const int slot, const int h) {
    const int c = u >> 1;
    const int buf = c & 1;
    if (h == 0) {
      __builtin_amdgcn_s_waitcnt(waitcnt(2 * 3 * NSUB, 15));
      asm volatile("" ::: "memory");
      dma_rows(buf ^ 1, c + 1);
      __builtin_amdgcn_sched_barrier(0);   // the wait above counts the weight loads after these
    }
    load_b((slot + P - 1) % P, u + P - 1);
    __builtin_amdgcn_sched_barrier(0);
    read_a(buf, h);
    mma(slot);
    __builtin_amdgcn_sched_barrier(0);
  };

  dma_rows(0, 0);
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
  asm volatile("" ::: "memory");
#pragma unroll
  for (int p = 0; p < P - 1; ++p) load_b(p, p);
  // nsteps is even; P steps per group, u % P the slot and u % 2 the half.
  static_assert(P % 2 == 0, "the group of P steps must keep halves in phase");
  int u = 0;
  for (; u + P <= nsteps; u += P) {
#pragma unroll
    for (int q = 0; q < P; ++q) step(u + q, q, q & 1);
  }
#pragma unroll
  for (int q = 0; q < P; ++q)
    if (u + q < nsteps) step(u + q, q, q & 1);

  // The last column requested a (clamped) next one: its LDS-DMA writes must
  // land before the partial sums reuse the stages.
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
  asm volatile("" ::: "memory");
  reduce_store<MI, NSUB>(acc, red, C, N, m0, mrows, n0, wave, tid);
}

template <int NSUB>
hipError_t launch_mx_nsub(const uint8_t *table, const uint8_t *scales, int64_t num_rows,
                          const int32_t *ids, int64_t ids_stride, const uint8_t *w_codes,
                          const uint8_t *w_scales, uint16_t *c, int32_t M, int32_t K, int32_t N,
                          int32_t *bad_ids, hipStream_t stream) {
  constexpr int P = 4;
  const int cols = K / ENGRAM_HEAD_DIM;
  const size_t lds = std::max(size_t(kSkinnyWaves) * kSkinnyM * red_stride<NSUB>() * sizeof(float),
                              size_t(cols) * kSkinnyM * sizeof(uint32_t) +
                                  size_t(kSkinnyWaves) * 2 * kMxStageBytes);
  const void *fn = reinterpret_cast<const void *>(&gemm_skinny_mx_kernel<NSUB, P>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  const dim3 grid = skinny_grid(M, N, 16 * NSUB, kSkinnyM);
  hipLaunchKernelGGL((gemm_skinny_mx_kernel<NSUB, P>), grid, dim3(kSkinnyWaves * 64), lds,
                     stream, table, scales, num_rows, ids, ids_stride, w_codes, w_scales, c, M,
                     N, K, bad_ids);
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
    case 1: return launch_q2k_mi<1>(table, num_rows, ids, ids_token_stride, w, c, M, K, N, bad_ids, stream);
    case 2: return launch_q2k_mi<2>(table, num_rows, ids, ids_token_stride, w, c, M, K, N, bad_ids, stream);
    case 3: return launch_q2k_mi<3>(table, num_rows, ids, ids_token_stride, w, c, M, K, N, bad_ids, stream);
    case 4: return launch_q2k_mi<4>(table, num_rows, ids, ids_token_stride, w, c, M, K, N, bad_ids, stream);
    default: return launch_q2k_mi<5>(table, num_rows, ids, ids_token_stride, w, c, M, K, N, bad_ids, stream);
  }
}

}  // namespace engram

namespace engram {

bool project_mx_skinny_supported(int32_t M, int32_t cols) {
  return M <= kSkinnyM && cols % kSkinnyWaves == 0 && cols <= kMxSkinnyMaxCols;
}

hipError_t launch_project_mx_skinny(const uint8_t *table, const uint8_t *scales, int64_t num_rows,
                                    const int32_t *ids, int64_t ids_token_stride, int32_t cols,
                                    const uint8_t *w_codes, const uint8_t *w_scales, uint16_t *c,
                                    int32_t M, int32_t N, int32_t *bad_ids, hipStream_t stream) {
  const int32_t K = cols * ENGRAM_HEAD_DIM;
#define ENGRAM_MX_NSUB(n)                                                                   \
  return launch_mx_nsub<n>(table, scales, num_rows, ids, ids_token_stride, w_codes, w_scales, \
                           c, M, K, N, bad_ids, stream)
  switch (skinny_nsub(N)) {
    case 1: ENGRAM_MX_NSUB(1);
    case 2: ENGRAM_MX_NSUB(2);
    case 3: ENGRAM_MX_NSUB(3);
    case 4: ENGRAM_MX_NSUB(4);
    default: ENGRAM_MX_NSUB(5);
  }
#undef ENGRAM_MX_NSUB
}

}  // namespace engram
