// Stage 3 for few tokens (decode): kv = rows x wkv^T when T is small.
//
// [spark engram_v41 page, overview stage 3]: the same bf16 projection as
// gemm.hip.  With a few dozen tokens the 256 x 256 tiles of gemm.hip leave
// most of the chip idle and most of each tile empty, while the work itself
// is bound by streaming wkv ((hc + 1) * dim rows of cols * 256 bf16, 252 MB
// in the DeepSeek-V4.1 shape) from HBM once.  This kernel is built for that:
//
//  - one workgroup per NT = 16 * NSUB output columns and per 64 tokens, with
//    NSUB chosen so that the column tiles about fill the 256 CUs;
//  - its 4 waves split K in four and each streams its quarter of the NT wkv
//    rows straight from HBM into MFMA B fragments (v_mfma_f32_16x16x32_bf16:
//    lane l holds 8 consecutive k of row l % 16, starting at k = 8 * (l / 16)),
//    with P steps of 32 k in flight per wave;
//  - the A fragments (the tokens' rows, a few hundred KB shared by every
//    workgroup) come from L2 the same way;
//  - the four partial sums are added in LDS in a fixed order, so results do
//    not depend on timing, and rounded to bf16 once.
#include <algorithm>

#include "gemm_common.hpp"

namespace engram {
namespace {

using namespace gemm;

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kSkinnyM = 64;             // tokens per workgroup
constexpr int kSkinnyWaves = 4;
constexpr int kSkinnyMaxTokens = 128;    // above this the 256 x 256 tiles of gemm.hip win

template <int NSUB>
constexpr int red_stride() { return 16 * NSUB + 4; }   // LDS row pitch (floats), bank spread

template <int NSUB, int P>
__global__ __launch_bounds__(kSkinnyWaves * 64, 1) void gemm_skinny_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, uint16_t *__restrict__ C,
    int M, int N, int K) {
  constexpr int NT = 16 * NSUB;
  constexpr int RS = red_stride<NSUB>();
  extern __shared__ __attribute__((aligned(16))) float red[];   // [waves][64][RS]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * NT;
  const int m0 = blockIdx.y * kSkinnyM;
  const int mrows = min(kSkinnyM, M - m0);

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

  u32x4 fa[P][4], fb[P][NSUB];
  auto load = [&](const int slot, int step) {
    const int k0 = kbeg + min(step, nsteps - 1) * 32;
#pragma unroll
    for (int j = 0; j < NSUB; ++j)
      fb[slot][j] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, voff + j * sub_step, k0 * 2, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      fa[slot][i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, voff + i * sub_step, k0 * 2, 0));
  };
  f32x4v acc[4][NSUB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NSUB; ++j) acc[i][j] = f32x4v{};
  auto mma = [&](const int slot) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
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

  // Partial sums -> LDS [wave][row][col]; D of a 16 x 16 block: lane l holds
  // column l % 16 of rows 4 * (l / 16) .. + 3.
  float *mine = red + wave * kSkinnyM * RS;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NSUB; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        mine[(16 * i + 4 * kg + e) * RS + 16 * j + r] = acc[i][j][e];
  __syncthreads();
  for (int idx = tid; idx < kSkinnyM * NT; idx += kSkinnyWaves * 64) {
    const int m = idx / NT, n = idx % NT;
    float s = red[m * RS + n];
#pragma unroll
    for (int w = 1; w < kSkinnyWaves; ++w) s += red[(w * kSkinnyM + m) * RS + n];
    if (m < mrows && n0 + n < N) C[int64_t(m0 + m) * N + n0 + n] = f32_to_bf16(s);
  }
}

template <int NSUB>
hipError_t launch_nsub(const uint16_t *a, const uint16_t *w, uint16_t *c, int32_t M, int32_t K,
                       int32_t N, hipStream_t stream) {
  constexpr int P = 4;
  const size_t lds = size_t(kSkinnyWaves) * kSkinnyM * red_stride<NSUB>() * sizeof(float);
  const void *fn = reinterpret_cast<const void *>(&gemm_skinny_kernel<NSUB, P>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  const dim3 grid((N + 16 * NSUB - 1) / (16 * NSUB), (M + kSkinnyM - 1) / kSkinnyM);
  hipLaunchKernelGGL((gemm_skinny_kernel<NSUB, P>), grid, dim3(kSkinnyWaves * 64), lds, stream,
                     a, w, c, M, N, K);
  return hipGetLastError();
}

}  // namespace

bool project_uses_skinny(int32_t M) { return M <= kSkinnyMaxTokens; }

hipError_t launch_project_skinny(const uint16_t *a, const uint16_t *w, uint16_t *c, int32_t M,
                                 int32_t K, int32_t N, hipStream_t stream) {
  // Column tiles of 16 * NSUB, NSUB as small as lets about one tile per CU
  // cover N (the wkv stream is what bounds the kernel).
  const int64_t per_cu = (int64_t(N) + 255) / 256;
  const int nsub = int(std::min<int64_t>(5, std::max<int64_t>(1, (per_cu + 15) / 16)));
  switch (nsub) {
    case 1: return launch_nsub<1>(a, w, c, M, K, N, stream);
    case 2: return launch_nsub<2>(a, w, c, M, K, N, stream);
    case 3: return launch_nsub<3>(a, w, c, M, K, N, stream);
    case 4: return launch_nsub<4>(a, w, c, M, K, N, stream);
    default: return launch_nsub<5>(a, w, c, M, K, N, stream);
  }
}

}  // namespace engram
