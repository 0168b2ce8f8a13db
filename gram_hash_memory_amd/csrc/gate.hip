// Stage 4: the Engram gate, in place on the fp32 highway.
//
// [spark engram_v41 page, overview stage 4]: normalised dot of stream and
// key, signed square root, sigmoid, h += gate * value on the fp32 [T, hc, H]
// highway.  [NeMo engram page, _engram_gate_core / compile_engram_gate]: the
// three hidden-dim reductions (stream RMS, key RMS, stream-key dot) are
// fused into one pass over the fp32 streams; masked tokens keep their
// streams.  [vLLM engram page, Engram]: one key per stream plus a shared
// value; clamp 1e-6 before the square root.
//
// One workgroup per token (or, for a few tokens, per token and stream: see
// launch_gate).  Every thread loads its 8-wide slices of all hc streams into
// registers, together with the matching key and value slices.
// It accumulates the 3*hc partial sums, and the sums are reduced with wave
// shuffles plus one LDS exchange.  Each thread then derives the hc gates and
// writes x + g * v from the registers, so h is read once and written once
// and the shared value once per token (not once per stream).  Masked tokens
// return before touching memory, which leaves them bit-for-bit unchanged.
//
// Several engram layers that act on the same highway one after the other
// (the forward's layers, with nothing in between) run in one pass: the
// streams stay in registers from one layer's gate to the next, so h is read
// and written once for all of them.  Each layer's arithmetic is the
// single-layer kernel's, on the same fp32 values, so the result is bit for
// bit that of separate calls.
#include "common.hpp"

namespace engram {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kVec = 8;                       // elements per thread per chunk

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ void bf16x8_to_f32(const u32x4 w, float *f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
}

// HC streams per workgroup; with SPLIT the workgroup handles stream
// blockIdx.x % hc of token blockIdx.x / hc only (HC = 1 then, hc the real
// stream count): the value is then read once per stream, but a decode batch
// of a few dozen tokens spreads over hc times more workgroups.
//
// Where a thread's slices are few (HC * NCH <= 8: the hc = 4, dim <= 4096
// shapes), a layer's key, value and q/k weight slices are loaded into
// registers in one batch before its sums start, and the key and value slices
// of the next layer are requested right behind them, so that they arrive
// while this layer reduces.  Each layer then waits on memory once, not three
// times (keys and weights, then the value after the reduction, then the next
// layer's keys).  Wider shapes keep the loads at their use: their streams
// alone fill most of the registers.
template <int HC, int NCH, bool SPLIT>
__global__ __launch_bounds__(kThreads) void gate_kernel(
    float *__restrict__ h, const GateLayers layers, const uint8_t *__restrict__ mask,
    int32_t dim, int32_t hc, float eps, float clamp, float dot_scale) {
  constexpr bool kBatch = HC * NCH <= 8;
  const int64_t t = SPLIT ? blockIdx.x / hc : blockIdx.x;
  const int s0 = SPLIT ? int(blockIdx.x % hc) : 0;   // first stream of this workgroup
  const int nstreams = SPLIT ? hc : HC;
  if (mask && mask[t] == 0) return;
  __shared__ float red[kWaves][3 * HC];

  float *ht = h + (t * nstreams + s0) * int64_t(dim);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float inv_dim = 1.0f / float(dim);
  auto i0_of = [&](int c) { return (int(threadIdx.x) + c * kThreads) * kVec; };
  float x[HC][NCH][kVec];
  float ssx[HC], ssk[HC], dot[HC];

  // Layer l's slices: key of stream s, the shared value, q/k weights.
  auto key_ptr = [&](int l, int s, int c) {
    return layers.kv[l] + t * (nstreams + 1) * int64_t(dim) + (s0 + s) * int64_t(dim) + i0_of(c);
  };
  auto val_ptr = [&](int l, int c) {
    return layers.kv[l] + t * (nstreams + 1) * int64_t(dim) + nstreams * int64_t(dim) + i0_of(c);
  };
  auto w_ptr = [&](const uint16_t *w, int s, int c) { return w + (s0 + s) * int64_t(dim) + i0_of(c); };
  auto ld = [](const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); };

  // Register copies (kBatch): this layer's operands and the next layer's
  // key and value.
  u32x4 key[HC][NCH], qw[HC][NCH], kw[HC][NCH], val[NCH];
  u32x4 key_next[HC][NCH], val_next[NCH];
  auto load_kv = [&](int l, u32x4 (&k)[HC][NCH], u32x4 (&v)[NCH]) {
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      if (i0_of(c) < dim) {
#pragma unroll
        for (int s = 0; s < HC; ++s) k[s][c] = ld(key_ptr(l, s, c));
        v[c] = ld(val_ptr(l, c));
      }
  };
  auto load_weights = [&](int l) {
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      if (i0_of(c) < dim)
#pragma unroll
        for (int s = 0; s < HC; ++s) {
          qw[s][c] = ld(w_ptr(layers.qw[l], s, c));
          kw[s][c] = ld(w_ptr(layers.kw[l], s, c));
        }
  };
  // Layer l's operands: from the registers (kBatch) or straight from memory.
  auto key_of = [&](int l, int s, int c) { return kBatch ? key[s][c] : ld(key_ptr(l, s, c)); };
  auto qw_of = [&](int l, int s, int c) { return kBatch ? qw[s][c] : ld(w_ptr(layers.qw[l], s, c)); };
  auto kw_of = [&](int l, int s, int c) { return kBatch ? kw[s][c] : ld(w_ptr(layers.kw[l], s, c)); };
  auto val_of = [&](int l, int c) { return kBatch ? val[c] : ld(val_ptr(l, c)); };

  // Layer l's partial sums over this thread's slices.
  auto accumulate = [&](int l) {
#pragma unroll
    for (int s = 0; s < HC; ++s) ssx[s] = ssk[s] = dot[s] = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (i0_of(c) < dim) {
#pragma unroll
        for (int s = 0; s < HC; ++s) {
          float kf[kVec], q[kVec], k[kVec];
          bf16x8_to_f32(key_of(l, s, c), kf);
          bf16x8_to_f32(qw_of(l, s, c), q);
          bf16x8_to_f32(kw_of(l, s, c), k);
#pragma unroll
          for (int e = 0; e < kVec; ++e) {
            const float xv = x[s][c][e];
            ssx[s] += xv * xv;
            ssk[s] += kf[e] * kf[e];
            dot[s] += (xv * q[e]) * (kf[e] * k[e]);
          }
        }
      }
    }
  };
  // Reduce the sums over the workgroup, derive the hc gates of layer l and
  // add gate * value to the streams in registers.
  auto finish = [&](int l) {
#pragma unroll
    for (int s = 0; s < HC; ++s) {
      const float a = wave_sum(ssx[s]), b = wave_sum(ssk[s]), d = wave_sum(dot[s]);
      if (lane == 0) {
        red[wave][3 * s] = a;
        red[wave][3 * s + 1] = b;
        red[wave][3 * s + 2] = d;
      }
    }
    __syncthreads();
    float g[HC];
#pragma unroll
    for (int s = 0; s < HC; ++s) {
      float a = 0.f, b = 0.f, d = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        a += red[w][3 * s];
        b += red[w][3 * s + 1];
        d += red[w][3 * s + 2];
      }
      const float rx = 1.0f / sqrtf(a * inv_dim + eps);
      const float rk = 1.0f / sqrtf(b * inv_dim + eps);
      const float av = dot_scale * d * rx * rk;
      const float mag = sqrtf(fmaxf(fabsf(av), clamp));
      const float z = av > 0.f ? mag : (av < 0.f ? -mag : 0.f);
      g[s] = 1.0f / (1.0f + expf(-z));
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (i0_of(c) < dim) {
        float v[kVec];
        bf16x8_to_f32(val_of(l, c), v);
#pragma unroll
        for (int s = 0; s < HC; ++s)
#pragma unroll
          for (int e = 0; e < kVec; ++e) x[s][c][e] = x[s][c][e] + g[s] * v[e];
      }
    }
  };

  // The streams, then (kBatch) layer 0's operands and layer 1's key and
  // value.  The scheduling fences keep the three groups in this order: a
  // wait for the first two then leaves the third in flight.
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (i0_of(c) < dim) {
#pragma unroll
      for (int s = 0; s < HC; ++s) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(ht + s * dim + i0_of(c));
        const f32x4 b = *reinterpret_cast<const f32x4 *>(ht + s * dim + i0_of(c) + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[s][c][e] = a[e];
          x[s][c][4 + e] = b[e];
        }
      }
    }
  }
  if constexpr (kBatch) {
    load_kv(0, key, val);
    load_weights(0);
    __builtin_amdgcn_sched_barrier(0);
    if (layers.n > 1) load_kv(1, key_next, val_next);
    __builtin_amdgcn_sched_barrier(0);
  }
  accumulate(0);
  finish(0);
  // Later layers read the streams from registers.
  for (int l = 1; l < layers.n; ++l) {
    __syncthreads();                               // every thread is done with red
    if constexpr (kBatch) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        val[c] = val_next[c];
#pragma unroll
        for (int s = 0; s < HC; ++s) key[s][c] = key_next[s][c];
      }
      load_weights(l);
      __builtin_amdgcn_sched_barrier(0);
      if (l + 1 < layers.n) load_kv(l + 1, key_next, val_next);
      __builtin_amdgcn_sched_barrier(0);
    }
    accumulate(l);
    finish(l);
  }

#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (i0_of(c) < dim) {
#pragma unroll
      for (int s = 0; s < HC; ++s) {
        f32x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = x[s][c][e];
          b[e] = x[s][c][4 + e];
        }
        *reinterpret_cast<f32x4 *>(ht + s * dim + i0_of(c)) = a;
        *reinterpret_cast<f32x4 *>(ht + s * dim + i0_of(c) + 4) = b;
      }
    }
  }
}

template <int HC, bool SPLIT>
hipError_t launch_hc(float *h, const GateLayers &ly, const uint8_t *mask, int32_t T, int32_t hc,
                     int32_t dim, float eps, float clamp, float dot_scale, hipStream_t stream) {
  const int nch = (dim + kThreads * kVec - 1) / (kThreads * kVec);
  const dim3 grid(SPLIT ? unsigned(T) * unsigned(hc) : unsigned(T)), block(kThreads);
  switch (nch) {
    case 1:
      hipLaunchKernelGGL((gate_kernel<HC, 1, SPLIT>), grid, block, 0, stream, h, ly, mask, dim,
                         hc, eps, clamp, dot_scale);
      break;
    case 2:
      hipLaunchKernelGGL((gate_kernel<HC, 2, SPLIT>), grid, block, 0, stream, h, ly, mask, dim,
                         hc, eps, clamp, dot_scale);
      break;
    default:
      hipLaunchKernelGGL((gate_kernel<HC, 4, SPLIT>), grid, block, 0, stream, h, ly, mask, dim,
                         hc, eps, clamp, dot_scale);
      break;
  }
  return hipGetLastError();
}

// Below this many workgroups a token-per-workgroup grid leaves most CUs idle.
constexpr int kSplitBelow = 1024;

}  // namespace

hipError_t launch_gate_layers(float *h, const GateLayers &ly, const uint8_t *mask, int32_t T,
                              int32_t hc, int32_t dim, float eps, float clamp, float dot_scale,
                              hipStream_t stream) {
  if (T < kSplitBelow && hc > 1)
    return launch_hc<1, true>(h, ly, mask, T, hc, dim, eps, clamp, dot_scale, stream);
  switch (hc) {
#define ENGRAM_GATE_HC(n) \
    case n: return launch_hc<n, false>(h, ly, mask, T, hc, dim, eps, clamp, dot_scale, stream);
    ENGRAM_GATE_HC(1) ENGRAM_GATE_HC(2) ENGRAM_GATE_HC(3) ENGRAM_GATE_HC(4)
    ENGRAM_GATE_HC(5) ENGRAM_GATE_HC(6) ENGRAM_GATE_HC(7)
#undef ENGRAM_GATE_HC
    default: return launch_hc<8, false>(h, ly, mask, T, hc, dim, eps, clamp, dot_scale, stream);
  }
}

hipError_t launch_gate(float *h, const uint16_t *kv, const uint16_t *qw, const uint16_t *kw,
                       const uint8_t *mask, int32_t T, int32_t hc, int32_t dim, float eps,
                       float clamp, float dot_scale, hipStream_t stream) {
  GateLayers ly{};
  ly.kv[0] = kv;
  ly.qw[0] = qw;
  ly.kw[0] = kw;
  ly.n = 1;
  return launch_gate_layers(h, ly, mask, T, hc, dim, eps, clamp, dot_scale, stream);
}

}  // namespace engram
