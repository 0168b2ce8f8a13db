// Stage 1: n-gram hash -> int32 row ids.
//
// [vLLM engram page, EngramLayout / NgramHashState.forward] and [NeMo engram
// page, DeepseekV41NgramHash.forward]: every position hashes orders
// 2..max_ngram over n_heads heads; each (order, head) column owns a prime-sized
// bucket range; missing or blocked history reads as the pad id.
//
// One thread per position.  Its history (max_ngram - 1 ids back, with the
// blocking rule) is resolved once and then shared by every layer.  The tables
// travel as kernel arguments: all lanes index them uniformly, so they are read
// with scalar loads.  The whole stage is a few hundred integer operations per
// position; it is bound by launch latency, not by bandwidth.
#include "common.hpp"

namespace engram {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void hash_kernel(
    const HashTables tab, int32_t T, int32_t n_seqs, int32_t depth,
    const int32_t *__restrict__ cids, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ doc_ids, const uint8_t *__restrict__ mask,
    const int32_t *__restrict__ lookback, const uint8_t *__restrict__ lookback_live,
    int32_t *__restrict__ ids) {
  const int32_t t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= T) return;

  // Chunk of t: the last s with cu[s] <= t (empty chunks are skipped over).
  int32_t lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int32_t s = lo;
  const int32_t start = max(cu[s], 0);

  // History: distance 0 is t itself; walking back, the first position that
  // is absent or not live, and everything before it, reads as pad_id.
  uint64_t hist[ENGRAM_MAX_NGRAM];
  hist[0] = uint64_t(int64_t(cids[t]));
  const int32_t own_doc = doc_ids ? doc_ids[t] : 1;
  bool blocked = own_doc == 0;          // a padding position has no history
  const uint64_t pad = uint64_t(int64_t(tab.pad_id));
#pragma unroll
  for (int k = 1; k < ENGRAM_MAX_NGRAM; ++k) {
    if (k >= tab.max_ngram) break;
    int32_t tokv = tab.pad_id;
    if (!blocked) {
      const int32_t q = t - k;
      bool live;
      if (q >= start) {
        live = (!mask || mask[q] != 0) && (!doc_ids || doc_ids[q] == own_doc);
        tokv = cids[q];
      } else {
        const int32_t j = depth - (start - q);   // lookback is oldest first
        if (!lookback || j < 0) {
          live = false;
        } else {
          const int64_t at = int64_t(s) * depth + j;
          live = !lookback_live || lookback_live[at] != 0;
          tokv = lookback[at];
        }
      }
      blocked = !live;
    }
    hist[k] = blocked ? pad : uint64_t(int64_t(tokv));
  }

  const int32_t cols = (tab.max_ngram - 1) * tab.n_heads;
  int32_t *out = ids + int64_t(t) * tab.n_layers * cols;
  for (int l = 0; l < tab.n_layers; ++l) {
    uint64_t mix = hist[0] * tab.mult[l][0];
    for (int n = 2; n <= tab.max_ngram; ++n) {
      mix ^= hist[n - 1] * tab.mult[l][n - 1];      // wraps mod 2^64
      const int c0 = (n - 2) * tab.n_heads;
      for (int j = 0; j < tab.n_heads; ++j) {
        const int c = c0 + j;
        out[l * cols + c] = int32_t(tab.offset[l][c] + uint32_t(mix % tab.prime[l][c]));
      }
    }
  }
}

}  // namespace

hipError_t launch_hash(const HashTables &tab, const engram_tokens &tok, int32_t *ids,
                       hipStream_t stream) {
  const int blocks = (tok.T + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(hash_kernel, dim3(blocks), dim3(kThreads), 0, stream, tab, tok.T,
                     tok.n_seqs, tok.lookback ? tok.lookback_depth : 0, tok.cids,
                     tok.cu_seqlens, tok.doc_ids, tok.token_mask, tok.lookback,
                     tok.lookback_live, ids);
  return hipGetLastError();
}

}  // namespace engram
