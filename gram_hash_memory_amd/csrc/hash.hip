// Stage 1: n-gram hash -> int32 row ids.
//
// [vLLM engram page, EngramLayout / NgramHashState.forward] and [NeMo engram
// page, DeepseekV41NgramHash.forward]: every position hashes orders
// 2..max_ngram over n_heads heads; each (order, head) column owns a prime-sized
// bucket range; missing or blocked history reads as the pad id.
//
// One thread per (position, column), so that even a decode batch of a few
// dozen tokens spreads over enough lanes; the column's order n fixes how many
// history positions (n - 1) the thread resolves.  The tables travel as kernel
// arguments: all lanes index them uniformly per layer, so they are read with
// scalar loads.  Sequence boundaries are searched in an LDS copy of
// cu_seqlens when it fits, which turns a chain of dependent global loads into
// one cooperative load.  Every history entry a thread may need is loaded
// before the walk that decides which of them count (an earlier dead or
// foreign position blocks the later ones), so the loads travel together:
// the positions inside the batch while cu_seqlens comes in, the lookback
// entries after the search.  All of them lie inside the batch or the
// sequence's lookback row whatever the walk decides.
#include "common.hpp"

namespace engram {
namespace {

constexpr int kThreads = 256;
constexpr int kCuLds = 4096;           // cu_seqlens entries searched in LDS

// x mod p for 64-bit x and a 31-bit prime p.  The quotient estimate from fp64
// is within a few units of floor(x / p) once p >= 2^12 (relative error of the
// three roundings <= 3.3 * 2^-53, and x / p < 2^52), so a couple of
// corrections make the remainder exact; smaller moduli take the integer
// division.  The difference x - q*p is formed mod 2^64, and its true value
// lies within a few p of 0, so reading it as int64 is exact.
__device__ __forceinline__ uint32_t mod_prime(uint64_t x, uint32_t p) {
  if (p < 4096u) return uint32_t(x % p);
  const uint64_t q = uint64_t(double(x) * (1.0 / double(p)));
  int64_t r = int64_t(x - q * uint64_t(p));
  while (r < 0) r += int64_t(p);
  while (r >= int64_t(p)) r -= int64_t(p);
  return uint32_t(r);
}

__global__ __launch_bounds__(kThreads) void hash_kernel(
    const HashTables tab, int32_t T, int32_t n_seqs, int32_t depth,
    const int32_t *__restrict__ cids, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ doc_ids, const uint8_t *__restrict__ mask,
    const int32_t *__restrict__ lookback, const uint8_t *__restrict__ lookback_live,
    int32_t *__restrict__ ids) {
  __shared__ int32_t cu_lds[kCuLds];
  const bool cu_in_lds = n_seqs + 1 <= kCuLds;
  const int32_t cols = (tab.max_ngram - 1) * tab.n_heads;
  const int64_t g = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const bool active = g < int64_t(T) * cols;
  const int32_t t = active ? int32_t(g / cols) : 0, c = active ? int32_t(g % cols) : 0;
  const int order = 2 + c / tab.n_heads;

  // First, with no load waiting on another: this thread's first entry of
  // the LDS copy of cu_seqlens, then the position itself and the ones
  // before it in the batch (distance k, clamped at 0; an absent mask or
  // document array reads stand-in bytes of cids, in bounds and unused).
  const int32_t cu_first = cu_in_lds && int(threadIdx.x) <= n_seqs ? cu[threadIdx.x] : 0;
  const uint8_t *mptr = mask ? mask : reinterpret_cast<const uint8_t *>(cids);
  const int32_t *dptr = doc_ids ? doc_ids : cids;
  const int32_t tok0 = cids[t], d0 = dptr[t];
  int32_t tokv[ENGRAM_MAX_NGRAM], dq[ENGRAM_MAX_NGRAM];
  uint32_t mq[ENGRAM_MAX_NGRAM];
  bool livev[ENGRAM_MAX_NGRAM];
#pragma unroll
  for (int k = 1; k < ENGRAM_MAX_NGRAM; ++k) {
    const int32_t q = max(t - k, 0);
    tokv[k] = cids[q];
    mq[k] = mptr[q];
    dq[k] = dptr[q];
  }
  if (cu_in_lds) {
    if (int(threadIdx.x) <= n_seqs) cu_lds[threadIdx.x] = cu_first;
    for (int i = threadIdx.x + kThreads; i <= n_seqs; i += kThreads) cu_lds[i] = cu[i];
    __syncthreads();
  }
  if (!active) return;
  const int32_t own_doc = doc_ids ? d0 : 1;
#pragma unroll
  for (int k = 1; k < ENGRAM_MAX_NGRAM; ++k)
    livev[k] = k < order && t - k >= 0 && (!mask || mq[k] != 0) && (!doc_ids || dq[k] == own_doc);

  // Chunk of t: the last s with cu[s] <= t (empty chunks are skipped over).
  int32_t lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if ((cu_in_lds ? cu_lds[mid] : cu[mid]) <= t) lo = mid; else hi = mid - 1;
  }
  const int32_t s = lo;
  const int32_t start = max(cu_in_lds ? cu_lds[s] : cu[s], 0);

  // Positions before the chunk come from the sequence's lookback row
  // (oldest first, entry depth - (start - q)), or are absent.  The row's
  // entries are loaded at clamped indices, then kept where they count.
  const bool has_lookback = lookback && depth > 0;
  const uint8_t *llptr =
      lookback_live ? lookback_live : reinterpret_cast<const uint8_t *>(lookback);
  int32_t lb_tok[ENGRAM_MAX_NGRAM];
  uint32_t lb_live[ENGRAM_MAX_NGRAM];
  if (has_lookback) {
#pragma unroll
    for (int k = 1; k < ENGRAM_MAX_NGRAM; ++k) {
      const int32_t j = depth - (start - (t - k));
      const int64_t at = int64_t(s) * depth + min(max(j, 0), depth - 1);
      lb_tok[k] = lookback[at];
      lb_live[k] = llptr[at];
    }
  }
#pragma unroll
  for (int k = 1; k < ENGRAM_MAX_NGRAM; ++k) {
    if (k < order && t - k < start) {
      const int32_t j = depth - (start - (t - k));
      livev[k] = has_lookback && j >= 0 && (!lookback_live || lb_live[k] != 0);
      tokv[k] = has_lookback ? lb_tok[k] : 0;
    }
  }

  // History: distance 0 is t itself; walking back, the first position that
  // is absent or not live, and everything before it, reads as pad_id.
  uint64_t hist[ENGRAM_MAX_NGRAM];
  hist[0] = uint64_t(int64_t(tok0));
  bool blocked = own_doc == 0;          // a padding position has no history
  const uint64_t pad = uint64_t(int64_t(tab.pad_id));
#pragma unroll
  for (int k = 1; k < ENGRAM_MAX_NGRAM; ++k) {
    if (k >= order) break;
    blocked = blocked || !livev[k];
    hist[k] = blocked ? pad : uint64_t(int64_t(tokv[k]));
  }

  int32_t *out = ids + int64_t(t) * tab.n_layers * cols + c;
  for (int l = 0; l < tab.n_layers; ++l) {
    uint64_t mix = hist[0] * tab.mult[l][0];
#pragma unroll
    for (int k = 1; k < ENGRAM_MAX_NGRAM; ++k)
      if (k < order) mix ^= hist[k] * tab.mult[l][k];   // products wrap mod 2^64
    out[l * cols] = int32_t(tab.offset[l][c] + mod_prime(mix, tab.prime[l][c]));
  }
}

// The lookback store after a batch, one thread per sequence: entry j (oldest
// first) becomes the position that precedes the sequence's next chunk by
// depth - j -- a position of this chunk, or an older entry of the store.  The
// thread reads all of its sequence's old entries before it writes any, so
// the update can run in place.  The chunk bounds are clamped to [0, T], so
// that malformed cu_seqlens cannot move an access outside the token arrays.
__global__ __launch_bounds__(kThreads) void history_kernel(
    int32_t T, int32_t n_seqs, int32_t depth, const int32_t *__restrict__ cids,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ doc_ids,
    const uint8_t *__restrict__ mask, int32_t *hist, uint8_t *live) {
  const int32_t s = int32_t(blockIdx.x) * kThreads + int32_t(threadIdx.x);
  if (s >= n_seqs) return;
  const int32_t start = min(max(cu[s], 0), T), end = min(max(cu[s + 1], 0), T);
  if (end <= start) return;                       // an empty chunk changes nothing
  int32_t *h = hist + int64_t(s) * depth;
  uint8_t *l = live + int64_t(s) * depth;
  int32_t old_tok[ENGRAM_MAX_NGRAM];
  bool old_live[ENGRAM_MAX_NGRAM];
#pragma unroll
  for (int j = 0; j < ENGRAM_MAX_NGRAM; ++j) {
    if (j < depth) {
      old_tok[j] = h[j];
      old_live[j] = l[j] != 0;
    }
  }
  // The next chunk continues the document of this chunk's last position; a
  // document change inside the chunk, or a padding document, ends the older
  // entries' usefulness.
  const int32_t last_doc = doc_ids ? doc_ids[end - 1] : 1;
  const bool old_ok = !doc_ids || (last_doc != 0 && doc_ids[start] == last_doc);
#pragma unroll
  for (int j = 0; j < ENGRAM_MAX_NGRAM; ++j) {
    if (j >= depth) break;
    const int32_t p = end - depth + j;
    int32_t tok = 0;
    bool ok = false;
    if (p >= start) {
      tok = cids[p];
      ok = (!mask || mask[p] != 0) && (!doc_ids || (last_doc != 0 && doc_ids[p] == last_doc));
    } else {
      const int32_t jo = depth - (start - p);
#pragma unroll
      for (int k = 0; k < ENGRAM_MAX_NGRAM; ++k)
        if (k == jo) {
          tok = old_tok[k];
          ok = old_live[k] && old_ok;
        }
    }
    h[j] = tok;
    l[j] = ok ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_history_update(const engram_tokens &tok, int32_t depth, int32_t *history,
                                 uint8_t *history_live, hipStream_t stream) {
  const int64_t blocks = (int64_t(tok.n_seqs) + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(history_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                     tok.T, tok.n_seqs, depth, tok.cids, tok.cu_seqlens, tok.doc_ids,
                     tok.token_mask,
                     history, history_live);
  return hipGetLastError();
}

hipError_t launch_hash(const HashTables &tab, const engram_tokens &tok, int32_t *ids,
                       hipStream_t stream) {
  const int64_t cols = int64_t(tab.max_ngram - 1) * tab.n_heads;
  const int64_t blocks = (int64_t(tok.T) * cols + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(hash_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, tab,
                     tok.T, tok.n_seqs, tok.lookback ? tok.lookback_depth : 0, tok.cids,
                     tok.cu_seqlens, tok.doc_ids, tok.token_mask, tok.lookback,
                     tok.lookback_live, ids);
  return hipGetLastError();
}

}  // namespace engram
