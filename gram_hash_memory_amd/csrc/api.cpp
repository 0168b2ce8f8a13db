// C ABI of libengram.so: host-side validation and dispatch (see include/engram.h).
//
// Every entry point checks all of its arguments before queuing anything, so
// ENGRAM_ERR_ARG and ENGRAM_ERR_UNSUPPORTED mean that nothing reached the GPU.
// ENGRAM_ERR_HIP reports a failed launch; in engram_forward, stages queued
// before the failing one may still run.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "common.hpp"

namespace {

thread_local char g_error[512] = "";

engram_status fail(engram_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return st;
}

// Prefixes the current message with the layer index (copied first: the
// message buffer is also the destination).
engram_status fail_layer(engram_status st, int layer) {
  char msg[sizeof(g_error)];
  std::memcpy(msg, g_error, sizeof(msg));
  return fail(st, "layer %d: %s", layer, msg);
}

engram_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ENGRAM_OK;
  return fail(ENGRAM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define REQUIRE(cond, ...)                                   \
  do {                                                       \
    if (!(cond)) return fail(ENGRAM_ERR_ARG, __VA_ARGS__);   \
  } while (0)
#define REQUIRE_SUP(cond, ...)                                       \
  do {                                                               \
    if (!(cond)) return fail(ENGRAM_ERR_UNSUPPORTED, __VA_ARGS__);   \
  } while (0)

constexpr int64_t kInt32Max = 2147483647;

engram_status check_hash_params(const engram_hash_params *p, engram::HashTables *tab) {
  REQUIRE(p, "engram_hash_params is NULL");
  REQUIRE_SUP(p->n_layers >= 1 && p->n_layers <= ENGRAM_MAX_LAYERS,
              "n_layers=%d outside 1..%d", p->n_layers, ENGRAM_MAX_LAYERS);
  REQUIRE_SUP(p->max_ngram >= 2 && p->max_ngram <= ENGRAM_MAX_NGRAM,
              "max_ngram=%d outside 2..%d", p->max_ngram, ENGRAM_MAX_NGRAM);
  REQUIRE(p->n_heads >= 1, "n_heads=%d < 1", p->n_heads);
  const int64_t cols = int64_t(p->max_ngram - 1) * p->n_heads;
  REQUIRE_SUP(cols <= ENGRAM_MAX_COLS, "(max_ngram-1)*n_heads=%lld > %d", (long long)cols,
              ENGRAM_MAX_COLS);
  REQUIRE(p->multipliers && p->primes && p->offsets, "hash table pointer is NULL");
  std::memset(tab, 0, sizeof(*tab));
  tab->n_layers = p->n_layers;
  tab->max_ngram = p->max_ngram;
  tab->n_heads = p->n_heads;
  tab->pad_id = p->pad_id;
  for (int l = 0; l < p->n_layers; ++l) {
    for (int k = 0; k < p->max_ngram; ++k)
      tab->mult[l][k] = uint64_t(p->multipliers[int64_t(l) * p->max_ngram + k]);
    for (int c = 0; c < cols; ++c) {
      const int64_t pr = p->primes[int64_t(l) * cols + c];
      const int64_t of = p->offsets[int64_t(l) * cols + c];
      REQUIRE(pr >= 1 && pr <= kInt32Max, "primes[%d][%d]=%lld outside [1, 2^31)", l, c,
              (long long)pr);
      REQUIRE(of >= 0 && of + pr <= kInt32Max + 1, "offsets[%d][%d]+primes exceeds 2^31", l,
              c);
      tab->prime[l][c] = uint32_t(pr);
      tab->offset[l][c] = uint32_t(of);
    }
  }
  return ENGRAM_OK;
}

engram_status check_tokens(const engram_tokens *t, int max_ngram) {
  REQUIRE(t, "engram_tokens is NULL");
  REQUIRE(t->T >= 0, "T=%d < 0", t->T);
  if (t->T == 0) return ENGRAM_OK;
  REQUIRE(t->n_seqs >= 1, "n_seqs=%d < 1", t->n_seqs);
  REQUIRE(t->cids && t->cu_seqlens, "cids or cu_seqlens is NULL");
  REQUIRE(aligned(t->cids, 4) && aligned(t->cu_seqlens, 4), "cids/cu_seqlens misaligned");
  REQUIRE(!t->doc_ids || aligned(t->doc_ids, 4), "doc_ids misaligned");
  REQUIRE(t->lookback_depth >= 0 && t->lookback_depth <= max_ngram - 1,
          "lookback_depth=%d outside 0..max_ngram-1=%d", t->lookback_depth, max_ngram - 1);
  REQUIRE(!t->lookback || aligned(t->lookback, 4), "lookback misaligned");
  REQUIRE(!(t->lookback_live && !t->lookback), "lookback_live given without lookback");
  return ENGRAM_OK;
}

engram_status check_rows_shape(engram_row_format fmt, int64_t num_rows, int64_t stride,
                               int32_t cols, int32_t T) {
  REQUIRE(fmt == ENGRAM_ROWS_Q2K || fmt == ENGRAM_ROWS_FP8_E4M3_E8M0, "unknown row format %d",
          int(fmt));
  REQUIRE(T >= 0, "T=%d < 0", T);
  REQUIRE(cols >= 1, "cols=%d < 1", cols);
  REQUIRE(num_rows >= 1, "num_rows=%lld < 1", (long long)num_rows);
  REQUIRE(stride >= cols, "ids_token_stride=%lld < cols=%d", (long long)stride, cols);
  return ENGRAM_OK;
}

engram_status check_rows_ptrs(engram_row_format fmt, const uint8_t *table, const uint8_t *scales,
                              const int32_t *ids, const uint16_t *rows, const int32_t *bad_ids) {
  REQUIRE(table && ids && rows, "table, ids or rows is NULL");
  REQUIRE(aligned(ids, 4), "ids misaligned");
  REQUIRE(aligned(rows, 16), "rows must be 16-byte aligned");
  REQUIRE(!bad_ids || aligned(bad_ids, 4), "bad_ids misaligned");
  if (fmt == ENGRAM_ROWS_Q2K) {
    REQUIRE(aligned(table, 4), "Q2_K table must be 4-byte aligned");
  } else {
    REQUIRE(scales, "FP8 rows need scales");
    REQUIRE(aligned(table, 16), "FP8 table must be 16-byte aligned");
  }
  return ENGRAM_OK;
}

engram_status check_project_shape(int32_t T, int32_t K, int32_t N) {
  REQUIRE(T >= 0, "T=%d < 0", T);
  REQUIRE(K > 0 && K % 64 == 0, "K=%d must be a positive multiple of 64", K);
  REQUIRE(N > 0, "N=%d must be positive", N);
  return ENGRAM_OK;
}

engram_status check_project_ptrs(const uint16_t *a, const uint16_t *w, const uint16_t *c) {
  REQUIRE(a && w && c, "rows, wkv or kv is NULL");
  REQUIRE(aligned(a, 16) && aligned(w, 16) && aligned(c, 16),
          "GEMM operands must be 16-byte aligned");
  return ENGRAM_OK;
}

engram_status check_gate_shape(int32_t T, int32_t hc, int32_t dim, float eps, float clamp) {
  REQUIRE(T >= 0, "T=%d < 0", T);
  REQUIRE_SUP(hc >= 1 && hc <= ENGRAM_MAX_HC, "hc=%d outside 1..%d", hc, ENGRAM_MAX_HC);
  REQUIRE_SUP(dim >= 8 && dim <= ENGRAM_MAX_DIM && dim % 8 == 0,
              "dim=%d must be a multiple of 8 in 8..%d", dim, ENGRAM_MAX_DIM);
  REQUIRE(eps >= 0.f && clamp >= 0.f, "eps and clamp must be >= 0");
  return ENGRAM_OK;
}

engram_status check_gate_ptrs(const float *h, const uint16_t *kv, const uint16_t *qw,
                              const uint16_t *kw) {
  REQUIRE(h && kv && qw && kw, "h, kv, q_weight or k_weight is NULL");
  REQUIRE(aligned(h, 16) && aligned(kv, 16) && aligned(qw, 16) && aligned(kw, 16),
          "gate operands must be 16-byte aligned");
  return ENGRAM_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

extern "C" {

const char *engram_last_error(void) { return g_error; }

// The marker lets a loader check the file's build id without loading it.
#ifndef ENGRAM_BUILD_ID
#define ENGRAM_BUILD_ID "unknown"
#endif
static const char g_build_id[] = "engram-build-id " ENGRAM_BUILD_ID;

const char *engram_build_id(void) { return g_build_id + sizeof("engram-build-id ") - 1; }

engram_status engram_hash(const engram_hash_params *params, const engram_tokens *tokens,
                          int32_t *ids, hipStream_t stream) {
  engram::HashTables tab;
  engram_status st = check_hash_params(params, &tab);
  if (st != ENGRAM_OK) return st;
  if ((st = check_tokens(tokens, params->max_ngram)) != ENGRAM_OK) return st;
  if (tokens->T == 0) return ENGRAM_OK;
  REQUIRE(ids && aligned(ids, 4), "ids is NULL or misaligned");
  return hip_status(engram::launch_hash(tab, *tokens, ids, stream), "engram_hash launch");
}

engram_status engram_history_update(const engram_tokens *tokens, int32_t depth,
                                    int32_t *history, uint8_t *history_live,
                                    hipStream_t stream) {
  REQUIRE(depth >= 1 && depth <= ENGRAM_MAX_NGRAM - 1, "depth=%d outside 1..%d", depth,
          ENGRAM_MAX_NGRAM - 1);
  engram_status st = check_tokens(tokens, ENGRAM_MAX_NGRAM);
  if (st != ENGRAM_OK) return st;
  if (tokens->T == 0) return ENGRAM_OK;              // every chunk is empty
  REQUIRE(history && history_live, "history or history_live is NULL");
  REQUIRE(aligned(history, 4), "history misaligned");
  return hip_status(engram::launch_history_update(*tokens, depth, history, history_live,
                                                  stream),
                    "engram_history_update launch");
}

engram_status engram_rows(engram_row_format fmt, const uint8_t *table, const uint8_t *scales,
                          int64_t num_rows, const int32_t *ids, int64_t ids_token_stride,
                          int32_t cols, int32_t T, uint16_t *rows, int32_t *bad_ids,
                          hipStream_t stream) {
  engram_status st = check_rows_shape(fmt, num_rows, ids_token_stride, cols, T);
  if (st != ENGRAM_OK) return st;
  if (T == 0) return ENGRAM_OK;
  if ((st = check_rows_ptrs(fmt, table, scales, ids, rows, bad_ids)) != ENGRAM_OK) return st;
  return hip_status(engram::launch_rows(fmt, table, scales, num_rows, ids, ids_token_stride,
                                        cols, T, rows, bad_ids, stream),
                    "engram_rows launch");
}

engram_status engram_project(const uint16_t *rows, const uint16_t *wkv, uint16_t *kv, int32_t T,
                             int32_t K, int32_t N, hipStream_t stream) {
  engram_status st = check_project_shape(T, K, N);
  if (st != ENGRAM_OK) return st;
  if (T == 0) return ENGRAM_OK;
  if ((st = check_project_ptrs(rows, wkv, kv)) != ENGRAM_OK) return st;
  return hip_status(engram::launch_project(rows, wkv, kv, T, K, N, stream),
                    "engram_project launch");
}

engram_status engram_project_q2k(const uint8_t *table, int64_t num_rows, const int32_t *ids,
                                 int64_t ids_token_stride, int32_t cols, const uint16_t *wkv,
                                 uint16_t *kv, int32_t T, int32_t N, int32_t *bad_ids,
                                 hipStream_t stream) {
  engram_status st = check_rows_shape(ENGRAM_ROWS_Q2K, num_rows, ids_token_stride, cols, T);
  if (st != ENGRAM_OK) return st;
  REQUIRE(int64_t(cols) * ENGRAM_HEAD_DIM <= kInt32Max, "cols=%d too large", cols);
  const int32_t K = cols * ENGRAM_HEAD_DIM;
  if ((st = check_project_shape(T, K, N)) != ENGRAM_OK) return st;
  REQUIRE_SUP(cols <= ENGRAM_Q2K_FUSED_MAX_COLS, "cols=%d exceeds the fused kernel's %d", cols,
              ENGRAM_Q2K_FUSED_MAX_COLS);
  REQUIRE_SUP(engram::project_q2k_supported(num_rows, cols),
              "Q2_K table of %lld rows exceeds the fused kernel's %lld bytes",
              (long long)num_rows, (long long)ENGRAM_Q2K_FUSED_MAX_BYTES);
  if (T == 0) return ENGRAM_OK;
  REQUIRE(table && aligned(table, 4), "table is NULL or not 4-byte aligned");
  REQUIRE(ids && aligned(ids, 4), "ids is NULL or misaligned");
  REQUIRE(!bad_ids || aligned(bad_ids, 4), "bad_ids misaligned");
  REQUIRE(wkv && kv && aligned(wkv, 16) && aligned(kv, 16),
          "wkv or kv is NULL or not 16-byte aligned");
  return hip_status(engram::launch_project_q2k(table, num_rows, ids, ids_token_stride, cols, wkv,
                                               kv, T, N, bad_ids, stream),
                    "engram_project_q2k launch");
}

engram_status engram_quantize_mxfp8(const uint16_t *w, int32_t N, int32_t K, uint8_t *codes,
                                    uint8_t *scales, hipStream_t stream) {
  REQUIRE(N >= 0, "N=%d < 0", N);
  REQUIRE(K > 0 && K % 32 == 0, "K=%d must be a positive multiple of 32", K);
  if (N == 0) return ENGRAM_OK;
  REQUIRE(w && codes && scales, "w, codes or scales is NULL");
  REQUIRE(aligned(w, 16) && aligned(codes, 16), "w and codes must be 16-byte aligned");
  return hip_status(engram::launch_quantize_mx(w, N, K, codes, scales, stream),
                    "engram_quantize_mxfp8 launch");
}

namespace {
engram_status check_project_mx(const uint8_t *table, const uint8_t *scales, int64_t num_rows,
                               const int32_t *ids, int64_t stride, int32_t cols,
                               const uint8_t *wc, const uint8_t *ws, const uint16_t *kv,
                               int32_t T, int32_t N, const int32_t *bad_ids) {
  engram_status st =
      check_rows_shape(ENGRAM_ROWS_FP8_E4M3_E8M0, num_rows, stride, cols, T);
  if (st != ENGRAM_OK) return st;
  REQUIRE(int64_t(cols) * ENGRAM_HEAD_DIM <= kInt32Max, "cols=%d too large", cols);
  const int32_t K = cols * ENGRAM_HEAD_DIM;
  if ((st = check_project_shape(T, K, N)) != ENGRAM_OK) return st;
  REQUIRE_SUP(engram::project_mx_supported(N, K),
              "MXFP8 weight of %d x %d bytes exceeds %lld", N, K,
              (long long)ENGRAM_MX_MAX_WEIGHT_BYTES);
  REQUIRE_SUP(int64_t(T) * stride * 4 <= ENGRAM_MX_MAX_WEIGHT_BYTES,
              "T * ids_token_stride * 4 exceeds %lld", (long long)ENGRAM_MX_MAX_WEIGHT_BYTES);
  if (T == 0) return ENGRAM_OK;
  REQUIRE(table && aligned(table, 16), "table is NULL or not 16-byte aligned");
  REQUIRE(scales && aligned(scales, 4), "scales is NULL or not 4-byte aligned");
  REQUIRE(ids && aligned(ids, 4), "ids is NULL or misaligned");
  REQUIRE(!bad_ids || aligned(bad_ids, 4), "bad_ids misaligned");
  REQUIRE(wc && aligned(wc, 16), "wkv codes are NULL or not 16-byte aligned");
  REQUIRE(ws && aligned(ws, 4), "wkv scales are NULL or not 4-byte aligned");
  REQUIRE(kv && aligned(kv, 16), "kv is NULL or not 16-byte aligned");
  return ENGRAM_OK;
}
}  // namespace

engram_status engram_project_fp8(const uint8_t *table, const uint8_t *scales, int64_t num_rows,
                                 const int32_t *ids, int64_t ids_token_stride, int32_t cols,
                                 const uint16_t *wkv, uint16_t *kv, int32_t T, int32_t N,
                                 int32_t *bad_ids, hipStream_t stream) {
  engram_status st =
      check_rows_shape(ENGRAM_ROWS_FP8_E4M3_E8M0, num_rows, ids_token_stride, cols, T);
  if (st != ENGRAM_OK) return st;
  REQUIRE(int64_t(cols) * ENGRAM_HEAD_DIM <= kInt32Max, "cols=%d too large", cols);
  const int32_t K = cols * ENGRAM_HEAD_DIM;
  if ((st = check_project_shape(T, K, N)) != ENGRAM_OK) return st;
  REQUIRE_SUP(int64_t(T) * ids_token_stride * 4 <= ENGRAM_FP8_FUSED_MAX_ID_BYTES,
              "T * ids_token_stride * 4 exceeds %lld", (long long)ENGRAM_FP8_FUSED_MAX_ID_BYTES);
  if (T == 0) return ENGRAM_OK;
  REQUIRE(table && aligned(table, 16), "table is NULL or not 16-byte aligned");
  REQUIRE(scales && aligned(scales, 4), "scales is NULL or not 4-byte aligned");
  REQUIRE(ids && aligned(ids, 4), "ids is NULL or misaligned");
  REQUIRE(!bad_ids || aligned(bad_ids, 4), "bad_ids misaligned");
  REQUIRE(wkv && kv && aligned(wkv, 16) && aligned(kv, 16),
          "wkv or kv is NULL or not 16-byte aligned");
  return hip_status(engram::launch_project_fp8(table, scales, num_rows, ids, ids_token_stride,
                                               cols, wkv, kv, T, N, bad_ids, stream),
                    "engram_project_fp8 launch");
}

engram_status engram_project_mxfp8(const uint8_t *table, const uint8_t *scales,
                                   int64_t num_rows, const int32_t *ids,
                                   int64_t ids_token_stride, int32_t cols,
                                   const uint8_t *wkv_codes, const uint8_t *wkv_scales,
                                   uint16_t *kv, int32_t T, int32_t N, int32_t *bad_ids,
                                   hipStream_t stream) {
  engram_status st = check_project_mx(table, scales, num_rows, ids, ids_token_stride, cols,
                                      wkv_codes, wkv_scales, kv, T, N, bad_ids);
  if (st != ENGRAM_OK || T == 0) return st;
  return hip_status(engram::launch_project_mx(table, scales, num_rows, ids, ids_token_stride,
                                              cols, wkv_codes, wkv_scales, kv, T, N, bad_ids,
                                              stream),
                    "engram_project_mxfp8 launch");
}

engram_status engram_stage_mxfp8(const uint8_t *table, const uint8_t *scales, int64_t num_rows,
                                 const int32_t *ids, int64_t ids_token_stride, int32_t cols,
                                 int32_t T, uint8_t *a_codes, uint8_t *a_scales,
                                 int32_t *bad_ids, hipStream_t stream) {
  engram_status st =
      check_rows_shape(ENGRAM_ROWS_FP8_E4M3_E8M0, num_rows, ids_token_stride, cols, T);
  if (st != ENGRAM_OK) return st;
  REQUIRE(int64_t(cols) * ENGRAM_HEAD_DIM <= kInt32Max, "cols=%d too large", cols);
  // one workgroup per 64 rows of the flattened [T * cols]
  REQUIRE_SUP(int64_t(T) * cols <= int64_t(kInt32Max) * 64, "T * cols too large");
  if (T == 0) return ENGRAM_OK;
  REQUIRE(table && aligned(table, 16), "table is NULL or not 16-byte aligned");
  REQUIRE(scales && aligned(scales, 4), "scales is NULL or not 4-byte aligned");
  REQUIRE(ids && aligned(ids, 4), "ids is NULL or misaligned");
  REQUIRE(!bad_ids || aligned(bad_ids, 4), "bad_ids misaligned");
  REQUIRE(a_codes && aligned(a_codes, 16), "a_codes is NULL or not 16-byte aligned");
  REQUIRE(a_scales && aligned(a_scales, 4), "a_scales is NULL or not 4-byte aligned");
  return hip_status(engram::launch_stage_mx(table, scales, num_rows, ids, ids_token_stride, cols,
                                            T, a_codes, a_scales, bad_ids, stream),
                    "engram_stage_mxfp8 launch");
}

namespace {
engram_status check_project_mx_staged(const uint8_t *a_codes, const uint8_t *a_scales,
                                      int32_t cols, const uint8_t *wc, const uint8_t *ws,
                                      const uint16_t *kv, int32_t T, int32_t N) {
  REQUIRE(cols >= 1 && int64_t(cols) * ENGRAM_HEAD_DIM <= kInt32Max, "cols=%d out of range",
          cols);
  const int32_t K = cols * ENGRAM_HEAD_DIM;
  engram_status st = check_project_shape(T, K, N);
  if (st != ENGRAM_OK) return st;
  REQUIRE_SUP(engram::project_mx_supported(N, K),
              "MXFP8 weight of %d x %d bytes exceeds %lld", N, K,
              (long long)ENGRAM_MX_MAX_WEIGHT_BYTES);
  REQUIRE_SUP(int64_t(T) * K <= ENGRAM_MX_MAX_WEIGHT_BYTES,
              "MXFP8 activation of %d x %d bytes exceeds %lld", T, K,
              (long long)ENGRAM_MX_MAX_WEIGHT_BYTES);
  if (T == 0) return ENGRAM_OK;
  REQUIRE(a_codes && aligned(a_codes, 16), "a_codes is NULL or not 16-byte aligned");
  REQUIRE(a_scales && aligned(a_scales, 4), "a_scales is NULL or not 4-byte aligned");
  REQUIRE(wc && aligned(wc, 16), "wkv codes are NULL or not 16-byte aligned");
  REQUIRE(ws && aligned(ws, 4), "wkv scales are NULL or not 4-byte aligned");
  REQUIRE(kv && aligned(kv, 16), "kv is NULL or not 16-byte aligned");
  return ENGRAM_OK;
}
}  // namespace

engram_status engram_project_mxfp8_staged(const uint8_t *a_codes, const uint8_t *a_scales,
                                          int32_t cols, const uint8_t *wkv_codes,
                                          const uint8_t *wkv_scales, uint16_t *kv, int32_t T,
                                          int32_t N, hipStream_t stream) {
  engram_status st =
      check_project_mx_staged(a_codes, a_scales, cols, wkv_codes, wkv_scales, kv, T, N);
  if (st != ENGRAM_OK || T == 0) return st;
  return hip_status(engram::launch_project_mx_staged(a_codes, a_scales, cols, wkv_codes,
                                                     wkv_scales, kv, T, N, stream),
                    "engram_project_mxfp8_staged launch");
}

engram_status engram_gate(float *h, const uint16_t *kv, const uint16_t *q_weight,
                          const uint16_t *k_weight, const uint8_t *token_mask, int32_t T,
                          int32_t hc, int32_t dim, float eps, float clamp, float dot_scale,
                          hipStream_t stream) {
  engram_status st = check_gate_shape(T, hc, dim, eps, clamp);
  if (st != ENGRAM_OK) return st;
  if (T == 0) return ENGRAM_OK;
  if ((st = check_gate_ptrs(h, kv, q_weight, k_weight)) != ENGRAM_OK) return st;
  return hip_status(engram::launch_gate(h, kv, q_weight, k_weight, token_mask, T, hc, dim, eps,
                                        clamp, dot_scale, stream),
                    "engram_gate launch");
}

engram_status engram_gate_layers(float *h, const uint16_t *const *kv,
                                 const uint16_t *const *q_weight,
                                 const uint16_t *const *k_weight, int32_t n_layers,
                                 const uint8_t *token_mask, int32_t T, int32_t hc, int32_t dim,
                                 float eps, float clamp, float dot_scale, hipStream_t stream) {
  REQUIRE_SUP(n_layers >= 1 && n_layers <= ENGRAM_MAX_LAYERS, "n_layers=%d outside 1..%d",
              n_layers, ENGRAM_MAX_LAYERS);
  engram_status st = check_gate_shape(T, hc, dim, eps, clamp);
  if (st != ENGRAM_OK) return st;
  if (T == 0) return ENGRAM_OK;
  REQUIRE(kv && q_weight && k_weight, "kv, q_weight or k_weight array is NULL");
  engram::GateLayers gl{};
  gl.n = n_layers;
  for (int l = 0; l < n_layers; ++l) {
    if ((st = check_gate_ptrs(h, kv[l], q_weight[l], k_weight[l])) != ENGRAM_OK)
      return fail_layer(st, l);
    gl.kv[l] = kv[l];
    gl.qw[l] = q_weight[l];
    gl.kw[l] = k_weight[l];
  }
  return hip_status(engram::launch_gate_layers(h, gl, token_mask, T, hc, dim, eps, clamp,
                                               dot_scale, stream),
                    "engram_gate_layers launch");
}

size_t engram_workspace_bytes(int32_t T, int32_t n_layers, int32_t cols, int32_t hc,
                              int32_t dim) {
  if (T < 0 || n_layers < 0 || cols < 0 || hc < 0 || dim < 0) return 0;
  const size_t t = size_t(T);
  return align256(t * n_layers * cols * sizeof(int32_t)) +
         align256(t * cols * ENGRAM_HEAD_DIM * sizeof(uint16_t)) +
         size_t(n_layers) * align256(t * (size_t(hc) + 1) * dim * sizeof(uint16_t));
}

}  // extern "C"

namespace {

// engram_forward on a given workspace (the caller's, or the static array of
// engram_forward_noalloc).
engram_status forward_impl(const engram_hash_params *params, const engram_tokens *tokens,
                           const engram_layer *layers, float *h, int32_t hc, int32_t dim,
                           float eps, float clamp, float dot_scale, void *workspace,
                           size_t workspace_bytes, int32_t *bad_ids, hipStream_t stream) {
  engram::HashTables tab;
  engram_status st = check_hash_params(params, &tab);
  if (st != ENGRAM_OK) return st;
  if ((st = check_tokens(tokens, params->max_ngram)) != ENGRAM_OK) return st;
  REQUIRE(layers, "layers is NULL");
  const int32_t T = tokens->T, L = params->n_layers;
  const int32_t cols = (params->max_ngram - 1) * params->n_heads;
  const int32_t K = cols * ENGRAM_HEAD_DIM;
  const int64_t N64 = int64_t(hc + 1) * dim;
  REQUIRE_SUP(N64 <= kInt32Max, "(hc+1)*dim too large");
  const int32_t N = int32_t(N64);
  if ((st = check_gate_shape(T, hc, dim, eps, clamp)) != ENGRAM_OK) return st;
  for (int l = 0; l < L; ++l) {
    const engram_layer &ly = layers[l];
    if ((st = check_rows_shape(ly.fmt, ly.num_rows, int64_t(L) * cols, cols, T)) != ENGRAM_OK)
      return fail_layer(st, l);
    int64_t max_row = 0;
    for (int c = 0; c < cols; ++c)
      max_row = std::max<int64_t>(max_row, int64_t(tab.offset[l][c]) + tab.prime[l][c]);
    REQUIRE(max_row <= ly.num_rows, "layer %d: offsets + primes reach row %lld > num_rows %lld",
            l, (long long)max_row, (long long)ly.num_rows);
  }
  if (T == 0) return ENGRAM_OK;
  const size_t need = engram_workspace_bytes(T, L, cols, hc, dim);
  REQUIRE(workspace && aligned(workspace, 256), "workspace is NULL or not 256-byte aligned");
  REQUIRE(workspace_bytes >= need, "workspace_bytes=%zu < required %zu", workspace_bytes, need);

  char *ws = static_cast<char *>(workspace);
  int32_t *ids = reinterpret_cast<int32_t *>(ws);
  ws += align256(size_t(T) * L * cols * sizeof(int32_t));
  uint16_t *rows = reinterpret_cast<uint16_t *>(ws);
  ws += align256(size_t(T) * K * sizeof(uint16_t));
  // MXFP8 layers beyond the weight-streaming form's token count stage their
  // rows in the same buffer: codes [T][K], then scales [T][K / 32].
  uint8_t *const mx_codes = reinterpret_cast<uint8_t *>(rows);
  uint8_t *const mx_scales = mx_codes + align256(size_t(T) * K);
  const bool mx_staged = !engram::project_mx_skinny_supported(T, cols) &&
                         int64_t(T) * K <= ENGRAM_MX_MAX_WEIGHT_BYTES;
  // one kv per layer: every projection runs before the one gate pass
  uint16_t *kv_all = reinterpret_cast<uint16_t *>(ws);
  const size_t kv_elems = align256(size_t(T) * N * sizeof(uint16_t)) / sizeof(uint16_t);
  uint16_t *kv = kv_all;

  for (int l = 0; l < L; ++l) {
    const engram_layer &ly = layers[l];
    if (ly.wkv_mx || ly.wkv_mx_scales) {
      REQUIRE(ly.fmt == ENGRAM_ROWS_FP8_E4M3_E8M0, "layer %d: wkv_mx needs an FP8 table", l);
      st = check_project_mx(ly.table, ly.scales, ly.num_rows, ids, int64_t(L) * cols, cols,
                            ly.wkv_mx, ly.wkv_mx_scales, kv, T, N, bad_ids);
    } else if ((st = check_rows_ptrs(ly.fmt, ly.table, ly.scales, ids, rows, bad_ids)) ==
               ENGRAM_OK) {
      st = check_project_ptrs(rows, ly.wkv, kv);
    }
    if (st != ENGRAM_OK || (st = check_gate_ptrs(h, kv, ly.q_weight, ly.k_weight)) != ENGRAM_OK)
      return fail_layer(st, l);
  }

  if ((st = hip_status(engram::launch_hash(tab, *tokens, ids, stream), "hash launch")) !=
      ENGRAM_OK)
    return st;
  engram::GateLayers gl{};
  gl.n = L;
  for (int l = 0; l < L; ++l) {
    const engram_layer &ly = layers[l];
    kv = kv_all + l * kv_elems;
    gl.kv[l] = kv;
    gl.qw[l] = ly.q_weight;
    gl.kw[l] = ly.k_weight;
    // Q2_K: the fused rows + projection (its weight-streaming form for few
    // tokens).  Few tokens with cols % 4 != 0: rows -> the weight-streaming
    // projection, which beats the fused 256 x 256 tiles there.  FP8 without
    // an MXFP8 weight: rows -> projection, which measures faster than
    // engram_project_fp8 (the rows kernel gathers whole rows once; the fused
    // kernel gathers 128-byte pieces of random rows for every tile column).
    if (ly.wkv_mx && mx_staged) {
      // MXFP8 with the 256 x 256 tiles: the rows are first staged into an
      // MXFP8 activation in the rows buffer, which the tiles then read as
      // they read the weight (the same kv bits as the gather form).
      if ((st = hip_status(engram::launch_stage_mx(ly.table, ly.scales, ly.num_rows,
                                                   ids + l * cols, int64_t(L) * cols, cols, T,
                                                   mx_codes, mx_scales, bad_ids, stream),
                           "MXFP8 staging launch")) != ENGRAM_OK)
        return st;
      if ((st = hip_status(engram::launch_project_mx_staged(mx_codes, mx_scales, cols, ly.wkv_mx,
                                                            ly.wkv_mx_scales, kv, T, N, stream),
                           "MXFP8 project launch")) != ENGRAM_OK)
        return st;
    } else if (ly.wkv_mx) {
      if ((st = hip_status(engram::launch_project_mx(ly.table, ly.scales, ly.num_rows,
                                                     ids + l * cols, int64_t(L) * cols, cols,
                                                     ly.wkv_mx, ly.wkv_mx_scales, kv, T, N,
                                                     bad_ids, stream),
                           "MXFP8 rows+project launch")) != ENGRAM_OK)
        return st;
    } else if (ly.fmt == ENGRAM_ROWS_Q2K && engram::project_q2k_supported(ly.num_rows, cols) &&
               (!engram::project_uses_skinny(T) ||
                engram::project_q2k_skinny_supported(T, cols))) {
      if ((st = hip_status(engram::launch_project_q2k(ly.table, ly.num_rows, ids + l * cols,
                                                      int64_t(L) * cols, cols, ly.wkv, kv, T,
                                                      N, bad_ids, stream),
                           "fused rows+project launch")) != ENGRAM_OK)
        return st;
    } else {
      if ((st = hip_status(engram::launch_rows(ly.fmt, ly.table, ly.scales, ly.num_rows,
                                               ids + l * cols, int64_t(L) * cols, cols, T, rows,
                                               bad_ids, stream),
                           "rows launch")) != ENGRAM_OK)
        return st;
      if ((st = hip_status(engram::launch_project(rows, ly.wkv, kv, T, K, N, stream),
                           "project launch")) != ENGRAM_OK)
        return st;
    }
  }
  // The projections do not depend on h; the gates of all layers, in layer
  // order, then take one pass over the highway.
  return hip_status(engram::launch_gate_layers(h, gl, tokens->token_mask, T, hc, dim, eps,
                                               clamp, dot_scale, stream),
                    "gate launch");
}

// ---- The allocation-free forward's workspace.  A file-scope device array,
// one copy per GPU, held from the module's load until the process ends.  In
// host code its name is only a host-side stand-in: every use goes through
// the device address hipGetSymbolAddress returns for the GPU in question,
// looked up once per device (with that device current) and kept here.
__device__ __align__(256) uint8_t scratch[ENGRAM_FORWARD_NOALLOC_MAX_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

engram_status scratch_for_stream(hipStream_t stream, void **out) {
  int cur = 0, dev = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  dev = cur;
  if (stream) {
    if ((e = hipStreamGetDevice(stream, &dev)) != hipSuccess)
      return hip_status(e, "hipStreamGetDevice");
  }
  REQUIRE_SUP(dev >= 0 && dev < kMaxDevices, "device %d beyond the %d this library tracks", dev,
              kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e, "hipSetDevice");
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ENGRAM_OK;
}

}  // namespace

extern "C" {

engram_status engram_forward(const engram_hash_params *params, const engram_tokens *tokens,
                             const engram_layer *layers, float *h, int32_t hc, int32_t dim,
                             float eps, float clamp, float dot_scale, void *workspace,
                             size_t workspace_bytes, int32_t *bad_ids, hipStream_t stream) {
  return forward_impl(params, tokens, layers, h, hc, dim, eps, clamp, dot_scale, workspace,
                      workspace_bytes, bad_ids, stream);
}

engram_status engram_forward_noalloc(const engram_hash_params *params,
                                     const engram_tokens *tokens, const engram_layer *layers,
                                     float *h, int32_t hc, int32_t dim, float eps, float clamp,
                                     float dot_scale, int32_t *bad_ids, hipStream_t stream) {
  engram::HashTables tab;
  engram_status st = check_hash_params(params, &tab);
  if (st != ENGRAM_OK) return st;
  if ((st = check_tokens(tokens, params->max_ngram)) != ENGRAM_OK) return st;
  const int32_t cols = (params->max_ngram - 1) * params->n_heads;
  const size_t need = engram_workspace_bytes(tokens->T, params->n_layers, cols, hc, dim);
  REQUIRE_SUP(need <= size_t(ENGRAM_FORWARD_NOALLOC_MAX_BYTES),
              "this shape needs %zu bytes of workspace, above the %u of the static array "
              "(use engram_forward with a workspace)",
              need, unsigned(ENGRAM_FORWARD_NOALLOC_MAX_BYTES));
  void *ws = nullptr;
  if (tokens->T > 0 && (st = scratch_for_stream(stream, &ws)) != ENGRAM_OK) return st;
  return forward_impl(params, tokens, layers, h, hc, dim, eps, clamp, dot_scale, ws,
                      size_t(ENGRAM_FORWARD_NOALLOC_MAX_BYTES), bad_ids, stream);
}

}  // extern "C"
