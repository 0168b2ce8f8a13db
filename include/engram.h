/*
 * engram.h -- C ABI of libengram.so: the DeepSeek-V4.1 Engram forward on one
 * AMD Instinct MI355X (gfx950).
 *
 * The forward has four stages: n-gram hash, quantised row gather and dequant,
 * bf16 projection, gate.  Each runs as a hand-written HIP kernel.  The stages
 * are described on three public pages:
 *   [spark] "Module engram_v41" (spark_model layers API docs): the overview's
 *           four numbered stages and the ENGRAM_ROW_BYTES constant;
 *   [NeMo]  "nemo_automodel.components.models.deepseek_v41.engram":
 *           DeepseekV41NgramHash.forward, DeepseekV41Engram.forward,
 *           _engram_gate_core, compile_engram_gate;
 *   [vLLM]  "vllm.models.deepseek_v41.common.engram": Engram,
 *           EngramLayout, NgramHashState.forward, ParallelEngramEmbedding,
 *           _engram_lookup_kernel, compute_hash_multipliers.
 *
 * Conventions for every entry point:
 *   - Memory.  The caller allocates every device buffer and keeps it alive
 *     until the queued work has finished.  The library allocates nothing and
 *     keeps no state between calls.  Small hash tables are passed as HOST
 *     arrays; they are read during the call and copied into kernel arguments.
 *   - Asynchrony.  Work is queued on `stream` (NULL = the legacy default
 *     stream) and the call returns without synchronising.
 *   - Errors.  All arguments are validated on the host before anything is
 *     launched: ENGRAM_ERR_ARG and ENGRAM_ERR_UNSUPPORTED mean nothing was
 *     queued.  ENGRAM_ERR_HIP means a launch failed (in engram_forward the
 *     stages queued before it may still run).  After any non-OK status
 *     engram_last_error() returns a message for the calling thread.
 *     The library does not read device memory to validate it: the contents
 *     of cu_seqlens and similar arrays are the caller's promise (the kernels
 *     still keep every access inside the buffers whose sizes are passed).
 *   - Empty input.  T == 0 returns ENGRAM_OK and queues nothing.
 *   - bf16 values are stored as uint16_t bit patterns (the upper half of an
 *     IEEE binary32).  Every conversion to bf16 rounds to nearest, ties to even.
 *   - Alignment.  Every device pointer must be 16-byte aligned, except
 *     `table` (4 bytes for Q2_K, 16 for FP8) and the byte masks (any alignment).
 *   - Concurrency.  Calls on different streams are independent.  Calls that
 *     write the same buffers must be ordered by the caller.
 */
#ifndef ENGRAM_H
#define ENGRAM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden visibility; only these entry points are exported. */
#if defined(ENGRAM_BUILDING_LIBRARY)
#define ENGRAM_API __attribute__((visibility("default")))
#else
#define ENGRAM_API
#endif

/* In C++ the enums get a fixed 32-bit underlying type, so that any int32
 * value a C caller passes is a valid value to compare (the checks reject
 * unknown ones) rather than undefined behaviour; the ABI is an int either way. */
#ifdef __cplusplus
#define ENGRAM_ENUM_BASE : int32_t
#else
#define ENGRAM_ENUM_BASE
#endif

typedef enum engram_status ENGRAM_ENUM_BASE {
  ENGRAM_OK = 0,
  ENGRAM_ERR_ARG = 1,          /* invalid argument: null, misaligned, bad size     */
  ENGRAM_ERR_UNSUPPORTED = 2,  /* valid for the method, beyond this library's limits */
  ENGRAM_ERR_HIP = 3           /* a HIP launch or runtime call failed             */
} engram_status;

typedef enum engram_row_format ENGRAM_ENUM_BASE {
  ENGRAM_ROWS_Q2K = 0,             /* one 84-byte Q2_K super-block per row        */
  ENGRAM_ROWS_FP8_E4M3_E8M0 = 1    /* 256 e4m3fn bytes + 8 e8m0 bytes per row     */
} engram_row_format;

#define ENGRAM_HEAD_DIM 256        /* values per table row                         */
#define ENGRAM_Q2K_ROW_BYTES 84    /* [spark] ENGRAM_ROW_BYTES                     */
#define ENGRAM_FP8_ROW_BYTES 256
#define ENGRAM_FP8_SCALE_BYTES 8   /* one e8m0 byte per 32 values                  */
#define ENGRAM_MAX_LAYERS 4        /* engram layers hashed in one call             */
#define ENGRAM_MAX_NGRAM 8         /* orders 2..max_ngram                          */
#define ENGRAM_MAX_COLS 64         /* (max_ngram - 1) * n_heads per layer          */
#define ENGRAM_MAX_HC 8            /* hyper-connection streams                     */
#define ENGRAM_MAX_DIM 8192        /* hidden size                                  */

/* Hash-table metadata of all engram layers ([vLLM] EngramLayout and
 * compute_hash_multipliers; the spark page ships them as checkpoint
 * metadata).  HOST pointers, read during the call.
 *   multipliers [n_layers][max_ngram]: entry k multiplies the token k
 *              positions back (k = 0: the current token); any int64.
 *   primes     [n_layers][cols]: bucket size of column c, in [1, 2^31).
 *   offsets    [n_layers][cols]: first row of column c, >= 0, with
 *              offsets + primes <= 2^31 so that every id fits int32.
 *   Column c = (n - 2) * n_heads + j holds order n (2..max_ngram), head j.
 *   pad_id: compressed id that stands in for absent or blocked history.
 */
typedef struct engram_hash_params {
  int32_t n_layers;            /* 1..ENGRAM_MAX_LAYERS                            */
  int32_t max_ngram;           /* 2..ENGRAM_MAX_NGRAM                             */
  int32_t n_heads;             /* >= 1, (max_ngram - 1) * n_heads <= MAX_COLS     */
  int32_t pad_id;
  const int64_t *multipliers;
  const int64_t *primes;
  const int64_t *offsets;
} engram_hash_params;

/* A batch of tokens: T positions split into n_seqs chunks.  DEVICE pointers.
 *   cids [T]: compressed token ids (the pages hash compressed ids; the
 *        token map that produces them is outside this library).
 *   cu_seqlens [n_seqs + 1]: chunk s is positions cu[s] .. cu[s+1]-1;
 *        cu[0] = 0, nondecreasing, cu[n_seqs] = T.
 *   doc_ids [T] or NULL: document of each position; 0 marks padding
 *        ([NeMo] DeepseekV41NgramHash.forward sequence_ids).
 *   token_mask [T] or NULL: 0 marks image/padding positions.  They block
 *        lookback through them, and the gate leaves them unchanged.
 *   lookback [n_seqs][lookback_depth] or NULL: the ids just before each
 *        chunk, oldest first, so lookback[s][depth-1] directly precedes
 *        position cu[s] ([vLLM] module docstring, NgramHashState.forward).
 *   lookback_live: same shape or NULL (all live); 0 = unusable entry.
 */
typedef struct engram_tokens {
  int32_t T;
  int32_t n_seqs;              /* >= 1 when T > 0                                 */
  int32_t lookback_depth;      /* 0..max_ngram-1                                  */
  const int32_t *cids;
  const int32_t *cu_seqlens;
  const int32_t *doc_ids;
  const uint8_t *token_mask;
  const int32_t *lookback;
  const uint8_t *lookback_live;
} engram_tokens;

/* One engram layer's resident weights.  DEVICE pointers.
 *   Q2K: table [num_rows][84], scales NULL.
 *   FP8: table [num_rows][256] e4m3fn codes, scales [num_rows][8] e8m0 bytes.
 *   wkv [(hc+1)*dim][cols*256] bf16, row-major (the projection's weight;
 *        output o = sum_k rows[k] * wkv[o][k]).
 *   q_weight, k_weight [hc][dim] bf16 (learned branch-norm weights).
 *   wkv_mx, wkv_mx_scales: NULL, or (FP8 layers only) the MXFP8 copy of wkv
 *        from engram_quantize_mxfp8, codes [(hc+1)*dim][cols*256] and scales
 *        [(hc+1)*dim][cols*8].  When given, the layer projects its raw FP8
 *        rows against them (engram_project_mxfp8) and wkv may be NULL.
 */
typedef struct engram_layer {
  engram_row_format fmt;
  int64_t num_rows;
  const uint8_t *table;
  const uint8_t *scales;
  const uint16_t *wkv;
  const uint16_t *q_weight;
  const uint16_t *k_weight;
  const uint8_t *wkv_mx;
  const uint8_t *wkv_mx_scales;
} engram_layer;

/* Stage 1 -- n-gram hash ([spark] overview stage 1; [vLLM] EngramLayout,
 * NgramHashState.forward; [NeMo] DeepseekV41NgramHash.forward).
 * For every position t, layer l, order n and head j (column c):
 *   tok_0 = cids[t]; tok_k = the id k positions back if that position and
 *     every position between it and t is live, else pad_id.  A position is
 *     live if it lies in t's chunk or in its lookback, is not masked, and
 *     (when doc_ids is given) has the same non-zero document as t.  A padding
 *     position (doc 0) has no history.  A dead lookback entry is not live.
 *   mix_n = XOR over k < n of (uint64)tok_k * (uint64)multipliers[l][k]
 *     (64-bit wrapping products; within 0 <= id < vocab none wrap).
 *   ids[t][l][c] = offsets[l][c] + mix_n mod primes[l][c].
 * Output ids: DEVICE int32 [T][n_layers][cols], fully overwritten.
 */
ENGRAM_API engram_status engram_hash(const engram_hash_params *params, const engram_tokens *tokens,
                          int32_t *ids, hipStream_t stream);

/* Lookback store for streaming decode ([vLLM] module docstring and
 * NgramHashState.forward: a decode step hashes against the ids just before
 * its chunk).  history DEVICE int32 [n_seqs][depth] and history_live DEVICE
 * [n_seqs][depth], oldest first, are updated IN PLACE to what the sequences'
 * next chunks need as lookback (pass them as tokens->lookback /
 * lookback_live of the next batch; start from all-zero history_live).  For
 * sequence s with chunk [start, end), entry j becomes position
 * p = end - depth + j:
 *   p >= start: cids[p]; live unless token_mask[p] == 0, and, with doc_ids,
 *     only if doc_ids[p] equals the document of position end - 1 and that
 *     is not 0 (the next chunk continues that document);
 *   p < start: the old entry depth - (start - p) (token 0, dead when that
 *     index is negative); it keeps its liveness, except that with doc_ids
 *     every older entry turns dead when doc_ids[start] differs from the
 *     document of position end - 1 or that document is 0.
 * An empty chunk leaves its sequence unchanged.  Uses tokens' T, n_seqs,
 * cids, cu_seqlens, doc_ids and token_mask (its lookback fields are
 * ignored: the store is the lookback).  Run it after the batch's hash on the
 * same stream.  1 <= depth <= ENGRAM_MAX_NGRAM - 1.
 */
ENGRAM_API engram_status engram_history_update(const engram_tokens *tokens, int32_t depth,
                                               int32_t *history, uint8_t *history_live,
                                               hipStream_t stream);

/* Stage 2 -- row gather + dequant to bf16 ([spark] overview stage 2,
 * ENGRAM_ROW_BYTES; [vLLM] _engram_lookup_kernel, bf16 mode).
 *   ids: DEVICE int32; row r of token t is ids[t * ids_token_stride + r],
 *        r < cols (pass ids + l * cols and stride n_layers * cols to use
 *        layer l of engram_hash's output).
 *   rows: DEVICE bf16 [T][cols * 256]; rows[t][r*256 + i] is value i of
 *        table row ids[t][r], fully overwritten.
 *   Q2_K value i of a block: bytes 0..15 hold (min << 4 | scale) per 16
 *     values, bytes 16..79 the 2-bit quants (value i: byte
 *     16 + 32*(i/128) + i%32, bits 2*((i%128)/32)), bytes 80..81 fp16 d,
 *     82..83 fp16 dmin; y = d*scale*q - dmin*min, rounded to bf16 once from
 *     its exact value for every finite d and dmin (non-finite d or dmin give
 *     unspecified inf/NaN values).
 *   FP8 value i: e4m3fn code times 2^(scales[row][i/32] - 127) (the byte is
 *     placed in the binary32 exponent field, so byte 0 gives 0), then bf16.
 *   An id outside [0, num_rows) yields a zero row; if bad_ids (DEVICE int32,
 *   nullable) is given, it is atomically incremented once per such row.
 */
ENGRAM_API engram_status engram_rows(engram_row_format fmt, const uint8_t *table, const uint8_t *scales,
                          int64_t num_rows, const int32_t *ids, int64_t ids_token_stride,
                          int32_t cols, int32_t T, uint16_t *rows, int32_t *bad_ids,
                          hipStream_t stream);

/* Stage 3 -- projection kv = rows x wkv^T ([spark] overview stage 3; [vLLM]
 * Engram, the wkv linear without bias).
 *   rows DEVICE bf16 [T][K], wkv DEVICE bf16 [N][K], kv DEVICE bf16 [T][N],
 *   all row-major; K % 64 == 0.  Products accumulate in fp32 on the matrix
 *   cores and each output is rounded to bf16 once.  T <= 128 (decode) runs a
 *   kernel that streams wkv once from HBM with K split four ways per
 *   workgroup; more tokens run 256 x 256 output tiles.  Either way the
 *   result does not depend on timing.
 */
ENGRAM_API engram_status engram_project(const uint16_t *rows, const uint16_t *wkv, uint16_t *kv,
                             int32_t T, int32_t K, int32_t N, hipStream_t stream);

/* Stages 2 + 3 fused for Q2_K tables ([spark] overview stages 2-3): kv =
 * bf16(dequant(table[ids])) x wkv^T without writing the bf16 rows to memory.
 * The projection reads each row's 84-byte block and dequantises it on chip.
 * kv is bit for bit what engram_rows followed by engram_project gives (same
 * values, same fp32 accumulation order) for T > 128, and for T <= 128 when
 * cols % 4 == 0 (then the weight-streaming form runs, whose four K quarters
 * are whole table columns); for T <= 128 with other column counts the
 * 256 x 256 tiles run and sum in another order than engram_project.
 *   table DEVICE Q2_K [num_rows][84], 4-byte aligned; ids, ids_token_stride,
 *   cols, bad_ids as for engram_rows (K = cols * 256); wkv DEVICE bf16 [N][K];
 *   kv DEVICE bf16 [T][N], 16-byte aligned, fully overwritten.
 *   Limits: num_rows * 84 <= ENGRAM_Q2K_FUSED_MAX_BYTES (the blocks are read
 *   through one 32-bit-offset buffer descriptor) and cols <=
 *   ENGRAM_Q2K_FUSED_MAX_COLS (each workgroup keeps its rows' block offsets in
 *   LDS); beyond either the call returns ENGRAM_ERR_UNSUPPORTED and
 *   engram_forward uses rows -> projection instead.
 */
#define ENGRAM_Q2K_FUSED_MAX_BYTES 2147483504LL
#define ENGRAM_Q2K_FUSED_MAX_COLS 32
ENGRAM_API engram_status engram_project_q2k(const uint8_t *table, int64_t num_rows,
                                 const int32_t *ids, int64_t ids_token_stride, int32_t cols,
                                 const uint16_t *wkv, uint16_t *kv, int32_t T, int32_t N,
                                 int32_t *bad_ids, hipStream_t stream);

/* Stages 2 + 3 fused for FP8 tables with the bf16 weight ([vLLM]
 * _engram_lookup_kernel, bf16 mode, then [spark] overview stage 3): kv =
 * bf16(dequant(table[ids])) x wkv^T without writing the bf16 rows to memory.
 * The projection reads each row's 256 codes and 8 scale bytes and converts
 * them on chip to the values engram_rows gives (e4m3fn code x 2^(byte -
 * 127), rounded to bf16; NaN codes and scale bytes 0 and 255 included), and
 * sums the same products in the same fp32 order as engram_project, so kv is
 * bit for bit what engram_rows followed by engram_project gives.  It runs
 * 256 x 256 output tiles whatever T is and needs no rows buffer (T * cols *
 * 512 bytes for engram_rows); it is about 4 % slower than engram_rows
 * followed by engram_project (measured at 16384 tokens: the fused kernel
 * gathers 128-byte pieces of random table rows for every column of tiles),
 * so engram_forward runs rows -> projection for FP8 layers.
 *   table DEVICE [num_rows][256] e4m3fn codes, 16-byte aligned; scales DEVICE
 *   [num_rows][8] e8m0, 4-byte aligned; ids, ids_token_stride, cols, bad_ids
 *   as for engram_rows (K = cols * 256; an id outside the table gives a zero
 *   row); wkv DEVICE bf16 [N][K]; kv DEVICE bf16 [T][N], 16-byte aligned,
 *   fully overwritten.
 *   Limit: T * ids_token_stride * 4 <= ENGRAM_FP8_FUSED_MAX_ID_BYTES (the ids
 *   are read through a 32-bit-offset buffer descriptor), else
 *   ENGRAM_ERR_UNSUPPORTED.  The table has no size limit (its rows are read
 *   through 64-bit addresses).
 */
#define ENGRAM_FP8_FUSED_MAX_ID_BYTES 2147483632LL
ENGRAM_API engram_status engram_project_fp8(const uint8_t *table, const uint8_t *scales,
                                            int64_t num_rows, const int32_t *ids,
                                            int64_t ids_token_stride, int32_t cols,
                                            const uint16_t *wkv, uint16_t *kv, int32_t T,
                                            int32_t N, int32_t *bad_ids, hipStream_t stream);

/* MXFP8 copy of a bf16 weight, for engram_project_mxfp8 ([vLLM] EngramBatch:
 * the WKV GEMM there takes MXFP8 operands, in the OCP MX v1.0 format).
 *   w DEVICE bf16 [N][K], K % 32 == 0; codes DEVICE [N][K] e4m3fn, 16-byte
 *   aligned; scales DEVICE [N][K/32] e8m0 (byte b means 2^(b-127)).
 *   Per 32 consecutive k of a row: amax = max |w|; scale byte =
 *   floor(log2 amax) - 8 + 127 clamped to 0..254 (127 when amax = 0); each
 *   code is w / 2^(byte-127) saturated to +-448 and rounded to the nearest
 *   E4M3 value, ties to even (negative zero keeps its sign).  Inf/NaN inputs
 *   are not supported.  Runs once per weight; the result is deterministic.
 */
ENGRAM_API engram_status engram_quantize_mxfp8(const uint16_t *w, int32_t N, int32_t K,
                                               uint8_t *codes, uint8_t *scales,
                                               hipStream_t stream);

/* Stages 2 + 3 for FP8 tables in MXFP8 ([vLLM] EngramBatch / wkv_input: FP8
 * rows with per-32 E8M0 scales are MX blocks already): kv[t][n] =
 * bf16(sum_k a[t][k] * w[n][k]), a[t][r*256 + i] = e4m3(table[ids[t][r]][i])
 * * 2^(scales[ids[t][r]][i/32] - 127), w = wkv_codes/wkv_scales likewise.
 * The rows are read raw by the block-scaled matrix cores and never
 * dequantised to memory: 256 x 256 output tiles of
 * v_mfma_scale_f32_32x32x64_f8f6f4, or, for T <= 64 with cols % 4 == 0 and
 * cols <= 64, a kernel that streams the weight once from HBM into
 * v_mfma_scale_f32_16x16x128_f8f6f4 with K split four ways per workgroup.
 * The matrix cores sum each instruction's 64 or 128 products below fp32
 * precision (probed: a product keeps only its bits down to 2^-13 of the
 * largest product beside it, truncated toward zero; on random e4m3 data the
 * error reaches 1.7e-4 of the sum of |products|); the instructions' results
 * accumulate in fp32 in a fixed order and
 * each output is rounded to bf16 once, so the result does not depend on
 * timing (but differs between the two forms in the last bits).
 *   table DEVICE [num_rows][256] e4m3fn codes, 16-byte aligned; scales DEVICE
 *   [num_rows][8], 4-byte aligned; ids, ids_token_stride, cols, bad_ids as for
 *   engram_rows (K = cols * 256; an id outside the table contributes 0);
 *   wkv_codes DEVICE [N][K], 16-byte aligned, and wkv_scales DEVICE [N][K/32],
 *   4-byte aligned, from engram_quantize_mxfp8; kv DEVICE bf16 [T][N], 16-byte
 *   aligned, fully overwritten.
 *   Limits: N * K <= ENGRAM_MX_MAX_WEIGHT_BYTES and T * ids_token_stride * 4 <=
 *   ENGRAM_MX_MAX_WEIGHT_BYTES (both are read through 32-bit-offset buffer
 *   descriptors); beyond either the call returns ENGRAM_ERR_UNSUPPORTED.  The
 *   table has no size limit (its rows are read through 64-bit addresses).
 */
#define ENGRAM_MX_MAX_WEIGHT_BYTES 2147483632LL
ENGRAM_API engram_status engram_project_mxfp8(const uint8_t *table, const uint8_t *scales,
                                              int64_t num_rows, const int32_t *ids,
                                              int64_t ids_token_stride, int32_t cols,
                                              const uint8_t *wkv_codes,
                                              const uint8_t *wkv_scales, uint16_t *kv,
                                              int32_t T, int32_t N, int32_t *bad_ids,
                                              hipStream_t stream);

/* The MXFP8 activation of FP8 rows, for engram_project_mxfp8_staged ([vLLM]
 * EngramBatch: the FP8 rows of a batch are staged into an MXFP8 buffer that
 * the WKV GEMM takes as its activation).  Row r of token t is copied as
 * stored: a_codes[t][r*256 + i] = table[ids[t][r]][i], a_scales[t][r*8 + b] =
 * scales[ids[t][r]][b].  An id outside the table gives zero codes and scale
 * bytes 127 (2^0; the row contributes exactly 0 to any product) and is
 * counted in bad_ids as engram_rows counts it.
 *   table, scales, num_rows, ids, ids_token_stride, cols, T, bad_ids as for
 *   engram_project_mxfp8; a_codes DEVICE [T][cols*256], 16-byte aligned;
 *   a_scales DEVICE [T][cols*8], 4-byte aligned; both fully overwritten.
 */
ENGRAM_API engram_status engram_stage_mxfp8(const uint8_t *table, const uint8_t *scales,
                                            int64_t num_rows, const int32_t *ids,
                                            int64_t ids_token_stride, int32_t cols, int32_t T,
                                            uint8_t *a_codes, uint8_t *a_scales,
                                            int32_t *bad_ids, hipStream_t stream);

/* engram_project_mxfp8 on a staged MXFP8 activation (engram_stage_mxfp8):
 * kv[t][n] = bf16(sum_k a[t][k] * w[n][k]) with a = a_codes/a_scales and w =
 * wkv_codes/wkv_scales as in engram_project_mxfp8.  Always the 256 x 256
 * tiles, reading the activation as they read the weight; the same kv bits as
 * engram_project_mxfp8's tile form on the rows that were staged (for every
 * T > 64, and for every T when cols % 4 != 0 or cols > 64).
 *   a_codes DEVICE [T][K], 16-byte aligned; a_scales DEVICE [T][K/32],
 *   4-byte aligned (K = cols * 256); wkv_codes, wkv_scales, kv, N as for
 *   engram_project_mxfp8.
 *   Limits: N * K and T * K <= ENGRAM_MX_MAX_WEIGHT_BYTES (32-bit-offset
 *   buffer descriptors); beyond either the call returns
 *   ENGRAM_ERR_UNSUPPORTED.
 */
ENGRAM_API engram_status engram_project_mxfp8_staged(const uint8_t *a_codes,
                                                     const uint8_t *a_scales, int32_t cols,
                                                     const uint8_t *wkv_codes,
                                                     const uint8_t *wkv_scales, uint16_t *kv,
                                                     int32_t T, int32_t N, hipStream_t stream);

/* Stage 4 -- gate, in place on the fp32 highway ([spark] overview stage 4;
 * [NeMo] _engram_gate_core, compile_engram_gate; [vLLM] Engram).
 *   h DEVICE fp32 [T][hc][dim], updated in place.
 *   kv DEVICE bf16 [T][(hc+1)*dim]: hc keys (stream-major), then the shared value.
 *   q_weight, k_weight DEVICE bf16 [hc][dim].  token_mask DEVICE [T] or NULL.
 *   For each token t with a non-zero mask and each stream s, in fp32:
 *     a = dot_scale * sum_i (x_i q_i)(key_i k_i) / (rms(x) rms(key)),
 *         rms(v) = sqrt(mean(v^2) + eps), x = h[t][s], key = key s of t;
 *     z = sign(a) * sqrt(max(|a|, clamp));  g = 1 / (1 + exp(-z));
 *     h[t][s][i] += g * value[i].
 *   Masked tokens are not written, so they stay unchanged bit for bit.
 *   Limits: 1 <= hc <= ENGRAM_MAX_HC, 8 <= dim <= ENGRAM_MAX_DIM, dim % 8 == 0.
 */
ENGRAM_API engram_status engram_gate(float *h, const uint16_t *kv, const uint16_t *q_weight,
                          const uint16_t *k_weight, const uint8_t *token_mask, int32_t T,
                          int32_t hc, int32_t dim, float eps, float clamp, float dot_scale,
                          hipStream_t stream);

/* Stage 4 for several layers in one pass: the gates of layers 0..n_layers-1,
 * in that order, on the same h (engram_forward's layers, which nothing
 * separates), with h read and written once.  The result is bit for bit that
 * of engram_gate called per layer in order.  kv, q_weight, k_weight: HOST
 * arrays [n_layers] of DEVICE pointers, each as for engram_gate;
 * 1 <= n_layers <= ENGRAM_MAX_LAYERS.  Other arguments as for engram_gate.
 */
ENGRAM_API engram_status engram_gate_layers(float *h, const uint16_t *const *kv,
                                            const uint16_t *const *q_weight,
                                            const uint16_t *const *k_weight, int32_t n_layers,
                                            const uint8_t *token_mask, int32_t T, int32_t hc,
                                            int32_t dim, float eps, float clamp,
                                            float dot_scale, hipStream_t stream);

/* Bytes of device workspace engram_forward needs for this shape: the ids,
 * one layer's rows and every layer's kv, each 256-byte aligned. */
ENGRAM_API size_t engram_workspace_bytes(int32_t T, int32_t n_layers, int32_t cols, int32_t hc,
                              int32_t dim);

/* The whole forward ([spark] overview, stages 1-4): hash every layer once,
 * then for each layer in order: rows -> projection -> gate on the same h.
 * The projections do not read h, so all of them run first, each into its own
 * kv, and one gate pass then applies the layers' gates in order with h held
 * in registers (h read and written once; the same bits as per-layer gates).
 * Q2_K layers within the limits of engram_project_q2k run rows -> projection
 * as that fused kernel (same kv bits) when T > 128, or when T <= 128 and
 * cols % 4 == 0; other few-token Q2_K layers run rows -> the weight-streaming
 * projection.  FP8 layers that carry wkv_mx run the MXFP8 projection instead
 * of rows -> projection: engram_project_mxfp8's weight-streaming form where
 * it applies (T <= 64, cols % 4 == 0, cols <= 64), else engram_stage_mxfp8
 * into the rows buffer -> engram_project_mxfp8_staged (T * K within its
 * limit; beyond it engram_project_mxfp8's gather tiles).
 *   layers: HOST array [params->n_layers] of DEVICE-pointer descriptors.
 *   workspace: DEVICE, at least engram_workspace_bytes(...) bytes, 256-byte
 *   aligned; its contents are scratch.  Every other argument is as for the
 *   per-stage calls; the gate mask is tokens->token_mask.  Validation also
 *   checks offsets + primes <= num_rows for every layer.
 */
ENGRAM_API engram_status engram_forward(const engram_hash_params *params, const engram_tokens *tokens,
                             const engram_layer *layers, float *h, int32_t hc, int32_t dim,
                             float eps, float clamp, float dot_scale, void *workspace,
                             size_t workspace_bytes, int32_t *bad_ids, hipStream_t stream);

/* engram_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, checks and results as engram_forward, without workspace
 * and workspace_bytes: the workspace is a static device array of
 * ENGRAM_FORWARD_NOALLOC_MAX_BYTES bytes that the library holds on every GPU
 * it runs on, from the first call there until the process ends (looked up,
 * not allocated: the call itself allocates nothing).  A shape whose
 * engram_workspace_bytes exceeds the array returns ENGRAM_ERR_UNSUPPORTED
 * (32 MiB: e.g. up to 512 tokens at 24 columns, hc = 4, dim = 4096).  The
 * GPU is the stream's (the current device for the NULL stream).  Every call
 * on one GPU uses the same array, which keeps the last call's contents:
 * calls that overlap in time on one GPU (other streams, other threads) race,
 * and the caller must order them.
 */
#define ENGRAM_FORWARD_NOALLOC_MAX_BYTES (32u << 20)
ENGRAM_API engram_status engram_forward_noalloc(const engram_hash_params *params,
                                                const engram_tokens *tokens,
                                                const engram_layer *layers, float *h,
                                                int32_t hc, int32_t dim, float eps, float clamp,
                                                float dot_scale, int32_t *bad_ids,
                                                hipStream_t stream);

/* Message for the calling thread's last non-OK status ("" if none). */
ENGRAM_API const char *engram_last_error(void);

/* Identity of the sources this library was built from: "sha256:" and the
 * hex digest of the kernel sources, headers and build script ("unknown" for
 * a build outside the package's build script).  A static string. */
ENGRAM_API const char *engram_build_id(void);

#ifdef __cplusplus
}
#endif
#endif /* ENGRAM_H */
