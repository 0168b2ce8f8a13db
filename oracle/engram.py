"""The four stages of the Engram forward, plainly -- oracle side, test infrastructure.

Sources (page title, then section):
* [spark] "Module engram_v41": the module overview's four numbered stages
  (hash, Q2_K rows, dense bf16 projection, gate in place on the fp32
  highway) and the ENGRAM_ROW_BYTES constant (one Q2_K super-block per row).
* [NeMo] "nemo_automodel.components.models.deepseek_v41.engram":
  DeepseekV41NgramHash.forward (no lookback across document, image or
  padding boundaries; a False token_mask blocks lookback through that
  position; sequence id 0 marks padding), DeepseekV41Engram.forward and
  _engram_gate_core (shapes, masked tokens keep their streams),
  compile_engram_gate (three hidden-dim reductions: stream RMS, key RMS,
  stream-key dot).
* [vLLM] "vllm.models.deepseek_v41.common.engram": module docstring
  (lookback ids just before each chunk), Engram (one key per hc copy plus
  a shared value; normalised dot, signed square root, sigmoid; clamp 1e-6),
  EngramLayout, NgramHashState.forward ([tokens, layers, cols] int32 ids,
  pad id for missing history), _engram_lookup_kernel (FP8 dequant, ids
  outside the table read as zero rows), compute_hash_multipliers.

Where the pages are silent this module takes the readings listed in the
design notes (A1..A19); each is named where it is used.
"""

from __future__ import annotations

import numpy as np

from .numerics import (bf16_round, bf16_bits, bf16_value, fp16_value,
                       e4m3fn_value, e8m0_scale)
from .mx import rows_fp8_mx, project_mxfp8

HEAD_DIM = 256          # values per table row
Q2K_ROW_BYTES = 84      # [spark] ENGRAM_ROW_BYTES: one Q2_K super-block
FP8_ROW_BYTES = 256     # e4m3 codes per row; plus 256 / 32 = 8 e8m0 scale bytes
FP8_BLOCK = 32          # values per e8m0 scale

_U64 = (1 << 64) - 1


# --------------------------------------------------------------------------- hash

def _history(t, seq_start, depth_avail, cids, doc_ids, token_mask, lb_row,
             lb_live_row, max_ngram, pad_id):
    """Token ids at distances 0..max_ngram-1 before position t (reading A5).

    Distance 0 is the token itself (reading A6: a masked token still hashes
    its own id).  Walking back, the first position that is absent or not
    live -- masked, padding (doc 0), another document, or a dead lookback
    entry -- and every position before it read as pad_id.
    """
    hist = [int(cids[t])]
    own_doc = None if doc_ids is None else int(doc_ids[t])
    blocked = own_doc == 0           # a padding token has no history (reading A7)
    for k in range(1, max_ngram):
        q = t - k
        tok = pad_id
        if not blocked:
            if q >= seq_start:
                live = True
                if token_mask is not None and not token_mask[q]:
                    live = False
                if own_doc is not None and int(doc_ids[q]) != own_doc:
                    live = False
                tok = int(cids[q])
            else:
                j = depth_avail - (seq_start - q)    # lookback is oldest first (A8)
                if lb_row is None or j < 0:
                    live = False
                else:
                    live = lb_live_row is None or bool(lb_live_row[j])
                    tok = int(lb_row[j])
            if not live:
                blocked = True
        hist.append(pad_id if blocked else tok)
    return hist


def hash_ids(cids, cu_seqlens, multipliers, primes, offsets, max_ngram, n_heads,
             pad_id, doc_ids=None, token_mask=None, lookback=None,
             lookback_live=None) -> np.ndarray:
    """n-gram hash ids, int32 [T, n_layers, (max_ngram-1)*n_heads].

    For layer l, order n in 2..max_ngram and head j (column c = (n-2)*n_heads + j):
        mix = XOR over k < n of (tok_k * multipliers[l][k])        (reading A1, A2)
        id  = offsets[l][c] + mix mod primes[l][c]                 (reading A3, A4)
    Tokens are 64-bit two's-complement values and products wrap mod 2**64;
    inside the method's domain (0 <= token < compressed vocab) no product
    wraps, which is why the pages bound the multipliers.

    cu_seqlens [n_seqs+1] splits the flat tokens into sequences (chunks);
    lookback [n_seqs, depth] holds the ids just before each chunk, oldest
    first, with lookback_live marking usable entries (all if None).
    """
    cids = np.asarray(cids)
    T = int(cids.shape[0])
    mult = [[int(v) & _U64 for v in row] for row in np.asarray(multipliers)]
    prm = [[int(v) for v in row] for row in np.asarray(primes)]
    off = [[int(v) for v in row] for row in np.asarray(offsets)]
    n_layers, cols = len(prm), (max_ngram - 1) * n_heads
    assert all(len(r) == max_ngram for r in mult)
    assert all(len(r) == cols for r in prm) and all(len(r) == cols for r in off)
    out = np.zeros((T, n_layers, cols), dtype=np.int64)
    cu = [int(v) for v in np.asarray(cu_seqlens)]
    depth = 0 if lookback is None else int(np.asarray(lookback).shape[1])
    for s in range(len(cu) - 1):
        lb_row = None if lookback is None or depth == 0 else np.asarray(lookback)[s]
        lb_live = None if lookback_live is None else np.asarray(lookback_live)[s]
        for t in range(cu[s], cu[s + 1]):
            hist = _history(t, cu[s], depth, cids, doc_ids, token_mask, lb_row,
                            lb_live, max_ngram, pad_id)
            for l in range(n_layers):
                mix = 0
                for n in range(1, max_ngram + 1):
                    mix ^= ((hist[n - 1] & _U64) * mult[l][n - 1]) & _U64
                    if n < 2:
                        continue
                    for j in range(n_heads):
                        c = (n - 2) * n_heads + j
                        out[t, l, c] = off[l][c] + mix % prm[l][c]
    if out.size and (out.max() > np.iinfo(np.int32).max):
        raise ValueError("hash id exceeds int32")
    return out.astype(np.int32)


def history_update(history, history_live, cids, cu_seqlens, doc_ids=None, token_mask=None):
    """The lookback store after a batch: (history, live), both [n_seqs, depth].

    [vLLM] module docstring and NgramHashState.forward: a decode step hashes
    its tokens against the ids just before its chunk (the lookback).  This
    defines the store a streaming caller keeps so that step i + 1's lookback
    is what step i leaves behind (reading A25).  Entry j of sequence s (oldest
    first) is position p = end - depth + j, end = cu_seqlens[s + 1], the
    position that precedes the sequence's next chunk by depth - j:
      * inside the chunk (p >= start): its token; live unless masked, and,
        with doc_ids, only if its document is the chunk's last position's
        and not padding (the next chunk continues that document);
      * before the chunk: the old entry start - p positions before the
        chunk, if the old store reaches that far (else token 0, dead); it
        keeps its liveness, except that with doc_ids a chunk whose first and
        last documents differ, or whose last document is padding, leaves
        every older entry dead.
    An empty chunk leaves the sequence's entries unchanged.
    """
    hist = np.array(history, dtype=np.int64, copy=True)
    live = np.array(history_live, dtype=np.uint8, copy=True)
    n_seqs, depth = hist.shape
    new_h = hist.copy()
    new_l = live.copy()
    cu = [int(v) for v in np.asarray(cu_seqlens)]
    for s in range(n_seqs):
        start, end = cu[s], cu[s + 1]
        if end == start:
            continue
        last_doc = None if doc_ids is None else int(doc_ids[end - 1])
        old_ok = last_doc is None or (last_doc != 0 and int(doc_ids[start]) == last_doc)
        for j in range(depth):
            p = end - depth + j
            if p >= start:
                tok = int(cids[p])
                ok = token_mask is None or bool(token_mask[p])
                if last_doc is not None:
                    ok = ok and last_doc != 0 and int(doc_ids[p]) == last_doc
            else:
                jo = depth - (start - p)
                if jo < 0:
                    tok, ok = 0, False
                else:
                    tok, ok = int(hist[s, jo]), bool(live[s, jo]) and old_ok
            new_h[s, j], new_l[s, j] = tok, 1 if ok else 0
    return new_h.astype(np.int32), new_l


# --------------------------------------------------------------------------- rows

def _q2k_dequant_blocks(blocks: np.ndarray) -> np.ndarray:
    """Exact float64 values of Q2_K super-blocks [M, 84] -> [M, 256] (reading A10, A11).

    Block bytes: 0..15 sixteen (min << 4 | scale) nibble pairs, one per 16
    values; 16..79 the 2-bit quants; 80..81 fp16 d; 82..83 fp16 dmin (both
    little-endian).  Value i uses quant byte 32*(i // 128) + i % 32 at bit
    2*((i % 128) // 32), and scale/min pair i // 16:
        y_i = d * scale * q - dmin * min
    In float64 every product and the difference are exact for all fp16 d, dmin.
    """
    blocks = np.asarray(blocks, dtype=np.uint8)
    sc = (blocks[:, 0:16] & 0x0F).astype(np.float64)
    mn = (blocks[:, 0:16] >> 4).astype(np.float64)
    qs = blocks[:, 16:80]
    d = fp16_value(blocks[:, 80].astype(np.uint16) | (blocks[:, 81].astype(np.uint16) << 8))
    dmin = fp16_value(blocks[:, 82].astype(np.uint16) | (blocks[:, 83].astype(np.uint16) << 8))
    y = np.empty((blocks.shape[0], HEAD_DIM), dtype=np.float64)
    for i in range(HEAD_DIM):
        byte = qs[:, 32 * (i // 128) + (i % 32)]
        q = ((byte >> (2 * ((i % 128) // 32))) & 3).astype(np.float64)
        b = i // 16
        y[:, i] = d * sc[:, b] * q - dmin * mn[:, b]
    return y


def rows_q2k(table, ids) -> np.ndarray:
    """bf16 bits [T, cols*256] of the Q2_K rows named by ids [T, cols].

    [spark] overview stage 2: one 84-byte block per 256-wide row, written
    as rows[t, c*256 + i].  Ids outside [0, num_rows) give zero rows
    ([vLLM] _engram_lookup_kernel: unowned ids read as zeros).
    """
    table = np.asarray(table, dtype=np.uint8)
    assert table.ndim == 2 and table.shape[1] == Q2K_ROW_BYTES
    ids = np.asarray(ids, dtype=np.int64)
    T, cols = ids.shape
    flat = ids.reshape(-1)
    ok = (flat >= 0) & (flat < table.shape[0])
    y = _q2k_dequant_blocks(table[np.where(ok, flat, 0)])
    y[~ok] = 0.0
    return bf16_bits(bf16_round(y)).reshape(T, cols * HEAD_DIM)


def rows_fp8(table, scales, ids) -> np.ndarray:
    """bf16 bits [T, cols*256] of FP8 rows: e4m3fn code x 2**(e8m0 byte - 127) (reading A12).

    [vLLM] _engram_lookup_kernel, bf16 mode: value i of a row takes scale
    byte i // 32 of the same row; the product is rounded to bf16.
    """
    table = np.asarray(table, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    assert table.shape[1] == FP8_ROW_BYTES and scales.shape[1] == FP8_ROW_BYTES // FP8_BLOCK
    ids = np.asarray(ids, dtype=np.int64)
    T, cols = ids.shape
    flat = ids.reshape(-1)
    ok = (flat >= 0) & (flat < table.shape[0])
    safe = np.where(ok, flat, 0)
    vals = e4m3fn_value(table[safe])
    scl = np.repeat(e8m0_scale(scales[safe]), FP8_BLOCK, axis=1)
    y = vals * scl
    y[~ok] = 0.0
    return bf16_bits(bf16_round(y)).reshape(T, cols * HEAD_DIM)


# --------------------------------------------------------------------- projection

def project(rows_bits, wkv_bits) -> np.ndarray:
    """kv = bf16(rows @ wkv^T), bf16 bits [T, N] ([spark] overview stage 3).

    rows [T, K] and wkv [N, K] are bf16 bits; the sum runs in float64 and is
    rounded to bf16 once.
    """
    a = bf16_value(rows_bits)
    b = bf16_value(wkv_bits)
    return bf16_bits(bf16_round(a @ b.T))


# --------------------------------------------------------------------------- gate

def gate(h, kv_bits, q_weight_bits, k_weight_bits, token_mask, eps, clamp,
         dot_scale, return_preact=False):
    """Gate the shared value into every stream; returns new fp32 h [T, hc, dim].

    [spark] stage 4, [vLLM] Engram, [NeMo] _engram_gate_core.  For each
    unmasked token t and stream s, with x = h[t,s], key = kv[t, s*dim:(s+1)*dim]
    (keys first, stream-major; value last -- reading A13):
        xn  = x   / sqrt(mean(x^2)   + eps) * q_weight[s]      (reading A15)
        kn  = key / sqrt(mean(key^2) + eps) * k_weight[s]
        a   = dot_scale * sum(xn * kn)                          (reading A14)
        z   = sign(a) * sqrt(max(|a|, clamp))                   (reading A16)
        g   = 1 / (1 + exp(-z))
        h[t,s] <- x + g * value
    Masked tokens keep their streams bit for bit (reading A17).  Everything
    runs in float64; the result is rounded to fp32 once (reading A19).
    With return_preact, also returns a [T, hc] (the scaled normalised dot).
    """
    h = np.asarray(h, dtype=np.float32)
    T, hc, dim = h.shape
    kv = bf16_value(kv_bits).reshape(T, (hc + 1) * dim)
    qw = bf16_value(q_weight_bits).reshape(hc, dim)
    kw = bf16_value(k_weight_bits).reshape(hc, dim)
    x = h.astype(np.float64)
    key = kv[:, : hc * dim].reshape(T, hc, dim)
    value = kv[:, hc * dim:]
    xn = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * qw
    kn = key / np.sqrt(np.mean(key * key, axis=-1, keepdims=True) + eps) * kw
    a = dot_scale * np.sum(xn * kn, axis=-1)
    z = np.sign(a) * np.sqrt(np.maximum(np.abs(a), clamp))
    g = 1.0 / (1.0 + np.exp(-z))
    new = (x + g[:, :, None] * value[:, None, :]).astype(np.float32)
    if token_mask is not None:
        keep = ~np.asarray(token_mask, dtype=bool)
        new[keep] = h[keep]
    if return_preact:
        return new, a
    return new


# ------------------------------------------------------------------------ forward

def forward(h, cids, cu_seqlens, hash_params, layers, eps, clamp, dot_scale,
            doc_ids=None, token_mask=None, lookback=None, lookback_live=None,
            return_intermediates=False):
    """Whole forward: hash every layer, then rows -> projection -> gate per layer.

    hash_params: dict(multipliers, primes, offsets, max_ngram, n_heads, pad_id).
    layers: list of dicts with 'fmt' ('q2k' or 'fp8'), 'table', 'scales'
    (fp8 only), 'wkv', 'q_weight', 'k_weight' (bf16 bits); they run in order
    on the same h (reading A18).  The gate mask is token_mask.  An fp8 layer
    that also carries 'wkv_mx' = (codes, scales) from mx.quantize_mxfp8 is
    projected in MXFP8 (mx.project_mxfp8 of the raw rows) instead.
    """
    ids = hash_ids(cids, cu_seqlens, hash_params["multipliers"], hash_params["primes"],
                   hash_params["offsets"], hash_params["max_ngram"],
                   hash_params["n_heads"], hash_params["pad_id"], doc_ids=doc_ids,
                   token_mask=token_mask, lookback=lookback,
                   lookback_live=lookback_live)
    h = np.asarray(h, dtype=np.float32)
    inter = []
    for l, layer in enumerate(layers):
        if layer["fmt"] == "q2k":
            rows = rows_q2k(layer["table"], ids[:, l, :])
        elif layer["fmt"] == "fp8" and layer.get("wkv_mx") is not None:
            # MXFP8 projection (oracle.mx): raw rows against the MXFP8 wkv copy
            a_codes, a_scales = rows_fp8_mx(layer["table"], layer["scales"], ids[:, l, :])
            rows = None
            kv = project_mxfp8(a_codes, a_scales, *layer["wkv_mx"])
        elif layer["fmt"] == "fp8":
            rows = rows_fp8(layer["table"], layer["scales"], ids[:, l, :])
        else:
            raise ValueError(layer["fmt"])
        if rows is not None:
            kv = project(rows, layer["wkv"])
        h = gate(h, kv, layer["q_weight"], layer["k_weight"], token_mask, eps, clamp,
                 dot_scale)
        inter.append({"rows": rows, "kv": kv})
    if return_intermediates:
        return h, ids, inter
    return h
