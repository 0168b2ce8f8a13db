"""ctypes binding of libengram.so, with the C entry points' names.

Argument marshalling only: every stage runs in the library's HIP kernels.
Device buffers are torch tensors on the GPU; the binding passes their data
pointers and the current torch stream (or the stream given).  Before each
call it checks that every device tensor is on the GPU, contiguous, of the
right dtype and large enough for the sizes passed.  The C library cannot see
buffer sizes, and a short buffer would make a kernel read out of bounds.

The library is loaded after torch, so it binds to the HIP runtime that torch
already loaded (both name the same soname), and torch streams are valid in it.
If libengram.so has not been built, importing this module raises ImportError:
there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libengram.so")

ENGRAM_OK, ENGRAM_ERR_ARG, ENGRAM_ERR_UNSUPPORTED, ENGRAM_ERR_HIP = 0, 1, 2, 3
ENGRAM_ROWS_Q2K, ENGRAM_ROWS_FP8_E4M3_E8M0 = 0, 1
HEAD_DIM, Q2K_ROW_BYTES, FP8_ROW_BYTES, FP8_SCALE_BYTES = 256, 84, 256, 8

EXPORTS = ("engram_hash", "engram_history_update", "engram_rows", "engram_project", "engram_project_q2k",
           "engram_project_fp8", "engram_quantize_mxfp8", "engram_project_mxfp8",
           "engram_stage_mxfp8", "engram_project_mxfp8_staged", "engram_gate",
           "engram_gate_layers", "engram_workspace_bytes", "engram_forward", "engram_last_error",
           "engram_build_id", "engram_forward_noalloc")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python gram_hash_memory_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)
_lib.engram_build_id.restype = c_char_p
BUILD_ID = _lib.engram_build_id().decode()


def _expected_build_id() -> str | None:
    # The build script beside this file hashes the sources it builds from.
    import importlib.util
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "build.py")
    if not os.path.exists(path):
        return None
    spec = importlib.util.spec_from_file_location("_engram_build_ids", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.build_id()


_want = _expected_build_id()
if _want is not None and BUILD_ID != _want:
    raise ImportError(f"{LIB_PATH} was built from other sources ({BUILD_ID}, sources are "
                      f"{_want}); rebuild with `python gram_hash_memory_amd/build.py`")


class _HashParams(ctypes.Structure):
    _fields_ = [("n_layers", c_int32), ("max_ngram", c_int32), ("n_heads", c_int32),
                ("pad_id", c_int32), ("multipliers", c_void_p), ("primes", c_void_p),
                ("offsets", c_void_p)]


class _Tokens(ctypes.Structure):
    _fields_ = [("T", c_int32), ("n_seqs", c_int32), ("lookback_depth", c_int32),
                ("cids", c_void_p), ("cu_seqlens", c_void_p), ("doc_ids", c_void_p),
                ("token_mask", c_void_p), ("lookback", c_void_p), ("lookback_live", c_void_p)]


class _Layer(ctypes.Structure):
    _fields_ = [("fmt", c_int), ("num_rows", c_int64), ("table", c_void_p),
                ("scales", c_void_p), ("wkv", c_void_p), ("q_weight", c_void_p),
                ("k_weight", c_void_p), ("wkv_mx", c_void_p), ("wkv_mx_scales", c_void_p)]


_P = ctypes.POINTER
_lib.engram_hash.argtypes = [_P(_HashParams), _P(_Tokens), c_void_p, c_void_p]
_lib.engram_history_update.argtypes = [_P(_Tokens), c_int32, c_void_p, c_void_p, c_void_p]
_lib.engram_rows.argtypes = [c_int, c_void_p, c_void_p, c_int64, c_void_p, c_int64, c_int32,
                             c_int32, c_void_p, c_void_p, c_void_p]
_lib.engram_project.argtypes = [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                c_void_p]
_lib.engram_project_q2k.argtypes = [c_void_p, c_int64, c_void_p, c_int64, c_int32, c_void_p,
                                    c_void_p, c_int32, c_int32, c_void_p, c_void_p]
_lib.engram_project_fp8.argtypes = [c_void_p, c_void_p, c_int64, c_void_p, c_int64, c_int32,
                                   c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p]
_lib.engram_quantize_mxfp8.argtypes = [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p]
_lib.engram_project_mxfp8.argtypes = [c_void_p, c_void_p, c_int64, c_void_p, c_int64, c_int32,
                                      c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_void_p,
                                      c_void_p]
_lib.engram_stage_mxfp8.argtypes = [c_void_p, c_void_p, c_int64, c_void_p, c_int64, c_int32,
                                    c_int32, c_void_p, c_void_p, c_void_p, c_void_p]
_lib.engram_project_mxfp8_staged.argtypes = [c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                             c_void_p, c_int32, c_int32, c_void_p]
_lib.engram_gate.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                             c_int32, c_int32, c_float, c_float, c_float, c_void_p]
_lib.engram_gate_layers.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                    c_int32, c_int32, c_int32, c_float, c_float, c_float,
                                    c_void_p]
_lib.engram_workspace_bytes.argtypes = [c_int32, c_int32, c_int32, c_int32, c_int32]
_lib.engram_workspace_bytes.restype = c_size_t
_lib.engram_forward.argtypes = [_P(_HashParams), _P(_Tokens), _P(_Layer), c_void_p, c_int32,
                                c_int32, c_float, c_float, c_float, c_void_p, c_size_t,
                                c_void_p, c_void_p]
_lib.engram_forward_noalloc.argtypes = [_P(_HashParams), _P(_Tokens), _P(_Layer), c_void_p,
                                        c_int32, c_int32, c_float, c_float, c_float, c_void_p,
                                        c_void_p]
_lib.engram_last_error.restype = c_char_p
for _name in ("engram_hash", "engram_history_update", "engram_rows", "engram_project", "engram_project_q2k",
              "engram_project_fp8", "engram_quantize_mxfp8", "engram_project_mxfp8",
              "engram_stage_mxfp8", "engram_project_mxfp8_staged", "engram_gate",
              "engram_gate_layers", "engram_forward", "engram_forward_noalloc"):
    getattr(_lib, _name).restype = c_int


class EngramError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"engram status {status}: {message}")
        self.status = status


def engram_last_error() -> str:
    return (_lib.engram_last_error() or b"").decode()


def engram_build_id() -> str:
    """sha256 of the sources the loaded library was built from."""
    return BUILD_ID


def _check(status: int) -> None:
    if status != ENGRAM_OK:
        raise EngramError(status, engram_last_error())


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _dptr(t, dtype, min_numel: int = 0, name: str = "tensor"):
    """Device pointer of a contiguous GPU tensor with at least min_numel elements."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < min_numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {min_numel}")
    return t.data_ptr()


class HashParams:
    """engram_hash_params: host tables, kept alive as long as this object."""

    def __init__(self, multipliers, primes, offsets, max_ngram: int, n_heads: int, pad_id: int):
        self.multipliers = np.ascontiguousarray(multipliers, dtype=np.int64)
        self.primes = np.ascontiguousarray(primes, dtype=np.int64)
        self.offsets = np.ascontiguousarray(offsets, dtype=np.int64)
        self.n_layers = int(self.primes.shape[0])
        self.max_ngram, self.n_heads, self.pad_id = int(max_ngram), int(n_heads), int(pad_id)
        self.cols = (self.max_ngram - 1) * self.n_heads
        if self.multipliers.shape != (self.n_layers, self.max_ngram) or \
                self.primes.shape != (self.n_layers, self.cols) or \
                self.offsets.shape != (self.n_layers, self.cols):
            raise ValueError("hash table shapes do not match n_layers/max_ngram/n_heads")
        self.c = _HashParams(self.n_layers, self.max_ngram, self.n_heads, self.pad_id,
                             self.multipliers.ctypes.data, self.primes.ctypes.data,
                             self.offsets.ctypes.data)

    @classmethod
    def from_dict(cls, d: dict) -> "HashParams":
        return cls(d["multipliers"], d["primes"], d["offsets"], d["max_ngram"], d["n_heads"],
                   d["pad_id"])


class Tokens:
    """engram_tokens over GPU tensors (kept alive as long as this object)."""

    def __init__(self, cids, cu_seqlens, doc_ids=None, token_mask=None, lookback=None,
                 lookback_live=None):
        self.T = int(cids.numel())
        self.n_seqs = int(cu_seqlens.numel()) - 1
        self.depth = 0 if lookback is None else int(lookback.shape[1])
        if lookback is not None and lookback.shape[0] != self.n_seqs:
            raise ValueError("lookback must have one row per sequence")
        self._keep = (cids, cu_seqlens, doc_ids, token_mask, lookback, lookback_live)
        self.c = _Tokens(self.T, self.n_seqs, self.depth,
                         _dptr(cids, torch.int32, self.T, "cids"),
                         _dptr(cu_seqlens, torch.int32, self.n_seqs + 1, "cu_seqlens"),
                         _dptr(doc_ids, torch.int32, self.T, "doc_ids"),
                         _dptr(token_mask, torch.uint8, self.T, "token_mask"),
                         _dptr(lookback, torch.int32, self.n_seqs * self.depth, "lookback"),
                         _dptr(lookback_live, torch.uint8, self.n_seqs * self.depth,
                               "lookback_live"))
        self.token_mask = token_mask


def engram_hash(params: HashParams, tokens: Tokens, ids: torch.Tensor, stream=None) -> None:
    """Stage 1: ids int32 [T, n_layers, cols] from the token batch."""
    p = _dptr(ids, torch.int32, tokens.T * params.n_layers * params.cols, "ids")
    _check(_lib.engram_hash(ctypes.byref(params.c), ctypes.byref(tokens.c), p, _stream(stream)))


def engram_history_update(tokens: Tokens, history, history_live, stream=None) -> None:
    """Update the lookback store (int32 and uint8 [n_seqs, depth]) in place after a batch."""
    depth = int(history.shape[1]) if history.dim() == 2 else 0
    n = tokens.n_seqs * depth
    _check(_lib.engram_history_update(ctypes.byref(tokens.c), depth,
                                      _dptr(history, torch.int32, n, "history"),
                                      _dptr(history_live, torch.uint8, n, "history_live"),
                                      _stream(stream)))


def engram_rows(fmt: int, table, scales, num_rows: int, ids, ids_token_stride: int, cols: int,
                T: int, rows, bad_ids=None, stream=None) -> None:
    """Stage 2: bf16 rows [T, cols*256] (int16 tensor of bf16 bits) from ids."""
    row_bytes = Q2K_ROW_BYTES if fmt == ENGRAM_ROWS_Q2K else FP8_ROW_BYTES
    need_ids = 0 if T <= 0 else (T - 1) * ids_token_stride + cols
    _check(_lib.engram_rows(
        int(fmt), _dptr(table, torch.uint8, num_rows * row_bytes, "table"),
        _dptr(scales, torch.uint8, num_rows * FP8_SCALE_BYTES, "scales"), int(num_rows),
        _dptr(ids, torch.int32, need_ids, "ids"), int(ids_token_stride), int(cols), int(T),
        _dptr(rows, torch.int16, T * cols * HEAD_DIM, "rows"),
        _dptr(bad_ids, torch.int32, 1, "bad_ids"), _stream(stream)))


def engram_project(rows, wkv, kv, T: int, K: int, N: int, stream=None) -> None:
    """Stage 3: kv [T, N] = rows [T, K] x wkv [N, K]^T (bf16 bits in int16 tensors)."""
    _check(_lib.engram_project(_dptr(rows, torch.int16, T * K, "rows"),
                               _dptr(wkv, torch.int16, N * K, "wkv"),
                               _dptr(kv, torch.int16, T * N, "kv"), int(T), int(K), int(N),
                               _stream(stream)))


def engram_project_q2k(table, num_rows: int, ids, ids_token_stride: int, cols: int, wkv, kv,
                       T: int, N: int, bad_ids=None, stream=None) -> None:
    """Stages 2 + 3 fused for a Q2_K table: kv [T, N] from ids, bit-identical
    to engram_rows followed by engram_project for T > 128, and for T <= 128
    when cols % 4 == 0 (its weight-streaming form)."""
    K = cols * HEAD_DIM
    need_ids = 0 if T <= 0 else (T - 1) * ids_token_stride + cols
    _check(_lib.engram_project_q2k(
        _dptr(table, torch.uint8, num_rows * Q2K_ROW_BYTES, "table"), int(num_rows),
        _dptr(ids, torch.int32, need_ids, "ids"), int(ids_token_stride), int(cols),
        _dptr(wkv, torch.int16, N * K, "wkv"), _dptr(kv, torch.int16, T * N, "kv"), int(T),
        int(N), _dptr(bad_ids, torch.int32, 1, "bad_ids"), _stream(stream)))


def engram_project_fp8(table, scales, num_rows: int, ids, ids_token_stride: int, cols: int, wkv,
                       kv, T: int, N: int, bad_ids=None, stream=None) -> None:
    """Stages 2 + 3 fused for an FP8 table with the bf16 weight: kv [T, N] from
    ids, bit-identical to engram_rows followed by engram_project."""
    K = cols * HEAD_DIM
    need_ids = 0 if T <= 0 else (T - 1) * ids_token_stride + cols
    _check(_lib.engram_project_fp8(
        _dptr(table, torch.uint8, num_rows * FP8_ROW_BYTES, "table"),
        _dptr(scales, torch.uint8, num_rows * FP8_SCALE_BYTES, "scales"), int(num_rows),
        _dptr(ids, torch.int32, need_ids, "ids"), int(ids_token_stride), int(cols),
        _dptr(wkv, torch.int16, N * K, "wkv"), _dptr(kv, torch.int16, T * N, "kv"), int(T),
        int(N), _dptr(bad_ids, torch.int32, 1, "bad_ids"), _stream(stream)))


def engram_quantize_mxfp8(w, N: int, K: int, codes, scales, stream=None) -> None:
    """MXFP8 copy of bf16 w [N, K]: codes uint8 [N, K] (e4m3fn), scales uint8 [N, K/32] (e8m0)."""
    _check(_lib.engram_quantize_mxfp8(_dptr(w, torch.int16, N * K, "w"), int(N), int(K),
                                      _dptr(codes, torch.uint8, N * K, "codes"),
                                      _dptr(scales, torch.uint8, N * (K // 32), "scales"),
                                      _stream(stream)))


def engram_project_mxfp8(table, scales, num_rows: int, ids, ids_token_stride: int, cols: int,
                         wkv_codes, wkv_scales, kv, T: int, N: int, bad_ids=None,
                         stream=None) -> None:
    """Stages 2 + 3 for an FP8 table in MXFP8: kv [T, N] from ids and the MXFP8 wkv."""
    K = cols * HEAD_DIM
    need_ids = 0 if T <= 0 else (T - 1) * ids_token_stride + cols
    _check(_lib.engram_project_mxfp8(
        _dptr(table, torch.uint8, num_rows * FP8_ROW_BYTES, "table"),
        _dptr(scales, torch.uint8, num_rows * FP8_SCALE_BYTES, "scales"), int(num_rows),
        _dptr(ids, torch.int32, need_ids, "ids"), int(ids_token_stride), int(cols),
        _dptr(wkv_codes, torch.uint8, N * K, "wkv_codes"),
        _dptr(wkv_scales, torch.uint8, N * (K // 32), "wkv_scales"),
        _dptr(kv, torch.int16, T * N, "kv"), int(T), int(N),
        _dptr(bad_ids, torch.int32, 1, "bad_ids"), _stream(stream)))


def engram_stage_mxfp8(table, scales, num_rows: int, ids, ids_token_stride: int, cols: int,
                       T: int, a_codes, a_scales, bad_ids=None, stream=None) -> None:
    """The MXFP8 activation of FP8 rows: codes [T, cols*256] and scales [T, cols*8]."""
    need_ids = 0 if T <= 0 else (T - 1) * ids_token_stride + cols
    _check(_lib.engram_stage_mxfp8(
        _dptr(table, torch.uint8, num_rows * FP8_ROW_BYTES, "table"),
        _dptr(scales, torch.uint8, num_rows * FP8_SCALE_BYTES, "scales"), int(num_rows),
        _dptr(ids, torch.int32, need_ids, "ids"), int(ids_token_stride), int(cols), int(T),
        _dptr(a_codes, torch.uint8, T * cols * HEAD_DIM, "a_codes"),
        _dptr(a_scales, torch.uint8, T * cols * FP8_SCALE_BYTES, "a_scales"),
        _dptr(bad_ids, torch.int32, 1, "bad_ids"), _stream(stream)))


def engram_project_mxfp8_staged(a_codes, a_scales, cols: int, wkv_codes, wkv_scales, kv, T: int,
                                N: int, stream=None) -> None:
    """kv [T, N] from a staged MXFP8 activation and the MXFP8 wkv."""
    K = cols * HEAD_DIM
    _check(_lib.engram_project_mxfp8_staged(
        _dptr(a_codes, torch.uint8, T * K, "a_codes"),
        _dptr(a_scales, torch.uint8, T * (K // 32), "a_scales"), int(cols),
        _dptr(wkv_codes, torch.uint8, N * K, "wkv_codes"),
        _dptr(wkv_scales, torch.uint8, N * (K // 32), "wkv_scales"),
        _dptr(kv, torch.int16, T * N, "kv"), int(T), int(N), _stream(stream)))


def engram_gate(h, kv, q_weight, k_weight, token_mask, T: int, hc: int, dim: int, eps: float,
                clamp: float, dot_scale: float, stream=None) -> None:
    """Stage 4: update fp32 h [T, hc, dim] in place."""
    _check(_lib.engram_gate(_dptr(h, torch.float32, T * hc * dim, "h"),
                            _dptr(kv, torch.int16, T * (hc + 1) * dim, "kv"),
                            _dptr(q_weight, torch.int16, hc * dim, "q_weight"),
                            _dptr(k_weight, torch.int16, hc * dim, "k_weight"),
                            _dptr(token_mask, torch.uint8, T, "token_mask"), int(T), int(hc),
                            int(dim), float(eps), float(clamp), float(dot_scale),
                            _stream(stream)))


def engram_gate_layers(h, kvs, q_weights, k_weights, token_mask, T: int, hc: int, dim: int,
                       eps: float, clamp: float, dot_scale: float, stream=None) -> None:
    """Stage 4 for several layers in one pass over h (layer order), as engram_forward runs it."""
    n = len(kvs)
    if not (len(q_weights) == len(k_weights) == n):
        raise ValueError("one kv, q_weight and k_weight per layer")
    arr = lambda ts, numel, name: (c_void_p * n)(*[_dptr(t, torch.int16, numel, name) for t in ts])
    kv_a = arr(kvs, T * (hc + 1) * dim, "kv")
    q_a = arr(q_weights, hc * dim, "q_weight")
    k_a = arr(k_weights, hc * dim, "k_weight")
    _check(_lib.engram_gate_layers(_dptr(h, torch.float32, T * hc * dim, "h"), kv_a, q_a, k_a, n,
                                   _dptr(token_mask, torch.uint8, T, "token_mask"), int(T),
                                   int(hc), int(dim), float(eps), float(clamp), float(dot_scale),
                                   _stream(stream)))


def engram_workspace_bytes(T: int, n_layers: int, cols: int, hc: int, dim: int) -> int:
    return int(_lib.engram_workspace_bytes(T, n_layers, cols, hc, dim))


class Layer:
    """engram_layer over GPU tensors (kept alive as long as this object)."""

    def __init__(self, fmt: int, table, scales, wkv, q_weight, k_weight, hc: int, dim: int,
                 cols: int, wkv_mx=None, wkv_mx_scales=None):
        row_bytes = Q2K_ROW_BYTES if fmt == ENGRAM_ROWS_Q2K else FP8_ROW_BYTES
        self.num_rows = int(table.numel()) // row_bytes
        self._keep = (table, scales, wkv, q_weight, k_weight, wkv_mx, wkv_mx_scales)
        n, k = (hc + 1) * dim, cols * HEAD_DIM
        self.c = _Layer(int(fmt), self.num_rows,
                        _dptr(table, torch.uint8, self.num_rows * row_bytes, "table"),
                        _dptr(scales, torch.uint8, self.num_rows * FP8_SCALE_BYTES, "scales"),
                        _dptr(wkv, torch.int16, n * k, "wkv"),
                        _dptr(q_weight, torch.int16, hc * dim, "q_weight"),
                        _dptr(k_weight, torch.int16, hc * dim, "k_weight"),
                        _dptr(wkv_mx, torch.uint8, n * k, "wkv_mx"),
                        _dptr(wkv_mx_scales, torch.uint8, n * (k // 32), "wkv_mx_scales"))


def engram_forward(params: HashParams, tokens: Tokens, layers, h, hc: int, dim: int,
                   eps: float, clamp: float, dot_scale: float, workspace,
                   bad_ids=None, stream=None) -> None:
    """Whole forward on h (fp32 [T, hc, dim], in place); workspace is a uint8 GPU tensor."""
    if len(layers) != params.n_layers:
        raise ValueError("one Layer per hashed layer is required")
    arr = (_Layer * len(layers))(*[l.c for l in layers])
    need = engram_workspace_bytes(tokens.T, params.n_layers, params.cols, hc, dim)
    ws = _dptr(workspace, torch.uint8, need, "workspace")
    _check(_lib.engram_forward(ctypes.byref(params.c), ctypes.byref(tokens.c), arr,
                               _dptr(h, torch.float32, tokens.T * hc * dim, "h"), int(hc),
                               int(dim), float(eps), float(clamp), float(dot_scale), ws,
                               int(workspace.numel()) if workspace is not None else 0,
                               _dptr(bad_ids, torch.int32, 1, "bad_ids"), _stream(stream)))


FORWARD_NOALLOC_MAX_BYTES = 32 << 20


def engram_forward_noalloc(params: HashParams, tokens: Tokens, layers, h, hc: int, dim: int,
                           eps: float, clamp: float, dot_scale: float, bad_ids=None,
                           stream=None) -> None:
    """engram_forward on the library's static device workspace (no allocation)."""
    if len(layers) != params.n_layers:
        raise ValueError("one Layer per hashed layer is required")
    arr = (_Layer * len(layers))(*[l.c for l in layers])
    _check(_lib.engram_forward_noalloc(ctypes.byref(params.c), ctypes.byref(tokens.c), arr,
                                       _dptr(h, torch.float32, tokens.T * hc * dim, "h"),
                                       int(hc), int(dim), float(eps), float(clamp),
                                       float(dot_scale), _dptr(bad_ids, torch.int32, 1, "bad_ids"),
                                       _stream(stream)))
