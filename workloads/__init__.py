"""Seeded synthetic inputs for the five Engram workloads.

This module only draws numbers: token ids, masks, table bytes, weights and
the highway.  It holds none of the method's arithmetic.  Both the HIP path
and the CPU oracle consume what it returns.

The hash-table metadata (primes, offsets, multipliers), which a real model
ships with its checkpoint, is read from tests/golden/hash_tables.json. That
file is written by tests/golden/make_hash_tables.py from the oracle's layout
rules.

Seeds: every array comes from numpy's PCG64 seeded with 1000 * config + tag:
ids 1, table 10 + layer, wkv 20 + layer, q/k weights 30 + layer, highway 40,
mask 50, lookback 60.  The decode and prefill workloads share the table,
wkv and q/k draws (seeded as the decode workload).  Large draws are split
into chunks with seed [1000 * config + tag, chunk] so that they can run in
parallel.
"""

from __future__ import annotations

import json
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from functools import lru_cache

import numpy as np

HEAD_DIM = 256
Q2K_ROW_BYTES = 84
FP8_SCALES_PER_ROW = 8

_HASH_TABLES = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "tests", "golden", "hash_tables.json")


@dataclass(frozen=True)
class Spec:
    index: int
    name: str
    seq_lens: tuple              # chunk length per sequence
    layer_ids: tuple             # engram layer ids (seed the multipliers)
    n_heads: int
    compressed_vocab: int        # compressed token-id space; ids drawn below it
    engram_vocab_size: int       # prime search start + 1
    num_rows: int                # table rows per layer
    fmt: str                     # 'q2k' or 'fp8'
    dim: int
    hc: int
    id_dist: str                 # 'uniform' or 'zipf'
    max_ngram: int = 4
    lookback_depth: int = 0
    doc_len: int = 0             # >0: documents of this many tokens (doc ids 1, 2, ...)
    mask: tuple = ()             # ('spans', n) or ('choice', n): exactly n masked tokens
    eps: float = 1e-6
    clamp: float = 1e-6
    pad_id: int = 0
    weight_seed_config: int = -1  # config whose table/wkv/q,k draws are reused (-1: own)

    @property
    def T(self) -> int:
        return int(sum(self.seq_lens))

    @property
    def cols(self) -> int:
        return (self.max_ngram - 1) * self.n_heads

    @property
    def K(self) -> int:
        return self.cols * HEAD_DIM

    @property
    def N(self) -> int:
        return (self.hc + 1) * self.dim

    @property
    def dot_scale(self) -> float:
        return 1.0 / math.sqrt(self.dim)


SPECS = (
    Spec(0, "tiny", (64,), (1,), 2, 1000, 2713, 16384, "q2k", 128, 2, "uniform"),
    Spec(1, "decode", (1,) * 64, (1,), 8, 131072, 174000, 4194304, "q2k", 4096, 4,
         "uniform", lookback_depth=3),
    Spec(2, "prefill", (2048,) * 4, (1,), 8, 131072, 174000, 4194304, "q2k", 4096, 4,
         "zipf", weight_seed_config=1),
    Spec(3, "two_layer", (2048,) * 2, (1, 14), 8, 131072, 174000, 4194304, "q2k", 4096,
         4, "uniform", doc_len=512, mask=("spans", 410)),
    Spec(4, "fp8", (2048,) * 8, (1,), 8, 131072, 698000, 16777216, "fp8", 4096, 4,
         "zipf", mask=("choice", 819)),
)


@dataclass
class Layer:
    fmt: str
    table: np.ndarray            # uint8 [R, 84] (q2k) or [R, 256] (fp8 e4m3 codes)
    scales: np.ndarray | None    # uint8 [R, 8] e8m0 bytes (fp8) or None
    wkv: np.ndarray              # uint16 bf16 bits [N, K]
    q_weight: np.ndarray         # uint16 bf16 bits [hc, dim]
    k_weight: np.ndarray         # uint16 bf16 bits [hc, dim]

    def as_dict(self) -> dict:
        return dict(fmt=self.fmt, table=self.table, scales=self.scales, wkv=self.wkv,
                    q_weight=self.q_weight, k_weight=self.k_weight)


@dataclass
class Workload:
    spec: Spec
    cids: np.ndarray             # int32 [T]
    cu_seqlens: np.ndarray       # int32 [S+1]
    doc_ids: np.ndarray | None   # int32 [T]
    token_mask: np.ndarray | None  # uint8 [T]; 0 = masked
    lookback: np.ndarray | None  # int32 [S, depth], oldest first
    lookback_live: np.ndarray | None  # uint8 [S, depth]
    hash_params: dict            # multipliers, primes, offsets, max_ngram, n_heads, pad_id
    layers: list = field(default_factory=list)
    h: np.ndarray | None = None  # float32 [T, hc, dim]


def hash_tables() -> dict:
    """The stored hash-table metadata, keyed by config index (as a string)."""
    with open(_HASH_TABLES) as f:
        return json.load(f)


def hash_params(spec: Spec) -> dict:
    entry = hash_tables()[str(spec.index)]
    return dict(multipliers=np.array(entry["multipliers"], dtype=np.int64),
                primes=np.array(entry["primes"], dtype=np.int64),
                offsets=np.array(entry["offsets"], dtype=np.int64),
                max_ngram=int(entry["max_ngram"]), n_heads=int(entry["n_heads"]),
                pad_id=int(entry["pad_id"]))


def _rng(cfg: int, tag: int, chunk: int | None = None) -> np.random.Generator:
    seed = 1000 * cfg + tag
    return np.random.default_rng(seed if chunk is None else [seed, chunk])


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _chunked(n_rows: int, chunk_rows: int, fill, workers: int = 8) -> None:
    starts = list(range(0, n_rows, chunk_rows))
    with ThreadPoolExecutor(max_workers=min(workers, max(1, len(starts)))) as ex:
        list(ex.map(lambda i_s: fill(i_s[0], i_s[1], min(i_s[1] + chunk_rows, n_rows)),
                    enumerate(starts)))


def q2k_table(cfg: int, layer: int, num_rows: int) -> np.ndarray:
    """Q2_K blocks: random scale/min nibbles and quants; fp16 d, dmin ~ U[1e-3, 1e-2]."""
    table = np.empty((num_rows, Q2K_ROW_BYTES), dtype=np.uint8)

    def fill(ci, a, b):
        g = _rng(cfg, 10 + layer, ci)
        table[a:b, :80] = g.integers(0, 256, size=(b - a, 80), dtype=np.uint8)
        dd = g.uniform(1e-3, 1e-2, size=(b - a, 2)).astype("<f2")
        table[a:b, 80:84] = dd.view(np.uint8).reshape(b - a, 4)
    _chunked(num_rows, 1 << 18, fill)
    return table


def fp8_table(cfg: int, layer: int, num_rows: int) -> tuple[np.ndarray, np.ndarray]:
    """e4m3fn codes of clip(N(0,1), +-448) and e8m0 scale bytes ~ U{119..127}."""
    table = np.empty((num_rows, HEAD_DIM), dtype=np.uint8)
    scales = np.empty((num_rows, FP8_SCALES_PER_ROW), dtype=np.uint8)

    def fill(ci, a, b):
        g = _rng(cfg, 10 + layer, ci)
        v = np.clip(g.standard_normal(size=(b - a, HEAD_DIM), dtype=np.float32), -448, 448)
        table[a:b] = _to_e4m3_codes(v)
        scales[a:b] = g.integers(119, 128, size=(b - a, FP8_SCALES_PER_ROW), dtype=np.uint8)
    _chunked(num_rows, 1 << 17, fill)
    return table, scales


def wkv_weight(cfg: int, layer: int, n_out: int, k: int) -> np.ndarray:
    """bf16 bits of N(0, 0.02) weights [n_out, k]."""
    out = np.empty((n_out, k), dtype=np.uint16)

    def fill(ci, a, b):
        g = _rng(cfg, 20 + layer, ci)
        out[a:b] = _to_bf16_bits(g.standard_normal(size=(b - a, k), dtype=np.float32) * 0.02)
    _chunked(n_out, 1024, fill)
    return out


def norm_weights(cfg: int, layer: int, hc: int, dim: int) -> tuple[np.ndarray, np.ndarray]:
    """bf16 bits of q_weight, k_weight ~ 1 + N(0, 0.1), each [hc, dim]."""
    g = _rng(cfg, 30 + layer)
    q = _to_bf16_bits(1.0 + 0.1 * g.standard_normal(size=(hc, dim)))
    k = _to_bf16_bits(1.0 + 0.1 * g.standard_normal(size=(hc, dim)))
    return q, k


def highway(cfg: int, T: int, hc: int, dim: int) -> np.ndarray:
    """fp32 N(0, 1) highway [T, hc, dim]."""
    h = np.empty((T, hc, dim), dtype=np.float32)

    def fill(ci, a, b):
        h[a:b] = _rng(cfg, 40, ci).standard_normal(size=(b - a, hc, dim), dtype=np.float32)
    _chunked(T, 512, fill)
    return h


def token_ids(spec: Spec) -> np.ndarray:
    g = _rng(spec.index, 1)
    V = spec.compressed_vocab
    if spec.id_dist == "uniform":
        return g.integers(0, V, size=spec.T, dtype=np.int64).astype(np.int32)
    ranks = np.arange(1, V + 1, dtype=np.float64)     # truncated Zipf(1.1) over ranks
    p = ranks ** -1.1
    p /= p.sum()
    return g.choice(V, size=spec.T, p=p).astype(np.int32)


def token_mask(spec: Spec) -> np.ndarray | None:
    if not spec.mask:
        return None
    kind, n = spec.mask
    g = _rng(spec.index, 50)
    T = spec.T
    live = np.ones(T, dtype=np.uint8)
    if kind == "choice":
        live[g.choice(T, size=n, replace=False)] = 0
        return live
    masked = 0                              # 'spans': random spans until exactly n
    while masked < n:
        start = int(g.integers(0, T))
        length = int(g.integers(1, 17))
        for p in range(start, min(start + length, T)):
            if live[p]:
                live[p] = 0
                masked += 1
                if masked == n:
                    break
    return live


def make_workload(index: int, *, with_weights: bool = True, with_h: bool = True) -> Workload:
    spec = SPECS[index]
    cu = np.zeros(len(spec.seq_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(spec.seq_lens)
    doc_ids = None
    if spec.doc_len:
        doc_ids = (1 + np.arange(spec.T) // spec.doc_len).astype(np.int32)
    lookback = lookback_live = None
    if spec.lookback_depth:
        g = _rng(spec.index, 60)
        lookback = g.integers(0, spec.compressed_vocab,
                              size=(len(spec.seq_lens), spec.lookback_depth),
                              dtype=np.int64).astype(np.int32)
        lookback_live = np.ones_like(lookback, dtype=np.uint8)
    wl = Workload(spec=spec, cids=token_ids(spec), cu_seqlens=cu, doc_ids=doc_ids,
                  token_mask=token_mask(spec), lookback=lookback,
                  lookback_live=lookback_live, hash_params=hash_params(spec))
    if with_weights:
        wcfg = spec.index if spec.weight_seed_config < 0 else spec.weight_seed_config
        for l in range(len(spec.layer_ids)):
            if spec.fmt == "q2k":
                table, scales = q2k_table(wcfg, l, spec.num_rows), None
            else:
                table, scales = fp8_table(wcfg, l, spec.num_rows)
            q, k = norm_weights(wcfg, l, spec.hc, spec.dim)
            wl.layers.append(Layer(spec.fmt, table, scales,
                                   wkv_weight(wcfg, l, spec.N, spec.K), q, k))
    if with_h:
        wl.h = highway(spec.index, spec.T, spec.hc, spec.dim)
    return wl


@lru_cache(maxsize=2)
def cached_workload(index: int) -> Workload:
    """make_workload, memoised (callers must not modify the arrays in place)."""
    return make_workload(index)
