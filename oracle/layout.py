"""Hash-table layout of the Engram n-gram hash (oracle side; test infrastructure).

The primes, offsets and multipliers are fixed per model; the spark page says
they ship as checkpoint metadata.  The vLLM page derives them as follows,
and this module restates those rules from their definitions:

* [vLLM engram page, EngramLayout] -- a position hashes as max_ngram - 1
  n-grams (orders 2..max_ngram), each split over n_heads heads; every
  (order, head) pair owns a prime-sized bucket range of the layer's table.
  Primes are handed out in order, never twice in the whole model, and the
  search restarts from engram_vocab_size - 1 for every order of every layer.
  The flat column order is order-major, head-minor, and each column's
  offset is the exclusive prefix sum of the column sizes before it.
* [vLLM engram page, find_next_prime] -- the next prime is the smallest
  prime strictly above the start that has not been handed out.
* [vLLM engram page, compute_hash_multipliers] -- one multiplier per
  (layer, lookback distance): numpy's default generator seeded with
  10007 * layer_id draws max_ngram int64 values uniformly from
  [0, max(1, (int64_max // vocab) // 2)), and each value r becomes 2r + 1,
  so it is odd and token * multiplier stays below 2**63 for tokens < vocab.
"""

from __future__ import annotations

import numpy as np

INT64_MAX = (1 << 63) - 1


def is_prime(n: int) -> bool:
    """Primality by trial division: the definition, nothing cleverer.

    The vLLM page uses a deterministic Miller-Rabin test valid below 2**32;
    for the sizes here (< 2**25) trial division is fast and plainly correct,
    and both give the same answer for every n < 2**32.
    """
    n = int(n)
    if n < 2:
        return False
    if n % 2 == 0:
        return n == 2
    d = 3
    while d * d <= n:
        if n % d == 0:
            return False
        d += 2
    return True


def next_unused_prime(start: int, seen: set[int]) -> int:
    """Smallest prime > start that is not in `seen` [vLLM engram page, find_next_prime]."""
    cand = int(start) + 1
    while cand in seen or not is_prime(cand):
        cand += 1
    return cand


def engram_layout(n_layers: int, max_ngram: int, n_heads: int,
                  engram_vocab_size: int) -> tuple[np.ndarray, np.ndarray]:
    """Per-layer bucket primes and offsets [vLLM engram page, EngramLayout].

    Returns (primes, offsets), both int64 of shape [n_layers, (max_ngram-1)*n_heads].
    Column c = (n - 2) * n_heads + j holds order n, head j.
    """
    if max_ngram < 2 or n_heads < 1 or n_layers < 1:
        raise ValueError("need max_ngram >= 2, n_heads >= 1, n_layers >= 1")
    seen: set[int] = set()
    primes = []
    for _layer in range(n_layers):
        layer_primes = []
        for _order in range(2, max_ngram + 1):
            cur = engram_vocab_size - 1          # restart per order
            for _head in range(n_heads):
                cur = next_unused_prime(cur, seen)
                seen.add(cur)
                layer_primes.append(cur)
        primes.append(layer_primes)
    primes = np.array(primes, dtype=np.int64)
    offsets = np.zeros_like(primes)
    for layer in range(n_layers):
        run = 0
        for c in range(primes.shape[1]):
            offsets[layer, c] = run
            run += int(primes[layer, c])
    return primes, offsets


def hash_multipliers(layer_ids, max_ngram: int, compressed_vocab: int) -> np.ndarray:
    """Odd per-(layer, distance) multipliers [vLLM engram page, compute_hash_multipliers].

    Returns int64 [len(layer_ids), max_ngram]; entry [l, k] multiplies the
    token k positions back (k = 0 is the current token).
    """
    bound = max(1, (INT64_MAX // int(compressed_vocab)) // 2)
    rows = []
    for layer_id in layer_ids:
        gen = np.random.default_rng(10007 * int(layer_id))
        draw = gen.integers(0, bound, size=(max_ngram,), dtype=np.int64)
        rows.append([2 * int(r) + 1 for r in draw])
    return np.array(rows, dtype=np.int64)
