"""Pins for the lookback store of streaming decode (oracle.history_update), CPU only.

* A hand-worked store: depth 3, a chunk shorter than the depth, a masked
  token, an empty chunk, a fresh (all dead) store, a chunk longer than the
  depth.
* The defining property: hashing a sequence chunk by chunk, each chunk
  against the store the previous chunks left (starting from an all-dead
  store), gives exactly the ids of hashing the whole sequence at once --
  for random chunk splits, several sequences per batch, masked tokens, and
  every order up to max_ngram = depth + 1.  A plausible slip (an off-by-one
  in the entry position, liveness lost or kept wrongly, the old entries in
  the wrong order) breaks it.
* Documents: a chunk that ends in a new document leaves the older entries
  dead, so the next chunk equals a sequence that starts at that document.
"""

import numpy as np
import pytest

import oracle
from oracle.layout import engram_layout, hash_multipliers


def test_handworked_store():
    hist = np.array([[7, 8, 9], [1, 2, 3], [4, 5, 6]], dtype=np.int32)
    live = np.array([[1, 1, 1], [0, 1, 1], [1, 1, 1]], dtype=np.uint8)
    # sequence 0: chunk [20, 21] -> entries (9, 20, 21), 9 keeps its liveness
    # sequence 1: empty chunk -> unchanged
    # sequence 2: chunk [30, 31, 32, 33] with 31 masked -> (31 dead, 32, 33)
    cids = np.array([20, 21, 30, 31, 32, 33], dtype=np.int32)
    cu = np.array([0, 2, 2, 6], dtype=np.int32)
    mask = np.array([1, 1, 1, 0, 1, 1], dtype=np.uint8)
    h, l = oracle.history_update(hist, live, cids, cu, token_mask=mask)
    assert h.tolist() == [[9, 20, 21], [1, 2, 3], [31, 32, 33]]
    assert l.tolist() == [[1, 1, 1], [0, 1, 1], [0, 1, 1]]
    # a masked token at the end of a one-token chunk: dead entry, older ones shift
    h2, l2 = oracle.history_update(h, l, np.array([40], np.int32), np.array([0, 1, 1, 1]),
                                   token_mask=np.array([0], np.uint8))
    assert h2[0].tolist() == [20, 21, 40] and l2[0].tolist() == [1, 1, 0]
    # a fresh store has no live entry, and a chunk of one token leaves 2 dead
    fresh_h = np.zeros((1, 3), np.int32)
    fresh_l = np.zeros((1, 3), np.uint8)
    h3, l3 = oracle.history_update(fresh_h, fresh_l, np.array([5], np.int32),
                                   np.array([0, 1]))
    assert h3[0].tolist() == [0, 0, 5] and l3[0].tolist() == [0, 0, 1]


def _tables(max_ngram, n_heads, vocab, seed):
    primes, offsets = engram_layout(1, max_ngram, n_heads, 1009 + seed)
    mult = hash_multipliers([1], max_ngram, vocab)
    return mult, primes, offsets


@pytest.mark.parametrize("max_ngram", [2, 3, 4, 5])
def test_streaming_chunks_equal_prefill(max_ngram):
    rng = np.random.default_rng(max_ngram)
    n_heads, vocab, depth = 2, 50, max_ngram - 1
    mult, primes, offsets = _tables(max_ngram, n_heads, vocab, max_ngram)
    n_seqs = 4
    lens = rng.integers(1, 30, n_seqs)
    seqs = [rng.integers(0, vocab, n).astype(np.int32) for n in lens]
    masks = [(rng.random(n) > 0.15).astype(np.uint8) for n in lens]
    want = [oracle.hash_ids(s, np.array([0, len(s)]), mult, primes, offsets, max_ngram,
                            n_heads, 0, token_mask=m) for s, m in zip(seqs, masks)]
    hist = np.zeros((n_seqs, depth), np.int32)
    live = np.zeros((n_seqs, depth), np.uint8)
    pos = [0] * n_seqs
    got = [[] for _ in range(n_seqs)]
    while any(p < len(s) for p, s in zip(pos, seqs)):
        # one batch: every sequence advances by a random chunk (possibly empty)
        take = [min(int(rng.integers(0, 5)), len(s) - p) for p, s in zip(pos, seqs)]
        cu = np.concatenate([[0], np.cumsum(take)]).astype(np.int32)
        cids = np.concatenate([s[p:p + k] for s, p, k in zip(seqs, pos, take)]).astype(np.int32)
        mask = np.concatenate([m[p:p + k] for m, p, k in zip(masks, pos, take)]).astype(np.uint8)
        ids = oracle.hash_ids(cids, cu, mult, primes, offsets, max_ngram, n_heads, 0,
                              token_mask=mask, lookback=hist, lookback_live=live)
        for i in range(n_seqs):
            got[i].append(ids[cu[i]:cu[i + 1]])
        hist, live = oracle.history_update(hist, live, cids, cu, token_mask=mask)
        pos = [p + k for p, k in zip(pos, take)]
    for i in range(n_seqs):
        assert np.array_equal(np.concatenate(got[i]), want[i]), i


def test_new_document_kills_older_entries():
    rng = np.random.default_rng(3)
    max_ngram, n_heads, vocab = 4, 2, 40
    mult, primes, offsets = _tables(max_ngram, n_heads, vocab, 3)
    a = rng.integers(0, vocab, 6).astype(np.int32)
    b = rng.integers(0, vocab, 2).astype(np.int32)      # new document, shorter than depth
    c = rng.integers(0, vocab, 4).astype(np.int32)      # continues document b
    hist = np.zeros((1, 3), np.int32)
    live = np.zeros((1, 3), np.uint8)
    hist, live = oracle.history_update(hist, live, a, np.array([0, 6]),
                                       doc_ids=np.ones(6, np.int32))
    ab = np.concatenate([a[-1:], b])
    doc = np.array([1, 2, 2], np.int32)
    hist, live = oracle.history_update(hist, live, ab, np.array([0, 3]), doc_ids=doc)
    assert live[0].tolist() == [0, 1, 1] and hist[0, 1:].tolist() == b.tolist()
    got = oracle.hash_ids(c, np.array([0, 4]), mult, primes, offsets, max_ngram, n_heads, 0,
                          lookback=hist, lookback_live=live)
    bc = np.concatenate([b, c])
    want = oracle.hash_ids(bc, np.array([0, 6]), mult, primes, offsets, max_ngram, n_heads, 0)
    assert np.array_equal(got, want[2:])
    # a padding document at the end leaves every entry dead
    h2, l2 = oracle.history_update(hist, live, np.array([9, 9], np.int32), np.array([0, 2]),
                                   doc_ids=np.array([0, 0], np.int32))
    assert not l2.any()
