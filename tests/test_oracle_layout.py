"""Pins of the hash-table layout: primes, offsets, multipliers, stored metadata."""

import json
import os

import numpy as np
import sympy

import oracle
from workloads import SPECS


def test_is_prime_matches_sympy():
    for n in list(range(0, 5000)) + list(range(174000, 174400)) + list(range(698000, 698200)):
        assert oracle.is_prime(n) == sympy.isprime(n), n


def test_layout_rule_against_sympy_nextprime():
    # EngramLayout: per layer and order, restart at engram_vocab_size - 1 and
    # take the next prime not handed out before (anywhere in the model).
    n_layers, max_ngram, n_heads, start = 2, 4, 3, 500
    primes, offsets = oracle.engram_layout(n_layers, max_ngram, n_heads, start)
    seen = set()
    expect = []
    for _ in range(n_layers):
        row = []
        for _ in range(max_ngram - 1):
            cur = start - 1
            for _ in range(n_heads):
                cur = sympy.nextprime(cur)
                while cur in seen:
                    cur = sympy.nextprime(cur)
                seen.add(cur)
                row.append(cur)
        expect.append(row)
    np.testing.assert_array_equal(primes, np.array(expect))
    # offsets: exclusive prefix sums within each layer
    for l in range(n_layers):
        assert offsets[l, 0] == 0
        np.testing.assert_array_equal(offsets[l, 1:], np.cumsum(primes[l])[:-1])
    # all primes distinct across the model, so bucket ranges never share a size
    assert len(set(primes.ravel().tolist())) == primes.size


def test_layout_of_every_workload_fits_its_table():
    # ParallelEngramEmbedding requires the head sizes to sum to at most the table rows.
    for spec in SPECS:
        primes, offsets = oracle.engram_layout(len(spec.layer_ids), spec.max_ngram,
                                               spec.n_heads, spec.engram_vocab_size)
        assert all(sympy.isprime(int(p)) for p in primes.ravel())
        assert (primes.sum(axis=1) <= spec.num_rows).all(), spec.name
        assert (offsets + primes <= np.iinfo(np.int32).max).all()


def test_tiny_layout_reading_a9():
    primes, offsets = oracle.engram_layout(1, 4, 2, 2713)
    assert primes.tolist() == [[2713, 2719, 2729, 2731, 2741, 2749]]
    assert offsets.tolist() == [[0, 2713, 5432, 8161, 10892, 13633]]
    assert primes.sum() == 16382 <= 16384


def test_multiplier_properties():
    # compute_hash_multipliers: odd, and bounded so token * multiplier < 2^63
    # for every token below the compressed vocab size; layers hash differently.
    for vocab in (1000, 131072, 2**20):
        m = oracle.hash_multipliers((1, 14, 30), 4, vocab)
        assert m.shape == (3, 4) and m.dtype == np.int64
        assert (m % 2 == 1).all()
        bound = max(1, ((2**63 - 1) // vocab) // 2)
        assert all(1 <= int(v) <= 2 * bound - 1 for v in m.ravel())
        assert all(int(v) * (vocab - 1) < 2**63 for v in m.ravel())
        assert len({tuple(r) for r in m.tolist()}) == 3
    # deterministic per layer id, independent of which other layers are listed
    a = oracle.hash_multipliers((14,), 4, 131072)
    b = oracle.hash_multipliers((1, 14), 4, 131072)
    np.testing.assert_array_equal(a[0], b[1])


def test_stored_hash_tables_match_the_oracle(golden_dir):
    with open(os.path.join(golden_dir, "hash_tables.json")) as f:
        stored = json.load(f)
    for spec in SPECS:
        e = stored[str(spec.index)]
        primes, offsets = oracle.engram_layout(len(spec.layer_ids), spec.max_ngram,
                                               spec.n_heads, spec.engram_vocab_size)
        mult = oracle.hash_multipliers(spec.layer_ids, spec.max_ngram, spec.compressed_vocab)
        assert e["primes"] == primes.tolist()
        assert e["offsets"] == offsets.tolist()
        assert e["multipliers"] == mult.tolist()
        assert e["max_ngram"] == spec.max_ngram and e["n_heads"] == spec.n_heads
