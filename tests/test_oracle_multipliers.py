"""Pins of the oracle's hash multipliers and of ids hashed with them.

The multiplier rule ([vLLM] "vllm.models.deepseek_v41.common.engram",
compute_hash_multipliers) draws from numpy's default generator.  Two pins
hold the oracle's use of that rule to something other than itself:

* literal multipliers and ids computed from the rule while the pages were
  surveyed (tests/golden/hash_worked_real_multipliers.json);
* a from-scratch restatement of the generator's published definition
  (SeedSequence entropy mixing, the PCG64 XSL-RR generator, Lemire's
  nearly-divisionless bounded integers), checked here against numpy and then
  used to recompute the multipliers for other layers and vocabularies.

A slip in the oracle -- another seed (layer_id instead of 10007 * layer_id),
another range ([1, bound) or the full bound), another odd mapping, or
another draw order -- fails both.
"""

import json
import os

import numpy as np
import pytest

import oracle

M32 = 0xFFFFFFFF
M64 = (1 << 64) - 1
M128 = (1 << 128) - 1


# ----------------------------------------------------------------- SeedSequence
# numpy's SeedSequence (NEP 19): the seed's 32-bit words are hashed into a
# pool of four words, every pool word is mixed with every other, and output
# words are hashed out of the pool in a cycle.

_INIT_A, _MULT_A = 0x43B0D7E5, 0x931E8875
_INIT_B, _MULT_B = 0x8B51F9DD, 0x58F38DED
_MIX_L, _MIX_R = 0xCA01F9DD, 0x4973F715
_POOL = 4


def _hashmix(value, const):
    value = (value ^ const[0]) & M32
    const[0] = (const[0] * _MULT_A) & M32
    value = (value * const[0]) & M32
    return value ^ (value >> 16)


def _mix(x, y):
    r = (_MIX_L * x - _MIX_R * y) & M32
    return r ^ (r >> 16)


def _seed_words(seed):
    words = []
    while True:
        words.append(seed & M32)
        seed >>= 32
        if seed == 0:
            return words


def _seed_pool(seed):
    entropy = _seed_words(seed)
    const = [_INIT_A]
    pool = [_hashmix(entropy[i] if i < len(entropy) else 0, const) for i in range(_POOL)]
    for src in range(_POOL):
        for dst in range(_POOL):
            if src != dst:
                pool[dst] = _mix(pool[dst], _hashmix(pool[src], const))
    for src in range(_POOL, len(entropy)):
        for dst in range(_POOL):
            pool[dst] = _mix(pool[dst], _hashmix(entropy[src], const))
    return pool


def _generate_u64(pool, n):
    const = _INIT_B
    words = []
    for i in range(2 * n):
        v = pool[i % _POOL] ^ const
        const = (const * _MULT_B) & M32
        v = (v * const) & M32
        words.append(v ^ (v >> 16))
    return [words[2 * i] | (words[2 * i + 1] << 32) for i in range(n)]   # little-endian pairs


# ----------------------------------------------------------------------- PCG64
# O'Neill's PCG: a 128-bit LCG, output = rotate-right of (high ^ low) by the
# top 6 bits of the state ("XSL-RR"); the generator steps, then outputs.

_PCG_MULT = (2549297995355413924 << 64) | 4865540595714422341


class _Pcg64:
    def __init__(self, seed):
        s = _generate_u64(_seed_pool(seed), 4)
        init_state = (s[0] << 64) | s[1]
        init_seq = (s[2] << 64) | s[3]
        self.inc = ((init_seq << 1) | 1) & M128
        self.state = 0
        self._step()
        self.state = (self.state + init_state) & M128
        self._step()

    def _step(self):
        self.state = (self.state * _PCG_MULT + self.inc) & M128

    def next_u64(self):
        self._step()
        x = ((self.state >> 64) ^ self.state) & M64
        rot = self.state >> 122
        return ((x >> rot) | (x << ((64 - rot) & 63))) & M64


def _bounded(gen, bound):
    """Uniform integer in [0, bound): Lemire's multiply-shift with rejection.

    This is the path numpy takes for 64-bit ranges wider than 2**32 - 1.
    """
    assert bound - 1 > M32
    m = gen.next_u64() * bound
    low = m & M64
    if low < bound:
        threshold = (-bound) % bound            # 2**64 mod bound
        while low < threshold:
            m = gen.next_u64() * bound
            low = m & M64
    return m >> 64


def _multipliers_from_definition(layer_id, max_ngram, vocab):
    bound = max(1, ((2**63 - 1) // vocab) // 2)
    gen = _Pcg64(10007 * layer_id)
    return [2 * _bounded(gen, bound) + 1 for _ in range(max_ngram)]


# ----------------------------------------------------------------------- tests

@pytest.fixture(scope="module")
def worked(golden_dir):
    with open(os.path.join(golden_dir, "hash_worked_real_multipliers.json")) as f:
        return json.load(f)


def test_generator_restatement_matches_numpy():
    # The restatement above is a second implementation of numpy's stream, not
    # the oracle's: check it draw for draw before it is used as a pin.
    for seed in (0, 1, 10007, 140098, 2**32 + 5, 2**70 + 3):
        ref = np.random.default_rng(seed)
        mine = _Pcg64(seed)
        for bound in (2**40 + 7, 2**62 - 1, 35184372088831):
            want = ref.integers(0, bound, size=6, dtype=np.int64).tolist()
            assert [_bounded(mine, bound) for _ in range(6)] == want, (seed, bound)


def test_literal_multipliers(worked):
    for case in worked["multipliers"]:
        got = oracle.hash_multipliers((case["layer_id"],), case["max_ngram"], case["vocab"])
        assert got.tolist() == [case["values"]], case
        assert _multipliers_from_definition(case["layer_id"], case["max_ngram"],
                                            case["vocab"]) == case["values"]


@pytest.mark.parametrize("vocab", [1000, 131072, 129280, 2**20])
def test_multipliers_against_the_restated_rule(vocab):
    layer_ids = (0, 1, 2, 14, 30, 61)
    got = oracle.hash_multipliers(layer_ids, 4, vocab)
    for row, layer_id in zip(got.tolist(), layer_ids):
        assert row == _multipliers_from_definition(layer_id, 4, vocab), (layer_id, vocab)
    # max_ngram changes how many are drawn, not the stream: a prefix.
    longer = oracle.hash_multipliers((14,), 6, vocab)
    assert longer[0, :4].tolist() == got[3].tolist()


def test_worked_ids_with_real_multipliers(worked):
    c = worked["tiny_sequence"]
    primes, offsets = oracle.engram_layout(1, c["max_ngram"], c["n_heads"],
                                           c["engram_vocab_size"])
    mult = np.array([_multipliers_from_definition(c["layer_id"], c["max_ngram"], c["vocab"])])
    cids = np.array(c["cids"], dtype=np.int32)
    cu = np.array([0, len(cids)], dtype=np.int32)
    ids = oracle.hash_ids(cids, cu, mult, primes, offsets, c["max_ngram"], c["n_heads"],
                          c["pad_id"])
    assert ids[:, 0, :].tolist() == c["ids"]
    m = c["masked"]
    ids_m = oracle.hash_ids(cids, cu, mult, primes, offsets, c["max_ngram"], c["n_heads"],
                            c["pad_id"], token_mask=np.array(m["token_mask"], dtype=np.uint8))
    assert ids_m[m["t"], 0, :].tolist() == m["ids_t"]
    # order 2 (columns 0, 1) sees only distance 1, which is live: unchanged
    assert ids_m[m["t"], 0, :2].tolist() == c["ids"][m["t"]][:2]
