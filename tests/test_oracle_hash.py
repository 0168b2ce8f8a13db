"""Pins of the oracle's n-gram hash: hand-worked ids and invariants the pages fix."""

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import workloads


def _load(golden_dir):
    with open(os.path.join(golden_dir, "hash_handworked.json")) as f:
        return json.load(f)


def _arr(case, key, dtype):
    return None if key not in case else np.array(case[key], dtype=dtype)


def test_handworked_cases(golden_dir):
    g = _load(golden_dir)
    p = g["params"]
    for case in g["cases"]:
        ids = oracle.hash_ids(np.array(case["cids"]), np.array(case["cu_seqlens"]),
                              np.array(p["multipliers"]), np.array(p["primes"]),
                              np.array(p["offsets"]), p["max_ngram"], p["n_heads"],
                              case["pad_id"], doc_ids=_arr(case, "doc_ids", np.int32),
                              token_mask=_arr(case, "token_mask", np.uint8),
                              lookback=_arr(case, "lookback", np.int32),
                              lookback_live=_arr(case, "lookback_live", np.uint8))
        assert ids[:, 0, :].tolist() == case["ids"], case["name"]


def test_handworked_two_layers(golden_dir):
    g = _load(golden_dir)["two_layer"]
    p = g["params"]
    ids = oracle.hash_ids(np.array(g["cids"]), np.array(g["cu_seqlens"]),
                          np.array(p["multipliers"]), np.array(p["primes"]),
                          np.array(p["offsets"]), p["max_ngram"], p["n_heads"], g["pad_id"])
    assert ids.shape == (3, 2, 4)
    assert ids[2, 1].tolist() == g["ids_t2_layer1"]


def _tiny_params():
    hp = workloads.hash_params(workloads.SPECS[0])
    return hp


def _hash(cids, cu, hp, **kw):
    return oracle.hash_ids(np.asarray(cids), np.asarray(cu), hp["multipliers"], hp["primes"],
                           hp["offsets"], hp["max_ngram"], hp["n_heads"], hp["pad_id"], **kw)


def test_ids_stay_in_their_bucket_on_every_workload():
    # EngramLayout: each (order, head) column owns [offset, offset + prime).
    for spec in workloads.SPECS[:4]:
        wl = workloads.make_workload(spec.index, with_weights=False, with_h=False)
        hp = wl.hash_params
        ids = _hash(wl.cids, wl.cu_seqlens, hp, doc_ids=wl.doc_ids, token_mask=wl.token_mask,
                    lookback=wl.lookback, lookback_live=wl.lookback_live)
        assert ids.shape == (spec.T, len(spec.layer_ids), spec.cols)
        lo = hp["offsets"][None]
        hi = lo + hp["primes"][None]
        assert ((ids >= lo) & (ids < hi)).all(), spec.name


def test_decode_with_lookback_equals_prefill():
    # Reading A8: hashing a chunk with the ids just before it supplied as
    # lookback gives the ids that hashing the whole sequence gives.
    hp = _tiny_params()
    rng = np.random.default_rng(5)
    seq = rng.integers(0, 1000, 40).astype(np.int32)
    full = _hash(seq, [0, 40], hp)
    depth = hp["max_ngram"] - 1
    for split in (1, 2, 3, 17, 39):
        lb = np.zeros((1, depth), dtype=np.int32)
        live = np.zeros((1, depth), dtype=np.uint8)
        have = seq[max(0, split - depth):split]
        lb[0, depth - len(have):] = have
        live[0, depth - len(have):] = 1
        tail = _hash(seq[split:], [0, 40 - split], hp, lookback=lb, lookback_live=live)
        np.testing.assert_array_equal(tail, full[split:])
    # token-by-token decode (64 one-token sequences, as the decode workload)
    lbs = np.zeros((40, depth), dtype=np.int32)
    lives = np.zeros((40, depth), dtype=np.uint8)
    for t in range(40):
        have = seq[max(0, t - depth):t]
        lbs[t, depth - len(have):] = have
        lives[t, depth - len(have):] = 1
    step = _hash(seq, np.arange(41), hp, lookback=lbs, lookback_live=lives)
    np.testing.assert_array_equal(step, full)


def test_mask_blocks_like_a_sequence_start():
    # NeMo hash: a False token_mask blocks all lookback through that position,
    # so position t with a mask at t-j hashes like the suffix t-j+1..t alone.
    hp = _tiny_params()
    rng = np.random.default_rng(6)
    seq = rng.integers(0, 1000, 30).astype(np.int32)
    for j in (1, 2, 3):
        t = 20
        mask = np.ones(30, dtype=np.uint8)
        mask[t - j] = 0
        got = _hash(seq, [0, 30], hp, token_mask=mask)[t]
        alone = _hash(seq[t - j + 1:t + 1], [0, j], hp)[-1]
        np.testing.assert_array_equal(got, alone)
        # positions before the mask are unaffected
        np.testing.assert_array_equal(_hash(seq, [0, 30], hp, token_mask=mask)[:t - j],
                                      _hash(seq, [0, 30], hp)[:t - j])


def test_document_boundary_blocks_like_a_sequence_start():
    hp = _tiny_params()
    rng = np.random.default_rng(7)
    seq = rng.integers(0, 1000, 24).astype(np.int32)
    docs = np.array([1] * 10 + [2] * 14, dtype=np.int32)
    got = _hash(seq, [0, 24], hp, doc_ids=docs)
    np.testing.assert_array_equal(got[:10], _hash(seq[:10], [0, 10], hp))
    np.testing.assert_array_equal(got[10:], _hash(seq[10:], [0, 14], hp))


def test_order_n_depends_only_on_last_n_tokens():
    hp = _tiny_params()
    rng = np.random.default_rng(8)
    seq = rng.integers(0, 1000, 12).astype(np.int32)
    base = _hash(seq, [0, 12], hp)
    H = hp["n_heads"]
    t = 10
    for dist in (1, 2, 3):
        other = seq.copy()
        other[t - dist] = (other[t - dist] + 1) % 1000
        changed = _hash(other, [0, 12], hp)
        for n in range(2, hp["max_ngram"] + 1):
            cols = slice((n - 2) * H, (n - 1) * H)
            if n <= dist:   # order n reads distances < n only
                np.testing.assert_array_equal(changed[t, :, cols], base[t, :, cols])


def test_first_position_reduces_to_single_product():
    # With no history every tok_k (k >= 1) is pad_id = 0, so every order's mix
    # is just token * m[0] and id = offset + (token * m[0]) mod prime.
    hp = _tiny_params()
    for tok in (0, 1, 999):
        ids = _hash(np.array([tok], dtype=np.int32), [0, 1], hp)[0, 0]
        m0 = int(hp["multipliers"][0, 0])
        want = [int(o) + (tok * m0) % int(p) for o, p in zip(hp["offsets"][0], hp["primes"][0])]
        assert ids.tolist() == want


@settings(max_examples=60, deadline=None)
@given(st.lists(st.integers(0, 999), min_size=1, max_size=12),
       st.lists(st.booleans(), min_size=12, max_size=12))
def test_hypothesis_range_and_mask_locality(toks, mask_bits):
    hp = _tiny_params()
    T = len(toks)
    mask = np.array(mask_bits[:T], dtype=np.uint8)
    ids = _hash(np.array(toks, dtype=np.int32), [0, T], hp, token_mask=mask)
    lo = hp["offsets"][None]
    assert ((ids >= lo) & (ids < lo + hp["primes"][None])).all()
    # a position's own mask bit never changes its own ids (reading A6)
    mask2 = mask.copy()
    mask2[-1] ^= 1
    ids2 = _hash(np.array(toks, dtype=np.int32), [0, T], hp, token_mask=mask2)
    np.testing.assert_array_equal(ids[-1], ids2[-1])


def test_empty_input():
    hp = _tiny_params()
    ids = _hash(np.zeros(0, dtype=np.int32), [0], hp)
    assert ids.shape == (0, 1, 6)
