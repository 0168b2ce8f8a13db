"""Pins of the oracle's projection and gate."""

from fractions import Fraction

import numpy as np
import pytest

import oracle


def _bits(x):
    return oracle.bf16_bits(oracle.bf16_round(np.asarray(x, dtype=np.float64)))


# --------------------------------------------------------------------- projection

def test_projection_equals_exactly_rounded_sum():
    # Brute force with exact rationals: bf16 values are dyadic, so the exact
    # dot product is a Fraction; rounding it to bf16 must give the oracle's
    # answer (a tie after a float64 sum is possible in principle but not here).
    rng = np.random.default_rng(0)
    T, K, N = 5, 48, 7
    a = _bits(rng.standard_normal((T, K)))
    b = _bits(0.02 * rng.standard_normal((N, K)))
    kv = oracle.bf16_value(oracle.project(a, b))
    av, bv = oracle.bf16_value(a), oracle.bf16_value(b)
    for t in range(T):
        for o in range(N):
            exact = sum(Fraction(float(x)) * Fraction(float(y)) for x, y in zip(av[t], bv[o]))
            want = oracle.bf16_round([float(exact)])[0]
            assert kv[t, o] == want


def test_projection_shapes_and_identity():
    # wkv = identity block picks columns out of rows: [T, K] x [N, K]^T -> [T, N].
    K = 16
    rng = np.random.default_rng(1)
    rows = _bits(rng.standard_normal((3, K)))
    eye = _bits(np.eye(K)[:5])
    kv = oracle.project(rows, eye)
    np.testing.assert_array_equal(kv, rows[:, :5])


# --------------------------------------------------------------------------- gate

def _gate_inputs(T=6, hc=3, dim=64, seed=0):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((T, hc, dim)).astype(np.float32)
    kv = _bits(0.125 * rng.standard_normal((T, (hc + 1) * dim)))
    qw = _bits(1 + 0.1 * rng.standard_normal((hc, dim)))
    kw = _bits(1 + 0.1 * rng.standard_normal((hc, dim)))
    return h, kv, qw, kw


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


@pytest.mark.parametrize("dim", [128, 4096])
@pytest.mark.parametrize("c", [0.5, -2.0])
def test_gate_closed_form_key_parallel_to_stream(dim, c):
    # Reading A14 special case: key = c * x with unit norm weights and eps = 0
    # makes the normalised dot sign(c) * dim, so with dot scale 1/sqrt(dim)
    # a = sign(c) * sqrt(dim), z = sign(c) * dim**(1/4) and g = sigmoid(z).
    # A unit value then shows g directly as h_new - x.
    rng = np.random.default_rng(2)
    T, hc = 3, 2
    x = oracle.bf16_round(rng.standard_normal((T, hc, dim)))   # key must be exact bf16
    key = c * x
    kv = np.concatenate([key.reshape(T, hc * dim), np.ones((T, dim))], axis=1)
    ones = _bits(np.ones((hc, dim)))
    h = x.astype(np.float32)
    new = oracle.gate(h, _bits(kv), ones, ones, None, 0.0, 1e-6, 1 / np.sqrt(dim))
    g = new.astype(np.float64) - x
    want = _sigmoid(np.sign(c) * dim ** 0.25)
    np.testing.assert_allclose(g, want, atol=4e-6)
    if dim == 128:   # values recorded in the design notes (A14)
        assert abs(want - (0.966547 if c > 0 else 0.033453)) < 1e-6


def test_gate_value_zero_is_identity_bitwise():
    h, kv, qw, kw = _gate_inputs()
    T, hc, dim = h.shape
    kv = kv.copy()
    kv[:, hc * dim:] = 0
    new = oracle.gate(h, kv, qw, kw, None, 1e-6, 1e-6, 1 / np.sqrt(dim))
    np.testing.assert_array_equal(new.view(np.uint32), h.view(np.uint32))


def test_gate_masked_tokens_unchanged_bitwise():
    h, kv, qw, kw = _gate_inputs()
    mask = np.array([1, 0, 1, 0, 0, 1], dtype=np.uint8)
    new = oracle.gate(h, kv, qw, kw, mask, 1e-6, 1e-6, 1 / 8)
    np.testing.assert_array_equal(new[mask == 0].view(np.uint32), h[mask == 0].view(np.uint32))
    assert (new[mask == 1] != h[mask == 1]).any()


def test_gate_in_open_unit_interval_and_odd_in_key():
    # g in (0, 1); z is odd in the key, so g(key) + g(-key) = 1.
    h, kv, qw, kw = _gate_inputs(T=16, seed=3)
    T, hc, dim = h.shape
    v = kv.copy()
    v[:, hc * dim:] = _bits(np.ones((T, dim)))
    neg = v.copy()
    neg[:, :hc * dim] ^= np.uint16(0x8000)            # flip key signs
    g1 = oracle.gate(h, v, qw, kw, None, 1e-6, 1e-6, 1 / 8).astype(np.float64) - h
    g2 = oracle.gate(h, neg, qw, kw, None, 1e-6, 1e-6, 1 / 8).astype(np.float64) - h
    assert (g1 > 0).all() and (g1 < 1).all()
    np.testing.assert_allclose(g1 + g2, 1.0, atol=1e-6)


def test_gate_norm_scaling_laws():
    # With eps = 0: scaling the stream or the key leaves a unchanged (RMS norm);
    # scaling q_weight by 4 scales a by 4 and so z by 2 (signed square root).
    h, kv, qw, kw = _gate_inputs(T=8, seed=4)
    T, hc, dim = h.shape
    kv1 = kv.copy()
    kv1[:, hc * dim:] = _bits(np.ones((T, dim)))

    def z_of(hh, kvv, qq, kk):
        g = oracle.gate(hh, kvv, qq, kk, None, 0.0, 1e-12, 1 / np.sqrt(dim)).astype(np.float64) - hh
        g = g.mean(axis=-1)
        return np.log(g / (1 - g))

    z0 = z_of(h, kv1, qw, kw)
    np.testing.assert_allclose(z_of(h * 4, kv1, qw, kw), z0, atol=1e-4)
    kv2 = kv1.copy()
    kv2[:, :hc * dim] = _bits(oracle.bf16_value(kv1[:, :hc * dim]) * 2)
    np.testing.assert_allclose(z_of(h, kv2, qw, kw), z0, atol=1e-4)
    qw4 = _bits(oracle.bf16_value(qw) * 4)
    np.testing.assert_allclose(z_of(h, kv1, qw4, kw), 2 * z0, atol=2e-4)
    kw4 = _bits(oracle.bf16_value(kw) * 4)
    np.testing.assert_allclose(z_of(h, kv1, qw, kw4), 2 * z0, atol=2e-4)


def test_gate_zero_dot_gives_half_and_clamp_floor():
    # a = 0 (zero key) -> z = 0 -> g = 1/2.  A tiny |a| is lifted to the clamp
    # before the square root: |z| = sqrt(clamp).
    T, hc, dim = 2, 1, 64
    h = np.ones((T, hc, dim), dtype=np.float32)
    kv = np.zeros((T, 2 * dim))
    kv[:, dim:] = 1.0
    ones = _bits(np.ones((hc, dim)))
    new = oracle.gate(h, _bits(kv), ones, ones, None, 1e-6, 1e-6, 1 / 8)
    np.testing.assert_allclose(new - 1.0, 0.5, atol=1e-7)
    kv[:, :dim] = 2.0 ** -40                 # a tiny positive dot
    new = oracle.gate(h, _bits(kv), ones, ones, None, 1.0, 0.25, 1 / 8)
    np.testing.assert_allclose(new - 1.0, _sigmoid(0.5), atol=1e-6)


def test_forward_composes_the_stages():
    import workloads
    wl = workloads.make_workload(0)
    s = wl.spec
    h, ids, inter = oracle.forward(wl.h, wl.cids, wl.cu_seqlens, wl.hash_params,
                                   [l.as_dict() for l in wl.layers], s.eps, s.clamp,
                                   s.dot_scale, return_intermediates=True)
    assert h.shape == (s.T, s.hc, s.dim) and h.dtype == np.float32
    rows = oracle.rows_q2k(wl.layers[0].table, ids[:, 0])
    np.testing.assert_array_equal(inter[0]["rows"], rows)
    kv = oracle.project(rows, wl.layers[0].wkv)
    np.testing.assert_array_equal(inter[0]["kv"], kv)
    np.testing.assert_array_equal(
        h, oracle.gate(wl.h, kv, wl.layers[0].q_weight, wl.layers[0].k_weight, None,
                       s.eps, s.clamp, s.dot_scale))
    assert np.abs(h - wl.h).max() > 0


# ------------------------------------------------------------ forward, two layers

def _two_layer_case():
    """Two tiny Q2_K layers with the real layout and multipliers of layer ids 1 and 14.

    Primes are unique across the model ([vLLM] EngramLayout), so layer 14's
    buckets differ from layer 1's and its ids differ too.
    """
    import workloads
    max_ngram, n_heads, vocab, start = 4, 2, 1000, 2713
    T, hc, dim = 48, 2, 128
    cols = (max_ngram - 1) * n_heads
    primes, offsets = oracle.engram_layout(2, max_ngram, n_heads, start)
    mult = oracle.hash_multipliers((1, 14), max_ngram, vocab)
    num_rows = int(primes.sum(axis=1).max()) + 7
    rng = np.random.default_rng(7)
    cids = rng.integers(0, vocab, size=T).astype(np.int32)
    cu = np.array([0, 20, T], dtype=np.int32)
    mask = np.ones(T, dtype=np.uint8)
    mask[[3, 4, 30]] = 0
    layers = []
    for l in range(2):
        q, k = workloads.norm_weights(900, l, hc, dim)
        layers.append(dict(fmt="q2k", table=workloads.q2k_table(900, l, num_rows), scales=None,
                           wkv=workloads.wkv_weight(900, l, (hc + 1) * dim, cols * 256),
                           q_weight=q, k_weight=k))
    h = workloads.highway(900, T, hc, dim)

    def params(sel):
        return dict(multipliers=mult[sel], primes=primes[sel], offsets=offsets[sel],
                    max_ngram=max_ngram, n_heads=n_heads, pad_id=0)
    return h, cids, cu, mask, layers, params, hc, dim


def _zero_value(layer, hc, dim):
    out = dict(layer)
    wkv = layer["wkv"].copy()
    wkv[hc * dim:] = 0                       # value rows of the projection -> value = 0
    out["wkv"] = wkv
    return out


def test_forward_two_layers_against_single_layers():
    # With the value gate-identity pinned above (value 0 leaves h bit for bit),
    # zeroing one layer's value must leave exactly the other layer's single-
    # layer forward: this pins that layer l hashes with layer l's multipliers
    # and buckets (ids[:, l]), gathers from layer l's table and gates with
    # layer l's weights, in order.
    h, cids, cu, mask, layers, params, hc, dim = _two_layer_case()
    args = (1e-6, 1e-6, 1 / np.sqrt(dim))
    both, ids, _ = oracle.forward(h, cids, cu, params([0, 1]), layers, *args, token_mask=mask,
                                  return_intermediates=True)
    assert (ids[:, 0] != ids[:, 1]).any(axis=1).all()
    only1 = oracle.forward(h, cids, cu, params([0]), layers[:1], *args, token_mask=mask)
    only2 = oracle.forward(h, cids, cu, params([1]), layers[1:], *args, token_mask=mask)
    first_only = oracle.forward(h, cids, cu, params([0, 1]),
                                [layers[0], _zero_value(layers[1], hc, dim)], *args,
                                token_mask=mask)
    second_only = oracle.forward(h, cids, cu, params([0, 1]),
                                 [_zero_value(layers[0], hc, dim), layers[1]], *args,
                                 token_mask=mask)
    np.testing.assert_array_equal(first_only.view(np.uint32), only1.view(np.uint32))
    np.testing.assert_array_equal(second_only.view(np.uint32), only2.view(np.uint32))
    # the layers really differ, and both act in the full forward
    assert np.abs(only1 - only2).max() > 1e-3
    assert np.abs(both - only1).max() > 1e-3 and np.abs(both - only2).max() > 1e-3


def test_forward_two_layers_apply_in_order():
    # Layer 2's gate reads the highway layer 1 left (reading A18): the full
    # forward equals layer 2's single-layer forward started from layer 1's
    # output; the other order gives a different highway.
    h, cids, cu, mask, layers, params, hc, dim = _two_layer_case()
    args = (1e-6, 1e-6, 1 / np.sqrt(dim))
    both = oracle.forward(h, cids, cu, params([0, 1]), layers, *args, token_mask=mask)
    after1 = oracle.forward(h, cids, cu, params([0]), layers[:1], *args, token_mask=mask)
    then2 = oracle.forward(after1, cids, cu, params([1]), layers[1:], *args, token_mask=mask)
    np.testing.assert_array_equal(both.view(np.uint32), then2.view(np.uint32))
    after2 = oracle.forward(h, cids, cu, params([1]), layers[1:], *args, token_mask=mask)
    then1 = oracle.forward(after2, cids, cu, params([0]), layers[:1], *args, token_mask=mask)
    assert np.abs(both - then1).max() > 0
    # masked tokens keep their streams through both layers
    np.testing.assert_array_equal(both[mask == 0].view(np.uint32), h[mask == 0].view(np.uint32))
