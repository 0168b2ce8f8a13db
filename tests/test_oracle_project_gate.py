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
