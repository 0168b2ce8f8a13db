"""CPU check of the arithmetic the Q2_K kernels use to reach the oracle's
bit-exact rows for every finite fp16 d and dmin (no GPU; numpy float32
stands in for the kernels' fp32 operations, one rounding per operation).

The kernels form y = d*scale*q - dmin*min and round it to bf16:
* fast path: one fp32 fused multiply-add, then fp32 -> bf16 to nearest even.
  d*scale (<= 15 significant bits), q*d*scale (<= 17) and dmin*min (<= 15)
  are exact in fp32; the difference is exact, so the bf16 rounding is the
  only one, whenever the two fp16 exponents (subnormals counted as exponent
  field 1) differ by -9 .. 7, or d or dmin is zero.  Then y is 2^min(E) times
  an integer below 92115 * 2^7 + 30705 or 92115 + 30705 * 2^9, both < 2^24.
* exact path, for the other blocks: the difference s = fl(a - b) and its
  rounding error e (Knuth's TwoSum, exact); s is rounded to odd with e (s if
  e == 0 or s is odd, else the fp32 neighbour of s on e's side); that value,
  rounded to bf16 to nearest even, is the bf16 rounding of the exact y
  (Boldo and Melquiond: rounding to odd at 24 bits, then to nearest at 8 <=
  24 - 2 bits, is one rounding to nearest).
"""

import numpy as np

import oracle

F = np.float32


def _f32_to_bf16_bits(x):
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def fp32_is_exact(d_bits, m_bits):
    """The kernels' per-block test for the fast path."""
    d_bits, m_bits = np.asarray(d_bits, np.int64), np.asarray(m_bits, np.int64)
    ed, em = (d_bits >> 10) & 31, (m_bits >> 10) & 31
    zero = ((d_bits & 0x7FFF) == 0) | ((m_bits & 0x7FFF) == 0)
    gap = np.maximum(ed, 1) - np.maximum(em, 1)
    return zero | (ed == 31) | (em == 31) | ((gap >= -9) & (gap <= 7))


def fast(dl, ml, q):
    return _f32_to_bf16_bits(F(q) * dl - ml)          # product exact: = fma rounding


def exact(dl, ml, q):
    a = (F(q) * dl).astype(F)                         # exact
    b = ml.astype(F)
    s = (a - b).astype(F)
    bv = (s - a).astype(F)
    av = (s - bv).astype(F)
    e = ((a - av).astype(F) + (-b - bv).astype(F)).astype(F)
    t = s.view(np.uint32).astype(np.int64)
    same = ((e.view(np.uint32) ^ s.view(np.uint32)) >> 31) == 0
    fix = (e != 0) & ((t & 1) == 0)
    t = np.where(fix, t + np.where(same, 1, -1), t)
    return _f32_to_bf16_bits(t.astype(np.uint32).view(np.float32))


def _values(blocks, path):
    """bf16 bits [B, 256] of Q2_K blocks by the given kernel arithmetic."""
    blocks = np.asarray(blocks, np.uint8)
    d = blocks[:, 80:82].copy().view("<f2").astype(F)[:, 0]
    dm = blocks[:, 82:84].copy().view("<f2").astype(F)[:, 0]
    out = np.empty((len(blocks), 256), np.uint16)
    for i in range(256):
        byte = blocks[:, 16 + 32 * (i // 128) + i % 32]
        q = ((byte >> (2 * ((i % 128) // 32))) & 3).astype(F)
        sc = (blocks[:, i // 16] & 15).astype(F)
        mn = (blocks[:, i // 16] >> 4).astype(F)
        out[:, i] = path(d * sc, dm * mn, q)
    return out


def _random_blocks(n, seed, lo=0, hi=0x7C00):
    rng = np.random.default_rng(seed)
    b = rng.integers(0, 256, (n, 84)).astype(np.uint8)
    for k in (80, 82):
        bits = rng.integers(lo, hi, n) | (rng.integers(0, 2, n) << 15)
        b[:, k], b[:, k + 1] = bits & 0xFF, bits >> 8
    return b


def _oracle(blocks):
    return oracle.rows_q2k(blocks, np.arange(len(blocks))[:, None])


def test_fast_path_is_exact_wherever_the_block_test_allows_it():
    blocks = _random_blocks(20000, 1)
    d_bits = blocks[:, 80].astype(np.int64) | (blocks[:, 81].astype(np.int64) << 8)
    m_bits = blocks[:, 82].astype(np.int64) | (blocks[:, 83].astype(np.int64) << 8)
    ok = fp32_is_exact(d_bits, m_bits)
    # also every exponent gap at its edges: -9 and 7 with the largest mantissas
    edge = []
    for ed in range(1, 31):
        for em in (ed - 7, ed + 9):
            if 1 <= em <= 30:
                b = _random_blocks(1, ed * 31 + em)[0]
                b[:16] = 0xFF                          # scale 15, min 15
                b[16:80] = 0xFF                        # q = 3
                dbits, mbits = (ed << 10) | 0x3FF, (em << 10) | 0x3FF
                b[80], b[81], b[82], b[83] = dbits & 0xFF, dbits >> 8, mbits & 0xFF, mbits >> 8
                edge.append(b)
    sel = np.concatenate([blocks[ok], np.stack(edge)])
    assert len(sel) > 5000
    np.testing.assert_array_equal(_values(sel, fast), _oracle(sel))


def test_exact_path_matches_the_oracle_for_every_finite_block():
    blocks = np.concatenate([_random_blocks(20000, 2), _random_blocks(2000, 3, 0, 0x400)])
    np.testing.assert_array_equal(_values(blocks, exact), _oracle(blocks))


def test_fast_path_alone_would_not_be_exact():
    # Why the exact path exists: on wide blocks the fp32 difference rounds,
    # and a second rounding to bf16 can land on the other side of a tie.
    blocks = _random_blocks(20000, 4)
    d_bits = blocks[:, 80].astype(np.int64) | (blocks[:, 81].astype(np.int64) << 8)
    m_bits = blocks[:, 82].astype(np.int64) | (blocks[:, 83].astype(np.int64) << 8)
    wide = blocks[~fp32_is_exact(d_bits, m_bits)]
    assert (_values(wide, fast) != _oracle(wide)).any()


def fp32_only_rows(blocks):
    """bf16 bits [B, 256] of Q2_K blocks evaluated with one fp32 fma per value
    and nothing else (the shortcut the kernels take only where it is exact)."""
    return _values(blocks, fast)
