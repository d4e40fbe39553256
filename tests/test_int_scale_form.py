"""The integer form of a key's fp16 block scales (host-side check of the
arithmetic the 32-row attention kernel relies on; no GPU).

A finite binary16 value s is m * 2^(e - 25) with e its exponent field (1 for
subnormals) and m its integer significand.  Over one key's nonzero block
scales, with emin the smallest e, s_b = M_b * 2^(emin - 25) where
M_b = m_b << (e_b - emin).  When every e_b - emin <= 3, sum_b M_b * S_b over
eight int32 block sums |S_b| <= 32 * 127 * 4 stays inside int32, so the
key's block-scaled logit is one exact integer times a power of two.
"""
from fractions import Fraction

import numpy as np

S_MAX = 32 * 127 * 4          # |int8 q| <= 127, |k| = |c - 4| <= 4


def split(bits: int):
    E, man = (bits >> 10) & 31, bits & 1023
    m = (man | 1024) if E else man
    e = (E if E else 1) if m else 31
    return m, e


def test_every_finite_fp16_splits_exactly():
    bits = np.arange(0, 0x7C00, dtype=np.uint16)          # +0 .. 65504
    vals = bits.view(np.float16).astype(np.float64)
    for b, v in zip(bits.tolist(), vals.tolist()):
        m, e = split(b)
        assert Fraction(v) == Fraction(m) * Fraction(2) ** (e - 25)
        assert m < 2048


def test_largest_sum_fits_int32():
    m_max = 2047 << 3
    assert m_max < 2 ** 14 < 2 ** 15                     # a positive int16 operand
    assert 8 * m_max * S_MAX < 2 ** 31
    # the case the GPU test builds: seven blocks three binades above the eighth
    assert S_MAX * (7 * m_max + 2047) < 2 ** 31


def test_key_sum_equals_the_scaled_sum():
    rng = np.random.default_rng(7)
    for _ in range(2000):
        emin = int(rng.integers(1, 28))
        es = emin + rng.integers(0, 4, size=8)
        es[int(rng.integers(0, 8))] = emin
        mans = rng.integers(0, 1024, size=8)
        bits = [(int(e) << 10) | int(mn) for e, mn in zip(es, mans)]
        if rng.random() < 0.2:
            bits[int(rng.integers(0, 8))] = 0                 # a zero block
        S = rng.integers(-S_MAX, S_MAX + 1, size=8)
        parts = [split(b) for b in bits]
        nz = [e for m, e in parts if m]
        if not nz:
            continue
        lo = min(nz)
        M = [m << (e - lo) if m else 0 for m, e in parts]
        acc = sum(int(a) * int(s) for a, s in zip(M, S))
        assert abs(acc) < 2 ** 31
        exact = sum(Fraction(np.array([b], dtype=np.uint16).view(np.float16)[0].item()) * int(s)
                    for b, s in zip(bits, S))
        assert Fraction(acc) * Fraction(2) ** (lo - 25) == exact
