"""The attention K mean: where the GPU's binary64 summation reproduces the exact
mean that the oracle defines.

The kernel sums the bf16 keys of each (head, channel) in binary64 and returns
fl32(fl64(S / Sk)).  Whenever every partial sum is exact (a sufficient condition
is sum|k| < 2^53 * q_min, q_min the finest quantum among the nonzero keys), S is
the exact sum and the only question is the two roundings of the quotient.  They
give the exactly rounded mean: a binary32 midpoint m (25 significant bits) can
only be the binary64 rounding of S / Sk if |S - m Sk| < 2^-53 * 2^e(m) * Sk,
which is less than one unit of the last place of a 53-bit S, so S = m Sk and
the tie is a true tie.  These CPU checks exercise that argument on random and
adversarial quotients.
"""
from fractions import Fraction

import numpy as np

import oracle


def _two_roundings(s: float, sk: int) -> np.float32:
    return np.float32(np.float64(s) / np.float64(sk))


def test_quotient_rounding_random():
    rng = np.random.default_rng(3)
    for _ in range(20000):
        sk = 16 * int(rng.integers(1, 65536))
        # a 53-bit sum at a random scale
        s = float(int(rng.integers(-(1 << 53) + 1, 1 << 53))) * 2.0 ** int(rng.integers(-180, 60))
        num, den = Fraction(s).numerator, Fraction(s).denominator * sk
        assert _two_roundings(s, sk) == np.float32(oracle._f32_nearest(num, den))


def test_quotient_rounding_next_to_binary32_midpoints():
    """S = m * Sk + t * ulp(S) for binary32 midpoints m and small t: the cases in
    which a double rounding could differ, if the argument were wrong."""
    rng = np.random.default_rng(4)
    checked = 0
    for _ in range(20000):
        sk = 16 * int(rng.integers(1, 65536))
        mant = (1 << 24) + 2 * int(rng.integers(0, 1 << 23)) + 1      # 25 bits, odd: a binary32 midpoint
        e = int(rng.integers(-140, 40))
        m = Fraction(mant) * Fraction(2) ** (e - 24)
        exact = m * sk
        s0 = float(exact)                                              # nearest binary64 to m * Sk
        for t in (-2, -1, 0, 1, 2):
            s = s0 + t * np.spacing(abs(s0)) if s0 != 0 else s0
            fs = Fraction(s)
            assert _two_roundings(s, sk) == np.float32(oracle._f32_nearest(fs.numerator, fs.denominator * sk))
            checked += 1
    assert checked == 100000


def test_quotient_rounding_subnormal_means():
    """Means below 2^-126 (binary32 subnormals), where the last place is 2^-149."""
    rng = np.random.default_rng(5)
    for _ in range(20000):
        sk = 16 * int(rng.integers(1, 65536))
        s = float(int(rng.integers(-(1 << 40), 1 << 40))) * 2.0 ** -133 * 2.0 ** int(rng.integers(-20, 10))
        fs = Fraction(s)
        assert _two_roundings(s, sk) == np.float32(oracle._f32_nearest(fs.numerator, fs.denominator * sk))
