"""Pins for the oracle's binary64 batch-1 GEMV (`oracle.gemv_f64`), the
reference the fused decode+GEMV is compared with. No GPU code is involved.

The GEMV is the forward product that consumes the decoded weights (EntQuant
summary, section 2, technical component 3; its future-work part proposes
fusing the decompression into that matrix multiply)."""
from fractions import Fraction

import numpy as np

import oracle


def _bf16_bits(v: np.ndarray) -> np.ndarray:
    return oracle.bf16_rne(np.asarray(v, np.float32))


def _bits_to_fraction(b: int) -> Fraction:
    return Fraction(float(np.array([b << 16], np.uint32).view(np.float32)[0]))


def test_hand_worked_2x2():
    # W = [[1, 2], [-1, 0.5]], x = [3, 1]: y = [1*3 + 2*1, -1*3 + 0.5*1] = [5, -2.5];
    # sum |W x| per row = [5, 3.5]
    w = np.array([[0x3F80, 0x4000], [0xBF80, 0x3F00]], np.uint16)
    x = np.array([0x4040, 0x3F80], np.uint16)
    y, a = oracle.gemv_f64(w, x)
    assert y.tolist() == [5.0, -2.5]
    assert a.tolist() == [5.0, 3.5]


def test_one_hot_selects_a_column_of_a_non_square_matrix():
    rng = np.random.default_rng(3)
    w = _bf16_bits(rng.standard_normal((5, 7)))
    for c in range(7):
        x = np.zeros(7, np.uint16)
        x[c] = 0x3F80  # 1.0
        y, _ = oracle.gemv_f64(w, x)
        exp = (w[:, c].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.array_equal(y, exp), c


def test_against_exact_rational_sum():
    # products of bf16 values are exact in binary64; the binary64 sum may
    # round, by at most (cols - 1) * 2^-53 * sum |w x|
    rng = np.random.default_rng(11)
    for rows, cols in [(3, 1), (4, 17), (6, 64), (2, 300)]:
        w = _bf16_bits(rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-8, 8, (rows, cols))))
        x = _bf16_bits(rng.standard_normal(cols))
        y, a = oracle.gemv_f64(w, x)
        for r in range(rows):
            exact = sum(_bits_to_fraction(int(w[r, c])) * _bits_to_fraction(int(x[c])) for c in range(cols))
            absum = sum(abs(_bits_to_fraction(int(w[r, c])) * _bits_to_fraction(int(x[c]))) for c in range(cols))
            assert abs(Fraction(y[r]) - exact) <= Fraction(max(cols - 1, 0), 2**53) * absum
            assert abs(Fraction(a[r]) - absum) <= Fraction(cols, 2**53) * absum


def test_cancellation_is_not_lost():
    # 2^20 + 1 - 2^20 in ascending order: every partial sum is exact in binary64
    w = _bf16_bits(np.array([[2.0**20, 1.0, -(2.0**20)]]))
    x = _bf16_bits(np.ones(3))
    y, a = oracle.gemv_f64(w, x)
    assert y[0] == 1.0 and a[0] == 2.0**21 + 1
