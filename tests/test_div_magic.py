"""The division-by-invariant-integer method the attention kernel's work-item decode uses
(Granlund and Montgomery, PLDI 1994, the 33-bit-multiplier case): for d >= 1, with
2^(l-1) < d <= 2^l, m = floor(2^32 (2^l - d) / d) + 1 and t = mulhi(m, x),
x / d = (t + ((x - t) >> min(l, 1))) >> max(l - 1, 0) for every 32-bit x.  Written out
here from that statement (the C++ header checks its own copy at compile time) and checked
against integer division: every divisor below 5000 against every dividend below 70000 and
random ones, and random large divisors with the edge dividends."""
import numpy as np


def _magic(d):
    l = 0
    while (1 << l) < d:
        l += 1
    return ((1 << 32) * ((1 << l) - d)) // d + 1, min(l, 1), max(l - 1, 0)


def _div(x, d):
    m, s1, s2 = _magic(d)
    x = np.asarray(x, np.uint64)
    t = (x * np.uint64(m)) >> np.uint64(32)
    return (t + ((x - t) >> np.uint64(s1))) >> np.uint64(s2)


def test_every_small_divisor():
    xs = np.arange(0, 70000, dtype=np.uint64)
    for d in range(1, 5000):
        assert np.array_equal(_div(xs, d), xs // np.uint64(d)), d


def test_random_divisors_and_edge_dividends():
    rng = np.random.default_rng(3)
    for d in [int(v) for v in rng.integers(5000, 1 << 32, 3000)] + [(1 << 31) - 1, 1 << 31,
                                                                     (1 << 32) - 1]:
        xs = np.concatenate([rng.integers(0, 1 << 32, 2000, dtype=np.uint64),
                             np.array([0, 1, d - 1, d, d + 1, (1 << 31), (1 << 32) - 1],
                                      np.uint64)])
        xs = xs[xs < (1 << 32)]
        assert np.array_equal(_div(xs, d), xs // np.uint64(d)), d
