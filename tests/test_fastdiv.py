"""The multiply-high division the kernels use to decode their work items
(Granlund and Montgomery, "Division by Invariant Integers using
Multiplication", PLDI 1994, section 4): for a divisor d with l = ceil(log2 d)
and m = floor(2^32 (2^l - d) / d) + 1, (mulhi(n, m) + n) >> l equals n // d
for every 0 <= n < 2^31.  Checked here exhaustively over small n and at
every multiple boundary of large n, for the divisors the index decodes meet
(head groups, column groups, spans, chains and batch sizes)."""
import numpy as np


def magic(d):
    if d <= 1:
        return 1, 0
    l = 0
    while (1 << l) < d:
        l += 1
    return ((1 << 32) * ((1 << l) - d)) // d + 1, l


def fdiv(n, m, l):
    n = n.astype(np.uint64)
    return ((n * np.uint64(m)) >> np.uint64(32)) + n >> np.uint64(l)


def check(d, n):
    m, l = magic(d)
    assert 0 < m < (1 << 32)
    got = fdiv(n, m, l)
    assert np.array_equal(got, n.astype(np.uint64) // np.uint64(d)), d


def test_small_numerators_exhaustive():
    n = np.arange(1 << 16, dtype=np.uint64)
    for d in range(1, 1025):
        check(d, n)


def test_large_numerators_at_quotient_boundaries():
    rng = np.random.default_rng(7)
    top = (1 << 31) - 1
    divisors = list(range(1, 300)) + [383, 384, 385, 1000, 1536, 4095, 4096, 4097,
                                      65535, 65536, 65537, 1 << 20, (1 << 20) + 1,
                                      (1 << 30) - 1, 1 << 30, (1 << 30) + 1]
    divisors += rng.integers(2, 1 << 31, 64).tolist()
    for d in divisors:
        q = rng.integers(0, top // d + 1, 4096, dtype=np.uint64)
        n = np.concatenate([q * np.uint64(d), q * np.uint64(d) + np.uint64(d - 1),
                            np.array([top, top - 1, 0], dtype=np.uint64)])
        n = n[n <= np.uint64(top)]
        check(d, n)
