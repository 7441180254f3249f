"""The exact division that locates a unit's piece in the prefill kernel.

The kernel divides by a handful of per-call divisors (units per workgroup,
the pieces' lengths, the K panels and the blocks per panel) with
host-computed multipliers: for d > 1,
l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1, and then
n / d = (t + ((n - t) >> 1)) >> (l - 1) with t = floor(n m / 2^32)
(Granlund and Montgomery, "Division by invariant integers using
multiplication", 1994). This checks the method itself against integer
division over the divisors the library can meet (1 .. 2^28) and all 32-bit
dividends at the edges; the GPU parity tests check the kernel's use of it.

Staging x divides a vector index idx < 2^14 by the vectors per row, kp * 32:
(idx >> 5) / kp with n = idx >> 5 < 2^9 is (n * m) >> (9 + l) for
l = ceil(log2 kp), m = ceil(2^(9 + l) / kp), one 24-bit multiply (the same
paper's round-up method for N-bit dividends).
"""
import random


def multiplier(d):
    if d <= 1:
        return 0, 0
    l = (d - 1).bit_length()  # ceil(log2 d)
    return ((1 << 32) * ((1 << l) - d)) // d + 1, l


def divide(n, m, l):
    if l == 0:
        return n
    t = (n * m) >> 32
    return (t + ((n - t) >> 1)) >> (l - 1)


def test_multiplier_fits_32_bits_and_shift_is_ceil_log2():
    for d in list(range(2, 70000)) + [2 ** 28, 2 ** 28 - 1, 3 << 26]:
        m, l = multiplier(d)
        assert 0 < m < 2 ** 32
        assert 2 ** (l - 1) < d <= 2 ** l


def test_division_is_exact():
    rng = random.Random(7)
    divisors = list(range(1, 3000)) + [2 ** k + e for k in range(1, 29) for e in (-1, 0, 1)]
    divisors += [rng.randrange(2, 2 ** 28) for _ in range(3000)]
    for d in divisors:
        m, l = multiplier(d)
        ns = [0, 1, d - 1, d, d + 1, 2 ** 31 - 1, 2 ** 31, 2 ** 32 - 1]
        ns += [q * d + r for q in (1, 2, 15, 16, 17, 1 << 10) for r in (0, d - 1)]
        ns += [rng.randrange(2 ** 32) for _ in range(20)]
        for n in ns:
            if 0 <= n < 2 ** 32:
                assert divide(n, m, l) == n // d, (n, d)


def row_multiplier(kp):
    l = (kp - 1).bit_length()  # ceil(log2 kp)
    return -(-(1 << (9 + l)) // kp), 9 + l


def test_staging_row_multiplier_is_exact():
    # every blocks-per-panel count up to 512 (x fits in LDS up to 312) and
    # every 9-bit quotient input
    for kp in range(1, 513):
        m, s = row_multiplier(kp)
        assert m < 2 ** 24
        for n in range(512):
            assert n * m < 2 ** 32
            assert (n * m) >> s == n // kp, (n, kp)
