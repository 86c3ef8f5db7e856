"""The patch-pooling kernel sums patch rows in fp64 in a fixed phase order and
relies on every partial sum being exact, so that its patch means (and the
top-s ranking built on them) equal the fp64 oracle's bit for bit in any
summation order.  The kernel states the condition: with p significant bits per
entry (8 for bf16, 24 for fp32), at most 2^12 rows and nonzero magnitudes
within a factor 2^r of each other, a sum spans p + r + 12 bits, so it is exact
for r <= 33 (bf16) or r <= 17 (fp32).  These CPU checks pin that bound: at the
bound, sequential fp64 sums in several orders equal the exact integer sum; a
bf16 counterexample at r = 36 is not exact.
"""

import numpy as np


def _entries(rng, n, p, r):
    # integers m * 2^e with p significant bits (m in [2^(p-1), 2^p)) and
    # e in [0, r - 1]: every nonzero magnitude lies within a factor 2^r of every other
    m = rng.integers(2 ** (p - 1), 2 ** p, n)
    e = rng.integers(0, r, n)
    sign = rng.choice([-1, 1], n)
    return [int(s) * int(mm) * (1 << int(ee)) for s, mm, ee in zip(sign, m, e)]


def _exact_in_every_order(vals, rng):
    exact = sum(vals)
    for order in (np.arange(len(vals)), np.arange(len(vals))[::-1], rng.permutation(len(vals))):
        acc = 0.0
        run = 0
        for i in order:
            acc += float(vals[i])
            run += vals[i]
            if acc != float(run) or int(acc) != run:
                return False
        assert int(acc) == exact
    return True


def test_bf16_and_fp32_bounds_hold():
    rng = np.random.default_rng(3)
    for p, r in ((8, 33), (24, 17)):
        for _ in range(3):
            assert _exact_in_every_order(_entries(rng, 4096, p, r), rng)


def test_bf16_counterexample_past_the_bound():
    # one entry 1 + 2^-7 and 4095 entries 2^36 (1 + 2^-7), scaled by 2^7 to integers:
    # the exact sum needs 8 + 36 + 12 = 56 bits, more than fp64 holds
    small = 129
    big = 129 << 36
    vals = [small] + [big] * 4095
    acc = 0.0
    for v in vals:
        acc += float(v)
    assert int(acc) != sum(vals)
