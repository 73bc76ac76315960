"""The compensated sum of squares the kernels use reaches the exact sum in any order (CPU).

The HIP kernels accumulate x^2 (exact in fp64 for an fp32 x) into (hi, lo)
pairs with Knuth's two-sum and combine the pairs across lanes, wavefronts,
tiles and chunks in a tree whose shape depends on the launch; the scale then
takes fl64(hi + lo).  Both oracles instead define the scale from the exact sum
rounded once.  Restated here in Python (IEEE fp64 arithmetic, the same
operations in the same order per step), the scheme runs over random splits
into leaves and random combine trees, and must give math.fsum of the squares
(the exact sum rounded once) every time.  This is the property that lets the
GPU reduce in any order and still match the oracles' scales bit for bit.
"""
import math
import random

import numpy as np
import pytest


def accumulate(hi, lo, x):
    """(hi, lo) += x * x with x * x exact: two-sum of hi and the square."""
    q = x * x
    s = hi + q
    bp = s - hi
    lo += (hi - (s - bp)) + (q - bp)
    return s, lo


def combine(a, b):
    """(hi, lo) pair sum, renormalised."""
    hi, lo = a
    bhi, blo = b
    s = hi + bhi
    bp = s - hi
    e = (hi - (s - bp)) + (bhi - bp)
    e = e + (lo + blo)
    h = s + e
    return h, e - (h - s)


def compensated(values, rng):
    """Random leaves accumulated in order, then combined in a random tree."""
    vals = [float(v) for v in values]
    cuts = sorted(rng.sample(range(1, len(vals)), min(len(vals) - 1, rng.randint(0, 40)))) if len(vals) > 1 else []
    pairs, start = [], 0
    for end in cuts + [len(vals)]:
        hi = lo = 0.0
        for v in vals[start:end]:
            hi, lo = accumulate(hi, lo, v)
        pairs.append((hi, lo))
        start = end
    while len(pairs) > 1:
        i = rng.randrange(len(pairs) - 1)
        pairs[i:i + 2] = [combine(pairs[i], pairs[i + 1])]
    hi, lo = pairs[0]
    return hi + lo


def _inputs(kind, n, rng):
    if kind == "normal":
        return rng.normal(0.0, 1e-3, n).astype(np.float32)
    if kind == "lognormal":
        return (rng.choice([-1.0, 1.0], n) * np.exp(rng.normal(-14.0, 4.0, n))).astype(np.float32)
    if kind == "mixed":
        x = rng.normal(0.0, 1.0, n) * 10.0 ** rng.integers(-18, 18, n)
        return x.astype(np.float32)
    # one large value over many tiny ones: the tiny squares must survive in lo
    x = np.full(n, np.float32(1e-4))
    x[n // 2] = np.float32(3e3)
    return x


@pytest.mark.parametrize("kind", ["normal", "lognormal", "mixed", "one_large"])
def test_compensated_sum_equals_exact_in_any_order(kind):
    nrng = np.random.default_rng(5)
    rng = random.Random(9)
    for n in (1, 7, 300, 5000):
        x = _inputs(kind, n, nrng)
        exact = math.fsum(float(v) * float(v) for v in x)
        for _ in range(6):
            assert compensated(x, rng) == exact, (kind, n)


def test_plain_fp64_sum_is_order_dependent():
    """Why the pair is needed: a plain fp64 sum of the same squares depends on
    the order for these inputs, so it could not match an exact-sum oracle."""
    x = _inputs("one_large", 5000, np.random.default_rng(5))
    sq = [float(v) * float(v) for v in x]
    forward = sum(sq)
    backward = sum(reversed(sq))
    assert forward != backward or forward != math.fsum(sq)
