"""Pins of the oracle's data-parallel averaging, fp32 accumulation and clip.

  * Inputs whose fp32 partial sums are all exact (small multiples of 2^-12)
    make the average the exact rational mean, correctly rounded once by the
    division -- independent of summation order.
  * A constructed input whose fp32 sum depends on the order pins the
    reading "ascending rank order, starting from +0".
  * For arbitrary inputs the recursive-summation error bound
    |err| <= (N - 1) u sum|x| (u = 2^-24) holds, plus the final rounding.
  * A constant gradient c on every rank has the mean c and the global norm
    |c| sqrt(Psi): an oracle that clipped the sum instead of the mean, or
    took the norm per rank, fails.
"""
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import _c


def rn32(x: Fr) -> np.float32:
    """Correct rounding of an exact rational to binary32 (ties to even)."""
    f = np.float32(float(x))
    lo = f if Fr(float(f)) <= x else np.nextafter(f, np.float32(-np.inf))
    hi = np.nextafter(lo, np.float32(np.inf))
    dl, dh = x - Fr(float(lo)), Fr(float(hi)) - x
    if dl < dh:
        return lo
    if dh < dl:
        return hi
    return lo if (int(np.array(lo).view(np.uint32)) & 1) == 0 else hi


def bf16(x):
    return _c.f32_to_bf16(np.asarray(x, np.float32))


@pytest.mark.parametrize("n", [1, 2, 3, 4, 7, 8, 64])
def test_exact_inputs_give_the_rounded_exact_mean(n):
    rng = np.random.default_rng(n)
    k = 257
    ranks = [(rng.integers(-128, 128, k) * 2.0 ** -12).astype(np.float32) for _ in range(n)]
    bits = [bf16(r) for r in ranks]
    assert all(np.array_equal(_c.bf16_to_f32(b), r) for b, r in zip(bits, ranks))
    out = _c.average(bits)
    out32 = _c.average(ranks)
    for i in range(k):
        want = rn32(sum(Fr(float(r[i])) for r in ranks) / n)
        assert out[i] == want and out32[i] == want


def test_summation_is_ascending_from_zero():
    # ranks hold 1, 2^-24, 2^-24, 2^-24.  Ascending: 1 + 2^-24 ties back to 1
    # three times -> 1, mean 0.25.  Descending would give 1 + 2^-22 first.
    vals = [1.0, 2.0 ** -24, 2.0 ** -24, 2.0 ** -24]
    bits = [bf16([v]) for v in vals]
    assert _c.average(bits)[0] == np.float32(0.25)
    rev = list(reversed(bits))
    assert _c.average(rev)[0] == np.float32(0.25 + 2.0 ** -24)


def test_fp32_summation_is_ascending_from_zero():
    # the same four values as fp32 rank buffers (the Megatron fp32 path):
    # descending, 3 * 2^-24 is summed first and 1 + 3 * 2^-24 ties to 1 + 2^-22
    bufs = [np.array([v], np.float32) for v in (1.0, 2.0 ** -24, 2.0 ** -24, 2.0 ** -24)]
    assert _c.average(bufs)[0] == np.float32(0.25)
    assert _c.average(list(reversed(bufs)))[0] == np.float32(0.25 + 2.0 ** -24)


@pytest.mark.parametrize("n", [2, 4, 8, 64])
def test_general_inputs_within_recursive_summation_bound(n):
    rng = np.random.default_rng(100 + n)
    k = 4096
    ranks = [bf16(rng.standard_normal(k) * 1e-3 * (1 + 99 * (rng.random(k) < 0.01)))
             for _ in range(n)]
    out = _c.average(ranks).astype(np.float64)
    x = np.stack([_c.bf16_to_f32(b).astype(np.float64) for b in ranks])
    exact = x.sum(0) / n           # fp64 sum of <= 64 bf16 values is exact
    bound = (n - 1) * 2.0 ** -24 * np.abs(x).sum(0) / n + np.spacing(np.abs(out).astype(np.float32))
    assert np.all(np.abs(out - exact) <= bound)


def test_fp32_accumulation_of_micro_batches():
    rng = np.random.default_rng(5)
    k, K = 1000, 4
    micro = [bf16(rng.integers(-100, 100, k) * 2.0 ** -10) for _ in range(K)]
    acc = np.zeros(k, np.float32)
    for mb in micro:
        _c.accumulate_bf16(acc, mb)
    exact = sum(_c.bf16_to_f32(mb).astype(np.float64) for mb in micro)
    assert np.array_equal(acc.astype(np.float64), exact)


def test_clip_norm_of_constant_gradient():
    psi = 4096                         # sqrt(psi) = 64
    c = 2.0 ** -3
    g = np.full(psi, c, np.float32)
    s = _c.sumsq(g)
    assert s == psi * c * c            # exact: 64.0
    coef = _c.clip_coef(s, 1.0)
    assert coef == np.float32(1.0 / (64 * c + 1e-6))
    assert _c.clip_coef(s, 100.0) == 1.0       # norm 8 < 100: no clip


def test_clip_coefficient_rounding():
    # fp64 norm, fp64 quotient, one rounding to fp32
    for s, mx in [(39.6 ** 2, 1.0), (2.0, 1.0), (1e-12, 1.0), (1e6, 0.5)]:
        want = min(1.0, float(np.float32(mx / (np.sqrt(s) + 1e-6))))
        assert _c.clip_coef(s, mx) == np.float32(want)
