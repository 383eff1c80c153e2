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


@pytest.mark.parametrize("c", [np.float32(1.0 / 39.6), np.float32(0.5), np.float32(0.3),
                               np.float32(1.0 / (8.0 + 1e-6)), np.nextafter(np.float32(1), np.float32(0))])
def test_scale_is_the_correctly_rounded_product(c):
    # g <- g * c rounds the exact product once to binary32 (ties to even),
    # checked against exact rationals; magnitudes span normal gradients,
    # outliers and the subnormal range, where a product by c < 1 loses bits
    rng = np.random.default_rng(int(c.view(np.uint32)))
    k = 3000
    mags = 10.0 ** rng.uniform(-42, 2, k)
    g = (mags * rng.choice([-1.0, 1.0], k)).astype(np.float32)
    g[:4] = [0.0, -0.0, 2.0 ** -149, -(2.0 ** -126)]
    want = [rn32(Fr(float(x)) * Fr(float(c))) for x in g]
    got = g.copy()
    _c.scale(got, float(c))
    for i in range(k):
        w, x = np.float32(want[i]), got[i]
        # a zero product keeps the sign of g (c > 0)
        if w == 0:
            w = np.float32(np.copysign(0.0, g[i]))
        assert x.view(np.uint32) == w.view(np.uint32), (i, g[i], x, w)


def test_scale_keeps_inf_and_nan():
    g = np.array([np.inf, -np.inf, np.nan], np.float32)
    _c.scale(g, 0.25)
    assert g[0] == np.inf and g[1] == -np.inf and np.isnan(g[2])


@pytest.mark.parametrize("n,k_exp,max_norm", [(4, -3, 1.0), (8, -7, 0.01), (2, 1, 3.0)])
def test_clipped_first_moment_is_the_scaled_constant_gradient(n, k_exp, max_norm):
    # every rank holds the constant gradient k = 2^k_exp over psi = 4096
    # elements, so the mean is k, the norm 64|k| exactly, and the clip
    # coefficient c = max_norm / (64|k| + 1e-6) < 1.  After one step from
    # zero state the first moment is (1 - b1) * (k * c): checked against
    # exact rationals through the C per-rank chain and through every
    # strategy of the simulation.  Dividing by c, or scaling by anything but
    # c, moves m by a factor near 1/c^2.
    from oracle import strategies
    psi = 4096
    k = 2.0 ** k_exp
    cfg = strategies.AdamConfig(max_grad_norm=max_norm)
    hp = cfg.hparams(1)
    c = np.float32(max_norm / (64.0 * k + 1e-6))
    assert c < 1
    omb1 = np.float32(1.0 - float(np.float32(cfg.beta1)))
    g_c = rn32(Fr(k) * Fr(float(c)))
    m_want = rn32(Fr(float(omb1)) * Fr(float(g_c)))
    exact = Fr(float(omb1)) * Fr(k) * Fr(float(c))
    assert abs(Fr(float(m_want)) - exact) <= 2 * Fr(float(np.spacing(np.float32(m_want))))

    ranks = [bf16(np.full(psi, k)) for _ in range(n)]
    coef = _c.clip_coef(_c.sumsq(_c.average(ranks)), max_norm)
    assert np.float32(coef) == c
    p = np.full(psi, 0.01, np.float32)
    m = np.zeros(psi, np.float32)
    v = np.zeros(psi, np.float32)
    out = np.empty(psi, np.uint16)
    _c.rank_step(hp, ranks, coef, p, m, v, out)
    assert np.all(m == m_want)

    for s in ("ddp", "zero2", "zero3", "megatron_do"):
        cl = strategies.make_cluster(s, [psi], n, np.full(psi, 0.01, np.float32))
        g = [[r] for r in ranks] if s == "megatron_do" else ranks
        strategies.step(cl, cfg, 1, g)
        assert np.all(strategies.full_state(cl)["m"] == m_want), s
