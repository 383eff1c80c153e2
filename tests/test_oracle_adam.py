"""Pins of the oracle's Adam / AdamW step to results fixed by the mathematics
of the update (Kingma & Ba 2015, Algorithm 1; Loshchilov & Hutter 2019), not
by re-running its formula:

  * t = 1 from m = v = 0: the bias-corrected moments are exactly g and g^2,
    so p1 = p0 - lr * g / (|g| + eps).
  * A constant gradient keeps m_hat = g and v_hat = g^2 at every t, so
    p_T = p0 - T * lr * g / (|g| + eps).
  * Two steps with gradients a then b: m_hat_2 = (b1 a + b) / (1 + b1) and
    v_hat_2 = (b2 a^2 + b^2) / (1 + b2) (the bias-corrected EMA of two terms,
    simplified by hand).
  * g = 0, no decay: nothing changes.  g = 0 with AdamW decay: p_T =
    p0 * (1 - lr wd)^T.  g = 0 with L2 decay: the effective gradient is
    wd * p, so the first step moves p by lr * sign(p) (to within eps).

The expected values are evaluated exactly (fractions) or in high precision
(decimal, for the square root), and the fp32 oracle must land within a few
fp32 ulps of them.  A plausible slip in the oracle -- a dropped bias
correction, beta1 and 1 - beta1 swapped, eps inside the square root, an
off-by-one in t, decay applied to the wrong quantity -- moves the result by
far more than that.
"""
from decimal import Decimal, getcontext
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import _c

getcontext().prec = 60

LR, B1, B2, EPS = 1e-3, 0.9, 0.999, 1e-8


def f32(x):
    return np.float32(x)


def ulp(x):
    x = np.float32(abs(x))
    return float(np.spacing(x)) if x != 0 else float(np.spacing(np.float32(0)))


def run(g_steps, p0, m0=0.0, v0=0.0, wd=0.0, decoupled=False, lr=LR, b1=B1, b2=B2, eps=EPS):
    """Run the oracle on a vector over len(g_steps) steps."""
    p = np.array(p0, np.float32)
    m = np.full_like(p, m0)
    v = np.full_like(p, v0)
    for t, g in enumerate(g_steps, start=1):
        hp = _c.hparams(lr, b1, b2, eps, wd, t, decoupled)
        _c.adam(hp, np.array(g, np.float32), p, m, v)
    return p, m, v


def dsqrt(fr):
    return Fr((Decimal(fr.numerator) / Decimal(fr.denominator)).sqrt())


def tol(k, *xs):
    """k fp32 ulps at the scale of the largest quantity involved (the
    subtraction p - lr * u rounds at that scale)."""
    return k * Fr(ulp(max(abs(float(x)) for x in xs)))


def exact_step(p, mh, vh, lr=LR, eps=EPS):
    """p - lr * mh / (sqrt(vh) + eps), with the fp32 hyper-parameters taken at
    their exact binary32 values."""
    lr, eps = Fr(float(f32(lr))), Fr(float(f32(eps)))
    return p - lr * mh / (dsqrt(vh) + eps)


G = [3.0e-4, -7.5e-4, 1.25e-3, -2.0e-2, 6.1e-8, -1.0e-8, 0.5, 1e-5]
P0 = [0.02, -0.013, 0.0071, 0.5, -1.0, 0.03, 1e-3, -0.25]


def test_first_step_from_zero_state():
    p, m, v = run([G], P0)
    for i in range(len(G)):
        g = Fr(float(f32(G[i])))
        want = exact_step(Fr(float(f32(P0[i]))), g, g * g)
        assert abs(Fr(float(p[i])) - want) <= tol(2, P0[i], p[i], LR), i


def test_first_step_moment_values():
    # m1 = (1 - b1) g and v1 = (1 - b2) g^2, with b1, b2 at their binary32
    # values, up to the roundings of the products
    p, m, v = run([G], P0)
    b1, b2 = Fr(float(f32(B1))), Fr(float(f32(B2)))
    for i in range(len(G)):
        g = Fr(float(f32(G[i])))
        assert abs(Fr(float(m[i])) - (1 - b1) * g) <= 2 * Fr(ulp(m[i]))
        assert abs(Fr(float(v[i])) - (1 - b2) * g * g) <= 3 * Fr(ulp(v[i]))


@pytest.mark.parametrize("T", [1, 2, 5, 10])
def test_constant_gradient_T_steps(T):
    p, _, _ = run([G] * T, P0)
    for i in range(len(G)):
        g = Fr(float(f32(G[i])))
        p0 = Fr(float(f32(P0[i])))
        step = Fr(float(f32(LR))) * g / (abs(g) + Fr(float(f32(EPS))))
        want = p0 - T * step
        # each step contributes a few roundings of size ulp(p)
        assert abs(Fr(float(p[i])) - want) <= tol(3 * T, P0[i], p[i], LR), (i, T)


def test_two_step_closed_form():
    a = [2.0e-3, -1.0e-3, 4.0e-4, 1.0e-2]
    b = [-5.0e-4, -3.0e-3, 4.0e-4, 2.5e-2]
    p0 = [0.1, -0.2, 0.3, -0.05]
    p, _, _ = run([a, b], p0)
    b1, b2 = Fr(float(f32(B1))), Fr(float(f32(B2)))
    for i in range(4):
        A, Bv = Fr(float(f32(a[i]))), Fr(float(f32(b[i])))
        # step 1 moves by lr * sign-ish(a), step 2 by the two-term EMA
        p1 = exact_step(Fr(float(f32(p0[i]))), A, A * A)
        mh2 = (b1 * A + Bv) / (1 + b1)
        vh2 = (b2 * A * A + Bv * Bv) / (1 + b2)
        want = exact_step(p1, mh2, vh2)
        assert abs(Fr(float(p[i])) - want) <= tol(8, p0[i], p[i], LR), i


def test_zero_gradient_no_decay_is_identity():
    p0 = np.array(P0, np.float32)
    p, m, v = run([[0.0] * 8] * 4, P0)
    assert np.array_equal(p, p0) and not m.any() and not v.any()


@pytest.mark.parametrize("T", [1, 3, 7])
def test_zero_gradient_adamw_decay(T):
    wd = 0.01
    p, _, _ = run([[0.0] * 8] * T, P0, wd=wd, decoupled=True)
    decay = Fr(1) - Fr(float(f32(LR))) * Fr(float(f32(wd)))
    for i in range(8):
        want = Fr(float(f32(P0[i]))) * decay ** T
        assert abs(Fr(float(p[i])) - want) <= tol(2 * T + 1, P0[i]), i


def test_zero_gradient_l2_decay_first_step():
    wd = 0.1
    p, m, _ = run([[0.0] * 8], P0, wd=wd, decoupled=False)
    for i in range(8):
        p0 = Fr(float(f32(P0[i])))
        ge = Fr(float(f32(wd))) * p0        # effective gradient, sign of p
        want = exact_step(p0, ge, ge * ge)
        assert abs(Fr(float(p[i])) - want) <= tol(4, P0[i], p[i], LR), i
        # the L2 term enters the moment, the AdamW term would not
        assert m[i] != 0


def test_update_opposes_gradient():
    p, _, _ = run([G], P0)
    for i in range(8):
        assert np.sign(np.float32(P0[i]) - p[i]) == np.sign(G[i])


def test_fp32_oracle_tracks_fp64_evaluation():
    """Over 10 steps of random N(0, 1e-3) gradients the fp32 oracle stays
    within a few fp32 ulps of the same update evaluated in fp64."""
    rng = np.random.default_rng(7)
    n = 4096
    p32 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m32 = np.zeros(n, np.float32); v32 = np.zeros(n, np.float32)
    p64, m64, v64 = p32.astype(np.float64), np.zeros(n), np.zeros(n)
    for t in range(1, 11):
        g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        for dec, wd in ((True, 0.01),):
            hp = _c.hparams(LR, B1, B2, EPS, wd, t, dec)
            _c.adam(hp, g, p32, m32, v32)
            _c.adam_f64(hp, g.astype(np.float64), p64, m64, v64)
    # per step: one rounding of p (<= 1 ulp(p)) plus the relative error of the
    # fp32 update u (a handful of roundings, < 16 * 2^-24) times lr
    T = 10
    bound = T * (np.spacing(np.abs(p32)).astype(np.float64) + LR * 16 * 2.0 ** -24)
    assert np.all(np.abs(p32 - p64) <= bound)
    # m is a sum of terms of size up to max|m|; each step rounds twice
    m_ulp = float(np.spacing(np.abs(m32).max()))
    assert np.abs(m32 - m64).max() <= T * 2 * m_ulp


@pytest.mark.parametrize("dtype", [np.uint16, np.float32])
@pytest.mark.parametrize("clip", [1.0, 0.37])
def test_rank_step_is_the_pinned_chain_in_order(dtype, clip):
    """The per-rank chain (the expected values of the GPU parity tests) is,
    bit for bit, the separately pinned steps in the pages' order: the rank
    mean, the clip scale when its coefficient is below 1, one Adam step, and
    the bf16 rounding of the updated master."""
    rng = np.random.default_rng(7)
    n, k = 5, 3000
    raw = [rng.standard_normal(k).astype(np.float32) * np.float32(1e-3) for _ in range(n)]
    ranks = [_c.f32_to_bf16(r) for r in raw] if dtype == np.uint16 else raw
    p0 = rng.standard_normal(k).astype(np.float32) * np.float32(0.02)
    m0 = rng.standard_normal(k).astype(np.float32) * np.float32(1e-4)
    v0 = rng.random(k).astype(np.float32) * np.float32(1e-7)
    hp = _c.hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 3, True)

    def chain(c):
        g = _c.average(ranks)
        if c < 1.0:
            _c.scale(g, c)
        p, m, v = p0.copy(), m0.copy(), v0.copy()
        _c.adam(hp, g, p, m, v)
        return p, m, v

    p, m, v = p0.copy(), m0.copy(), v0.copy()
    out = np.empty(k, np.uint16)
    _c.rank_step(hp, ranks, clip, p, m, v, out)
    pe, me, ve = chain(clip)
    for got, want in ((p, pe), (m, me), (v, ve)):
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert np.array_equal(out, _c.f32_to_bf16(pe))
    # the cast is of the new master, and a coefficient below 1 changes the step
    assert (out != _c.f32_to_bf16(p0)).mean() > 0.5
    if clip < 1.0:
        assert not np.array_equal(pe, chain(1.0)[0])
