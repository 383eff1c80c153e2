"""Structural invariants of the oracle's strategy simulation.

  * DDP all-reduce + replicated Adam and ZeRO reduce-scatter + sharded Adam +
    all-gather give identical parameters (every replica "takes the same
    optimizer step", "Data Parallel, ZeRO and FSDP", section "Plain data
    parallel (DDP)"; all-reduce = reduce-scatter + all-gather, "dp-zero-fsdp",
    concepts).  Bit-exact, for every strategy, with and without clipping.
  * Padding stays zero; every DDP replica ends identical.
  * Resuming: steps 1..k then k+1..T equal steps 1..T (the step counter is an
    input).
  * Splitting the buffer into more buckets changes nothing (the update is
    elementwise and the clip norm is taken over the whole flat buffer).
"""
import numpy as np
import pytest
import torch

from oracle import _c, strategies
from synthetic import grad_bits, master_init, small_workload

STRATS = ["ddp", "zero1", "zero1_allreduce", "zero2", "zero3", "fsdp", "megatron_do"]


def _inputs(units, n, steps, outliers=0.0, cfg=14):
    """Model-order inputs (no padding): master and per-step, per-rank grads."""
    w = small_workload(units, n, steps=steps, cfg=cfg, outlier_frac=outliers)
    P = sum(units)
    master = master_init(w, P).numpy()
    grads = [[grad_bits(w, t, q, P).numpy().view(np.uint16) for q in range(n)]
             for t in range(steps)]
    return master, grads


def _run(strategy, units, n, master, grads, cfg, t0=1, cl=None):
    cl = cl or strategies.make_cluster(strategy, units, n, master)
    for i, g in enumerate(grads):
        gg = [[x] for x in g] if strategy == "megatron_do" else g
        strategies.step(cl, cfg, t0 + i, gg)
    return cl


@pytest.mark.parametrize("clip", [None, 1e-3])
def test_all_strategies_give_identical_parameters(clip):
    units, n = [300, 41, 1000], 4
    master, grads = _inputs(units, n, 3, outliers=0.01)
    cfg = strategies.AdamConfig(weight_decay=0.01, decoupled=True, max_grad_norm=clip)
    ref = _run("ddp", units, n, master, grads, cfg)
    ref_p = strategies.full_params(ref)
    ref_s = strategies.full_state(ref)
    for q in range(n):                          # replicas stay identical
        assert np.array_equal(ref.ranks[q].params, ref_p)
    for s in STRATS[1:]:
        cl = _run(s, units, n, master, grads, cfg)
        for q in range(n):
            assert np.array_equal(strategies.full_params(cl, q), ref_p), s
        st = strategies.full_state(cl)
        for k in ("master", "m", "v"):
            assert np.array_equal(st[k], ref_s[k]), (s, k)


def test_clip_is_active_and_changes_the_result():
    units, n = [512], 4
    master, grads = _inputs(units, n, 2)
    a = _run("zero2", units, n, master, grads, strategies.AdamConfig())
    b = _run("zero2", units, n, master, grads, strategies.AdamConfig(max_grad_norm=1e-4))
    # the first moment carries the clipped gradient
    assert not np.array_equal(strategies.full_state(a)["m"], strategies.full_state(b)["m"])


def test_padding_stays_zero():
    units, n = [13, 27, 2], 4
    master, grads = _inputs(units, n, 3)
    cl = _run("zero3", units, n, master, grads, strategies.AdamConfig(weight_decay=0.1, decoupled=True))
    lay = cl.layouts[0]
    full = strategies.full_params(cl, padded=True)
    st = strategies.full_state(cl, padded=True)
    for U in lay.units:
        pad = slice(U.flat_off + U.numel, U.flat_off + U.padded)
        assert not full[pad].any() and not st["master"][pad].any()
        assert not st["m"][pad].any() and not st["v"][pad].any()


@pytest.mark.parametrize("k", [1, 2, 4])
def test_resume_equals_uninterrupted(k):
    units, n, T = [200, 56], 4, 5
    master, grads = _inputs(units, n, T)
    cfg = strategies.AdamConfig()
    full = _run("zero2", units, n, master, grads, cfg)
    part = _run("zero2", units, n, master, grads[:k], cfg)
    part = _run("zero2", units, n, master, grads[k:], cfg, t0=k + 1, cl=part)
    assert np.array_equal(strategies.full_params(full), strategies.full_params(part))


def test_bucketing_does_not_change_the_result():
    n = 4
    master, grads = _inputs([1024], n, 3)
    cfg = strategies.AdamConfig(max_grad_norm=1e-3)
    one = _run("zero2", [1024], n, master, grads, cfg)
    four = _run("zero2", [256] * 4, n, master, grads, cfg)
    assert np.array_equal(strategies.full_params(one), strategies.full_params(four))


def test_megatron_micro_batches_sum_in_fp32():
    """K micro-batch grads summed into fp32 main_grad, then averaged over
    ranks, equal DDP driven by the fp32 totals."""
    units, n, K = [96], 4, 4
    P = 96
    rng = np.random.default_rng(3)
    master = (rng.standard_normal(P) * 0.02).astype(np.float32)
    micro = [[_c.f32_to_bf16((rng.standard_normal(P) * 1e-3).astype(np.float32))
              for _ in range(K)] for _ in range(n)]
    cl = strategies.make_cluster("megatron_do", units, n, master)
    strategies.step(cl, strategies.AdamConfig(), 1, micro, micro=K)
    tot = []
    for q in range(n):
        acc = np.zeros(P, np.float32)
        for k in range(K):
            acc = (acc + _c.bf16_to_f32(micro[q][k])).astype(np.float32)
        tot.append(acc)
    g = _c.average(tot)
    p, m, v = master.copy(), np.zeros(P, np.float32), np.zeros(P, np.float32)
    _c.adam(strategies.AdamConfig().hparams(1), g, p, m, v)
    assert np.array_equal(strategies.full_params(cl), _c.f32_to_bf16(p))
