"""Pins of the FSDP linear-layer oracle (oracle/linear.py).

  * Finite differences of L = sum(Y * G) with Y = X W fix dL/dX = G W^T and
    dL/dW = X^T G independently of those formulas (central differences on
    tiny fp64 inputs; L is linear in each operand, so the difference is exact
    up to rounding).
  * Data parallelism over the batch: sum_q X_q^T dY_q = [X_0; ...]^T [dY_0; ...]
    and the reduce-scattered rows tile the mean gradient exactly once.
  * The all-gather of torch.chunk row shards rebuilds W.
"""
import numpy as np
import torch

from oracle import linear
from oracle.layout import plan_rows


def test_gradients_match_finite_differences():
    rng = np.random.default_rng(0)
    b, i, o = 3, 5, 4
    x, w, g = rng.standard_normal((b, i)), rng.standard_normal((i, o)), rng.standard_normal((b, o))
    loss = lambda x_, w_: float(np.sum(linear.forward(w_, x_) * g))
    dx, dw = linear.backward(w, x, g)
    h = 1e-3
    for (p, q) in [(0, 0), (1, 3), (2, 4)]:
        e = np.zeros_like(x); e[p, q] = h
        fd = (loss(x + e, w) - loss(x - e, w)) / (2 * h)
        assert abs(fd - dx[p, q]) < 1e-9
    for (p, q) in [(0, 0), (4, 3), (2, 1)]:
        e = np.zeros_like(w); e[p, q] = h
        fd = (loss(x, w + e) - loss(x, w - e)) / (2 * h)
        assert abs(fd - dw[p, q]) < 1e-9


def test_data_parallel_identity_and_reduce_scatter_tiling():
    rng = np.random.default_rng(1)
    n, b, i, o = 4, 6, 10, 7
    xs = [rng.standard_normal((b, i)) for _ in range(n)]
    dys = [rng.standard_normal((b, o)) for _ in range(n)]
    w = rng.standard_normal((i, o))
    dws = [linear.backward(w, xq, dq)[1] for xq, dq in zip(xs, dys)]
    whole = np.concatenate(xs).T @ np.concatenate(dys)
    assert np.allclose(sum(dws), whole, rtol=0, atol=1e-12)
    parts = [linear.reduce_scatter_mean(plan_rows([(i, o)], n, r), dws, o) for r in range(n)]
    c = parts[0].shape[0]
    stacked = np.concatenate(parts)
    assert np.allclose(stacked[:i], whole / n, rtol=0, atol=1e-12)
    assert not stacked[i:].any()          # padding rows stay zero
    assert c == -(-i // n)


def test_gather_rebuilds_w_from_torch_chunk_shards():
    n, i, o = 4, 10, 3
    w = np.arange(i * o, dtype=np.float64).reshape(i, o)
    lay = plan_rows([(i, o)], n, 0)
    c = lay.units[0].shard // o
    shards = []
    for ch in torch.chunk(torch.from_numpy(w), n, dim=0):
        pad = np.zeros((c, o)); pad[:ch.shape[0]] = ch.numpy()
        shards.append(pad)
    while len(shards) < n:
        shards.append(np.zeros((c, o)))
    assert np.array_equal(linear.gather_rows(lay, shards, i, o), w)


def test_gemm_bound_covers_fp32_accumulation():
    rng = np.random.default_rng(2)
    a = rng.standard_normal((16, 3000)).astype(np.float32)
    b = rng.standard_normal((3000, 16)).astype(np.float32)
    exact = a.astype(np.float64) @ b.astype(np.float64)
    acc = np.zeros((16, 16), np.float32)
    for k in range(3000):                       # naive sequential fp32 accumulation
        acc = (acc + np.outer(a[:, k], b[k, :]).astype(np.float32)).astype(np.float32)
    assert np.all(np.abs(acc - exact) <= linear.gemm_bound(a.astype(np.float64),
                                                           b.astype(np.float64)))
