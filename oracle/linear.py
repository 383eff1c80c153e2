"""A hand-written FSDP linear layer, from one rank's point of view, on N
simulated ranks ("dp-zero-fsdp", follow-up on writing one FSDP linear layer
by hand): each rank stores 1/N of the rows of W; forward all-gathers the
full W, computes X W for its local batch and frees W; backward all-gathers
W again to compute dX, computes the full-shape dW locally and
reduce-scatters it so each rank keeps its 1/N of the rows.

Readings taken:
  * W is (in_features x out_features), Y = X W as the page writes it; the
    rows of W (in_features) are sharded FSDP2-style: torch.chunk rows per
    rank, zero-padded to ceil(in / N) rows (oracle.layout.plan_rows).
  * The reduce-scatter averages over the N ranks (like the data-parallel
    gradient average).
  * Arithmetic is exact (fp64 on bf16-valued inputs: every product is exact
    and the sums have far more precision than the fp32 being checked); the
    comparison against an fp32-accumulating implementation uses the
    standard bound |fl(sum) - sum| <= gamma_K sum |a_k b_k|.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).
"""
from typing import List, Sequence

import numpy as np

from . import _c
from .layout import Layout


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact fp64 values."""
    return _c.bf16_to_f32(np.ascontiguousarray(bits, np.uint16)).astype(np.float64)


def gather_rows(lay: Layout, shards: Sequence[np.ndarray], rows: int, cols: int) -> np.ndarray:
    """All-gather of the row shards (each c x cols) into the full rows x cols
    matrix (padding rows dropped)."""
    c = lay.units[0].shard // cols
    full = np.concatenate([np.asarray(s).reshape(c, cols) for s in shards], axis=0)
    return full[:rows]


def forward(w_full: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Y = X W, exact."""
    return x @ w_full


def backward(w_full: np.ndarray, x: np.ndarray, dy: np.ndarray):
    """(dX, dW) of L with dL/dY = dY: dX = dY W^T, dW = X^T dY, exact."""
    return dy @ w_full.T, x.T @ dy


def reduce_scatter_mean(lay: Layout, dws: Sequence[np.ndarray], cols: int) -> np.ndarray:
    """Rank lay.rank's rows of (sum_q dW_q) / N, padded to its c rows."""
    n = lay.n_ranks
    c = lay.units[0].shard // cols
    rows = dws[0].shape[0]
    total = sum(dws) / n
    out = np.zeros((c, cols))
    first = lay.rank * c
    take = max(0, min(c, rows - first))
    out[:take] = total[first:first + take]
    return out


def gamma(k: int) -> float:
    u = 2.0 ** -24
    return k * u / (1 - k * u)


def gemm_bound(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Elementwise bound on |fl32(A B) - A B| for fp32 accumulation of K
    exact products (any order): gamma_K (|A| |B|)."""
    return gamma(a.shape[1]) * (np.abs(a) @ np.abs(b))
