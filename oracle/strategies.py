"""One optimizer step of N simulated data-parallel ranks under DDP, ZeRO-1/2/3,
FSDP and the Megatron distributed optimizer, on numpy buffers.

The arithmetic is the plain definition: average the N ranks' gradients, take
one Adam step on the fp32 master state, round to bf16, lay the result out in
the flat buffer.  Sharding changes who computes an element and where it is
stored, never its value:
  * DDP: a full replica per GPU; the mean of the rank gradients reaches
    every replica and all of them apply the same optimizer step ("Data
    Parallel, ZeRO and FSDP", section "Plain data parallel (DDP)"; "Behind
    the scenes...", section on DDP).
  * all-reduce = reduce-scatter (sum, each GPU keeps its 1/N) + all-gather
    (concatenate the 1/N slices) ("dp-zero-fsdp", concepts; "Behind the
    scenes...", section "ZeRO: The Dial Between DDP and FSDP").
  * ZeRO-1 shards the optimizer state, ZeRO-2 also the gradients, ZeRO-3 also
    the parameters; FSDP is PyTorch's ZeRO-3 ("dp-zero-fsdp", concepts).
  * Megatron distributed optimizer: bf16 params and fp32 gradients (summed in
    fp32) replicated, fp32 main param / m / v sharded ("dp-zero-fsdp",
    worked example, the note under the Megatron row).

Each rank object holds exactly the model-state buffers that its strategy
keeps between steps, so `model_state_bytes()` can be checked against the
pages' closed forms, and every collective appends its per-GPU volume in
elements to a log, counted the pages' way (an all-reduce of P elements is
P + P, a reduce-scatter P, an all-gather P; "dp-zero-fsdp", derivation of the
per-GPU communication volume).
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

from . import _c
from .layout import Layout, plan, plan_rows

STRATEGIES = ("ddp", "zero1", "zero1_allreduce", "zero2", "zero3", "fsdp", "fsdp2", "megatron_do")
SHARDED_PARAMS = ("zero3", "fsdp", "fsdp2")


@dataclass
class AdamConfig:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    decoupled: bool = False          # True = AdamW
    max_grad_norm: Optional[float] = None

    def hparams(self, step: int):
        return _c.hparams(self.lr, self.beta1, self.beta2, self.eps,
                          self.weight_decay, step, self.decoupled)


@dataclass
class RankState:
    params: np.ndarray                    # bf16 bits; full or shard
    grads: Optional[np.ndarray]           # bf16 bits or fp32; full or shard
    master: np.ndarray                    # fp32 master (shard unless DDP)
    m: np.ndarray
    v: np.ndarray

    def model_state_bytes(self) -> int:
        arrays = [self.params, self.grads, self.master, self.m, self.v]
        return int(sum(a.nbytes for a in arrays if a is not None))


@dataclass
class Cluster:
    strategy: str
    layouts: List[Layout]                 # one per rank
    ranks: List[RankState]
    comm_log: List = field(default_factory=list)

    @property
    def n(self) -> int:
        return len(self.ranks)


def pad(lay: Layout, x: np.ndarray) -> np.ndarray:
    """Model-order buffer (sum of n_u) -> padded flat buffer (zeros at each
    unit's tail)."""
    out = np.zeros(lay.flat_len, x.dtype)
    o = 0
    for U in lay.units:
        out[U.flat_off:U.flat_off + U.numel] = x[o:o + U.numel]
        o += U.numel
    assert o == x.size
    return out


def unpad(lay: Layout, full: np.ndarray) -> np.ndarray:
    return np.concatenate([full[U.flat_off:U.flat_off + U.numel] for U in lay.units])


def _shard_of(full: np.ndarray, lay: Layout) -> np.ndarray:
    """The rank's owned elements of a full flat buffer, unit by unit."""
    return np.concatenate([full[b:b + n] for b, _, n in lay.owned_runs()])


def _place(full: np.ndarray, lay: Layout, shard: np.ndarray) -> None:
    for b, s, n in lay.owned_runs():
        full[b:b + n] = shard[s:s + n]


def all_gather(layouts: Sequence[Layout], shards: Sequence[np.ndarray]) -> np.ndarray:
    """Concatenate every rank's slice into the full flat buffer."""
    full = np.empty(layouts[0].flat_len, shards[0].dtype)
    for lay, sh in zip(layouts, shards):
        _place(full, lay, sh)
    return full


def make_cluster(strategy: str, unit_numel: Sequence, n_ranks: int,
                 master0: np.ndarray) -> Cluster:
    """N ranks holding the initial state.  master0 is the fp32 master in
    model order (sum of the unit sizes, no padding); bf16 params start as its
    rounding; m = v = 0; padding positions are zero.  For "fsdp2" the units
    are (rows, cols) parameter shapes."""
    if strategy not in STRATEGIES:
        raise ValueError(strategy)
    sharded = strategy != "ddp"
    if strategy == "fsdp2":
        layouts = [plan_rows(unit_numel, n_ranks, r) for r in range(n_ranks)]
    else:
        layouts = [plan(unit_numel, n_ranks, r, sharded) for r in range(n_ranks)]
    P = layouts[0].flat_len
    assert master0.dtype == np.float32 and master0.size == sum(U.numel for U in layouts[0].units)
    master0 = pad(layouts[0], master0)
    params_full = _c.f32_to_bf16(master0)
    ranks = []
    for lay in layouts:
        if strategy == "ddp":
            master = master0.copy()
            grads = np.zeros(P, np.uint16)
            params = params_full.copy()
        else:
            master = _shard_of(master0, lay).copy()
            if strategy in ("zero1", "zero1_allreduce"):
                grads = np.zeros(P, np.uint16)
            elif strategy == "megatron_do":
                grads = np.zeros(P, np.float32)      # fp32 main_grad, full
            else:
                grads = np.zeros(lay.shard_len, np.uint16)
            params = (_shard_of(params_full, lay).copy()
                      if strategy in SHARDED_PARAMS else params_full.copy())
        ranks.append(RankState(params, grads, master,
                               np.zeros_like(master), np.zeros_like(master)))
    return Cluster(strategy, layouts, ranks)


def _clip_coefficient(cfg: AdamConfig, full_mean_grad: np.ndarray) -> float:
    """Global L2 norm over the whole averaged gradient, in flat index order."""
    if cfg.max_grad_norm is None or cfg.max_grad_norm <= 0:
        return 1.0
    return _c.clip_coef(_c.sumsq(full_mean_grad), cfg.max_grad_norm)


def step(cl: Cluster, cfg: AdamConfig, t: int, grads: Sequence, micro: int = 1) -> None:
    """One optimizer step of every rank.

    grads[q] is rank q's full gradient from its backward pass, in model
    order (bf16 bits, no padding), or, for the Megatron distributed
    optimizer, a list of `micro` such arrays (one per micro-batch), which are
    summed into the fp32 main gradient first.
    """
    N, s, lay0 = cl.n, cl.strategy, cl.layouts[0]
    P = lay0.flat_len
    hp = cfg.hparams(t)

    if s == "megatron_do":
        for q in range(N):
            cl.ranks[q].grads[:] = 0.0
            for k in range(micro):
                _c.accumulate_bf16(cl.ranks[q].grads, pad(lay0, grads[q][k]))
        full_grads = [cl.ranks[q].grads for q in range(N)]
    else:
        full_grads = [pad(lay0, np.ascontiguousarray(g)) for g in grads]
        assert all(g.dtype == np.uint16 and g.size == P for g in full_grads)

    if s == "ddp":
        # all-reduce: every replica receives the same average
        cl.comm_log.append(("all_reduce", 2 * P))
        g_mean = _c.average(full_grads)
        c = _clip_coefficient(cfg, g_mean)
        if c < 1.0:
            _c.scale(g_mean, c)
        for q in range(N):
            R = cl.ranks[q]
            R.grads[:] = full_grads[q]
            _c.adam(hp, g_mean.copy(), R.master, R.m, R.v)
            R.params[:] = _c.f32_to_bf16(R.master)
        return

    # sharded strategies: reduce-scatter of the average (ZeRO-1 may instead
    # all-reduce and keep its slice; same values)
    if s == "zero1_allreduce":
        cl.comm_log.append(("all_reduce", 2 * P))
    else:
        cl.comm_log.append(("reduce_scatter", P))
    if s in SHARDED_PARAMS:
        # forward and backward each all-gather the parameters once
        cl.comm_log.append(("all_gather_forward", P))
        cl.comm_log.append(("all_gather_backward", P))
    g_mean_full = _c.average(full_grads)
    shards = [_shard_of(g_mean_full, lay) for lay in cl.layouts]
    c = _clip_coefficient(cfg, g_mean_full)
    new_param_shards = []
    for q in range(N):
        R, lay = cl.ranks[q], cl.layouts[q]
        g = shards[q]
        if c < 1.0:
            _c.scale(g, c)
        if s in ("zero1", "zero1_allreduce"):
            R.grads[:] = full_grads[q]
        elif s != "megatron_do":
            R.grads[:] = _shard_of(full_grads[q], lay)
        _c.adam(hp, g, R.master, R.m, R.v)
        new_param_shards.append(_c.f32_to_bf16(R.master))
    if s in SHARDED_PARAMS:
        for q in range(N):
            cl.ranks[q].params[:] = new_param_shards[q]
    else:
        cl.comm_log.append(("all_gather", P))
        full = all_gather(cl.layouts, new_param_shards)
        for q in range(N):
            cl.ranks[q].params[:] = full


def full_params(cl: Cluster, q: int = 0, padded: bool = False) -> np.ndarray:
    """Rank q's view of the full bf16 parameter buffer (gathered, not logged,
    for ZeRO-3 / FSDP), in model order unless `padded`."""
    if cl.strategy in SHARDED_PARAMS:
        full = all_gather(cl.layouts, [R.params for R in cl.ranks])
    else:
        full = cl.ranks[q].params.copy()
    return full if padded else unpad(cl.layouts[0], full)


def full_state(cl: Cluster, padded: bool = False) -> Dict[str, np.ndarray]:
    """master / m / v over the whole buffer, in model order unless `padded`."""
    if cl.strategy == "ddp":
        R = cl.ranks[0]
        out = {"master": R.master.copy(), "m": R.m.copy(), "v": R.v.copy()}
    else:
        out = {k: all_gather(cl.layouts, [getattr(R, k) for R in cl.ranks])
               for k in ("master", "m", "v")}
    return out if padded else {k: unpad(cl.layouts[0], x) for k, x in out.items()}


def comm_elements_per_step(cl: Cluster, steps: int = 1) -> int:
    return sum(n for _, n in cl.comm_log) // steps
