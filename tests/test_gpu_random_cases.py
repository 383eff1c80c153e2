"""GPU parity on seeded random configurations: the fused step through the
C ABI against the oracle, bit for bit, over layouts, rank counts, index
modes and both memory formats drawn together rather than one at a time.

Each case draws: 1-6 units of 0 to 20,000 elements (ragged tails, empty
units, slices that are not multiples of 4), N from 1 to 64, a sharded
strategy, Adam / AdamW / L2, a state chunk (three arrays or 4 to 8192), a
gradient chunk (one buffer per rank, or rows of 4 to 4096 elements per rank),
per-rank index modes (with a gradient chunk: every rank shard-indexed, or,
from a second generator, a random set of ranks full-indexed in buffers of
their own beside the receive buffer, at least one rank left in it), and
whole-range or per-unit calls; two steps each.
"""
import numpy as np
import pytest
import torch

from oracle import strategies
from gpu_ranks import GpuRanks, bind, draw, oracle_cfg
from synthetic import small_workload

pytestmark = pytest.mark.gpu
zs = None


def setup_module(module):
    global zs
    from fsdp_sharded_optimizer_shard_amd import zs as _zs
    zs = _zs
    bind(_zs)
    assert torch.cuda.is_available()


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 16, 64]))
    units = []
    for _ in range(int(rng.integers(1, 7))):
        kind = rng.integers(0, 4)
        units.append(0 if kind == 0 else int(rng.integers(1, 100)) if kind == 1 else
                     int(rng.integers(1000, 20000)) if kind == 2 else
                     2048 * int(rng.integers(1, 5)) + int(rng.integers(-3, 4)))
    if sum(units) == 0:
        units.append(777)
    strategy = str(rng.choice(["zero1", "zero2", "zero3", "fsdp"]))
    decay = str(rng.choice(["none", "adamw", "l2"]))
    E = int(rng.choice([0, 4, 8, 64, 1024, 8192]))
    GE = int(rng.choice([0, 0, 4, 16, 256, 4096]))
    if GE:
        modes = [zs.INDEX_SHARD] * n
        alt = np.random.default_rng(5000 + seed)
        if n > 1 and alt.integers(0, 2):
            for q in alt.choice(n, int(alt.integers(1, n)), replace=False):
                modes[int(q)] = zs.INDEX_FULL
    else:
        modes = [int(x) for x in rng.choice([zs.INDEX_FULL, zs.INDEX_SHARD], n)]
    per_unit = bool(rng.integers(0, 2))
    return units, n, strategy, decay, E, GE, modes, per_unit


@pytest.mark.parametrize("seed", range(32))
def test_random_configuration(seed):
    units, n, strategy, decay, E, GE, modes, per_unit = _case(seed)
    kw = {"adamw": dict(weight_decay=0.01, decoupled=True),
          "l2": dict(weight_decay=0.1, decoupled=False)}.get(decay, {})
    w = small_workload(units, n, strategy, steps=2, cfg=40 + seed % 7, outlier_frac=0.01, **kw)
    master0, grads = draw(w, w.steps)
    oc = strategies.make_cluster(strategy, units, n, master0)
    g = GpuRanks(w, master0, oc, state_chunk=E, grad_chunk=GE)
    what = (f"seed {seed}: units {units} N={n} {strategy} {decay} E={E} GE={GE} "
            f"per_unit={per_unit}")
    for t in range(w.steps):
        strategies.step(oc, oracle_cfg(w), t + 1, grads[t])
        g.step_fused(t + 1, grads[t], modes, per_unit=per_unit)
        g.check(f"{what} step {t + 1}")
