"""FSDP2 per-parameter dim-0 sharding in the oracle.

Pins:
  * rank r's rows of a parameter are exactly torch.chunk(param, N, dim=0)[r]
    (a library routine; ranks past the last chunk hold nothing), and the
    padded slices tile every parameter once;
  * FSDP2 gives bit-identical parameters and state to DDP (the strategy only
    changes who holds what, "dp-zero-fsdp", follow-up "FSDP2 vs FSDP1");
  * each rank's held bytes are 16 Psi / N when N divides every row count.
"""
import numpy as np
import pytest
import torch

from oracle import closed_forms as cf
from oracle import strategies
from oracle.layout import plan_rows, valid_rows

SHAPES = [[(10, 3)], [(9, 4), (1, 5), (0, 2), (17, 1)], [(64, 8), (8, 64), (7, 7)],
          [(128256 // 512, 16), (3, 1024)]]


@pytest.mark.parametrize("shapes", SHAPES)
@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 16])
def test_rows_match_torch_chunk(shapes, n):
    owners = {}
    for r in range(n):
        lay = plan_rows(shapes, n, r)
        for u, ((rows, cols), U) in enumerate(zip(shapes, lay.units)):
            param = torch.arange(rows * cols).reshape(rows, cols)
            chunks = torch.chunk(param, n, dim=0) if rows else ()
            first, cnt = valid_rows(lay, u)
            want = chunks[r].reshape(-1).tolist() if r < len(chunks) else []
            got = list(range(first * cols, (first + cnt) * cols))
            assert got == want, (shapes, n, r, u)
            b, e = lay.owned(u)
            assert e - b == U.shard and U.shard * n == U.padded
            for f in range(b, e):
                assert f not in owners
                owners[f] = (r, u)
    assert sorted(owners) == list(range(plan_rows(shapes, n, 0).flat_len))


def test_fsdp2_equals_ddp_bit_exact():
    shapes = [(9, 4), (1, 5), (17, 3), (12, 8)]
    n = 4
    psi = sum(r * c for r, c in shapes)
    rng = np.random.default_rng(0)
    master = (rng.standard_normal(psi) * 0.02).astype(np.float32)
    from oracle import _c
    cfg = strategies.AdamConfig(weight_decay=0.01, decoupled=True, max_grad_norm=0.01)
    ddp = strategies.make_cluster("ddp", [psi], n, master)
    f2 = strategies.make_cluster("fsdp2", shapes, n, master)
    for t in range(3):
        grads = [_c.f32_to_bf16((rng.standard_normal(psi) * 1e-3).astype(np.float32))
                 for _ in range(n)]
        strategies.step(ddp, cfg, t + 1, grads)
        strategies.step(f2, cfg, t + 1, grads)
    assert np.array_equal(strategies.full_params(ddp), strategies.full_params(f2))
    a, b = strategies.full_state(ddp), strategies.full_state(f2)
    for k in ("master", "m", "v"):
        assert np.array_equal(a[k], b[k])


def test_fsdp2_rank_holds_16_psi_over_n():
    shapes = [(8, 3), (16, 5)]
    psi = sum(r * c for r, c in shapes)
    cl = strategies.make_cluster("fsdp2", shapes, 8, np.zeros(psi, np.float32))
    for R in cl.ranks:
        assert R.model_state_bytes() == cf.model_state_bytes("fsdp2", psi, 8)
