"""Pins of the oracle's flat-buffer layout.

  * Brute force on tiny inputs: every flat index of the padded buffer has
    exactly one (rank, unit, local) owner, the owned ranges of the N ranks
    tile each unit, and each rank owns L_u / N elements of unit u ("each rank
    keeps and updates only its own 1/N", "dp-zero-fsdp", concepts).
  * Padding is minimal: n_u <= L_u < n_u + N, L_u a multiple of N.
  * The Llama-70B unit table (hidden 8192, FFN 28672, 64 q / 8 kv heads of
    128, vocabulary 128256, 80 layers, untied embedding and head) gives
    70,553,706,496 parameters and 1,102,401,664 per rank at N = 64; at 16
    bytes per parameter that is the ~17.5 GB per GPU of "Data Parallel, ZeRO
    and FSDP", section "70B model, full shard" (which rounds Psi to 70e9).
"""
import itertools

import pytest

from oracle import closed_forms as cf
from oracle.layout import owner_of, padding_mask, plan
from synthetic import llama70b_units

CASES = [([1], 1), ([5], 2), ([7, 1, 0, 9], 3), ([16], 4), ([13, 27, 2], 4), ([3, 3, 3], 8),
         ([100, 1, 64], 64)]


@pytest.mark.parametrize("units,n", CASES)
def test_every_flat_index_has_one_owner(units, n):
    lays = [plan(units, n, r) for r in range(n)]
    P = lays[0].flat_len
    seen = {}
    for r, lay in enumerate(lays):
        for u, U in enumerate(lay.units):
            b, e = lay.owned(u)
            assert e - b == U.shard
            for j, f in enumerate(range(b, e)):
                assert f not in seen
                seen[f] = (r, u, j)
                assert owner_of(lay, f) == (r, u, j)
    assert sorted(seen) == list(range(P))


@pytest.mark.parametrize("units,n", CASES)
def test_padding_is_minimal_and_at_unit_tails(units, n):
    lay = plan(units, n, 0)
    mask = padding_mask(lay)
    assert len(mask) == lay.flat_len
    for U, nu in zip(lay.units, units):
        assert U.padded % n == 0 and nu <= U.padded < nu + n
        assert U.shard * n == U.padded
        seg = mask[U.flat_off:U.flat_off + U.padded]
        assert seg == [False] * nu + [True] * (U.padded - nu)
    assert lay.shard_len * n == lay.flat_len


@pytest.mark.parametrize("units", [[10], [3, 9, 1]])
def test_ddp_is_one_unsharded_replica(units):
    for r in range(4):
        lay = plan(units, 4, r, sharded=False)
        assert lay.flat_len == sum(units) == lay.shard_len
        assert [lay.owned(u) for u in range(len(units))] == \
               [(U.flat_off, U.flat_off + U.numel) for U in lay.units]


def test_llama70b_unit_table():
    units = llama70b_units()
    assert len(units) == 81
    assert sum(units) == 70_553_706_496
    lay = plan(units, 64, 63)
    assert all(U.padded == U.numel for U in lay.units)        # all multiples of 64
    assert lay.units[0].shard == 13_369_600 and lay.units[80].shard == 32_833_664
    assert lay.shard_len == 1_102_401_664
    gb = float(cf.gb(16 * lay.shard_len))
    assert abs(gb - 17.5) < 0.2


def test_gpt2_buckets_and_7b_shard():
    lay = plan([25_000_000] * 4 + [24_439_808], 8, 3)
    assert lay.flat_len == 124_439_808
    assert [U.shard for U in lay.units] == [3_125_000] * 4 + [3_054_976]
    assert lay.shard_len == 15_554_976
    lay = plan([7_240_000_000], 8, 7)
    assert lay.shard_len == 905_000_000 and lay.owned(0) == (6_335_000_000, 7_240_000_000)
