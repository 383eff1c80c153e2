"""Pins of the oracle's accounting to the numbers the pages print.

Three independent things must agree:
  1. the pages' printed values (tests/golden/*.txt, each with its citation);
  2. the closed-form functions in oracle.closed_forms;
  3. what the strategy simulation actually holds (bytes of the buffers each
     simulated rank keeps) and moves (its collective log), and what a
     hop-by-hop ring simulation sends.
"""
from fractions import Fraction as Fr

import numpy as np
import pytest

from conftest import load_golden
from oracle import closed_forms as cf
from oracle import ring, strategies

STRATS = ["ddp", "zero1", "zero1_allreduce", "zero2", "zero3", "fsdp", "megatron_do"]


def test_worked_example_7b_n8_memory():
    g = load_golden("worked_example_7b_n8.txt")
    psi, n = int(g["psi"]), int(g["n"])
    gb = lambda s: cf.gb(cf.model_state_bytes(s, psi, n))
    assert gb("ddp") == Fr(g["ddp_gb"]).limit_denominator()
    assert gb("zero1") == Fr(str(g["zero1_gb"]))
    assert gb("zero2") == Fr(str(g["zero2_gb"]))
    assert gb("zero3") == Fr(str(g["zero3_gb"]))
    assert gb("fsdp") == Fr(str(g["fsdp_gb"]))
    assert gb("megatron_do") == Fr(str(g["megatron_do_gb"]))
    assert cf.gb(cf.megatron_unsharded_bytes(psi)) == Fr(str(g["megatron_unsharded_gb"]))
    # the page splits each entry into the replicated and the 1/N part
    assert cf.gb(4 * psi) == Fr(str(g["zero1_replicated_gb"]))
    assert cf.gb(Fr(12 * psi, n)) == Fr(str(g["zero1_sharded_gb"]))
    assert cf.gb(2 * psi) == Fr(str(g["zero2_replicated_gb"]))
    assert cf.gb(Fr(14 * psi, n)) == Fr(str(g["zero2_sharded_gb"]))
    assert cf.gb(6 * psi) == Fr(str(g["megatron_do_replicated_gb"]))
    assert cf.gb(Fr(12 * psi, n)) == Fr(str(g["megatron_do_sharded_gb"]))


def test_worked_example_7b_n8_communication():
    g = load_golden("worked_example_7b_n8.txt")
    for s in STRATS:
        assert cf.comm_elements(s, 1) == int(g[f"{s}_comm_psi"]), s


def test_k8ai_full_shard_and_ring():
    g = load_golden("data_parallel_k8ai.txt")
    psi = int(g["full_shard_psi"])
    # 16 x 70e9 / 64 ~ 17.5 GB; at N = 8, 140 GB
    assert cf.gb(cf.model_state_bytes("fsdp", psi, int(g["full_shard_n64"]))) == Fr(str(g["full_shard_n64_gb"]))
    assert cf.gb(cf.model_state_bytes("fsdp", psi, int(g["full_shard_n8"]))) == int(g["full_shard_n8_gb"])
    assert cf.model_state_bytes("ddp", 1, 1) == int(g["bytes_per_param"])
    assert Fr(cf.comm_elements("zero3", 1), cf.comm_elements("ddp", 1)) == Fr(str(g["zero3_vs_ddp"]))
    S = int(g["ring_psi"]) * int(g["ring_bytes_per_param"])
    assert cf.gb(S) == int(g["ring_s_gb"])
    # exact expression at N = 8 is 24.5 GB; the page's 28 GB is the large-N limit
    assert cf.gb(cf.ring_allreduce_bytes_per_gpu(S, 8)) == Fr("24.5")
    assert cf.gb(cf.ring_allreduce_bytes_per_gpu(S, 10 ** 9)) < int(g["ring_limit_gb"])
    assert int(g["ring_limit_gb"]) - cf.gb(cf.ring_allreduce_bytes_per_gpu(S, 10 ** 6)) < Fr(1, 1000)


def test_page1_mistral_accounting():
    """Page 1 counts 2 + 2 + 8 bytes (no fp32 master): reproduce its
    roundings with Mistral's parameter count."""
    g = load_golden("what_each_gpu_holds_mistral7b.txt")
    psi = g["psi"]
    params, grads, mv = 2 * psi / 1e9, 2 * psi / 1e9, 8 * psi / 1e9
    assert round(params) == g["params_gb_approx"]
    assert round(grads) == g["grads_gb_approx"]
    assert round(mv) == g["adam_mv_gb_approx"]
    assert round(params + grads + mv) == g["total_gb_approx"]
    assert round(g["total_gb_approx"] / g["fsdp_n"]) == g["fsdp_per_gpu_gb_approx"]


@pytest.mark.parametrize("strategy", STRATS)
@pytest.mark.parametrize("n", [2, 4, 8])
def test_simulated_ranks_hold_the_closed_form_bytes(strategy, n):
    """The buffers each simulated rank keeps between steps add up to the
    pages' closed form (Psi a multiple of N so there is no padding)."""
    psi = 96 * n
    cl = strategies.make_cluster(strategy, [psi], n, np.zeros(psi, np.float32))
    for R in cl.ranks:
        assert R.model_state_bytes() == cf.model_state_bytes(strategy, psi, n)


@pytest.mark.parametrize("strategy", STRATS)
def test_simulated_collectives_move_the_closed_form_volume(strategy):
    n, psi = 4, 64
    cl = strategies.make_cluster(strategy, [psi], n, np.zeros(psi, np.float32))
    cfg = strategies.AdamConfig()
    zeros = np.zeros(psi, np.uint16)
    grads = [[zeros] if strategy == "megatron_do" else zeros for _ in range(n)]
    strategies.step(cl, cfg, 1, grads)
    assert strategies.comm_elements_per_step(cl) == cf.comm_elements(strategy, psi)


@pytest.mark.parametrize("n", [2, 3, 4, 8])
def test_ring_simulation_sends_2_n_minus_1_over_n(n):
    P = 24 * n
    rng = np.random.default_rng(n)
    # multiples of 2^-12 of modest size: every fp32 partial sum is exact, so
    # the ring's rotated order gives the exact sum
    bufs = [(rng.integers(-512, 512, P) * 2.0 ** -12).astype(np.float32) for _ in range(n)]
    full, sent = ring.all_reduce(bufs)
    exact = sum(b.astype(np.float64) for b in bufs)
    for q in range(n):
        assert np.array_equal(full[q].astype(np.float64), exact)
        assert Fr(sent[q]) == cf.ring_allreduce_bytes_per_gpu(P * 4, n)
    # bus bandwidth: per-GPU bytes / S is exactly the busbw factor
    assert Fr(sent[0], P * 4) == cf.busbw(1, n)
    # all-reduce == reduce-scatter then all-gather, and reduce-scatter leaves
    # rank q with chunk q of the sum
    red, sent_rs = ring.reduce_scatter(bufs)
    c = P // n
    for q in range(n):
        assert np.array_equal(red[q].astype(np.float64), exact[q * c:(q + 1) * c])
        assert Fr(sent_rs[q]) == Fr(n - 1, n) * P * 4
