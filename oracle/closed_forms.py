"""The pages' closed forms for per-GPU model-state bytes and per-GPU
communication volume, as exact rationals.

  * Mixed-precision Adam keeps 16 bytes per parameter: bf16 param 2 + bf16
    grad 2 + fp32 master, m, v 12 ("dp-zero-fsdp", concepts, "Model states:
    16 Psi bytes").
  * Per-GPU bytes: DDP 16 Psi; ZeRO-1 4 Psi + 12 Psi/N; ZeRO-2 2 Psi +
    14 Psi/N; ZeRO-3 / FSDP 16 Psi/N; Megatron distributed optimizer
    6 Psi + 12 Psi/N, and 18 Psi unsharded ("dp-zero-fsdp", figure 1 and
    worked example "7B, N = 8"; "Data Parallel, ZeRO and FSDP", ZeRO/FSDP
    table).
  * Per-GPU communication in elements: DDP 2 Psi; ZeRO-2 reduce-scatter Psi +
    all-gather Psi = 2 Psi; ZeRO-3 / FSDP 3 Psi = 1.5x DDP; ZeRO-1 2 Psi with
    a reduce-scatter, 3 Psi if it all-reduces the gradients
    ("dp-zero-fsdp", derivation and follow-up on ZeRO-1 vs ZeRO-2).
  * Ring all-reduce bytes per GPU 2 (N-1)/N x S ("Data Parallel, ZeRO and
    FSDP", section "Communication cost").

These are the pages' formulas, checked in the tests against the numbers the
pages print and against the buffers the strategy simulation actually holds
and moves.  1 GB = 1e9 bytes.
"""
from fractions import Fraction as Fr

MODEL_STATE_BYTES = {
    "ddp": lambda psi, n: 16 * psi,
    "zero1": lambda psi, n: 4 * psi + Fr(12 * psi, n),
    "zero1_allreduce": lambda psi, n: 4 * psi + Fr(12 * psi, n),
    "zero2": lambda psi, n: 2 * psi + Fr(14 * psi, n),
    "zero3": lambda psi, n: Fr(16 * psi, n),
    "fsdp": lambda psi, n: Fr(16 * psi, n),
    "fsdp2": lambda psi, n: Fr(16 * psi, n),
    "megatron_do": lambda psi, n: 6 * psi + Fr(12 * psi, n),
}

COMM_ELEMENTS = {
    "ddp": lambda psi: 2 * psi,
    "zero1": lambda psi: 2 * psi,
    "zero1_allreduce": lambda psi: 3 * psi,
    "zero2": lambda psi: 2 * psi,
    "zero3": lambda psi: 3 * psi,
    "fsdp": lambda psi: 3 * psi,
    "fsdp2": lambda psi: 3 * psi,
    "megatron_do": lambda psi: 2 * psi,
}


def model_state_bytes(strategy: str, psi: int, n: int) -> Fr:
    return Fr(MODEL_STATE_BYTES[strategy](psi, n))


def megatron_unsharded_bytes(psi: int) -> int:
    """bf16 param 2 + fp32 grad 4 + fp32 main param, m, v 12 = 18 per param."""
    return 18 * psi


def comm_elements(strategy: str, psi: int) -> int:
    return COMM_ELEMENTS[strategy](psi)


def ring_allreduce_bytes_per_gpu(size_bytes, n: int) -> Fr:
    return Fr(2 * (n - 1), n) * Fr(size_bytes)


def busbw(algbw, n: int) -> Fr:
    return Fr(algbw) * Fr(2 * (n - 1), n)


def gb(x) -> Fr:
    return Fr(x) / Fr(10 ** 9)
