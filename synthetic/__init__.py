"""Seeded synthetic workloads shared by the tests, the smoke check and the
benchmark.  It holds the workload shapes and the random draws only -- none of
the optimizer's arithmetic -- and imports neither the HIP binding nor the
oracle.

Every draw comes from its own torch.Generator seeded by
    seed = ((((cfg * 16 + kind) * 1024 + step) * 128 + rank) * 128 + unit)
with kind 0 = gradient, 1 = master init, 2 = outlier mask, 3 = micro-batch
gradient (the micro-batch index rides in `unit`), 4 = a peer's parameter
shard for the gather.  CPU and GPU generators give
different streams for one seed, so a test draws on one device and copies the
bits to the other.

Workloads (sizes from the pages' model scales; the optimizer step depends only
on parameter counts and unit shapes, never on data, so synthetic draws stand
in for the pages' Mistral-7B / Alpaca fine-tune and for the GPT-2-small and
Llama-70B shapes):
  0  tiny ZeRO-2 shard step: Psi = 2^20, N = 4, one unit
  1  GPT-2-small flat buffer: Psi = 124,439,808, N = 8, 25M-element buckets
  2  Mistral-7B ZeRO-3 rank shard: Psi = 7.24e9, N = 8, shard 905,000,000
  3  Megatron distributed optimizer, Psi = 7.24e9, N = 8, 4 micro-batches
  4  Llama-70B FSDP full shard, N = 64, 80 layer units + 1 root unit
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import torch

# --------------------------------------------------------------- shapes --

LLAMA70B_HIDDEN = 8192
LLAMA70B_FFN = 28672
LLAMA70B_QHEADS, LLAMA70B_KVHEADS, LLAMA70B_HEAD = 64, 8, 128
LLAMA70B_VOCAB = 128256
LLAMA70B_LAYERS = 80


def llama70b_units() -> List[int]:
    """Per-layer FSDP units (q, k, v, o, gate, up, down, two RMSNorm weights)
    followed by the root unit (token embedding, final norm, untied lm_head)."""
    h, f = LLAMA70B_HIDDEN, LLAMA70B_FFN
    kv = LLAMA70B_KVHEADS * LLAMA70B_HEAD
    q = LLAMA70B_QHEADS * LLAMA70B_HEAD
    layer = h * q + 2 * h * kv + q * h + 3 * h * f + 2 * h
    root = 2 * LLAMA70B_VOCAB * h + h
    return [layer] * LLAMA70B_LAYERS + [root]


MISTRAL7B_HIDDEN, MISTRAL7B_FFN, MISTRAL7B_KV, MISTRAL7B_VOCAB, MISTRAL7B_LAYERS = (
    4096, 14336, 1024, 32000, 32)


def mistral7b_shapes() -> List[Tuple[int, int]]:
    """(rows, cols) of every Mistral-7B parameter in module order (dim 0 =
    output features; 1-D norm weights are (H, 1)): embedding, 32 x (input
    norm, q, k, v, o, post-attention norm, gate, up, down), final norm,
    untied lm_head.  7,241,732,096 elements."""
    h, f, kv, V = MISTRAL7B_HIDDEN, MISTRAL7B_FFN, MISTRAL7B_KV, MISTRAL7B_VOCAB
    layer = [(h, 1), (h, h), (kv, h), (kv, h), (h, h), (h, 1), (f, h), (f, h), (h, f)]
    return [(V, h)] + layer * MISTRAL7B_LAYERS + [(h, 1), (V, h)]


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    strategy: str
    n_ranks: int
    units: Tuple[int, ...]
    steps: int
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    decoupled: bool = False
    max_grad_norm: Optional[float] = None
    grad_std: float = 1e-3
    master_std: float = 0.02
    outlier_frac: float = 0.0
    outlier_scale: float = 100.0
    micro_batches: int = 1
    grad_dtype: str = "bf16"          # dtype of the buffers that are reduced
    grads_full_flat: bool = True      # rank grads indexed over the full buffer

    @property
    def psi(self) -> int:
        return sum(self.units)


WORKLOADS = {
    0: Workload(0, "tiny ZeRO-2 shard step (Psi=2^20, N=4)", "zero2", 4,
                (1 << 20,), 10),
    1: Workload(1, "GPT-2-small flat buffer (Psi=124,439,808, N=8, 25M buckets)",
                "zero2", 8, (25_000_000,) * 4 + (24_439_808,), 5,
                weight_decay=0.01, decoupled=True, max_grad_norm=1.0,
                outlier_frac=0.01),
    2: Workload(2, "Mistral-7B ZeRO-3 rank shard (Psi=7.24e9, N=8)", "zero3", 8,
                (7_240_000_000,), 3, grads_full_flat=False),
    3: Workload(3, "Megatron distributed optimizer (Psi=7.24e9, N=8, 4 micro-batches)",
                "megatron_do", 8, (7_240_000_000,), 1, micro_batches=4,
                grad_dtype="fp32", grads_full_flat=False),
    4: Workload(4, "Llama-70B FSDP full shard (N=64, 80 layers + root)", "fsdp", 64,
                tuple(llama70b_units()), 1, grads_full_flat=False),
}

# ---------------------------------------------------------------- draws --

KIND_GRAD, KIND_MASTER, KIND_OUTLIER, KIND_MICRO, KIND_PEER = 0, 1, 2, 3, 4


def seed(cfg: int, kind: int, step: int, rank: int, unit: int = 0) -> int:
    return ((((cfg * 16 + kind) * 1024 + step) * 128 + rank) * 128 + unit)


def _gen(s: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def normal_f32(n: int, std: float, s: int, device="cpu") -> torch.Tensor:
    x = torch.randn(n, generator=_gen(s, device), device=device, dtype=torch.float32)
    return x.mul_(std)


def to_bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """bf16 bit patterns (int16 view) of a float32 tensor, via torch's cast."""
    return x.to(torch.bfloat16).view(torch.int16)


def grad_bits(w: Workload, step: int, rank: int, n: int, device="cpu",
              unit: int = 0, kind: int = KIND_GRAD) -> torch.Tensor:
    """One rank's gradient draw of n elements as bf16 bits (int16 tensor):
    N(0, grad_std), and for workloads with outliers an independent
    Bernoulli(outlier_frac) mask whose entries are scaled by outlier_scale
    before the single rounding to bf16."""
    x = normal_f32(n, w.grad_std, seed(w.cfg, kind, step, rank, unit), device)
    if w.outlier_frac > 0:
        u = torch.rand(n, generator=_gen(seed(w.cfg, KIND_OUTLIER, step, rank, unit), device),
                       device=device)
        x = torch.where(u < w.outlier_frac, x * w.outlier_scale, x)
    return to_bf16_bits(x)


def peer_bits(w: Workload, rank: int, n: int, device="cpu", unit: int = 0) -> torch.Tensor:
    """A peer rank's parameter shard for the gather: n uniformly random
    16-bit patterns (int16 tensor; every bf16 pattern, NaNs and Infs
    included, is equally likely), distinct per rank and unit."""
    g = _gen(seed(w.cfg, KIND_PEER, 0, rank, unit), device)
    return torch.randint(-32768, 32768, (n,), generator=g, device=device, dtype=torch.int16)


def master_init(w: Workload, n: int, device="cpu", rank: int = 0, unit: int = 0) -> torch.Tensor:
    return normal_f32(n, w.master_std, seed(w.cfg, KIND_MASTER, 0, rank, unit), device)


def small_workload(units, n_ranks: int, strategy: str = "zero2", steps: int = 3,
                   cfg: int = 15, **kw) -> Workload:
    """A test-sized workload with the same draw recipe."""
    return Workload(cfg, f"test {strategy} N={n_ranks} units={list(units)}", strategy,
                    n_ranks, tuple(int(u) for u in units), steps, **kw)
