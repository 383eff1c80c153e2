"""MI355X-native sharded mixed-precision optimizer step (ZeRO-1/2/3, FSDP,
DDP, Megatron distributed optimizer) for one data-parallel rank, behind the
C ABI in include/zero_shard.h.

    from fsdp_sharded_optimizer_shard_amd import zs
    L = zs.shard_init("zero3", world_n=8, rank=7, unit_numel=[7_240_000_000])
    zs.adam_step(L, 0, 1, zs.adam_cfg(step=1), master, m, v, params,
                 zs.INDEX_SHARD, grads=zs.Grads(rank_grads, zs.BF16, zs.INDEX_SHARD))

The binding is loaded lazily so that importing the package does not need the
built library; using `zs` without it raises ImportError (no fallback).
"""
import importlib

__all__ = ["zs", "build"]


def __getattr__(name):
    if name == "zs":
        return importlib.import_module("._lib", __name__)
    if name == "build":
        return importlib.import_module(".build", __name__)
    raise AttributeError(name)
