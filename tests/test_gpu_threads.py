"""Calls from several host threads at once, each on its own stream with its
own buffers, give the same bits as the same calls made one after another
from one thread (the library keeps no shared mutable state besides
per-device caches and a per-thread error message)."""
import threading

import numpy as np
import pytest
import torch

from synthetic import grad_bits, small_workload

pytestmark = pytest.mark.gpu

zs = None
DEV = "cuda:0"


def setup_module(module):
    global zs
    from fsdp_sharded_optimizer_shard_amd import zs as _zs
    zs = _zs


def _bits(t):
    return t.cpu().numpy().view(np.uint32 if t.dtype == torch.float32 else np.uint16)


def test_concurrent_threads_match_sequential():
    units, n, T, steps = [6000, 2500, 1111], 4, 4, 5
    w = small_workload(units, n, "zero3", cfg=14)
    lays = [zs.shard_init("zero3", n, r, units) for r in range(n)]
    S, P = lays[0].shard_len, lays[0].flat_len
    peers = [grad_bits(w, 9, q, S, device=DEV) for q in range(n)]

    def job(k):
        # thread k runs rank k % n of its own copy of the state
        r = k % n
        grads = [grad_bits(w, k, q, S, device=DEV) for q in range(n)]
        g = torch.Generator(device="cpu")
        g.manual_seed(k)
        st = [(torch.randn(S, generator=g) * 0.02).to(DEV), torch.zeros(S, device=DEV),
              torch.zeros(S, device=DEV), torch.zeros(P, dtype=torch.int16, device=DEV)]
        return r, grads, st

    def run(r, grads, st, stream):
        with torch.cuda.stream(stream):
            for t in range(1, steps + 1):
                zs.adam_step(lays[r], 0, len(units), zs.adam_cfg(step=t), st[0], st[1], st[2],
                             st[3], grads=zs.Grads(grads, zs.BF16, zs.INDEX_SHARD))
                zs.gather_params(lays[r], 0, len(units),
                                 [None if q == r else peers[q] for q in range(n)], st[3])

    seq = [job(k) for k in range(T)]
    par = [job(k) for k in range(T)]
    torch.cuda.synchronize()
    s0 = torch.cuda.Stream()
    for r, grads, st in seq:
        run(r, grads, st, s0)
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream() for _ in range(T)]
    errors = []

    def worker(k):
        try:
            run(*par[k], streams[k])
        except Exception as e:          # reported below, in the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(T)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k in range(T):
        for a, b in zip(seq[k][2], par[k][2]):
            assert np.array_equal(_bits(a), _bits(b)), f"thread {k}"
