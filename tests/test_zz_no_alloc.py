"""The entry point that allocates nothing, zero_adam_step_clip_noalloc,
against the three calls it stands for (zero_reduce_shard with caller-owned
sum-of-squares partials, zero_clip_coef into a caller-owned coefficient,
zero_adam_step from the reduced gradient), through the C ABI, on the same
inputs: master, m, v, the bf16 parameters, the averaged gradient and the
norm must be bit-identical.  Two calls in a row share the library's static
buffer, the second on a smaller range than the first, so a stale partial
left by the first call would show in the second's norm."""
import numpy as np
import pytest
import torch

from synthetic import grad_bits, master_init, small_workload

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(strategy, units, n, r, cfg_id):
    from fsdp_sharded_optimizer_shard_amd import zs
    w = small_workload(units, n, strategy, cfg=cfg_id, weight_decay=0.01, decoupled=True)
    L = zs.shard_init(strategy, n, r, units)
    P, S = L.flat_len, L.shard_len
    grads = [grad_bits(w, 0, q, P, device=DEV) for q in range(n)]
    master0 = master_init(w, S, device=DEV, rank=r)
    return w, L, grads, master0


def _bits(t):
    x = t.cpu().numpy()
    return x.view({4: np.uint32, 8: np.uint64, 2: np.uint16}[x.itemsize])


def _state(L, master0, E):
    """master, m, v: three arrays, or views of one chunked buffer (E > 0)
    holding master0 and zeros."""
    S = L.shard_len
    if not E:
        return [master0.clone(), torch.zeros(S, device=DEV), torch.zeros(S, device=DEV)]
    rows = -(-S // E)
    buf = torch.zeros(L.state_len, device=DEV)
    col = torch.zeros(rows * E, device=DEV)
    col[:S] = master0
    buf.view(rows, 3, E)[:, 0, :].copy_(col.view(rows, E))
    return list(L.state_views(buf)) + [buf]


def _both_paths(strategy, units, n, r, cfg_id, max_norm, steps, state_chunk=0, grad_chunk=0):
    from fsdp_sharded_optimizer_shard_amd import zs
    w, L, grads, master0 = _case(strategy, units, n, r, cfg_id)
    if state_chunk:
        L = L.chunk_state(state_chunk)
    U, P, S = len(units), L.flat_len, L.shard_len
    G = zs.Grads(grads, zs.BF16, zs.INDEX_FULL)
    if grad_chunk:
        # rank q's shard slices, chunked into one buffer (rows of grad_chunk
        # elements per rank)
        E = grad_chunk
        rows = -(-S // E)
        owned = torch.cat([torch.arange(L.query(u)["rank_flat_off"],
                                        L.query(u)["rank_flat_off"] + L.query(u)["shard_len"])
                           for u in range(U)]).to(DEV)
        gbuf = torch.zeros(L.grad_len(E), dtype=torch.int16, device=DEV)
        col = torch.zeros(rows * E, dtype=torch.int16, device=DEV)
        for q in range(n):
            col[:S] = grads[q][owned]
            gbuf.view(rows, n, E)[:, q, :].copy_(col.view(rows, E))
        G = zs.Grads.chunked(gbuf, n, E)
    out = {}
    for path in ("three_calls", "noalloc"):
        st = _state(L, master0, state_chunk)
        full = torch.zeros(P, dtype=torch.int16, device=DEV)
        gout = torch.empty(S, device=DEV)
        norm = torch.empty(1, dtype=torch.float64, device=DEV)
        for t in range(1, steps + 1):
            cfg = zs.adam_cfg(weight_decay=w.weight_decay, decoupled=w.decoupled, step=t)
            if path == "three_calls":
                count = zs.reduce_partials_count(L, 0, U)
                partials = torch.empty(count, dtype=torch.float64, device=DEV)
                coef = torch.empty(1, device=DEV)
                zs.reduce_shard(L, 0, U, G, gout, partials, count)
                zs.clip_coef(partials, count, max_norm, coef, norm)
                zs.adam_step(L, 0, U, cfg, *st[:3], full, zs.INDEX_FULL, grad_fp32=gout,
                             clip_coef=coef)
                out["coef"] = float(coef.item())
            else:
                zs.adam_step_clip_noalloc(L, 0, U, cfg, max_norm, G, gout, *st[:3], full,
                                          zs.INDEX_FULL, norm_out=norm)
        torch.cuda.synchronize()
        state = {"state": _bits(st[3])} if state_chunk else {
            "master": _bits(st[0]), "m": _bits(st[1]), "v": _bits(st[2])}
        out[path] = dict(state, params=_bits(full), grad=_bits(gout), norm=_bits(norm))
    return out


def test_two_calls_in_a_row_match_the_three_call_path():
    # first a larger DDP replica (the norm over the whole buffer), then a
    # smaller ZeRO-2 rank shard (the norm over that shard), both clipped
    first = _both_paths("ddp", [300_000, 123_457], 8, 0, 21, 0.05, steps=2)
    second = _both_paths("zero2", [5000, 777, 64], 4, 1, 22, 0.01, steps=1)
    for name, res in (("first call", first), ("second call", second)):
        assert res["coef"] < 1.0, f"{name}: the clip must be active"
        for k, want in res["three_calls"].items():
            got = res["noalloc"][k]
            nbad = int(np.count_nonzero(got != want))
            assert nbad == 0, f"{name}: {k}: {nbad} of {want.size} differ"


def test_chunked_gradients_call_matches_the_three_call_path():
    # the rank gradients chunked into one buffer, on a chunked state and on
    # three arrays
    for E in (1024, 0):
        res = _both_paths("zero3", [20_000, 333, 4099], 8, 5, 24, 0.005, steps=2, state_chunk=E,
                          grad_chunk=512)
        assert res["coef"] < 1.0
        for k, want in res["three_calls"].items():
            got = res["noalloc"][k]
            nbad = int(np.count_nonzero(got != want))
            assert nbad == 0, f"chunked gradients, state chunk {E}: {k}: {nbad} of {want.size} differ"


def test_chunked_state_call_matches_the_three_call_path():
    # the same entry point on a layout whose master, m and v form one
    # chunked buffer, after the calls above have left the static buffer
    # holding their partials
    res = _both_paths("zero3", [20_000, 333, 4099], 8, 3, 23, 0.005, steps=2, state_chunk=1024)
    assert res["coef"] < 1.0
    for k, want in res["three_calls"].items():
        got = res["noalloc"][k]
        nbad = int(np.count_nonzero(got != want))
        assert nbad == 0, f"chunked state: {k}: {nbad} of {want.size} differ"
