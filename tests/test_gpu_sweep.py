"""GPU parity of the two-stream FSDP sweep (zero_fsdp_sweep).

The sweep must give exactly what per-unit zero_adam_step + zero_gather_params
give -- which the oracle pins -- for every in-flight cap, on two streams or
one, with distinct per-unit buffers or a ring of reused ones, per-unit rank
gradients as N buffers or one chunked receive buffer, bf16 or fp32, on fixed
and on ten seeded random configurations.  Also the full
Llama-70B sweep (N = 64, 81 units) with a ring of two unit buffers and
chunked receive buffers, sampled.
"""
import numpy as np
import pytest
import torch

from oracle import _c, strategies
from chunked import grad_buffer, state_buffer, state_pos
from gather_check import assert_gathered
from synthetic import WORKLOADS, grad_bits, master_init, peer_bits, small_workload

pytestmark = pytest.mark.gpu
zs = None
DEV = "cuda:0"


def setup_module(module):
    global zs
    from fsdp_sharded_optimizer_shard_amd import zs as _zs
    zs = _zs


def h16(t):
    return t.cpu().numpy().view(np.uint16)


def h32(t):
    return t.cpu().numpy()


@pytest.mark.parametrize("cap,two,E,GE,fp32", [
    (0, True, 0, 0, False), (1, True, 0, 0, False), (2, True, 0, 0, False),
    (3, True, 0, 0, False), (2, False, 0, 0, False), (2, True, 16, 0, False),
    (0, True, 2048, 0, False), (2, True, 0, 4, False), (1, True, 16, 64, False),
    (2, False, 2048, 1024, False), (2, True, 0, 0, True), (1, True, 2048, 64, True)])
def test_sweep_small_ragged_matches_oracle(cap, two, E, GE, fp32):
    """E > 0: master, m and v in one chunked buffer of E-element chunks.
    GE > 0: each unit's rank gradients in one chunked receive buffer of
    GE-element rows per rank.  fp32: the rank gradients as fp32 (the bf16
    draws widened, so the sums and the oracle's results are the same)."""
    _sweep_case([4096, 100, 8192 + 3, 8, 0, 64 * 33, 5000, 2048 * 3], 8, 5, cap, two, E, GE,
                seed=cap, fp32=fp32)


@pytest.mark.parametrize("seed", range(10))
def test_sweep_random_configuration(seed):
    """Seeded random sweeps: 1-9 units of 0 to 12,000 elements, N up to 64,
    any rank, cap 0-3 on one or two streams, both memory formats."""
    rng = np.random.default_rng(500 + seed)
    units = [int(rng.choice([0, rng.integers(1, 50), rng.integers(100, 12000)]))
             for _ in range(int(rng.integers(1, 10)))]
    if sum(units) == 0:
        units.append(999)
    n = int(rng.choice([2, 3, 4, 8, 16, 64]))
    r = int(rng.integers(0, n))
    cap, two = int(rng.integers(0, 4)), bool(rng.integers(0, 2))
    E = int(rng.choice([0, 4, 64, 8192]))
    GE = int(rng.choice([0, 4, 16, 4096]))
    _sweep_case(units, n, r, cap, two, E, GE, seed=100 + seed)


def _sweep_case(units, n, r, cap, two, E, GE, seed, fp32=False):
    w = small_workload(units, n, "fsdp", steps=2, cfg=10, weight_decay=0.01, decoupled=True)
    psi = sum(units)
    master0 = master_init(w, psi).numpy()
    oc = strategies.make_cluster("fsdp", units, n, master0)
    olay = oc.layouts[r]
    L = zs.shard_init("fsdp", n, r, units)
    U = len(units)
    idx = np.concatenate([np.arange(b, b + k) for b, _, k in olay.owned_runs()])
    mfull = strategies.pad(olay, master0)
    S = L.shard_len
    if E:
        L = L.chunk_state(E)
        rows = -(-S // E)
        col = np.zeros(rows * E, np.float32)
        col[:S] = mfull[idx]
        buf_h = np.zeros((rows, 3, E), np.float32)
        buf_h[:, 0, :] = col.reshape(rows, E)
        buf = torch.from_numpy(buf_h.reshape(-1)).to(DEV)
        master, m, v = L.state_views(buf)
    else:
        master = torch.from_numpy(mfull[idx].copy()).to(DEV)
        m = torch.zeros(S, device=DEV)
        v = torch.zeros(S, device=DEV)
    rng = np.random.default_rng(seed)
    q = [L.query(u) for u in range(U)]
    peers_h = [[rng.integers(0, 1 << 16, x["shard_len"], dtype=np.uint16) for _ in range(n)]
               for x in q]
    peers = [[torch.from_numpy(p.view(np.int16)).to(DEV) for p in pu] for pu in peers_h]
    fulls = [torch.zeros(max(1, x["padded_len"]), dtype=torch.int16, device=DEV) for x in q]
    gs = torch.cuda.Stream() if two else None
    for t in range(w.steps):
        grads = [grad_bits(w, t, k, psi).numpy().view(np.uint16) for k in range(n)]
        strategies.step(oc, strategies.AdamConfig(weight_decay=0.01, decoupled=True), t + 1, grads)
        padded = [strategies.pad(olay, g) for g in grads]
        if fp32:
            # bf16 bit patterns widened to fp32 (exact)
            padded = [(p.astype(np.uint32) << 16).view(np.float32) for p in padded]
        gdt = np.float32 if fp32 else np.uint16
        ios = []
        for u, x in enumerate(q):
            b, s = x["rank_flat_off"], x["shard_len"]
            if GE:
                # rows of GE elements of each rank's slice, in rank order; a
                # zero-size unit still gets pointers one chunk apart
                rows = max(1, -(-s // GE))
                cells = np.zeros((rows, n, GE), gdt)
                for k, p in enumerate(padded):
                    col = np.zeros(rows * GE, gdt)
                    col[:s] = p[b:b + s]
                    cells[:, k, :] = col.reshape(rows, GE)
                flat = cells.reshape(-1)
                recv = torch.from_numpy(flat if fp32 else flat.view(np.int16)).to(DEV)
                rg = [recv[k * GE:] for k in range(n)]
            elif s:
                rg = [torch.from_numpy((p[b:b + s] if fp32 else
                                        p[b:b + s].view(np.int16)).copy()).to(DEV)
                      for p in padded]
            else:
                # a zero-size unit still needs non-NULL rank buffers (NULL =
                # missing replica)
                rg = [torch.zeros(1, dtype=torch.float32 if fp32 else torch.int16,
                                  device=DEV)] * n
            ios.append((rg, [None if k == r else peers[u][k] for k in range(n)], fulls[u]))
        zs.fsdp_sweep(L, 0, U, zs.adam_cfg(weight_decay=0.01, decoupled=True, step=t + 1),
                      zs.FP32 if fp32 else zs.BF16, ios, master, m, v, cap, gather_stream=gs,
                      grad_chunk=GE)
        torch.cuda.synchronize()
    st = strategies.full_state(oc, padded=True)
    if E:
        b = h32(buf).reshape(-1, 3, E)
        got = [b[:, k, :].reshape(-1)[:S] for k in range(3)]
    else:
        got = [h32(master), h32(m), h32(v)]
    for name, x in zip(("master", "m", "v"), got):
        assert np.array_equal(x.view(np.uint32), st[name][idx].view(np.uint32)), name
    want_params = strategies.full_params(oc, padded=True)
    for u, x in enumerate(q):
        if x["padded_len"] == 0:
            continue
        got = h16(fulls[u])
        s = x["shard_len"]
        for k in range(n):
            seg = got[k * s:(k + 1) * s]
            if k == r:
                F = x["flat_off"]
                assert np.array_equal(seg, want_params[F + r * s:F + (r + 1) * s]), (u, "own")
            else:
                assert np.array_equal(seg, peers_h[u][k]), (u, k)


@pytest.mark.parametrize("E", [0, 8192])
def test_sweep_ring_of_two_buffers_full_llama70b(E):
    """The whole 81-unit sweep at N = 64 with K = 2 and two unit buffers
    reused in turn, every unit's 64 rank gradients read from one chunked
    receive buffer, master, m and v as three arrays or (E > 0, the bench's
    configuration) one chunked buffer; every unit's state sampled against
    the oracle, the last two units' buffers checked."""
    w = WORKLOADS[4]
    n, r = w.n_ranks, w.n_ranks - 1
    units = list(w.units)
    U = len(units)
    L = zs.shard_init("fsdp", n, r, units)
    if E:
        L = L.chunk_state(E)
    q = [L.query(u) for u in range(U)]
    smax = max(x["shard_len"] for x in q)
    GE = zs.GRAD_CHUNK_DEFAULT
    # every unit reads elements [0, s_u) of each rank's draw: the prefix of
    # one receive buffer laid out for the largest unit
    grads = [grad_bits(w, 0, k, smax, device=DEV) for k in range(n)]
    recv, _ = grad_buffer(smax, n, GE, lambda k: grads[k])
    peers = [peer_bits(w, k, smax, device=DEV) for k in range(n)]
    ring = [torch.zeros(n * smax, dtype=torch.int16, device=DEV) for _ in range(2)]
    master0 = torch.empty(L.shard_len, device=DEV)
    for u, x in enumerate(q):
        so, su = x["shard_off"], x["shard_len"]
        master0[so:so + su] = master_init(w, su, device=DEV, rank=r, unit=u)
    if E:
        sbuf = state_buffer(L, master0)
        master, m, v = L.state_views(sbuf)
        arrays = None
    else:
        master, m, v = (master0, torch.zeros(L.shard_len, device=DEV),
                        torch.zeros(L.shard_len, device=DEV))
        arrays = (master, m, v)

    def at(k, i):
        # part k (master, m, v) of the state at shard indices i, the positions
        # checked on the host against the buffer they index
        if arrays is None:
            p, t = state_pos(E, i) + k * E, sbuf
        else:
            p, t = i, arrays[k]
        assert p.min() >= 0 and p.max() < t.numel()
        return t[torch.from_numpy(p).to(DEV)]
    rng = np.random.default_rng(44)
    samp = {}
    for u, x in enumerate(q):
        idx = np.unique(np.concatenate([rng.integers(0, x["shard_len"], 2048),
                                        [0, x["shard_len"] - 1]])).astype(np.int64)
        samp[u] = (idx, h32(at(0, x["shard_off"] + idx)).copy())
    gsamp = {}
    for u, x in enumerate(q):
        t_idx = torch.from_numpy(samp[u][0]).to(DEV)
        gsamp[u] = [h16(g[t_idx]) for g in grads]
    rg = [recv[k * GE:] for k in range(n)]
    ios = [(rg, [None if k == r else peers[k] for k in range(n)], ring[u % 2]) for u in range(U)]
    gs = torch.cuda.Stream()
    zs.fsdp_sweep(L, 0, U, zs.adam_cfg(step=1), zs.BF16, ios, master, m, v, 2, gather_stream=gs,
                  grad_chunk=GE)
    torch.cuda.synchronize()
    hp = _c.hparams(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, False)
    for u, x in enumerate(q):
        idx, p_h = samp[u]
        m_h = np.zeros(idx.size, np.float32)
        v_h = np.zeros(idx.size, np.float32)
        par_h = np.empty(idx.size, np.uint16)
        _c.rank_step(hp, gsamp[u], 1.0, p_h, m_h, v_h, par_h)
        ai = x["shard_off"] + idx
        assert np.array_equal(h32(at(0, ai)).view(np.uint32), p_h.view(np.uint32)), u
        assert np.array_equal(h32(at(1, ai)).view(np.uint32), m_h.view(np.uint32)), u
        assert np.array_equal(h32(at(2, ai)).view(np.uint32), v_h.view(np.uint32)), u
        if u >= U - 2:
            s = x["shard_len"]
            ub = ring[u % 2]
            own = h16(ub[r * s + torch.from_numpy(idx).to(DEV)])
            assert np.array_equal(own, par_h), u
            assert_gathered(ub, 0, s, [None if k == r else peers[k] for k in range(n)], idx,
                            f"sweep unit {u} gather")
