"""Shared pieces of the GPU parity tests: device/host conversions, the
chunked state and gradient formats built on the host, the bit-exact
comparisons, and GpuRanks, which runs all N simulated ranks of a sharded
strategy through the C ABI next to the oracle's cluster.  Index arithmetic
and copies only; the optimizer arithmetic is the library's (GPU) and the
oracle's (CPU)."""
import numpy as np
import torch

from oracle import _c, strategies
from synthetic import grad_bits, master_init

zs = None


def bind(module):
    """Called from a test module's setup: the library's binding."""
    global zs
    zs = module


DEV = "cuda:0"


def dev_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV)


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def host_bf16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def owned_index(lay):
    """Flat indices of a rank's slices, in shard order (oracle layout)."""
    return np.concatenate([np.arange(b, b + k, dtype=np.int64) for b, _, k in lay.owned_runs()])


def chunk_state(master, m, v, E):
    """One chunked state buffer (chunks of E master, E m, E v values) holding
    three shard-length arrays; the tail of the last chunk stays zero."""
    S = master.size
    n = -(-S // E)
    buf = np.zeros((n, 3, E), np.float32)
    for k, x in enumerate((master, m, v)):
        col = np.zeros(n * E, np.float32)
        col[:S] = x
        buf[:, k, :] = col.reshape(n, E)
    return buf.reshape(-1)


def chunk_grads(xs, E):
    """One chunked gradient buffer (rows of E elements of each of the N
    ranks in order) holding N shard-length arrays; row tails stay zero."""
    S, n = xs[0].size, len(xs)
    rows = -(-S // E)
    buf = np.zeros((rows, n, E), xs[0].dtype)
    for q, x in enumerate(xs):
        col = np.zeros(rows * E, x.dtype)
        col[:S] = x
        buf[:, q, :] = col.reshape(rows, E)
    return buf.reshape(-1)


def unchunk_state(buf, E, S):
    """(master, m, v) of shard length S out of a chunked state buffer."""
    b = np.asarray(buf).reshape(-1, 3, E)
    return tuple(np.ascontiguousarray(b[:, k, :].reshape(-1)[:S]) for k in range(3))


def assert_f32_close(got, want, what):
    """Bit-exact, and within the stated tolerance (reported together)."""
    diff = np.abs(got.astype(np.float64) - want.astype(np.float64))
    tol_ok = np.all((diff <= 1e-6 * np.maximum(1.0, np.abs(want))) | (got == want) |
                    (np.isnan(got) & np.isnan(want)))
    exact = np.array_equal(got.view(np.uint32), want.view(np.uint32))
    nbad = int(np.count_nonzero(got.view(np.uint32) != want.view(np.uint32)))
    assert tol_ok and exact, f"{what}: {nbad} of {got.size} differ, max |d| {diff.max():.3e}"


def assert_bf16_equal(got, want, what):
    d = np.abs(got.astype(np.int32) - want.astype(np.int32))
    nbad = int(np.count_nonzero(d))
    assert nbad == 0, f"{what}: {nbad} of {got.size} bf16 differ, max {d.max()} ulp-steps"


def cfg_of(w, t):
    return zs.adam_cfg(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                       weight_decay=w.weight_decay, decoupled=w.decoupled, step=t)


def oracle_cfg(w):
    return strategies.AdamConfig(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, w.decoupled,
                                 w.max_grad_norm)


def draw(w, steps):
    psi = w.psi
    master0 = master_init(w, psi).numpy()
    grads = [[grad_bits(w, t, q, psi).numpy().view(np.uint16) for q in range(w.n_ranks)]
             for t in range(steps)]
    return master0, grads


class GpuRanks:
    """All N simulated ranks of one sharded strategy on the GPU, each with
    its own shard state, writing its bf16 slice into one shared full flat
    buffer (the all-gather is implicit) or, for ZeRO-3, into its own shard
    buffer followed by zero_gather_params."""

    def __init__(self, w, master0, oracle_cluster, state_chunk=0, grad_chunk=0):
        self.w = w
        self.n = w.n_ranks
        self.oc = oracle_cluster
        self.E = state_chunk
        self.GE = grad_chunk
        self.lays = [zs.shard_init(w.strategy, self.n, r, list(w.units)) for r in range(self.n)]
        if state_chunk:
            self.lays = [L.chunk_state(state_chunk) for L in self.lays]
        self.U = len(w.units)
        lay0 = oracle_cluster.layouts[0]
        mfull = strategies.pad(lay0, master0)
        self.P = lay0.flat_len
        self.full = dev_bf16(_c.f32_to_bf16(mfull))
        self.state = []
        self.bufs = []
        for r in range(self.n):
            idx = owned_index(oracle_cluster.layouts[r])
            L = self.lays[r]
            S = L.shard_len
            if state_chunk:
                z = np.zeros(S, np.float32)
                buf = dev_f32(chunk_state(mfull[idx], z, z, state_chunk))
                self.bufs.append(buf)
                self.state.append(list(L.state_views(buf)))
            else:
                self.state.append([dev_f32(mfull[idx]), torch.zeros(S, device=DEV),
                                   torch.zeros(S, device=DEV)])

    def host_state(self, r):
        """(master, m, v) of rank r as shard-length host arrays."""
        if self.E:
            return unchunk_state(host_f32(self.bufs[r]), self.E, self.lays[r].shard_len)
        return tuple(host_f32(x) for x in self.state[r])

    def rank_grads(self, grads_t, r, index_modes, dtype):
        lay0 = self.oc.layouts[0]
        idx = owned_index(self.oc.layouts[r])
        xs = []
        for q in range(self.n):
            full = strategies.pad(lay0, grads_t[q])
            if dtype == zs.FP32:
                full = _c.bf16_to_f32(full)
            xs.append(full if index_modes[q] == zs.INDEX_FULL else full[idx])
        if self.GE:
            return xs          # host arrays; chunked per call by chunked_grads
        return [dev_f32(x) if dtype == zs.FP32 else dev_bf16(x) for x in xs]

    def chunked_grads(self, xs, dtype, lo=0, hi=None, index_modes=None, flo=0):
        """zs.Grads over one chunked receive buffer holding shard elements
        [lo, hi) of every shard-indexed rank's gradient.  A full-indexed
        rank keeps its own buffer from flat element `flo` on; its slot in
        the receive buffer holds NaN, which no result may show."""
        full = [q for q in range(self.n)
                if index_modes is not None and index_modes[q] == zs.INDEX_FULL]
        k = len(next(x for q, x in enumerate(xs) if q not in full)[lo:hi])
        hole = (np.full(k, np.nan, np.float32) if dtype == zs.FP32 else
                np.full(k, 0x7FC0, np.uint16))
        buf = chunk_grads([hole if q in full else x[lo:hi] for q, x in enumerate(xs)], self.GE)
        dev = dev_f32 if dtype == zs.FP32 else dev_bf16
        own = {q: dev(xs[q][flo:]) for q in full}
        return zs.Grads.chunked(dev(buf), self.n, self.GE, dtype, full=own)

    def grads_of(self, bufs, dtype, index_modes):
        """zs.Grads over rank_grads' result (one chunked buffer, or N)."""
        if self.GE:
            return self.chunked_grads(bufs, dtype, index_modes=index_modes)
        return zs.Grads(bufs, dtype, list(index_modes))

    def step_fused(self, t, grads_t, index_modes, dtype=None, per_unit=False):
        dtype = zs.BF16 if dtype is None else dtype
        c = cfg_of(self.w, t)
        for r, L in enumerate(self.lays):
            bufs = self.rank_grads(grads_t, r, index_modes, dtype)
            if self.GE:
                # chunked gradients are counted from the range's start: one
                # receive buffer per call; a chunked state is passed from its
                # start for every range, three state arrays move with the unit
                for u0, u1 in ([(u, u + 1) for u in range(self.U)] if per_unit else
                               [(0, self.U)]):
                    q = L.query(u0)
                    so, fo = q["shard_off"], q["flat_off"]
                    hi = so + sum(L.query(u)["shard_len"] for u in range(u0, u1))
                    if hi == so:
                        continue
                    G = self.chunked_grads(bufs, dtype, so, hi, index_modes, fo)
                    q0 = index_modes.index(zs.INDEX_SHARD)
                    assert (G._keep[q0].numel() + q0 * self.GE ==
                            L.grad_len(self.GE, u0, u1))
                    st = self.state[r] if self.E else [x[so:] for x in self.state[r]]
                    zs.adam_step(L, u0, u1, c, *st, self.full[fo:], zs.INDEX_FULL, grads=G)
                continue
            if not per_unit:
                G = zs.Grads(bufs, dtype, list(index_modes))
                zs.adam_step(L, 0, self.U, c, *self.state[r], self.full, zs.INDEX_FULL, grads=G)
                continue
            # one call per unit, every pointer moved to the unit's start
            for u in range(self.U):
                q = L.query(u)
                so, fo = q["shard_off"], q["flat_off"]
                ptrs = [b[so:] if index_modes[k] == zs.INDEX_SHARD else b[fo:]
                        for k, b in enumerate(bufs)]
                G = zs.Grads(ptrs, dtype, list(index_modes))
                # three arrays move with the unit; a chunked state is always
                # passed from its start
                st = self.state[r] if self.E else [x[so:] for x in self.state[r]]
                zs.adam_step(L, u, u + 1, c, *st, self.full[fo:], zs.INDEX_FULL, grads=G)

    def step_two_pass(self, t, grads_t, max_norm):
        """reduce every rank -> global clip coefficient -> Adam from fp32."""
        c = cfg_of(self.w, t)
        counts = [zs.reduce_partials_count(L, 0, self.U) for L in self.lays]
        partials = torch.empty(sum(counts), dtype=torch.float64, device=DEV)
        gshard = []
        off = 0
        modes = [zs.INDEX_SHARD if self.GE else zs.INDEX_FULL] * self.n
        for r, L in enumerate(self.lays):
            bufs = self.rank_grads(grads_t, r, modes, zs.BF16)
            g = torch.empty(L.shard_len, device=DEV)
            zs.reduce_shard(L, 0, self.U, self.grads_of(bufs, zs.BF16, modes), g,
                            partials[off:], counts[r])
            off += counts[r]
            gshard.append(g)
        coef = torch.empty(1, device=DEV)
        norm = torch.empty(1, dtype=torch.float64, device=DEV)
        zs.clip_coef(partials, partials.numel(), max_norm, coef, norm)
        for r, L in enumerate(self.lays):
            zs.adam_step(L, 0, self.U, c, *self.state[r], self.full, zs.INDEX_FULL,
                         grad_fp32=gshard[r], clip_coef=coef)
        return gshard, coef, norm

    def check(self, what):
        torch.cuda.synchronize()
        assert_bf16_equal(host_bf16(self.full), strategies.full_params(self.oc, padded=True),
                          f"{what}: params")
        st = strategies.full_state(self.oc, padded=True)
        for r in range(self.n):
            idx = owned_index(self.oc.layouts[r])
            got = self.host_state(r)
            for k, name in enumerate(("master", "m", "v")):
                assert_f32_close(got[k], st[name][idx], f"{what}: rank {r} {name}")
