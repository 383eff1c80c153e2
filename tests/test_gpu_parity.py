"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: bit-exact for layouts, gathered parameters and every fp32 result (the
kernels follow the oracle's operation order: fp32, one rounding per
operation, ascending rank sum, IEEE division and square root), which is
stricter than the stated floating-point tolerance |d| <= 1e-6 max(1, |x|)
on master / m / v and 1 bf16 ulp on parameters; the tolerance is also
asserted so a failure reports both.  The only value that may differ is the
fp64 global norm (summation order); its fp32 clip coefficient must match.

Small cases span several 2048-element tiles, ragged tails, zero padding,
slices that are not multiples of 8 (scalar path), N in {1, 2, 3, 4, 5, 8,
64}, bf16 and fp32 gradients, full- and shard-indexed rank buffers, AdamW and
L2 decay, whole-range and per-unit calls, three state arrays or a chunked
state, one buffer per rank gradient or all N chunked into one.  The
full-size 7B / N = 8 shard is checked after 3 steps in the launch
configuration the benchmark times: on sampled elements (with the gather
into the 7.24e9-element buffer), and element by element over all
905,000,000 elements.
"""
import numpy as np
import pytest
import torch

from oracle import _c, strategies
from gather_check import assert_gathered
from synthetic import WORKLOADS, grad_bits, master_init, peer_bits, small_workload

pytestmark = pytest.mark.gpu

zs = None


def setup_module(module):
    global zs
    from fsdp_sharded_optimizer_shard_amd import zs as _zs
    zs = _zs
    assert torch.cuda.is_available()


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

    def chunked_grads(self, xs, dtype, lo=0, hi=None):
        """zs.Grads over one chunked receive buffer holding shard elements
        [lo, hi) of every rank's shard-indexed gradient."""
        buf = chunk_grads([x[lo:hi] for x in xs], self.GE)
        d = dev_f32(buf) if dtype == zs.FP32 else dev_bf16(buf)
        return zs.Grads.chunked(d, self.n, self.GE, dtype)

    def grads_of(self, bufs, dtype, index_modes):
        """zs.Grads over rank_grads' result (one chunked buffer, or N)."""
        if self.GE:
            return self.chunked_grads(bufs, dtype)
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
                    G = self.chunked_grads(bufs, dtype, so, hi)
                    assert G._keep[0].numel() == L.grad_len(self.GE, u0, u1)
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


# ------------------------------------------------------------ cases --

def test_config0_tiny_zero2_ten_steps():
    """Psi = 2^20, N = 4, Adam, 10 steps, all four ranks into one buffer;
    checked bit-exactly after every step (and DDP == ZeRO in the oracle)."""
    w = WORKLOADS[0]
    master0, grads = draw(w, w.steps)
    oc = strategies.make_cluster("zero2", list(w.units), w.n_ranks, master0)
    ddp = strategies.make_cluster("ddp", list(w.units), w.n_ranks, master0)
    g = GpuRanks(w, master0, oc)
    for t in range(w.steps):
        strategies.step(oc, oracle_cfg(w), t + 1, grads[t])
        strategies.step(ddp, oracle_cfg(w), t + 1, grads[t])
        g.step_fused(t + 1, grads[t], [zs.INDEX_FULL] * w.n_ranks)
        g.check(f"config 0 step {t + 1}")
    assert np.array_equal(strategies.full_params(ddp), strategies.full_params(oc))


CASES = [
    # units, N, strategy, decay, index modes
    ([5000, 333, 20000], 4, "zero2", "adamw", "full"),
    ([4097, 1, 0, 7], 3, "zero2", "l2", "shard"),
    ([2048 * 3 + 5], 5, "zero3", "none", "mixed"),
    ([640, 6400, 64000], 8, "fsdp", "adamw", "shard"),
    ([129 * 64, 64, 1], 64, "fsdp", "none", "shard"),
    ([3333], 1, "zero2", "adamw", "full"),
    ([100, 10000], 2, "zero1", "l2", "full"),
]


def _w(units, n, strategy, decay, cfg=12, steps=3):
    kw = {}
    if decay == "adamw":
        kw = dict(weight_decay=0.01, decoupled=True)
    elif decay == "l2":
        kw = dict(weight_decay=0.1, decoupled=False)
    return small_workload(units, n, strategy, steps=steps, cfg=cfg, outlier_frac=0.01, **kw)


def _modes(kind, n):
    if kind == "full":
        return [zs.INDEX_FULL] * n
    if kind == "shard":
        return [zs.INDEX_SHARD] * n
    return [zs.INDEX_FULL if q % 2 == 0 else zs.INDEX_SHARD for q in range(n)]


@pytest.mark.parametrize("units,n,strategy,decay,modes", CASES)
def test_fused_step_small_layouts(units, n, strategy, decay, modes):
    w = _w(units, n, strategy, decay)
    master0, grads = draw(w, w.steps)
    oc = strategies.make_cluster(strategy, units, n, master0)
    g = GpuRanks(w, master0, oc)
    for t in range(w.steps):
        strategies.step(oc, oracle_cfg(w), t + 1, grads[t])
        g.step_fused(t + 1, grads[t], _modes(modes, n))
        g.check(f"{units} N={n} step {t + 1}")


def test_per_unit_calls_equal_whole_range():
    units, n = [4096, 100, 8192 + 3, 8], 4
    w = _w(units, n, "fsdp", "adamw")
    master0, grads = draw(w, 2)
    oc = strategies.make_cluster("fsdp", units, n, master0)
    g = GpuRanks(w, master0, oc)
    for t in range(2):
        strategies.step(oc, oracle_cfg(w), t + 1, grads[t])
        g.step_fused(t + 1, grads[t], _modes("mixed", n), per_unit=True)
        g.check(f"per-unit step {t + 1}")


CHUNK_CASES = [
    # units, N, strategy, decay, index modes, state chunk
    ([5000, 333, 20000], 4, "zero2", "adamw", "full", 8192),
    ([4097, 1, 0, 7], 3, "zero2", "l2", "shard", 4),
    ([2048 * 3 + 5], 5, "zero3", "none", "mixed", 1024),
    ([640, 6400, 64000], 8, "fsdp", "adamw", "shard", 8),
    ([129 * 64, 64, 1], 64, "fsdp", "none", "shard", 16384),
]


@pytest.mark.parametrize("units,n,strategy,decay,modes,E", CHUNK_CASES)
def test_fused_step_chunked_state(units, n, strategy, decay, modes, E):
    """The fused step with master, m and v in one chunked buffer: results
    equal the oracle's bit for bit.  Chunks of 4 and 8 put every 4-element
    group at a chunk edge; units with shard offsets that are not multiples
    of 4 run the scalar path across chunk edges."""
    w = _w(units, n, strategy, decay)
    master0, grads = draw(w, w.steps)
    oc = strategies.make_cluster(strategy, units, n, master0)
    g = GpuRanks(w, master0, oc, state_chunk=E)
    for t in range(w.steps):
        strategies.step(oc, oracle_cfg(w), t + 1, grads[t])
        g.step_fused(t + 1, grads[t], _modes(modes, n))
        g.check(f"{units} N={n} E={E} step {t + 1}")


@pytest.mark.parametrize("E", [4, 64, 4096])
def test_per_unit_calls_on_chunked_state(E):
    """One call per unit on a chunked state (each passed from the buffer's
    start) equals the oracle, with unit shard offsets 1024, 25, 2048+..."""
    units, n = [4096, 100, 8192 + 3, 8], 4
    w = _w(units, n, "fsdp", "adamw")
    master0, grads = draw(w, 2)
    oc = strategies.make_cluster("fsdp", units, n, master0)
    g = GpuRanks(w, master0, oc, state_chunk=E)
    for t in range(2):
        strategies.step(oc, oracle_cfg(w), t + 1, grads[t])
        g.step_fused(t + 1, grads[t], _modes("mixed", n), per_unit=True)
        g.check(f"per-unit chunked E={E} step {t + 1}")


def test_two_pass_clip_on_chunked_state():
    """reduce -> clip coefficient -> Adam from fp32 on a chunked state."""
    units, n, max_norm = [25000, 25000, 24439], 8, 1e-4
    w = small_workload(units, n, "zero2", steps=2, cfg=11, weight_decay=0.01, decoupled=True,
                       max_grad_norm=max_norm, outlier_frac=0.01)
    master0, grads = draw(w, w.steps)
    oc = strategies.make_cluster("zero2", units, n, master0)
    g = GpuRanks(w, master0, oc, state_chunk=2048)
    for t in range(w.steps):
        strategies.step(oc, oracle_cfg(w), t + 1, grads[t])
        g.step_two_pass(t + 1, grads[t], max_norm)
        g.check(f"chunked clip step {t + 1}")


def test_table_step_on_chunked_state():
    """zero_adam_step_table (scalars read on the device from a step table)
    on a chunked state, three steps with the counter advanced on the device."""
    units, n, E = [5000, 777, 64], 4, 64
    w = _w(units, n, "zero3", "adamw")
    master0, grads = draw(w, w.steps)
    oc = strategies.make_cluster("zero3", units, n, master0)
    g = GpuRanks(w, master0, oc, state_chunk=E)
    table = zs.adam_table_device([cfg_of(w, t + 1) for t in range(w.steps)], DEV)
    counter = torch.ones(1, dtype=torch.int64, device=DEV)
    modes = _modes("mixed", n)
    for t in range(w.steps):
        strategies.step(oc, oracle_cfg(w), t + 1, grads[t])
        for r, L in enumerate(g.lays):
            G = zs.Grads(g.rank_grads(grads[t], r, modes, zs.BF16), zs.BF16, modes)
            zs.adam_step_table(L, 0, g.U, table, w.steps, counter, *g.state[r], g.full,
                               zs.INDEX_FULL, grads=G)
        zs.step_advance(counter)
        g.check(f"table on chunked state, step {t + 1}")


@pytest.mark.parametrize("E", [0, 1024])
def test_fp32_gradients_megatron(E):
    """fp32 rank gradients (the Megatron main_grad) through the fused path,
    with three state arrays and with a chunked state."""
    units, n = [8192 * 3 + 17], 8
    w = _w(units, n, "megatron_do", "none")
    master0, grads = draw(w, 2)
    oc = strategies.make_cluster("megatron_do", units, n, master0)
    g = GpuRanks(w, master0, oc, state_chunk=E)
    for t in range(2):
        strategies.step(oc, oracle_cfg(w), t + 1, [[x] for x in grads[t]])
        g.step_fused(t + 1, grads[t], _modes("mixed", n), dtype=zs.FP32)
        g.check(f"megatron fp32 step {t + 1}")


GRAD_CHUNK_CASES = [
    # units, N, strategy, decay, state chunk, gradient chunk
    ([5000, 333, 20000], 4, "zero2", "adamw", 8192, 16384),
    ([4097, 1, 0, 7], 3, "zero2", "l2", 0, 4),
    ([2048 * 3 + 5], 5, "zero3", "none", 1024, 8),
    ([640, 6400, 64000], 8, "fsdp", "adamw", 8192, 1024),
    ([129 * 64, 64, 1], 64, "fsdp", "none", 16384, 64),
]


@pytest.mark.parametrize("units,n,strategy,decay,E,GE", GRAD_CHUNK_CASES)
def test_fused_step_chunked_grads(units, n, strategy, decay, E, GE):
    """The N rank gradients in one chunked buffer (rows of GE elements per
    rank), with three state arrays or a chunked state: bit for bit the
    oracle's results.  N = 3 and 5 give rows that are not a power of two;
    chunks of 4 and 8 put every 4-element group at a chunk edge; units with
    shard offsets that are not multiples of 4 run the scalar path."""
    w = _w(units, n, strategy, decay)
    master0, grads = draw(w, w.steps)
    oc = strategies.make_cluster(strategy, units, n, master0)
    g = GpuRanks(w, master0, oc, state_chunk=E, grad_chunk=GE)
    for t in range(w.steps):
        strategies.step(oc, oracle_cfg(w), t + 1, grads[t])
        g.step_fused(t + 1, grads[t], _modes("shard", n))
        g.check(f"{units} N={n} E={E} GE={GE} step {t + 1}")


@pytest.mark.parametrize("E,GE", [(0, 4), (64, 4096), (4, 16)])
def test_per_unit_calls_on_chunked_grads(E, GE):
    """One call per unit, each with its own chunked receive buffer (unit
    shard offsets 1024, 1049, 3097, ...: vector and scalar slices, and
    unit lengths that are not multiples of the chunk)."""
    units, n = [4096, 100, 8192 + 3, 8], 4
    w = _w(units, n, "fsdp", "adamw")
    master0, grads = draw(w, 2)
    oc = strategies.make_cluster("fsdp", units, n, master0)
    g = GpuRanks(w, master0, oc, state_chunk=E, grad_chunk=GE)
    for t in range(2):
        strategies.step(oc, oracle_cfg(w), t + 1, grads[t])
        g.step_fused(t + 1, grads[t], _modes("shard", n), per_unit=True)
        g.check(f"per-unit chunked grads E={E} GE={GE} step {t + 1}")


def test_fp32_chunked_grads_megatron():
    """fp32 rank gradients in one chunked buffer through the fused path."""
    units, n = [8192 * 3 + 17], 8
    w = _w(units, n, "megatron_do", "none")
    master0, grads = draw(w, 2)
    oc = strategies.make_cluster("megatron_do", units, n, master0)
    g = GpuRanks(w, master0, oc, state_chunk=1024, grad_chunk=2048)
    for t in range(2):
        strategies.step(oc, oracle_cfg(w), t + 1, [[x] for x in grads[t]])
        g.step_fused(t + 1, grads[t], _modes("shard", n), dtype=zs.FP32)
        g.check(f"megatron fp32 chunked grads step {t + 1}")


def test_two_pass_clip_on_chunked_grads():
    """reduce_shard from chunked gradients -> clip coefficient -> Adam from
    fp32; the coefficient must equal the oracle's."""
    units, n, max_norm = [25000, 25000, 24439], 8, 1e-4
    w = small_workload(units, n, "zero2", steps=2, cfg=11, weight_decay=0.01, decoupled=True,
                       max_grad_norm=max_norm, outlier_frac=0.01)
    master0, grads = draw(w, w.steps)
    oc = strategies.make_cluster("zero2", units, n, master0)
    g = GpuRanks(w, master0, oc, state_chunk=2048, grad_chunk=8192)
    lay0 = oc.layouts[0]
    for t in range(w.steps):
        g_mean = _c.average([strategies.pad(lay0, x) for x in grads[t]])
        want_coef = _c.clip_coef(_c.sumsq(g_mean), max_norm)
        strategies.step(oc, oracle_cfg(w), t + 1, grads[t])
        gshard, coef, _ = g.step_two_pass(t + 1, grads[t], max_norm)
        torch.cuda.synchronize()
        assert coef.item() == np.float32(want_coef)
        for r in range(n):
            idx = owned_index(oc.layouts[r])
            assert_f32_close(host_f32(gshard[r]), g_mean[idx], f"reduced grad rank {r}")
        g.check(f"chunked grads clip step {t + 1}")


@pytest.mark.parametrize("max_norm", [1.0, 1e-4])
def test_two_pass_clip(max_norm):
    """reduce_shard -> clip_coef -> adam_step(grad_fp32, clip_coef), AdamW,
    1 % outliers, several buckets; the coefficient must equal the oracle's."""
    units, n = [25000, 25000, 24439], 8
    w = small_workload(units, n, "zero2", steps=3, cfg=11, weight_decay=0.01, decoupled=True,
                       max_grad_norm=max_norm, outlier_frac=0.01)
    master0, grads = draw(w, w.steps)
    oc = strategies.make_cluster("zero2", units, n, master0)
    g = GpuRanks(w, master0, oc)
    lay0 = oc.layouts[0]
    for t in range(w.steps):
        g_mean = _c.average([strategies.pad(lay0, x) for x in grads[t]])
        sumsq = _c.sumsq(g_mean)
        want_coef = _c.clip_coef(sumsq, max_norm)
        strategies.step(oc, oracle_cfg(w), t + 1, grads[t])
        gshard, coef, norm = g.step_two_pass(t + 1, grads[t], max_norm)
        torch.cuda.synchronize()
        assert abs(norm.item() - np.sqrt(sumsq)) <= 1e-12 * np.sqrt(sumsq)
        assert coef.item() == np.float32(want_coef)
        for r in range(n):
            idx = owned_index(oc.layouts[r])
            assert_f32_close(host_f32(gshard[r]), g_mean[idx], f"reduced grad rank {r}")
        g.check(f"clip {max_norm} step {t + 1}")


def test_ddp_variant():
    """Full-replica averaging + replicated Adam: every replica's library call
    produces the oracle's DDP replica."""
    units, n = [3000, 50000], 4
    w = _w(units, n, "ddp", "adamw")
    master0, grads = draw(w, 2)
    oc = strategies.make_cluster("ddp", units, n, master0)
    lays = [zs.shard_init("ddp", n, r, units) for r in range(n)]
    P = lays[0].flat_len
    assert P == sum(units)
    reps = [[dev_f32(master0), torch.zeros(P, device=DEV), torch.zeros(P, device=DEV),
             torch.zeros(P, dtype=torch.int16, device=DEV)] for _ in range(n)]
    for t in range(2):
        strategies.step(oc, oracle_cfg(w), t + 1, grads[t])
        G = zs.Grads([dev_bf16(x) for x in grads[t]], zs.BF16, zs.INDEX_FULL)
        for r in range(n):
            zs.adam_step(lays[r], 0, 2, cfg_of(w, t + 1), *reps[r][:3], reps[r][3], zs.INDEX_FULL,
                         grads=G)
    torch.cuda.synchronize()
    want = strategies.full_params(oc)
    for r in range(n):
        assert_bf16_equal(host_bf16(reps[r][3]), want, f"ddp replica {r}")
        assert_f32_close(host_f32(reps[r][0]), oc.ranks[r].master, f"ddp replica {r} master")


@pytest.mark.parametrize("units,n", [([5000, 333, 20000], 4), ([7, 2048 * 5 + 3], 8),
                                     ([64 * 129, 64], 64)])
def test_gather_params(units, n):
    rng = np.random.default_rng(n)
    lays_o = [strategies.plan(units, n, r) for r in range(n)]
    S = lays_o[0].shard_len
    shards = [rng.integers(0, 1 << 16, S, dtype=np.uint16) for _ in range(n)]
    want = strategies.all_gather(lays_o, shards)
    L = zs.shard_init("zero3", n, n - 1, units)
    sentinel = np.full(L.flat_len, 0xABCD, np.uint16)
    full = dev_bf16(sentinel)
    dsh = [dev_bf16(s) for s in shards]
    zs.gather_params(L, 0, len(units), [None if q == n - 1 else dsh[q] for q in range(n)], full)
    torch.cuda.synchronize()
    got = host_bf16(full)
    own = owned_index(lays_o[n - 1])
    mask = np.ones(L.flat_len, bool)
    mask[own] = False
    assert np.array_equal(got[mask], want[mask])
    assert np.all(got[own] == 0xABCD)          # the NULL (own) slot is not touched
    zs.gather_params(L, 0, len(units), dsh, full)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(full), want)


@pytest.mark.parametrize("n,off", [(1, 0), (8 * 2048 * 3 + 5, 0), (100_003, 1), (4096, 3)])
def test_grad_accumulate(n, off):
    rng = np.random.default_rng(n)
    acc0 = (rng.standard_normal(n + off) * 1e-3).astype(np.float32)
    micro = [_c.f32_to_bf16((rng.standard_normal(n + off) * 1e-3).astype(np.float32))
             for _ in range(4)]
    acc = dev_f32(acc0)
    for mb in micro:
        d = dev_bf16(mb)
        zs.grad_accumulate(acc[off:], d[off:], n)
    torch.cuda.synchronize()
    want = acc0.copy()
    for mb in micro:
        part = want[off:].copy()
        _c.accumulate_bf16(part, np.ascontiguousarray(mb[off:]))
        want[off:] = part
    assert_f32_close(host_f32(acc), want, "accumulate")


# --------------------------------------------------- full-size config 2 --

def _sample_index(S, rng):
    idx = rng.integers(0, S, 1 << 20)
    edges = np.concatenate([np.arange(0, 4096), np.arange(S - 4096, S)])
    return np.unique(np.concatenate([idx, edges])).astype(np.int64)


def test_config2_full_size_sampled():
    """Mistral-7B ZeRO-3 rank shard: 905,000,000 elements, N = 8, rank 7,
    3 Adam steps through the fused path in the benchmark's launch (state
    chunked at the library default, the 8 rank gradients chunked into one
    buffer), then the gather of the 7 peer shards; sampled elements against
    the oracle."""
    w = WORKLOADS[2]
    n, r = w.n_ranks, w.n_ranks - 1
    E, GE = zs.STATE_CHUNK_DEFAULT, zs.GRAD_CHUNK_DEFAULT
    L = zs.shard_init("zero3", n, r, list(w.units)).chunk_state(E)
    S = L.shard_len
    assert S == 905_000_000
    rng = np.random.default_rng(2)
    idx = _sample_index(S, rng)
    pos = torch.from_numpy((idx // E) * 3 * E + idx % E).to(DEV)
    tidx = torch.from_numpy(idx).to(DEV)
    master = master_init(w, S, device=DEV, rank=r)
    rows, grows = -(-S // E), -(-S // GE)
    st = torch.zeros(L.state_len, device=DEV)
    col = torch.zeros(rows * E, device=DEV)
    col[:S] = master
    st.view(rows, 3, E)[:, 0, :].copy_(col.view(rows, E))
    del col
    own = torch.empty(S, dtype=torch.int16, device=DEV)
    p_h = master[tidx].cpu().numpy()
    del master
    m_h = np.zeros(idx.size, np.float32)
    v_h = np.zeros(idx.size, np.float32)
    par_h = np.empty(idx.size, np.uint16)
    for t in range(w.steps):
        gbuf = torch.zeros(L.grad_len(GE), dtype=torch.int16, device=DEV)
        col = torch.zeros(grows * GE, dtype=torch.int16, device=DEV)
        samp = []
        for q in range(n):
            col[:S] = grad_bits(w, t, q, S, device=DEV)
            samp.append(host_bf16(col[tidx]))
            gbuf.view(grows, n, GE)[:, q, :].copy_(col.view(grows, GE))
        del col
        zs.adam_step(L, 0, 1, cfg_of(w, t + 1), *L.state_views(st), own, zs.INDEX_SHARD,
                     grads=zs.Grads.chunked(gbuf, n, GE))
        torch.cuda.synchronize()
        del gbuf
        _c.rank_step(oracle_cfg(w).hparams(t + 1), samp, 1.0, p_h, m_h, v_h, par_h)
    torch.cuda.synchronize()
    assert_f32_close(host_f32(st[pos]), p_h, "config 2 master")
    assert_f32_close(host_f32(st[pos + E]), m_h, "config 2 m")
    assert_f32_close(host_f32(st[pos + 2 * E]), v_h, "config 2 v")
    assert_bf16_equal(host_bf16(own[tidx]), par_h, "config 2 bf16 shard")
    # all-gather data movement into the full 7.24e9-element buffer: random
    # peer shards, every slot at the sampled positions and its edges
    peers = [peer_bits(w, q, S, device=DEV) for q in range(n - 1)] + [own]
    full = torch.empty(L.flat_len, dtype=torch.int16, device=DEV)
    zs.gather_params(L, 0, 1, peers, full)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(full[r * S + tidx]), par_h), "gather: own slot"
    assert_gathered(full, 0, S, peers, idx, "config 2 gather")


def test_config2_full_shard_every_element():
    """The same Mistral-7B rank shard (905,000,000 elements, N = 8, rank 7,
    3 fused Adam steps), compared element by element over the whole shard:
    the oracle steps every element from the same gradients, streamed from
    the GPU in 32M-element chunks, and master, m, v and the bf16 shard must
    be bit-identical everywhere -- for three state arrays with eight rank
    buffers, and side by side for the benchmark's launch: the chunked state
    and the rank gradients chunked into one buffer."""
    w = WORKLOADS[2]
    n, r = w.n_ranks, w.n_ranks - 1
    L = zs.shard_init("zero3", n, r, list(w.units))
    S = L.shard_len
    CH = 1 << 25
    E = zs.STATE_CHUNK_DEFAULT
    assert CH % E == 0
    LC = L.chunk_state(E)
    master = master_init(w, S, device=DEV, rank=r)
    m = torch.zeros(S, device=DEV)
    v = torch.zeros(S, device=DEV)
    own = torch.empty(S, dtype=torch.int16, device=DEV)
    rows = -(-S // E)
    st_c = torch.zeros(LC.state_len, device=DEV)
    col = torch.zeros(rows * E, device=DEV)
    col[:S] = master
    st_c.view(rows, 3, E)[:, 0, :].copy_(col.view(rows, E))
    del col
    own_c = torch.empty(S, dtype=torch.int16, device=DEV)
    p_h = master.cpu().numpy()
    m_h = np.zeros(S, np.float32)
    v_h = np.zeros(S, np.float32)
    par_h = np.empty(S, np.uint16)
    tmp = np.empty(CH, np.float32)
    GE = zs.GRAD_CHUNK_DEFAULT
    grows = -(-S // GE)
    for t in range(w.steps):
        grads = [grad_bits(w, t, q, S, device=DEV) for q in range(n)]
        G = zs.Grads(grads, zs.BF16, zs.INDEX_SHARD)
        zs.adam_step(L, 0, 1, cfg_of(w, t + 1), master, m, v, own, zs.INDEX_SHARD, grads=G)
        gbuf = torch.zeros(LC.grad_len(GE), dtype=torch.int16, device=DEV)
        col = torch.zeros(grows * GE, dtype=torch.int16, device=DEV)
        for q in range(n):
            col[:S] = grads[q]
            gbuf.view(grows, n, GE)[:, q, :].copy_(col.view(grows, GE))
        del col
        zs.adam_step(LC, 0, 1, cfg_of(w, t + 1), *LC.state_views(st_c), own_c, zs.INDEX_SHARD,
                     grads=zs.Grads.chunked(gbuf, n, GE))
        hp = oracle_cfg(w).hparams(t + 1)
        for off in range(0, S, CH):
            k = min(CH, S - off)
            g = [host_bf16(gq[off:off + k]) for gq in grads]
            _c.rank_step(hp, g, 1.0, p_h[off:off + k], m_h[off:off + k], v_h[off:off + k],
                         par_h[off:off + k], tmp[:k])
        torch.cuda.synchronize()
        del grads, G, gbuf
    bad = {}
    for name, dev_t, want in (("master", master, p_h), ("m", m, m_h), ("v", v, v_h)):
        nbad = 0
        for off in range(0, S, CH):
            got = host_f32(dev_t[off:off + CH])
            nbad += int(np.count_nonzero(got.view(np.uint32) !=
                                         want[off:off + CH].view(np.uint32)))
        bad[name] = nbad
    nbad = {"master": 0, "m": 0, "v": 0}
    for off in range(0, S, CH):
        k = min(CH, S - off)
        got = unchunk_state(host_f32(st_c[off // E * 3 * E:(off + k + E - 1) // E * 3 * E]), E, k)
        for name, x, want in zip(("master", "m", "v"), got, (p_h, m_h, v_h)):
            nbad[name] += int(np.count_nonzero(x.view(np.uint32) !=
                                               want[off:off + k].view(np.uint32)))
    bad.update({f"chunked state and gradients: {k}": x for k, x in nbad.items()})
    for name, o in (("bf16 shard", own), ("chunked state and gradients: bf16 shard", own_c)):
        nb = 0
        for off in range(0, S, CH):
            nb += int(np.count_nonzero(host_bf16(o[off:off + CH]) != par_h[off:off + CH]))
        bad[name] = nb
    assert not any(bad.values()), f"elements differing from the oracle: {bad}"
