"""The library's calls under HIP graph capture (torch.cuda.CUDAGraph).

The library records no memset and allocates nothing, so a caller may capture
its launches in a graph. Each graph here is replayed several times. Between
the replays the program runs eager work of its own and synchronizes the
device. Every replay's output is compared bit for bit with the same calls
run eagerly on a second copy of the state, so a replay that reused stale
arguments or skipped a node would show.
"""
import numpy as np
import pytest
import torch

from synthetic import grad_bits, small_workload

pytestmark = pytest.mark.gpu

zs = None
DEV = "cuda:0"
REPLAYS = 4


def setup_module(module):
    global zs
    from fsdp_sharded_optimizer_shard_amd import zs as _zs
    zs = _zs


def _bits(t):
    return t.detach().cpu().numpy().view(np.uint32 if t.dtype == torch.float32 else np.uint16)


def _same(a, b, what):
    assert np.array_equal(_bits(a), _bits(b)), what


def _noise():
    # eager work of the program's own between replays
    x = torch.randn(1 << 20, device=DEV)
    return float((x * x).sum())


def _state(S, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    master = (torch.randn(S, generator=g) * 0.02).to(DEV)
    m = (torch.randn(S, generator=g) * 1e-4).to(DEV)
    v = (torch.rand(S, generator=g) * 1e-7).to(DEV)
    return master, m, v


def _replay_and_compare(capture, eager, outputs_g, outputs_e):
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        capture()
    for rep in range(REPLAYS):
        eager()
        graph.replay()
        _noise()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(outputs_g, outputs_e)):
            _same(a, b, f"replay {rep}, output {k}")


def test_fused_step_and_gather_in_a_graph():
    units, n, r = [5000, 3000, 777], 4, 1
    L = zs.shard_init("zero3", n, r, units)
    S, P = L.shard_len, L.flat_len
    w = small_workload(units, n, "zero3", cfg=12)
    grads = [grad_bits(w, 0, q, S, device=DEV) for q in range(n)]
    peers = [None if q == r else grad_bits(w, 1, q, S, device=DEV) for q in range(n)]
    cfg = zs.adam_cfg(lr=1e-3, weight_decay=0.01, decoupled=True, step=3)
    G = list(_state(S, 5)) + [torch.zeros(P, dtype=torch.int16, device=DEV)]
    E = [t.clone() for t in G]

    def step(st):
        zs.adam_step(L, 0, len(units), cfg, st[0], st[1], st[2], st[3],
                     grads=zs.Grads(grads, zs.BF16, zs.INDEX_SHARD))
        zs.gather_params(L, 0, len(units), peers, st[3])

    W = [t.clone() for t in G]          # warm-up call before capture
    step(W)
    torch.cuda.synchronize()
    _replay_and_compare(lambda: step(G), lambda: step(E), G, E)


@pytest.mark.parametrize("GE", [0, 512])
def test_chunked_state_steps_in_a_graph(GE):
    # master, m and v in one chunked buffer (and, GE > 0, the rank gradients
    # in one chunked receive buffer, the benchmark's launch): the fused step
    # with its gather, then the two-pass path, captured and replayed
    units, n, r, E = [5000, 3000, 777], 4, 1, 1024
    L = zs.shard_init("zero3", n, r, units).chunk_state(E)
    S, P = L.shard_len, L.flat_len
    w = small_workload(units, n, "zero3", cfg=12)
    if GE:
        recv = grad_bits(w, 0, 0, L.grad_len(GE), device=DEV)
        grads = [recv[q * GE:] for q in range(n)]
    else:
        grads = [grad_bits(w, 0, q, S, device=DEV) for q in range(n)]
    peers = [None if q == r else grad_bits(w, 1, q, S, device=DEV) for q in range(n)]
    cfg = zs.adam_cfg(lr=1e-3, weight_decay=0.01, decoupled=True, step=3)
    npart = zs.reduce_partials_count(L, 0, len(units))

    def buffers():
        g = torch.Generator(device="cpu")
        g.manual_seed(11)
        st = (torch.randn(L.state_len, generator=g) * 1e-3).abs().to(DEV)
        return [st, torch.zeros(P, dtype=torch.int16, device=DEV), torch.empty(S, device=DEV),
                torch.empty(npart, dtype=torch.float64, device=DEV), torch.empty(1, device=DEV)]

    def step(b):
        G = zs.Grads(grads, zs.BF16, zs.INDEX_SHARD, GE)
        zs.adam_step(L, 0, len(units), cfg, *L.state_views(b[0]), b[1], grads=G)
        zs.gather_params(L, 0, len(units), peers, b[1])
        zs.reduce_shard(L, 0, len(units), G, b[2], b[3], npart)
        zs.clip_coef(b[3], npart, 1e-3, b[4])
        zs.adam_step(L, 0, len(units), cfg, *L.state_views(b[0]), b[1], grad_fp32=b[2],
                     clip_coef=b[4])

    G_, E_ = buffers(), buffers()
    step(buffers())
    torch.cuda.synchronize()
    _replay_and_compare(lambda: step(G_), lambda: step(E_), G_, E_)


def test_launches_with_the_occupancy_reservation_in_a_graph():
    # the fused and apply passes and the gather reserve LDS (their occupancy
    # caps) only for launches of more blocks than fit on the GPU at once, 5
    # and 13 per CU (the reduce pass runs uncapped): a shard of 2.5 million
    # elements (2442 step tiles of 1024; 1222 gather tiles of 2048 for each
    # of 3 sources) takes both paths, under capture
    units, n, r = [8_000_000, 2_000_003], 4, 1
    L = zs.shard_init("zero3", n, r, units)
    S, P = L.shard_len, L.flat_len
    assert S > 256 * 5 * 1024
    gather_tiles = sum(-(-L.query(u)["shard_len"] // 2048) for u in range(len(units)))
    assert gather_tiles * (n - 1) > 256 * 13
    w = small_workload(units, n, "zero3", cfg=12)
    grads = [grad_bits(w, 0, q, S, device=DEV) for q in range(n)]
    peers = [None if q == r else grad_bits(w, 1, q, S, device=DEV) for q in range(n)]
    cfg = zs.adam_cfg(lr=1e-3, step=4)
    npart = zs.reduce_partials_count(L, 0, len(units))

    def buffers():
        master, m, v = _state(S, 7)
        return [master, m, v, torch.zeros(P, dtype=torch.int16, device=DEV),
                master.clone(), m.clone(), v.clone(), torch.zeros(P, dtype=torch.int16, device=DEV),
                torch.empty(S, device=DEV), torch.empty(npart, dtype=torch.float64, device=DEV),
                torch.empty(1, device=DEV)]

    def step(b):
        G = zs.Grads(grads, zs.BF16, zs.INDEX_SHARD)
        zs.adam_step(L, 0, len(units), cfg, b[0], b[1], b[2], b[3], grads=G)
        zs.gather_params(L, 0, len(units), peers, b[3])
        zs.reduce_shard(L, 0, len(units), G, b[8], b[9], npart)
        zs.clip_coef(b[9], npart, 1e-3, b[10])
        zs.adam_step(L, 0, len(units), cfg, b[4], b[5], b[6], b[7], grad_fp32=b[8],
                     clip_coef=b[10])

    G_, E_ = buffers(), buffers()
    step(buffers())
    torch.cuda.synchronize()
    _replay_and_compare(lambda: step(G_), lambda: step(E_), G_, E_)
    assert float(E_[10]) < 1.0


def test_two_pass_clip_in_a_graph():
    units, n, r = [25000, 9001], 4, 2
    L = zs.shard_init("zero2", n, r, units)
    S, P = L.shard_len, L.flat_len
    w = small_workload(units, n, "zero2", cfg=12)
    grads = [grad_bits(w, 0, q, P, device=DEV) for q in range(n)]
    cfg = zs.adam_cfg(lr=1e-3, step=2)
    npart = zs.reduce_partials_count(L, 0, len(units))

    def buffers():
        master, m, v = _state(S, 6)
        return [master, m, v, torch.zeros(P, dtype=torch.int16, device=DEV),
                torch.empty(S, device=DEV), torch.empty(npart, dtype=torch.float64, device=DEV),
                torch.empty(1, device=DEV), torch.empty(1, dtype=torch.float64, device=DEV)]

    def step(b):
        master, m, v, out, gsh, part, coef, norm = b
        zs.reduce_shard(L, 0, len(units), zs.Grads(grads, zs.BF16, zs.INDEX_FULL), gsh,
                        part, npart)
        # a small max_norm, so that the coefficient is below 1 and applied
        zs.clip_coef(part, npart, 1e-3, coef, norm)
        zs.adam_step(L, 0, len(units), cfg, master, m, v, out, grad_fp32=gsh, clip_coef=coef)

    G, E = buffers(), buffers()
    step(buffers())
    torch.cuda.synchronize()
    _replay_and_compare(lambda: step(G), lambda: step(E), G, E)
    assert float(E[6]) < 1.0


def test_table_clip_steps_replayed_from_one_graph():
    """The two-pass clip path captured once, [reduce with partials, clip
    coefficient, zero_adam_step_table from the fp32 gradient, step advance],
    replays as steps 1..T with a learning-rate schedule and new gradients
    each step, bit-identical to the eager path with zero_adam_step."""
    units, n, r, T = [25000, 9001], 4, 2, 4
    L = zs.shard_init("zero2", n, r, units)
    S, P = L.shard_len, L.flat_len
    U = len(units)
    w = small_workload(units, n, "zero2", cfg=12)
    npart = zs.reduce_partials_count(L, 0, U)
    cfgs = [zs.adam_cfg(lr=1e-3 * (1.0 - 0.2 * k), weight_decay=0.01, decoupled=True,
                        step=k + 1) for k in range(T)]
    table = zs.adam_table_device(cfgs, DEV)
    counter = torch.ones(1, dtype=torch.int64, device=DEV)
    grads = [torch.empty(P, dtype=torch.int16, device=DEV) for _ in range(n)]
    gr = zs.Grads(grads, zs.BF16, zs.INDEX_FULL)

    def buffers():
        master, m, v = _state(S, 11)
        return [master, m, v, torch.zeros(P, dtype=torch.int16, device=DEV),
                torch.empty(S, device=DEV), torch.empty(npart, dtype=torch.float64, device=DEV),
                torch.empty(1, device=DEV)]

    def two_pass(b, adam):
        master, m, v, out, gsh, part, coef = b
        zs.reduce_shard(L, 0, U, gr, gsh, part, npart)
        # a small max_norm, so that the coefficient is below 1 and applied
        zs.clip_coef(part, npart, 1e-3, coef)
        adam(master, m, v, out, gsh, coef)

    G, E = buffers(), buffers()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        two_pass(G, lambda *a: zs.adam_step_table(L, 0, U, table, T, counter, *a[:4],
                                                  grad_fp32=a[4], clip_coef=a[5]))
        zs.step_advance(counter)
    for k in range(T):
        for q in range(n):
            grads[q].copy_(grad_bits(w, k, q, P, device=DEV))
        two_pass(E, lambda *a: zs.adam_step(L, 0, U, cfgs[k], *a[:4], grad_fp32=a[4],
                                            clip_coef=a[5]))
        graph.replay()
        _noise()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(G, E)):
            _same(a, b, f"step {k + 1}, output {i}")
        assert float(E[6]) < 1.0
        assert int(counter.item()) == k + 2


@pytest.mark.parametrize("ao,bo", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_gemm_in_a_graph(ao, bo):
    M, N, K = 264, 520, 200
    gen = torch.Generator(device="cpu")
    gen.manual_seed(100 + 2 * ao + bo)
    A = (torch.randn((K, M) if ao else (M, K), generator=gen)).to(torch.bfloat16).to(DEV)
    B = (torch.randn((K, N) if bo else (N, K), generator=gen)).to(torch.bfloat16).to(DEV)
    order = (zs.K_INNER, zs.K_OUTER)
    Cg = torch.empty((M, N), device=DEV)
    Ce = torch.empty((M, N), device=DEV)

    def run(C):
        zs.gemm_bf16(M, N, K, A.view(torch.int16), A.shape[1], order[ao], B.view(torch.int16),
                     B.shape[1], order[bo], C, N, zs.FP32)

    def eager():
        Cg.fill_(float("nan"))           # each replay must rewrite every element
        run(Ce)

    run(Ce)
    torch.cuda.synchronize()
    _replay_and_compare(lambda: run(Cg), eager, [Cg], [Ce])


def test_two_stream_sweep_in_a_graph():
    """The FSDP sweep forks its gather stream from the capturing step stream
    through events and joins it back before returning, so the whole
    two-stream schedule is captured as one graph."""
    units, n, r = [4096, 1000, 2500, 777], 4, 3
    U = len(units)
    L = zs.shard_init("fsdp", n, r, units)
    q = [L.query(u) for u in range(U)]
    S = L.shard_len
    w = small_workload(units, n, "fsdp", cfg=12)
    grads = [[grad_bits(w, 0, k, q[u]["shard_len"], device=DEV, unit=u) for k in range(n)]
             for u in range(U)]
    peers = [[None if k == r else grad_bits(w, 1, k, q[u]["shard_len"], device=DEV, unit=u)
              for k in range(n)] for u in range(U)]
    cfg = zs.adam_cfg(lr=1e-3, weight_decay=0.01, decoupled=True, step=2)
    gs = torch.cuda.Stream()

    def buffers():
        return list(_state(S, 7)) + [torch.zeros(x["padded_len"], dtype=torch.int16, device=DEV)
                                     for x in q]

    def sweep(b):
        ios = [(grads[u], peers[u], b[3 + u]) for u in range(U)]
        zs.fsdp_sweep(L, 0, U, cfg, zs.BF16, ios, b[0], b[1], b[2], 2, gather_stream=gs)

    G, E = buffers(), buffers()
    sweep(buffers())
    torch.cuda.synchronize()
    _replay_and_compare(lambda: sweep(G), lambda: sweep(E), G, E)


def test_linear_layer_in_a_graph():
    # forward and backward of the FSDP linear layer, padding rows included
    inf, outf, n, r, batch = 200, 136, 4, 1, 64
    L = zs.shard_init_rows("fsdp2", n, r, [(inf, outf)])
    s = L.query(0)["shard_len"]
    P = L.flat_len
    gen = torch.Generator(device="cpu")
    gen.manual_seed(8)

    def bf(*shape):
        return torch.randn(shape, generator=gen).to(torch.bfloat16).view(torch.int16).to(DEV)

    shards = [bf(s) for _ in range(n)]
    x, dy = bf(batch, inf), bf(batch, outf)

    def buffers():
        return [torch.zeros(P, dtype=torch.int16, device=DEV),
                torch.empty((batch, outf), device=DEV), torch.empty((batch, inf), device=DEV),
                torch.empty(P, device=DEV)]

    def layer(b):
        w_full, y, dx, dw = b
        zs.fsdp_linear_forward(L, 0, shards, batch, x, w_full, y, zs.FP32)
        zs.fsdp_linear_backward(L, 0, shards, batch, x, dy, w_full, dx, dw, zs.FP32)

    def eager():
        for t in G[1:]:
            t.fill_(float("nan"))
        layer(E)

    G, E = buffers(), buffers()
    layer(buffers())
    torch.cuda.synchronize()
    _replay_and_compare(lambda: layer(G), eager, G, E)


def test_table_steps_replayed_from_one_graph():
    """One captured step [zero_adam_step_table, gather, zero_step_advance]
    replays as steps 1..T with a learning-rate schedule, each replay
    bit-identical to zero_adam_step with that step's configuration; a
    counter past the table leaves every buffer untouched."""
    units, n, r, T = [5000, 3000, 777], 4, 1, 5
    L = zs.shard_init("zero3", n, r, units)
    S, P = L.shard_len, L.flat_len
    w = small_workload(units, n, "zero3", cfg=13)
    grads = [grad_bits(w, 0, q, S, device=DEV) for q in range(n)]
    peers = [None if q == r else grad_bits(w, 1, q, S, device=DEV) for q in range(n)]
    cfgs = [zs.adam_cfg(lr=1e-3 * (1.0 - 0.15 * k), weight_decay=0.01, decoupled=True,
                        step=k + 1) for k in range(T)]
    table = zs.adam_table_device(cfgs, DEV)
    counter = torch.zeros(1, dtype=torch.int64, device=DEV)
    G = list(_state(S, 9)) + [torch.zeros(P, dtype=torch.int16, device=DEV)]
    E = [t.clone() for t in G]
    gr = zs.Grads(grads, zs.BF16, zs.INDEX_SHARD)

    def table_step(st):
        zs.adam_step_table(L, 0, len(units), table, T, counter, st[0], st[1], st[2], st[3],
                           grads=gr)
        zs.gather_params(L, 0, len(units), peers, st[3])
        zs.step_advance(counter)

    # warm-up with the counter at 0: no entry, so nothing is written
    W = [t.clone() for t in G]
    zs.adam_step_table(L, 0, len(units), table, T, counter, W[0], W[1], W[2], W[3], grads=gr)
    torch.cuda.synchronize()
    for a, b in zip(W, G):
        _same(a, b, "counter 0 must leave the state untouched")
    counter.fill_(1)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        table_step(G)
    for k in range(T):
        zs.adam_step(L, 0, len(units), cfgs[k], E[0], E[1], E[2], E[3], grads=gr)
        zs.gather_params(L, 0, len(units), peers, E[3])
        graph.replay()
        _noise()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(G, E)):
            _same(a, b, f"step {k + 1}, output {i}")
        assert int(counter.item()) == k + 2
    before = [t.clone() for t in G]
    graph.replay()                      # counter T + 1: past the table
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(G, before)):
        _same(a, b, f"past the table, output {i}")


@pytest.mark.parametrize("GE", [0, 64])
def test_table_sweep_replayed_from_one_graph(GE):
    """One captured two-stream zero_fsdp_sweep_table call replays as the
    sweeps of steps 1..T (a learning-rate schedule), each bit-identical to
    zero_fsdp_sweep with that step's configuration; GE > 0 with each unit's
    rank gradients in one chunked receive buffer."""
    units, n, r, T = [4096, 1000, 2500, 777], 4, 3, 4
    U = len(units)
    L = zs.shard_init("fsdp", n, r, units)
    q = [L.query(u) for u in range(U)]
    S = L.shard_len
    w = small_workload(units, n, "fsdp", cfg=12)
    if GE:
        recv = [grad_bits(w, 0, 0, L.grad_len(GE, u, u + 1), device=DEV, unit=u)
                for u in range(U)]
        grads = [[recv[u][k * GE:] for k in range(n)] for u in range(U)]
    else:
        grads = [[grad_bits(w, 0, k, q[u]["shard_len"], device=DEV, unit=u) for k in range(n)]
                 for u in range(U)]
    peers = [[None if k == r else grad_bits(w, 1, k, q[u]["shard_len"], device=DEV, unit=u)
              for k in range(n)] for u in range(U)]
    cfgs = [zs.adam_cfg(lr=2e-3 * (1.0 - 0.2 * k), weight_decay=0.01, decoupled=True, step=k + 1)
            for k in range(T)]
    table = zs.adam_table_device(cfgs, DEV)
    counter = torch.ones(1, dtype=torch.int64, device=DEV)
    gs = torch.cuda.Stream()

    def buffers():
        return list(_state(S, 11)) + [torch.zeros(x["padded_len"], dtype=torch.int16, device=DEV)
                                      for x in q]

    def ios(b):
        return [(grads[u], peers[u], b[3 + u]) for u in range(U)]

    G, E = buffers(), buffers()
    W = buffers()
    zs.fsdp_sweep(L, 0, U, cfgs[0], zs.BF16, ios(W), W[0], W[1], W[2], 2, gather_stream=gs,
                  grad_chunk=GE)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        zs.fsdp_sweep_table(L, 0, U, table, T, counter, zs.BF16, ios(G), G[0], G[1], G[2], 2,
                            gather_stream=gs, grad_chunk=GE)
    for k in range(T):
        zs.fsdp_sweep(L, 0, U, cfgs[k], zs.BF16, ios(E), E[0], E[1], E[2], 2, gather_stream=gs,
                      grad_chunk=GE)
        graph.replay()
        _noise()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(G, E)):
            _same(a, b, f"step {k + 1}, output {i}")
        assert int(counter.item()) == k + 2
