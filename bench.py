"""Benchmark: one data-parallel rank's sharded optimizer step on one MI355X.

Default workload (the headline): the Mistral-7B-sized ZeRO-3 rank shard --
Psi = 7.24e9, N = 8 simulated ranks, this GPU is rank 7 and owns
905,000,000 elements.  Inputs are synthetic and resident in HBM before
timing: 8 bf16 rank-gradient shards ~N(0, 1e-3), fp32 master ~N(0, 0.02),
m = v = 0, 7 peer bf16 parameter shards.  One step is the whole hot path:
  1. zero_adam_step, fused: reduce the 8 rank gradients in fp32, divide by
     8, Adam (lr 1e-3, betas 0.9 / 0.999, eps 1e-8), round to bf16 and store
     this rank's slice into the 7.24e9-element flat parameter buffer;
  2. zero_gather_params: pack the 7 peer shards into the flat buffer.
Every timed step is a real optimizer step (t increases).

Prints one JSON line.  value = shard parameters updated per second.
roofline: the fused kernel's algorithmic bytes (42 B per shard element:
16 gradient + 12 state read + 12 state write + 2 bf16) over its mean
duration from HIP events on the launch stream, against 8 TB/s.
cpu_baseline: the CPU oracle (single thread) timed on a bounded sample of
the same shard (the first elements, streamed in chunks from the GPU).

--config 0 | 1 | 3 | 4 measures the other workloads instead (same JSON
shape, their own metric): the tiny ZeRO-2 step, the GPT-2-small buffer with
the global-norm clip, the Megatron distributed optimizer (fp32 main-gradient
accumulation of 4 micro-batches + fp32 reduce + Adam + gather), and the
Llama-70B FSDP full shard at N = 64 swept unit by unit.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "fused_step_7b_n8_counters.md")
KERNELS_SRC = os.path.join(ROOT, "fsdp_sharded_optimizer_shard_amd", "csrc", "kernels.hip")
GEMM_COUNTERS = os.path.join(ROOT, "profiles", "gemm_fsdp_linear_mistral_up_counters.md")
GEMM_SRC = os.path.join(ROOT, "fsdp_sharded_optimizer_shard_amd", "csrc", "gemm.hip")
HEADLINE_METRIC = "shard optimizer-step params/sec at 7B N=8; achieved HBM GB/s vs peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--ddp-buckets", action="store_true",
                    help="config 1 only: one DDP replica, each bucket's reduce launched as "
                         "backward would produce it (last bucket first), then clip + AdamW")
    ap.add_argument("--fsdp-linear", action="store_true",
                    help="the hand-written FSDP linear layer (Mistral-7B MLP up projection, "
                         "in 4096, out 14336, 4096 tokens per rank, N=8, rank 7) instead of a "
                         "config")
    ap.add_argument("--vs-library", action="store_true",
                    help="with --fsdp-linear: also time the three GEMMs against torch.mm "
                         "(hipBLASLt) on the same operands, alternately")
    ap.add_argument("--vs-torch", action="store_true",
                    help="headline workload: also time the same step composed from PyTorch "
                         "ops (rank sum, torch.optim.Adam(fused=True), bf16 cast) on the same "
                         "inputs, alternating with the fused kernel")
    ap.add_argument("--one-stream", action="store_true",
                    help="config 4 only: skip the two-stream sweep, so a kernel trace holds "
                         "only launches that do not overlap")
    ap.add_argument("--fsdp2", action="store_true",
                    help="config 2 only: the exact Mistral-7B per-parameter dim-0 layout "
                         "(291 parameters) instead of one flat unit")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=12.0,
                    help="oracle time budget for the CPU baseline (headline and --config 4); 0 skips it")
    ap.add_argument("--placements", type=int, default=3,
                    help="headline workload: time the step on this many fresh allocations of "
                         "its buffers and report the median one (physical placement moves the "
                         "fused kernel by up to ~15 %%)")
    ap.add_argument("--calibrate-mix", type=int, default=0, metavar="PLACEMENTS",
                    help="instead of a step: the fused 7B step against zero_stream_mix (its "
                         "streams without the arithmetic, its reads, its writes) on this many "
                         "fresh placements")
    ap.add_argument("--state-chunk", type=int, default=None, metavar="E",
                    help="master, m and v of every workload as one buffer of E-element "
                         "chunks (zero_layout_chunk_state); 0 keeps three arrays; default: "
                         "the library's ZERO_STATE_CHUNK_DEFAULT")
    ap.add_argument("--grad-chunk", type=int, default=None, metavar="E",
                    help="the rank gradients of the 7B step, of each rank of --config 1, of "
                         "the peers of --config 3 and of each unit of --config 4 as one "
                         "receive buffer of rows of E elements per rank (zero_grads.chunk); 0 "
                         "keeps one buffer per rank (full-indexed for --config 1); default: "
                         "the library's ZERO_GRAD_CHUNK_DEFAULT")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="instead of a step, run a plain bf16 copy of BYTES through "
                         "zero_gather_params (counter calibration)")
    return ap.parse_args()


class Phases:
    """HIP-event timing of named phases on one stream; several launches of
    one phase in a step are summed, and each launch is also kept.  A phase
    run with chain=True starts at the previous phase's end event instead of
    an event of its own: for launches issued back to back with nothing else
    enqueued between them, it halves the events (each costs a few
    microseconds of stream time, which adds up over short kernels)."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.marks = []        # (name, start_event, end_event) in launch order

    def run(self, name, fn, chain=False):
        E = self.torch.cuda.Event
        if chain and self.marks:
            a = self.marks[-1][2]
        else:
            a = E(enable_timing=True)
            a.record(self.stream)
        b = E(enable_timing=True)
        fn()
        b.record(self.stream)
        self.marks.append((name, a, b))

    def summary(self, steps):
        per = {}
        for name, a, b in self.marks:
            per.setdefault(name, []).append(a.elapsed_time(b))
        return {k: {"ms_per_step": sum(v) / steps, "launches_per_step": len(v) // steps,
                    "ms_per_launch_mean": sum(v) / len(v), "ms_per_launch_min": min(v),
                    "ms_per_launch_median": sorted(v)[len(v) // 2],
                    "ms_per_launch_max": max(v)}
                for k, v in per.items()}


def timed(args, torch, step):
    """warmup, then exactly `steps` steps between synchronisations; returns
    (wall ms per step, phase summary)."""
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    ph = Phases(torch, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(ph)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return 1e3 * wall / args.steps, ph.summary(args.steps)


def phase(ph, name, fn, chain=False):
    if ph is None:
        fn()
    else:
        ph.run(name, fn, chain)


def roofline(name, bytes_per_launch, ms_per_launch, traffic=None, counters=COUNTERS):
    gbps = bytes_per_launch / (ms_per_launch * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": name, "achieved": gbps, "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS, "traffic": traffic,
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                            "copy-calibrated)",
            "traffic_source": (f"the committed counter summary {os.path.relpath(counters, ROOT)}, "
                               "taken on the kernel source whose sha256 it records; not measured "
                               "in this run (null when the source has changed since or no "
                               "summary covers this kernel)"),
            "algorithmic_bytes": bytes_per_launch}


def base_line(args, metric, value, unit, ms, workload, **config):
    return {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic (seeded N(0,1e-3) bf16 rank grads, N(0,0.02) fp32 master)",
            "config": {"workload": workload, **config}}


def add_rates(kernels, name, bytes_per_launch):
    k = kernels[name]
    k["bytes_per_launch"] = bytes_per_launch
    k["gbps"] = bytes_per_launch / (k["ms_per_launch_mean"] * 1e-3) / 1e9


# ------------------------------------------------------------ workloads --

class State:
    """One shard's fp32 master, m and v in the layout's state format: three
    arrays, or one buffer of E-element chunks (master | m | v per chunk)."""

    def __init__(self, torch, L, master0):
        S, E = L.shard_len, L.state_chunk
        self.E, self.buf = E, None
        if E == 0:
            self.views = (master0, torch.zeros(S, device=master0.device),
                          torch.zeros(S, device=master0.device))
            return
        rows = -(-S // E)
        self.buf = torch.zeros(L.state_len, device=master0.device)
        col = torch.zeros(rows * E, device=master0.device)
        col[:S] = master0
        self.buf.view(rows, 3, E)[:, 0, :].copy_(col.view(rows, E))
        del col
        self.views = L.state_views(self.buf)

    def master(self, off, n):
        """The master values of shard elements [off, off + n) (a tensor)."""
        if self.E == 0:
            return self.views[0][off:off + n]
        E = self.E
        r0, r1 = off // E, -(-(off + n) // E)
        return self.buf.view(-1, 3, E)[r0:r1, 0, :].reshape(-1)[off - r0 * E:off - r0 * E + n]


def state_desc(E):
    return ("three fp32 arrays (master, m, v)" if E == 0 else
            f"one fp32 buffer of {E}-element chunks, master | m | v per chunk")


class RankGrads:
    """The N ranks' shard-indexed bf16 gradients of S elements each (a
    shard, or the largest unit's slice for per-unit calls): N buffers, or
    one receive buffer of rows of E elements per rank (rank q's element i at
    (i // E) N E + q E + i % E), the chunked format zero_grads.chunk names."""

    def __init__(self, torch, zs, draws, E):
        self.zs, self.E, self.N, self.S = zs, E, len(draws), draws[0].numel()
        self._grads = None
        if E == 0:
            self.bufs, self.buf = list(draws), None
            return
        rows, dev = -(-self.S // E), draws[0].device
        self.bufs = None
        self.buf = torch.zeros(rows * self.N * E, dtype=torch.int16, device=dev)
        cells = self.buf.view(rows, self.N, E)
        col = torch.zeros(rows * E, dtype=torch.int16, device=dev)
        for q, d in enumerate(draws):
            col[:self.S] = d
            cells[:, q, :].copy_(col.view(rows, E))
        del col

    @property
    def grads(self):
        """The zs.Grads the library takes (made on first use)."""
        if self._grads is None:
            zs = self.zs
            self._grads = (zs.Grads(self.bufs, zs.BF16, zs.INDEX_SHARD) if self.E == 0 else
                           zs.Grads.chunked(self.buf, self.N, self.E))
        return self._grads

    @property
    def ptrs(self):
        """Rank q's pointer for each q, as the library takes them."""
        return self.bufs if self.E == 0 else [self.buf[q * self.E:] for q in range(self.N)]

    def rank(self, q, off, n):
        """Rank q's gradient for shard elements [off, off + n) (a tensor)."""
        if self.E == 0:
            return self.bufs[q][off:off + n]
        E = self.E
        r0, r1 = off // E, -(-(off + n) // E)
        return self.buf.view(-1, self.N, E)[r0:r1, q, :].reshape(-1)[off - r0 * E:off - r0 * E + n]

    def ranks(self):
        """One sliceable per rank: ranks()[q][a:b] is rank q's [a, b)."""
        me = self

        class _Rank:
            def __init__(self, q):
                self.q = q

            def __getitem__(self, sl):
                return me.rank(self.q, sl.start, sl.stop - sl.start)

        return [_Rank(q) for q in range(self.N)]


def grad_desc(E, N):
    return (f"{N} bf16 buffers, one per rank" if E == 0 else
            f"one bf16 buffer of rows of {E} elements per rank, {N} ranks per row")


def headline_buffers(torch, zs, w, L, S, N, r, dev, rank_peers=True, grad_chunk=0):
    """A fresh allocation of the headline step's buffers (one placement)."""
    from synthetic import grad_bits, master_init
    draws = [grad_bits(w, 0, q, S, device=dev) for q in range(N)]
    grads = RankGrads(torch, zs, draws, grad_chunk)
    assert grad_chunk == 0 or grads.buf.numel() == L.grad_len(grad_chunk)
    del draws
    st = State(torch, L, master_init(w, S, device=dev, rank=r))
    full = torch.empty(L.flat_len, dtype=torch.int16, device=dev)
    peers = ([torch.full((S,), q + 1, dtype=torch.int16, device=dev) for q in range(N - 1)]
             if rank_peers else [])
    torch.cuda.synchronize()
    return grads, st, full, peers


def state_chunk(args, zs):
    return zs.STATE_CHUNK_DEFAULT if args.state_chunk is None else args.state_chunk


def grad_chunk(args, zs):
    return zs.GRAD_CHUNK_DEFAULT if args.grad_chunk is None else args.grad_chunk


def release(torch, *objs):
    """Drop the tensors and return their memory to the device, so that the
    next allocation is a fresh placement."""
    for o in objs:
        if isinstance(o, list):
            o.clear()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def run_headline(args, torch, zs, np):
    """The step on `args.placements` fresh allocations of its buffers, each
    timed as the contract says (warmup, then exactly `steps` steps); the
    line reports the placement with the median step time, and every
    placement's times under "placements"."""
    from synthetic import WORKLOADS
    dev = torch.device("cuda:0")
    w = WORKLOADS[2]
    N, r = w.n_ranks, w.n_ranks - 1
    if args.fsdp2:
        from synthetic import mistral7b_shapes
        L = zs.shard_init_rows("fsdp2", N, r, mistral7b_shapes())
    else:
        L = zs.shard_init("zero3", N, r, list(w.units))
    L = L.chunk_state(state_chunk(args, zs))
    GE = grad_chunk(args, zs)
    S = L.shard_len
    U = L.info()["n_units"]
    print(f"# setup: {w.name}, rank {r}, shard {S} elements, {U} units, "
          f"{args.placements} placements, state: {state_desc(L.state_chunk)}, "
          f"gradients: {grad_desc(GE, N)}", file=sys.stderr, flush=True)
    fused_b, gather_b = 42 * S, 4 * (N - 1) * S
    runs = []
    cpu = cmp = None
    for k in range(args.placements):
        grads, st, full, peers = headline_buffers(torch, zs, w, L, S, N, r, dev, grad_chunk=GE)
        master, m, v = st.views
        shard_ptrs = peers + [None]                  # own slice is written by the step
        G = grads.grads
        t = [0]

        def step(ph):
            t[0] += 1
            cfg = zs.adam_cfg(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, step=t[0])
            phase(ph, "fused_reduce_adam_cast",
                  lambda: zs.adam_step(L, 0, U, cfg, master, m, v, full, zs.INDEX_FULL, grads=G))
            phase(ph, "gather_7_peers", lambda: zs.gather_params(L, 0, U, shard_ptrs, full))

        ms, kern = timed(args, torch, step)
        add_rates(kern, "fused_reduce_adam_cast", fused_b)
        add_rates(kern, "gather_7_peers", gather_b)
        runs.append((ms, kern))
        print(f"# placement {k}: {ms:.3f} ms per step, fused "
              f"{kern['fused_reduce_adam_cast']['ms_per_launch_mean']:.3f} ms, gather "
              f"{kern['gather_7_peers']['ms_per_launch_mean']:.3f} ms", file=sys.stderr,
              flush=True)
        if k == args.placements - 1:
            if args.cpu_baseline_seconds > 0:
                cpu = cpu_baseline(w, grads.ranks(), st.master, S, r, args.cpu_baseline_seconds)
            if args.vs_torch:
                cmp = step_vs_torch(torch, zs, L, U, w, grads, st, full, G, r, S)
        del G, shard_ptrs
        release(torch, peers)
        del grads, st, master, m, v, full, peers
        torch.cuda.empty_cache()
    order = sorted(range(len(runs)), key=lambda i: runs[i][0])
    ms, kern = runs[order[len(order) // 2]]
    out = base_line(args, HEADLINE_METRIC, S / (ms * 1e-3), "params/s", ms,
                    ("Mistral-7B FSDP2 per-parameter (291 params, dim-0 rows) " if args.fsdp2
                     else "Mistral-7B ZeRO-3 ") +
                    "rank shard step: reduce 8 bf16 rank grads + Adam + "
                    "bf16 cast into the flat buffer + gather of 7 peer shards",
                    psi=L.flat_len, n_ranks=N, rank=r, shard_elems=S, units=U,
                    state_layout=state_desc(L.state_chunk), grad_layout=grad_desc(GE, N),
                    algorithmic_bytes_per_step=fused_b + gather_b)
    out["step_gbps"] = (fused_b + gather_b) / (ms * 1e-3) / 1e9
    out["state_gbps_16psi_over_n"] = 16 * S / (ms * 1e-3) / 1e9
    out["kernels"] = kern
    out["placements"] = {
        "what": "the step timed on each fresh allocation of its buffers (warmup, then `steps` "
                "steps each); value, ms_per_step, kernels and roofline are the median "
                "placement's",
        "ms_per_step": [x[0] for x in runs],
        "fused_ms_per_launch": [x[1]["fused_reduce_adam_cast"]["ms_per_launch_mean"]
                                for x in runs],
        "gather_ms_per_launch": [x[1]["gather_7_peers"]["ms_per_launch_mean"] for x in runs],
        "median_index": order[len(order) // 2]}
    out["roofline"] = roofline("fused_reduce_adam_cast (step_kernel<fused, N=8, bf16>)", fused_b,
                               kern["fused_reduce_adam_cast"]["ms_per_launch_mean"],
                               counter_traffic())
    out["cpu_baseline"] = cpu
    if cmp is not None:
        out["torch_comparison"] = cmp
    return out


def step_vs_torch(torch, zs, L, U, w, grads, st, full, G, r, S, rounds=5, iters=5):
    """The rank's reduce + Adam + bf16 cast composed from PyTorch ops on the
    same inputs: the fp32 sum of the N bf16 gradients in rank order (in-place
    mixed-dtype adds), one division by N, torch.optim.Adam(fused=True) on an
    fp32 copy of the master, and the bf16 cast into the rank's slice of the
    flat buffer.  Timed alternately with zero_adam_step (the fused kernel),
    `iters` steps per round, on the current stream with HIP events.  The
    PyTorch side gets each rank's gradient as its own contiguous tensor (a
    copy when the kernel's are chunked)."""
    N = grads.N
    master, m, v = st.views
    gb = [grads.rank(q, 0, S).contiguous().view(torch.bfloat16) for q in range(N)]
    own = full.view(torch.bfloat16)[r * S:(r + 1) * S]
    p = torch.nn.Parameter(st.master(0, S).detach().clone())
    acc = torch.empty(S, device=master.device)
    try:
        opt = torch.optim.Adam([p], lr=w.lr, betas=(w.beta1, w.beta2), eps=w.eps, fused=True)
        kind = "torch.optim.Adam(fused=True)"
    except (RuntimeError, ValueError):
        opt = torch.optim.Adam([p], lr=w.lr, betas=(w.beta1, w.beta2), eps=w.eps, foreach=True)
        kind = "torch.optim.Adam(foreach=True)"

    def torch_step():
        acc.copy_(gb[0])
        for q in range(1, N):
            acc.add_(gb[q])
        acc.div_(N)
        p.grad = acc
        opt.step()
        own.copy_(p.detach())

    t = [1000]

    def ours():
        t[0] += 1
        cfg = zs.adam_cfg(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, step=t[0])
        zs.adam_step(L, 0, U, cfg, master, m, v, full, zs.INDEX_FULL, grads=G)

    E = torch.cuda.Event
    res = {"ours": [], "torch": []}
    for fn in (ours, torch_step):        # warm-up
        fn()
    for _ in range(rounds):
        for name, fn in (("ours", ours), ("torch", torch_step)):
            a, b = E(enable_timing=True), E(enable_timing=True)
            a.record()
            for _ in range(iters):
                fn()
            b.record()
            b.synchronize()
            res[name].append(a.elapsed_time(b) / iters)
    mo, mt = sum(res["ours"]) / rounds, sum(res["torch"]) / rounds
    return {"torch_pipeline": kind + " after an fp32 rank sum; bf16 cast into the flat buffer",
            "ms_ours": mo, "ms_torch": mt, "speedup": mt / mo,
            "ms_ours_range": [min(res["ours"]), max(res["ours"])],
            "ms_torch_range": [min(res["torch"]), max(res["torch"])]}


def run_tiny(args, torch, zs, np):
    """Config 0: Psi = 2^20, N = 4, all four ranks' fused steps into one
    shared flat buffer (cache-resident, launch-bound: not a roofline point)."""
    from synthetic import WORKLOADS, grad_bits, master_init
    dev = torch.device("cuda:0")
    w = WORKLOADS[0]
    N = w.n_ranks
    lays = [zs.shard_init("zero2", N, r, list(w.units)).chunk_state(state_chunk(args, zs))
            for r in range(N)]
    S, P = lays[0].shard_len, lays[0].flat_len
    grads = [grad_bits(w, 0, q, P, device=dev) for q in range(N)]
    G = zs.Grads(grads, zs.BF16, zs.INDEX_FULL)
    full = torch.empty(P, dtype=torch.int16, device=dev)
    st = [State(torch, lays[r], master_init(w, S, device=dev, rank=r)).views for r in range(N)]
    t = [0]

    def step(ph):
        t[0] += 1
        cfg = zs.adam_cfg(step=t[0])
        for r in range(N):
            phase(ph, "fused_reduce_adam_cast",
                  lambda r=r: zs.adam_step(lays[r], 0, 1, cfg, *st[r], full, zs.INDEX_FULL,
                                           grads=G), chain=r > 0)

    ms, kern = timed(args, torch, step)
    b = (2 * N + 26) * S
    add_rates(kern, "fused_reduce_adam_cast", b)
    out = base_line(args, "tiny ZeRO-2 step params/sec (Psi=2^20, N=4, all ranks)",
                    P / (ms * 1e-3), "params/s", ms,
                    "tiny ZeRO-2 step: 4 ranks x fused reduce + Adam + bf16 into one buffer",
                    psi=w.psi, n_ranks=N, shard_elems=S,
                    state_layout=state_desc(lays[0].state_chunk))
    out["kernels"] = kern
    out["roofline"] = roofline("step_kernel<fused, N=4, bf16> (cache-resident; not a roofline "
                               "point)", b, kern["fused_reduce_adam_cast"]["ms_per_launch_mean"])
    out["cpu_baseline"] = None
    # The same four launches captured once in a HIP graph and replayed: this
    # workload is launch-bound, and a graph removes the per-launch host cost.
    # A graph keeps the step number of its capture, which does not change
    # the work timed.
    cfg = zs.adam_cfg(step=t[0] + 1)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for r in range(N):
            zs.adam_step(lays[r], 0, 1, cfg, *st[r], full, zs.INDEX_FULL, grads=G)
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    g_ms = 1e3 * (time.perf_counter() - t0) / args.steps
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(None)
    torch.cuda.synchronize()
    out["graph_replay"] = {"ms_per_step": g_ms,
                           "eager_ms_per_step": 1e3 * (time.perf_counter() - t0) / args.steps,
                           "what": "one step's four fused launches captured in a HIP graph, "
                                   "against the same launches issued eagerly (no timing events)"}
    return out


def run_gpt2_clip(args, torch, zs, np):
    """Config 1: Psi = 124,439,808, N = 8, five 25M buckets, all 8 ranks:
    reduce (with sum-of-squares partials) -> clip coefficient -> AdamW from
    the fp32 gradient."""
    from synthetic import WORKLOADS, grad_bits, master_init
    dev = torch.device("cuda:0")
    w = WORKLOADS[1]
    N, U = w.n_ranks, len(w.units)
    lays = [zs.shard_init("zero2", N, r, list(w.units)).chunk_state(state_chunk(args, zs))
            for r in range(N)]
    S, P = lays[0].shard_len, lays[0].flat_len
    GE = grad_chunk(args, zs)
    grads = [grad_bits(w, 0, q, P, device=dev) for q in range(N)]
    if GE:
        # each rank reads its slices of the N gradients from its own
        # receive buffer (rows of GE elements per rank): what a bucketed
        # reduce-scatter leaves on it
        recv = []
        for L in lays:
            own = torch.cat([torch.arange(L.query(u)["rank_flat_off"],
                                          L.query(u)["rank_flat_off"] + L.query(u)["shard_len"],
                                          device=dev) for u in range(U)])
            recv.append(RankGrads(torch, zs, [g[own] for g in grads], GE))
            assert recv[-1].buf.numel() == L.grad_len(GE)
        Gr = [x.grads for x in recv]
    else:
        Gr = [zs.Grads(grads, zs.BF16, zs.INDEX_FULL)] * N
    full = torch.empty(P, dtype=torch.int16, device=dev)
    st = [State(torch, L, master_init(w, L.shard_len, device=dev, rank=r)).views
          for r, L in enumerate(lays)]
    gsh = [torch.empty(L.shard_len, device=dev) for L in lays]
    counts = [zs.reduce_partials_count(L, 0, U) for L in lays]
    offs = [sum(counts[:r]) for r in range(N)]
    partials = torch.empty(sum(counts), dtype=torch.float64, device=dev)
    coef = torch.empty(1, device=dev)
    t = [0]

    def step(ph):
        t[0] += 1
        cfg = zs.adam_cfg(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                          weight_decay=w.weight_decay, decoupled=w.decoupled, step=t[0])
        # the 17 launches go back to back: each one's events start at the
        # previous one's end
        for r in range(N):
            phase(ph, "reduce_with_sumsq",
                  lambda r=r: zs.reduce_shard(lays[r], 0, U, Gr[r], gsh[r], partials[offs[r]:],
                                              counts[r]), chain=r > 0)
        phase(ph, "clip_coef", lambda: zs.clip_coef(partials, partials.numel(),
                                                    w.max_grad_norm, coef), chain=True)
        for r in range(N):
            phase(ph, "adamw_apply_cast",
                  lambda r=r: zs.adam_step(lays[r], 0, U, cfg, *st[r], full, zs.INDEX_FULL,
                                           grad_fp32=gsh[r], clip_coef=coef), chain=True)

    ms, kern = timed(args, torch, step)
    rb, ab = (2 * N + 4) * S, 30 * S
    add_rates(kern, "reduce_with_sumsq", rb)
    add_rates(kern, "adamw_apply_cast", ab)
    kern["clip_coef"]["bytes_per_launch"] = 8 * partials.numel() + 4
    dom = max(("reduce_with_sumsq", rb), ("adamw_apply_cast", ab),
              key=lambda x: kern[x[0]]["ms_per_step"])
    out = base_line(args, "GPT-2-small clipped AdamW step params/sec (N=8, all ranks)",
                    P / (ms * 1e-3), "params/s", ms,
                    "GPT-2-small flat buffer, 5 x 25M buckets, N=8: reduce + global-norm clip "
                    "+ AdamW + bf16 for all 8 ranks",
                    psi=w.psi, n_ranks=N, shard_elems=S, buckets=list(w.units),
                    state_layout=state_desc(lays[0].state_chunk),
                    grad_layout=("per rank: " + grad_desc(GE, N)) if GE else
                    f"{N} full-indexed bf16 gradient buffers, read by every rank")
    out["step_gbps"] = N * (rb + ab) / (ms * 1e-3) / 1e9
    out["kernels"] = kern
    out["roofline"] = roofline(dom[0], dom[1], kern[dom[0]]["ms_per_launch_mean"])
    out["cpu_baseline"] = None
    # The same 17 launches captured once in a HIP graph and replayed. The
    # Adam launches read their scalars from a device table at a device step
    # counter that the graph advances, so each replay is the next step.
    n_rep = args.warmup + args.steps
    table = zs.adam_table_device(
        [zs.adam_cfg(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                     weight_decay=w.weight_decay, decoupled=w.decoupled, step=t[0] + 1 + k)
         for k in range(n_rep)], dev)
    counter = torch.ones(1, dtype=torch.int64, device=dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for r in range(N):
            zs.reduce_shard(lays[r], 0, U, Gr[r], gsh[r], partials[offs[r]:], counts[r])
        zs.clip_coef(partials, partials.numel(), w.max_grad_norm, coef)
        for r in range(N):
            zs.adam_step_table(lays[r], 0, U, table, n_rep, counter, *st[r], full,
                               zs.INDEX_FULL, grad_fp32=gsh[r], clip_coef=coef)
        zs.step_advance(counter)
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    g_ms = 1e3 * (time.perf_counter() - t0) / args.steps
    assert int(counter.item()) == n_rep + 1, "the graph did not advance the step counter"
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(None)
    torch.cuda.synchronize()
    out["graph_replay"] = {"ms_per_step": g_ms, "params_per_s": P / (g_ms * 1e-3),
                           "eager_ms_per_step": 1e3 * (time.perf_counter() - t0) / args.steps,
                           "what": "one step's 17 launches captured in a HIP graph with "
                                   "table-driven Adam scalars, each replay the next step; "
                                   "against the same launches issued eagerly (no timing events)"}
    return out


def run_gpt2_ddp_buckets(args, torch, zs, np):
    """Config 1 as DDP with bucket-as-ready reduction: one replica; the 5
    gradient buckets are reduced (all-reduce arithmetic over the 8 ranks)
    one launch each, last bucket first, then the global clip coefficient and
    one AdamW call over the whole replica."""
    from synthetic import WORKLOADS, grad_bits, master_init
    dev = torch.device("cuda:0")
    w = WORKLOADS[1]
    N, U = w.n_ranks, len(w.units)
    L = zs.shard_init("ddp", N, 0, list(w.units)).chunk_state(state_chunk(args, zs))
    P = L.flat_len
    grads = [grad_bits(w, 0, q, P, device=dev) for q in range(N)]
    fo = [L.query(u)["flat_off"] for u in range(U)]
    Gu = [zs.Grads([g[fo[u]:] for g in grads], zs.BF16, zs.INDEX_FULL) for u in range(U)]
    tiles = [zs.reduce_partials_count(L, u, u + 1) for u in range(U)]
    offs = [sum(tiles[:u]) for u in range(U)]
    partials = torch.empty(sum(tiles), dtype=torch.float64, device=dev)
    g = torch.empty(P, device=dev)
    coef = torch.empty(1, device=dev)
    p, m, v = State(torch, L, master_init(w, P, device=dev)).views
    out = torch.empty(P, dtype=torch.int16, device=dev)
    t = [0]

    def step(ph):
        t[0] += 1
        cfg = zs.adam_cfg(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                          weight_decay=w.weight_decay, decoupled=w.decoupled, step=t[0])
        for u in reversed(range(U)):
            phase(ph, f"reduce_bucket_{u}",
                  lambda u=u: zs.reduce_shard(L, u, u + 1, Gu[u], g[fo[u]:], partials[offs[u]:],
                                              tiles[u]), chain=u < U - 1)
        phase(ph, "clip_coef", lambda: zs.clip_coef(partials, partials.numel(),
                                                    w.max_grad_norm, coef), chain=True)
        phase(ph, "adamw_apply_cast",
              lambda: zs.adam_step(L, 0, U, cfg, p, m, v, out, zs.INDEX_FULL, grad_fp32=g,
                                   clip_coef=coef), chain=True)

    ms, kern = timed(args, torch, step)
    for u in range(U):
        add_rates(kern, f"reduce_bucket_{u}", (2 * N + 4) * w.units[u])
    add_rates(kern, "adamw_apply_cast", 30 * P)
    out_line = base_line(args, "GPT-2-small DDP bucket-as-ready step params/sec (one replica)",
                         P / (ms * 1e-3), "params/s", ms,
                         "GPT-2-small DDP replica, N=8: per-bucket reduce launches (last bucket "
                         "first) + global clip + one AdamW",
                         psi=w.psi, n_ranks=N, buckets=list(w.units),
                         state_layout=state_desc(L.state_chunk))
    out_line["kernels"] = kern
    out_line["roofline"] = roofline("adamw_apply_cast", 30 * P,
                                    kern["adamw_apply_cast"]["ms_per_launch_mean"])
    out_line["cpu_baseline"] = None
    return out_line


def run_megatron(args, torch, zs, np):
    """Config 3: Psi = 7.24e9, N = 8, rank 7: four bf16 micro-batch
    gradients accumulated into the fp32 main gradient over the whole buffer,
    then the fused fp32 reduce (7 peer fp32 shards + own main gradient) +
    Adam + bf16 into the replicated buffer, then the gather of 7 peers."""
    from synthetic import KIND_MICRO, WORKLOADS, grad_bits, master_init
    dev = torch.device("cuda:0")
    w = WORKLOADS[3]
    N, r = w.n_ranks, w.n_ranks - 1
    L = zs.shard_init("megatron_do", N, r, list(w.units)).chunk_state(state_chunk(args, zs))
    S, P = L.shard_len, L.flat_len
    main = torch.zeros(P, device=dev)
    micro = grad_bits(w, 0, r, P, device=dev, kind=KIND_MICRO)
    GE = grad_chunk(args, zs)
    if GE:
        # the 7 peers' fp32 shards in one receive buffer (rows of GE elements
        # per rank; the own rank's slot unused) beside the own full-indexed
        # main gradient
        rows = -(-S // GE)
        recv = torch.zeros(rows * N * GE, device=dev)
        assert recv.numel() == L.grad_len(GE)
        col = torch.zeros(rows * GE, device=dev)
        for q in range(N - 1):
            col[:S].normal_(0, 1e-3)
            recv.view(rows, N, GE)[:, q, :].copy_(col.view(rows, GE))
        del col
        G = zs.Grads.chunked(recv, N, GE, zs.FP32, full={r: main})
        grad_layout = (f"own fp32 main gradient full-indexed; the {N - 1} peers' fp32 shards in "
                       f"one buffer of rows of {GE} elements per rank, {N} rank slots per row")
    else:
        peers32 = [torch.empty(S, device=dev).normal_(0, 1e-3) for _ in range(N - 1)]
        G = zs.Grads(peers32 + [main], zs.FP32, [zs.INDEX_SHARD] * (N - 1) + [zs.INDEX_FULL])
        grad_layout = f"own fp32 main gradient full-indexed; {N - 1} fp32 peer shard buffers"
    master, m, v = State(torch, L, master_init(w, S, device=dev, rank=r)).views
    replica = torch.empty(P, dtype=torch.int16, device=dev)
    peers16 = [torch.full((S,), q + 1, dtype=torch.int16, device=dev) for q in range(N - 1)]
    torch.cuda.synchronize()
    t = [0]

    def step(ph):
        t[0] += 1
        cfg = zs.adam_cfg(step=t[0])
        main.zero_()
        for _ in range(w.micro_batches):
            phase(ph, "accumulate_fp32", lambda: zs.grad_accumulate(main, micro, P))
        phase(ph, "fused_fp32_reduce_adam_cast",
              lambda: zs.adam_step(L, 0, 1, cfg, master, m, v, replica, zs.INDEX_FULL, grads=G))
        phase(ph, "gather_7_peers", lambda: zs.gather_params(L, 0, 1, peers16 + [None], replica))

    ms, kern = timed(args, torch, step)
    acc_b, fb, gb = 10 * P, (4 * N + 26) * S, 4 * (N - 1) * S
    add_rates(kern, "accumulate_fp32", acc_b)
    add_rates(kern, "fused_fp32_reduce_adam_cast", fb)
    add_rates(kern, "gather_7_peers", gb)
    opt_ms = (kern["fused_fp32_reduce_adam_cast"]["ms_per_step"]
              + kern["gather_7_peers"]["ms_per_step"])
    out = base_line(args, "Megatron distributed-optimizer step shard params/sec (7B, N=8)",
                    S / (ms * 1e-3), "params/s", ms,
                    "Megatron DO, Psi=7.24e9, N=8, rank 7: 4 micro-batch fp32 accumulations "
                    "over the whole buffer + fp32 reduce + Adam + bf16 + gather of 7 peers "
                    "(the step also zeroes main_grad with torch, untimed per phase)",
                    psi=w.psi, n_ranks=N, rank=r, shard_elems=S, micro_batches=w.micro_batches,
                    state_layout=state_desc(L.state_chunk), grad_layout=grad_layout)
    out["optimizer_only_shard_params_per_s"] = S / (opt_ms * 1e-3)
    out["kernels"] = kern
    dom = max(("accumulate_fp32", acc_b), ("fused_fp32_reduce_adam_cast", fb),
              key=lambda x: kern[x[0]]["ms_per_launch_mean"])
    out["roofline"] = roofline(dom[0], dom[1], kern[dom[0]]["ms_per_launch_mean"])
    out["cpu_baseline"] = None
    return out


def run_fsdp70b(args, torch, zs, np):
    """Config 4: Llama-70B FSDP full shard, N = 64, rank 63: for each of the
    81 units, fused reduce of 64 rank gradients + Adam + bf16 into the
    unit's full buffer, then the gather of the unit's 63 peer shards.  The
    per-unit working buffers are allocated once at the largest unit."""
    from synthetic import WORKLOADS, grad_bits
    dev = torch.device("cuda:0")
    w = WORKLOADS[4]
    N, r = w.n_ranks, w.n_ranks - 1
    units = list(w.units)
    L = zs.shard_init("fsdp", N, r, units).chunk_state(state_chunk(args, zs))
    S, SE, GE = L.shard_len, L.state_chunk, grad_chunk(args, zs)
    q = [L.query(u) for u in range(len(units))]
    smax = max(x["shard_len"] for x in q)
    # one set of unit receive buffers, sized for the largest unit and
    # reused by every unit (each reads the first s_u elements per rank)
    rg = RankGrads(torch, zs, [grad_bits(w, 0, k, smax, device=dev) for k in range(N)], GE)
    G = rg.grads
    st = State(torch, L, torch.empty(S, device=dev).normal_(0, 0.02))
    master, m, v = st.views
    full_unit = torch.empty(N * smax, dtype=torch.int16, device=dev)
    peers = [torch.full((smax,), k + 1, dtype=torch.int16, device=dev) for k in range(N - 1)]
    torch.cuda.synchronize()
    t = [0]

    def step(ph):
        t[0] += 1
        cfg = zs.adam_cfg(step=t[0])
        for u, x in enumerate(q):
            # three arrays are passed from the unit's first element, a
            # chunked state from its start
            so = 0 if SE else x["shard_off"]
            phase(ph, "fused_reduce64_adam_cast",
                  lambda u=u, so=so: zs.adam_step(L, u, u + 1, cfg, master[so:], m[so:], v[so:],
                                                  full_unit, zs.INDEX_FULL, grads=G), chain=u > 0)
            phase(ph, "gather_63_peers",
                  lambda u=u: zs.gather_params(L, u, u + 1, peers + [None], full_unit),
                  chain=True)

    ms, kern = timed(args, torch, step)
    fb, gb = (2 * N + 26) * S, 4 * (N - 1) * S
    for name, b in (("fused_reduce64_adam_cast", fb), ("gather_63_peers", gb)):
        k = kern[name]
        k["bytes_per_step"] = b
        k["gbps"] = b / (k["ms_per_step"] * 1e-3) / 1e9

    # the same sweep through zero_fsdp_sweep: one stream, then two streams
    # with the step of unit u+1 overlapping the gather of unit u (cap 2,
    # two unit buffers reused in turn)
    ring = [full_unit, torch.empty(N * smax, dtype=torch.int16, device=dev)]
    peer_list = peers + [None]
    gstream = torch.cuda.Stream()
    sweeps = {}
    variants = [("sweep_one_stream", 1, None, [full_unit])]
    if not args.one_stream:
        variants.append(("sweep_two_streams_cap2", 2, gstream, ring))
    for label, cap, gs, bufs in variants:
        ios = [(rg.ptrs, peer_list, bufs[u % len(bufs)]) for u in range(len(units))]

        def sweep_step(ph, cap=cap, gs=gs, ios=ios):
            t[0] += 1
            cfg = zs.adam_cfg(step=t[0])
            phase(ph, "sweep", lambda: zs.fsdp_sweep(L, 0, len(units), cfg, zs.BF16, ios, master,
                                                     m, v, cap, gather_stream=gs,
                                                     grad_chunk=GE))
        sms, _ = timed(args, torch, sweep_step)
        sweeps[label] = {"ms_per_step": sms, "shard_params_per_s": S / (sms * 1e-3),
                         "gbps": (fb + gb) / (sms * 1e-3) / 1e9}
    best = min(sweeps.values(), key=lambda x: x["ms_per_step"])["ms_per_step"]
    out = base_line(args, "Llama-70B FSDP per-unit sweep shard params/sec (N=64)",
                    S / (best * 1e-3), "params/s", best,
                    "Llama-70B FSDP full shard, N=64, rank 63: 81 units x (fused reduce of 64 "
                    "rank grads + Adam + bf16 into the unit buffer, gather of 63 peers); value "
                    "is the faster zero_fsdp_sweep variant",
                    psi=w.psi, n_ranks=N, rank=r, shard_elems=S, units=len(units),
                    state_layout=state_desc(SE), grad_layout="per unit: " + grad_desc(GE, N))
    out["per_unit_calls_ms_per_step"] = ms
    out["sweeps"] = sweeps
    out["kernels"] = kern
    fk = kern["fused_reduce64_adam_cast"]
    out["roofline"] = roofline("step_kernel<fused, N=64, bf16> (81 launches, summed)", fb,
                               fk["ms_per_step"])
    out["cpu_baseline"] = None
    if args.cpu_baseline_seconds > 0:
        # one layer unit x 64 ranks on the CPU, extrapolated to the 81 units
        s0 = q[0]["shard_len"]
        out["cpu_baseline"] = cpu_baseline(w, rg.ranks(), st.master, s0, r,
                                           args.cpu_baseline_seconds,
                                           what="rank-{r} shard of layer unit 0", total=S)
    return out


MFMA_BF16_PEAK_TFLOPS = 2500.0


def run_fsdp_linear(args, torch, zs, np):
    """One rank's FSDP linear-layer training step, N = 8 simulated ranks:
    forward (all-gather W, Y = X W), backward for this rank (re-gather,
    dX = dY W^T, dW = X^T dY) and the other 7 ranks' local dW (simulated),
    the reduce-scatter of the 8 dW into this rank's rows, and Adam on the W
    shard.  The GEMMs read X, W and dY in place."""
    from synthetic import small_workload, grad_bits
    dev = torch.device("cuda:0")
    N, r, inf, outf, batch = 8, 7, 4096, 14336, 4096
    L = zs.shard_init_rows("fsdp2", N, r, [(inf, outf)])
    S, Lu = L.shard_len, L.query(0)["padded_len"]
    w = small_workload([inf * outf], N, "fsdp2", cfg=5)
    shards = [grad_bits(w, 0, q, S, device=dev) for q in range(N)]
    xs = [torch.randn(batch, inf, device=dev).to(torch.bfloat16).view(torch.int16) for _ in range(N)]
    dys = [(torch.randn(batch, outf, device=dev) * 1e-2).to(torch.bfloat16).view(torch.int16)
           for _ in range(N)]
    w_full = torch.empty(Lu, dtype=torch.int16, device=dev)
    y = torch.empty((batch, outf), dtype=torch.int16, device=dev)
    dx = torch.empty((batch, inf), dtype=torch.int16, device=dev)
    dws = [torch.empty(Lu, device=dev) for _ in range(N)]
    gshard = torch.empty(S, device=dev)
    master = torch.randn(S, device=dev) * 0.02
    m = torch.zeros(S, device=dev)
    v = torch.zeros(S, device=dev)
    own = torch.empty(S, dtype=torch.int16, device=dev)
    G = zs.Grads(dws, zs.FP32, zs.INDEX_FULL)
    KI, KO = zs.K_INNER, zs.K_OUTER
    t = [0]

    def step(ph):
        t[0] += 1
        phase(ph, "gather_w", lambda: zs.gather_params(L, 0, 1, shards, w_full))
        # Y = X W (W read in place as a K-outer operand)
        phase(ph, "gemm_forward", lambda: zs.gemm_bf16(batch, outf, inf, xs[r], inf, KI, w_full,
                                                       outf, KO, y, outf, zs.BF16))
        phase(ph, "gather_w", lambda: zs.gather_params(L, 0, 1, shards, w_full))
        # dX = dY W^T
        phase(ph, "gemm_dx", lambda: zs.gemm_bf16(batch, inf, outf, dys[r], outf, KI, w_full, outf,
                                                  KI, dx, inf, zs.BF16))
        # every rank's dW = X^T dY (fp32), both operands K-outer
        for q in range(N):
            phase(ph, "gemm_dw", lambda q=q: zs.gemm_bf16(inf, outf, batch, xs[q], inf, KO, dys[q],
                                                          outf, KO, dws[q], outf, zs.FP32))
        phase(ph, "reduce_scatter_dw", lambda: zs.reduce_shard(L, 0, 1, G, gshard))
        phase(ph, "adam_shard", lambda: zs.adam_step(L, 0, 1, zs.adam_cfg(step=t[0]), master, m, v,
                                                     own, zs.INDEX_SHARD, grad_fp32=gshard))

    ms, kern = timed(args, torch, step)
    flops = 2.0 * batch * inf * outf
    for name, count in (("gemm_forward", 1), ("gemm_dx", 1), ("gemm_dw", N)):
        k = kern[name]
        k["flops_per_launch"] = flops
        k["tflops"] = flops * count / (k["ms_per_step"] * 1e-3) / 1e12
    kern["reduce_scatter_dw"]["gbps"] = (4 * N + 4) * S / (
        kern["reduce_scatter_dw"]["ms_per_step"] * 1e-3) / 1e9
    out = base_line(args, "FSDP linear-layer training step tokens/sec per rank "
                          "(Mistral-7B MLP up projection, N=8)",
                    batch / (ms * 1e-3), "tokens/s", ms,
                    "hand-written FSDP linear layer, W 4096 x 14336 row-sharded over 8 ranks, "
                    "4096 tokens per rank: gather + Y = X W, gather + dX, the 8 ranks' dW, "
                    "reduce-scatter of dW, Adam on the shard",
                    in_features=inf, out_features=outf, tokens_per_rank=batch, n_ranks=N, rank=r)
    out["dtype"] = "bf16 (fp32 accumulate)"
    out["kernels"] = kern
    gemm_ms = sum(kern[k]["ms_per_step"] for k in ("gemm_forward", "gemm_dx", "gemm_dw"))
    out["gemm_tflops"] = flops * (N + 2) / (gemm_ms * 1e-3) / 1e12
    out["roofline"] = {"bound": "mfma", "kernel": "gemm_kernel (bf16, fp32 accumulate), "
                                                   "all 10 launches of the step",
                       "achieved": out["gemm_tflops"], "peak": MFMA_BF16_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": out["gemm_tflops"] / MFMA_BF16_PEAK_TFLOPS,
                       "traffic": counter_traffic(GEMM_COUNTERS, GEMM_SRC, "gemm_hip_sha256",
                                                  "gemm_traffic_bytes_per_step"),
                       "traffic_unit": "HBM bytes of the 10 GEMM launches of one step "
                                       "(rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"}
    out["cpu_baseline"] = None
    if args.vs_library:
        out["library_comparison"] = gemm_vs_library(torch, zs, xs[r], w_full, dys[r], y, dx,
                                                    dws[r], batch, inf, outf)
    return out


def gemm_vs_library(torch, zs, x, w, dy, y, dx, dw, batch, inf, outf, rounds=5, iters=10):
    """The three GEMMs of the linear layer, timed alternately with
    zero_gemm_bf16 and with torch.mm (hipBLASLt) on the same operands and
    streams; TFLOP/s as mean (min-max) over the rounds."""
    KI, KO = zs.K_INNER, zs.K_OUTER
    xb, wb = x.view(torch.bfloat16).view(batch, inf), w.view(torch.bfloat16).view(inf, outf)
    dyb = dy.view(torch.bfloat16).view(batch, outf)
    yb, dxb = y.view(torch.bfloat16), dx.view(torch.bfloat16)
    cases = {
        "gemm_forward": (lambda: zs.gemm_bf16(batch, outf, inf, x, inf, KI, w, outf, KO, y, outf,
                                              zs.BF16),
                         lambda: torch.mm(xb, wb, out=yb)),
        "gemm_dx": (lambda: zs.gemm_bf16(batch, inf, outf, dy, outf, KI, w, outf, KI, dx, inf,
                                         zs.BF16),
                    lambda: torch.mm(dyb, wb.t(), out=dxb)),
        "gemm_dw": (lambda: zs.gemm_bf16(inf, outf, batch, x, inf, KO, dy, outf, KO, dw, outf,
                                         zs.FP32),
                    lambda: torch.mm(xb.t(), dyb, out_dtype=torch.float32)),
    }
    flops = 2.0 * batch * inf * outf
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for name, fns in cases.items():
        tf = [[], []]
        for f in fns:
            f()
        torch.cuda.synchronize()
        for _ in range(rounds):
            for i, f in enumerate(fns):
                e0.record()
                for _ in range(iters):
                    f()
                e1.record()
                torch.cuda.synchronize()
                tf[i].append(flops / (e0.elapsed_time(e1) / iters * 1e-3) / 1e12)
        ours, lib = (sum(v) / len(v) for v in tf)
        res[name] = {"ours_tflops": ours, "ours_range": [min(tf[0]), max(tf[0])],
                     "torch_mm_tflops": lib, "torch_mm_range": [min(tf[1]), max(tf[1])],
                     "ours_over_torch_mm": ours / lib}
    return res


def calibrate_copy(args, torch, zs, np):
    dev = torch.device("cuda:0")
    n = args.calibrate_copy // 2
    L = zs.shard_init("zero2", 1, 0, [n])
    src = torch.ones(n, dtype=torch.int16, device=dev)
    dst = torch.empty(n, dtype=torch.int16, device=dev)
    for _ in range(3):
        zs.gather_params(L, 0, 1, [src], dst)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        zs.gather_params(L, 0, 1, [src], dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    return {"calibrate_copy_bytes": 2 * n, "ms": ms, "GBps": 4 * n / ms / 1e6}


def calibrate_mix(args, torch, zs, np, rounds=5):
    """The fused 7B / N = 8 step against the ceiling of its own access
    pattern, on `args.calibrate_mix` fresh placements of the headline's
    buffers: zero_adam_step (fused), then zero_stream_mix with the same
    streams and launch shape and no optimizer arithmetic, its reads alone and
    its writes alone, timed alternately (HIP events, one launch each, median
    of `rounds` per placement)."""
    from synthetic import WORKLOADS
    dev = torch.device("cuda:0")
    w = WORKLOADS[2]
    N, r = w.n_ranks, w.n_ranks - 1
    L = zs.shard_init("zero3", N, r, list(w.units)).chunk_state(state_chunk(args, zs))
    S, SE, GE = L.shard_len, L.state_chunk, grad_chunk(args, zs)
    kinds = {"fused_step": 42 * S, "step_streams_no_math": 42 * S, "reads_only": 28 * S,
             "writes_only": 14 * S}
    E = torch.cuda.Event
    per = {k: [] for k in kinds}
    for pl in range(args.calibrate_mix):
        rg, st, full, _ = headline_buffers(torch, zs, w, L, S, N, r, dev, rank_peers=False,
                                           grad_chunk=GE)
        master, m, v = st.views
        own = full[r * S:(r + 1) * S]
        G, grads = rg.grads, rg.ptrs
        t = [0]

        def fused():
            t[0] += 1
            cfg = zs.adam_cfg(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, step=t[0])
            zs.adam_step(L, 0, 1, cfg, master, m, v, full, zs.INDEX_FULL, grads=G)

        fns = {"fused_step": fused,
               "step_streams_no_math": lambda: zs.stream_mix(zs.MIX_STEP_STREAMS, grads, master,
                                                             m, v, own, S, state_chunk=SE,
                                                             grad_chunk=GE),
               "reads_only": lambda: zs.stream_mix(zs.MIX_READS, grads, master, m, v, own, S,
                                                   state_chunk=SE, grad_chunk=GE),
               "writes_only": lambda: zs.stream_mix(zs.MIX_WRITES, grads, master, m, v, own, S,
                                                    state_chunk=SE, grad_chunk=GE)}
        got = {k: [] for k in kinds}
        names = list(kinds)
        for rd in range(rounds + 1):
            for i in range(len(names)):
                k = names[(i + rd) % len(names)]
                a, b = E(enable_timing=True), E(enable_timing=True)
                a.record()
                fns[k]()
                b.record()
                b.synchronize()
                if rd:
                    got[k].append(a.elapsed_time(b))
        for k in kinds:
            per[k].append(sorted(got[k])[len(got[k]) // 2])
        print("# placement %d: %s" % (pl, ", ".join(f"{k} {per[k][-1]:.3f} ms" for k in kinds)),
              file=sys.stderr, flush=True)
        del G, own, grads
        release(torch)
        del rg, st, master, m, v, full
        torch.cuda.empty_cache()
    med = {k: sorted(x)[len(x) // 2] for k, x in per.items()}
    return {"calibrate_mix": {
        "workload": "Mistral-7B ZeRO-3 rank shard, N=8, 905,000,000 elements",
        "state_layout": state_desc(SE), "grad_layout": grad_desc(GE, N),
        "placements": args.calibrate_mix, "rounds_per_placement": rounds,
        "ms_per_placement": per,
        "ms_median": med,
        "GBps_median": {k: kinds[k] / (med[k] * 1e-3) / 1e9 for k in kinds},
        "bytes_per_launch": kinds,
        "fused_over_no_math_per_placement": [a / b for a, b in
                                             zip(per["fused_step"], per["step_streams_no_math"])],
        "reads_plus_writes_ms_per_placement": [a + b for a, b in
                                               zip(per["reads_only"], per["writes_only"])]}}


def counter_traffic(path=COUNTERS, src=KERNELS_SRC, sha_key="kernels_hip_sha256",
                    key="fused_traffic_bytes_per_launch"):
    """HBM bytes from a committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary
    (already scaled by the copy calibration), or None if that summary was
    taken on a different version of the kernel source."""
    import hashlib
    try:
        kv = dict(line.split(": ", 1) for line in open(path).read().splitlines()
                  if line.startswith((sha_key + ": ", key + ": ")))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if kv.get(sha_key) != sha:
            return None
        return float(kv[key])
    except (OSError, KeyError, ValueError):
        return None


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, grads, master_of, S, r, budget_s, what="rank-{r} shard", total=None):
    """The oracle, as it stands, on the first elements of the same shard:
    16M-element chunks are copied from the GPU and stepped (step 1) until the
    single-threaded oracle has run for `budget_s` seconds or the S elements
    are done; only oracle time is counted.  Each chunk is also stepped by
    the same oracle function on all host cores, each thread taking a
    contiguous slice (ctypes releases the GIL), and both results must be
    bit-identical.  With `total`, the sample is one part of a `total`-element
    shard and the time for all of it is extrapolated."""
    import concurrent.futures as cf

    import numpy as np

    from oracle import _c

    cores = len(os.sched_getaffinity(0))
    pool = cf.ThreadPoolExecutor(cores)
    chunk = 1 << 24
    hp = _c.hparams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, 1, w.decoupled)
    done, spent, spent_all, same = 0, 0.0, 0.0, True
    while spent < budget_s and done < S:
        n = min(chunk, S - done)
        g = [x[done:done + n].cpu().numpy().view(np.uint16) for x in grads]
        p0 = master_of(done, n).cpu().numpy()
        p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
        out, tmp = np.empty(n, np.uint16), np.empty(n, np.float32)
        t0 = time.perf_counter()
        _c.rank_step(hp, g, 1.0, p, m, v, out, tmp)
        spent += time.perf_counter() - t0
        pa, ma, va = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
        outa, tmpa = np.empty(n, np.uint16), np.empty(n, np.float32)
        cuts = [n * k // cores for k in range(cores + 1)]

        def part(k):
            lo, hi = cuts[k], cuts[k + 1]
            if hi > lo:
                _c.rank_step(hp, [x[lo:hi] for x in g], 1.0, pa[lo:hi], ma[lo:hi], va[lo:hi],
                             outa[lo:hi], tmpa[lo:hi])

        t0 = time.perf_counter()
        list(pool.map(part, range(cores)))
        spent_all += time.perf_counter() - t0
        same = same and np.array_equal(out, outa) and np.array_equal(p.view(np.uint32),
                                                                     pa.view(np.uint32))
        done += n
    pool.shutdown()
    assert same, "the oracle on all cores must match the single-threaded oracle"
    sample = (f"first {done} of {S} elements of the {what.format(r=r)}, step 1, "
              f"{chunk}-element chunks, {spent:.1f} s of oracle time "
              f"(reduce {len(grads)} bf16 ranks + Adam + bf16 cast)")
    if total:
        sample += (f"; the whole {total}-element shard would take {spent * total / done:.1f} s "
                   f"(extrapolated)")
    return {"value": done / spent, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": sample, "cpu_model": host_cpu_model(),
            "all_cores": {"value": done / spent_all, "unit": "params/s", "cores": cores,
                          "how": "the same oracle function on contiguous slices, one host "
                                 "thread per core; bit-identical to the single-threaded run"}}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build simulates the N data-parallel ranks "
              "inside one GPU's memory and has no multi-GPU path; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.one_stream and (args.config != 4 or args.fsdp_linear):
        print("--one-stream applies to --config 4 only.", file=sys.stderr)
        sys.exit(2)
    if args.vs_library and not args.fsdp_linear:
        print("--vs-library applies to --fsdp-linear only.", file=sys.stderr)
        sys.exit(2)
    if args.vs_torch and (args.fsdp_linear or args.fsdp2 or args.config != 2 or
                          args.calibrate_copy or args.calibrate_mix):
        print("--vs-torch applies to the headline workload (--config 2) only.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from fsdp_sharded_optimizer_shard_amd import zs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.placements < 1:
        print("--placements must be >= 1.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_mix:
        out = calibrate_mix(args, torch, zs, np)
    elif args.calibrate_copy:
        out = calibrate_copy(args, torch, zs, np)
    elif args.fsdp_linear:
        out = run_fsdp_linear(args, torch, zs, np)
    else:
        run = {0: run_tiny, 1: run_gpt2_ddp_buckets if args.ddp_buckets else run_gpt2_clip,
               2: run_headline, 3: run_megatron, 4: run_fsdp70b}[args.config]
        out = run(args, torch, zs, np)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
