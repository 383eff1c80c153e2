"""Benchmark: one data-parallel rank's sharded optimizer step on one MI355X.

Workload (default): the Mistral-7B-sized ZeRO-3 rank shard -- Psi =
7.24e9, N = 8 simulated ranks, this GPU is rank 7 and owns 905,000,000
elements.  Inputs are synthetic and resident in HBM before timing: 8 bf16
rank-gradient shards ~N(0, 1e-3), fp32 master ~N(0, 0.02), m = v = 0,
7 peer bf16 parameter shards.  One step is the whole hot path:
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
BYTES_FUSED = 42          # per shard element, bf16 grads, N = 8
BYTES_GATHER_PER_PEER = 4  # read 2 + write 2 per element per peer slice


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-baseline-seconds", type=float, default=12.0,
                    help="oracle time budget for the CPU baseline; 0 skips it")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="instead of the step, run a plain bf16 copy of BYTES through "
                         "zero_gather_params (counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build simulates the N data-parallel ranks "
              "inside one GPU's memory and has no multi-GPU path; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from fsdp_sharded_optimizer_shard_amd import zs
    from synthetic import WORKLOADS, grad_bits, master_init

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    if args.calibrate_copy:
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
        print(json.dumps({"calibrate_copy_bytes": 2 * n, "ms": ms, "GBps": 4 * n / ms / 1e6}),
              flush=True)
        return

    w = WORKLOADS[2]
    N, r = w.n_ranks, w.n_ranks - 1
    L = zs.shard_init("zero3", N, r, list(w.units))
    S = L.shard_len
    q0 = L.query(0)
    print(f"# setup: {w.name}, rank {r}, shard {S} elements", file=sys.stderr, flush=True)

    grads = [grad_bits(w, 0, q, S, device=dev) for q in range(N)]
    master = master_init(w, S, device=dev, rank=r)
    m = torch.zeros(S, device=dev)
    v = torch.zeros(S, device=dev)
    full = torch.empty(L.flat_len, dtype=torch.int16, device=dev)
    peers = [torch.full((S,), q + 1, dtype=torch.int16, device=dev) for q in range(N - 1)]
    shard_ptrs = peers + [None]                      # own slice is written by the step
    G = zs.Grads(grads, zs.BF16, zs.INDEX_SHARD)
    torch.cuda.synchronize()

    t_state = [0]

    def step(ev=None):
        t_state[0] += 1
        cfg = zs.adam_cfg(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, step=t_state[0])
        if ev:
            ev[0].record(stream)
        zs.adam_step(L, 0, 1, cfg, master, m, v, full, zs.INDEX_FULL, grads=G, stream=stream)
        if ev:
            ev[1].record(stream)
        zs.gather_params(L, 0, 1, shard_ptrs, full, stream=stream)
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    fused_ms = [e[0].elapsed_time(e[1]) for e in evs]
    gather_ms = [e[1].elapsed_time(e[2]) for e in evs]
    step_ms = [e[0].elapsed_time(e[2]) for e in evs]
    ms_per_step = 1e3 * wall / args.steps
    fused_avg = float(np.mean(fused_ms))
    gather_avg = float(np.mean(gather_ms))
    fused_gbps = BYTES_FUSED * S / (fused_avg * 1e-3) / 1e9
    gather_gbps = BYTES_GATHER_PER_PEER * (N - 1) * S / (gather_avg * 1e-3) / 1e9
    step_bytes = (BYTES_FUSED + BYTES_GATHER_PER_PEER * (N - 1)) * S

    cpu = None
    if args.cpu_baseline_seconds > 0:
        cpu = cpu_baseline(w, grads, master, S, r, args.cpu_baseline_seconds)

    out = {
        "metric": "shard optimizer-step params/sec at 7B N=8; achieved HBM GB/s vs peak",
        "value": S / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1e-3) bf16 rank grads, N(0,0.02) fp32 master)",
        "config": {
            "workload": "Mistral-7B ZeRO-3 rank shard step: reduce 8 bf16 rank grads + Adam + "
                        "bf16 cast into the flat buffer + gather of 7 peer shards",
            "psi": w.psi, "n_ranks": N, "rank": r, "shard_elems": S,
            "rank_flat_offset": q0["rank_flat_off"],
            "algorithmic_bytes_per_step": step_bytes,
        },
        "step_gbps": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "state_gbps_16psi_over_n": 16 * S / (ms_per_step * 1e-3) / 1e9,
        "kernels": {
            "fused_reduce_adam_cast": {"ms_mean": fused_avg, "ms_min": float(np.min(fused_ms)),
                                       "ms_max": float(np.max(fused_ms)), "gbps": fused_gbps,
                                       "bytes_per_elem": BYTES_FUSED},
            "gather_7_peers": {"ms_mean": gather_avg, "ms_min": float(np.min(gather_ms)),
                               "gbps": gather_gbps,
                               "bytes_per_elem": BYTES_GATHER_PER_PEER * (N - 1)},
            "step_events_ms_mean": float(np.mean(step_ms)),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "fused_reduce_adam_cast (step_kernel<fused, N=8, bf16>)",
            "achieved": fused_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": fused_gbps / HBM_PEAK_GBPS,
            "traffic": counter_traffic(),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                            "copy-calibrated)",
            "algorithmic_bytes": BYTES_FUSED * S,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def counter_traffic():
    """HBM bytes per launch of the fused kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary (already scaled by the copy calibration),
    or None if that summary was taken on a different kernels.hip."""
    import hashlib
    try:
        kv = dict(line.split(": ", 1) for line in open(COUNTERS).read().splitlines()
                  if line.startswith(("kernels_hip_sha256: ", "fused_traffic_bytes_per_launch: ")))
        sha = hashlib.sha256(open(KERNELS_SRC, "rb").read()).hexdigest()
        if kv.get("kernels_hip_sha256") != sha:
            return None
        return float(kv["fused_traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(w, grads, master, S, r, budget_s):
    """The oracle, single-threaded, on the first elements of the same shard:
    16M-element chunks are copied from the GPU and stepped (step 1) until the
    oracle has run for `budget_s` seconds; only oracle time is counted."""
    import numpy as np
    import torch

    from oracle import _c

    chunk = 1 << 24
    hp = _c.hparams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, 1, w.decoupled)
    done, spent = 0, 0.0
    while spent < budget_s and done < S:
        n = min(chunk, S - done)
        g = [x[done:done + n].cpu().numpy().view(np.uint16) for x in grads]
        p = master[done:done + n].cpu().numpy().copy()
        m = np.zeros(n, np.float32)
        v = np.zeros(n, np.float32)
        out = np.empty(n, np.uint16)
        tmp = np.empty(n, np.float32)
        t0 = time.perf_counter()
        _c.rank_step(hp, g, 1.0, p, m, v, out, tmp)
        spent += time.perf_counter() - t0
        done += n
    return {"value": done / spent, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"first {done} of {S} elements of the rank-{r} shard, step 1, "
                      f"{chunk}-element chunks, {spent:.1f} s of oracle time "
                      f"(reduce 8 bf16 ranks + Adam + bf16 cast)"}


if __name__ == "__main__":
    main()
