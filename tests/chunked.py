"""Device buffers in the library's chunked formats for the full-size GPU
tests: the optimizer state (rows of E master, E m, E v values) and the N
rank gradients (rows of E elements of each rank in rank order).  Index
arithmetic and copies only; no optimizer arithmetic."""
import numpy as np
import torch


def state_pos(E, i):
    """Offset of shard element i's master in a chunked state (m: + E, v: + 2E)."""
    return (i // E) * (3 * E) + i % E


def state_buffer(L, master):
    """A chunked state buffer of layout L holding `master` (device fp32,
    shard length) and zero m and v."""
    E, S = L.state_chunk, L.shard_len
    rows = -(-S // E)
    buf = torch.zeros(L.state_len, device=master.device)
    col = torch.zeros(rows * E, device=master.device)
    col[:S] = master
    buf.view(rows, 3, E)[:, 0, :].copy_(col.view(rows, E))
    return buf


def grad_buffer(S, n, E, draw, tidx=None):
    """One receive buffer of S elements per rank for n ranks in chunks of E
    (ceil(S / E) rows of n chunks, as Layout.grad_len counts) filled with
    draw(q), a device int16 tensor of S elements, for each rank q; and,
    with tidx (a device index tensor), each rank's values at those
    positions as host uint16 arrays."""
    rows = -(-S // E)
    first = draw(0)
    buf = torch.zeros(rows * n * E, dtype=torch.int16, device=first.device)
    col = torch.zeros(rows * E, dtype=torch.int16, device=first.device)
    samples = []
    for q in range(n):
        col[:S] = first if q == 0 else draw(q)
        if tidx is not None:
            samples.append(col[tidx].cpu().numpy().view(np.uint16))
        buf.view(rows, n, E)[:, q, :].copy_(col.view(rows, E))
    return buf, samples
