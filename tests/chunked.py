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


def grad_buffer(S, n, E, draw, tidx=None, hole=()):
    """One receive buffer of S elements per rank for n ranks in chunks of E
    (ceil(S / E) rows of n chunks, as Layout.grad_len counts) filled with
    draw(q), a device tensor of S elements (int16 bf16 bits or fp32), for
    each rank q not in `hole`; the chunks of the ranks in `hole` (a rank's
    own full-indexed gradient, kept elsewhere) hold NaN.  With tidx (a
    device index tensor), also each drawn rank's values at those positions
    as host arrays (uint16 for bf16), None for a hole."""
    rows = -(-S // E)
    buf = col = None
    samples = []
    for q in range(n):
        if q in hole:
            samples.append(None)
            continue
        x = draw(q)
        if buf is None:
            buf = torch.zeros(rows * n * E, dtype=x.dtype, device=x.device)
            col = torch.zeros(rows * E, dtype=x.dtype, device=x.device)
        col[:S] = x
        del x
        if tidx is not None:
            h = col[tidx].cpu().numpy()
            samples.append(h.view(np.uint16) if h.dtype == np.int16 else h)
        buf.view(rows, n, E)[:, q, :].copy_(col.view(rows, E))
    for q in hole:
        if buf.dtype == torch.int16:
            buf.view(rows, n, E)[:, q, :] = 0x7FC0
        else:
            buf.view(rows, n, E)[:, q, :] = float("nan")
    return buf, samples
