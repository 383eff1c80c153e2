"""A ring reduce-scatter / all-gather / all-reduce over N simulated ranks that
moves chunks between neighbours one hop at a time and counts the bytes each
rank sends.

Used to pin the communication-cost statements of the pages by brute force:
  * ring all-reduce moves about 2 (N-1)/N x S bytes per GPU per step, S the
    gradient size ("Data Parallel, ZeRO and FSDP", section "Communication
    cost");
  * busbw = algbw x 2 (N-1)/N ("Data Parallel, ZeRO and FSDP", section "Bus
    bandwidth");
  * all-reduce = reduce-scatter + all-gather ("dp-zero-fsdp", concepts;
    "Behind the scenes...", section "ZeRO: The Dial Between DDP and FSDP").

The ring adds in a rotated rank order, so its sums equal the oracle's
ascending-order sums only where fp32 addition is exact; tests use such
inputs.
"""
from typing import List, Sequence, Tuple

import numpy as np


def _chunks(P: int, N: int) -> List[Tuple[int, int]]:
    if P % N:
        raise ValueError("ring simulation needs P divisible by N")
    c = P // N
    return [(i * c, (i + 1) * c) for i in range(N)]


def reduce_scatter(bufs: Sequence[np.ndarray]):
    """Returns (per-rank reduced chunk q, bytes sent per rank).  Rank q ends
    with the full sum of chunk q.  Inputs are fp32 arrays of equal length."""
    N = len(bufs)
    work = [np.array(b, dtype=np.float32, copy=True) for b in bufs]
    ch = _chunks(work[0].size, N)
    sent = [0] * N
    for k in range(N - 1):
        # all sends of one step happen "at once": snapshot what is sent
        msgs = []
        for q in range(N):
            c = (q - k - 1) % N
            lo, hi = ch[c]
            msgs.append((q, c, work[q][lo:hi].copy()))
            sent[q] += (hi - lo) * work[q].itemsize
        for q, c, data in msgs:
            dst = (q + 1) % N
            lo, hi = ch[c]
            work[dst][lo:hi] = data + work[dst][lo:hi]
    out = [work[q][ch[q][0]:ch[q][1]].copy() for q in range(N)]
    return out, sent


def all_gather(chunks: Sequence[np.ndarray]):
    """Rank q starts with chunk q; returns (per-rank full buffer, bytes sent
    per rank)."""
    N = len(chunks)
    c = chunks[0].size
    P = c * N
    have = [np.full(P, np.nan, dtype=chunks[0].dtype) for _ in range(N)]
    for q in range(N):
        have[q][q * c:(q + 1) * c] = chunks[q]
    sent = [0] * N
    for k in range(N - 1):
        msgs = []
        for q in range(N):
            ci = (q - k) % N
            msgs.append((q, ci, have[q][ci * c:(ci + 1) * c].copy()))
            sent[q] += c * chunks[0].itemsize
        for q, ci, data in msgs:
            have[(q + 1) % N][ci * c:(ci + 1) * c] = data
    return have, sent


def all_reduce(bufs: Sequence[np.ndarray]):
    """Ring all-reduce (sum) as reduce-scatter followed by all-gather."""
    red, sent1 = reduce_scatter(bufs)
    full, sent2 = all_gather(red)
    return full, [a + b for a, b in zip(sent1, sent2)]
