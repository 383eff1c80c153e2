"""Checks of gathered flat buffers against the peer shards that went in.

The gather is a bit copy, so the expected value of every gathered element
is the input element itself: peer shard q's element j must sit at
base + q * s + j.  Checked at the sampled positions and at both edges of
every slot (64 elements each side), for every peer slot."""
import numpy as np
import torch

EDGE = 64


def assert_gathered(full, base, s, peers, idx, what, skip=()):
    """full: the device buffer; base: offset of the unit's flat start;
    s: slice length; peers: list of device shards (None to skip), each
    addressed from that unit's first element; idx: host int64 sample of
    slice positions."""
    dev = full.device
    e = min(EDGE, s)
    pos = np.unique(np.concatenate([idx, np.arange(e), np.arange(s - e, s)])).astype(np.int64)
    tpos = torch.from_numpy(pos).to(dev)
    for q, p in enumerate(peers):
        if p is None or q in skip:
            continue
        got = full[base + q * s + tpos].cpu().numpy().view(np.uint16)
        want = p[tpos].cpu().numpy().view(np.uint16)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (f"{what}: slot {q}, {bad.size} of {pos.size} positions differ, "
                               f"first at slice position {pos[bad[0]]}")
