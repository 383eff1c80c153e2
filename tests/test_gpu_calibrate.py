"""zero_stream_mix on the GPU: the calibration kernels do exactly what the
header says on a small ragged tile count (several 2048-element tiles plus a
partial one), so a rate measured with them is a rate of those streams.

  MIX_STEP_STREAMS  master, m, v each gain the fp32 rank sum (ranks added in
                    order from +0); param holds the upper 16 bits of the new
                    master;
  MIX_READS         nothing changes;
  MIX_WRITES        master = m = v = the group index j (the first element of
                    the element's 4-element group), param = the low and high
                    halves of j, alternately.
With a state chunk E the same holds at the chunked positions (element i of
master at (i / E) 3E + i % E, m and v E and 2E further), and the rest of the
buffer is left alone.
"""
import numpy as np
import pytest
import torch

from fsdp_sharded_optimizer_shard_amd import zs

pytestmark = pytest.mark.gpu


def _setup(n, n_ranks, seed):
    rng = np.random.default_rng(seed)
    dev = torch.device("cuda:0")
    g = [rng.integers(0, 1 << 16, n, dtype=np.uint16) for _ in range(n_ranks)]
    # finite bf16 values only (exponent field below 0xff)
    for x in g:
        x &= 0xbfff
    st = [rng.standard_normal(n).astype(np.float32) for _ in range(3)]
    dg = [torch.from_numpy(x.view(np.int16)).to(dev) for x in g]
    ds = [torch.from_numpy(x.copy()).to(dev) for x in st]
    param = torch.zeros(n, dtype=torch.int16, device=dev)
    return g, st, dg, ds, param


@pytest.mark.parametrize("n_ranks", [8, 3])
def test_step_streams_add_the_rank_sum(n_ranks):
    n = 3 * 2048 + 4 * 37
    g, st, dg, ds, param = _setup(n, n_ranks, 11 + n_ranks)
    zs.stream_mix(zs.MIX_STEP_STREAMS, dg, *ds, param, n)
    torch.cuda.synchronize()
    acc = np.zeros(n, np.float32)
    for x in g:
        acc = acc + (x.astype(np.uint32) << 16).view(np.float32)
    for before, after in zip(st, ds):
        assert np.array_equal((before + acc).view(np.uint32), after.cpu().numpy().view(np.uint32))
    want = (ds[0].cpu().numpy().view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(param.cpu().numpy().view(np.uint16), want)


def test_reads_change_nothing_and_writes_fill_the_index():
    n = 2 * 2048 + 4 * 5
    g, st, dg, ds, param = _setup(n, 8, 5)
    zs.stream_mix(zs.MIX_READS, dg, *ds, param, n)
    torch.cuda.synchronize()
    for before, after in zip(st, ds):
        assert np.array_equal(before.view(np.uint32), after.cpu().numpy().view(np.uint32))
    assert not param.any()
    zs.stream_mix(zs.MIX_WRITES, dg, *ds, param, n)
    torch.cuda.synchronize()
    j = (np.arange(n) // 4 * 4).astype(np.int64)
    for after in ds:
        assert np.array_equal(after.cpu().numpy(), j.astype(np.float32))
    half = np.where(np.arange(n) % 2 == 0, j & 0xffff, (j >> 16) & 0xffff).astype(np.uint16)
    assert np.array_equal(param.cpu().numpy().view(np.uint16), half)


def test_step_streams_on_a_chunked_state():
    n, E, n_ranks = 3 * 2048 + 4 * 37, 1024, 8
    rng = np.random.default_rng(9)
    dev = torch.device("cuda:0")
    g = [rng.integers(0, 1 << 16, n, dtype=np.uint16) & 0xbfff for _ in range(n_ranks)]
    rows = -(-n // E)
    buf = rng.standard_normal(rows * 3 * E).astype(np.float32)
    dbuf = torch.from_numpy(buf.copy()).to(dev)
    dg = [torch.from_numpy(x.view(np.int16)).to(dev) for x in g]
    param = torch.zeros(n, dtype=torch.int16, device=dev)
    views = (dbuf[0:], dbuf[E:], dbuf[2 * E:])
    zs.stream_mix(zs.MIX_STEP_STREAMS, dg, *views, param, n, state_chunk=E)
    torch.cuda.synchronize()
    acc = np.zeros(n, np.float32)
    for x in g:
        acc = acc + (x.astype(np.uint32) << 16).view(np.float32)
    i = np.arange(n)
    pos = (i // E) * 3 * E + i % E
    want = buf.copy()
    for k in range(3):
        want[pos + k * E] = buf[pos + k * E] + acc
    got = dbuf.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert np.array_equal(param.cpu().numpy().view(np.uint16),
                          (got[pos].view(np.uint32) >> 16).astype(np.uint16))


@pytest.mark.parametrize("n_ranks", [8, 3])
def test_step_streams_on_chunked_gradients(n_ranks):
    """The rank values come from the chunked positions (element i of rank q
    at (i / G) N G + q G + i % G of one buffer); the rest of it is unread."""
    n, E, G = 3 * 2048 + 4 * 37, 1024, 512
    rng = np.random.default_rng(21 + n_ranks)
    dev = torch.device("cuda:0")
    grows = -(-n // G)
    gbuf = rng.integers(0, 1 << 16, grows * n_ranks * G, dtype=np.uint16) & 0xbfff
    dg = torch.from_numpy(gbuf.view(np.int16)).to(dev)
    rows = -(-n // E)
    buf = rng.standard_normal(rows * 3 * E).astype(np.float32)
    dbuf = torch.from_numpy(buf.copy()).to(dev)
    param = torch.zeros(n, dtype=torch.int16, device=dev)
    zs.stream_mix(zs.MIX_STEP_STREAMS, [dg[q * G:] for q in range(n_ranks)],
                  dbuf[0:], dbuf[E:], dbuf[2 * E:], param, n, state_chunk=E, grad_chunk=G)
    torch.cuda.synchronize()
    i = np.arange(n)
    acc = np.zeros(n, np.float32)
    for q in range(n_ranks):
        x = gbuf[(i // G) * n_ranks * G + q * G + i % G]
        acc = acc + (x.astype(np.uint32) << 16).view(np.float32)
    pos = (i // E) * 3 * E + i % E
    want = buf.copy()
    for k in range(3):
        want[pos + k * E] = buf[pos + k * E] + acc
    got = dbuf.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
