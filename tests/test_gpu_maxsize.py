"""GPU parity past 2^31 elements: element indices that no longer fit in 32
bits, on the fused step, the gather and the fp32 accumulation.

The workloads stop at 1.1e9 elements per shard, where byte offsets already
pass 2^31 but element indices do not. Here one unit holds 2^31 + 4099
elements, so the last group of four is ragged and takes the scalar path;
one case runs a shard of that length in the chunked state and chunked
gradient formats. Inputs are drawn on the device. The elements compared lie
around index 2^31, at both ends and at random. Each is checked bit for bit
against the oracle run on the same values. Peak device memory is about
45 GB.
"""
import numpy as np
import pytest
import torch

from oracle import _c

pytestmark = pytest.mark.gpu

zs = None
DEV = "cuda:0"
BIG = (1 << 31) + 4099


def setup_module(module):
    global zs
    from fsdp_sharded_optimizer_shard_amd import zs as _zs
    zs = _zs


def _samples(n, seed):
    rng = np.random.default_rng(seed)
    parts = [np.arange(0, 64), np.arange((1 << 31) - 2048, min(n, (1 << 31) + 2048)),
             np.arange(n - 2048, n), rng.integers(0, n, 4096)]
    return np.unique(np.concatenate(parts)).astype(np.int64)


def _bf16_randn(n, scale, gen):
    t = torch.randn(n, device=DEV, generator=gen)
    t.mul_(scale)
    out = t.to(torch.bfloat16).view(torch.int16)
    del t
    return out


def _at(t, ti):
    return t[ti].cpu().numpy().copy()


def _same_bits(got, want, what):
    view = np.uint32 if got.dtype == np.float32 else np.uint16
    bad = np.count_nonzero(got.view(view) != want.view(view))
    assert bad == 0, f"{what}: {bad} of {got.size} sampled elements differ"


def _release():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_fused_step_past_2_31_elements():
    n = BIG
    L = zs.shard_init("zero2", 1, 0, [n])
    assert L.shard_len == n
    gen = torch.Generator(device=DEV)
    gen.manual_seed(31)
    master = torch.randn(n, device=DEV, generator=gen)
    master.mul_(0.02)
    grad = _bf16_randn(n, 1e-3, gen)
    m = torch.zeros(n, device=DEV)
    v = torch.zeros(n, device=DEV)
    out = torch.empty(n, dtype=torch.int16, device=DEV)
    idx = _samples(n, 31)
    ti = torch.from_numpy(idx).to(DEV)
    p_h, g_h = _at(master, ti), _at(grad, ti).view(np.uint16)
    cfg = zs.adam_cfg(lr=1e-3, weight_decay=0.01, decoupled=True, step=1)
    zs.adam_step(L, 0, 1, cfg, master, m, v, out,
                 grads=zs.Grads([grad], zs.BF16, zs.INDEX_FULL))
    torch.cuda.synchronize()
    m_h = np.zeros(idx.size, np.float32)
    v_h = np.zeros(idx.size, np.float32)
    par_h = np.empty(idx.size, np.uint16)
    _c.rank_step(_c.hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1, True), [g_h], 1.0, p_h, m_h,
                 v_h, par_h)
    _same_bits(_at(master, ti), p_h, "master")
    _same_bits(_at(m, ti), m_h, "m")
    _same_bits(_at(v, ti), v_h, "v")
    _same_bits(_at(out, ti).view(np.uint16), par_h, "bf16 param")
    del master, grad, m, v, out, ti
    _release()


def test_gather_past_2_31_elements():
    # rank 0 of two; the peer's slice of the flat buffer lies past 2^31
    n = BIG
    L = zs.shard_init("zero3", 2, 0, [n])
    s = L.query(0)["shard_len"]
    assert 2 * s > (1 << 31)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(32)
    peer = torch.randint(-32768, 32768, (s,), dtype=torch.int16, device=DEV, generator=gen)
    full = torch.zeros(2 * s, dtype=torch.int16, device=DEV)
    zs.gather_params(L, 0, 1, [None, peer], full)
    torch.cuda.synchronize()
    j = _samples(s, 32)
    j = j[j < s]
    tj = torch.from_numpy(j).to(DEV)
    _same_bits(_at(full, tj + s).view(np.uint16), _at(peer, tj).view(np.uint16), "peer slice")
    assert not _at(full, tj).any()          # this rank's own slice is not the gather's
    del peer, full, tj
    _release()


def test_grad_accumulate_past_2_31_elements():
    n = BIG
    gen = torch.Generator(device=DEV)
    gen.manual_seed(33)
    acc = torch.randn(n, device=DEV, generator=gen)
    acc.mul_(1e-3)
    micro = _bf16_randn(n, 1e-3, gen)
    idx = _samples(n, 33)
    ti = torch.from_numpy(idx).to(DEV)
    a_h, mb_h = _at(acc, ti), _at(micro, ti).view(np.uint16)
    zs.grad_accumulate(acc, micro, n)
    torch.cuda.synchronize()
    _c.accumulate_bf16(a_h, np.ascontiguousarray(mb_h))
    _same_bits(_at(acc, ti), a_h, "main gradient")
    del acc, micro, ti
    _release()


def test_chunked_formats_past_2_31_shard_elements():
    # two ranks, each with a shard of 2^31 + 4099 elements: the chunked
    # state and the chunked receive buffer of both ranks' gradients are
    # addressed with shard indices past 2^31 (and buffer offsets past 2^32)
    n, E, GE = BIG, 8192, 16384
    L = zs.shard_init("zero3", 2, 1, [2 * n]).chunk_state(E)
    assert L.shard_len == n
    gen = torch.Generator(device=DEV)
    gen.manual_seed(34)
    st = torch.empty(L.state_len, device=DEV)
    st.normal_(0.0, 0.02, generator=gen)
    st.view(-1, 3, E)[:, 2, :].abs_()            # v >= 0
    recv = torch.empty(L.grad_len(GE), dtype=torch.int16, device=DEV)
    step = 1 << 30
    for off in range(0, recv.numel(), step):
        k = min(step, recv.numel() - off)
        recv[off:off + k] = _bf16_randn(k, 1e-3, gen)
    out = torch.empty(n, dtype=torch.int16, device=DEV)
    idx = _samples(n, 34)
    pos = torch.from_numpy((idx // E) * 3 * E + idx % E).to(DEV)
    gpos = [torch.from_numpy((idx // GE) * 2 * GE + q * GE + idx % GE).to(DEV) for q in range(2)]
    p_h, m_h, v_h = _at(st, pos), _at(st, pos + E), _at(st, pos + 2 * E)
    g_h = [_at(recv, gp).view(np.uint16) for gp in gpos]
    cfg = zs.adam_cfg(lr=1e-3, weight_decay=0.01, decoupled=True, step=3)
    zs.adam_step(L, 0, 1, cfg, *L.state_views(st), out, zs.INDEX_SHARD,
                 grads=zs.Grads.chunked(recv, 2, GE))
    torch.cuda.synchronize()
    par_h = np.empty(idx.size, np.uint16)
    _c.rank_step(_c.hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 3, True), g_h, 1.0, p_h, m_h, v_h,
                 par_h)
    _same_bits(_at(st, pos), p_h, "master")
    _same_bits(_at(st, pos + E), m_h, "m")
    _same_bits(_at(st, pos + 2 * E), v_h, "v")
    _same_bits(_at(out, torch.from_numpy(idx).to(DEV)).view(np.uint16), par_h, "bf16 param")
    del st, recv, out, pos, gpos
    _release()
