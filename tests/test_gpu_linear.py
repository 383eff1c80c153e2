"""GPU parity of the MFMA GEMM, the transpose and the FSDP linear layer
against the exact oracle (oracle/linear.py).

fp32 GEMM results must lie within gamma_K (|A| |B|) of the exact product
(products of bf16 values are exact in fp32, so this is the standard
rounding-error bound of an fp32 dot product in any order); bf16 results
within that plus half a bf16 ulp.  The reduce-scatter of dW adds the fp32
sum over ranks: (N - 1) u sum_q |dW_q| / N.
"""
import numpy as np
import pytest
import torch

from oracle import _c, linear
from oracle.layout import plan_rows

pytestmark = pytest.mark.gpu
zs = None
DEV = "cuda:0"
U32 = 2.0 ** -24


def setup_module(module):
    global zs
    from fsdp_sharded_optimizer_shard_amd import zs as _zs
    zs = _zs


def rand_bf16(rng, shape, scale=1.0):
    return _c.f32_to_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


def dev16(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV)


def host16(t):
    return t.cpu().numpy().view(np.uint16)


def check_f32(got, exact, bound, what):
    err = np.abs(got.astype(np.float64) - exact)
    assert np.all(err <= bound), f"{what}: max err {err.max():.3e}, worst excess " \
                                 f"{(err - bound).max():.3e}"


@pytest.mark.parametrize("M,N,K,extra", [(128, 128, 32, 0), (1, 1, 8, 0), (200, 300, 72, 8),
                                         (257, 129, 4096, 16), (64, 1000, 520, 0)])
def test_gemm_nt_within_fp32_bound(M, N, K, extra):
    rng = np.random.default_rng(M * 7 + N)
    lda = ldb = K + extra
    A = rand_bf16(rng, (M, lda))
    B = rand_bf16(rng, (N, ldb))
    a = linear.bf16_values(A)[:, :K]
    b = linear.bf16_values(B)[:, :K]
    exact = a @ b.T
    bound = linear.gemm_bound(a, b.T)
    C = torch.full((M, N + 3), 7.0, device=DEV)
    zs.gemm_bf16_nt(M, N, K, dev16(A), lda, dev16(B), ldb, C, N + 3, zs.FP32)
    Cb = torch.zeros((M, N), dtype=torch.int16, device=DEV)
    zs.gemm_bf16_nt(M, N, K, dev16(A), lda, dev16(B), ldb, Cb, N, zs.BF16)
    torch.cuda.synchronize()
    c = C.cpu().numpy()
    check_f32(c[:, :N], exact, bound, "fp32 C")
    assert np.all(c[:, N:] == 7.0)                       # columns past N untouched
    cb = linear.bf16_values(host16(Cb))
    check_f32(cb, exact, bound + 2.0 ** -8 * (np.abs(exact) + bound), "bf16 C")


ORDERS = [(0, 0), (1, 0), (0, 1), (1, 1)]


@pytest.mark.parametrize("ao,bo", ORDERS)
@pytest.mark.parametrize("M,N,K,pad", [(8, 8, 8, 0), (200, 312, 72, 8), (264, 520, 200, 16),
                                       (520, 256, 1096, 0), (3104, 2904, 136, 8),
                                       (2040, 9448, 72, 0), (256, 264, 40, 0),
                                       (136, 256, 256, 8), (272, 528, 1024, 0)])
def test_gemm_operand_orders_within_fp32_bound(ao, bo, M, N, K, pad):
    """Every operand order (K-inner: stored rows x K; K-outer: stored K x
    rows), ragged in M, N and K, with leading dimensions wider than the
    matrix.  K runs through 1, 2, 3, 5, 7, 8, 32 and 35 stages of 32, with
    and without a partial last stage; 256 and 1024 end on whole stages, and
    1024 and 1096 run the four-stage steady loop.  On a 256-CU part the
    small shapes run as 128 x 256 half tiles only, 3104 x 2904 (156 tiles)
    as whole tiles only, and 2040 x 9448 (296 tiles) as one wave of whole
    tiles plus 80 half tiles."""
    rng = np.random.default_rng(M + 3 * N + 7 * K + 11 * ao + 13 * bo)
    a = rand_bf16(rng, (M, K))
    b = rand_bf16(rng, (N, K))
    def stored(x, outer):
        rows, k = x.shape
        st = np.full((k, rows + pad) if outer else (rows, k + pad), 0x7FC0, np.uint16)
        if outer:
            st[:, :rows] = x.T
        else:
            st[:, :k] = x
        return st
    A, B = stored(a, ao), stored(b, bo)
    av, bv = linear.bf16_values(a), linear.bf16_values(b)
    exact = av @ bv.T
    bound = linear.gemm_bound(av, bv.T)
    C = torch.full((M, N + 5), 7.0, device=DEV)
    Cb = torch.zeros((M, N), dtype=torch.int16, device=DEV)
    order = (zs.K_INNER, zs.K_OUTER)
    zs.gemm_bf16(M, N, K, dev16(A), A.shape[1], order[ao], dev16(B), B.shape[1], order[bo], C,
                 N + 5, zs.FP32)
    zs.gemm_bf16(M, N, K, dev16(A), A.shape[1], order[ao], dev16(B), B.shape[1], order[bo], Cb,
                 N, zs.BF16)
    torch.cuda.synchronize()
    c = C.cpu().numpy()
    check_f32(c[:, :N], exact, bound, "fp32 C")
    assert np.all(c[:, N:] == 7.0)          # columns past N untouched (the padding holds NaN)
    cb = linear.bf16_values(host16(Cb))
    check_f32(cb, exact, bound + 2.0 ** -8 * (np.abs(exact) + bound), "bf16 C")


def test_gemm_at_the_leading_dimension_limits():
    """The largest leading dimensions the host accepts: a K-inner A with
    lda = 2^22 (a 256-row panel then spans 255 * 2^23 bytes, just under the
    2^31 of a buffer offset) and a K-outer B with ldb = 2^25 (k row 31 of a
    stage at 31 * 2^26 bytes).  M = 264 runs one whole tile and one half
    tile.  Rows past M and columns past N of C stay untouched."""
    M, N, K = 264, 136, 40
    lda, ldb = 1 << 22, 1 << 25
    rng = np.random.default_rng(22)
    a = rand_bf16(rng, (M, K))
    b = rand_bf16(rng, (N, K))
    A = torch.zeros((M, lda), dtype=torch.int16, device=DEV)        # 2.2 GB
    A[:, :K] = dev16(a)
    B = torch.zeros((K, ldb), dtype=torch.int16, device=DEV)        # 2.7 GB
    B[:, :N] = dev16(np.ascontiguousarray(b.T))
    av, bv = linear.bf16_values(a), linear.bf16_values(b)
    exact = av @ bv.T
    bound = linear.gemm_bound(av, bv.T)
    C = torch.full((M + 2, N + 5), 7.0, device=DEV)
    zs.gemm_bf16(M, N, K, A, lda, zs.K_INNER, B, ldb, zs.K_OUTER, C, N + 5, zs.FP32)
    torch.cuda.synchronize()
    c = C.cpu().numpy()
    del A, B
    torch.cuda.empty_cache()
    check_f32(c[:M, :N], exact, bound, "fp32 C")
    assert np.all(c[:, N:] == 7.0) and np.all(c[M:, :] == 7.0)


def test_gemm_k_zero_writes_zeros():
    C = torch.full((16, 24), 3.0, device=DEV)
    buf = torch.zeros(64, dtype=torch.int16, device=DEV)
    zs.gemm_bf16(16, 24, 0, buf, 16, zs.K_OUTER, buf, 24, zs.K_OUTER, C, 24, zs.FP32)
    torch.cuda.synchronize()
    assert not C.cpu().numpy().any()


def test_transpose_exact():
    rng = np.random.default_rng(3)
    for rows, cols in [(1, 1), (64, 64), (130, 77), (1000, 33)]:
        x = rng.integers(0, 1 << 16, (rows, cols), dtype=np.uint16)
        out = torch.zeros((cols, rows + 5), dtype=torch.int16, device=DEV)
        zs.transpose_bf16(rows, cols, dev16(x), cols, out, rows + 5)
        torch.cuda.synchronize()
        got = host16(out)
        assert np.array_equal(got[:, :rows], x.T)
        assert not got[:, rows:].any()


def _layer(n, rank, inf, outf, batch, seed):
    rng = np.random.default_rng(seed)
    lay = plan_rows([(inf, outf)], n, rank)
    L = zs.shard_init_rows("fsdp2", n, rank, [(inf, outf)])
    c = lay.units[0].shard // outf
    w = rand_bf16(rng, (inf, outf), 0.02)
    shards = []
    for q in range(n):
        sh = np.zeros((c, outf), np.uint16)
        take = max(0, min(c, inf - q * c))
        sh[:take] = w[q * c:q * c + take]
        shards.append(sh)
    xs = [rand_bf16(rng, (batch, inf)) for _ in range(n)]
    dys = [rand_bf16(rng, (batch, outf), 1e-2) for _ in range(n)]
    return lay, L, c, w, shards, xs, dys


def _run_layer(L, n, rank, inf, outf, batch, c, shards, xs, dys):
    Lu = L.query(0)["padded_len"]
    dsh = [dev16(s) for s in shards]
    w_full = torch.empty(Lu, dtype=torch.int16, device=DEV)
    y = torch.empty((batch, outf), device=DEV)
    zs.fsdp_linear_forward(L, 0, dsh, batch, dev16(xs[rank]), w_full, y, zs.FP32)
    dws, dx = [], None
    for q in range(n):
        dw = torch.full((Lu,), 9.0, device=DEV)
        dxq = torch.empty((batch, inf), device=DEV)
        zs.fsdp_linear_backward(L, 0, dsh, batch, dev16(xs[q]), dev16(dys[q]), w_full, dxq, dw,
                                zs.FP32)
        dws.append(dw)
        if q == rank:
            dx = dxq
    shard = torch.empty(L.shard_len, device=DEV)
    zs.reduce_shard(L, 0, 1, zs.Grads(dws, zs.FP32, zs.INDEX_FULL), shard)
    torch.cuda.synchronize()
    return y.cpu().numpy(), dx.cpu().numpy(), [d.cpu().numpy() for d in dws], shard.cpu().numpy()


@pytest.mark.parametrize("n,rank,inf,outf,batch", [(3, 2, 200, 48, 64), (4, 0, 256, 128, 128),
                                                   (8, 5, 96, 520, 40)])
def test_fsdp_linear_layer_matches_oracle(n, rank, inf, outf, batch):
    lay, L, c, w, shards, xs, dys = _layer(n, rank, inf, outf, batch, seed=inf + outf)
    y, dx, dws, shard = _run_layer(L, n, rank, inf, outf, batch, c, shards, xs, dys)
    W = linear.gather_rows(lay, [linear.bf16_values(s) for s in shards], inf, outf)
    assert np.array_equal(W, linear.bf16_values(w))
    X = [linear.bf16_values(x) for x in xs]
    DY = [linear.bf16_values(d) for d in dys]
    check_f32(y, linear.forward(W, X[rank]), linear.gemm_bound(X[rank], W), "Y")
    ex_dx, _ = linear.backward(W, X[rank], DY[rank])
    check_f32(dx, ex_dx, linear.gemm_bound(DY[rank], W.T), "dX")
    exact_dw = []
    bounds = []
    for q in range(n):
        _, e = linear.backward(W, X[q], DY[q])
        exact_dw.append(e)
        b = linear.gemm_bound(X[q].T, DY[q])
        bounds.append(b)
        got = dws[q].reshape(-1, outf)
        check_f32(got[:inf], e, b, f"dW rank {q}")
        assert np.all(got[inf:] == 0.0), "padding rows of dW must be zero"
    want = linear.reduce_scatter_mean(lay, exact_dw, outf)
    sum_abs = sum(np.abs(e) + b for e, b in zip(exact_dw, bounds))
    bound_rows = (sum(bounds) + (n - 1) * U32 * sum_abs) / n + U32 * np.abs(sum(exact_dw) / n)
    bd = np.zeros_like(want)
    take = max(0, min(c, inf - rank * c))
    bd[:take] = bound_rows[rank * c:rank * c + take]
    check_f32(shard.reshape(c, outf), want, bd, "reduce-scattered dW shard")


def test_fsdp_linear_mistral_mlp_up_sampled():
    """in 4096, out 14336 (Mistral-7B MLP up projection), 4096 tokens per
    rank, N = 8, rank 7; sampled outputs against exact dot products."""
    n, rank, inf, outf, batch = 8, 7, 4096, 14336, 4096
    lay, L, c, w, shards, xs, dys = _layer(n, rank, inf, outf, batch, seed=11)
    y, dx, dws, shard = _run_layer(L, n, rank, inf, outf, batch, c, shards, xs, dys)
    W = linear.bf16_values(w)
    X = [linear.bf16_values(x) for x in xs]
    DY = [linear.bf16_values(d) for d in dys]
    rng = np.random.default_rng(5)
    for _ in range(2000):
        i, j = rng.integers(0, batch), rng.integers(0, outf)
        a, b = X[rank][i], W[:, j]
        assert abs(y[i, j] - a @ b) <= linear.gamma(inf) * (np.abs(a) @ np.abs(b))
        k = rng.integers(0, inf)
        a, b = DY[rank][i], W[k]
        assert abs(dx[i, k] - a @ b) <= linear.gamma(outf) * (np.abs(a) @ np.abs(b))
        # this rank's rows of the mean dW
        rr = rank * c + rng.integers(0, c)
        ex = [X[q][:, rr] @ DY[q][:, j] for q in range(n)]
        bq = [linear.gamma(batch) * (np.abs(X[q][:, rr]) @ np.abs(DY[q][:, j])) for q in range(n)]
        bound = (sum(bq) + (n - 1) * U32 * sum(abs(e) + b for e, b in zip(ex, bq))) / n \
            + U32 * abs(sum(ex) / n)
        assert abs(shard[(rr - rank * c) * outf + j] - sum(ex) / n) <= bound
