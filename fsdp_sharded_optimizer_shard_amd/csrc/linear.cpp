// A hand-written FSDP linear layer for one rank ("DP, ZeRO-1/2/3, FSDP"
// notes, follow-up on writing one FSDP linear layer by hand): every rank
// stores 1/N of the rows of W; forward all-gathers the full W and computes
// X W for the local batch; backward all-gathers W again, computes dX and the
// full-shape dW locally; the reduce-scatter of dW over the ranks is
// zero_reduce_shard on the N ranks' dW buffers.
//
// W is unit `unit` of a row layout (zero_shard_init_rows) with rows =
// in_features and cols = out_features, so Y = X W takes (batch x in) to
// (batch x out).  The contractions run on the MFMA GEMM, which reads each
// operand in place, contiguous along K or along its rows, so no transposed
// copy is made.  The batch is the K of the dW product, hence the GEMM's
// multiple-of-8 rule on it.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace zs {
zero_status zero_rows_fill(float *p, int64_t ld, int64_t r0, int64_t r1, int64_t cols,
                           hipStream_t s);
zero_status gemm_check(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                       int32_t a_order, const uint16_t *B, int64_t ldb, int32_t b_order,
                       const void *C, int64_t ldc, int32_t c_dtype);
}

namespace {

struct Dims {
    int64_t in, out, in_pad;
};

zero_status layer_dims(const zero_layout *L, int32_t unit, Dims *d)
{
    if (!L)
        return zs::fail(ZERO_ERR_INVALID_ARG, "layout is NULL");
    if (unit < 0 || unit >= L->n_units)
        return zs::fail(ZERO_ERR_INVALID_ARG, "unit %d outside [0, %d)", unit, L->n_units);
    d->out = L->cols[unit];
    d->in = L->numel[unit] / d->out;
    d->in_pad = L->padded[unit] / d->out;
    return ZERO_OK;
}

// The shards the gather reads: every one present and 2-byte aligned (the
// gather's own checks), so that a layer call fails before its first launch.
zero_status check_shards(const zero_layout *L, const uint16_t *const *w_shards)
{
    for (int32_t q = 0; q < L->parts; ++q) {
        if (!w_shards[q])
            return zs::fail(ZERO_ERR_INVALID_ARG, "W shard of rank %d is NULL", q);
        if (reinterpret_cast<uintptr_t>(w_shards[q]) % 2)
            return zs::fail(ZERO_ERR_ALIGNMENT, "W shard of rank %d is misaligned", q);
    }
    return ZERO_OK;
}

}  // namespace

extern "C" {

zero_status zero_fsdp_linear_forward(const zero_layout *L, int32_t unit,
                                     const uint16_t *const *w_shards, int64_t batch,
                                     const uint16_t *x, uint16_t *w_full, void *y,
                                     int32_t y_dtype, void *stream)
{
    Dims d;
    zero_status st = layer_dims(L, unit, &d);
    if (st != ZERO_OK)
        return st;
    if (!w_shards || !x || !w_full || !y || batch < 0)
        return zs::fail(ZERO_ERR_INVALID_ARG, "w_shards, x, w_full, y and batch >= 0 are "
                        "required");
    if ((st = check_shards(L, w_shards)) != ZERO_OK)
        return st;
    if (d.in % 8 || d.out % 8)
        return zs::fail(ZERO_ERR_UNSUPPORTED, "in_features and out_features must be "
                        "multiples of 8");
    // every check before the first launch: the GEMM's too
    if ((st = zs::gemm_check(batch, d.out, d.in, x, d.in, ZERO_K_INNER, w_full, d.out,
                             ZERO_K_OUTER, y, d.out, y_dtype)) != ZERO_OK)
        return st;
    if ((st = zero_gather_params(L, unit, unit + 1, w_shards, L->parts, w_full, stream)) != ZERO_OK)
        return st;
    // Y = X W: a(i, k) = X[i][k], b(j, k) = W[k][j]
    return zero_gemm_bf16(batch, d.out, d.in, x, d.in, ZERO_K_INNER, w_full, d.out, ZERO_K_OUTER,
                          y, d.out, y_dtype, stream);
}

zero_status zero_fsdp_linear_backward(const zero_layout *L, int32_t unit,
                                      const uint16_t *const *w_shards, int64_t batch,
                                      const uint16_t *x, const uint16_t *dy, uint16_t *w_full,
                                      void *dx, int32_t dx_dtype, float *dw_full, void *stream)
{
    Dims d;
    zero_status st = layer_dims(L, unit, &d);
    if (st != ZERO_OK)
        return st;
    if (!w_shards || !x || !dy || !w_full || !dx || !dw_full || batch < 0)
        return zs::fail(ZERO_ERR_INVALID_ARG, "every buffer and batch >= 0 are required");
    if ((st = check_shards(L, w_shards)) != ZERO_OK)
        return st;
    if (d.in % 8 || d.out % 8 || batch % 8)
        return zs::fail(ZERO_ERR_UNSUPPORTED, "in_features, out_features and batch must be "
                        "multiples of 8");
    // every check before the first launch: both GEMMs' too
    if ((st = zs::gemm_check(batch, d.in, d.out, dy, d.out, ZERO_K_INNER, w_full, d.out,
                             ZERO_K_INNER, dx, d.in, dx_dtype)) != ZERO_OK ||
        (st = zs::gemm_check(d.in, d.out, batch, x, d.in, ZERO_K_OUTER, dy, d.out, ZERO_K_OUTER,
                             dw_full, d.out, ZERO_FP32)) != ZERO_OK)
        return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // re-gather W (FSDP frees it after forward)
    if ((st = zero_gather_params(L, unit, unit + 1, w_shards, L->parts, w_full, stream)) != ZERO_OK)
        return st;
    // dX = dY W^T: a(i, k) = dY[i][k], b(j, k) = W[j][k]
    if ((st = zero_gemm_bf16(batch, d.in, d.out, dy, d.out, ZERO_K_INNER, w_full, d.out,
                             ZERO_K_INNER, dx, d.in, dx_dtype, stream)) != ZERO_OK)
        return st;
    // dW = X^T dY, fp32, full shape: a(i, k) = X[k][i], b(j, k) = dY[k][j]
    if ((st = zero_gemm_bf16(d.in, d.out, batch, x, d.in, ZERO_K_OUTER, dy, d.out, ZERO_K_OUTER,
                             dw_full, d.out, ZERO_FP32, stream)) != ZERO_OK)
        return st;
    // padding rows of the row-sharded layout hold zero gradient
    return zs::zero_rows_fill(dw_full, d.out, d.in, d.in_pad, d.out, s);
}

}  // extern "C"
