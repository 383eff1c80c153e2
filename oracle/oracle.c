/*
 * Plain CPU oracle for one data-parallel rank's sharded mixed-precision
 * optimizer step (DDP / ZeRO-1/2/3 / FSDP / Megatron distributed optimizer).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark do.  It shares no code,
 * header or constant with the HIP library: every routine below is written
 * here from the published definition it names.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fPIC -shared (see build.py).
 * x86-64 SSE arithmetic rounds every float operation to binary32 once, and
 * -ffp-contract=off forbids fusing a multiply into an add, so each line below
 * is exactly one IEEE-754 round-to-nearest-even operation in the stated type.
 *
 * What is computed, and where the pages define it:
 *  - Data-parallel averaging (all-reduce / reduce-scatter arithmetic): every
 *    rank's gradient is summed and divided by N so that every replica holds
 *    the mean ("Data Parallel, ZeRO and FSDP", section "Plain data parallel
 *    (DDP)"; "dp-zero-fsdp", concepts: DDP, reduce-scatter and all-gather).
 *    Reading taken: fp32 sum in ascending rank order, then one division by N.
 *  - Mixed-precision Adam state: bf16 param and grad, fp32 master / m / v
 *    ("dp-zero-fsdp", concepts: Model states 16 bytes per parameter).  The
 *    pages do not write Adam's update; it is Kingma & Ba (2015), Algorithm 1
 *    (bias-corrected moments, epsilon added outside the square root), with
 *    Loshchilov & Hutter (2019) decoupled weight decay for AdamW and the
 *    classic L2 form (g + wd * p) for plain Adam with weight decay.
 *  - fp32 gradient accumulation for the Megatron distributed optimizer
 *    ("dp-zero-fsdp", worked example 7B / N = 8, Megatron row note).
 *  - bf16 rounding: IEEE-754 round to nearest, ties to even, on the upper
 *    16 bits of the binary32 pattern; NaN becomes the quiet NaN 0x7FC0.
 *  - Global gradient-norm clipping is not on the pages; reading taken:
 *    PyTorch clip_grad_norm_ semantics (L2 norm of the averaged gradient over
 *    all parameters, coefficient max_norm / (norm + 1e-6), applied if < 1).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---------------------------------------------------------------- bf16 -- */

static float bf16_bits_to_float(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16; /* bf16 is the top half of binary32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint16_t float_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) /* any NaN */
        return (uint16_t)0x7fc0u;
    /* Round to nearest even on bit 16: add 0x7fff plus the lowest kept bit;
       a carry out of the low half bumps the kept part (and may carry into
       the exponent, which is the correct rounding to the next binade / Inf). */
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7fffu + keep_lsb;
    return (uint16_t)(u >> 16);
}

void orc_bf16_to_f32(const uint16_t *in, float *out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = bf16_bits_to_float(in[i]);
}

void orc_f32_to_bf16(const float *in, uint16_t *out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = float_to_bf16_rne(in[i]);
}

/* ------------------------------------------------------- DP averaging -- */

/* out[i] = (G_0[i] + G_1[i] + ... + G_{N-1}[i]) / N, sum in fp32, ranks in
   ascending order, starting from +0. */
void orc_average_bf16(int32_t n_ranks, const uint16_t *const *ranks,
                      int64_t count, float *out)
{
    const float n = (float)n_ranks;
    for (int64_t i = 0; i < count; ++i) {
        float acc = 0.0f;
        for (int32_t q = 0; q < n_ranks; ++q)
            acc = acc + bf16_bits_to_float(ranks[q][i]);
        out[i] = acc / n;
    }
}

void orc_average_f32(int32_t n_ranks, const float *const *ranks, int64_t count,
                     float *out)
{
    const float n = (float)n_ranks;
    for (int64_t i = 0; i < count; ++i) {
        float acc = 0.0f;
        for (int32_t q = 0; q < n_ranks; ++q)
            acc = acc + ranks[q][i];
        out[i] = acc / n;
    }
}

/* Megatron-style fp32 main-gradient accumulation of one bf16 micro-batch
   gradient: acc[i] = acc[i] + float(micro[i]). */
void orc_accumulate_bf16(float *acc, const uint16_t *micro, int64_t count)
{
    for (int64_t i = 0; i < count; ++i)
        acc[i] = acc[i] + bf16_bits_to_float(micro[i]);
}

/* ------------------------------------------------------------- clipping -- */

/* Sum of squares in fp64, sequential in index order.  (double)g * (double)g
   is exact (24-bit significands), so only the additions round. */
double orc_sumsq_f32(const float *g, int64_t count)
{
    double s = 0.0;
    for (int64_t i = 0; i < count; ++i) {
        double x = (double)g[i];
        s = s + x * x;
    }
    return s;
}

/* Clip coefficient from the global sum of squares: fp64 norm, fp64 quotient,
   one rounding to fp32, clamped at 1. */
float orc_clip_coef(double sumsq, float max_norm)
{
    double norm = sqrt(sumsq);
    float c = (float)((double)max_norm / (norm + 1e-6));
    return c < 1.0f ? c : 1.0f;
}

void orc_scale_f32(float *g, int64_t count, float c)
{
    for (int64_t i = 0; i < count; ++i)
        g[i] = g[i] * c;
}

/* ----------------------------------------------------------------- Adam -- */

typedef struct {
    float lr;
    float beta1;
    float beta2;
    float eps;
    float weight_decay;
    int64_t step;      /* t, starting at 1 */
    int32_t decoupled; /* 1: AdamW (decoupled), 0: L2 added to the gradient */
    int32_t _pad;
} orc_adam_hparams;

/* Step-dependent scalars, each evaluated in fp64 from the fp32
   hyper-parameters and rounded once to fp32. */
typedef struct {
    float one_minus_b1, one_minus_b2, bias1, bias2, decay;
} orc_adam_scalars;

static orc_adam_scalars adam_scalars(const orc_adam_hparams *h)
{
    orc_adam_scalars s;
    double b1 = (double)h->beta1, b2 = (double)h->beta2, t = (double)h->step;
    s.one_minus_b1 = (float)(1.0 - b1);
    s.one_minus_b2 = (float)(1.0 - b2);
    s.bias1 = (float)(1.0 - pow(b1, t));
    s.bias2 = (float)(1.0 - pow(b2, t));
    s.decay = (float)(1.0 - (double)h->lr * (double)h->weight_decay);
    return s;
}

/* One Adam / AdamW step on fp32 state, in place.  Per element:
 *   (L2 form)  g <- g + wd * p
 *   (AdamW)    p <- p * (1 - lr * wd)
 *   m <- b1 * m + (1 - b1) * g
 *   v <- b2 * v + (1 - b2) * g^2
 *   p <- p - lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
 */
void orc_adam_f32(const orc_adam_hparams *h, int64_t count, const float *grad,
                  float *p, float *m, float *v)
{
    const orc_adam_scalars s = adam_scalars(h);
    const float b1 = h->beta1, b2 = h->beta2, lr = h->lr, eps = h->eps;
    const float wd = h->weight_decay;
    for (int64_t i = 0; i < count; ++i) {
        float g = grad[i];
        float pi = p[i];
        if (wd != 0.0f) {
            if (h->decoupled)
                pi = pi * s.decay;
            else
                g = g + wd * pi;
        }
        float mi = b1 * m[i] + s.one_minus_b1 * g;
        float vi = b2 * v[i] + s.one_minus_b2 * (g * g);
        float m_hat = mi / s.bias1;
        float v_hat = vi / s.bias2;
        float denom = sqrtf(v_hat) + eps;
        pi = pi - lr * (m_hat / denom);
        p[i] = pi;
        m[i] = mi;
        v[i] = vi;
    }
}

/* The same update carried out entirely in fp64 (constants included).  Used
   only to bound the rounding error of the fp32 oracle. */
void orc_adam_f64(const orc_adam_hparams *h, int64_t count, const double *grad,
                  double *p, double *m, double *v)
{
    const double b1 = (double)h->beta1, b2 = (double)h->beta2;
    const double lr = (double)h->lr, eps = (double)h->eps;
    const double wd = (double)h->weight_decay, t = (double)h->step;
    const double bias1 = 1.0 - pow(b1, t), bias2 = 1.0 - pow(b2, t);
    for (int64_t i = 0; i < count; ++i) {
        double g = grad[i];
        double pi = p[i];
        if (wd != 0.0) {
            if (h->decoupled)
                pi = pi * (1.0 - lr * wd);
            else
                g = g + wd * pi;
        }
        double mi = b1 * m[i] + (1.0 - b1) * g;
        double vi = b2 * v[i] + (1.0 - b2) * (g * g);
        pi = pi - lr * ((mi / bias1) / (sqrt(vi / bias2) + eps));
        p[i] = pi;
        m[i] = mi;
        v[i] = vi;
    }
}

/* ---------------------------------------------- one rank, one element run -- */

/* The whole per-element chain for a contiguous run of owned elements, as the
   separate steps above applied in order: average the N rank gradients, scale
   by the clip coefficient when it is below 1, take the Adam step, round the
   new master to bf16.  Temporary storage for the averaged gradient is the
   caller's (count floats). */
void orc_rank_step_bf16(const orc_adam_hparams *h, int32_t n_ranks,
                        const uint16_t *const *ranks, int64_t count,
                        float clip_coef, float *tmp_grad, float *p, float *m,
                        float *v, uint16_t *param_out)
{
    orc_average_bf16(n_ranks, ranks, count, tmp_grad);
    if (clip_coef < 1.0f)
        orc_scale_f32(tmp_grad, count, clip_coef);
    orc_adam_f32(h, count, tmp_grad, p, m, v);
    orc_f32_to_bf16(p, param_out, count);
}

void orc_rank_step_f32(const orc_adam_hparams *h, int32_t n_ranks,
                       const float *const *ranks, int64_t count,
                       float clip_coef, float *tmp_grad, float *p, float *m,
                       float *v, uint16_t *param_out)
{
    orc_average_f32(n_ranks, ranks, count, tmp_grad);
    if (clip_coef < 1.0f)
        orc_scale_f32(tmp_grad, count, clip_coef);
    orc_adam_f32(h, count, tmp_grad, p, m, v);
    orc_f32_to_bf16(p, param_out, count);
}
