/*
 * A C program that drives libzeroshard through its C ABI alone, with no
 * Python and no torch: it allocates device memory with hipMalloc, runs three
 * optimizer steps of one ZeRO-3 rank (fused reduce of 4 bf16 rank gradients
 * + Adam + bf16 cast, then the gather of the 3 peer shards) on a ragged
 * three-unit layout, and compares every element of master, m, v and the full
 * bf16 buffer with the C oracle (oracle/liboracle.so) run on the same inputs.
 * The same steps run a second time side by side in the chunked formats: the
 * state in one buffer of 64-element chunks (zero_layout_chunk_state) and the
 * 4 rank gradients in one receive buffer of 16-element rows per rank
 * (zero_grads.chunk).
 *
 * Test infrastructure: built by __graft_entry__.build(), run by
 * tests/test_gpu_capi_c.py.  Prints "capi demo ok" and exits 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zero_shard.h"

/* The oracle's parameter block and per-rank chain (oracle/oracle.c). */
typedef struct {
    float lr, beta1, beta2, eps, weight_decay;
    int64_t step;
    int32_t decoupled, pad;
} orc_hparams;
void orc_rank_step_bf16(const orc_hparams *h, int32_t n_ranks, const uint16_t *const *ranks,
                        int64_t count, float clip_coef, float *tmp_grad, float *p, float *m,
                        float *v, uint16_t *param_out);

#define N_RANKS 4
#define RANK 1
#define N_UNITS 3
#define STEPS 3
#define STATE_CHUNK 64
#define GRAD_CHUNK 16

#define HIP(x)                                                                          \
    do {                                                                                \
        hipError_t e_ = (x);                                                            \
        if (e_ != hipSuccess) {                                                         \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
            exit(1);                                                                    \
        }                                                                               \
    } while (0)
#define ZS(x)                                                                             \
    do {                                                                                  \
        zero_status s_ = (x);                                                             \
        if (s_ != ZERO_OK) {                                                              \
            fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, zero_status_str(s_), \
                    zero_last_error());                                                   \
            exit(1);                                                                      \
        }                                                                                 \
    } while (0)

/* splitmix64: the inputs' generator */
static uint64_t rng_state = 0x5eed;
static uint64_t next64(void)
{
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}
static float uniform(float scale) { return scale * ((float)(next64() >> 40) / 8388608.0f - 1.0f); }
static uint16_t bf16_bits(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    return (uint16_t)(u >> 16);
}

static void *dev_copy(const void *host, size_t bytes)
{
    void *d = NULL;
    HIP(hipMalloc(&d, bytes));
    HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

int main(void)
{
    const int64_t numel[N_UNITS] = {5000, 3000, 777};
    zero_layout *L = NULL;
    ZS(zero_shard_init(&L, ZERO_STAGE3, N_RANKS, RANK, N_UNITS, numel));
    int64_t P = 0, S = 0;
    ZS(zero_layout_info(L, &P, &S, NULL, NULL, NULL, NULL));
    int64_t flat_off[N_UNITS], shard_len[N_UNITS], shard_off[N_UNITS];
    for (int u = 0; u < N_UNITS; ++u)
        ZS(zero_layout_query(L, u, NULL, NULL, &flat_off[u], &shard_len[u], &shard_off[u], NULL));

    /* host inputs */
    uint16_t *grads[N_RANKS], *peers[N_RANKS];
    for (int q = 0; q < N_RANKS; ++q) {
        grads[q] = malloc(S * 2);
        peers[q] = malloc(S * 2);
        for (int64_t i = 0; i < S; ++i) {
            grads[q][i] = bf16_bits(uniform(1e-3f));
            peers[q][i] = bf16_bits(uniform(0.02f));
        }
    }
    float *p = malloc(S * 4), *m = calloc(S, 4), *v = calloc(S, 4), *tmp = malloc(S * 4);
    uint16_t *own = malloc(S * 2), *full = malloc(P * 2), *want = malloc(P * 2);
    for (int64_t i = 0; i < S; ++i)
        p[i] = uniform(0.02f);

    /* the chunked formats: a copy of the layout with master, m and v in one
       buffer of E-element chunks (master at (i / E) 3E + i % E), and the
       rank gradients in one buffer of rows of GE elements per rank (rank q's
       element i at (i / GE) N GE + q GE + i % GE) */
    zero_layout *LC = NULL;
    ZS(zero_layout_chunk_state(L, STATE_CHUNK, &LC));
    int64_t E = 0, SL = 0;
    ZS(zero_layout_state(LC, &E, &SL));
    const int64_t GE = GRAD_CHUNK, grows = (S + GE - 1) / GE;
    float *hs = calloc(SL, 4);
    uint16_t *hrecv = calloc(grows * N_RANKS * GE, 2);
    for (int64_t i = 0; i < S; ++i) {
        hs[(i / E) * 3 * E + i % E] = p[i];
        for (int q = 0; q < N_RANKS; ++q)
            hrecv[(i / GE) * N_RANKS * GE + q * GE + i % GE] = grads[q][i];
    }

    /* device buffers */
    const void *dg[N_RANKS];
    const uint16_t *dpeer[N_RANKS];
    for (int q = 0; q < N_RANKS; ++q) {
        dg[q] = dev_copy(grads[q], S * 2);
        dpeer[q] = q == RANK ? NULL : dev_copy(peers[q], S * 2);
    }
    float *dp = dev_copy(p, S * 4), *dm = dev_copy(m, S * 4), *dv = dev_copy(v, S * 4);
    float *ds = dev_copy(hs, SL * 4);
    const uint16_t *drecv = dev_copy(hrecv, grows * N_RANKS * GE * 2);
    const void *dgc[N_RANKS];
    for (int q = 0; q < N_RANKS; ++q)
        dgc[q] = drecv + q * GE;
    uint16_t *dfull = NULL, *dfull2 = NULL;
    HIP(hipMalloc((void **)&dfull, P * 2));
    HIP(hipMalloc((void **)&dfull2, P * 2));
    HIP(hipMemset(dfull, 0xff, P * 2));
    HIP(hipMemset(dfull2, 0xff, P * 2));
    HIP(hipDeviceSynchronize());

    const zero_grads g = {dg, NULL, N_RANKS, ZERO_BF16, ZERO_INDEX_SHARD, 0};
    const zero_grads gc = {dgc, NULL, N_RANKS, ZERO_BF16, ZERO_INDEX_SHARD, GRAD_CHUNK};
    for (int t = 1; t <= STEPS; ++t) {
        const zero_adam_cfg cfg = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, 1, t};
        ZS(zero_adam_step(L, 0, N_UNITS, &cfg, NULL, ZERO_INDEX_SHARD, NULL, &g, dp, dm, dv,
                          dfull, ZERO_INDEX_FULL, NULL));
        ZS(zero_gather_params(L, 0, N_UNITS, dpeer, N_RANKS, dfull, NULL));
        ZS(zero_adam_step(LC, 0, N_UNITS, &cfg, NULL, ZERO_INDEX_SHARD, NULL, &gc, ds, ds + E,
                          ds + 2 * E, dfull2, ZERO_INDEX_FULL, NULL));
        ZS(zero_gather_params(LC, 0, N_UNITS, dpeer, N_RANKS, dfull2, NULL));
        const orc_hparams h = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, t, 1, 0};
        orc_rank_step_bf16(&h, N_RANKS, (const uint16_t *const *)grads, S, 1.0f, tmp, p, m, v,
                           own);
    }
    HIP(hipDeviceSynchronize());

    /* expected full buffer: this rank's slices from the oracle, peers' as given */
    for (int u = 0; u < N_UNITS; ++u)
        for (int q = 0; q < N_RANKS; ++q)
            memcpy(want + flat_off[u] + q * shard_len[u],
                   (q == RANK ? own : peers[q]) + shard_off[u], shard_len[u] * 2);

    float *gp = malloc(S * 4), *gm = malloc(S * 4), *gv = malloc(S * 4);
    HIP(hipMemcpy(gp, dp, S * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(gm, dm, S * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(gv, dv, S * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(full, dfull, P * 2, hipMemcpyDeviceToHost));
    const int bad = memcmp(gp, p, S * 4) != 0 || memcmp(gm, m, S * 4) != 0 ||
                    memcmp(gv, v, S * 4) != 0 || memcmp(full, want, P * 2) != 0;
    HIP(hipMemcpy(hs, ds, SL * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(full, dfull2, P * 2, hipMemcpyDeviceToHost));
    int bad_chunked = memcmp(full, want, P * 2) != 0;
    for (int64_t i = 0; i < S; ++i) {
        const float *x = hs + (i / E) * 3 * E + i % E;
        bad_chunked |= memcmp(x, p + i, 4) != 0 || memcmp(x + E, m + i, 4) != 0 ||
                       memcmp(x + 2 * E, v + i, 4) != 0;
    }
    zero_shard_destroy(LC);
    zero_shard_destroy(L);
    if (bad || bad_chunked) {
        fprintf(stderr, "capi demo: results differ from the oracle (%s)\n",
                bad ? "separate buffers" : "chunked formats");
        return 1;
    }
    printf("capi demo ok: %d ranks, %d units, shard %lld, flat %lld, %d steps, bit-exact, "
           "separate buffers and chunked formats\n",
           N_RANKS, N_UNITS, (long long)S, (long long)P, STEPS);
    return 0;
}
