// Host side of libzeroshard: layout planning, queries and error reporting.
//
// The layout is the FSDP1-style flat parameter ("DP, ZeRO-1/2/3, FSDP"
// notes, follow-up "FSDP2 vs FSDP1": flatten a group of parameters,
// concatenate, then shard), cut into N equal slices per unit so that each
// rank keeps and updates only its own 1/N (same notes, concepts "ZeRO-1 / 2
// / 3").  Each unit is zero-padded at its tail to a multiple of N.  Under
// DDP nothing is sharded ("Data Parallel, ZeRO and FSDP", plain DDP).
// zero_shard_init_rows pads and slices in whole dim-0 rows instead: FSDP2
// shards each parameter on its own along dim 0 (same notes, "FSDP2 vs
// FSDP1"), with torch.chunk row counts.  zero_layout_chunk_state copies a
// layout and records a chunked format for its fp32 master, m and v (one
// buffer, chunks of E master, E m, E v values): a memory layout the notes
// leave open ("Model states" fixes only what is kept per parameter).
#include <cstdarg>
#include <cstdio>
#include <new>

#include "internal.h"

namespace zs {

static thread_local std::string g_last_error;

zero_status fail(zero_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

void clear_error() { g_last_error.clear(); }

zero_status check_range(const zero_layout *L, int32_t unit_begin, int32_t unit_end)
{
    if (!L)
        return fail(ZERO_ERR_INVALID_ARG, "layout is NULL");
    if (unit_begin < 0 || unit_end > L->n_units || unit_begin > unit_end)
        return fail(ZERO_ERR_INVALID_ARG, "unit range [%d, %d) outside [0, %d)",
                    unit_begin, unit_end, L->n_units);
    return ZERO_OK;
}

zero_status check_state(const zero_layout *L, const float *master, const float *m,
                        const float *v)
{
    const int64_t E = L->state_chunk;
    if (E > 0 && master && (m != master + E || v != master + 2 * E))
        return fail(ZERO_ERR_INVALID_ARG, "chunked state (chunk %lld): m and v must be master + "
                    "chunk and master + 2 chunk, master the start of the state buffer",
                    (long long)E);
    return ZERO_OK;
}

}  // namespace zs

extern "C" {

// Shared planner: unit u has rows[u] rows of cols[u] elements; padding and
// slicing are in whole rows (cols = 1 gives the element-granular layout).
static zero_status plan_layout(zero_layout **out, zero_strategy strategy, int32_t world_n,
                               int32_t rank, int32_t n_units, const int64_t *rows,
                               const int64_t *cols)
{
    using zs::fail;
    if (!out)
        return fail(ZERO_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (strategy < ZERO_DDP || strategy > ZERO_MEGATRON_DO)
        return fail(ZERO_ERR_INVALID_ARG, "unknown strategy %d", (int)strategy);
    if (world_n < 1)
        return fail(ZERO_ERR_INVALID_ARG, "world_n must be >= 1 (got %d)", world_n);
    if (rank < 0 || rank >= world_n)
        return fail(ZERO_ERR_INVALID_ARG, "rank %d outside [0, %d)", rank, world_n);
    if (n_units < 1 || !rows)
        return fail(ZERO_ERR_INVALID_ARG, "need at least one unit and a size array");

    zero_layout *L = new (std::nothrow) zero_layout;
    if (!L)
        return fail(ZERO_ERR_OOM, "host allocation of the layout failed");
    try {
        const bool sharded = strategy != ZERO_DDP;
        L->strategy = strategy;
        L->world_n = world_n;
        L->rank = sharded ? rank : 0;
        L->parts = sharded ? world_n : 1;
        L->n_units = n_units;
        L->numel.resize(n_units);
        L->cols.resize(n_units);
        L->padded.resize(n_units);
        L->slice.resize(n_units);
        L->flat_off.resize(n_units + 1);
        L->shard_off.resize(n_units + 1);
        const int64_t P = L->parts;
        const int64_t kMax = INT64_MAX / 4;  // keeps every byte offset representable
        int64_t F = 0, R = 0;
        for (int32_t u = 0; u < n_units; ++u) {
            const int64_t nr = rows[u];
            const int64_t c = cols ? cols[u] : 1;
            if (nr < 0 || c < 1) {
                delete L;
                return fail(ZERO_ERR_INVALID_ARG, "unit %d has negative size or cols < 1", u);
            }
            if (nr > kMax - P || c > kMax / (nr + P) || F > kMax - (nr + P) * c) {
                delete L;
                return fail(ZERO_ERR_INVALID_ARG, "layout size overflows at unit %d", u);
            }
            const int64_t chunk_rows = (nr + P - 1) / P;
            L->numel[u] = nr * c;
            L->cols[u] = c;
            L->slice[u] = chunk_rows * c;
            L->padded[u] = chunk_rows * c * P;
            L->flat_off[u] = F;
            L->shard_off[u] = R;
            F += L->padded[u];
            R += L->slice[u];
        }
        L->flat_off[n_units] = F;
        L->shard_off[n_units] = R;
    } catch (const std::bad_alloc &) {
        delete L;
        return fail(ZERO_ERR_OOM, "host allocation of the unit tables failed");
    }
    *out = L;
    zs::clear_error();
    return ZERO_OK;
}

zero_status zero_shard_init(zero_layout **out, zero_strategy strategy, int32_t world_n,
                            int32_t rank, int32_t n_units, const int64_t *unit_numel)
{
    return plan_layout(out, strategy, world_n, rank, n_units, unit_numel, nullptr);
}

zero_status zero_shard_init_rows(zero_layout **out, zero_strategy strategy, int32_t world_n,
                                 int32_t rank, int32_t n_units, const int64_t *unit_rows,
                                 const int64_t *unit_cols)
{
    if (!unit_cols)
        return zs::fail(ZERO_ERR_INVALID_ARG, "unit_cols is NULL");
    return plan_layout(out, strategy, world_n, rank, n_units, unit_rows, unit_cols);
}

void zero_shard_destroy(zero_layout *layout) { delete layout; }

zero_status zero_layout_chunk_state(const zero_layout *L, int64_t chunk, zero_layout **out)
{
    using zs::fail;
    if (!out)
        return fail(ZERO_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!L)
        return fail(ZERO_ERR_INVALID_ARG, "layout is NULL");
    if (chunk != 0 && (chunk < ZERO_STATE_CHUNK_MIN || chunk > ZERO_STATE_CHUNK_MAX ||
                       (chunk & (chunk - 1)) != 0))
        return fail(ZERO_ERR_INVALID_ARG, "state chunk must be 0 or a power of two in [%d, %d] "
                    "(got %lld)", ZERO_STATE_CHUNK_MIN, ZERO_STATE_CHUNK_MAX, (long long)chunk);
    zero_layout *C = nullptr;
    try {
        C = new zero_layout(*L);
    } catch (const std::bad_alloc &) {
        delete C;
        return fail(ZERO_ERR_OOM, "host allocation of the layout copy failed");
    }
    C->state_chunk = chunk;
    *out = C;
    zs::clear_error();
    return ZERO_OK;
}

zero_status zero_layout_state(const zero_layout *L, int64_t *chunk, int64_t *state_len)
{
    if (!L)
        return zs::fail(ZERO_ERR_INVALID_ARG, "layout is NULL");
    const int64_t E = L->state_chunk, S = L->shard_off[L->n_units];
    if (chunk)
        *chunk = E;
    if (state_len) {
        if (E == 0) {
            *state_len = S;
        } else {
            const int64_t n_chunks = (S + E - 1) / E;
            if (n_chunks > INT64_MAX / 4 / (3 * E))
                return zs::fail(ZERO_ERR_INVALID_ARG, "state length overflows");
            *state_len = n_chunks * 3 * E;
        }
    }
    zs::clear_error();
    return ZERO_OK;
}

zero_status zero_layout_info(const zero_layout *L, int64_t *flat_len, int64_t *shard_len,
                             int32_t *n_units, int32_t *world_n, int32_t *rank,
                             int32_t *strategy)
{
    if (!L)
        return zs::fail(ZERO_ERR_INVALID_ARG, "layout is NULL");
    if (flat_len) *flat_len = L->flat_off[L->n_units];
    if (shard_len) *shard_len = L->shard_off[L->n_units];
    if (n_units) *n_units = L->n_units;
    if (world_n) *world_n = L->world_n;
    if (rank) *rank = L->rank;
    if (strategy) *strategy = L->strategy;
    return ZERO_OK;
}

zero_status zero_layout_query(const zero_layout *L, int32_t unit, int64_t *numel,
                              int64_t *padded_len, int64_t *flat_off, int64_t *shard_len,
                              int64_t *shard_off, int64_t *rank_flat_off)
{
    if (!L)
        return zs::fail(ZERO_ERR_INVALID_ARG, "layout is NULL");
    if (unit < 0 || unit >= L->n_units)
        return zs::fail(ZERO_ERR_INVALID_ARG, "unit %d outside [0, %d)", unit, L->n_units);
    if (numel) *numel = L->numel[unit];
    if (padded_len) *padded_len = L->padded[unit];
    if (flat_off) *flat_off = L->flat_off[unit];
    if (shard_len) *shard_len = L->slice[unit];
    if (shard_off) *shard_off = L->shard_off[unit];
    if (rank_flat_off) *rank_flat_off = L->flat_off[unit] + (int64_t)L->rank * L->slice[unit];
    return ZERO_OK;
}

zero_status zero_layout_rows(const zero_layout *L, int32_t unit, int64_t *cols,
                             int64_t *first_row, int64_t *row_count)
{
    if (!L)
        return zs::fail(ZERO_ERR_INVALID_ARG, "layout is NULL");
    if (unit < 0 || unit >= L->n_units)
        return zs::fail(ZERO_ERR_INVALID_ARG, "unit %d outside [0, %d)", unit, L->n_units);
    const int64_t c = L->cols[unit];
    const int64_t rows = L->numel[unit] / c;
    const int64_t chunk = L->slice[unit] / c;
    int64_t first = (int64_t)L->rank * chunk;
    first = first < rows ? first : rows;
    const int64_t left = rows - first;
    if (cols) *cols = c;
    if (first_row) *first_row = first;
    if (row_count) *row_count = left < chunk ? left : chunk;
    return ZERO_OK;
}

const char *zero_status_str(zero_status s)
{
    switch (s) {
    case ZERO_OK: return "ok";
    case ZERO_ERR_INVALID_ARG: return "invalid argument";
    case ZERO_ERR_ALIGNMENT: return "misaligned pointer";
    case ZERO_ERR_OOM: return "out of host memory";
    case ZERO_ERR_HIP: return "HIP runtime error";
    case ZERO_ERR_UNSUPPORTED: return "unsupported";
    }
    return "unknown status";
}

const char *zero_last_error(void) { return zs::g_last_error.c_str(); }

}  // extern "C"
