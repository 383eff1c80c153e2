// FSDP per-unit sweep: a two-stream scheduler over the library's own entry
// points.  Unit u's reduce + Adam + cast runs on the step stream; its
// gather runs on the gather stream once that step is done (an all-gather
// carries every rank's updated shard), while the step stream moves on to
// unit u + 1.  An in-flight cap -- the analogue of FSDP's
// limit_all_gathers ("DP, ZeRO-1/2/3, FSDP" notes, follow-ups on FSDP's
// separate all-gather stream and prefetch) -- makes the step of unit u wait
// for the gather of unit u - cap.
//
// Events are created per call (no device memory) and destroyed before
// returning; destroying a recorded event is safe while it is pending.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "internal.h"

namespace {

struct Events {
    std::vector<hipEvent_t> ev;
    ~Events()
    {
        for (hipEvent_t e : ev)
            (void)hipEventDestroy(e);
    }
    zero_status make(size_t n)
    {
        ev.reserve(n);
        for (size_t i = 0; i < n; ++i) {
            hipEvent_t e = nullptr;
            const hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableTiming);
            if (err != hipSuccess)
                return zs::fail(ZERO_ERR_HIP, "hipEventCreateWithFlags: %s", hipGetErrorString(err));
            ev.push_back(e);
        }
        return ZERO_OK;
    }
};

zero_status hip_check(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return zs::fail(ZERO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ZERO_OK;
}


// The schedule shared by both sweeps: validation of the per-unit buffers,
// then per unit step_unit(u, grads, so, unit_full) on the step stream and
// its gather on the gather stream.  `finish` runs on the step stream after
// the last unit's step.
template <typename StepUnit, typename Finish>
zero_status sweep(const zero_layout *L, int32_t ub, int32_t ue, int32_t grad_dtype,
                  int32_t grad_chunk, const zero_unit_io *io, float *master, float *m, float *v,
                  int32_t max_inflight, void *step_stream, void *gather_stream,
                  StepUnit step_unit, Finish finish)
{
    zero_status st = zs::check_range(L, ub, ue);
    if (st != ZERO_OK)
        return st;
    if (!io && ue > ub)
        return zs::fail(ZERO_ERR_INVALID_ARG, "io is required");
    if (max_inflight < 0)
        return zs::fail(ZERO_ERR_INVALID_ARG, "max_inflight must be >= 0");
    if (grad_dtype != ZERO_BF16 && grad_dtype != ZERO_FP32)
        return zs::fail(ZERO_ERR_INVALID_ARG, "unknown gradient dtype %d", grad_dtype);
    if (!master || !m || !v)
        return zs::fail(ZERO_ERR_INVALID_ARG, "master, m and v are required");
    if (reinterpret_cast<uintptr_t>(master) % 4 || reinterpret_cast<uintptr_t>(m) % 4 ||
        reinterpret_cast<uintptr_t>(v) % 4)
        return zs::fail(ZERO_ERR_ALIGNMENT, "misaligned state buffer");
    if ((st = zs::check_state(L, master, m, v)) != ZERO_OK)
        return st;
    if (L->world_n > ZERO_MAX_RANKS_PER_CALL)
        return zs::fail(ZERO_ERR_UNSUPPORTED, "at most %d rank buffers per call (got %d)",
                        ZERO_MAX_RANKS_PER_CALL, L->world_n);
    const int32_t n = L->world_n;
    // validate every unit's buffers before anything is launched
    for (int32_t u = ub; u < ue; ++u) {
        const zero_unit_io &x = io[u - ub];
        if (!x.rank_grads || !x.peer_shards || !x.unit_full)
            return zs::fail(ZERO_ERR_INVALID_ARG, "unit %d: rank_grads, peer_shards and "
                            "unit_full are required", u);
        const uintptr_t elem = grad_dtype == ZERO_BF16 ? 2 : 4;
        for (int32_t q = 0; q < n; ++q) {
            if (!x.rank_grads[q])
                return zs::fail(ZERO_ERR_INVALID_ARG, "unit %d: gradient buffer of rank %d is "
                                "NULL (missing replica)", u, q);
            if (reinterpret_cast<uintptr_t>(x.rank_grads[q]) % elem)
                return zs::fail(ZERO_ERR_ALIGNMENT, "unit %d: gradient buffer of rank %d is "
                                "misaligned", u, q);
        }
        for (int32_t q = 0; q < L->parts; ++q)
            if (reinterpret_cast<uintptr_t>(x.peer_shards[q]) % 2)
                return zs::fail(ZERO_ERR_ALIGNMENT, "unit %d: peer shard %d is misaligned", u, q);
        if (reinterpret_cast<uintptr_t>(x.unit_full) % 2)
            return zs::fail(ZERO_ERR_ALIGNMENT, "unit %d: unit_full is misaligned", u);
        if (L->parts > 1 && x.peer_shards[L->rank])
            return zs::fail(ZERO_ERR_INVALID_ARG, "unit %d: this rank's own peer_shards entry "
                            "must be NULL (the step writes that slice)", u);
        const zero_grads g{x.rank_grads, nullptr, n, grad_dtype, ZERO_INDEX_SHARD, grad_chunk};
        if ((st = zs::check_grads(L, &g)) != ZERO_OK) {
            const std::string why = zero_last_error();
            return zs::fail(st, "unit %d: %s", u, why.c_str());
        }
    }
    const hipStream_t ss = static_cast<hipStream_t>(step_stream);
    const hipStream_t gs = static_cast<hipStream_t>(gather_stream);
    const bool two = ss != gs;
    const size_t U = (size_t)(ue - ub);
    Events stepped, gathered;
    if (two && ((st = stepped.make(U)) != ZERO_OK || (st = gathered.make(U)) != ZERO_OK))
        return st;
    for (int32_t u = ub; u < ue; ++u) {
        const size_t k = (size_t)(u - ub);
        const zero_unit_io &x = io[k];
        if (two && max_inflight > 0 && k >= (size_t)max_inflight &&
            (st = hip_check(hipStreamWaitEvent(ss, gathered.ev[k - max_inflight], 0),
                            "hipStreamWaitEvent")) != ZERO_OK)
            return st;
        const zero_grads g{x.rank_grads, nullptr, n, grad_dtype, ZERO_INDEX_SHARD, grad_chunk};
        // three state arrays: the unit's step gets them from the unit's
        // first element; a chunked state is always passed from its start
        const int64_t so = L->state_chunk ? 0 : L->shard_off[u] - L->shard_off[ub];
        if ((st = step_unit(u, g, so, x.unit_full)) != ZERO_OK)
            return st;
        if (two) {
            if ((st = hip_check(hipEventRecord(stepped.ev[k], ss), "hipEventRecord")) != ZERO_OK ||
                (st = hip_check(hipStreamWaitEvent(gs, stepped.ev[k], 0), "hipStreamWaitEvent")) !=
                    ZERO_OK)
                return st;
        }
        st = zero_gather_params(L, u, u + 1, x.peer_shards, L->parts, x.unit_full, gather_stream);
        if (st != ZERO_OK)
            return st;
        if (two && (st = hip_check(hipEventRecord(gathered.ev[k], gs), "hipEventRecord")) != ZERO_OK)
            return st;
    }
    if ((st = finish()) != ZERO_OK)
        return st;
    if (two && U > 0)
        return hip_check(hipStreamWaitEvent(ss, gathered.ev[U - 1], 0), "hipStreamWaitEvent");
    return ZERO_OK;
}

}  // namespace

extern "C" zero_status zero_fsdp_sweep(const zero_layout *L, int32_t ub, int32_t ue,
                                       const zero_adam_cfg *cfg, int32_t grad_dtype,
                                       int32_t grad_chunk, const zero_unit_io *io,
                                       float *master, float *m, float *v,
                                       int32_t max_inflight, void *step_stream,
                                       void *gather_stream)
{
    if (!cfg)
        return zs::fail(ZERO_ERR_INVALID_ARG, "cfg is required");
    return sweep(L, ub, ue, grad_dtype, grad_chunk, io, master, m, v, max_inflight, step_stream,
                 gather_stream,
                 [&](int32_t u, const zero_grads &g, int64_t so, uint16_t *full) {
                     return zero_adam_step(L, u, u + 1, cfg, nullptr, ZERO_INDEX_SHARD, nullptr,
                                           &g, master + so, m + so, v + so, full,
                                           ZERO_INDEX_FULL, step_stream);
                 },
                 [] { return ZERO_OK; });
}

extern "C" zero_status zero_fsdp_sweep_table(const zero_layout *L, int32_t ub, int32_t ue,
                                             const zero_adam_table_entry *table,
                                             int64_t n_entries, int64_t *step_counter,
                                             int32_t grad_dtype, int32_t grad_chunk,
                                             const zero_unit_io *io,
                                             float *master, float *m, float *v,
                                             int32_t max_inflight, void *step_stream,
                                             void *gather_stream)
{
    if (!table || !step_counter || n_entries < 1)
        return zs::fail(ZERO_ERR_INVALID_ARG, "table, step_counter and n_entries >= 1 are "
                        "required");
    if (reinterpret_cast<uintptr_t>(table) % 4 || reinterpret_cast<uintptr_t>(step_counter) % 8)
        return zs::fail(ZERO_ERR_ALIGNMENT, "misaligned step table or counter");
    return sweep(L, ub, ue, grad_dtype, grad_chunk, io, master, m, v, max_inflight, step_stream,
                 gather_stream,
                 [&](int32_t u, const zero_grads &g, int64_t so, uint16_t *full) {
                     return zero_adam_step_table(L, u, u + 1, table, n_entries, step_counter,
                                                 nullptr, ZERO_INDEX_SHARD, nullptr, &g,
                                                 master + so, m + so, v + so, full,
                                                 ZERO_INDEX_FULL, step_stream);
                 },
                 [&] { return zero_step_advance(step_counter, step_stream); });
}
