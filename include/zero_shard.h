/*
 * zero_shard.h -- C ABI of the per-rank sharded mixed-precision optimizer
 * step for one AMD Instinct MI355X (gfx950) GPU.
 *
 * One data-parallel rank's step, seen from its own GPU, with the N ranks'
 * gradient buffers resident in this GPU's memory:
 *   reduce    the N ranks' gradients into this rank's 1/N slice, in fp32,
 *             divided by N -- the arithmetic of a reduce-scatter
 *             ("DP, ZeRO-1/2/3, FSDP" notes, concepts "reduce-scatter and
 *             all-gather"; "Data Parallel, ZeRO and FSDP", plain DDP);
 *   adam      Adam / AdamW on the slice's fp32 master, m and v (the 12 bytes
 *             per parameter that ZeRO shards; "DP, ZeRO-1/2/3, FSDP" notes,
 *             concepts "Model states" and "ZeRO-1 / 2 / 3"); the update
 *             equations are Kingma & Ba (2015) Algorithm 1, with
 *             Loshchilov & Hutter (2019) decoupled decay for AdamW;
 *   cast      the new master rounded to bf16 (round to nearest even) and
 *             stored at the rank's offsets of the flat parameter buffer;
 *   gather    the other ranks' bf16 slices packed into the full flat buffer
 *             -- the data movement of an all-gather.
 * Plus the DDP variant (no sharding: every replica averages and updates the
 * whole buffer) and the Megatron distributed-optimizer pieces (fp32 main
 * gradient accumulation; fp32 gradients reduced; "DP, ZeRO-1/2/3, FSDP"
 * notes, worked example, note under the Megatron row).
 *
 * LAYOUT (FSDP1-style flat parameter; "DP, ZeRO-1/2/3, FSDP" notes,
 * follow-up "FSDP2 vs FSDP1"): the parameters form units u = 0..U-1 of n_u
 * elements (a layer, or a gradient bucket).  Each unit is padded with zeros
 * at its tail to L_u = ceil(n_u / N) * N and the units are concatenated:
 *     F_u = sum_{j<u} L_j          (flat offset of unit u)
 *     s_u = L_u / N                (each rank's slice of unit u)
 *     R_u = sum_{j<u} s_j          (offset of unit u in a rank's shard)
 * Rank r owns flat elements [F_u + r*s_u, F_u + (r+1)*s_u) of every unit.
 * Under ZERO_DDP nothing is sharded: s_u = L_u = n_u and every rank "owns"
 * the whole buffer.
 *
 * RANGES AND INDEXING.  Every compute call covers a contiguous range of
 * units [unit_begin, unit_end) and every buffer pointer passed to it
 * addresses the first element of that range:
 *   ZERO_INDEX_FULL  buffer over the flat layout: element j of rank q's
 *                    slice of unit u is at (F_u - F_begin) + q*s_u + j;
 *   ZERO_INDEX_SHARD buffer over one rank's shard: element j of unit u is at
 *                    (R_u - R_begin) + j.
 * With unit_begin = 0 these are plain whole-buffer offsets; with a single
 * unit they address per-unit buffers (FSDP's gather / free per unit).
 * fp32 master, m and v are always shard-indexed: three such arrays, or, on a
 * layout made by zero_layout_chunk_state, one buffer over the whole shard
 * addressed from its start whatever the range.
 *
 * CONVENTIONS.
 *   - Lengths are element counts (int64_t).  Data pointers are DEVICE
 *     pointers owned by the caller; pointer ARRAYS (rank lists) and config
 *     structs are HOST memory, read during the call only.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every compute call
 *     only enqueues work on it and never synchronises.
 *   - Arguments are validated on the host before anything is launched; on
 *     any error nothing is launched and no buffer is touched.  Launch
 *     failures return ZERO_ERR_HIP.  zero_last_error() returns a text
 *     description of the last error on the calling thread.
 *   - The library allocates no device memory; a layout is host memory only
 *     and is immutable after init (safe to share between threads).
 *   - Every compute call only launches kernels (no memset, no copy, no
 *     allocation), so it may be captured into a HIP graph and replayed.
 *     zero_fsdp_sweep forks its gather stream from the step stream through
 *     events and joins it back before returning, so a capture of the step
 *     stream takes in both.  A graph keeps the argument values of its
 *     capture, the Adam step number included.
 *   - Calls that write disjoint buffers may run concurrently on different
 *     streams.  An fp32 buffer pointer must be 4-byte aligned and a bf16
 *     one 2-byte aligned; 16-byte aligned buffers with slice offsets that are
 *     multiples of 8 take the 128-bit vector path, others a scalar path with
 *     identical results.
 *   - At most ZERO_MAX_RANKS_PER_CALL rank buffers per reduce call.
 *   - Arithmetic: fp32, one IEEE-754 rounding per operation, no fused
 *     multiply-add; the N ranks are summed in ascending rank order from +0
 *     and the sum divided by N; results do not depend on the launch shape.
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZERO_MAX_RANKS_PER_CALL 64

typedef enum zero_status {
    ZERO_OK = 0,
    ZERO_ERR_INVALID_ARG = 1, /* null / out-of-range / inconsistent argument */
    ZERO_ERR_ALIGNMENT = 2,   /* pointer not aligned to its element size     */
    ZERO_ERR_OOM = 3,         /* host allocation failed                       */
    ZERO_ERR_HIP = 4,         /* a HIP runtime call or launch failed          */
    ZERO_ERR_UNSUPPORTED = 5  /* valid request outside this library's limits  */
} zero_status;

/* Who holds what ("DP, ZeRO-1/2/3, FSDP" notes, figure 1 and worked example;
   "Data Parallel, ZeRO and FSDP", ZeRO/FSDP table).  Only ZERO_DDP changes
   the layout (unsharded); the others record the caller's strategy. */
typedef enum zero_strategy {
    ZERO_DDP = 0,
    ZERO_STAGE1 = 1,
    ZERO_STAGE2 = 2,
    ZERO_STAGE3 = 3,
    ZERO_FSDP = 4,
    ZERO_MEGATRON_DO = 5
} zero_strategy;

typedef enum zero_dtype { ZERO_BF16 = 0, ZERO_FP32 = 1 } zero_dtype;

typedef enum zero_index { ZERO_INDEX_FULL = 0, ZERO_INDEX_SHARD = 1 } zero_index;

typedef struct zero_layout zero_layout;

/* The N ranks' gradient buffers for one call, all of one dtype (bf16 as raw
   uint16 bit patterns, or fp32).

   Chunked gradients (chunk = E > 0): the shard-indexed contributions to
   this rank's part of the call's range sit in one receive buffer R of
   ceil(S/E) rows, each row holding E elements of rank 0, then E of rank 1,
   ..., then E of rank N-1 (S = the range's shard length).  Rank q's
   gradient for element i of the range (counted from its first element, as
   for every shard-indexed buffer) is at R + (i / E) N E + q E + i % E, and
   ptrs[q] must be R + qE elements (ZERO_ERR_INVALID_ARG otherwise; at
   least one rank shard-indexed).  A full-indexed rank -- a rank's own
   main gradient, as in the Megatron distributed optimizer -- keeps its own
   buffer at ptrs[q]; its slot in R is never read.  A per-unit call
   therefore takes a per-unit receive buffer.
   The same bytes and sums as N separate buffers, read from one region
   instead of N: it is the receive buffer a rank would let its peers fill
   in a reduce-scatter.  On one MI355X the 7B / N = 8 fused step (state
   chunked either way) takes 0.956 x the time of eight separate buffers
   with E = 16384 (0.934-1.014 over six buffer placements; 2048-32768 all
   within 0.4 % of it).  E is a power of two in [ZERO_STATE_CHUNK_MIN,
   ZERO_STATE_CHUNK_MAX]. */
#define ZERO_GRAD_CHUNK_DEFAULT 16384 /* the measured best on MI355X */
typedef struct zero_grads {
    const void *const *ptrs; /* host array of n device pointers, rank order;
                                a NULL entry is an error (missing replica)  */
    const uint8_t *index;    /* host array of n zero_index values, or NULL
                                for all `index_all`                          */
    int32_t n;               /* must equal the layout's world_n             */
    int32_t dtype;           /* zero_dtype                                  */
    int32_t index_all;       /* zero_index used when `index` is NULL        */
    int32_t chunk;           /* 0: one buffer per rank; E: chunked (above)  */
} zero_grads;

/* Adam / AdamW hyper-parameters of one step.  The step scalars 1 - beta1,
   1 - beta2, 1 - beta1^t, 1 - beta2^t and 1 - lr*wd are evaluated in fp64
   from these fp32 values and rounded once to fp32. */
typedef struct zero_adam_cfg {
    float lr;
    float beta1;        /* in [0, 1) */
    float beta2;        /* in [0, 1) */
    float eps;          /* >= 0 */
    float weight_decay; /* >= 0; 0 disables both decay forms */
    int32_t decoupled;  /* 1: AdamW, p *= 1 - lr*wd; 0: L2, g += wd*p */
    int64_t step;       /* t >= 1, supplied by the caller every call */
} zero_adam_cfg;

/* ------------------------------------------------------------ layout -- */

/* Plan the layout of one rank: `n_units` units of unpadded sizes
   `unit_numel` (host array, each >= 0, at least one unit), `world_n` >= 1
   ranks, this rank `rank` in [0, world_n).  Host memory only; no HIP call.
   *out receives a layout to free with zero_shard_destroy.
   Source: "DP, ZeRO-1/2/3, FSDP" notes, concepts "ZeRO-1 / 2 / 3" (the
   model states are cut into N parts by data-parallel rank; each rank keeps
   and updates only its part) and "FSDP" (the model is split into units),
   and the follow-up "FSDP2 vs FSDP1" (FSDP1 flattens and concatenates a
   unit's parameters into one flat buffer and shards that); "Data Parallel,
   ZeRO and FSDP", section "ZeRO and FSDP".  The padding of each unit to a
   multiple of N is this layout's reading (the pages do not say how an
   uneven unit is cut). */
zero_status zero_shard_init(zero_layout **out, zero_strategy strategy,
                            int32_t world_n, int32_t rank, int32_t n_units,
                            const int64_t *unit_numel);

/* FSDP2-style per-parameter dim-0 sharding ("DP, ZeRO-1/2/3, FSDP" notes,
   follow-up "FSDP2 vs FSDP1": every parameter sharded on its own along dim
   0, so a rank holds whole rows and its sharded state dict needs no
   gather).  Unit u is a parameter of unit_rows[u] x unit_cols[u] elements
   (row-major; unit_cols >= 1, unit_rows >= 0).  It is cut into chunks of
   c_u = ceil(rows / N) rows (the torch.chunk rule): rank r holds rows
   [r c_u, min((r+1) c_u, rows)), padded with zero rows to c_u rows, so
   s_u = c_u * cols and L_u = N * s_u.  Offsets F_u, R_u and every other
   call work exactly as for zero_shard_init. */
zero_status zero_shard_init_rows(zero_layout **out, zero_strategy strategy,
                                 int32_t world_n, int32_t rank,
                                 int32_t n_units, const int64_t *unit_rows,
                                 const int64_t *unit_cols);

void zero_shard_destroy(zero_layout *layout);

/* Whole-layout sizes: padded flat length sum L_u, this rank's shard length
   sum s_u.  Any output pointer may be NULL. */
zero_status zero_layout_info(const zero_layout *layout, int64_t *flat_len,
                             int64_t *shard_len, int32_t *n_units,
                             int32_t *world_n, int32_t *rank,
                             int32_t *strategy);

/* Per-unit numbers (see LAYOUT): n_u, L_u, F_u, s_u, R_u and the rank's
   flat offset F_u + r*s_u.  Any output pointer may be NULL.  These are the
   offsets of the flat-buffer sharding that zero_shard_init plans (same
   source): where unit u sits in the flat buffer, where its slice sits in a
   rank's shard, and which flat elements this rank owns. */
zero_status zero_layout_query(const zero_layout *layout, int32_t unit,
                              int64_t *numel, int64_t *padded_len,
                              int64_t *flat_off, int64_t *shard_len,
                              int64_t *shard_off, int64_t *rank_flat_off);

/* The rows of unit u this rank really holds (the rest of its slice is
   padding): *cols (1 for element-granular layouts), *first_row and
   *row_count (0 when this rank's chunk lies past the end).  For an
   element-granular layout rows are elements.  Any output may be NULL. */
zero_status zero_layout_rows(const zero_layout *layout, int32_t unit,
                             int64_t *cols, int64_t *first_row,
                             int64_t *row_count);

/* Chunked optimizer state.  The pages fix what a rank keeps per parameter
   (fp32 master, m and v: "DP, ZeRO-1/2/3, FSDP" notes, concepts "Model
   states"), not where it lies in memory.  *out receives a copy of `layout`
   (free it with zero_shard_destroy) whose master, m and v live in ONE
   buffer, interleaved in chunks of E = `chunk` elements: shard element i of
   master is at state[(i / E) * 3E + i % E], of m at E further, of v at 2E
   further.  Every call that takes master, m and v on such a layout expects
   master = state, m = state + E, v = state + 2E, where `state` is the start
   of a buffer of zero_layout_state(...) floats covering the whole shard,
   whatever the call's unit range (else ZERO_ERR_INVALID_ARG); the kernels
   add the range's shard offset themselves.  Results are bit-identical to
   the three-array layout; only addresses change.  The fused step reads and
   writes each chunk's three parts next to each other instead of in three
   arrays gigabytes apart, which HBM serves faster: on one MI355X the
   7B / N = 8 step kernel takes 0.938 x the three-array time with
   E = 8192 (0.910-0.982 over six buffer placements).  chunk = 0 gives the
   three-array format back; otherwise `chunk` is a power of two in
   [ZERO_STATE_CHUNK_MIN, ZERO_STATE_CHUNK_MAX]. */
#define ZERO_STATE_CHUNK_MIN 4
#define ZERO_STATE_CHUNK_MAX 16777216
#define ZERO_STATE_CHUNK_DEFAULT 8192 /* the measured best on MI355X */
zero_status zero_layout_chunk_state(const zero_layout *layout, int64_t chunk,
                                    zero_layout **out);

/* The layout's state format: *chunk = 0 (three arrays of shard_len floats,
   *state_len = shard_len) or E (one buffer of *state_len =
   ceil(shard_len / E) * 3E floats).  Either output may be NULL. */
zero_status zero_layout_state(const zero_layout *layout, int64_t *chunk,
                              int64_t *state_len);

/* ------------------------------------------------------------ reduce -- */

/* Reduce-scatter arithmetic: for every element of this rank's slices of
   units [unit_begin, unit_end),
       out[i] = (G_0[i] + G_1[i] + ... + G_{N-1}[i]) / N      (fp32)
   with G_q indexed as grads->index says.  `out` is fp32, indexed as
   `out_index` says: ZERO_INDEX_SHARD for this rank's reduce-scatter result,
   ZERO_INDEX_FULL to write this rank's slices into a full flat buffer (the
   N ranks' calls together then form the all-reduce).
   If `sumsq_partials` is non-NULL it receives exactly
   zero_reduce_partials_count(...) fp64 partial sums of out[i]^2 (each square
   exact in fp64; one partial per 1024-element tile of a unit slice, summed
   in a fixed order), for the global-norm clip; `n_partials` is the capacity
   of that buffer.
   Source: "DP, ZeRO-1/2/3, FSDP" notes, concepts "reduce-scatter and
   all-gather" (a reduce-scatter sums the ranks' buffers and leaves each
   rank 1/N of the result; with the all-gather it makes an all-reduce);
   "Data Parallel, ZeRO and FSDP", section "Plain data parallel (DDP)"
   (after the all-reduce every replica holds the mean gradient) and section
   "ZeRO and FSDP" (gradients are reduce-scattered so that each GPU keeps
   its shard).  Summing in ascending rank order is this library's reading. */
zero_status zero_reduce_shard(const zero_layout *layout, int32_t unit_begin,
                              int32_t unit_end, const zero_grads *grads,
                              float *out, int32_t out_index,
                              double *sumsq_partials,
                              int64_t n_partials, void *stream);

/* Number of fp64 partials zero_reduce_shard writes for a range: one per
   1024-element tile of every unit slice in the range (a fixed function of
   the range, independent of the device and of the launch width). */
int64_t zero_reduce_partials_count(const zero_layout *layout,
                                   int32_t unit_begin, int32_t unit_end);

/* Global gradient-norm clip coefficient.  Not on the pages: the
   GPT-2-small workload with a global-norm clip at 1.0 names it, and the
   reading taken is PyTorch's clip_grad_norm_:
   norm = sqrt(sum of the n partials in fp64, in
   a fixed order for a given n: strided per-thread sums, then a fixed tree),
   *coef_out = min(1, fp32(max_norm / (norm + 1e-6))).
   `partials`, `coef_out` (one float) and `norm_out` (one double, may be
   NULL) are device pointers.  n >= 1, max_norm > 0. */
zero_status zero_clip_coef(const double *partials, int64_t n, float max_norm,
                           float *coef_out, double *norm_out, void *stream);

/* ------------------------------------------------ no allocation -- */

/* Capacity of the library's static device buffer of sum-of-squares partials
   (4 MiB of fp64 per GPU, held until the process ends). */
#define ZERO_NOALLOC_MAX_PARTIALS 524288

/* For callers that cannot allocate device memory: code under HIP graph
   capture, tight serving loops, harnesses that forbid hipMalloc.  The
   two-pass clipped step of one range -- zero_reduce_shard into `grad_out`
   (fp32, shard-indexed) with sum-of-squares partials, zero_clip_coef over
   those partials (max_norm > 0), then zero_adam_step from `grad_out` scaled
   by the coefficient -- with the partials and the coefficient kept in a
   static device array of the library instead of caller buffers.  Results
   are those of that three-call sequence, bit for bit.  The norm is the
   norm of this call's range: the whole buffer under ZERO_DDP, this rank's
   shard otherwise (a global norm over several ranks needs every rank's
   partials: use the three calls).  `norm_out` (device double, may be NULL)
   receives the norm.  The range may need at most ZERO_NOALLOC_MAX_PARTIALS
   partials (zero_reduce_partials_count; 536,870,912 elements per rank),
   else ZERO_ERR_UNSUPPORTED.  The call allocates nothing and calls no
   allocating routine; every argument is checked on the host before the
   first HIP call.  Calls on one GPU share its array, so calls that overlap
   in time on one GPU (other streams, other host threads) race; calls in
   one stream order are safe, each overwriting what it uses before reading
   it. */
zero_status zero_adam_step_clip_noalloc(const zero_layout *layout, int32_t unit_begin,
                                        int32_t unit_end, const zero_adam_cfg *cfg,
                                        float max_norm, const zero_grads *grads,
                                        float *grad_out, float *master, float *m, float *v,
                                        uint16_t *param_out, int32_t param_index,
                                        double *norm_out, void *stream);

/* --------------------------------------------------------- Adam step -- */

/* Adam / AdamW on this rank's slices of units [unit_begin, unit_end), then
   bf16 rounding of the new master into `param_out`.
   Source: "DP, ZeRO-1/2/3, FSDP" notes, concepts "Model states" (bf16
   parameter and gradient, fp32 master, m and v: 12 of the 16 bytes per
   parameter) and "ZeRO-1 / 2 / 3" (each rank updates only its part); the
   update itself is Kingma & Ba (2015) Algorithm 1 and, for AdamW,
   Loshchilov & Hutter (2019), as the pages leave it to the optimizer.
   Gradient source, exactly one of:
     grad_fp32 != NULL: fp32 averaged gradient, indexed as `grad_index`
                        says: ZERO_INDEX_SHARD for a reduce-scatter result
                        (zero_reduce_shard on this layout), ZERO_INDEX_FULL
                        for an all-reduce result over this layout's whole
                        flat buffer (zero_reduce_shard of every rank's
                        layout with out_index = ZERO_INDEX_FULL -- ZeRO-1
                        implemented with all-reduce, "DP, ZeRO-1/2/3, FSDP"
                        notes, follow-up on the ZeRO-1 / ZeRO-2
                        communication gap); multiplied by *clip_coef (a
                        device float; NULL means 1);
     grads != NULL:     fused path -- the N ranks' buffers are reduced
                        (as zero_reduce_shard) in the same pass, so each
                        byte crosses HBM once.  clip_coef must be NULL.
   master, m, v: shard-indexed fp32, updated in place.
   param_out: bf16 (uint16) written at the rank's offsets; `param_index`
   says whether it is the full flat buffer (ZERO_INDEX_FULL: elements of
   the other ranks are not touched) or the rank's own shard buffer
   (ZERO_INDEX_SHARD, ZeRO-3 / FSDP). */
zero_status zero_adam_step(const zero_layout *layout, int32_t unit_begin,
                           int32_t unit_end, const zero_adam_cfg *cfg,
                           const float *grad_fp32, int32_t grad_index,
                           const float *clip_coef,
                           const zero_grads *grads, float *master, float *m,
                           float *v, uint16_t *param_out, int32_t param_index,
                           void *stream);

/* Step scalars read on the device, for graph replay.  A captured graph keeps
   the arguments of its capture, so zero_adam_step replayed from a graph
   would repeat one step number (and one learning rate).
   zero_adam_step_table instead reads the step's scalars when its kernels
   run, from entry (*step_counter - 1) of a table that the caller fills once
   on the host with zero_adam_table_fill and copies to the device.
   zero_step_advance increments the counter on the device.  A graph of
   [zero_adam_step_table, ..., zero_step_advance] then replays as steps 1,
   2, 3, ... with the arithmetic of zero_adam_step, bit for bit.
   The entry is the set of fp32 scalars of one step, each evaluated in fp64
   from that step's configuration and rounded once (as zero_adam_step). */
typedef struct zero_adam_table_entry {
    float lr, beta1, beta2, eps, weight_decay;
    float one_minus_beta1, one_minus_beta2;
    float bias1, bias2;  /* 1 - beta1^t, 1 - beta2^t of the entry's step t */
    float decay;         /* 1 - lr * weight_decay */
    int32_t has_decay;   /* weight_decay != 0 */
    int32_t decoupled;
} zero_adam_table_entry;

/* host_out[k] = the step scalars of cfgs[k], k < n (host arrays; each cfg
   validated as in zero_adam_step).  cfgs[k].step is the t of entry k,
   normally k + 1; lr may change from entry to entry (a schedule). */
zero_status zero_adam_table_fill(const zero_adam_cfg *cfgs, int64_t n,
                                 zero_adam_table_entry *host_out);

/* zero_adam_step with the scalars of table[*step_counter - 1].  `table` is
   a device array of n_entries >= 1 entries (4-byte aligned), `step_counter`
   a device int64 (8-byte aligned), both read when the kernels run; a
   counter outside [1, n_entries] leaves every buffer untouched.  The other
   arguments, and the host-side errors, are those of zero_adam_step. */
zero_status zero_adam_step_table(const zero_layout *layout, int32_t unit_begin,
                                 int32_t unit_end, const zero_adam_table_entry *table,
                                 int64_t n_entries, const int64_t *step_counter,
                                 const float *grad_fp32, int32_t grad_index,
                                 const float *clip_coef, const zero_grads *grads,
                                 float *master, float *m, float *v, uint16_t *param_out,
                                 int32_t param_index, void *stream);

/* *step_counter += 1 on the device, in stream order (device int64,
   8-byte aligned). */
zero_status zero_step_advance(int64_t *step_counter, void *stream);

/* ------------------------------------------------------------ gather -- */

/* All-gather data movement (source: "DP, ZeRO-1/2/3, FSDP" notes, concepts
   "reduce-scatter and all-gather": an all-gather puts the ranks' 1/N
   slices back together into the whole; "Data Parallel, ZeRO and FSDP",
   section "ZeRO and FSDP": a layer's parameter shards are all-gathered
   before it runs): for every rank q < n with shards[q] != NULL
   and every element j of rank q's slice of unit u in the range,
       param_full[(F_u - F_begin) + q*s_u + j] = shards[q][(R_u - R_begin) + j]
   Bit copies.  `shards` is a host array of n = world_n device pointers
   (NULL entries are skipped -- typically this rank's own, already written by
   zero_adam_step); param_full is the full flat bf16 buffer of the range. */
zero_status zero_gather_params(const zero_layout *layout, int32_t unit_begin,
                               int32_t unit_end, const uint16_t *const *shards,
                               int32_t n, uint16_t *param_full, void *stream);

/* ------------------------------------------------------ FSDP sweep -- */

/* One unit's buffers for zero_fsdp_sweep. */
typedef struct zero_unit_io {
    const void *const *rank_grads;      /* host array of world_n device pointers:
                                           this unit's rank gradients, each
                                           indexed over this rank's slice of the
                                           unit (s_u elements, unit-local); or,
                                           with grad_chunk > 0, the pointers of
                                           this unit's chunked receive buffer
                                           (zero_grads.chunk)                  */
    const uint16_t *const *peer_shards; /* host array of world_n device pointers
                                           (s_u bf16 each) gathered into the
                                           unit buffer; NULL entries skipped,
                                           this rank's own entry must be NULL  */
    uint16_t *unit_full;                /* device, L_u bf16: the unit's full
                                           flat parameters                     */
} zero_unit_io;

/* The FSDP per-unit sweep as a two-stream pipeline ("DP, ZeRO-1/2/3, FSDP"
   notes, follow-up on how FSDP hides communication: the all-gather runs on
   its own stream, the next unit's gather is prefetched, and
   limit_all_gathers bounds how many gathered units exist at once).
   For every unit u in [unit_begin, unit_end), in order:
     on step_stream:   the fused reduce of io[u].rank_grads (grad_dtype) +
                       Adam + bf16 of this rank's slice into io[u].unit_full
                       (zero_adam_step on the single unit; master, m and v
                       are shard-indexed from unit_begin, as everywhere, or
                       a chunked state from its start);
     on gather_stream: after that step, zero_gather_params of
                       io[u].peer_shards into io[u].unit_full (an all-gather
                       carries every rank's updated shard, so it follows the
                       step of its unit).
   max_inflight caps the pipeline: the step of unit u waits until the
   gather of unit u - max_inflight has finished.  1 makes the sweep
   sequential, 2 double-buffers (the step of unit u+1 overlaps the gather of
   unit u), 0 means no cap.  When the call's work completes on step_stream,
   every gather has completed too (step_stream waits for the last one).
   gather_stream may equal step_stream (sequential).  Results are identical
   to per-unit zero_adam_step + zero_gather_params calls.  Host-side errors
   launch nothing; a HIP error part-way returns ZERO_ERR_HIP with the units
   before it enqueued.  `io` is a host array of (unit_end - unit_begin)
   entries.  grad_chunk = 0 takes each unit's rank gradients as world_n
   buffers; E > 0 as one chunked receive buffer per unit, as
   zero_grads.chunk describes, checked for every unit before anything is
   launched. */
zero_status zero_fsdp_sweep(const zero_layout *layout, int32_t unit_begin,
                            int32_t unit_end, const zero_adam_cfg *cfg,
                            int32_t grad_dtype, int32_t grad_chunk,
                            const zero_unit_io *io,
                            float *master, float *m, float *v,
                            int32_t max_inflight, void *step_stream,
                            void *gather_stream);

/* zero_fsdp_sweep with each unit's step as zero_adam_step_table (scalars of
   table[*step_counter - 1], read on the device), then *step_counter += 1 on
   step_stream after the last unit's step: a graph captured from one call
   replays as the sweeps of steps 1, 2, 3, ... .  Arguments and errors
   otherwise as zero_fsdp_sweep and zero_adam_step_table. */
zero_status zero_fsdp_sweep_table(const zero_layout *layout, int32_t unit_begin,
                                  int32_t unit_end, const zero_adam_table_entry *table,
                                  int64_t n_entries, int64_t *step_counter,
                                  int32_t grad_dtype, int32_t grad_chunk,
                                  const zero_unit_io *io,
                                  float *master, float *m, float *v,
                                  int32_t max_inflight, void *step_stream,
                                  void *gather_stream);

/* ------------------------------------------------------- accumulation -- */

/* Megatron-style fp32 main-gradient accumulation of one micro-batch:
   main_grad[i] = main_grad[i] + float(micro_bf16[i]) for i < n.
   Source: "DP, ZeRO-1/2/3, FSDP" notes, worked example "7B, N = 8", the
   note under the Megatron distributed-optimizer row (the gradient is kept
   and accumulated in fp32: 4 bytes per parameter, replicated); the bf16
   micro-batch gradient is this library's reading (the model is bf16). */
zero_status zero_grad_accumulate(float *main_grad, const uint16_t *micro_bf16,
                                 int64_t n, void *stream);

/* ---------------------------------------------- rate calibration -- */

/* HBM rate of the fused step's memory traffic without its arithmetic, for
   measuring the step kernel against the ceiling of its own access pattern
   (a measurement aid, not part of the optimizer step).  Over elements
   i < n, with the launch shape, tile walk and per-lane element ownership of
   zero_adam_step's fused kernel, and every buffer indexed from 0:
     ZERO_MIX_STEP_STREAMS  reads the n_ranks bf16 grads[q][i] and master[i],
                            m[i], v[i]; writes master[i] + s, m[i] + s and
                            v[i] + s (s = the fp32 sum of the rank values) and
                            param[i] = the upper 16 bits of the new master[i];
     ZERO_MIX_READS         the same reads, nothing written;
     ZERO_MIX_WRITES        the same writes, nothing read (master, m, v and
                            param receive values derived from i).
   Per element the step streams are 2*n_ranks + 12 bytes read and 14 bytes
   written, as in the fused step.  `grads` is a host array of n_ranks device
   pointers; 1 <= n_ranks <= ZERO_MAX_RANKS_PER_CALL; n must be a multiple of
   4 and every buffer 16-byte aligned (ZERO_ERR_INVALID_ARG /
   ZERO_ERR_ALIGNMENT otherwise, nothing launched).  `state_chunk` = 0 takes
   master, m and v as three arrays; a power of two E in
   [ZERO_STATE_CHUNK_MIN, ZERO_STATE_CHUNK_MAX] takes them in the chunked
   format of zero_layout_chunk_state (m = master + E, v = master + 2E), so
   the calibration covers the same addresses as a chunked-state step.
   Likewise `grad_chunk` = 0 takes n_ranks separate gradient buffers, and a
   power of two E in the same bounds takes them chunked as zero_grads.chunk
   describes (grads[q] = grads[0] + qE; element i of rank q at
   grads[q] + (i / E) n_ranks E + i % E). */
typedef enum {
    ZERO_MIX_STEP_STREAMS = 0,
    ZERO_MIX_READS = 1,
    ZERO_MIX_WRITES = 2
} zero_mix_kind;

zero_status zero_stream_mix(int32_t kind, const uint16_t *const *grads, int32_t n_ranks,
                            float *master, float *m, float *v, uint16_t *param, int64_t n,
                            int64_t state_chunk, int64_t grad_chunk, void *stream);

/* ----------------------------------------------- FSDP linear layer -- */

/* How a GEMM operand is stored.  K_INNER: A as M x K, B as N x K (row-major,
   K contiguous).  K_OUTER: A as K x M, B as K x N (row-major, M or N
   contiguous). */
typedef enum {
    ZERO_K_INNER = 0,
    ZERO_K_OUTER = 1
} zero_operand_order;

/* C[i][j] = sum_{k < K} a(i, k) * b(j, k) for i < M, j < N on the MFMA
   units, where a(i, k) = A[i * lda + k] (K_INNER) or A[k * lda + i]
   (K_OUTER), and b(j, k) = B[j * ldb + k] (K_INNER) or B[k * ldb + j]
   (K_OUTER).  So with B K_OUTER this is C = A B, with both K_INNER
   C = A B^T, with both K_OUTER C = A^T B.  A and B are bf16 bits; C is
   row-major with leading dimension ldc, fp32 (c_dtype ZERO_FP32) or bf16
   rounded to nearest even (ZERO_BF16).  Accumulation is fp32 in the
   kernel's own order (error within the usual gamma_K bound of fp32 dot
   products).  Needs K, lda and ldb multiples of 8, M (N) a multiple of 8
   when A (B) is K_OUTER, lda >= K or M and ldb >= K or N by order,
   ldc >= N, and 16-byte aligned A and B.  Operands are read through 32-bit
   buffer offsets, so a K_INNER operand's leading dimension must be at most
   2^22 = 4,194,304 elements and a K_OUTER one's at most 2^25 = 33,554,432.
   C may span at most 4,194,303 tiles of 256 x 256 (the launch, up to two
   512-thread blocks per tile, stays below 2^32 work-items).
   ZERO_ERR_UNSUPPORTED or ZERO_ERR_ALIGNMENT otherwise, with nothing
   launched.  M = 0 or N = 0 is
   a no-op; K = 0 writes zeros.  All pointers are device memory owned by the
   caller. */
zero_status zero_gemm_bf16(int64_t M, int64_t N, int64_t K, const uint16_t *A,
                           int64_t lda, int32_t a_order, const uint16_t *B,
                           int64_t ldb, int32_t b_order, void *C, int64_t ldc,
                           int32_t c_dtype, void *stream);

/* zero_gemm_bf16 with both operands K_INNER: C = A B^T. */
zero_status zero_gemm_bf16_nt(int64_t M, int64_t N, int64_t K, const uint16_t *A,
                              int64_t lda, const uint16_t *B, int64_t ldb,
                              void *C, int64_t ldc, int32_t c_dtype,
                              void *stream);

/* dst[c * ldd + r] = src[r * lds + c] for r < rows, c < cols (bf16 bits). */
zero_status zero_transpose_bf16(int64_t rows, int64_t cols, const uint16_t *src,
                                int64_t lds, uint16_t *dst, int64_t ldd,
                                void *stream);

/* A hand-written FSDP linear layer ("DP, ZeRO-1/2/3, FSDP" notes, follow-up
   on writing one FSDP linear layer: each rank stores 1/N of the rows of W;
   forward all-gathers W and computes X W; backward all-gathers W again,
   computes dX and the full-shape dW locally, and reduce-scatters dW into
   each rank's rows).  W is unit `unit` of a row layout
   (zero_shard_init_rows): rows = in_features (in), cols = out_features
   (out), so rank r's W shard is its c_u x out rows.
   forward:  w_full = all-gather(w_shards) (device, L_u bf16 workspace);
             y = x W (x: batch x in bf16; y: batch x out, y_dtype).
   backward: w_full = all-gather(w_shards) again; dx = dy W^T (dy: batch x
             out bf16; dx: batch x in, dx_dtype); dw_full = x^T dy (fp32,
             the padded unit: in rows then zeroed padding rows, L_u
             elements).  The reduce-scatter of the N ranks' dw_full is
             zero_reduce_shard (fp32 grads, ZERO_INDEX_FULL) on this unit,
             and zero_adam_step(grad_fp32 = its output) steps the shard.
   Every GEMM reads its operands in place (zero_gemm_bf16 with K_OUTER
   operands), so no transposed copies are made.
   `w_shards` is a host array of world_n device pointers (s_u bf16 each, this
   rank's own included).  in and out must be multiples of 8, and batch too
   for the backward; x, dy, w_full and the shards 16-byte aligned. */
zero_status zero_fsdp_linear_forward(const zero_layout *layout, int32_t unit,
                                     const uint16_t *const *w_shards,
                                     int64_t batch, const uint16_t *x,
                                     uint16_t *w_full, void *y, int32_t y_dtype,
                                     void *stream);

zero_status zero_fsdp_linear_backward(const zero_layout *layout, int32_t unit,
                                      const uint16_t *const *w_shards,
                                      int64_t batch, const uint16_t *x,
                                      const uint16_t *dy, uint16_t *w_full,
                                      void *dx, int32_t dx_dtype,
                                      float *dw_full, void *stream);

/* ---------------------------------------------------------- errors -- */

const char *zero_status_str(zero_status status);
const char *zero_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_SHARD_H */
