// Internal declarations shared by the host layout code and the HIP
// launchers of libzeroshard.  Not part of the C ABI.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "zero_shard.h"

struct zero_layout {
    int32_t strategy;
    int32_t world_n;  // N: ranks whose gradients are averaged
    int32_t rank;     // r (0 under DDP)
    int32_t parts;    // N when sharded, 1 under DDP
    int32_t n_units;
    // Per unit u (size n_units), and the prefix tables F and R (size n_units + 1).
    std::vector<int64_t> numel;      // n_u
    std::vector<int64_t> cols;       // elements per padding row (1: per element)
    std::vector<int64_t> padded;     // L_u
    std::vector<int64_t> slice;      // s_u
    std::vector<int64_t> flat_off;   // F_u, F_{U} = flat length
    std::vector<int64_t> shard_off;  // R_u, R_{U} = shard length
    // 0: master, m and v are three shard-indexed arrays.  Otherwise a power
    // of two E: one buffer of chunks of E elements, each chunk holding E
    // master, then E m, then E v values (zero_layout_chunk_state).
    int64_t state_chunk = 0;
};

namespace zs {

// Records a message for zero_last_error() and returns `st`.
zero_status fail(zero_status st, const char *fmt, ...)
    __attribute__((format(printf, 2, 3)));
void clear_error();

// Validates a unit range of a layout.
zero_status check_range(const zero_layout *L, int32_t unit_begin, int32_t unit_end);

// Checks master, m and v against the layout's state format: under a chunked
// state m and v must be master + E and master + 2E.
zero_status check_state(const zero_layout *L, const float *master, const float *m,
                        const float *v);

// Checks a call's rank gradient buffers against the layout: count, dtype,
// pointers, index modes and, for chunked gradients, the chunk and the
// pointers one chunk apart.
zero_status check_grads(const zero_layout *L, const zero_grads *g);

}  // namespace zs
