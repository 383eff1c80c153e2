// Host-only driver for the layout planner, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_layout_sanitized.py.  It drives
// zero_shard_init / zero_shard_init_rows / the queries through random and
// adversarial sizes (zero-length units, huge units, overflow, bad ranks)
// and checks the invariants the planner promises: offsets are prefix sums
// of padded lengths, slices tile each unit, every error returns a status
// and leaves *out NULL.  Exit status 0 means no invariant failed and the
// sanitizers reported nothing.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "zero_shard.h"

static int failures = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            ++failures;                                                 \
        }                                                               \
    } while (0)

static void check_layout(const zero_layout *L, int32_t n, const std::vector<int64_t> &numel,
                         const std::vector<int64_t> &cols)
{
    int64_t flat = 0, shard = 0, F = 0, S = 0;
    int32_t U = 0, N = 0, r = 0, strat = 0;
    CHECK(zero_layout_info(L, &F, &S, &U, &N, &r, &strat) == ZERO_OK);
    CHECK(U == (int32_t)numel.size() && N == n);
    for (int32_t u = 0; u < U; ++u) {
        int64_t nu, pl, fo, sl, so, rfo, c, fr, rc;
        CHECK(zero_layout_query(L, u, &nu, &pl, &fo, &sl, &so, &rfo) == ZERO_OK);
        CHECK(zero_layout_rows(L, u, &c, &fr, &rc) == ZERO_OK);
        CHECK(nu == numel[u] && c == cols[u]);
        CHECK(fo == flat && so == shard);
        const int64_t parts = strat == ZERO_DDP ? 1 : n;
        CHECK(pl == sl * parts && pl >= nu && pl - nu < parts * c);
        CHECK(sl % c == 0);
        CHECK(rfo == fo + (int64_t)r * sl);
        CHECK(fr >= 0 && rc >= 0 && rc * c <= sl && (fr + rc) * c <= nu);
        flat += pl;
        shard += sl;
    }
    CHECK(F == flat && S == shard);
    int64_t dummy;
    CHECK(zero_layout_query(L, U, &dummy, nullptr, nullptr, nullptr, nullptr, nullptr) ==
          ZERO_ERR_INVALID_ARG);
    CHECK(zero_layout_query(L, -1, &dummy, nullptr, nullptr, nullptr, nullptr, nullptr) ==
          ZERO_ERR_INVALID_ARG);
}

int main()
{
    std::mt19937_64 rng(20260101);
    const zero_strategy strategies[] = {ZERO_DDP, ZERO_STAGE1, ZERO_STAGE2, ZERO_STAGE3, ZERO_FSDP,
                                        ZERO_MEGATRON_DO};
    for (int it = 0; it < 4000; ++it) {
        const int32_t n = 1 + (int32_t)(rng() % 130);
        const int32_t r = (int32_t)(rng() % n);
        const int32_t U = 1 + (int32_t)(rng() % 40);
        const bool rows = rng() % 2;
        std::vector<int64_t> num(U), cols(U, 1), nrows(U);
        for (int32_t u = 0; u < U; ++u) {
            const int kind = (int)(rng() % 4);
            nrows[u] = kind == 0 ? 0 : kind == 1 ? (int64_t)(rng() % 7) : (int64_t)(rng() % 100000);
            if (rows)
                cols[u] = 1 + (int64_t)(rng() % 5000);
            num[u] = nrows[u] * cols[u];
        }
        const zero_strategy s = strategies[rng() % 6];
        zero_layout *L = nullptr;
        const zero_status st = rows ? zero_shard_init_rows(&L, s, n, r, U, nrows.data(), cols.data())
                                    : zero_shard_init(&L, s, n, r, U, num.data());
        CHECK(st == ZERO_OK && L);
        if (L) {
            check_layout(L, n, num, cols);
            // a chunked-state copy: the same layout, its state length
            const int64_t E = (int64_t)1 << (2 + (int)(rng() % 23));   // 4 .. 2^24
            zero_layout *C = nullptr;
            CHECK(zero_layout_chunk_state(L, E, &C) == ZERO_OK && C);
            if (C) {
                check_layout(C, n, num, cols);
                int64_t e = -1, len = -1, S = -1;
                CHECK(zero_layout_info(L, nullptr, &S, nullptr, nullptr, nullptr, nullptr) == ZERO_OK);
                CHECK(zero_layout_state(C, &e, &len) == ZERO_OK);
                CHECK(e == E && len == (S + E - 1) / E * 3 * E);
                CHECK(zero_layout_state(L, &e, &len) == ZERO_OK && e == 0 && len == S);
                zero_shard_destroy(C);
            }
            zero_layout *B = (zero_layout *)&rng;  // refused: *out becomes NULL
            CHECK(zero_layout_chunk_state(L, E + 1 + (E == 4 ? 1 : 0), &B) == ZERO_ERR_INVALID_ARG && !B);
            zero_shard_destroy(L);
        }
    }
    {
        zero_layout *C = (zero_layout *)&rng;
        CHECK(zero_layout_chunk_state(nullptr, 8, &C) == ZERO_ERR_INVALID_ARG && !C);
        CHECK(zero_layout_chunk_state(nullptr, 8, nullptr) == ZERO_ERR_INVALID_ARG);
        CHECK(zero_layout_state(nullptr, nullptr, nullptr) == ZERO_ERR_INVALID_ARG);
        // a state length past the representable byte range is refused
        const int64_t big = (int64_t)1 << 60;
        zero_layout *L = nullptr, *D = nullptr;
        CHECK(zero_shard_init(&L, ZERO_DDP, 1, 0, 1, &big) == ZERO_OK && L);
        CHECK(zero_layout_chunk_state(L, (int64_t)1 << 24, &D) == ZERO_OK && D);
        int64_t len = 0;
        CHECK(zero_layout_state(D, nullptr, &len) == ZERO_ERR_INVALID_ARG);
        CHECK(zero_layout_state(L, nullptr, &len) == ZERO_OK && len == big);
        zero_shard_destroy(D);
        zero_shard_destroy(L);
    }
    // adversarial sizes: every one is refused, and *out is left NULL
    const int64_t huge[] = {INT64_MAX, INT64_MAX / 2, (int64_t)1 << 62};
    for (int64_t h : huge) {
        zero_layout *L = (zero_layout *)&rng;  // must be overwritten with NULL
        CHECK(zero_shard_init(&L, ZERO_FSDP, 64, 0, 1, &h) == ZERO_ERR_INVALID_ARG && !L);
        const int64_t two[] = {((int64_t)1 << 60), ((int64_t)1 << 60)};
        L = (zero_layout *)&rng;
        CHECK(zero_shard_init(&L, ZERO_FSDP, 8, 0, 2, two) == ZERO_ERR_INVALID_ARG && !L);
        const int64_t r1 = (int64_t)1 << 40, c1 = (int64_t)1 << 30;
        L = (zero_layout *)&rng;
        CHECK(zero_shard_init_rows(&L, ZERO_FSDP, 8, 0, 1, &r1, &c1) == ZERO_ERR_INVALID_ARG && !L);
    }
    const int64_t one = 10, neg = -1, zero_cols = 0;
    zero_layout *L = nullptr;
    CHECK(zero_shard_init(&L, ZERO_FSDP, 0, 0, 1, &one) == ZERO_ERR_INVALID_ARG);
    CHECK(zero_shard_init(&L, ZERO_FSDP, 4, 4, 1, &one) == ZERO_ERR_INVALID_ARG);
    CHECK(zero_shard_init(&L, ZERO_FSDP, 4, -1, 1, &one) == ZERO_ERR_INVALID_ARG);
    CHECK(zero_shard_init(&L, ZERO_FSDP, 4, 0, 0, &one) == ZERO_ERR_INVALID_ARG);
    CHECK(zero_shard_init(&L, ZERO_FSDP, 4, 0, 1, &neg) == ZERO_ERR_INVALID_ARG);
    CHECK(zero_shard_init(&L, (zero_strategy)17, 4, 0, 1, &one) == ZERO_ERR_INVALID_ARG);
    CHECK(zero_shard_init(nullptr, ZERO_FSDP, 4, 0, 1, &one) == ZERO_ERR_INVALID_ARG);
    CHECK(zero_shard_init(&L, ZERO_FSDP, 4, 0, 1, nullptr) == ZERO_ERR_INVALID_ARG);
    CHECK(zero_shard_init_rows(&L, ZERO_FSDP, 4, 0, 1, &one, &zero_cols) == ZERO_ERR_INVALID_ARG);
    CHECK(zero_shard_init_rows(&L, ZERO_FSDP, 4, 0, 1, &one, nullptr) == ZERO_ERR_INVALID_ARG);
    CHECK(zero_layout_info(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) ==
          ZERO_ERR_INVALID_ARG);
    CHECK(zero_last_error()[0] != '\0');
    zero_shard_destroy(nullptr);
    for (int s = -1; s <= 6; ++s)
        CHECK(zero_status_str((zero_status)s) != nullptr);
    std::printf("layout sanitized driver: %d failures\n", failures);
    return failures ? 1 : 0;
}
