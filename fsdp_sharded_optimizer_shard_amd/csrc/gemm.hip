// bf16 GEMM on MFMA (gfx950) and a bf16 transpose: the dense contractions of
// a hand-written FSDP linear layer ("DP, ZeRO-1/2/3, FSDP" notes, follow-up
// on writing one FSDP linear layer by hand).
//
//   zero_gemm_bf16:     C[i][j] = sum_k a(i, k) b(j, k), fp32 accumulation, C
//                       fp32 or bf16 (round to nearest even).  Each operand is
//                       stored either K-inner (A as M x K, B as N x K) or
//                       K-outer (A as K x M, B as K x N), so X W, dY W^T and
//                       X^T dY all run without a separate transpose.
//   zero_gemm_bf16_nt:  the K-inner / K-inner case.
//   zero_transpose_bf16: dst[c][r] = src[r][c].
//
// GEMM tiling.  A 256-thread block (4 waves, one per SIMD) owns a 256 x 256
// tile of C; each wave owns 128 x 128 as 4 x 4 tiles of
// v_mfma_f32_32x32x16_bf16, so its 256 fp32 accumulators per lane live in
// the accumulation registers.  K advances 64 at a time through two LDS
// buffers of 256 x 64 bf16 per operand (128 KB).  LDS rows are 128 bytes
// with the 16-byte chunk c of row r stored at position c ^ s(r),
// s(r) = (r ^ (r >> 3)) & 7, which keeps both the staging writes and the
// fragment reads free of bank conflicts.
//
// Staging.  A K-inner operand is read as 16-byte chunks along K (thread t:
// rows t/8 + 32 i, chunk t % 8).  A K-outer operand is read as one 8 x 8
// block per thread (k-block t / 32, row-block t % 32) that is transposed in
// registers with v_perm_b32 before it is written to LDS, so the fragment
// reads are the same for both orders.
//
// Pipeline per K tile of 64 (four MFMA substeps of k = 16): the global loads
// of the next tile are issued during the first substep; the fragment reads
// of substep s + 1 are issued during the MFMAs of substep s; the next tile is
// written to the other LDS buffer during the first half of the last substep,
// then one barrier, then the next tile's first fragments are read during the
// second half.  sched_group_barrier fixes that interleave.
//
// Tile order.  Block b runs on XCD b % 8; each XCD gets a contiguous range of
// tiles, walked 4 tile rows at a time, so the blocks that share an L2 share
// A rows and B columns.
//
// MFMA 32x32x16 bf16 lane layout (checked on the device against an exact
// CPU product): lane l holds A row (l % 32), k = 8 (l / 32) .. +7, and B
// column (l % 32) at the same k; accumulator v of lane l is row
// 8 (v / 4) + 4 (l / 32) + (v % 4), column l % 32.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "internal.h"

namespace zs {
namespace {

constexpr int kGT = 256;  // threads per GEMM block
constexpr int kBM = 256, kBN = 256, kBK = 64;
// Tile rows walked together.  Paired runs of the Mistral-7B MLP layer's
// GEMMs (distinct operands per launch): 4 rows beat 8 by 9 % on the dW
// products and 1-2 % on the others; 2, 6 and 16 were slower than 4.
constexpr int kGroupM = 4;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// LDS position (in elements) of the 16-byte chunk `c` of tile row `r`.
__device__ __forceinline__ int lds_pos(int r, int c)
{
    return r * kBK + ((c ^ ((r ^ (r >> 3)) & 7)) * 8);
}

// Staging of one operand's R x 64 tile (R = 256, or 128 for a half tile).
// K-inner: thread t reads the 16-byte chunks (row t/8 + 32 i, k chunk t % 8),
// i < R / 32.  K-outer: thread t reads the block of rows RB (t % 32) .. +RB-1
// (RB = R / 32) at k = 8 (t / 32) .. +7 -- eight loads of RB elements -- and
// transposes it in registers into RB chunks of 8 k values.  Both give R / 32
// LDS writes per thread.  Rows past the matrix are clamped to real rows
// (K-outer: to the last RB; rows % 8 == 0): they only feed C rows or
// columns that are never stored.
template <int R, bool KOUTER>
struct Stage {
    static constexpr int RB = R / 32;              // K-outer rows per block
    static constexpr int NL = KOUTER ? 8 : R / 32;  // global loads per thread
    static constexpr int NW = R / 32;               // LDS writes per thread
};

template <int R, bool KOUTER>
__device__ __forceinline__ void tile_sources(const uint16_t *(&src)[8], const uint16_t *base,
                                             int64_t ld, int64_t row0, int64_t rows, int t)
{
    constexpr int RB = Stage<R, KOUTER>::RB;
    if (!KOUTER) {
#pragma unroll
        for (int i = 0; i < R / 32; ++i) {
            int64_t row = row0 + (t >> 3) + 32 * i;
            row = row < rows ? row : rows - 1;
            src[i] = base + row * ld + (t & 7) * 8;
        }
    } else {
        int64_t c = row0 + (t & 31) * RB;
        c = c < rows ? c : rows - RB;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            src[i] = base + (int64_t)((t >> 5) * 8 + i) * ld + c;
    }
}

template <int R, bool KOUTER>
__device__ __forceinline__ void tile_dests(int (&dst)[8], int t)
{
    constexpr int RB = Stage<R, KOUTER>::RB;
#pragma unroll
    for (int i = 0; i < R / 32; ++i)
        dst[i] = KOUTER ? lds_pos((t & 31) * RB + i, t >> 5) : lds_pos((t >> 3) + 32 * i, t & 7);
}

// k offset, within the tile, of the data thread t stages.
template <bool KOUTER>
__device__ __forceinline__ int tile_kofs(int t)
{
    return KOUTER ? (t >> 5) * 8 : (t & 7) * 8;
}

// Global -> registers for the tile at k0.  MASKED: the tile runs past K; the
// thread's 8 k values are all in range or all out (K % 8 == 0) and out of
// range ones read as zero.
template <int R, bool KOUTER, bool MASKED>
__device__ __forceinline__ void tile_load(u32x4 (&v)[8], const uint16_t *const (&src)[8],
                                          int64_t ld, int64_t k0, int64_t K, int kofs)
{
    const int64_t adv = KOUTER ? k0 * ld : k0;
    const bool ok = !MASKED || k0 + kofs < K;
#pragma unroll
    for (int i = 0; i < Stage<R, KOUTER>::NL; ++i) {
        if (!KOUTER || R == 256) {
            if (MASKED)
                v[i] = ok ? *reinterpret_cast<const u32x4 *>(src[i] + adv) : u32x4{0u, 0u, 0u, 0u};
            else
                v[i] = *reinterpret_cast<const u32x4 *>(src[i] + adv);
        } else {  // K-outer half tile: 4 rows (8 bytes) per load
            u32x2 h;
            if (MASKED)
                h = ok ? *reinterpret_cast<const u32x2 *>(src[i] + adv) : u32x2{0u, 0u};
            else
                h = *reinterpret_cast<const u32x2 *>(src[i] + adv);
            v[i][0] = h[0];
            v[i][1] = h[1];
        }
    }
}

// Registers -> LDS.  K-outer: v[i] holds rows 0..RB-1 at k = i; row j's
// eight k values are gathered with v_perm_b32 (low or high halves of a pair).
template <int R, bool KOUTER>
__device__ __forceinline__ void tile_store(const u32x4 (&v)[8], uint16_t *lds, const int (&dst)[8])
{
#pragma unroll
    for (int j = 0; j < Stage<R, KOUTER>::NW; ++j) {
        u32x4 w;
        if (!KOUTER) {
            w = v[j];
        } else {
            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                w[q] = __builtin_amdgcn_perm(v[2 * q + 1][j >> 1], v[2 * q][j >> 1], sel);
        }
        *reinterpret_cast<u32x4 *>(lds + dst[j]) = w;
    }
}

// XCD-contiguous order over a range of `n` blocks: block i of the range runs
// on XCD (first + i) % 8, and each XCD gets a contiguous run of the range.
__device__ __forceinline__ int xcd_order(int i, int n)
{
    const int per = n / 8, rem = n % 8, x = i % 8;
    return x * per + (x < rem ? x : rem) + i / 8;
}

// Grouped order: big tile `logical` -> (tile row, tile column), kGroupM tile
// rows at a time.
__device__ __forceinline__ void grouped(int logical, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int gsz = kGroupM * tiles_n;
    const int g = logical / gsz;
    const int first_m = g * kGroupM;
    const int gm = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
    const int in_g = logical - g * gsz;
    tm = first_m + in_g % gm;
    tn = in_g / gm;
}

// One BM x 256 tile of C (BM = 256, or 128 for half tiles): 4 waves, each
// (BM / 2) x 128 as (BM / 64) x 4 MFMA tiles.
template <int BM, bool A_KOUTER, bool B_KOUTER, bool OUT_BF16>
__device__ __forceinline__ void gemm_tile(int64_t M, int64_t N, int64_t K,
                                          const uint16_t *__restrict__ A, int64_t lda,
                                          const uint16_t *__restrict__ B, int64_t ldb,
                                          void *__restrict__ C, int64_t ldc, int64_t m0,
                                          int64_t n0, uint16_t (*As)[kBM * kBK],
                                          uint16_t (*Bs)[kBN * kBK])
{
    constexpr int TM = BM / 64, TN = 4;  // 32 x 32 MFMA tiles per wave
    constexpr int NF = TM + TN;          // fragment reads per substep
    constexpr int NMF = TM * TN;         // MFMAs per substep
    constexpr int NG = Stage<BM, A_KOUTER>::NL + Stage<kBN, B_KOUTER>::NL;  // global loads
    constexpr int NW = Stage<BM, A_KOUTER>::NW + Stage<kBN, B_KOUTER>::NW;  // LDS writes

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = (wave >> 1) * (BM / 2), wn = (wave & 1) * (kBN / 2);
    const int fr = lane & 31, fh = lane >> 5;

    const uint16_t *sa[8], *sb[8];
    tile_sources<BM, A_KOUTER>(sa, A, lda, m0, M, t);
    tile_sources<kBN, B_KOUTER>(sb, B, ldb, n0, N, t);
    int da[8], db[8];
    tile_dests<BM, A_KOUTER>(da, t);
    tile_dests<kBN, B_KOUTER>(db, t);
    const int ka = tile_kofs<A_KOUTER>(t), kb = tile_kofs<B_KOUTER>(t);

    // Fragment read positions for the four substeps.
    int fa_pos[TM][4], fb_pos[TN][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
            fa_pos[i][s] = lds_pos(wm + 32 * i + fr, 2 * s + fh);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            fb_pos[j][s] = lds_pos(wn + 32 * j + fr, 2 * s + fh);
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[i][j][v] = 0.0f;

    u32x4 ra[8], rb[8];
    bf16x8 fa0[TM], fb0[TN], fa1[TM], fb1[TN];

    auto frags = [&](int buf, int s, bf16x8 (&fa)[TM], bf16x8 (&fb)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
            fa[i] = *reinterpret_cast<const bf16x8 *>(&As[buf][fa_pos[i][s]]);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            fb[j] = *reinterpret_cast<const bf16x8 *>(&Bs[buf][fb_pos[j][s]]);
    };
    auto mma = [&](const bf16x8 (&fa)[TM], const bf16x8 (&fb)[TN], int lo, int hi) {
#pragma unroll
        for (int q = 0; q < NMF; ++q)
            if (q >= lo && q < hi)
                acc[q / TN][q % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    fa[q / TN], fb[q % TN], acc[q / TN][q % TN], 0, 0, 0);
    };
    auto load = [&](int64_t k0, bool masked) {
        if (masked) {
            tile_load<BM, A_KOUTER, true>(ra, sa, lda, k0, K, ka);
            tile_load<kBN, B_KOUTER, true>(rb, sb, ldb, k0, K, kb);
        } else {
            tile_load<BM, A_KOUTER, false>(ra, sa, lda, k0, K, ka);
            tile_load<kBN, B_KOUTER, false>(rb, sb, ldb, k0, K, kb);
        }
    };
    auto store = [&](int buf) {
        tile_store<BM, A_KOUTER>(ra, As[buf], da);
        tile_store<kBN, B_KOUTER>(rb, Bs[buf], db);
    };
    // Interleave: per fragment read, NMF / NF MFMAs (and optionally NG / NF
    // global loads).
    auto interleave_reads = [&](bool with_loads) {
#pragma unroll
        for (int q = 0; q < NF; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, NMF / NF, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);         // LDS read
            if (with_loads)
                __builtin_amdgcn_sched_group_barrier(0x020, NG / NF, 0);  // global read
        }
    };

    // One K tile.  next: 0 none, 1 full tile, 2 tile running past K.
    auto tile = [&](int64_t kt, int next) {
        const int cur = (int)(kt & 1);
        if (next)
            load((kt + 1) * kBK, next == 2);
        frags(cur, 1, fa1, fb1);
        mma(fa0, fb0, 0, NMF);
        interleave_reads(next != 0);
        frags(cur, 2, fa0, fb0);
        mma(fa1, fb1, 0, NMF);
        interleave_reads(false);
        frags(cur, 3, fa1, fb1);
        mma(fa0, fb0, 0, NMF);
        interleave_reads(false);
        mma(fa1, fb1, 0, NMF / 2);
        if (next) {
            store(cur ^ 1);
#pragma unroll
            for (int q = 0; q < NMF / 2; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
                __builtin_amdgcn_sched_group_barrier(0x200, NW / (NMF / 2), 0);  // LDS write
            }
        }
        __syncthreads();
        if (next) {
            frags(cur ^ 1, 0, fa0, fb0);
            mma(fa1, fb1, NMF / 2, NMF);
#pragma unroll
            for (int q = 0; q < NF; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
        } else {
            mma(fa1, fb1, NMF / 2, NMF);
        }
    };

    const int64_t kt_n = (K + kBK - 1) / kBK;
    const int64_t kt_full = K / kBK;
    load(0, kt_full == 0);
    store(0);
    __syncthreads();
    frags(0, 0, fa0, fb0);
    // Tiles before `last_full_next` prefetch a full tile; then at most one
    // prefetches the partial tail; the last prefetches nothing.
    const int64_t last_full_next = kt_full < kt_n ? kt_full - 1 : kt_n - 1;
    int64_t kt = 0;
    for (; kt < last_full_next; ++kt)
        tile(kt, 1);
    if (kt < kt_n - 1) {
        tile(kt, 2);
        ++kt;
    }
    tile(kt, 0);

#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * fh + (v & 3);
                const int64_t col = n0 + wn + 32 * j + fr;
                if (row < M && col < N) {
                    if (OUT_BF16)
                        static_cast<uint16_t *>(C)[row * ldc + col] =
                            (uint16_t)f32_to_bf16_rne(acc[i][j][v]);
                    else
                        static_cast<float *>(C)[row * ldc + col] = acc[i][j][v];
                }
            }
}

// Blocks [0, n_big) compute whole 256 x 256 tiles (big tiles 0 .. n_big-1 in
// grouped order); the remaining blocks split the last big tiles into
// 128 x 256 halves, two blocks per tile, so a partial last wave of big
// tiles becomes a wave of half-length work.
template <bool A_KOUTER, bool B_KOUTER, bool OUT_BF16>
__global__ __launch_bounds__(kGT) void gemm_kernel(int64_t M, int64_t N, int64_t K,
                                                   const uint16_t *__restrict__ A, int64_t lda,
                                                   const uint16_t *__restrict__ B, int64_t ldb,
                                                   void *__restrict__ C, int64_t ldc, int tiles_m,
                                                   int tiles_n, int n_big)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBN * kBK];
    const int b = blockIdx.x;
    int tm, tn;
    if (b < n_big) {
        grouped(xcd_order(b, n_big), tiles_m, tiles_n, tm, tn);
        gemm_tile<kBM, A_KOUTER, B_KOUTER, OUT_BF16>(M, N, K, A, lda, B, ldb, C, ldc,
                                                     (int64_t)tm * kBM, (int64_t)tn * kBN, As, Bs);
    } else {
        const int h = xcd_order(b - n_big, (int)gridDim.x - n_big);
        grouped(n_big + h / 2, tiles_m, tiles_n, tm, tn);
        gemm_tile<kBM / 2, A_KOUTER, B_KOUTER, OUT_BF16>(
            M, N, K, A, lda, B, ldb, C, ldc, (int64_t)tm * kBM + (h & 1) * (kBM / 2),
            (int64_t)tn * kBN, As, Bs);
    }
}

// 64 x 64 tiles through LDS (one padding column against bank conflicts):
// reads along src rows and writes along dst rows are both coalesced.
constexpr int kTT = 64;
__global__ __launch_bounds__(256) void transpose_kernel(int64_t rows, int64_t cols,
                                                        const uint16_t *__restrict__ src,
                                                        int64_t lds, uint16_t *__restrict__ dst,
                                                        int64_t ldd)
{
    __shared__ uint16_t t[kTT][kTT + 2];
    const int64_t r0 = (int64_t)blockIdx.y * kTT, c0 = (int64_t)blockIdx.x * kTT;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int i = ty; i < kTT; i += 4) {
        const int64_t r = r0 + i, c = c0 + tx;
        t[i][tx] = (r < rows && c < cols) ? src[r * lds + c] : (uint16_t)0;
    }
    __syncthreads();
    for (int i = ty; i < kTT; i += 4) {
        const int64_t c = c0 + i, r = r0 + tx;  // dst row c, column r
        if (c < cols && r < rows)
            dst[c * ldd + r] = t[tx][i];
    }
}

// Fills rows [r0, r1) x cols of an fp32 matrix with zeros (a kernel, so it
// is safe inside captured graphs).
__global__ __launch_bounds__(256) void zero_rows_kernel(float *p, int64_t ld, int64_t r0,
                                                        int64_t r1, int64_t cols)
{
    const int64_t n = (r1 - r0) * cols;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * 256)
        p[(r0 + i / cols) * ld + i % cols] = 0.0f;
}

bool a16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Compute units of the current device (cached per device).
int cu_count()
{
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        dev = -1;
    if (dev >= 0 && dev < 64 && cache[dev] > 0)
        return cache[dev];
    int n = 0;
    if (dev < 0 || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                       hipSuccess || n <= 0)
        n = 256;
    if (dev >= 0 && dev < 64)
        cache[dev] = n;
    return n;
}

zero_status launched(const char *what)
{
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(ZERO_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return ZERO_OK;
}

}  // namespace

zero_status zero_rows_fill(float *p, int64_t ld, int64_t r0, int64_t r1, int64_t cols,
                           hipStream_t s)
{
    if (r1 <= r0 || cols <= 0)
        return ZERO_OK;
    const int64_t n = (r1 - r0) * cols;
    int64_t grid = (n + 255) / 256;
    grid = grid > 65536 ? 65536 : grid;
    (void)hipGetLastError();
    hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)grid), dim3(256), 0, s, p, ld, r0, r1,
                       cols);
    return launched("zero_rows");
}

}  // namespace zs

extern "C" {

zero_status zero_gemm_bf16(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                           int32_t a_order, const uint16_t *B, int64_t ldb, int32_t b_order,
                           void *C, int64_t ldc, int32_t c_dtype, void *stream)
{
    using zs::fail;
    if (M < 0 || N < 0 || K < 0)
        return fail(ZERO_ERR_INVALID_ARG, "negative GEMM size");
    if ((a_order != ZERO_K_INNER && a_order != ZERO_K_OUTER) ||
        (b_order != ZERO_K_INNER && b_order != ZERO_K_OUTER))
        return fail(ZERO_ERR_INVALID_ARG, "unknown operand order (%d, %d)", a_order, b_order);
    if (c_dtype != ZERO_BF16 && c_dtype != ZERO_FP32)
        return fail(ZERO_ERR_INVALID_ARG, "unknown C dtype %d", c_dtype);
    if (M == 0 || N == 0)
        return ZERO_OK;
    if (!A || !B || !C)
        return fail(ZERO_ERR_INVALID_ARG, "A, B and C are required");
    const bool ao = a_order == ZERO_K_OUTER, bo = b_order == ZERO_K_OUTER;
    if (K % 8 || lda % 8 || ldb % 8)
        return fail(ZERO_ERR_UNSUPPORTED, "GEMM needs K, lda and ldb multiples of 8");
    if ((ao && M % 8) || (bo && N % 8))
        return fail(ZERO_ERR_UNSUPPORTED, "a K-outer operand needs its M or N a multiple of 8");
    if (lda < (ao ? M : K) || ldb < (bo ? N : K) || ldc < N)
        return fail(ZERO_ERR_INVALID_ARG, "leading dimension too small (lda %lld, ldb %lld, "
                    "ldc %lld)", (long long)lda, (long long)ldb, (long long)ldc);
    if (!zs::a16(A) || !zs::a16(B))
        return fail(ZERO_ERR_ALIGNMENT, "A and B must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(C) % (c_dtype == ZERO_BF16 ? 2 : 4))
        return fail(ZERO_ERR_ALIGNMENT, "C is misaligned");
    const int64_t tm = (M + zs::kBM - 1) / zs::kBM, tn = (N + zs::kBN - 1) / zs::kBN;
    if (tm > INT_MAX / 2 / tn)
        return fail(ZERO_ERR_UNSUPPORTED, "too many GEMM tiles for one launch");
    // One block per CU at a time (128 KB of LDS).  A last wave of at most
    // half the CUs runs as twice as many half tiles.
    const int64_t T = tm * tn, P = zs::cu_count();
    const int64_t rem = T % P;
    const int64_t n_big = rem > 0 && rem <= P / 2 ? T - rem : T;
    const dim3 grid((unsigned)(n_big + 2 * (T - n_big))), block(zs::kGT);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int code = (ao ? 1 : 0) | (bo ? 2 : 0) | (c_dtype == ZERO_BF16 ? 4 : 0);
    (void)hipGetLastError();
#define ZS_GEMM(AO, BO, BF)                                                                      \
    hipLaunchKernelGGL((zs::gemm_kernel<AO, BO, BF>), grid, block, 0, s, M, N, K, A, lda, B, ldb, \
                       C, ldc, (int)tm, (int)tn, (int)n_big)
    switch (code) {
    case 0: ZS_GEMM(false, false, false); break;
    case 1: ZS_GEMM(true, false, false); break;
    case 2: ZS_GEMM(false, true, false); break;
    case 3: ZS_GEMM(true, true, false); break;
    case 4: ZS_GEMM(false, false, true); break;
    case 5: ZS_GEMM(true, false, true); break;
    case 6: ZS_GEMM(false, true, true); break;
    default: ZS_GEMM(true, true, true); break;
    }
#undef ZS_GEMM
    return zs::launched("gemm");
}

zero_status zero_gemm_bf16_nt(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                              const uint16_t *B, int64_t ldb, void *C, int64_t ldc,
                              int32_t c_dtype, void *stream)
{
    return zero_gemm_bf16(M, N, K, A, lda, ZERO_K_INNER, B, ldb, ZERO_K_INNER, C, ldc, c_dtype,
                          stream);
}

zero_status zero_transpose_bf16(int64_t rows, int64_t cols, const uint16_t *src, int64_t lds,
                                uint16_t *dst, int64_t ldd, void *stream)
{
    using zs::fail;
    if (rows < 0 || cols < 0)
        return fail(ZERO_ERR_INVALID_ARG, "negative transpose size");
    if (rows == 0 || cols == 0)
        return ZERO_OK;
    if (!src || !dst || lds < cols || ldd < rows)
        return fail(ZERO_ERR_INVALID_ARG, "transpose needs src, dst, lds >= cols, ldd >= rows");
    if (reinterpret_cast<uintptr_t>(src) % 2 || reinterpret_cast<uintptr_t>(dst) % 2)
        return fail(ZERO_ERR_ALIGNMENT, "transpose buffers are misaligned");
    if ((rows + zs::kTT - 1) / zs::kTT > 65535 || (cols + zs::kTT - 1) / zs::kTT > INT_MAX)
        return fail(ZERO_ERR_UNSUPPORTED, "transpose too large for one launch");
    const dim3 grid((unsigned)((cols + zs::kTT - 1) / zs::kTT),
                    (unsigned)((rows + zs::kTT - 1) / zs::kTT));
    (void)hipGetLastError();
    hipLaunchKernelGGL(zs::transpose_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                       rows, cols, src, lds, dst, ldd);
    return zs::launched("transpose");
}

}  // extern "C"
