// bf16 GEMM on MFMA (gfx950) and a bf16 transpose: the dense contractions of
// a hand-written FSDP linear layer ("DP, ZeRO-1/2/3, FSDP" notes, follow-up
// on writing one FSDP linear layer by hand).
//
//   zero_gemm_bf16_nt:  C[M x N] = A[M x K] * B[N x K]^T, A and B bf16
//                       row-major (K contiguous in both -- the operand layout
//                       the MFMA fragments want), fp32 accumulation, C fp32
//                       or bf16 (round to nearest even).
//   zero_transpose_bf16: dst[c][r] = src[r][c].
//
// GEMM tiling: 256-thread blocks (4 waves) own a 128 x 128 tile of C; each
// wave owns 64 x 64 as 2 x 2 tiles of v_mfma_f32_32x32x16_bf16.  K advances
// 32 at a time through double-buffered LDS tiles (rows padded to 40 bf16),
// loaded with 128-bit global loads; the next K-tile is fetched into
// registers while the current one feeds the MFMAs, and one barrier per K
// step separates the two LDS buffers.
//
// MFMA 32x32x16 bf16 lane layout (checked on the device against an exact
// CPU product): lane l holds A row (l % 32), k = 8 (l / 32) .. +7, and B
// column (l % 32) at the same k; accumulator v of lane l is row
// 8 (v / 4) + 4 (l / 32) + (v % 4), column l % 32.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace zs {
namespace {

constexpr int kGT = 256;          // threads per GEMM block
constexpr int kBM = 128, kBN = 128, kBK = 32;
constexpr int kLdsRow = kBK + 8;  // padded LDS row (bf16 elements), 80 bytes

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// One 128 x 32 bf16 tile of a K-contiguous matrix: 512 chunks of 8
// elements, two per thread; rows past `rows` and k past K read as zero.
struct TileRegs {
    u32x4 v[2];
};

__device__ __forceinline__ void load_tile(TileRegs &r, const uint16_t *base, int64_t ld,
                                          int64_t row0, int64_t rows, int64_t k0, int64_t K)
{
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = threadIdx.x + h * kGT;
        const int64_t row = row0 + (c >> 2);
        const int64_t k = k0 + (c & 3) * 8;
        if (row < rows && k < K)
            r.v[h] = *reinterpret_cast<const u32x4 *>(base + row * ld + k);
        else
            r.v[h] = u32x4{0u, 0u, 0u, 0u};
    }
}

__device__ __forceinline__ void store_tile(const TileRegs &r, uint16_t *lds)
{
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = threadIdx.x + h * kGT;
        *reinterpret_cast<u32x4 *>(lds + (c >> 2) * kLdsRow + (c & 3) * 8) = r.v[h];
    }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(kGT) void gemm_nt_kernel(int64_t M, int64_t N, int64_t K,
                                                      const uint16_t *__restrict__ A, int64_t lda,
                                                      const uint16_t *__restrict__ B, int64_t ldb,
                                                      void *__restrict__ C, int64_t ldc)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kLdsRow];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBN * kLdsRow];

    const int64_t m0 = (int64_t)blockIdx.y * kBM;
    const int64_t n0 = (int64_t)blockIdx.x * kBN;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const int fr = lane & 31;          // fragment row / column
    const int fk = (lane >> 5) * 8;    // fragment k offset

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[i][j][v] = 0.0f;

    const int64_t kt_n = (K + kBK - 1) / kBK;
    TileRegs ra, rb;
    load_tile(ra, A, lda, m0, M, 0, K);
    load_tile(rb, B, ldb, n0, N, 0, K);
    store_tile(ra, As[0]);
    store_tile(rb, Bs[0]);
    __syncthreads();

    for (int64_t kt = 0; kt < kt_n; ++kt) {
        const int cur = (int)(kt & 1);
        if (kt + 1 < kt_n) {
            load_tile(ra, A, lda, m0, M, (kt + 1) * kBK, K);
            load_tile(rb, B, ldb, n0, N, (kt + 1) * kBK, K);
        }
#pragma unroll
        for (int ks = 0; ks < kBK; ks += 16) {
            bf16x8 fa[2], fb[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                fa[t] = *reinterpret_cast<const bf16x8 *>(
                    &As[cur][(wm + 32 * t + fr) * kLdsRow + ks + fk]);
                fb[t] = *reinterpret_cast<const bf16x8 *>(
                    &Bs[cur][(wn + 32 * t + fr) * kLdsRow + ks + fk]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j],
                                                                         0, 0, 0);
        }
        if (kt + 1 < kt_n) {
            store_tile(ra, As[cur ^ 1]);
            store_tile(rb, Bs[cur ^ 1]);
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
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

zero_status zero_gemm_bf16_nt(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                              const uint16_t *B, int64_t ldb, void *C, int64_t ldc,
                              int32_t c_dtype, void *stream)
{
    using zs::fail;
    if (M < 0 || N < 0 || K < 0)
        return fail(ZERO_ERR_INVALID_ARG, "negative GEMM size");
    if (M == 0 || N == 0)
        return ZERO_OK;
    if (!A || !B || !C)
        return fail(ZERO_ERR_INVALID_ARG, "A, B and C are required");
    if (c_dtype != ZERO_BF16 && c_dtype != ZERO_FP32)
        return fail(ZERO_ERR_INVALID_ARG, "unknown C dtype %d", c_dtype);
    if (K % 8 || lda < K || ldb < K || ldc < N || lda % 8 || ldb % 8)
        return fail(ZERO_ERR_UNSUPPORTED, "GEMM needs K, lda and ldb multiples of 8, "
                    "lda, ldb >= K and ldc >= N");
    if (!zs::a16(A) || !zs::a16(B))
        return fail(ZERO_ERR_ALIGNMENT, "A and B must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(C) % (c_dtype == ZERO_BF16 ? 2 : 4))
        return fail(ZERO_ERR_ALIGNMENT, "C is misaligned");
    if ((M + zs::kBM - 1) / zs::kBM > 65535)
        return fail(ZERO_ERR_UNSUPPORTED, "M too large for one launch");
    const dim3 grid((unsigned)((N + zs::kBN - 1) / zs::kBN), (unsigned)((M + zs::kBM - 1) / zs::kBM));
    const hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (c_dtype == ZERO_BF16)
        hipLaunchKernelGGL(zs::gemm_nt_kernel<true>, grid, dim3(zs::kGT), 0, s, M, N, K, A, lda, B,
                           ldb, C, ldc);
    else
        hipLaunchKernelGGL(zs::gemm_nt_kernel<false>, grid, dim3(zs::kGT), 0, s, M, N, K, A, lda,
                           B, ldb, C, ldc);
    return zs::launched("gemm");
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
    if ((rows + zs::kTT - 1) / zs::kTT > 65535)
        return fail(ZERO_ERR_UNSUPPORTED, "too many rows for one launch");
    const dim3 grid((unsigned)((cols + zs::kTT - 1) / zs::kTT),
                    (unsigned)((rows + zs::kTT - 1) / zs::kTT));
    (void)hipGetLastError();
    hipLaunchKernelGGL(zs::transpose_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                       rows, cols, src, lds, dst, ldd);
    return zs::launched("transpose");
}

}  // extern "C"
