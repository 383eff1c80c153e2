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
// GEMM tiling.  A 512-thread block (8 waves, two per SIMD) owns a 256 x 256
// tile of C; each wave owns 128 x 64 as 4 x 2 tiles of
// v_mfma_f32_32x32x16_bf16 (128 fp32 accumulators per lane), so while one
// wave of a SIMD waits on its fragment reads the other issues MFMAs.  K
// advances 32 at a time through four LDS stages of 256 x 32 bf16 per
// operand (128 KB in all).
//
// Loads.  Operands go from HBM straight into LDS with buffer_load ... lds
// (16 bytes per lane, 1 KB per wave instruction): no register staging and
// no LDS write instructions.  The DMA of tile k + 3 is issued at the start
// of tile k, into the stage tile k - 1 has just released, so three tiles of
// loads are in flight.  Each block's buffer descriptors end at the
// operand's last element, so rows past M or N and k past K read as zero
// without touching memory.
//
// LDS layouts.  A K-inner stage has 64-byte rows (32 k); 16-byte chunk c of
// row r sits at slot c ^ ((r >> 2) & 3), which keeps the fragment reads
// (ds_read_b128) free of bank conflicts.  A K-outer stage is k-major (one
// 2R-byte row per k); its 32-byte units are permuted per k row (unit_pos), and a
// fragment is two ds_read_b64_tr_b16 that transpose 4 x 4 blocks of 16-bit
// values across each 16-lane group.  A DMA lane's global address is chosen
// so that it lands in the swizzled slot.  Both layouts read without bank
// conflicts (rocprofv3 SQ_LDS_BANK_CONFLICT reads 0).
//
// Pipeline per K tile of 32 (two MFMA substeps of 16): DMA of tile k + 3;
// substep 0 under the fragment reads of substep 1; half of substep 1; wait
// for this wave's DMA of tile k + 1 (two tiles may stay in flight) and its
// LDS reads, then one barrier; the rest of substep 1 under the reads of
// tile k + 1's first substep.  sched_group_barrier fixes that interleave.
// Measured against the previous design (register staging, two 64-k LDS
// buffers, one tile ahead), paired on the Mistral-7B MLP shapes with random
// operands: dX +8.5 %, forward +4.2 %, dW +6.7 %, 8192^3 +9.1 %; then eight
// waves instead of four (128 x 128 each): dX +4.9 %, forward +15 %, dW +9 %;
// a 2 x 4 wave grid (128 x 64 per wave) rather than 4 x 2 adds about 1 %
// and needs no register spills.  Every step gave bit-identical results.
//
// Tile order.  Block b runs on XCD b % 8; each XCD gets a contiguous range of
// tiles, walked 4 tile rows at a time, so the blocks that share an L2 share
// A rows and B columns.
//
// Both operands K-inner (dY W^T): 16x16x32 MFMAs and 64-k stage pairs
// (gemm_tile_kp, below), so that every DMA instruction moves whole cache
// lines; a pair lands every second tile, so only those tiles need a
// barrier.
//
// MFMA 32x32x16 bf16 lane layout (checked on the device against an exact
// CPU product): lane l holds A row (l % 32), k = 8 (l / 32) .. +7, and B
// column (l % 32) at the same k; accumulator v of lane l is row
// 8 (v / 4) + 4 (l / 32) + (v % 4), column l % 32.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstdint>
#include <type_traits>

#include "internal.h"

namespace zs {
namespace {

constexpr int kNW = 8;          // waves per GEMM block: two per SIMD
constexpr int kGT = 64 * kNW;   // threads per GEMM block
constexpr int kBM = 256, kBN = 256, kBK = 32;
constexpr int kStages = 4;                 // LDS stages of kBK
constexpr int kStage = kBM * kBK * 2;      // bytes of one operand's stage
constexpr uint32_t kOOB = 0x80000000u;     // a buffer offset past every range
// Tile rows walked together.  Paired runs of the Mistral-7B MLP layer's
// GEMMs (distinct operands per launch): 4 rows beat 8 by 9 % on the dW
// products and 1-2 % on the others; 2, 6 and 16 were slower than 4.
constexpr int kGroupM = 4;

#define ZS_LDS __attribute__((address_space(3)))
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
template <int V>
using IC = std::integral_constant<int, V>;

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// K-inner stage of the 32x32x16 tile: byte offset of the 16-byte chunk c
// (of 4) of row r, swizzled by (r >> 2) & 3 so that the fragment reads are
// free of bank conflicts.
__device__ __forceinline__ int ki_swz(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int ki_pos(int r, int c) { return r * 64 + ((c ^ ki_swz(r)) << 4); }

// Buffer descriptor over `bytes` bytes from `base` (clamped to 2^31 - 1;
// the host bounds every offset below that).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes)
{
    int64_t n = bytes < 0 ? 0 : bytes;
    n = n > 0x7fffffffLL ? 0x7fffffffLL : n;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n, 0x00020000);
}

// s_waitcnt vmcnt(V) lgkmcnt(0) (expcnt not waited).
template <int V>
__device__ __forceinline__ void wait_vm_lgkm0()
{
    static_assert(V >= 0 && V < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((V & 15) | ((V >> 4) << 14) | (0x7 << 4));
}

// A scheduling sequence of NQ groups sharing out NM MFMAs, NR LDS reads and
// NV global loads in order.
template <int NQ, int NM, int NR, int NV, int Q = 0>
__device__ __forceinline__ void seq()
{
    if constexpr (Q < NQ) {
        constexpr int m = NM * (Q + 1) / NQ - NM * Q / NQ;
        constexpr int r = NR * (Q + 1) / NQ - NR * Q / NQ;
        constexpr int v = NV * (Q + 1) / NQ - NV * Q / NQ;
        if constexpr (m > 0)
            __builtin_amdgcn_sched_group_barrier(0x008, m, 0);
        if constexpr (r > 0)
            __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
        if constexpr (v > 0)
            __builtin_amdgcn_sched_group_barrier(0x020, v, 0);
        seq<NQ, NM, NR, NV, Q + 1>();
    }
}

// One operand's R x 32 stage.  Each of the 8 waves issues R / 128 DMA
// instructions of 1 KB; instruction n of wave w fills stage bytes
// [1024 I, 1024 I + 1024), I = w + 8 n, lane l landing at 16 l.
//   K-inner (rows of 64 B): rows 16 I .. +15; lane l takes row 16 I + l / 4
//     and stage slot l % 4, which holds k chunk slot ^ ((row >> 2) & 3).
//   K-outer (k-major, 2R bytes per k row): KPI = 1024 / 2R k rows per
//     instruction; lane l takes k row KPI I + l / (64 / KPI) and 16 bytes of
//     it.  The 32-byte unit of rows 16 u .. 16 u + 15 in k row kr sits at
//     unit_pos(u, kr) = u ^ (kr & 3) ^ ((u & 1) << 2): the transposing reads
//     of two neighbouring 16-row units then fall in different 128-byte
//     halves of the banks (2-way conflicts without the last term).
template <int R, bool KOUTER>
struct Op {
    static constexpr int NI = R / (16 * kNW);          // DMA instructions per wave per stage
    static constexpr int KPI = 1024 / (2 * R);         // K-outer: k rows per instruction
    static constexpr int NRD = KOUTER ? 2 : 1;         // LDS reads per fragment
};

__device__ __forceinline__ int unit_pos(int u, int kr) { return u ^ (kr & 3) ^ ((u & 1) << 2); }
// Inverse of unit_pos for one k row.
__device__ __forceinline__ int unit_at(int pos, int kr)
{
    const int x = pos ^ (kr & 3);
    return x ^ ((x & 1) << 2);
}

template <int R, bool KOUTER>
__device__ __forceinline__ uint32_t dma_offset(int64_t ld, int wave, int lane, int n)
{
    const int I = wave + kNW * n;
    if (!KOUTER) {
        const int r = 16 * I + (lane >> 2), c = (lane & 3) ^ ki_swz(r);
        return (uint32_t)((r * ld + 8 * c) * 2);
    }
    constexpr int KPI = Op<R, true>::KPI, LPR = 64 / KPI;  // lanes per k row
    const int kr = KPI * I + lane / LPR, w = (lane % LPR) * 16;
    const int lu = unit_at(w >> 5, kr), half = (w >> 4) & 1;
    return (uint32_t)((kr * ld + lu * 16 + half * 8) * 2);
}

// The k offset within the stage of a K-inner lane's chunk (for the K tail).
__device__ __forceinline__ int dma_kofs(int wave, int lane, int n)
{
    const int r = 16 * (wave + kNW * n) + (lane >> 2);
    return 8 * ((lane & 3) ^ ki_swz(r));
}

// First LDS read offset of the fragment of rows w0 .. w0 + 31 at k
// 16 s + 8 fh .. +7 (fh = lane / 32).  K-inner: one ds_read_b128.
// K-outer: two ds_read_b64_tr_b16, the second 4 k rows further; within
// 16-lane group g (lanes 16 g .. of each half-wave), lane j reads 8 bytes of
// k row 16 s + 8 fh + j / 4 at row offset 4 (j % 4) of unit (w0 + 16 g) / 16,
// and the transpose hands each lane the four k values of one row.
template <int R, bool KOUTER>
__device__ __forceinline__ int frag_offset(int w0, int s, int lane)
{
    const int fr = lane & 31, fh = lane >> 5;
    if (!KOUTER)
        return ki_pos(w0 + fr, 2 * s + fh);
    const int g = (lane >> 4) & 1, j = lane & 15, m = j >> 2, q = j & 3;
    const int kr = 16 * s + 8 * fh + m;  // the second read's k row kr + 4 has the same unit_pos
    return kr * (2 * R) + unit_pos((w0 + 16 * g) >> 4, kr) * 32 + q * 8;
}

template <int R, bool KOUTER>
__device__ __forceinline__ bf16x8 frag_read(const ZS_LDS char *stage, int off)
{
    if (!KOUTER)
        return *reinterpret_cast<const ZS_LDS bf16x8 *>(stage + off);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ZS_LDS s16x4 *)(stage + off));
    const s16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((ZS_LDS s16x4 *)(stage + off + 4 * (2 * R)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
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

// One BM x 256 tile of C (BM = 256, or 128 for half tiles): 8 waves in a
// 2 x 4 grid, each (BM / 2) x 64 as (BM / 64) x 2 MFMA tiles, over K
// stages of 32 (two
// substeps of 16).  Tile kt lives in LDS stage kt % 4; its DMA went out at
// the start of tile kt - 3, so three tiles of loads are in flight and no
// register staging or LDS write instruction is involved.
template <int BM, bool A_KOUTER, bool B_KOUTER, bool OUT_BF16>
__device__ __forceinline__ void gemm_tile(int64_t M, int64_t N, int64_t K,
                                          const uint16_t *__restrict__ A, int64_t lda,
                                          const uint16_t *__restrict__ B, int64_t ldb,
                                          void *__restrict__ C, int64_t ldc, int64_t m0, int64_t n0,
                                          ZS_LDS char *const (&As)[kStages],
                                          ZS_LDS char *const (&Bs)[kStages])
{
    constexpr int TM = BM / 64, TN = 2;  // 32 x 32 MFMA tiles per wave
    constexpr int NF = TM + TN;          // fragments per substep
    constexpr int NMF = TM * TN;         // MFMAs per substep
    constexpr int NRD = TM * Op<BM, A_KOUTER>::NRD + TN * Op<kBN, B_KOUTER>::NRD;
    constexpr int NIA = Op<BM, A_KOUTER>::NI, NIB = Op<kBN, B_KOUTER>::NI;
    constexpr int D = NIA + NIB;         // DMA instructions per wave per tile

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = (wave >> 2) * (BM / 2), wn = (wave & 3) * (kBN / 4);
    const int fr = lane & 31, fh = lane >> 5;

    uint32_t va[4], vb[4];
    int ka[4], kb[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        va[n] = n < NIA ? dma_offset<BM, A_KOUTER>(lda, wave, lane, n) : 0u;
        vb[n] = n < NIB ? dma_offset<kBN, B_KOUTER>(ldb, wave, lane, n) : 0u;
        ka[n] = kb[n] = dma_kofs(wave, lane, n);
    }
    int fa_off[TM][2], fb_off[TN][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
            fa_off[i][s] = frag_offset<BM, A_KOUTER>(wm + 32 * i, s, lane);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            fb_off[j][s] = frag_offset<kBN, B_KOUTER>(wn + 32 * j, s, lane);
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[i][j][v] = 0.0f;

    const int64_t kt_n = (K + kBK - 1) / kBK, kt_full = K / kBK;
    // Descriptors end at each operand's last element: rows past M or N and
    // k rows past K read as zero without a memory access.
    auto rs_a = [&](int64_t k0) {
        return A_KOUTER ? rsrc(A + k0 * lda + m0, ((K - 1 - k0) * lda + M - m0) * 2)
                        : rsrc(A + m0 * lda + k0, ((M - 1 - m0) * lda + K - k0) * 2);
    };
    auto rs_b = [&](int64_t k0) {
        return B_KOUTER ? rsrc(B + k0 * ldb + n0, ((K - 1 - k0) * ldb + N - n0) * 2)
                        : rsrc(B + n0 * ldb + k0, ((N - 1 - n0) * ldb + K - k0) * 2);
    };
    // DMA of tile kt into stage S.  WHOLE: the tile lies inside K, so no
    // lane needs the K-inner tail mask.
    auto dma = [&](auto st, auto whole, int64_t kt) {
        constexpr int S = decltype(st)::value;
        constexpr bool WHOLE = decltype(whole)::value != 0;
        const int64_t k0 = kt * kBK;
        const __amdgpu_buffer_rsrc_t ra = rs_a(k0), rb = rs_b(k0);
#pragma unroll
        for (int n = 0; n < NIA; ++n) {
            const uint32_t o = !WHOLE && !A_KOUTER && k0 + ka[n] >= K ? kOOB : va[n];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (ZS_LDS void *)(As[S] + (wave + kNW * n) * 1024),
                                                     16, o, 0, 0, 0);
        }
#pragma unroll
        for (int n = 0; n < NIB; ++n) {
            const uint32_t o = !WHOLE && !B_KOUTER && k0 + kb[n] >= K ? kOOB : vb[n];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (ZS_LDS void *)(Bs[S] + (wave + kNW * n) * 1024),
                                                     16, o, 0, 0, 0);
        }
    };
    bf16x8 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    auto frags = [&](auto st, int s, bf16x8 (&fa)[TM], bf16x8 (&fb)[TN]) {
        constexpr int S = decltype(st)::value;
#pragma unroll
        for (int i = 0; i < TM; ++i)
            fa[i] = frag_read<BM, A_KOUTER>(As[S], fa_off[i][s]);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            fb[j] = frag_read<kBN, B_KOUTER>(Bs[S], fb_off[j][s]);
    };
    auto mma = [&](const bf16x8 (&fa)[TM], const bf16x8 (&fb)[TN], int lo, int hi) {
#pragma unroll
        for (int q = 0; q < NMF; ++q)
            if (q >= lo && q < hi)
                acc[q / TN][q % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    fa[q / TN], fb[q % TN], acc[q / TN][q % TN], 0, 0, 0);
    };
    // This wave's DMA for the tiles after `kt1` (at most two) is allowed to
    // stay in flight; everything up to tile kt1 and every LDS read is done.
    auto wait_for = [&](int64_t kt1) {
        const int64_t after = kt_n - 1 - kt1;
        if (after >= 2)
            wait_vm_lgkm0<2 * D>();
        else if (after == 1)
            wait_vm_lgkm0<D>();
        else
            wait_vm_lgkm0<0>();
    };
    // Tile kt in stage S: DMA tile kt + 3 into the stage tile kt - 1 used,
    // substep 0 under the reads of substep 1, half of substep 1, wait for tile
    // kt + 1 and barrier, then the rest under the reads of tile kt + 1's
    // first substep.  STEADY: tiles kt + 1 .. kt + 3 exist and lie inside K.
    auto tile = [&](auto st, auto steady, int64_t kt) {
        constexpr int S = decltype(st)::value;
        constexpr bool STEADY = decltype(steady)::value != 0;
        constexpr int SN = (S + kStages - 1) % kStages, S1 = (S + 1) % kStages;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (STEADY)
            dma(IC<SN>{}, IC<1>{}, kt + kStages - 1);
        else if (kt + kStages - 1 < kt_n)
            dma(IC<SN>{}, IC<0>{}, kt + kStages - 1);
        frags(IC<S>{}, 1, fa1, fb1);
        mma(fa0, fb0, 0, NMF);
        if constexpr (STEADY)
            seq<NF, NMF, NRD, D>();
        else
            seq<NF, NMF, NRD, 0>();
        mma(fa1, fb1, 0, NMF / 2);
        __builtin_amdgcn_sched_group_barrier(0x008, NMF / 2, 0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (STEADY)
            wait_vm_lgkm0<2 * D>();
        else
            wait_for(kt + 1);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (STEADY || kt + 1 < kt_n)
            frags(IC<S1>{}, 0, fa0, fb0);
        mma(fa1, fb1, NMF / 2, NMF);
        seq<NF, NMF / 2, NRD, 0>();
    };

    if (kt_n > 0) {
        dma(IC<0>{}, IC<0>{}, 0);
        if (kt_n > 1)
            dma(IC<1>{}, IC<0>{}, 1);
        if (kt_n > 2)
            dma(IC<2>{}, IC<0>{}, 2);
        wait_for(0);
        __builtin_amdgcn_s_barrier();
        frags(IC<0>{}, 0, fa0, fb0);
        int64_t kt = 0;
        // Groups of four tiles whose DMA targets (tiles kt + 3 .. kt + 6) lie
        // inside K, then the last few tiles with checks.
        for (; kt + 2 * kStages - 1 <= kt_full; kt += kStages) {
            tile(IC<0>{}, IC<1>{}, kt);
            tile(IC<1>{}, IC<1>{}, kt + 1);
            tile(IC<2>{}, IC<1>{}, kt + 2);
            tile(IC<3>{}, IC<1>{}, kt + 3);
        }
        for (; kt < kt_n; kt += kStages) {
            tile(IC<0>{}, IC<0>{}, kt);
            if (kt + 1 < kt_n)
                tile(IC<1>{}, IC<0>{}, kt + 1);
            if (kt + 2 < kt_n)
                tile(IC<2>{}, IC<0>{}, kt + 2);
            if (kt + 3 < kt_n)
                tile(IC<3>{}, IC<0>{}, kt + 3);
        }
    }

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

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Both operands K-inner (dY W^T) run on 16x16x32 MFMAs with K in 64-k stage
// pairs: a K-inner row chunk of one 32-k tile is 64 bytes, half a cache line,
// so one DMA instruction would touch 16 lines; a pair buffer holds 64 k per
// row, and each DMA instruction moves 8 whole 128-byte rows.  Two pair
// buffers per operand (128 KB).  The pair of tiles 2p, 2p + 1 is fetched at
// the start of tile 2p - 3, once the reads of pair p - 2 are done, and first
// read during tile 2p - 1: two tiles of lead, as with single stages.
// Paired against single 32-k stages: dX +10.6 %, bit-identical.
// Row r of a pair buffer holds k 0..63 of the pair as eight 16-byte chunks,
// chunk c at slot c ^ ((r >> 1) & 7); one DMA instruction moves 8 whole
// 128-byte rows.
__device__ __forceinline__ int kp_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int kp_pos(int r, int c) { return r * 128 + ((c ^ kp_swz(r)) << 4); }
__device__ __forceinline__ uint32_t kp_dma_offset(int64_t ld, int wave, int lane, int n)
{
    const int r = 8 * (wave + kNW * n) + (lane >> 3), c = (lane & 7) ^ kp_swz(r);
    return (uint32_t)((r * ld + 8 * c) * 2);
}
__device__ __forceinline__ int kp_kofs(int wave, int lane, int n)
{
    const int r = 8 * (wave + kNW * n) + (lane >> 3);
    return 8 * ((lane & 7) ^ kp_swz(r));
}
constexpr int kPair = kBM * 128;  // bytes of one operand's pair buffer

template <int BM, bool OUT_BF16>
__device__ __forceinline__ void gemm_tile_kp(int64_t M, int64_t N, int64_t K,
                                             const uint16_t *__restrict__ A, int64_t lda,
                                             const uint16_t *__restrict__ B, int64_t ldb,
                                             void *__restrict__ C, int64_t ldc, int64_t m0, int64_t n0,
                                             ZS_LDS char *A0, ZS_LDS char *A1, ZS_LDS char *B0,
                                             ZS_LDS char *B1)
{
    auto Ab = [&](auto pb) -> ZS_LDS char * {
        if constexpr (decltype(pb)::value == 0) return A0; else return A1;
    };
    auto Bb = [&](auto pb) -> ZS_LDS char * {
        if constexpr (decltype(pb)::value == 0) return B0; else return B1;
    };
    constexpr int TM = BM / 32, TN = 4;
    constexpr int NF = TM + TN, NMF = TM * TN;
    constexpr int NPA = BM / (8 * kNW), NPB = kBN / (8 * kNW);
    constexpr int DP = NPA + NPB;  // DMA instructions per wave per pair
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = (wave >> 2) * (BM / 2), wn = (wave & 3) * (kBN / 4);
    const int r16 = lane & 15, g = lane >> 4;

    uint32_t va[4], vb[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        va[n] = n < NPA ? kp_dma_offset(lda, wave, lane, n) : 0u;
        vb[n] = n < NPB ? kp_dma_offset(ldb, wave, lane, n) : 0u;
    }
    const int fa_off[2] = {kp_pos(wm + r16, g), kp_pos(wm + r16, 4 + g)};
    const int fb_off[2] = {kp_pos(wn + r16, g), kp_pos(wn + r16, 4 + g)};

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t kt_n = (K + kBK - 1) / kBK;
    const int64_t np_n = (kt_n + 1) / 2, np_full = K / (2 * kBK);
    auto dma = [&](auto pb, auto whole, int64_t p) {
        constexpr int P = decltype(pb)::value;
        constexpr bool WHOLE = decltype(whole)::value != 0;
        const int64_t k0 = p * 2 * kBK;
        const __amdgpu_buffer_rsrc_t ra = rsrc(A + m0 * lda + k0, ((M - 1 - m0) * lda + K - k0) * 2);
        const __amdgpu_buffer_rsrc_t rb = rsrc(B + n0 * ldb + k0, ((N - 1 - n0) * ldb + K - k0) * 2);
#pragma unroll
        for (int n = 0; n < NPA; ++n) {
            const uint32_t o = !WHOLE && k0 + kp_kofs(wave, lane, n) >= K ? kOOB : va[n];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (ZS_LDS void *)(Ab(IC<P>{}) + (wave + kNW * n) * 1024), 16, o, 0, 0, 0);
        }
#pragma unroll
        for (int n = 0; n < NPB; ++n) {
            const uint32_t o = !WHOLE && k0 + kp_kofs(wave, lane, n) >= K ? kOOB : vb[n];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (ZS_LDS void *)(Bb(IC<P>{}) + (wave + kNW * n) * 1024), 16, o, 0, 0, 0);
        }
    };
    bf16x8 fa[2][TM], fb[2][TN];
    // fragments of a tile held in pair buffer P, half H, into set F
    auto frags = [&](auto pb, auto hb, auto set) {
        constexpr int P = decltype(pb)::value, H = decltype(hb)::value, F = decltype(set)::value;
#pragma unroll
        for (int j = 0; j < TN; ++j)
            fb[F][j] = *reinterpret_cast<const ZS_LDS bf16x8 *>(Bb(IC<P>{}) + fb_off[H] + j * 2048);
#pragma unroll
        for (int i = 0; i < TM; ++i)
            fa[F][i] = *reinterpret_cast<const ZS_LDS bf16x8 *>(Ab(IC<P>{}) + fa_off[H] + i * 2048);
    };
    auto mma = [&](auto set) {
        constexpr int F = decltype(set)::value;
#pragma unroll
        for (int q = 0; q < NMF; ++q)
            acc[q / TN][q % TN] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[F][q / TN], fb[F][q % TN], acc[q / TN][q % TN], 0, 0, 0);
    };
    // Tile kt (TI = kt mod 4): odd tiles wait for tile kt + 1's pair and
    // their own fragment reads, then a barrier: after it every wave's part of
    // that pair has landed and no wave still reads the buffer the pair
    // before it used, so the DMA of the pair two ahead goes there.  Even
    // tiles only wait for their own reads: tile kt + 1 is the other half of
    // the pair already in place, and no DMA is issued, so they need no
    // barrier (paired on the dX shape: 1.022 x faster, bit-identical).
    // Read tile kt + 1's fragments under tile kt's MFMAs.
    auto tile = [&](auto ti, auto steady, int64_t kt) {
        constexpr int TI = decltype(ti)::value;
        constexpr bool STEADY = decltype(steady)::value != 0;
        constexpr bool ODD = TI & 1;
        constexpr int F = TI & 1;
        constexpr int T1 = (TI + 1) & 3;                 // tile kt + 1 mod 4
        constexpr int P1 = (T1 >> 1) & 1, H1 = T1 & 1;   // its buffer and half
        constexpr int PN = (((TI + 3) >> 1)) & 1;        // buffer of pair (kt + 3) / 2
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ODD) {
            wait_vm_lgkm0<0>();
            __builtin_amdgcn_s_barrier();
        } else {
            wait_vm_lgkm0<DP>();
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ODD) {
            const int64_t p = (kt + 3) / 2;
            if constexpr (STEADY)
                dma(IC<PN>{}, IC<1>{}, p);
            else if (p < np_n)
                dma(IC<PN>{}, IC<0>{}, p);
        }
        if (STEADY || kt + 1 < kt_n)
            frags(IC<P1>{}, IC<H1>{}, IC<F ^ 1>{});
        mma(IC<F>{});
        if constexpr (STEADY && ODD)
            seq<NF, NMF, NF, DP>();
        else
            seq<NF, NMF, NF, 0>();
    };
    if (kt_n > 0) {
        dma(IC<0>{}, IC<0>{}, 0);
        if (np_n > 1) {
            dma(IC<1>{}, IC<0>{}, 1);
            wait_vm_lgkm0<DP>();
        } else {
            wait_vm_lgkm0<0>();
        }
        __builtin_amdgcn_s_barrier();
        frags(IC<0>{}, IC<0>{}, IC<0>{});
        int64_t kt = 0;
        // steady: the pairs this group issues, (kt + 4) / 2 and (kt + 6) / 2,
        // lie inside K
        for (; (kt + 6) / 2 < np_full; kt += 4) {
            tile(IC<0>{}, IC<1>{}, kt);
            tile(IC<1>{}, IC<1>{}, kt + 1);
            tile(IC<2>{}, IC<1>{}, kt + 2);
            tile(IC<3>{}, IC<1>{}, kt + 3);
        }
        for (; kt < kt_n; kt += 4) {
            tile(IC<0>{}, IC<0>{}, kt);
            if (kt + 1 < kt_n) tile(IC<1>{}, IC<0>{}, kt + 1);
            if (kt + 2 < kt_n) tile(IC<2>{}, IC<0>{}, kt + 2);
            if (kt + 3 < kt_n) tile(IC<3>{}, IC<0>{}, kt + 3);
        }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t row = m0 + wm + 16 * i + 4 * g + v;
                const int64_t col = n0 + wn + 16 * j + r16;
                if (row < M && col < N) {
                    if (OUT_BF16)
                        static_cast<uint16_t *>(C)[row * ldc + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][v]);
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
    // One array per stage and operand, so the compiler can tell the LDS a
    // DMA writes from the LDS the fragment reads use.
    __shared__ __attribute__((aligned(1024))) char a0[kStage], a1[kStage], a2[kStage], a3[kStage];
    __shared__ __attribute__((aligned(1024))) char b0[kStage], b1[kStage], b2[kStage], b3[kStage];
    ZS_LDS char *const As[kStages] = {(ZS_LDS char *)a0, (ZS_LDS char *)a1, (ZS_LDS char *)a2,
                                      (ZS_LDS char *)a3};
    ZS_LDS char *const Bs[kStages] = {(ZS_LDS char *)b0, (ZS_LDS char *)b1, (ZS_LDS char *)b2,
                                      (ZS_LDS char *)b3};
    const int b = blockIdx.x;
    int tm, tn;
    if (b < n_big) {
        grouped(xcd_order(b, n_big), tiles_m, tiles_n, tm, tn);
        gemm_tile<kBM, A_KOUTER, B_KOUTER, OUT_BF16>(M, N, K, A, lda, B, ldb, C, ldc,
                                                     (int64_t)tm * kBM, (int64_t)tn * kBN, As,
                                                     Bs);
    } else {
        const int h = xcd_order(b - n_big, (int)gridDim.x - n_big);
        grouped(n_big + h / 2, tiles_m, tiles_n, tm, tn);
        const int64_t hm0 = (int64_t)tm * kBM + (h & 1) * (kBM / 2);
        gemm_tile<kBM / 2, A_KOUTER, B_KOUTER, OUT_BF16>(M, N, K, A, lda, B, ldb, C, ldc, hm0,
                                                         (int64_t)tn * kBN, As, Bs);
    }
}

// The both-K-inner order: gemm_tile_kp with its pair buffers, whole tiles and
// half tiles as in gemm_kernel.
template <bool OUT_BF16>
__global__ __launch_bounds__(kGT) void gemm_kernel_kp(int64_t M, int64_t N, int64_t K,
                                                      const uint16_t *__restrict__ A, int64_t lda,
                                                      const uint16_t *__restrict__ B, int64_t ldb,
                                                      void *__restrict__ C, int64_t ldc, int tiles_m,
                                                      int tiles_n, int n_big)
{
    __shared__ __attribute__((aligned(1024))) char pa0[kPair], pa1[kPair];
    __shared__ __attribute__((aligned(1024))) char pb0[kPair], pb1[kPair];
    const int b = blockIdx.x;
    int tm, tn;
    if (b < n_big) {
        grouped(xcd_order(b, n_big), tiles_m, tiles_n, tm, tn);
        gemm_tile_kp<kBM, OUT_BF16>(M, N, K, A, lda, B, ldb, C, ldc, (int64_t)tm * kBM,
                                    (int64_t)tn * kBN, (ZS_LDS char *)pa0, (ZS_LDS char *)pa1,
                                    (ZS_LDS char *)pb0, (ZS_LDS char *)pb1);
    } else {
        const int h = xcd_order(b - n_big, (int)gridDim.x - n_big);
        grouped(n_big + h / 2, tiles_m, tiles_n, tm, tn);
        const int64_t hm0 = (int64_t)tm * kBM + (h & 1) * (kBM / 2);
        gemm_tile_kp<kBM / 2, OUT_BF16>(M, N, K, A, lda, B, ldb, C, ldc, hm0, (int64_t)tn * kBN,
                                        (ZS_LDS char *)pa0, (ZS_LDS char *)pa1, (ZS_LDS char *)pb0,
                                        (ZS_LDS char *)pb1);
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

// Compute units of the current device, cached per device (atomics: calls
// may come from several host threads at once).
int cu_count()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        dev = -1;
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0)
            return c;
    }
    int n = 0;
    if (dev < 0 || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                       hipSuccess || n <= 0)
        n = 256;
    if (dev >= 0 && dev < 64)
        cache[dev].store(n, std::memory_order_relaxed);
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

namespace zs {

// Every argument check of zero_gemm_bf16, with nothing launched; composite
// calls (the FSDP linear layer) run it for each of their GEMMs before their
// first launch.
zero_status gemm_check(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                       int32_t a_order, const uint16_t *B, int64_t ldb, int32_t b_order,
                       const void *C, int64_t ldc, int32_t c_dtype)
{
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
    // The kernel reads a K-inner operand's 256-row panel (at most 510 ld + 64
    // bytes from its start) and a K-outer operand's 32 k rows (at most
    // 62 ld + 512) through 32-bit buffer offsets below 2^31.
    const int64_t ki_max = int64_t(1) << 22, ko_max = int64_t(1) << 25;
    if (lda > (ao ? ko_max : ki_max) || ldb > (bo ? ko_max : ki_max))
        return fail(ZERO_ERR_UNSUPPORTED, "leading dimension too large for 32-bit operand offsets "
                    "(lda %lld, ldb %lld; K-inner at most %lld, K-outer at most %lld)",
                    (long long)lda, (long long)ldb, (long long)ki_max, (long long)ko_max);
    // The dispatch counts the grid in work-items, 32 bits wide, and the grid
    // has up to two blocks per tile.
    const int64_t tm = (M + zs::kBM - 1) / zs::kBM, tn = (N + zs::kBN - 1) / zs::kBN;
    constexpr int64_t kMaxTiles = int64_t(0xffffffffu) / (2 * zs::kGT);
    if (tm > kMaxTiles / tn)
        return fail(ZERO_ERR_UNSUPPORTED, "too many GEMM tiles for one launch (%lld x %lld)",
                    (long long)tm, (long long)tn);
    if (!zs::a16(A) || !zs::a16(B))
        return fail(ZERO_ERR_ALIGNMENT, "A and B must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(C) % (c_dtype == ZERO_BF16 ? 2 : 4))
        return fail(ZERO_ERR_ALIGNMENT, "C is misaligned");
    return ZERO_OK;
}

}  // namespace zs

extern "C" {

zero_status zero_gemm_bf16(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                           int32_t a_order, const uint16_t *B, int64_t ldb, int32_t b_order,
                           void *C, int64_t ldc, int32_t c_dtype, void *stream)
{
    const zero_status st = zs::gemm_check(M, N, K, A, lda, a_order, B, ldb, b_order, C, ldc,
                                          c_dtype);
    if (st != ZERO_OK || M == 0 || N == 0)
        return st;
    const bool ao = a_order == ZERO_K_OUTER, bo = b_order == ZERO_K_OUTER;
    const int64_t tm = (M + zs::kBM - 1) / zs::kBM, tn = (N + zs::kBN - 1) / zs::kBN;
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
    case 0:
        hipLaunchKernelGGL((zs::gemm_kernel_kp<false>), grid, block, 0, s, M, N, K, A, lda, B, ldb,
                           C, ldc, (int)tm, (int)tn, (int)n_big);
        break;
    case 4:
        hipLaunchKernelGGL((zs::gemm_kernel_kp<true>), grid, block, 0, s, M, N, K, A, lda, B, ldb,
                           C, ldc, (int)tm, (int)tn, (int)n_big);
        break;
    case 1: ZS_GEMM(true, false, false); break;
    case 2: ZS_GEMM(false, true, false); break;
    case 3: ZS_GEMM(true, true, false); break;
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
    if ((rows + zs::kTT - 1) / zs::kTT > 65535 ||
        (cols + zs::kTT - 1) / zs::kTT > int64_t(0xffffffffu) / 256)
        return fail(ZERO_ERR_UNSUPPORTED, "transpose too large for one launch");
    const dim3 grid((unsigned)((cols + zs::kTT - 1) / zs::kTT),
                    (unsigned)((rows + zs::kTT - 1) / zs::kTT));
    (void)hipGetLastError();
    hipLaunchKernelGGL(zs::transpose_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                       rows, cols, src, lds, dst, ldd);
    return zs::launched("transpose");
}

}  // extern "C"
