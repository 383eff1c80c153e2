// HIP kernels (gfx950 / CDNA4) and compute entry points of libzeroshard.
//
// Everything here is HBM-bound streaming: per shard element the fused step
// reads N gradients (2N bytes bf16 or 4N fp32) and the fp32 master, m, v
// (12 bytes), and writes master, m, v (12) and the bf16 parameter (2), for
// about N + 20 flops -- far below the machine balance, so there is no
// contraction and no MFMA.  The design rules that matter are the memory ones:
//   * the step kernel walks 1024-element tiles in 256-thread blocks, each
//     lane owning one group of 4 consecutive elements, so that every load /
//     store instruction of a wave covers one contiguous run (fp32 streams in
//     128-bit accesses, bf16 streams in 64-bit ones) and whole lines are
//     written by one instruction -- rocprof FETCH_SIZE / WRITE_SIZE equal the
//     algorithmic bytes; the gather and the accumulation walk 2048-element
//     tiles;
//   * the step kernel runs at most 5 blocks (20 waves) per CU (3 in its
//     N = 64 specialisation) and the gather at most 13 (26 waves): fewer
//     requests in flight mix the read and write streams better; the
//     read-dominated reduce pass runs uncapped (measured below, at
//     launch_one and at the gather launch);
//   * one pass: the reduce over ranks, the Adam update and the bf16 cast are
//     fused so each byte crosses HBM once;
//   * one launch covers a tile space that concatenates the slices of many
//     units (FSDP layers, gradient buckets), so small units do not pay one
//     launch and one ramp-down each; by default one block per tile (see
//     blocks_per_cu_override for the measurement behind that choice), with
//     the tiles dealt to the 8 XCDs in contiguous ranges (tile_walk);
//   * the N rank streams are loaded in groups of 8 before they are summed,
//     keeping 8 loads per thread in flight without holding all N.
//
// Arithmetic (identical on every launch shape): fp32, one rounding per
// operation, no contraction into FMA (pragma below plus -ffp-contract=off),
// IEEE division and square root (the compiler's correctly-rounded
// sequences), rank sum in ascending order from +0 then divided by N (times
// the exact reciprocal when N is a power of two, which rounds identically).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstddef>
#include <cstdlib>
#include <cstring>

#include "internal.h"

#pragma clang fp contract(off)

namespace zs {
namespace {

constexpr int kTile = 2048;                 // elements per gather / accumulate tile
constexpr int kVec = 8;                     // gather: bf16 elements per 16-byte chunk
constexpr int kMaxSegs = 32;                // units per launch (kernarg table)
constexpr int kStepTile = 1024;             // elements per step-kernel tile
constexpr int kStepThreads = 256;           // step kernel: one 4-element group per lane
constexpr int kStepBlocksPerCU = 5;         // step kernel occupancy cap (LDS reservation)
constexpr int kStep64BlocksPerCU = 3;       // the same for the N = 64 specialisation
constexpr int kGatherBlocksPerCU = 13;      // gather occupancy cap (LDS reservation)
constexpr int kAccThreads = 512;            // accumulate: one 4-element group per lane
constexpr int kWaveElems = 256;             // elements one wave covers (64 lanes x 4)
static_assert(kStepTile == kStepThreads * 4 && kTile == kAccThreads * 4, "one group per lane");
constexpr int kClipThreads = 1024;          // one block sums the clip partials
constexpr int kMaxRanks = ZERO_MAX_RANKS_PER_CALL;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// One unit's slice inside a launch's tile space.
struct Seg {
    int64_t len;        // s_u: elements of the slice
    int64_t shard_off;  // R_u - R_begin: slice start in shard-indexed buffers
    int64_t full_off;   // (F_u - F_begin) + r*s_u: slice start in full buffers
    int64_t tile0;      // first tile of this slice
    int64_t vec;        // 1 if both offsets are multiples of 4 (vector path)
};

// The step scalars; the same layout as zero_adam_table_entry, so a table of
// them in device memory can be read as is.
struct AdamScalars {
    float lr, b1, b2, eps, wd;
    float omb1, omb2, bias1, bias2, decay;
    int32_t has_wd, decoupled;
};
static_assert(sizeof(AdamScalars) == sizeof(zero_adam_table_entry), "table entry layout");
static_assert(offsetof(AdamScalars, omb1) == offsetof(zero_adam_table_entry, one_minus_beta1) &&
                  offsetof(AdamScalars, decay) == offsetof(zero_adam_table_entry, decay) &&
                  offsetof(AdamScalars, has_wd) == offsetof(zero_adam_table_entry, has_decay) &&
                  offsetof(AdamScalars, decoupled) == offsetof(zero_adam_table_entry, decoupled),
              "table entry layout");

// kFused / kReduce / kApply are the optimizer step's passes.  The last
// three measure HBM rates of the fused pass's exact streams, tile walk and
// launch shape with the Adam arithmetic taken out (zero_stream_mix).
enum Mode { kFused = 0, kReduce = 1, kApply = 2, kMix = 3, kReadOnly = 4, kWriteOnly = 5 };

struct StepArgs {
    const void *grads[kMaxRanks];
    uint64_t full_mask;  // bit q: rank q's buffer is full-indexed
    int32_t n_ranks;
    int32_t n_segs;
    int64_t n_tiles;
    float inv_n;         // exact 1/N when N is a power of two
    float n_f;           // (float)N
    int32_t pow2;
    int32_t vec_ptrs;    // every base pointer is 16-byte aligned
    float *master, *m, *v;
    int64_t st_base;     // chunked state: shard index of the range's first element
    int32_t st_shift;    // 0: three state arrays; else log2 of the state chunk
    int32_t g_shift;     // 0: one buffer per rank; else log2 of the gradient chunk
    const float *gin;    // kApply: averaged gradient
    int32_t gin_full;    // kApply: 1 if gin is full-indexed, 0 if shard-indexed
    int32_t _pad2;
    const float *clip;   // kApply: device clip coefficient or null
    float *gout;         // kReduce: averaged gradient
    int32_t gout_full;   // kReduce: 1 if gout is full-indexed, 0 if shard-indexed
    int32_t _pad3;
    double *partials;    // kReduce: one fp64 sum of squares per tile, or null
    uint16_t *pout;      // bf16 parameter output
    int32_t pout_full;   // 1: full-indexed, 0: shard-indexed
    float sink_key;      // kReadOnly: a value no element equals (NaN)
    AdamScalars sc;
    const AdamScalars *table;  // non-null: scalars from table[*step - 1] instead of sc
    const int64_t *step;
    int64_t n_table;
    Seg seg[kMaxSegs];
};

// ------------------------------------------------------------ helpers --

// Tiles a block walks.  The default launch has one block per tile.  With
// `by_xcd`, the tiles are dealt out so that each XCD (block b runs on XCD
// b % 8) gets a contiguous eighth of the tile space, walked in order: each
// XCD's L2 and address translation then see one compact window per stream
// instead of a slice of every window.  Paired runs (same process, same
// buffers) measured it 2-4 % faster for the gather and the fp32
// accumulation, 1.4 % for the fused bf16 step (up to 2 % where the buffer
// placement was slow), neutral for the reduce and the fp32 fused step, and
// 1-5 % slower for the apply pass, which therefore keeps the plain order.
// A persistent width (ZERO_SHARD_BLOCKS_PER_CU) walks the tiles with a grid
// stride instead.  Every tile is visited exactly once.
struct TileWalk {
    int64_t t, end, stride;
};

__device__ __forceinline__ TileWalk tile_walk(int64_t n_tiles, bool by_xcd)
{
    if (by_xcd && (int64_t)gridDim.x == n_tiles) {
        const int64_t i = blockIdx.x, per = n_tiles / 8, rem = n_tiles % 8, x = i % 8;
        const int64_t t = x * per + (x < rem ? x : rem) + i / 8;
        return {t, t + 1, 1};
    }
    return {(int64_t)blockIdx.x, n_tiles, (int64_t)gridDim.x};
}

// The segment holding tile t: the last s with seg[s].tile0 <= t (seg[0].tile0
// is 0).  A binary search -- at most 5 dependent scalar loads for 32
// segments -- because with one block per tile every block looks its segment
// up from scratch, and for a light kernel (the gather moves 16 bytes per
// thread) a linear scan over the table costs more than the copy.
template <typename SegT>
__device__ __forceinline__ int find_seg(const SegT *seg, int n_segs, int64_t t)
{
    int lo = 0, hi = n_segs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seg[mid].tile0 <= t)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// IEEE round to nearest even on bit 16; every NaN becomes 0x7FC0.
__device__ __forceinline__ uint32_t to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <typename T>
__device__ __forceinline__ T ld_nt(const T *p) { return __builtin_nontemporal_load(p); }
template <typename T>
__device__ __forceinline__ void st_nt(T *p, T x) { __builtin_nontemporal_store(x, p); }

__device__ __forceinline__ void adam1(const AdamScalars &s, float g, float &p, float &m, float &v)
{
    if (s.has_wd) {
        if (s.decoupled)
            p = p * s.decay;
        else
            g = g + s.wd * p;
    }
    m = s.b1 * m + s.omb1 * g;
    v = s.b2 * v + s.omb2 * (g * g);
    const float m_hat = m / s.bias1;
    const float v_hat = v / s.bias2;
    const float denom = sqrtf(v_hat) + s.eps;
    p = p - s.lr * (m_hat / denom);
}

__device__ __forceinline__ float mean_of(const StepArgs &a, float sum)
{
    return a.pow2 ? sum * a.inv_n : sum / a.n_f;
}

// Offset of shard element `si` (relative to the range) in master, m and v.
// Three arrays: si itself.  Chunked state (chunk E = 2^st_shift): element
// i = st_base + si sits at (i / E) 3E + i % E from master (m and v are
// master + E and master + 2E).  A 4-aligned group of 4 never crosses a
// chunk, so the vector path keeps one 16-byte access per lane and stream.
__device__ __forceinline__ int64_t st_at(const StepArgs &a, int64_t si)
{
    if (a.st_shift == 0)
        return si;
    const int64_t i = a.st_base + si;
    const int sh = a.st_shift;
    return ((i >> sh) * 3 << sh) + (i & (((int64_t)1 << sh) - 1));
}

// Offset of shard element `si` (relative to the range) in a shard-indexed
// rank gradient.  One buffer per rank: si itself.  Chunked gradients (chunk
// E = 2^g_shift, N ranks in one buffer): element si of rank q sits at
// (si / E) N E + si % E from rank q's pointer, which is rank 0's + qE.  A
// group of 4 at a 4-aligned si never crosses a chunk.
__device__ __forceinline__ int64_t g_at(const StepArgs &a, int n, int64_t si)
{
    if (a.g_shift == 0)
        return si;
    const int sh = a.g_shift;
    return ((si >> sh) * n << sh) + (si & (((int64_t)1 << sh) - 1));
}

// Sum of the N rank gradients for G groups of 4 consecutive elements, group
// h at shard index si[h] / full index fi[h] (vector path).  Each rank is
// added in ascending order, from +0.
template <int NR, bool BF16, int G>
__device__ __forceinline__ void reduce_groups(const StepArgs &a, const int64_t *si,
                                              const int64_t *fi, float (*acc)[4])
{
    const int n = NR > 0 ? NR : a.n_ranks;
    int64_t gi[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        gi[h] = g_at(a, n, si[h]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc[h][e] = 0.0f;
    }
    // one group of 8 rank loads in flight per thread; other waves hide the
    // latency between groups (unrolling further only raises register use)
#pragma unroll 1
    for (int q0 = 0; q0 < n; q0 += 8) {
        if (BF16) {
            u32x2 w[8][G];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int q = q0 + k;
                if (q < n) {
                    const bool full = (a.full_mask >> q) & 1;
                    const uint16_t *base = static_cast<const uint16_t *>(a.grads[q]);
#pragma unroll
                    for (int h = 0; h < G; ++h)
                        w[k][h] = ld_nt(reinterpret_cast<const u32x2 *>(base + (full ? fi[h] : gi[h])));
                }
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (q0 + k < n) {
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        acc[h][0] = acc[h][0] + bf16lo(w[k][h].x);
                        acc[h][1] = acc[h][1] + bf16hi(w[k][h].x);
                        acc[h][2] = acc[h][2] + bf16lo(w[k][h].y);
                        acc[h][3] = acc[h][3] + bf16hi(w[k][h].y);
                    }
                }
            }
        } else {
            f32x4 w[8][G];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int q = q0 + k;
                if (q < n) {
                    const bool full = (a.full_mask >> q) & 1;
                    const float *base = static_cast<const float *>(a.grads[q]);
#pragma unroll
                    for (int h = 0; h < G; ++h)
                        w[k][h] = ld_nt(reinterpret_cast<const f32x4 *>(base + (full ? fi[h] : gi[h])));
                }
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (q0 + k < n) {
#pragma unroll
                    for (int h = 0; h < G; ++h)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[h][e] = acc[h][e] + w[k][h][e];
                }
            }
        }
    }
}

// Sum of the N rank gradients for one element (scalar path).
template <int NR, bool BF16>
__device__ __forceinline__ float reduce1(const StepArgs &a, int64_t si, int64_t fi)
{
    const int n = NR > 0 ? NR : a.n_ranks;
    float acc = 0.0f;
    const int64_t gi = g_at(a, n, si);
    for (int q = 0; q < n; ++q) {
        const int64_t i = ((a.full_mask >> q) & 1) ? fi : gi;
        const float x = BF16 ? bf16f(static_cast<const uint16_t *>(a.grads[q])[i])
                             : static_cast<const float *>(a.grads[q])[i];
        acc = acc + x;
    }
    return acc;
}

// Wave-wide fp64 sum in a fixed butterfly order; every lane gets the total.
__device__ __forceinline__ double wave_sum(double x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x = x + __shfl_xor(x, off, 64);
    return x;
}

// Block-wide fp64 sum in a fixed order (wave butterflies, then the waves in
// order); the total is valid in thread 0.  Ends with a barrier so the LDS
// slots can be reused by the next call.
template <int THREADS>
__device__ double block_sum(double x)
{
    __shared__ double lds[THREADS / 64];
    x = wave_sum(x);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
        lds[wave] = x;
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x == 0)
        for (int w = 0; w < THREADS / 64; ++w)
            t = t + lds[w];
    __syncthreads();
    return t;
}

// -------------------------------------------------------- step kernel --
//
// Element ownership in a 1024-element tile: the step kernel runs 256-thread
// blocks; wave w covers [256w, 256w + 256) and lane l owns the 4-element
// group at 256w + 4l.  Every load or store instruction of a wave therefore
// covers one contiguous run -- 512 bytes of a bf16 stream, 1 KiB of an fp32
// stream -- so caches and HBM see whole lines written by one instruction.
// (With 8 contiguous elements per lane, each 16-byte fp32 store instruction
// filled only every other 16 bytes of its span and lines were written back
// in halves; 8 elements per lane with 128-bit bf16 loads and a
// v_permlane32_swap hand-off that keeps the fp32 instructions on whole lines
// measured 1.6 % slower than this.)  One group per lane keeps the kernel near
// 55 VGPRs; two groups per lane (91 VGPRs) measured 2-3 % slower.

// The fused / reduce / apply work for G full groups of 4 elements.
template <int MODE, int NR, bool BF16, int G>
__device__ __forceinline__ void step_groups(const StepArgs &a, const AdamScalars &sc,
                                            const Seg &sg, const int64_t *j,
                                            float coef, double &sq)
{
    int64_t si[G], fi[G], xi[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        si[h] = sg.shard_off + j[h];
        fi[h] = sg.full_off + j[h];
        xi[h] = st_at(a, si[h]);
    }
    float p[G][4], m[G][4], v[G][4], g[G][4];
    if constexpr (MODE == kWriteOnly) {
        // the fused pass's four write streams, with values from the index
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float x = (float)j[h];
            st_nt(reinterpret_cast<f32x4 *>(a.master + xi[h]), f32x4{x, x, x, x});
            st_nt(reinterpret_cast<f32x4 *>(a.m + xi[h]), f32x4{x, x, x, x});
            st_nt(reinterpret_cast<f32x4 *>(a.v + xi[h]), f32x4{x, x, x, x});
            st_nt(reinterpret_cast<u32x2 *>(a.pout + (a.pout_full ? fi[h] : si[h])),
                  u32x2{(uint32_t)j[h], (uint32_t)j[h]});
        }
        return;
    }
    if (MODE != kReduce) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const f32x4 pv = ld_nt(reinterpret_cast<const f32x4 *>(a.master + xi[h]));
            const f32x4 mv = ld_nt(reinterpret_cast<const f32x4 *>(a.m + xi[h]));
            const f32x4 vv = ld_nt(reinterpret_cast<const f32x4 *>(a.v + xi[h]));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p[h][e] = pv[e];
                m[h][e] = mv[e];
                v[h][e] = vv[e];
            }
        }
    }
    if (MODE == kApply) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const f32x4 gv =
                ld_nt(reinterpret_cast<const f32x4 *>(a.gin + (a.gin_full ? fi[h] : si[h])));
#pragma unroll
            for (int e = 0; e < 4; ++e)
                g[h][e] = gv[e] * coef;
        }
    } else {
        float acc[G][4];
        reduce_groups<NR, BF16, G>(a, si, fi, acc);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                g[h][e] = MODE >= kMix ? acc[h][e] : mean_of(a, acc[h][e]);
    }
    if constexpr (MODE == kReadOnly) {
        // every loaded value feeds a comparison the host makes false
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = ((g[h][e] + p[h][e]) + m[h][e]) + v[h][e];
                if (x == a.sink_key)
                    a.master[xi[h] + e] = x;
            }
        return;
    }
    if (MODE == kReduce) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sq = sq + (double)g[h][e] * (double)g[h][e];
            st_nt(reinterpret_cast<f32x4 *>(a.gout + (a.gout_full ? fi[h] : si[h])),
                  f32x4{g[h][0], g[h][1], g[h][2], g[h][3]});
        }
        return;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (MODE == kMix) {
                p[h][e] = p[h][e] + g[h][e];
                m[h][e] = m[h][e] + g[h][e];
                v[h][e] = v[h][e] + g[h][e];
            } else {
                adam1(sc, g[h][e], p[h][e], m[h][e], v[h][e]);
            }
        }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        st_nt(reinterpret_cast<f32x4 *>(a.master + xi[h]), f32x4{p[h][0], p[h][1], p[h][2], p[h][3]});
        st_nt(reinterpret_cast<f32x4 *>(a.m + xi[h]), f32x4{m[h][0], m[h][1], m[h][2], m[h][3]});
        st_nt(reinterpret_cast<f32x4 *>(a.v + xi[h]), f32x4{v[h][0], v[h][1], v[h][2], v[h][3]});
        u32x2 w;
        if constexpr (MODE == kMix) {
            // the upper halves: a bf16 stream without the rounding
            w.x = (__float_as_uint(p[h][0]) >> 16) | (__float_as_uint(p[h][1]) & 0xffff0000u);
            w.y = (__float_as_uint(p[h][2]) >> 16) | (__float_as_uint(p[h][3]) & 0xffff0000u);
        } else {
            w.x = to_bf16(p[h][0]) | (to_bf16(p[h][1]) << 16);
            w.y = to_bf16(p[h][2]) | (to_bf16(p[h][3]) << 16);
        }
        st_nt(reinterpret_cast<u32x2 *>(a.pout + (a.pout_full ? fi[h] : si[h])), w);
    }
}

// The same work one element at a time: ragged tails and unaligned slices.
template <int MODE, int NR, bool BF16>
__device__ __forceinline__ void step_scalar(const StepArgs &a, const AdamScalars &sc,
                                            const Seg &sg, int64_t j,
                                            int64_t cnt, float coef, double &sq)
{
    if constexpr (MODE >= kMix) {
        return;  // zero_stream_mix accepts whole 16-byte aligned groups only
    } else {
    const int64_t si = sg.shard_off + j;
    const int64_t fi = sg.full_off + j;
    const int64_t oi = a.pout_full ? fi : si;
    for (int64_t e = 0; e < cnt; ++e) {
        float g;
        if (MODE == kApply)
            g = a.gin[(a.gin_full ? fi : si) + e] * coef;
        else
            g = mean_of(a, reduce1<NR, BF16>(a, si + e, fi + e));
        if (MODE == kReduce) {
            a.gout[(a.gout_full ? fi : si) + e] = g;
            sq = sq + (double)g * (double)g;
        } else {
            const int64_t x = st_at(a, si + e);
            float p = a.master[x], m = a.m[x], v = a.v[x];
            adam1(sc, g, p, m, v);
            a.master[x] = p;
            a.m[x] = m;
            a.v[x] = v;
            a.pout[oi + e] = (uint16_t)to_bf16(p);
        }
    }
    }
}

template <int MODE, int NR, bool BF16>
__global__ __launch_bounds__(kStepThreads) void step_kernel(const StepArgs a)
{
    AdamScalars sc = a.sc;
    if (MODE != kReduce && a.table) {
        // the whole grid reads one counter: a value outside the table
        // leaves every buffer untouched
        const int64_t t = *a.step;
        if (t < 1 || t > a.n_table)
            return;
        sc = a.table[t - 1];
    }
    const float coef = (MODE == kApply && a.clip) ? *a.clip : 1.0f;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const TileWalk tw = tile_walk(a.n_tiles, MODE != kApply);
    for (int64_t t = tw.t; t < tw.end; t += tw.stride) {
        const Seg &sg = a.seg[find_seg(a.seg, a.n_segs, t)];
        const int64_t j[1] = {(t - sg.tile0) * kStepTile + wave * kWaveElems + lane * 4};
        const bool vec = sg.vec && a.vec_ptrs;
        double sq = 0.0;  // kReduce: this thread's sum of squares in this tile
        if (j[0] < sg.len) {
            if (vec && j[0] + 4 <= sg.len)
                step_groups<MODE, NR, BF16, 1>(a, sc, sg, j, coef, sq);
            else
                step_scalar<MODE, NR, BF16>(a, sc, sg, j[0], sg.len - j[0] < 4 ? sg.len - j[0] : 4,
                                            coef, sq);
        }
        if (MODE == kReduce && a.partials) {
            // every thread takes part; threads past the slice end add 0
            const double b = block_sum<kStepThreads>(sq);
            if (threadIdx.x == 0)
                a.partials[t] = b;
        }
    }
}

// ------------------------------------------------------ gather kernel --

struct GSeg {
    int64_t len;        // s_u
    int64_t shard_off;  // R_u - R_begin
    int64_t flat_base;  // F_u - F_begin
    int64_t tile0;
    int64_t vec;        // len, shard_off, flat_base all multiples of 8
};

struct GatherArgs {
    const uint16_t *src[kMaxRanks];
    int32_t rank_of[kMaxRanks];
    int32_t n_src;
    int32_t n_segs;
    int64_t n_tiles;
    uint16_t *dst;
    int32_t vec_ptrs;
    int32_t _pad;
    GSeg seg[kMaxSegs];
};

// blockIdx.y selects the source rank; x walks the tiles of every slice.
// 128-thread blocks: thread i copies the 8-element chunks at 8i and
// 1024 + 8i of its tile (each wave instruction moves 1 KiB contiguous).
// Paired runs measured this 0.1-4.6 % faster for 7 sources and 0.6-1.1 %
// for 63 than 256 threads with one chunk each.
constexpr int kGatherThreads = 128;
__global__ __launch_bounds__(kGatherThreads) void gather_kernel(const GatherArgs a)
{
    const int y = blockIdx.y;
    const uint16_t *src = a.src[y];
    const int64_t q = a.rank_of[y];
    const TileWalk tw = tile_walk(a.n_tiles, true);
    for (int64_t t = tw.t; t < tw.end; t += tw.stride) {
        const GSeg &sg = a.seg[find_seg(a.seg, a.n_segs, t)];
#pragma unroll
        for (int h = 0; h < kTile / (kGatherThreads * kVec); ++h) {
            const int64_t j = (t - sg.tile0) * kTile + (int64_t)h * (kGatherThreads * kVec) +
                              (int64_t)threadIdx.x * kVec;
            if (j >= sg.len)
                continue;
            const int64_t si = sg.shard_off + j;
            const int64_t di = sg.flat_base + q * sg.len + j;
            if (sg.vec && a.vec_ptrs && j + kVec <= sg.len) {
                st_nt(reinterpret_cast<u32x4 *>(a.dst + di),
                      ld_nt(reinterpret_cast<const u32x4 *>(src + si)));
            } else {
                const int64_t cnt = (sg.len - j) < kVec ? (sg.len - j) : kVec;
                for (int64_t e = 0; e < cnt; ++e)
                    a.dst[di + e] = src[si + e];
            }
        }
    }
}

// ------------------------------------------------- accumulate kernel --

// 512-thread blocks, lane l of wave w owns the 4-element group at 256w + 4l
// of each 2048-element tile (paired runs on a 4e9-element buffer: 1.2-2 %
// faster than 256 threads with two groups per lane; capping its occupancy
// as the step kernel does measured 3.5-7 % slower).
__global__ __launch_bounds__(kAccThreads) void accumulate_kernel(float *acc,
                                                                  const uint16_t *micro,
                                                                  int64_t n, int32_t vec)
{
    const int64_t lane_off = (threadIdx.x >> 6) * kWaveElems + (threadIdx.x & 63) * 4;
    const TileWalk tw = tile_walk((n + kTile - 1) / kTile, true);
    for (int64_t t = tw.t; t < tw.end; t += tw.stride) {
        const int64_t i = t * kTile + lane_off;
        if (i >= n)
            continue;
        if (vec && i + 4 <= n) {
            f32x4 *ap = reinterpret_cast<f32x4 *>(acc + i);
            f32x4 x = ld_nt(ap);
            const u32x2 w = ld_nt(reinterpret_cast<const u32x2 *>(micro + i));
            x.x = x.x + bf16lo(w.x);
            x.y = x.y + bf16hi(w.x);
            x.z = x.z + bf16lo(w.y);
            x.w = x.w + bf16hi(w.y);
            st_nt(ap, x);
        } else {
            const int64_t cnt = (n - i) < 4 ? (n - i) : 4;
            for (int64_t e = 0; e < cnt; ++e)
                acc[i + e] = acc[i + e] + bf16f(micro[i + e]);
        }
    }
}

// ---------------------------------------------------- step counter --

// *step += 1, one lane (a graph node that advances the table step).
__global__ __launch_bounds__(64) void step_advance_kernel(int64_t *step)
{
    if (threadIdx.x == 0)
        *step = *step + 1;
}

// ------------------------------------------------------- clip kernel --

// One block of 1024 threads: thread i sums partials i, i + 1024, ... into
// kClipAcc independent fp64 accumulators (the k-th of its elements goes to
// accumulator k mod kClipAcc, so that many loads are in flight: the kernel
// is bound by load latency), adds them in order, then a fixed-order block
// sum.  The order is fixed for a given n, so the result is deterministic.
constexpr int kClipAcc = 16;
__global__ __launch_bounds__(kClipThreads) void clip_kernel(const double *partials, int64_t n,
                                                            float max_norm, float *coef,
                                                            double *norm_out)
{
    double s[kClipAcc];
#pragma unroll
    for (int k = 0; k < kClipAcc; ++k)
        s[k] = 0.0;
    int64_t i = threadIdx.x;
    for (; i + (kClipAcc - 1) * kClipThreads < n; i += kClipAcc * kClipThreads) {
#pragma unroll
        for (int k = 0; k < kClipAcc; ++k)
            s[k] = s[k] + partials[i + k * kClipThreads];
    }
    // fewer than kClipAcc elements of this thread remain
#pragma unroll
    for (int k = 0; k < kClipAcc; ++k)
        if (i + (int64_t)k * kClipThreads < n)
            s[k] = s[k] + partials[i + k * kClipThreads];
    double t = 0.0;
#pragma unroll
    for (int k = 0; k < kClipAcc; ++k)
        t = t + s[k];
    const double total = block_sum<kClipThreads>(t);
    if (threadIdx.x == 0) {
        const double norm = sqrt(total);
        const float c = (float)((double)max_norm / (norm + 1e-6));
        *coef = c < 1.0f ? c : 1.0f;
        if (norm_out)
            *norm_out = norm;
    }
}

// ------------------------------------------------------------- host --

// Compute units of the current device, cached per device (atomics: calls
// may come from several host threads at once).
int device_cus()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int cus = cached[dev].load(std::memory_order_relaxed);
    if (cus <= 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cached[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

// Launch width.  Default: one block per tile.  Measured on
// MI355X (7B / N = 8 step, paired runs over six buffer placements) this beat
// a persistent grid sized to the resident occupancy by 6 % on the fused
// kernel and 12 % on the gather: the dispatcher hands out blocks in tile
// order, which keeps the active window of every stream compact, and it
// balances the tail by itself.  ZERO_SHARD_BLOCKS_PER_CU=K (1..64) selects a
// persistent grid of K blocks per CU instead (0 = the default).  Read once.
int blocks_per_cu_override()
{
    static int v = [] {
        const char *e = std::getenv("ZERO_SHARD_BLOCKS_PER_CU");
        if (!e || !*e)
            return 0;
        const int x = std::atoi(e);
        return (x >= 0 && x <= 64) ? x : 0;
    }();
    return v;
}

template <typename Kernel>
int resident_blocks(Kernel kernel, int threads, size_t lds = 0)
{
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, threads, lds) != hipSuccess ||
        nb < 1)
        nb = 4;
    return nb;
}

// `resident` (blocks of the kernel that fit on one CU) caps the persistent
// width so a persistent grid is fully resident from the start.  The
// dispatch packet counts a grid dimension in work-items, 32 bits wide, so
// blocks x threads must stay below 2^32.  Every kernel walks its tiles with
// a grid stride, so capping the width there keeps any tile count
// launchable.
int64_t stream_grid(int64_t n_tiles, int resident, int threads)
{
    const int o = blocks_per_cu_override();
    int64_t g = (int64_t)0xffffffffu / threads;
    if (o != 0) {
        const int64_t p = (int64_t)device_cus() * (o < resident ? o : resident);
        g = p < g ? p : g;
    }
    return n_tiles < g ? n_tiles : g;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t tiles_of(int64_t len) { return (len + kTile - 1) / kTile; }
int64_t step_tiles_of(int64_t len) { return (len + kStepTile - 1) / kStepTile; }

// LDS bytes reserved per block so that at most CAP blocks share a CU (the
// kernels themselves use no LDS beyond a few bytes for the clip partials).
// From the device's LDS per CU (160 KiB on gfx950: 32 KiB per step block,
// 12 KiB per gather block), cached per device.
template <int CAP>
size_t lds_reserve()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return (size_t)(((160 * 1024) / CAP) & ~1023);
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        int lds = 0;
        if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
                hipSuccess ||
            lds <= 0)
            lds = 160 * 1024;
        v = (lds / CAP) & ~1023;
        v = v > 64 * 1024 ? 64 * 1024 : (v < 1024 ? 1024 : v);
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return (size_t)v;
}


// Splits a unit range into launches of at most kMaxSegs units each and
// calls fn(first_unit, last_unit_exclusive).
template <typename F>
zero_status for_each_chunk(int32_t ub, int32_t ue, F fn)
{
    for (int32_t u0 = ub; u0 < ue; u0 += kMaxSegs) {
        const int32_t u1 = (ue - u0) > kMaxSegs ? u0 + kMaxSegs : ue;
        const zero_status st = fn(u0, u1);
        if (st != ZERO_OK)
            return st;
    }
    return ZERO_OK;
}

// Fills the segment table for units [u0, u1) of a call whose range starts
// at `ub`; returns the number of tiles.  `abs_index`: the launch addresses a
// chunked state by absolute shard index, so a slice takes the vector path
// only if its absolute shard offset is a multiple of 4 as well.
int64_t fill_segs(const zero_layout *L, int32_t ub, int32_t u0, int32_t u1, Seg *seg,
                  int32_t *n_segs, bool abs_index = false)
{
    int64_t tiles = 0;
    int32_t k = 0;
    for (int32_t u = u0; u < u1; ++u) {
        const int64_t len = L->slice[u];
        if (len == 0)
            continue;
        Seg &s = seg[k++];
        s.len = len;
        s.shard_off = L->shard_off[u] - L->shard_off[ub];
        s.full_off = L->flat_off[u] - L->flat_off[ub] + (int64_t)L->rank * len;
        s.tile0 = tiles;
        s.vec = (s.shard_off % 4 == 0 && s.full_off % 4 == 0 &&
                 (!abs_index || L->shard_off[u] % 4 == 0)) ? 1 : 0;
        tiles += step_tiles_of(len);
    }
    *n_segs = k;
    return tiles;
}

}  // namespace

zero_status check_grads(const zero_layout *L, const zero_grads *g)
{
    if (g->n != L->world_n)
        return fail(ZERO_ERR_INVALID_ARG, "grads->n = %d but the layout has world_n = %d", g->n,
                    L->world_n);
    if (g->n > kMaxRanks)
        return fail(ZERO_ERR_UNSUPPORTED, "at most %d rank buffers per call (got %d)", kMaxRanks,
                    g->n);
    if (g->dtype != ZERO_BF16 && g->dtype != ZERO_FP32)
        return fail(ZERO_ERR_INVALID_ARG, "unknown gradient dtype %d", g->dtype);
    if (!g->ptrs)
        return fail(ZERO_ERR_INVALID_ARG, "grads->ptrs is NULL");
    if (!g->index && g->index_all != ZERO_INDEX_FULL && g->index_all != ZERO_INDEX_SHARD)
        return fail(ZERO_ERR_INVALID_ARG, "unknown index_all %d", g->index_all);
    const uintptr_t elem = g->dtype == ZERO_BF16 ? 2 : 4;
    for (int q = 0; q < g->n; ++q) {
        if (!g->ptrs[q])
            return fail(ZERO_ERR_INVALID_ARG, "gradient buffer of rank %d is NULL (missing replica)",
                        q);
        if (reinterpret_cast<uintptr_t>(g->ptrs[q]) % elem)
            return fail(ZERO_ERR_ALIGNMENT, "gradient buffer of rank %d is misaligned", q);
        if (g->index && g->index[q] != ZERO_INDEX_FULL && g->index[q] != ZERO_INDEX_SHARD)
            return fail(ZERO_ERR_INVALID_ARG, "unknown index %d for rank %d", g->index[q], q);
    }
    if (g->chunk == 0)
        return ZERO_OK;
    const int64_t E = g->chunk;
    if (E < ZERO_STATE_CHUNK_MIN || E > ZERO_STATE_CHUNK_MAX || (E & (E - 1)))
        return fail(ZERO_ERR_INVALID_ARG,
                    "grads->chunk = %d: 0 or a power of two in [%d, %d]", g->chunk,
                    ZERO_STATE_CHUNK_MIN, ZERO_STATE_CHUNK_MAX);
    const int64_t S = L->shard_off[L->n_units];
    if ((S + E - 1) / E > INT64_MAX / 4 / E / g->n)
        return fail(ZERO_ERR_INVALID_ARG, "chunked gradients of %lld elements per rank overflow",
                    (long long)S);
    // The shard-indexed ranks share one receive buffer: rank q's pointer is
    // the buffer's start + q chunks.  A full-indexed rank (a rank's own
    // main gradient) keeps its own buffer, and its slot in the receive
    // buffer is never read.
    const char *base = nullptr;
    for (int q = 0; q < g->n; ++q) {
        if ((g->index ? g->index[q] : g->index_all) != ZERO_INDEX_SHARD)
            continue;
        const char *want = base ? base + (int64_t)q * E * (int64_t)elem : nullptr;
        if (!base)
            base = static_cast<const char *>(g->ptrs[q]) - (int64_t)q * E * (int64_t)elem;
        else if (static_cast<const char *>(g->ptrs[q]) != want)
            return fail(ZERO_ERR_INVALID_ARG,
                        "chunked gradients: rank %d's pointer must be the receive buffer's "
                        "start + %d chunk elements",
                        q, q);
    }
    if (!base)
        return fail(ZERO_ERR_INVALID_ARG, "chunked gradients need a shard-indexed rank");
    return ZERO_OK;
}

namespace {

void fill_grads(const zero_grads *g, StepArgs &a, bool &all_aligned)
{
    a.n_ranks = g->n;
    if (g->chunk)
        a.g_shift = __builtin_ctz((unsigned)g->chunk);
    a.full_mask = 0;
    for (int q = 0; q < g->n; ++q) {
        a.grads[q] = g->ptrs[q];
        const int ix = g->index ? g->index[q] : g->index_all;
        if (ix == ZERO_INDEX_FULL)
            a.full_mask |= (uint64_t)1 << q;
        all_aligned = all_aligned && aligned16(g->ptrs[q]);
    }
    const int n = g->n;
    a.pow2 = (n & (n - 1)) == 0;
    a.inv_n = 1.0f / (float)n;  // exact when pow2
    a.n_f = (float)n;
}

AdamScalars make_scalars(const zero_adam_cfg *c)
{
    AdamScalars s;
    const double b1 = c->beta1, b2 = c->beta2, t = (double)c->step;
    s.lr = c->lr;
    s.b1 = c->beta1;
    s.b2 = c->beta2;
    s.eps = c->eps;
    s.wd = c->weight_decay;
    s.omb1 = (float)(1.0 - b1);
    s.omb2 = (float)(1.0 - b2);
    s.bias1 = (float)(1.0 - std::pow(b1, t));
    s.bias2 = (float)(1.0 - std::pow(b2, t));
    s.decay = (float)(1.0 - (double)c->lr * (double)c->weight_decay);
    s.has_wd = c->weight_decay != 0.0f;
    s.decoupled = c->decoupled ? 1 : 0;
    return s;
}

// Occupancy of the step kernel.  Its launches reserve LDS so that at most 5
// of its 256-thread blocks (20 waves) run on a CU at once.  Paired runs over
// ten buffer placements (the 7B / N = 8 fused step, the apply pass and the
// N = 64 Llama-70B unit), against the former 512-thread / 2048-element tiles
// at full occupancy: fused 0.964 x (0.947-0.982 per placement), apply
// 0.955 x, N = 64 0.973 x; the same 256-thread tiles at full occupancy
// 0.985 x, with a 16-wave cap 0.965 x, 8 or 12 waves 0.99 x.  With fewer
// requests in flight the memory controllers mix the read and write streams
// better; the kernel's time is that of its memory traffic (the same streams
// without the arithmetic run no faster; zero_stream_mix).
//
// The N = 64 specialisation (the Llama-70B units) runs at most 3 blocks per
// CU: with its 64 rank gradients in one chunked receive buffer, paired over
// eight placements of one layer unit, 3 blocks took 0.970 x the time of 5
// (0.967-0.998; 2 blocks 0.968 x, 4 blocks 1.000 x, 6 blocks 1.013 x);
// with 64 separate rank buffers every cap from 2 to 6 is within 0.4 %.  The
// same sweep at N = 8 keeps 5 (4 equal, 3 1.12 x, 6 1.025 x).
//
// The reduce pass, four fifths reads, runs uncapped: on the GPT-2-small
// rank shard (8 full-indexed rank buffers) full occupancy took 0.962 x the
// time of 5 blocks per CU (0.956-0.969, eight placements; 6 or 8 blocks
// the same, 4 blocks 1.12 x), on a 1e8-element shard 0.988 x.  The apply
// pass keeps 5 (full occupancy 1.020 x on the GPT-2 shard, 1.023 x on the
// 7B shard; 4 blocks equal).
//
// A launch whose tiles fit on the GPU at once under the cap never has more
// in flight than the cap allows, so it reserves nothing: small launches (a
// tiny shard, one bucket of a few tiles) keep the plain dispatch.
template <int MODE, int NR>
constexpr int step_cap()
{
    return MODE == kReduce ? 0 : NR == 64 ? kStep64BlocksPerCU : kStepBlocksPerCU;
}

template <int CAP>
size_t step_lds(int64_t n_tiles)
{
    if constexpr (CAP == 0)
        return 0;
    else
        return n_tiles > (int64_t)device_cus() * CAP ? lds_reserve<CAP>() : 0;
}

template <int MODE, int NR, bool BF16>
void launch_one(const StepArgs &a, hipStream_t st)
{
    constexpr int cap = step_cap<MODE, NR>();
    const size_t lds = step_lds<cap>(a.n_tiles);
    static const int resident =
        resident_blocks(step_kernel<MODE, NR, BF16>, kStepThreads, step_lds<cap>(INT64_MAX));
    const int64_t blocks = stream_grid(a.n_tiles, resident, kStepThreads);
    hipLaunchKernelGGL((step_kernel<MODE, NR, BF16>), dim3((unsigned)blocks), dim3(kStepThreads),
                       lds, st, a);
}

template <int MODE, bool BF16>
void launch_step(const StepArgs &a, hipStream_t st)
{
    if constexpr (MODE == kApply) {
        launch_one<kApply, 1, true>(a, st);
    } else {
        switch (a.n_ranks) {
        case 1: launch_one<MODE, 1, BF16>(a, st); break;
        case 2: launch_one<MODE, 2, BF16>(a, st); break;
        case 4: launch_one<MODE, 4, BF16>(a, st); break;
        case 8: launch_one<MODE, 8, BF16>(a, st); break;
        case 64: launch_one<MODE, 64, BF16>(a, st); break;
        default: launch_one<MODE, 0, BF16>(a, st); break;
        }
    }
}

// The calibration modes take bf16 rank buffers; N = 8 (the 7B step) has the
// fused kernel's specialisation, other counts the generic loop.
template <int MODE>
zero_status launch_mix(const StepArgs &a, hipStream_t st)
{
    (void)hipGetLastError();
    if (a.n_ranks == 8)
        launch_one<MODE, 8, true>(a, st);
    else
        launch_one<MODE, 0, true>(a, st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(ZERO_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ZERO_OK;
}

template <int MODE>
zero_status launch_mode(StepArgs &a, bool bf16, hipStream_t st)
{
    (void)hipGetLastError();  // clear a stale error so the check below is ours
    if (MODE == kApply || bf16)
        launch_step<MODE, true>(a, st);
    else
        launch_step<MODE, false>(a, st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(ZERO_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ZERO_OK;
}

zero_status check_cfg(const zero_adam_cfg *cfg)
{
    if (!cfg)
        return fail(ZERO_ERR_INVALID_ARG, "cfg is NULL");
    if (cfg->step < 1)
        return fail(ZERO_ERR_INVALID_ARG, "step must be >= 1 (got %lld)", (long long)cfg->step);
    if (!(cfg->beta1 >= 0.0f && cfg->beta1 < 1.0f) || !(cfg->beta2 >= 0.0f && cfg->beta2 < 1.0f))
        return fail(ZERO_ERR_INVALID_ARG, "betas must lie in [0, 1)");
    if (!std::isfinite(cfg->lr) || !(cfg->eps >= 0.0f) || !std::isfinite(cfg->eps) ||
        !(cfg->weight_decay >= 0.0f) || !std::isfinite(cfg->weight_decay))
        return fail(ZERO_ERR_INVALID_ARG, "lr, eps and weight_decay must be finite, eps, wd >= 0");
    return ZERO_OK;
}

// The Adam step with its scalars either in the launch (table == nullptr) or
// read on the device from table[*step - 1].
zero_status adam_launch(const zero_layout *L, int32_t ub, int32_t ue, const AdamScalars &sc,
                        const AdamScalars *table, int64_t n_table, const int64_t *step,
                        const float *grad_fp32, int32_t grad_index, const float *clip_coef,
                        const zero_grads *grads, float *master, float *m, float *v,
                        uint16_t *param_out, int32_t param_index, void *stream)
{
    zero_status st;
    if ((grad_fp32 != nullptr) == (grads != nullptr))
        return fail(ZERO_ERR_INVALID_ARG, "give exactly one of grad_fp32 and grads");
    if (grads && clip_coef)
        return fail(ZERO_ERR_INVALID_ARG, "clip_coef needs the two-pass path (grad_fp32)");
    if (!master || !m || !v || !param_out)
        return fail(ZERO_ERR_INVALID_ARG, "master, m, v and param_out are required");
    if (param_index != ZERO_INDEX_FULL && param_index != ZERO_INDEX_SHARD)
        return fail(ZERO_ERR_INVALID_ARG, "unknown param_index %d", param_index);
    if (grad_index != ZERO_INDEX_FULL && grad_index != ZERO_INDEX_SHARD)
        return fail(ZERO_ERR_INVALID_ARG, "unknown grad_index %d", grad_index);
    if (reinterpret_cast<uintptr_t>(master) % 4 || reinterpret_cast<uintptr_t>(m) % 4 ||
        reinterpret_cast<uintptr_t>(v) % 4 || reinterpret_cast<uintptr_t>(param_out) % 2 ||
        reinterpret_cast<uintptr_t>(grad_fp32) % 4 || reinterpret_cast<uintptr_t>(clip_coef) % 4)
        return fail(ZERO_ERR_ALIGNMENT, "misaligned state / parameter buffer");
    if (grads && (st = check_grads(L, grads)) != ZERO_OK)
        return st;
    if ((st = check_state(L, master, m, v)) != ZERO_OK)
        return st;
    const int64_t E = L->state_chunk;
    return for_each_chunk(ub, ue, [&](int32_t u0, int32_t u1) -> zero_status {
        StepArgs a;
        std::memset(&a, 0, sizeof a);
        bool al = aligned16(master) && aligned16(m) && aligned16(v) && aligned16(param_out);
        if (grads)
            fill_grads(grads, a, al);
        else
            al = al && aligned16(grad_fp32);
        a.vec_ptrs = al;
        a.n_tiles = fill_segs(L, ub, u0, u1, a.seg, &a.n_segs, E > 0);
        if (a.n_tiles == 0)
            return ZERO_OK;
        a.master = master;
        a.m = m;
        a.v = v;
        if (E > 0) {
            a.st_base = L->shard_off[ub];
            a.st_shift = __builtin_ctzll((unsigned long long)E);
        }
        a.gin = grad_fp32;
        a.gin_full = grad_index == ZERO_INDEX_FULL;
        a.clip = clip_coef;
        a.pout = param_out;
        a.pout_full = param_index == ZERO_INDEX_FULL;
        a.sc = sc;
        a.table = table;
        a.step = step;
        a.n_table = n_table;
        const hipStream_t s = static_cast<hipStream_t>(stream);
        if (grads)
            return launch_mode<kFused>(a, grads->dtype == ZERO_BF16, s);
        return launch_mode<kApply>(a, true, s);
    });
}

}  // namespace
}  // namespace zs

// Device memory for the one entry point that allocates nothing
// (zero_adam_step_clip_noalloc): the fp64 sum-of-squares partials of the
// reduce, then the clip coefficient (a float in the first 4 bytes of slot
// kNoAllocPartials).  Each GPU the library runs on holds its own copy until
// the process ends.  Host code never passes `scratch` itself to a kernel:
// the host-side name is not a device address.  It uses the address
// hipGetSymbolAddress returns for the current device (noalloc_scratch).
constexpr int64_t kNoAllocPartials = ZERO_NOALLOC_MAX_PARTIALS;
static __device__ __align__(256) double scratch[kNoAllocPartials + 32];

namespace zs {
namespace {

// The device address of `scratch` on the current device, looked up once per
// device (hipGetSymbolAddress with that device current) and kept; several
// host threads may race to look it up, and all store the same address.
zero_status noalloc_scratch(double **out)
{
    static std::atomic<double *> cached[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(ZERO_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64)
        return fail(ZERO_ERR_UNSUPPORTED, "device %d: at most 64 devices are supported", dev);
    double *p = cached[dev].load(std::memory_order_acquire);
    if (!p) {
        void *addr = nullptr;
        e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !addr)
            return fail(ZERO_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        p = static_cast<double *>(addr);
        cached[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return ZERO_OK;
}

}  // namespace
}  // namespace zs

using namespace zs;

extern "C" {

int64_t zero_reduce_partials_count(const zero_layout *L, int32_t ub, int32_t ue)
{
    if (check_range(L, ub, ue) != ZERO_OK)
        return -1;
    int64_t total = 0;
    for_each_chunk(ub, ue, [&](int32_t u0, int32_t u1) {
        Seg seg[kMaxSegs];
        int32_t ns = 0;
        total += fill_segs(L, ub, u0, u1, seg, &ns);
        return ZERO_OK;
    });
    return total;
}

zero_status zero_reduce_shard(const zero_layout *L, int32_t ub, int32_t ue,
                              const zero_grads *grads, float *out, int32_t out_index,
                              double *partials, int64_t n_partials, void *stream)
{
    zero_status st = check_range(L, ub, ue);
    if (st != ZERO_OK)
        return st;
    if (!grads || !out)
        return fail(ZERO_ERR_INVALID_ARG, "grads and out are required");
    if ((st = check_grads(L, grads)) != ZERO_OK)
        return st;
    if (reinterpret_cast<uintptr_t>(out) % 4)
        return fail(ZERO_ERR_ALIGNMENT, "out is misaligned");
    if (out_index != ZERO_INDEX_FULL && out_index != ZERO_INDEX_SHARD)
        return fail(ZERO_ERR_INVALID_ARG, "unknown out_index %d", out_index);
    if (partials) {
        if (reinterpret_cast<uintptr_t>(partials) % 8)
            return fail(ZERO_ERR_ALIGNMENT, "sumsq_partials is misaligned");
        const int64_t need = zero_reduce_partials_count(L, ub, ue);
        if (n_partials < need)
            return fail(ZERO_ERR_INVALID_ARG, "sumsq_partials holds %lld, the call writes %lld",
                        (long long)n_partials, (long long)need);
    }
    int64_t poff = 0;
    return for_each_chunk(ub, ue, [&](int32_t u0, int32_t u1) -> zero_status {
        StepArgs a;
        std::memset(&a, 0, sizeof a);
        bool al = aligned16(out);
        fill_grads(grads, a, al);
        a.vec_ptrs = al;
        a.n_tiles = fill_segs(L, ub, u0, u1, a.seg, &a.n_segs);
        if (a.n_tiles == 0)
            return ZERO_OK;
        a.gout = out;
        a.gout_full = out_index == ZERO_INDEX_FULL;
        a.partials = partials ? partials + poff : nullptr;
        poff += a.n_tiles;
        return launch_mode<kReduce>(a, grads->dtype == ZERO_BF16, static_cast<hipStream_t>(stream));
    });
}

zero_status zero_clip_coef(const double *partials, int64_t n, float max_norm, float *coef_out,
                           double *norm_out, void *stream)
{
    if (!partials || !coef_out || n < 1)
        return fail(ZERO_ERR_INVALID_ARG, "partials, coef_out and n >= 1 are required");
    if (!(max_norm > 0.0f) || !std::isfinite(max_norm))
        return fail(ZERO_ERR_INVALID_ARG, "max_norm must be finite and > 0");
    if (reinterpret_cast<uintptr_t>(partials) % 8 || reinterpret_cast<uintptr_t>(coef_out) % 4 ||
        reinterpret_cast<uintptr_t>(norm_out) % 8)
        return fail(ZERO_ERR_ALIGNMENT, "misaligned clip buffers");
    (void)hipGetLastError();
    hipLaunchKernelGGL(clip_kernel, dim3(1), dim3(kClipThreads), 0, static_cast<hipStream_t>(stream),
                       partials, n, max_norm, coef_out, norm_out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(ZERO_ERR_HIP, "clip launch failed: %s", hipGetErrorString(e));
    return ZERO_OK;
}

zero_status zero_adam_step(const zero_layout *L, int32_t ub, int32_t ue,
                           const zero_adam_cfg *cfg, const float *grad_fp32, int32_t grad_index,
                           const float *clip_coef, const zero_grads *grads, float *master,
                           float *m, float *v, uint16_t *param_out, int32_t param_index,
                           void *stream)
{
    zero_status st = check_range(L, ub, ue);
    if (st != ZERO_OK)
        return st;
    if ((st = check_cfg(cfg)) != ZERO_OK)
        return st;
    return adam_launch(L, ub, ue, make_scalars(cfg), nullptr, 0, nullptr, grad_fp32, grad_index,
                       clip_coef, grads, master, m, v, param_out, param_index, stream);
}

zero_status zero_adam_step_clip_noalloc(const zero_layout *L, int32_t ub, int32_t ue,
                                        const zero_adam_cfg *cfg, float max_norm,
                                        const zero_grads *grads, float *grad_out, float *master,
                                        float *m, float *v, uint16_t *param_out,
                                        int32_t param_index, double *norm_out, void *stream)
{
    // every check on the host first: on error nothing is launched and no HIP
    // call is made
    zero_status st = check_range(L, ub, ue);
    if (st != ZERO_OK)
        return st;
    if ((st = check_cfg(cfg)) != ZERO_OK)
        return st;
    if (!(max_norm > 0.0f) || !std::isfinite(max_norm))
        return fail(ZERO_ERR_INVALID_ARG, "max_norm must be finite and > 0");
    if (!grads || !grad_out)
        return fail(ZERO_ERR_INVALID_ARG, "grads and grad_out are required");
    if ((st = check_grads(L, grads)) != ZERO_OK)
        return st;
    if (!master || !m || !v || !param_out)
        return fail(ZERO_ERR_INVALID_ARG, "master, m, v and param_out are required");
    if (param_index != ZERO_INDEX_FULL && param_index != ZERO_INDEX_SHARD)
        return fail(ZERO_ERR_INVALID_ARG, "unknown param_index %d", param_index);
    if (reinterpret_cast<uintptr_t>(grad_out) % 4 || reinterpret_cast<uintptr_t>(master) % 4 ||
        reinterpret_cast<uintptr_t>(m) % 4 || reinterpret_cast<uintptr_t>(v) % 4 ||
        reinterpret_cast<uintptr_t>(param_out) % 2 || reinterpret_cast<uintptr_t>(norm_out) % 8)
        return fail(ZERO_ERR_ALIGNMENT, "misaligned gradient, state, parameter or norm buffer");
    if ((st = check_state(L, master, m, v)) != ZERO_OK)
        return st;
    const int64_t n = zero_reduce_partials_count(L, ub, ue);
    if (n > kNoAllocPartials)
        return fail(ZERO_ERR_UNSUPPORTED,
                    "the range needs %lld sum-of-squares partials; the library's static buffer "
                    "holds %lld (ranges up to %lld elements per rank)",
                    (long long)n, (long long)kNoAllocPartials,
                    (long long)kNoAllocPartials * kStepTile);
    if (n == 0)
        return ZERO_OK;  // every unit of the range is empty
    double *sp = nullptr;
    if ((st = noalloc_scratch(&sp)) != ZERO_OK)
        return st;
    float *coef = reinterpret_cast<float *>(sp + kNoAllocPartials);
    // the three calls of the two-pass path, on the static buffer; their own
    // checks pass, as every argument was checked above
    if ((st = zero_reduce_shard(L, ub, ue, grads, grad_out, ZERO_INDEX_SHARD, sp, n, stream)) !=
        ZERO_OK)
        return st;
    if ((st = zero_clip_coef(sp, n, max_norm, coef, norm_out, stream)) != ZERO_OK)
        return st;
    return zero_adam_step(L, ub, ue, cfg, grad_out, ZERO_INDEX_SHARD, coef, nullptr, master, m, v,
                          param_out, param_index, stream);
}

zero_status zero_adam_table_fill(const zero_adam_cfg *cfgs, int64_t n,
                                 zero_adam_table_entry *host_out)
{
    if (!cfgs || !host_out || n < 1)
        return fail(ZERO_ERR_INVALID_ARG, "cfgs, host_out and n >= 1 are required");
    for (int64_t k = 0; k < n; ++k) {
        const zero_status st = check_cfg(&cfgs[k]);
        if (st != ZERO_OK)
            return fail(st, "entry %lld: %s", (long long)k, zero_last_error());
    }
    for (int64_t k = 0; k < n; ++k) {
        const AdamScalars sc = make_scalars(&cfgs[k]);
        std::memcpy(&host_out[k], &sc, sizeof sc);
    }
    return ZERO_OK;
}

zero_status zero_adam_step_table(const zero_layout *L, int32_t ub, int32_t ue,
                                 const zero_adam_table_entry *table, int64_t n_entries,
                                 const int64_t *step_counter, const float *grad_fp32,
                                 int32_t grad_index, const float *clip_coef,
                                 const zero_grads *grads, float *master, float *m, float *v,
                                 uint16_t *param_out, int32_t param_index, void *stream)
{
    zero_status st = check_range(L, ub, ue);
    if (st != ZERO_OK)
        return st;
    if (!table || !step_counter || n_entries < 1)
        return fail(ZERO_ERR_INVALID_ARG, "table, step_counter and n_entries >= 1 are required");
    if (reinterpret_cast<uintptr_t>(table) % 4 || reinterpret_cast<uintptr_t>(step_counter) % 8)
        return fail(ZERO_ERR_ALIGNMENT, "misaligned step table or counter");
    AdamScalars none;
    std::memset(&none, 0, sizeof none);
    return adam_launch(L, ub, ue, none, reinterpret_cast<const AdamScalars *>(table), n_entries,
                       step_counter, grad_fp32, grad_index, clip_coef, grads, master, m, v,
                       param_out, param_index, stream);
}

zero_status zero_step_advance(int64_t *step_counter, void *stream)
{
    if (!step_counter)
        return fail(ZERO_ERR_INVALID_ARG, "step_counter is NULL");
    if (reinterpret_cast<uintptr_t>(step_counter) % 8)
        return fail(ZERO_ERR_ALIGNMENT, "step_counter is misaligned");
    (void)hipGetLastError();
    hipLaunchKernelGGL(step_advance_kernel, dim3(1), dim3(64), 0,
                       static_cast<hipStream_t>(stream), step_counter);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(ZERO_ERR_HIP, "step advance launch failed: %s", hipGetErrorString(e));
    return ZERO_OK;
}

zero_status zero_gather_params(const zero_layout *L, int32_t ub, int32_t ue,
                               const uint16_t *const *shards, int32_t n, uint16_t *param_full,
                               void *stream)
{
    zero_status st = check_range(L, ub, ue);
    if (st != ZERO_OK)
        return st;
    if (!shards || !param_full)
        return fail(ZERO_ERR_INVALID_ARG, "shards and param_full are required");
    if (n != L->parts)
        return fail(ZERO_ERR_INVALID_ARG, "n = %d but the layout has %d slices per unit", n,
                    L->parts);
    if (reinterpret_cast<uintptr_t>(param_full) % 2)
        return fail(ZERO_ERR_ALIGNMENT, "param_full is misaligned");
    for (int q = 0; q < n; ++q)
        if (reinterpret_cast<uintptr_t>(shards[q]) % 2)
            return fail(ZERO_ERR_ALIGNMENT, "shard of rank %d is misaligned", q);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // batches of at most kMaxRanks non-null sources
    for (int q0 = 0; q0 < n; q0 += kMaxRanks) {
        st = for_each_chunk(ub, ue, [&](int32_t u0, int32_t u1) -> zero_status {
            GatherArgs a;
            std::memset(&a, 0, sizeof a);
            bool al = aligned16(param_full);
            for (int q = q0; q < n && q < q0 + kMaxRanks; ++q) {
                if (!shards[q])
                    continue;
                a.src[a.n_src] = shards[q];
                a.rank_of[a.n_src] = q;
                al = al && aligned16(shards[q]);
                ++a.n_src;
            }
            if (a.n_src == 0)
                return ZERO_OK;
            int64_t tiles = 0;
            int32_t k = 0;
            for (int32_t u = u0; u < u1; ++u) {
                const int64_t len = L->slice[u];
                if (len == 0)
                    continue;
                GSeg &g = a.seg[k++];
                g.len = len;
                g.shard_off = L->shard_off[u] - L->shard_off[ub];
                g.flat_base = L->flat_off[u] - L->flat_off[ub];
                g.tile0 = tiles;
                g.vec = (len % kVec == 0 && g.shard_off % kVec == 0 && g.flat_base % kVec == 0);
                tiles += tiles_of(len);
            }
            a.n_segs = k;
            a.n_tiles = tiles;
            a.dst = param_full;
            a.vec_ptrs = al;
            if (tiles == 0)
                return ZERO_OK;
            // default: one block per (tile, source) -- paired runs on the 7-
            // and 63-source shapes measured 6.2-6.3 TB/s against 5.4-5.6 with
            // each block walking n_src tiles; a persistent override spreads
            // its width over the sources.  A launch of more blocks than fit
            // at once reserves LDS so that at most kGatherBlocksPerCU of them
            // (26 waves) share a CU: paired over ten buffer placements on
            // two boxes, 0.989 x (0.975-0.997) for 7 sources of the 7B
            // shard and 0.990 x (0.981-0.996) for 63 sources of a
            // Llama-70B layer unit, against full occupancy (32 waves);
            // 14 and 12 blocks were within 0.3 % of it, 10 blocks 2.8 %
            // slower.
            const size_t lds = tiles * a.n_src > (int64_t)device_cus() * kGatherBlocksPerCU
                                   ? lds_reserve<kGatherBlocksPerCU>()
                                   : 0;
            static const int resident = resident_blocks(gather_kernel, kGatherThreads,
                                                        lds_reserve<kGatherBlocksPerCU>());
            int64_t gx = blocks_per_cu_override() == 0
                             ? stream_grid(tiles, resident, kGatherThreads)
                             : stream_grid(tiles, resident, kGatherThreads) / a.n_src;
            gx = gx < 1 ? 1 : gx;
            (void)hipGetLastError();
            hipLaunchKernelGGL(gather_kernel, dim3((unsigned)gx, (unsigned)a.n_src),
                               dim3(kGatherThreads), lds, s, a);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return fail(ZERO_ERR_HIP, "gather launch failed: %s", hipGetErrorString(e));
            return ZERO_OK;
        });
        if (st != ZERO_OK)
            return st;
    }
    return ZERO_OK;
}

zero_status zero_stream_mix(int32_t kind, const uint16_t *const *grads, int32_t n_ranks,
                            float *master, float *m, float *v, uint16_t *param, int64_t n,
                            int64_t state_chunk, int64_t grad_chunk, void *stream)
{
    if (kind != ZERO_MIX_STEP_STREAMS && kind != ZERO_MIX_READS && kind != ZERO_MIX_WRITES)
        return fail(ZERO_ERR_INVALID_ARG, "unknown stream-mix kind %d", kind);
    if (n_ranks < 1 || n_ranks > kMaxRanks)
        return fail(ZERO_ERR_INVALID_ARG, "n_ranks must lie in [1, %d] (got %d)", kMaxRanks,
                    n_ranks);
    if (n < 0 || n % 4)
        return fail(ZERO_ERR_INVALID_ARG, "n must be a non-negative multiple of 4 (got %lld)",
                    (long long)n);
    if (!grads || !master || !m || !v || !param)
        return fail(ZERO_ERR_INVALID_ARG, "grads, master, m, v and param are required");
    const int64_t E = state_chunk;
    if (E != 0 && (E < ZERO_STATE_CHUNK_MIN || E > ZERO_STATE_CHUNK_MAX || (E & (E - 1)) != 0))
        return fail(ZERO_ERR_INVALID_ARG, "state_chunk must be 0 or a power of two in [%d, %d] "
                    "(got %lld)", ZERO_STATE_CHUNK_MIN, ZERO_STATE_CHUNK_MAX, (long long)E);
    if (E > 0 && (m != master + E || v != master + 2 * E))
        return fail(ZERO_ERR_INVALID_ARG, "chunked state: m and v must be master + state_chunk "
                    "and master + 2 state_chunk");
    const int64_t GE = grad_chunk;
    if (GE != 0 &&
        (GE < ZERO_STATE_CHUNK_MIN || GE > ZERO_STATE_CHUNK_MAX || (GE & (GE - 1)) != 0))
        return fail(ZERO_ERR_INVALID_ARG, "grad_chunk must be 0 or a power of two in [%d, %d] "
                    "(got %lld)", ZERO_STATE_CHUNK_MIN, ZERO_STATE_CHUNK_MAX, (long long)GE);
    bool al = aligned16(master) && aligned16(m) && aligned16(v) && aligned16(param);
    for (int q = 0; q < n_ranks; ++q) {
        if (!grads[q])
            return fail(ZERO_ERR_INVALID_ARG, "gradient buffer of rank %d is NULL", q);
        if (GE > 0 && grads[q] != grads[0] + q * GE)
            return fail(ZERO_ERR_INVALID_ARG, "chunked gradients: rank %d's pointer must be "
                        "rank 0's + %d grad_chunk elements", q, q);
        al = al && aligned16(grads[q]);
    }
    if (!al)
        return fail(ZERO_ERR_ALIGNMENT, "every buffer must be 16-byte aligned");
    if (n == 0)
        return ZERO_OK;
    StepArgs a;
    std::memset(&a, 0, sizeof a);
    for (int q = 0; q < n_ranks; ++q)
        a.grads[q] = grads[q];
    a.n_ranks = n_ranks;
    a.vec_ptrs = 1;
    a.n_segs = 1;
    a.seg[0].len = n;
    a.seg[0].vec = 1;
    a.n_tiles = step_tiles_of(n);
    a.master = master;
    a.m = m;
    a.v = v;
    if (E > 0)
        a.st_shift = __builtin_ctzll((unsigned long long)E);
    if (GE > 0)
        a.g_shift = __builtin_ctzll((unsigned long long)GE);
    a.pout = param;
    a.sink_key = __builtin_nanf("");
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (kind == ZERO_MIX_STEP_STREAMS)
        return launch_mix<kMix>(a, s);
    if (kind == ZERO_MIX_READS)
        return launch_mix<kReadOnly>(a, s);
    return launch_mix<kWriteOnly>(a, s);
}

zero_status zero_grad_accumulate(float *main_grad, const uint16_t *micro, int64_t n, void *stream)
{
    if (!main_grad || !micro || n < 0)
        return fail(ZERO_ERR_INVALID_ARG, "main_grad, micro and n >= 0 are required");
    if (reinterpret_cast<uintptr_t>(main_grad) % 4 || reinterpret_cast<uintptr_t>(micro) % 2)
        return fail(ZERO_ERR_ALIGNMENT, "misaligned accumulation buffers");
    if (n == 0)
        return ZERO_OK;
    const int64_t tiles = tiles_of(n);
    static const int resident = resident_blocks(accumulate_kernel, kAccThreads);
    const int64_t grid = stream_grid(tiles, resident, kAccThreads);
    const int32_t vec = aligned16(main_grad) && aligned16(micro);
    (void)hipGetLastError();
    hipLaunchKernelGGL(accumulate_kernel, dim3((unsigned)grid), dim3(kAccThreads), 0,
                       static_cast<hipStream_t>(stream), main_grad, micro, n, vec);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(ZERO_ERR_HIP, "accumulate launch failed: %s", hipGetErrorString(e));
    return ZERO_OK;
}

}  // extern "C"
