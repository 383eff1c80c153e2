// HIP kernels (gfx950 / CDNA4) and compute entry points of libzeroshard.
//
// Everything here is HBM-bound streaming: per shard element the fused step
// reads N gradients (2N bytes bf16 or 4N fp32) and the fp32 master, m, v
// (12 bytes), and writes master, m, v (12) and the bf16 parameter (2), for
// about N + 20 flops -- far below the machine balance, so there is no
// contraction and no MFMA.  The design rules that matter are the memory ones:
//   * 256-thread blocks, each thread owns 8 consecutive elements of a
//     2048-element tile, so every stream moves in 128-bit loads/stores
//     (one per bf16 stream, two per fp32 stream) and a wave covers whole
//     128-byte lines;
//   * one pass: the reduce over ranks, the Adam update and the bf16 cast are
//     fused so each byte crosses HBM once;
//   * persistent grid-stride launch over a tile space that concatenates the
//     slices of many units (FSDP layers, gradient buckets), so small units do
//     not pay one launch and one ramp-down each;
//   * the N rank streams are loaded in groups of 8 before they are summed,
//     keeping 8 x 16 bytes per thread in flight without holding all N.
//
// Arithmetic (identical on every launch shape): fp32, one rounding per
// operation, no contraction into FMA (pragma below plus -ffp-contract=off),
// IEEE division and square root (the compiler's correctly-rounded
// sequences), rank sum in ascending order from +0 then divided by N (times
// the exact reciprocal when N is a power of two, which rounds identically).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>

#include "internal.h"

#pragma clang fp contract(off)

namespace zs {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8;                     // elements per thread per tile
constexpr int kTile = kThreads * kVec;      // elements per tile
constexpr int kMaxSegs = 32;                // units per launch (kernarg table)
constexpr int kReduceGrid = 2048;           // fixed so the partial count is fixed
constexpr int kMaxRanks = ZERO_MAX_RANKS_PER_CALL;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One unit's slice inside a launch's tile space.
struct Seg {
    int64_t len;        // s_u: elements of the slice
    int64_t shard_off;  // R_u - R_begin: slice start in shard-indexed buffers
    int64_t full_off;   // (F_u - F_begin) + r*s_u: slice start in full buffers
    int64_t tile0;      // first tile of this slice
    int64_t vec;        // 1 if both offsets are multiples of 8 (vector path)
};

struct AdamScalars {
    float lr, b1, b2, eps, wd;
    float omb1, omb2, bias1, bias2, decay;
    int32_t has_wd, decoupled;
};

enum Mode { kFused = 0, kReduce = 1, kApply = 2 };

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
    const float *gin;    // kApply: shard-indexed averaged gradient
    const float *clip;   // kApply: device clip coefficient or null
    float *gout;         // kReduce: shard-indexed averaged gradient
    double *partials;    // kReduce: one fp64 sum of squares per block, or null
    uint16_t *pout;      // bf16 parameter output
    int32_t pout_full;   // 1: full-indexed, 0: shard-indexed
    int32_t _pad;
    AdamScalars sc;
    Seg seg[kMaxSegs];
};

// ------------------------------------------------------------ helpers --

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

// Sum of the N rank gradients for 8 consecutive elements (vector path).
template <int NR, bool BF16>
__device__ __forceinline__ void reduce8(const StepArgs &a, int64_t si, int64_t fi, float acc[8])
{
    const int n = NR > 0 ? NR : a.n_ranks;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        acc[k] = 0.0f;
    // one group of 8 rank loads in flight per thread; other waves hide the
    // latency between groups (unrolling further only raises register use)
#pragma unroll 1
    for (int q0 = 0; q0 < n; q0 += 8) {
        if (BF16) {
            u32x4 w[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int q = q0 + k;
                if (q < n) {
                    const int64_t i = ((a.full_mask >> q) & 1) ? fi : si;
                    w[k] = ld_nt(reinterpret_cast<const u32x4 *>(
                        static_cast<const uint16_t *>(a.grads[q]) + i));
                }
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (q0 + k < n) {
                    acc[0] = acc[0] + bf16lo(w[k].x);
                    acc[1] = acc[1] + bf16hi(w[k].x);
                    acc[2] = acc[2] + bf16lo(w[k].y);
                    acc[3] = acc[3] + bf16hi(w[k].y);
                    acc[4] = acc[4] + bf16lo(w[k].z);
                    acc[5] = acc[5] + bf16hi(w[k].z);
                    acc[6] = acc[6] + bf16lo(w[k].w);
                    acc[7] = acc[7] + bf16hi(w[k].w);
                }
            }
        } else {
            f32x4 w[8][2];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int q = q0 + k;
                if (q < n) {
                    const int64_t i = ((a.full_mask >> q) & 1) ? fi : si;
                    const f32x4 *p = reinterpret_cast<const f32x4 *>(
                        static_cast<const float *>(a.grads[q]) + i);
                    w[k][0] = ld_nt(p);
                    w[k][1] = ld_nt(p + 1);
                }
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (q0 + k < n) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[e] = acc[e] + w[k][0][e];
                        acc[4 + e] = acc[4 + e] + w[k][1][e];
                    }
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
    for (int q = 0; q < n; ++q) {
        const int64_t i = ((a.full_mask >> q) & 1) ? fi : si;
        const float x = BF16 ? bf16f(static_cast<const uint16_t *>(a.grads[q])[i])
                             : static_cast<const float *>(a.grads[q])[i];
        acc = acc + x;
    }
    return acc;
}

// Block-wide fp64 sum in a fixed order (wave shuffles, then waves 0..3).
__device__ double block_sum(double x)
{
    __shared__ double lds[kThreads / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x = x + __shfl_xor(x, off, 64);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
        lds[wave] = x;
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x == 0)
        for (int w = 0; w < kThreads / 64; ++w)
            t = t + lds[w];
    return t;  // valid in thread 0
}

// -------------------------------------------------------- step kernel --

template <int MODE, int NR, bool BF16>
__global__ __launch_bounds__(kThreads) void step_kernel(const StepArgs a)
{
    double sq = 0.0;
    const float coef = (MODE == kApply && a.clip) ? *a.clip : 1.0f;
    int s = 0;
    for (int64_t t = blockIdx.x; t < a.n_tiles; t += gridDim.x) {
        while (s + 1 < a.n_segs && t >= a.seg[s + 1].tile0)
            ++s;
        const Seg &sg = a.seg[s];
        const int64_t j = (t - sg.tile0) * kTile + (int64_t)threadIdx.x * kVec;
        if (j >= sg.len)
            continue;
        const int64_t si = sg.shard_off + j;
        const int64_t fi = sg.full_off + j;
        const int64_t oi = a.pout_full ? fi : si;

        if (sg.vec && a.vec_ptrs && j + kVec <= sg.len) {
            // ---------------- vector path: 8 elements, 128-bit accesses
            float g[8];
            f32x4 p0, p1, m0, m1, v0, v1;
            if (MODE != kReduce) {
                const f32x4 *pp = reinterpret_cast<const f32x4 *>(a.master + si);
                const f32x4 *mp = reinterpret_cast<const f32x4 *>(a.m + si);
                const f32x4 *vp = reinterpret_cast<const f32x4 *>(a.v + si);
                p0 = ld_nt(pp); p1 = ld_nt(pp + 1);
                m0 = ld_nt(mp); m1 = ld_nt(mp + 1);
                v0 = ld_nt(vp); v1 = ld_nt(vp + 1);
            }
            if (MODE == kApply) {
                const f32x4 *gp = reinterpret_cast<const f32x4 *>(a.gin + si);
                const f32x4 g0 = ld_nt(gp), g1 = ld_nt(gp + 1);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    g[e] = g0[e] * coef;
                    g[4 + e] = g1[e] * coef;
                }
            } else {
                float acc[8];
                reduce8<NR, BF16>(a, si, fi, acc);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    g[e] = mean_of(a, acc[e]);
            }
            if (MODE == kReduce) {
                f32x4 g0, g1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    g0[e] = g[e];
                    g1[e] = g[4 + e];
                    sq = sq + (double)g[e] * (double)g[e];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sq = sq + (double)g[4 + e] * (double)g[4 + e];
                f32x4 *gp = reinterpret_cast<f32x4 *>(a.gout + si);
                st_nt(gp, g0);
                st_nt(gp + 1, g1);
            } else {
                float p[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
                float m[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
                float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    adam1(a.sc, g[e], p[e], m[e], v[e]);
                f32x4 *pp = reinterpret_cast<f32x4 *>(a.master + si);
                f32x4 *mp = reinterpret_cast<f32x4 *>(a.m + si);
                f32x4 *vp = reinterpret_cast<f32x4 *>(a.v + si);
                st_nt(pp, f32x4{p[0], p[1], p[2], p[3]});
                st_nt(pp + 1, f32x4{p[4], p[5], p[6], p[7]});
                st_nt(mp, f32x4{m[0], m[1], m[2], m[3]});
                st_nt(mp + 1, f32x4{m[4], m[5], m[6], m[7]});
                st_nt(vp, f32x4{v[0], v[1], v[2], v[3]});
                st_nt(vp + 1, f32x4{v[4], v[5], v[6], v[7]});
                u32x4 w;
                w.x = to_bf16(p[0]) | (to_bf16(p[1]) << 16);
                w.y = to_bf16(p[2]) | (to_bf16(p[3]) << 16);
                w.z = to_bf16(p[4]) | (to_bf16(p[5]) << 16);
                w.w = to_bf16(p[6]) | (to_bf16(p[7]) << 16);
                st_nt(reinterpret_cast<u32x4 *>(a.pout + oi), w);
            }
        } else {
            // ---------------- scalar path: ragged tail or unaligned slice
            const int64_t cnt = (sg.len - j) < kVec ? (sg.len - j) : kVec;
            for (int64_t e = 0; e < cnt; ++e) {
                float g;
                if (MODE == kApply)
                    g = a.gin[si + e] * coef;
                else
                    g = mean_of(a, reduce1<NR, BF16>(a, si + e, fi + e));
                if (MODE == kReduce) {
                    a.gout[si + e] = g;
                    sq = sq + (double)g * (double)g;
                } else {
                    float p = a.master[si + e], m = a.m[si + e], v = a.v[si + e];
                    adam1(a.sc, g, p, m, v);
                    a.master[si + e] = p;
                    a.m[si + e] = m;
                    a.v[si + e] = v;
                    a.pout[oi + e] = (uint16_t)to_bf16(p);
                }
            }
        }
    }
    if (MODE == kReduce && a.partials) {
        const double total = block_sum(sq);
        if (threadIdx.x == 0)
            a.partials[blockIdx.x] = total;
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
__global__ __launch_bounds__(kThreads) void gather_kernel(const GatherArgs a)
{
    const int y = blockIdx.y;
    const uint16_t *src = a.src[y];
    const int64_t q = a.rank_of[y];
    int s = 0;
    for (int64_t t = blockIdx.x; t < a.n_tiles; t += gridDim.x) {
        while (s + 1 < a.n_segs && t >= a.seg[s + 1].tile0)
            ++s;
        const GSeg &sg = a.seg[s];
        const int64_t j = (t - sg.tile0) * kTile + (int64_t)threadIdx.x * kVec;
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

// ------------------------------------------------- accumulate kernel --

__global__ __launch_bounds__(kThreads) void accumulate_kernel(float *acc, const uint16_t *micro,
                                                              int64_t n, int32_t vec)
{
    const int64_t stride = (int64_t)gridDim.x * kTile;
    for (int64_t b = (int64_t)blockIdx.x * kTile; b < n; b += stride) {
        const int64_t i = b + (int64_t)threadIdx.x * kVec;
        if (i >= n)
            continue;
        if (vec && i + kVec <= n) {
            f32x4 *ap = reinterpret_cast<f32x4 *>(acc + i);
            f32x4 a0 = ld_nt(ap), a1 = ld_nt(ap + 1);
            const u32x4 w = ld_nt(reinterpret_cast<const u32x4 *>(micro + i));
            a0.x = a0.x + bf16lo(w.x); a0.y = a0.y + bf16hi(w.x);
            a0.z = a0.z + bf16lo(w.y); a0.w = a0.w + bf16hi(w.y);
            a1.x = a1.x + bf16lo(w.z); a1.y = a1.y + bf16hi(w.z);
            a1.z = a1.z + bf16lo(w.w); a1.w = a1.w + bf16hi(w.w);
            st_nt(ap, a0);
            st_nt(ap + 1, a1);
        } else {
            const int64_t cnt = (n - i) < kVec ? (n - i) : kVec;
            for (int64_t e = 0; e < cnt; ++e)
                acc[i + e] = acc[i + e] + bf16f(micro[i + e]);
        }
    }
}

// ------------------------------------------------------- clip kernel --

// One block: per-thread strided fp64 sums, then a fixed-order block sum.
__global__ __launch_bounds__(kThreads) void clip_kernel(const double *partials, int64_t n,
                                                        float max_norm, float *coef,
                                                        double *norm_out)
{
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += kThreads)
        s = s + partials[i];
    const double total = block_sum(s);
    if (threadIdx.x == 0) {
        const double norm = sqrt(total);
        const float c = (float)((double)max_norm / (norm + 1e-6));
        *coef = c < 1.0f ? c : 1.0f;
        if (norm_out)
            *norm_out = norm;
    }
}

// ------------------------------------------------------------- host --

int device_cus()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (!cached[dev]) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
}

int blocks_per_cu()
{
    static int v = [] {
        const char *e = std::getenv("ZERO_SHARD_BLOCKS_PER_CU");
        const int x = e ? std::atoi(e) : 0;
        return (x >= 1 && x <= 64) ? x : 8;
    }();
    return v;
}

int64_t stream_grid(int64_t n_tiles)
{
    const int64_t g = (int64_t)device_cus() * blocks_per_cu();
    return n_tiles < g ? n_tiles : g;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t tiles_of(int64_t len) { return (len + kTile - 1) / kTile; }

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
// at `ub`; returns the number of tiles.
int64_t fill_segs(const zero_layout *L, int32_t ub, int32_t u0, int32_t u1, Seg *seg,
                  int32_t *n_segs)
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
        s.vec = (s.shard_off % kVec == 0 && s.full_off % kVec == 0) ? 1 : 0;
        tiles += tiles_of(len);
    }
    *n_segs = k;
    return tiles;
}

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
    return ZERO_OK;
}

void fill_grads(const zero_grads *g, StepArgs &a, bool &all_aligned)
{
    a.n_ranks = g->n;
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

template <int MODE, bool BF16>
void launch_step(const StepArgs &a, int64_t grid, hipStream_t st)
{
    const dim3 g((unsigned)grid), b(kThreads);
    if constexpr (MODE == kApply) {
        hipLaunchKernelGGL((step_kernel<kApply, 1, true>), g, b, 0, st, a);
        return;
    } else {
    switch (a.n_ranks) {
    case 1: hipLaunchKernelGGL((step_kernel<MODE, 1, BF16>), g, b, 0, st, a); break;
    case 2: hipLaunchKernelGGL((step_kernel<MODE, 2, BF16>), g, b, 0, st, a); break;
    case 4: hipLaunchKernelGGL((step_kernel<MODE, 4, BF16>), g, b, 0, st, a); break;
    case 8: hipLaunchKernelGGL((step_kernel<MODE, 8, BF16>), g, b, 0, st, a); break;
    case 64: hipLaunchKernelGGL((step_kernel<MODE, 64, BF16>), g, b, 0, st, a); break;
    default: hipLaunchKernelGGL((step_kernel<MODE, 0, BF16>), g, b, 0, st, a); break;
    }
    }
}

template <int MODE>
zero_status launch_mode(StepArgs &a, bool bf16, int64_t grid, hipStream_t st)
{
    (void)hipGetLastError();  // clear a stale error so the check below is ours
    if (MODE == kApply || bf16)
        launch_step<MODE, true>(a, grid, st);
    else
        launch_step<MODE, false>(a, grid, st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(ZERO_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
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
        const int64_t tiles = fill_segs(L, ub, u0, u1, seg, &ns);
        total += tiles < kReduceGrid ? tiles : kReduceGrid;
        return ZERO_OK;
    });
    return total;
}

zero_status zero_reduce_shard(const zero_layout *L, int32_t ub, int32_t ue,
                              const zero_grads *grads, float *out, double *partials,
                              int64_t n_partials, void *stream)
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
        const int64_t grid = a.n_tiles < kReduceGrid ? a.n_tiles : kReduceGrid;
        a.partials = partials ? partials + poff : nullptr;
        poff += grid;
        return launch_mode<kReduce>(a, grads->dtype == ZERO_BF16, grid,
                                    static_cast<hipStream_t>(stream));
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
    hipLaunchKernelGGL(clip_kernel, dim3(1), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       partials, n, max_norm, coef_out, norm_out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(ZERO_ERR_HIP, "clip launch failed: %s", hipGetErrorString(e));
    return ZERO_OK;
}

zero_status zero_adam_step(const zero_layout *L, int32_t ub, int32_t ue,
                           const zero_adam_cfg *cfg, const float *grad_fp32,
                           const float *clip_coef, const zero_grads *grads, float *master,
                           float *m, float *v, uint16_t *param_out, int32_t param_index,
                           void *stream)
{
    zero_status st = check_range(L, ub, ue);
    if (st != ZERO_OK)
        return st;
    if (!cfg)
        return fail(ZERO_ERR_INVALID_ARG, "cfg is NULL");
    if (cfg->step < 1)
        return fail(ZERO_ERR_INVALID_ARG, "step must be >= 1 (got %lld)", (long long)cfg->step);
    if (!(cfg->beta1 >= 0.0f && cfg->beta1 < 1.0f) || !(cfg->beta2 >= 0.0f && cfg->beta2 < 1.0f))
        return fail(ZERO_ERR_INVALID_ARG, "betas must lie in [0, 1)");
    if (!std::isfinite(cfg->lr) || !(cfg->eps >= 0.0f) || !std::isfinite(cfg->eps) ||
        !(cfg->weight_decay >= 0.0f) || !std::isfinite(cfg->weight_decay))
        return fail(ZERO_ERR_INVALID_ARG, "lr, eps and weight_decay must be finite, eps, wd >= 0");
    if ((grad_fp32 != nullptr) == (grads != nullptr))
        return fail(ZERO_ERR_INVALID_ARG, "give exactly one of grad_fp32 and grads");
    if (grads && clip_coef)
        return fail(ZERO_ERR_INVALID_ARG, "clip_coef needs the two-pass path (grad_fp32)");
    if (!master || !m || !v || !param_out)
        return fail(ZERO_ERR_INVALID_ARG, "master, m, v and param_out are required");
    if (param_index != ZERO_INDEX_FULL && param_index != ZERO_INDEX_SHARD)
        return fail(ZERO_ERR_INVALID_ARG, "unknown param_index %d", param_index);
    if (reinterpret_cast<uintptr_t>(master) % 4 || reinterpret_cast<uintptr_t>(m) % 4 ||
        reinterpret_cast<uintptr_t>(v) % 4 || reinterpret_cast<uintptr_t>(param_out) % 2 ||
        reinterpret_cast<uintptr_t>(grad_fp32) % 4 || reinterpret_cast<uintptr_t>(clip_coef) % 4)
        return fail(ZERO_ERR_ALIGNMENT, "misaligned state / parameter buffer");
    if (grads && (st = check_grads(L, grads)) != ZERO_OK)
        return st;
    const AdamScalars sc = make_scalars(cfg);
    return for_each_chunk(ub, ue, [&](int32_t u0, int32_t u1) -> zero_status {
        StepArgs a;
        std::memset(&a, 0, sizeof a);
        bool al = aligned16(master) && aligned16(m) && aligned16(v) && aligned16(param_out);
        if (grads)
            fill_grads(grads, a, al);
        else
            al = al && aligned16(grad_fp32);
        a.vec_ptrs = al;
        a.n_tiles = fill_segs(L, ub, u0, u1, a.seg, &a.n_segs);
        if (a.n_tiles == 0)
            return ZERO_OK;
        a.master = master;
        a.m = m;
        a.v = v;
        a.gin = grad_fp32;
        a.clip = clip_coef;
        a.pout = param_out;
        a.pout_full = param_index == ZERO_INDEX_FULL;
        a.sc = sc;
        const int64_t grid = stream_grid(a.n_tiles);
        const hipStream_t s = static_cast<hipStream_t>(stream);
        if (grads)
            return launch_mode<kFused>(a, grads->dtype == ZERO_BF16, grid, s);
        return launch_mode<kApply>(a, true, grid, s);
    });
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
            int64_t gx = stream_grid(tiles) / a.n_src;
            gx = gx < 1 ? 1 : gx;
            (void)hipGetLastError();
            hipLaunchKernelGGL(gather_kernel, dim3((unsigned)gx, (unsigned)a.n_src), dim3(kThreads),
                               0, s, a);
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

zero_status zero_grad_accumulate(float *main_grad, const uint16_t *micro, int64_t n, void *stream)
{
    if (!main_grad || !micro || n < 0)
        return fail(ZERO_ERR_INVALID_ARG, "main_grad, micro and n >= 0 are required");
    if (reinterpret_cast<uintptr_t>(main_grad) % 4 || reinterpret_cast<uintptr_t>(micro) % 2)
        return fail(ZERO_ERR_ALIGNMENT, "misaligned accumulation buffers");
    if (n == 0)
        return ZERO_OK;
    const int64_t tiles = tiles_of(n);
    const int64_t grid = stream_grid(tiles);
    const int32_t vec = aligned16(main_grad) && aligned16(micro);
    (void)hipGetLastError();
    hipLaunchKernelGGL(accumulate_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), main_grad, micro, n, vec);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(ZERO_ERR_HIP, "accumulate launch failed: %s", hipGetErrorString(e));
    return ZERO_OK;
}

}  // extern "C"
