// msda.hip -- gfx950 (MI355X, CDNA4) kernels and C ABI of the multi-scale
// deformable attention (MSDeformAttn) sampling core.  The operation, layouts
// and error behaviour are specified in include/msda.h.
//
// Vocabulary.  An "item" is one (batch b, query q, head m); it owns L*K
// sampling points and D channels.  A group of G = D/4 lanes serves one item,
// lane c holding channels 4c..4c+3, so each neighbour fetch of a point is one
// coalesced read of the head's row of D values (16 bytes per lane for fp32,
// 8 for bf16).  Per-point coordinate work (pixel coordinate, floor, the four
// neighbours' offsets and weights) is done once per point, by one thread,
// into LDS, and the lane groups read it from there.
//
// Forward (msda_fwd_kernel): per item, sum over its points of A * bilinear
// sample, accumulated in registers, one store per item.
//
// Backward (msda_backward) runs as a pipeline on the caller's stream:
//   1. bwd_dots_kernel: per point the four <grad_out, neighbour row> dot
//      products, reduced across the lane group with DPP, give
//      grad_attn_weight and grad_sampling_loc.  The same pass counts, per
//      8x8-pixel tile of grad_value ("bin"), how many points have a
//      neighbour in it (LDS histogram, one global add per bin per workgroup).
//   2. bin_scan_kernel: exclusive scan of the counts -> bin offsets, and a
//      work list of (bin, chunk of at most kChunk points).
//   3. bin_scatter_kernel: every point's index is written into each bin it
//      touches (LDS ranks, one global reservation per bin per workgroup).
//   4. grad_value_tile_kernel: per work item, the points of the chunk push
//      A * w * grad_out into private LDS copies of the 8x8xD tile -- each
//      half-wave (or wave) owns one copy, so plain read-modify-writes never
//      race -- then the copies are summed and every pixel is written once.
//      Only bins split over several chunks add into grad_value atomically.
// fp32 atomics on this chip run at a few hundred G lane-ops/s whether they
// target LDS or memory, so scattering the 4*D contributions of every point
// with atomics would cost milliseconds at the encoder shape; the binned
// pipeline replaces them with integer LDS atomics and plain LDS traffic.
//
// value and grad_value are addressed through raw buffer descriptors whose
// size is the batch slice.  A neighbour outside the map gets the offset
// kOOB, beyond every slice, so its fetch returns zeros without a branch; the
// same range check keeps an inconsistent level table from touching other
// memory.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msda.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxLevels = 16;
constexpr uint32_t kOOB = 0x80000000u;     // byte offset past every slice (slices < 2^31 B)
constexpr int kRsrcWord3 = 0x00020000;     // gfx9 buffer descriptor word 3 (raw, 32-bit data)
constexpr int kSetupLdsBytes = 36 * 1024;  // per-workgroup budget for the point tables
constexpr int kTileShift = 3;              // grad_value tiles of 8x8 pixels
constexpr int kTile = 1 << kTileShift;
constexpr int kTilePx = kTile * kTile;
constexpr int kChunk = 2048;               // points per grad_value work item, at most
constexpr int kHistLds = 4096;             // bins of one (batch, head) kept in an LDS histogram
constexpr int kScatterQueries = 64;        // queries per scatter workgroup
constexpr int kScanThreads = 1024;
constexpr int kTileGrid = 2048;            // persistent workgroups of the tile kernel

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

// Four consecutive channels of a value row, widened to fp32.  `off32` is the
// row's byte offset in fp32 units (row index * D * 4), `ch` the first channel.
template <typename VT> struct Row4;

template <> struct Row4<float> {
    __device__ __forceinline__ static float4 load(rsrc_t r, uint32_t off32, int ch) {
        auto u = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off32 + 4u * ch), 0, 0);
        return make_float4(__uint_as_float(u[0]), __uint_as_float(u[1]),
                           __uint_as_float(u[2]), __uint_as_float(u[3]));
    }
};

// bfloat16 bits in uint16_t: widening is a 16-bit left shift, exact.
template <> struct Row4<uint16_t> {
    __device__ __forceinline__ static float4 load(rsrc_t r, uint32_t off32, int ch) {
        auto u = __builtin_amdgcn_raw_buffer_load_b64(r, (int)((off32 >> 1) + 2u * ch), 0, 0);
        return make_float4(__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u),
                           __uint_as_float(u[1] << 16), __uint_as_float(u[1] & 0xffff0000u));
    }
};

template <int CTRL> __device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the G lanes of an aligned lane group (G a power of two <= 64);
// every lane of the group receives the sum.
template <int G> __device__ __forceinline__ float group_sum(float v) {
    if constexpr (G >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (G >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (G >= 8) v += dpp<0x141>(v);   // row_half_mirror: the other quad of 8
    if constexpr (G >= 16) v += dpp<0x140>(v);  // row_mirror: the other half of 16
    if constexpr (G >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (G >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// Level table staged in LDS.  lvl[l] = (H, W, start, first bin of the level);
// a level whose pixels do not fit inside value, or whose tiles would not fit
// the bin stride, becomes (0, 0, 0, first bin) and has no pixel and no bin.
struct LevelLds {
    int4 lvl[kMaxLevels];
    int tw[kMaxLevels];  // tiles along W
    int nbins;           // bins of one (batch, head)
};

__device__ __forceinline__ void stage_levels(LevelLds *s, const int64_t *shapes,
                                             const int64_t *starts, int L, int Nv, int nb_max) {
    const int t = threadIdx.x;
    if (t < L) {
        const int64_t H = shapes[2 * t], W = shapes[2 * t + 1], S = starts[t];
        const bool ok = H >= 1 && W >= 1 && H <= Nv && W <= Nv && S >= 0 && S <= Nv &&
                        H * W <= (int64_t)Nv - S;
        s->lvl[t] = ok ? make_int4((int)H, (int)W, (int)S, 0) : make_int4(0, 0, 0, 0);
    }
    __syncthreads();
    if (t == 0) {
        int tb = 0;
        for (int l = 0; l < L; ++l) {
            int4 v = s->lvl[l];
            const int tw = (v.y + kTile - 1) >> kTileShift, th = (v.x + kTile - 1) >> kTileShift;
            int n = tw * th;
            if (n > nb_max - tb) {  // keep every bin inside the caller's workspace
                v = make_int4(0, 0, 0, 0);
                n = 0;
            }
            v.w = tb;
            s->lvl[l] = v;
            s->tw[l] = n ? tw : 0;
            tb += n;
        }
        s->nbins = tb;
    }
    __syncthreads();
}

// Neighbours of one sampling point, in the order TL (x0,y0), TR (x0+1,y0),
// BL (x0,y0+1), BR (x0+1,y0+1).
struct Neighbours {
    uint4 off;       // fp32-unit byte offsets of the rows in the batch slice, or kOOB
    float4 w;        // bilinear weights, 0 outside the map
    float fx, fy;    // fractional parts of the pixel coordinate
    int xi, yi;      // x0, y0 clamped to [-1, W] x [-1, H]
    uint32_t valid;  // bit c: neighbour c inside the map
};

__device__ __forceinline__ Neighbours neighbours(float u, float v, int4 lvl, uint32_t row_stride,
                                                 uint32_t head_off) {
    const int H = lvl.x, W = lvl.y, S = lvl.z;
    Neighbours n;
    // one rounding, the same as the CPU check: x = u*W - 0.5, y = v*H - 0.5
    const float x = __builtin_fmaf(u, (float)W, -0.5f);
    const float y = __builtin_fmaf(v, (float)H, -0.5f);
    const float x0 = floorf(x), y0 = floorf(y);
    n.fx = x - x0;
    n.fy = y - y0;
    // NaN compares false, so non-finite coordinates leave every neighbour out
    const bool vx0 = x0 >= 0.f && x0 <= (float)(W - 1);
    const bool vx1 = x0 >= -1.f && x0 <= (float)(W - 2);
    const bool vy0 = y0 >= 0.f && y0 <= (float)(H - 1);
    const bool vy1 = y0 >= -1.f && y0 <= (float)(H - 2);
    // clamp first so the conversion is defined for every input
    n.xi = (int)fminf(fmaxf(x0, -1.f), (float)W);
    n.yi = (int)fminf(fmaxf(y0, -1.f), (float)H);
    const int pTL = S + n.yi * W + n.xi;
    const uint32_t oTL = (uint32_t)pTL * row_stride + head_off;
    const bool vTL = vx0 && vy0, vTR = vx1 && vy0, vBL = vx0 && vy1, vBR = vx1 && vy1;
    n.off.x = vTL ? oTL : kOOB;
    n.off.y = vTR ? oTL + row_stride : kOOB;
    n.off.z = vBL ? oTL + (uint32_t)W * row_stride : kOOB;
    n.off.w = vBR ? oTL + (uint32_t)(W + 1) * row_stride : kOOB;
    const float gx = 1.f - n.fx, gy = 1.f - n.fy;
    n.w.x = vTL ? gx * gy : 0.f;
    n.w.y = vTR ? n.fx * gy : 0.f;
    n.w.z = vBL ? gx * n.fy : 0.f;
    n.w.w = vBR ? n.fx * n.fy : 0.f;
    n.valid = (vTL ? 1u : 0u) | (vTR ? 2u : 0u) | (vBL ? 4u : 0u) | (vBR ? 8u : 0u);
    return n;
}

// The distinct grad_value tiles (bins, relative to the (batch, head)) that
// hold at least one of the point's neighbours inside the map.
__device__ __forceinline__ int point_bins(const Neighbours &n, int4 lvl, int tw, int bins[4]) {
    if (!n.valid) return 0;
    const int tx0 = n.xi >> kTileShift, tx1 = (n.xi + 1) >> kTileShift;
    const int ty0 = n.yi >> kTileShift, ty1 = (n.yi + 1) >> kTileShift;
    const bool sx = tx1 != tx0, sy = ty1 != ty0;
    const bool vTL = n.valid & 1u, vTR = n.valid & 2u, vBL = n.valid & 4u, vBR = n.valid & 8u;
    int k = 0;
    if (vTL || (!sx && vTR) || (!sy && vBL) || (!sx && !sy && vBR))
        bins[k++] = lvl.w + ty0 * tw + tx0;
    if (sx && (vTR || (!sy && vBR))) bins[k++] = lvl.w + ty0 * tw + tx1;
    if (sy && (vBL || (!sx && vBR))) bins[k++] = lvl.w + ty1 * tw + tx0;
    if (sx && sy && vBR) bins[k++] = lvl.w + ty1 * tw + tx1;
    return k;
}

__device__ __forceinline__ void fma4(float4 &acc, float w, const float4 &v) {
    acc.x = __builtin_fmaf(w, v.x, acc.x);
    acc.y = __builtin_fmaf(w, v.y, acc.y);
    acc.z = __builtin_fmaf(w, v.z, acc.z);
    acc.w = __builtin_fmaf(w, v.w, acc.w);
}

__device__ __forceinline__ float dot4(const float4 &a, const float4 &b) {
    return __builtin_fmaf(a.w, b.w, __builtin_fmaf(a.z, b.z, __builtin_fmaf(a.y, b.y, a.x * b.x)));
}

__device__ __forceinline__ float pick(const float4 &v, int c) {
    return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

// Workgroup ids are dispatched round-robin over the 8 XCDs (workgroup k runs
// on XCD k % 8), and each XCD has its own L2.  Mapping id k to the logical
// index below gives every XCD one contiguous range of the work, so the value
// rows, grad_out rows and points one XCD touches stay together in its L2.
// The mapping is a permutation of [0, total): results never depend on it.
constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_contiguous(int k, int total) {
    const int per = total / kXcds, rem = total % kXcds;
    const int x = k % kXcds, j = k / kXcds;
    return x * per + min(x, rem) + j;
}

struct Dims {
    int Nv, Nq, M, L, K;
    int PC;      // points per chunk (point-table kernels)
    int PS;      // LDS stride per item (PC rounded to an odd count, for bank spread)
    int b0;      // first batch of this launch
    int nblk;    // workgroups per batch (forward) or per (batch, head) (backward)
    int nb_max;      // bin stride per (batch, head) in the workspace
    int accumulate;  // grad_value already holds a gradient to add to
};

// Workspace of the backward pipeline (all 32-bit words).
struct Work {
    uint32_t *counts;      // [B][nb_max][M] points per bin
    uint32_t *start;       // [B][nb_max][M] first entry of each bin in `sorted`
    uint32_t *cursor;      // [B][nb_max][M] next free entry while scattering
    uint2 *items;          // [work_max] (bin, chunk)
    uint32_t *work_total;  // [1]
    uint32_t *sorted;      // [4 * points] point indices grouped by bin
};

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <int D, typename VT>
__global__ void __launch_bounds__(kThreads)
msda_fwd_kernel(const VT *__restrict__ value, const int64_t *__restrict__ shapes,
                const int64_t *__restrict__ starts, const float *__restrict__ loc,
                const float *__restrict__ attn, float *__restrict__ out, Dims dm) {
    constexpr int G = D / 4;
    constexpr int IPB = kThreads / G;
    __shared__ LevelLds s_lv;
    extern __shared__ __align__(16) unsigned char smem[];
    uint4 *s_off = reinterpret_cast<uint4 *>(smem);
    float4 *s_w = reinterpret_cast<float4 *>(s_off + IPB * dm.PS);

    const int M = dm.M, K = dm.K, LK = dm.L * dm.K;
    const int NqM = dm.Nq * M;
    const int wg = xcd_contiguous(blockIdx.x, gridDim.x);
    const int b = wg / dm.nblk + dm.b0;
    const int item0 = (wg % dm.nblk) * IPB;
    const int nitems = min(IPB, NqM - item0);
    const uint32_t row_stride = (uint32_t)M * D * 4u;

    stage_levels(&s_lv, shapes, starts, dm.L, dm.Nv, 0x7fffffff);

    const size_t slice = (size_t)dm.Nv * M * D;
    const rsrc_t vr = make_rsrc(value + (size_t)b * slice, (uint32_t)(slice * sizeof(VT)));
    const size_t pt0 = ((size_t)b * NqM + item0) * LK;

    const int it = threadIdx.x / G, c = threadIdx.x % G;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);

    for (int j0 = 0; j0 < LK; j0 += dm.PC) {
        const int pc = min(dm.PC, LK - j0);
        if (j0) __syncthreads();  // previous chunk consumed
        for (int idx = threadIdx.x; idx < nitems * pc; idx += kThreads) {
            const int i1 = idx / pc, jj = idx - i1 * pc, j = j0 + jj;
            const size_t p = pt0 + (size_t)i1 * LK + j;
            const float2 uv = reinterpret_cast<const float2 *>(loc)[p];
            const float A = attn[p];
            const int m = (item0 + i1) % M;
            Neighbours n = neighbours(uv.x, uv.y, s_lv.lvl[j / K], row_stride,
                                      (uint32_t)m * D * 4u);
            s_off[i1 * dm.PS + jj] = n.off;
            // skip outside neighbours outright, so a non-finite A cannot leak through them
            s_w[i1 * dm.PS + jj] = make_float4((n.valid & 1u) ? A * n.w.x : 0.f,
                                               (n.valid & 2u) ? A * n.w.y : 0.f,
                                               (n.valid & 4u) ? A * n.w.z : 0.f,
                                               (n.valid & 8u) ? A * n.w.w : 0.f);
        }
        __syncthreads();
        if (it < nitems) {
            const uint4 *po = s_off + it * dm.PS;
            const float4 *pw = s_w + it * dm.PS;
#pragma unroll 4
            for (int jj = 0; jj < pc; ++jj) {
                const uint4 o = po[jj];
                const float4 w = pw[jj];
                const float4 v0 = Row4<VT>::load(vr, o.x, 4 * c);
                const float4 v1 = Row4<VT>::load(vr, o.y, 4 * c);
                const float4 v2 = Row4<VT>::load(vr, o.z, 4 * c);
                const float4 v3 = Row4<VT>::load(vr, o.w, 4 * c);
                fma4(acc, w.x, v0);
                fma4(acc, w.y, v1);
                fma4(acc, w.z, v2);
                fma4(acc, w.w, v3);
            }
        }
    }
    if (it < nitems) {
        float4 *o = reinterpret_cast<float4 *>(out + ((size_t)b * NqM + item0 + it) * D) + c;
        *o = acc;
    }
}

// ---------------------------------------------------------------------------
// backward 1: grad_attn_weight, grad_sampling_loc, bin counts
// Workgroup = (batch b, head m, IPB consecutive queries).
// ---------------------------------------------------------------------------
template <int D, typename VT>
__global__ void __launch_bounds__(kThreads)
bwd_dots_kernel(const VT *__restrict__ value, const int64_t *__restrict__ shapes,
                const int64_t *__restrict__ starts, const float *__restrict__ loc,
                const float *__restrict__ attn, const float *__restrict__ grad_out,
                float *__restrict__ grad_loc, float *__restrict__ grad_attn,
                uint32_t *__restrict__ counts, int hist_cap, Dims dm) {
    constexpr int G = D / 4;
    constexpr int IPB = kThreads / G;
    __shared__ LevelLds s_lv;
    extern __shared__ __align__(16) unsigned char smem[];
    uint4 *s_off = reinterpret_cast<uint4 *>(smem);
    float4 *s_w = reinterpret_cast<float4 *>(s_off + IPB * dm.PS);
    float4 *s_aux = s_w + IPB * dm.PS;    // (fx, fy, A, valid bits)
    float4 *s_dot = s_aux + IPB * dm.PS;  // <g, row> of the four neighbours
    uint32_t *s_hist = reinterpret_cast<uint32_t *>(s_dot + IPB * dm.PS);

    const int M = dm.M, K = dm.K, LK = dm.L * dm.K, Nq = dm.Nq;
    const int wg = xcd_contiguous(blockIdx.x, gridDim.x);
    const int bm = wg / dm.nblk + dm.b0 * M;
    const int m = bm % M, b = bm / M;
    const int q0 = (wg % dm.nblk) * IPB;
    const int nitems = min(IPB, Nq - q0);
    const uint32_t row_stride = (uint32_t)M * D * 4u;
    const uint32_t head_off = (uint32_t)m * D * 4u;

    stage_levels(&s_lv, shapes, starts, dm.L, dm.Nv, dm.nb_max);
    const int nbins = s_lv.nbins;
    const bool lds_hist = nbins <= hist_cap;
    // bins are laid out (batch, tile, head): tile i of this (b, m) is gcount[i * M]
    uint32_t *gcount = counts + (size_t)b * dm.nb_max * M + m;
    if (lds_hist)
        for (int i = threadIdx.x; i < nbins; i += kThreads) s_hist[i] = 0u;

    const size_t slice = (size_t)dm.Nv * M * D;
    const rsrc_t vr = make_rsrc(value + (size_t)b * slice, (uint32_t)(slice * sizeof(VT)));
    const size_t row0 = ((size_t)b * Nq + q0) * M + m;  // item row of query q0
    const size_t pt0 = row0 * LK;

    const int it = threadIdx.x / G, c = threadIdx.x % G;
    // The lane's grad_out row is read through a buffer load: with plain pointer
    // loads the load/store vectorizer of the ROCm 7.2 compiler merged a float4
    // element into a neighbouring scalar load's address chain (wrong channel).
    float4 g4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (it < nitems) {
        const rsrc_t go = make_rsrc(grad_out + row0 * D,
                                    (uint32_t)(((size_t)(nitems - 1) * M + 1) * D * 4));
        auto u = __builtin_amdgcn_raw_buffer_load_b128(
            go, (int)((uint32_t)it * M * D * 4u + 16u * c), 0, 0);
        g4 = make_float4(__uint_as_float(u[0]), __uint_as_float(u[1]), __uint_as_float(u[2]),
                         __uint_as_float(u[3]));
    }

    for (int j0 = 0; j0 < LK; j0 += dm.PC) {
        const int pc = min(dm.PC, LK - j0);
        __syncthreads();  // histogram zeroed / previous chunk consumed
        for (int idx = threadIdx.x; idx < nitems * pc; idx += kThreads) {
            const int i1 = idx / pc, jj = idx - i1 * pc, j = j0 + jj;
            const size_t p = pt0 + (size_t)i1 * M * LK + j;
            const float2 uv = reinterpret_cast<const float2 *>(loc)[p];
            const float A = attn[p];
            const int l = j / K;
            const int4 lvl = s_lv.lvl[l];
            Neighbours n = neighbours(uv.x, uv.y, lvl, row_stride, head_off);
            s_off[i1 * dm.PS + jj] = n.off;
            s_w[i1 * dm.PS + jj] = n.w;
            s_aux[i1 * dm.PS + jj] = make_float4(n.fx, n.fy, A, __uint_as_float(n.valid));
            int bins[4];
            const int nb = point_bins(n, lvl, s_lv.tw[l], bins);
            for (int k = 0; k < nb; ++k) {
                if (lds_hist)
                    atomicAdd(&s_hist[bins[k]], 1u);
                else
                    atomicAdd(&gcount[(size_t)bins[k] * M], 1u);
            }
        }
        __syncthreads();
        if (it < nitems) {
            const int base = it * dm.PS;
#pragma unroll 2
            for (int jj = 0; jj < pc; ++jj) {
                const uint4 o = s_off[base + jj];
                const float4 v0 = Row4<VT>::load(vr, o.x, 4 * c);
                const float4 v1 = Row4<VT>::load(vr, o.y, 4 * c);
                const float4 v2 = Row4<VT>::load(vr, o.z, 4 * c);
                const float4 v3 = Row4<VT>::load(vr, o.w, 4 * c);
                const float d0 = group_sum<G>(dot4(g4, v0));
                const float d1 = group_sum<G>(dot4(g4, v1));
                const float d2 = group_sum<G>(dot4(g4, v2));
                const float d3 = group_sum<G>(dot4(g4, v3));
                if (c == 0) s_dot[base + jj] = make_float4(d0, d1, d2, d3);
            }
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < nitems * pc; idx += kThreads) {
            const int i1 = idx / pc, jj = idx - i1 * pc, j = j0 + jj;
            const size_t p = pt0 + (size_t)i1 * M * LK + j;
            const float4 d = s_dot[i1 * dm.PS + jj];
            const float4 w = s_w[i1 * dm.PS + jj];
            const float4 ax = s_aux[i1 * dm.PS + jj];
            const int4 lvl = s_lv.lvl[j / K];
            float ga = 0.f, gx = 0.f, gy = 0.f;
            if (__float_as_uint(ax.w) != 0u) {
                const float fx = ax.x, fy = ax.y, A = ax.z;
                ga = w.x * d.x + w.y * d.y + w.z * d.z + w.w * d.w;
                gx = A * (float)lvl.y * ((1.f - fy) * (d.y - d.x) + fy * (d.w - d.z));
                gy = A * (float)lvl.x * ((1.f - fx) * (d.z - d.x) + fx * (d.w - d.y));
            }
            grad_attn[p] = ga;
            reinterpret_cast<float2 *>(grad_loc)[p] = make_float2(gx, gy);
        }
    }
    if (lds_hist) {
        __syncthreads();
        for (int i = threadIdx.x; i < nbins; i += kThreads) {
            const uint32_t v = s_hist[i];
            if (v) atomicAdd(&gcount[(size_t)i * M], v);
        }
    }
}

// ---------------------------------------------------------------------------
// backward 2: scan of the bin counts, work list of (bin, chunk)
// One workgroup of kScanThreads; bins are visited in (batch, head, bin) order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void block_exclusive_scan2(uint32_t &a, uint32_t &b, uint32_t *s_a,
                                                      uint32_t *s_b, uint32_t &tot_a,
                                                      uint32_t &tot_b) {
    const int t = threadIdx.x;
    s_a[t] = a;
    s_b[t] = b;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
        const uint32_t xa = t >= off ? s_a[t - off] : 0u;
        const uint32_t xb = t >= off ? s_b[t - off] : 0u;
        __syncthreads();
        s_a[t] += xa;
        s_b[t] += xb;
        __syncthreads();
    }
    tot_a = s_a[kScanThreads - 1];
    tot_b = s_b[kScanThreads - 1];
    a = s_a[t] - a;  // exclusive
    b = s_b[t] - b;
    __syncthreads();
}

__global__ void __launch_bounds__(kScanThreads)
bin_scan_kernel(const int64_t *__restrict__ shapes, const int64_t *__restrict__ starts,
                const uint32_t *__restrict__ counts, uint32_t *__restrict__ start,
                uint32_t *__restrict__ cursor, uint2 *__restrict__ items,
                uint32_t *__restrict__ work_total, int B, Dims dm) {
    constexpr int kPer = 8;
    __shared__ LevelLds s_lv;
    __shared__ uint32_t s_a[kScanThreads], s_b[kScanThreads];
    stage_levels(&s_lv, shapes, starts, dm.L, dm.Nv, dm.nb_max);
    const int nbins = s_lv.nbins;
    // bins in (batch, tile, head) order; entry g maps to bin (b*nb_max + tile)*M + m
    const int64_t per_b = (int64_t)nbins * dm.M;
    const int64_t n = (int64_t)B * per_b;
    uint32_t carry_e = 0, carry_c = 0;
    for (int64_t base = 0; base < n; base += (int64_t)kScanThreads * kPer) {
        uint32_t cnt[kPer], e = 0, ch = 0;
        const int64_t g0 = base + (int64_t)threadIdx.x * kPer;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int64_t g = g0 + i;
            cnt[i] = 0;
            if (g < n) cnt[i] = counts[(g / per_b) * dm.nb_max * dm.M + g % per_b];
            e += cnt[i];
            ch += (cnt[i] + kChunk - 1) / kChunk;
        }
        uint32_t tot_e, tot_c;
        block_exclusive_scan2(e, ch, s_a, s_b, tot_e, tot_c);
        e += carry_e;
        ch += carry_c;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int64_t g = g0 + i;
            if (g < n) {
                const uint32_t bin = (uint32_t)((g / per_b) * dm.nb_max * dm.M + g % per_b);
                start[bin] = e;
                cursor[bin] = e;
                const uint32_t nch = (cnt[i] + kChunk - 1) / kChunk;
                for (uint32_t k = 0; k < nch; ++k) items[ch + k] = make_uint2(bin, k);
                e += cnt[i];
                ch += nch;
            }
        }
        carry_e += tot_e;
        carry_c += tot_c;
    }
    if (threadIdx.x == 0) *work_total = carry_c;
}

// ---------------------------------------------------------------------------
// backward 3: scatter point indices into their bins
// Workgroup = (batch b, head m, kScatterQueries consecutive queries).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads)
bin_scatter_kernel(const int64_t *__restrict__ shapes, const int64_t *__restrict__ starts,
                   const float *__restrict__ loc, uint32_t *__restrict__ cursor,
                   uint32_t *__restrict__ sorted, int hist_cap, Dims dm) {
    __shared__ LevelLds s_lv;
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *s_cnt = reinterpret_cast<uint32_t *>(smem);  // [hist_cap] counts, then ranks
    uint32_t *s_base = s_cnt + hist_cap;                    // [hist_cap] reserved offsets

    const int M = dm.M, K = dm.K, LK = dm.L * dm.K, Nq = dm.Nq;
    const int wg = xcd_contiguous(blockIdx.x, gridDim.x);
    const int bm = wg / dm.nblk + dm.b0 * M;
    const int m = bm % M, b = bm / M;
    const int q0 = (wg % dm.nblk) * kScatterQueries;
    const int nq = min(kScatterQueries, Nq - q0);
    const size_t row0 = ((size_t)b * Nq + q0) * M + m;
    const int npts = nq * LK;

    stage_levels(&s_lv, shapes, starts, dm.L, dm.Nv, dm.nb_max);
    const int nbins = s_lv.nbins;
    uint32_t *gcur = cursor + (size_t)b * dm.nb_max * M + m;  // tile i at gcur[i * M]
    if (nbins > hist_cap) {  // too many bins for LDS: reserve one slot at a time
        for (int idx = threadIdx.x; idx < npts; idx += kThreads) {
            const int i1 = idx / LK, j = idx - i1 * LK;
            const size_t p = (row0 + (size_t)i1 * M) * LK + j;
            const float2 uv = reinterpret_cast<const float2 *>(loc)[p];
            const int l = j / K;
            Neighbours n = neighbours(uv.x, uv.y, s_lv.lvl[l], 0u, 0u);
            int bins[4];
            const int nb = point_bins(n, s_lv.lvl[l], s_lv.tw[l], bins);
            for (int k = 0; k < nb; ++k)
                sorted[atomicAdd(&gcur[(size_t)bins[k] * M], 1u)] = (uint32_t)p;
        }
        return;
    }
    for (int i = threadIdx.x; i < nbins; i += kThreads) s_cnt[i] = 0u;
    __syncthreads();
    for (int idx = threadIdx.x; idx < npts; idx += kThreads) {
        const int i1 = idx / LK, j = idx - i1 * LK;
        const size_t p = (row0 + (size_t)i1 * M) * LK + j;
        const float2 uv = reinterpret_cast<const float2 *>(loc)[p];
        const int l = j / K;
        Neighbours n = neighbours(uv.x, uv.y, s_lv.lvl[l], 0u, 0u);
        int bins[4];
        const int nb = point_bins(n, s_lv.lvl[l], s_lv.tw[l], bins);
        for (int k = 0; k < nb; ++k) atomicAdd(&s_cnt[bins[k]], 1u);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nbins; i += kThreads) {
        const uint32_t v = s_cnt[i];
        s_base[i] = v ? atomicAdd(&gcur[(size_t)i * M], v) : 0u;
        s_cnt[i] = 0u;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < npts; idx += kThreads) {
        const int i1 = idx / LK, j = idx - i1 * LK;
        const size_t p = (row0 + (size_t)i1 * M) * LK + j;
        const float2 uv = reinterpret_cast<const float2 *>(loc)[p];
        const int l = j / K;
        Neighbours n = neighbours(uv.x, uv.y, s_lv.lvl[l], 0u, 0u);
        int bins[4];
        const int nb = point_bins(n, s_lv.lvl[l], s_lv.tw[l], bins);
        for (int k = 0; k < nb; ++k)
            sorted[s_base[bins[k]] + atomicAdd(&s_cnt[bins[k]], 1u)] = (uint32_t)p;
    }
}

// ---------------------------------------------------------------------------
// backward 4: grad_value, one 8x8 tile (and chunk of its points) per work item
//
// The chunk is walked in sub-chunks of kSubRows(D) points.  For each, the
// points' grad_out rows are staged in LDS (one read of each row), and the
// points are counting-sorted in LDS by the cell of their top-left neighbour
// (a 9x9 grid: the tile plus one column and row before it).  Pixel (x, y) of
// the tile receives from the points of four cells, in four roles: top-left
// from cell (x, y), top-right from (x-1, y), bottom-left from (x, y-1),
// bottom-right from (x-1, y-1).  A lane owns (pixel, 4-channel quad) pairs
// and sums A * w * grad_out over those lists in registers across all
// sub-chunks, so no two lanes ever add into the same value and the loop
// iterations are independent.  Each pixel is written once per work item.
// ---------------------------------------------------------------------------
constexpr int kTileThreads = 512;
constexpr int kCellsW = kTile + 1;
constexpr int kCells = kCellsW * kCellsW;
constexpr int kStageBytes = 32 * 1024;  // grad_out rows staged per sub-chunk

template <int D>
__global__ void __launch_bounds__(kTileThreads)
grad_value_tile_kernel(const int64_t *__restrict__ shapes, const int64_t *__restrict__ starts,
                       const float *__restrict__ loc, const float *__restrict__ attn,
                       const float *__restrict__ grad_out, const uint32_t *__restrict__ counts,
                       const uint32_t *__restrict__ start, const uint2 *__restrict__ items,
                       const uint32_t *__restrict__ work_total,
                       const uint32_t *__restrict__ sorted, float *__restrict__ grad_value,
                       Dims dm) {
    constexpr int kQuads = D / 4;
    constexpr int kSub = kStageBytes / (D * 4) < 512 ? kStageBytes / (D * 4) : 512;  // points per sub-chunk
    constexpr int kOwn = (kTilePx * kQuads + kTileThreads - 1) / kTileThreads;  // pairs per lane
    __shared__ LevelLds s_lv;
    __shared__ float4 s_g[kSub * kQuads];  // staged grad_out rows
    __shared__ float4 s_w[kSub];           // A * bilinear weight of each neighbour
    __shared__ uint32_t s_item[kSub];      // (b, q, m) row of the point
    __shared__ uint16_t s_cell[kSub];      // cell of the point's top-left neighbour
    __shared__ uint16_t s_ent[kSub];       // points ordered by cell
    __shared__ uint32_t s_cnt[kCells + 1];
    __shared__ uint32_t s_cur[kCells];

    const int M = dm.M, LK = dm.L * dm.K;
    stage_levels(&s_lv, shapes, starts, dm.L, dm.Nv, dm.nb_max);
    const uint32_t total = *work_total;
    const int tid = threadIdx.x;
    // The work list is in (batch, level, tile, head) order and workgroup k
    // (dispatched to XCD k % 8) takes items k, k + grid, ...  With 8 heads the
    // XCDs therefore split the work by head: every XCD gets the same mix of
    // tiles, and the grad_out rows it gathers are those of one head.
    for (uint32_t w = blockIdx.x; w < total; w += gridDim.x) {
        const uint2 wk = items[w];
        const uint32_t bin = wk.x;  // (b * nb_max + tile) * M + m
        const int m = (int)(bin % (uint32_t)M);
        const uint32_t bt = bin / (uint32_t)M;
        const int b = (int)(bt / (uint32_t)dm.nb_max);
        const int lb = (int)(bt - (uint32_t)b * dm.nb_max);
        int l = 0;
        while (l + 1 < dm.L && s_lv.lvl[l + 1].w <= lb) ++l;
        const int4 lvl = s_lv.lvl[l];
        const int tw = s_lv.tw[l];
        const int ty = (lb - lvl.w) / tw, tx = (lb - lvl.w) - ty * tw;
        const int x0t = tx * kTile, y0t = ty * kTile;
        const uint32_t cnt = counts[bin];
        const uint32_t s0 = start[bin] + wk.y * kChunk;
        const int n = (int)min((uint32_t)kChunk, cnt - wk.y * kChunk);
        const bool whole = cnt <= (uint32_t)kChunk;

        float4 acc[kOwn];
#pragma unroll
        for (int o = 0; o < kOwn; ++o) acc[o] = make_float4(0.f, 0.f, 0.f, 0.f);

        for (int sub = 0; sub < n; sub += kSub) {
            const int ns = min(kSub, n - sub);
            for (int i = tid; i < kCells; i += kTileThreads) s_cnt[i] = 0u;
            __syncthreads();
            for (int i = tid; i < ns; i += kTileThreads) {
                const uint32_t p = sorted[s0 + sub + i];
                const float2 uv = reinterpret_cast<const float2 *>(loc)[p];
                const float A = attn[p];
                const Neighbours nb = neighbours(uv.x, uv.y, lvl, 0u, 0u);
                // a point of this bin has a neighbour inside the tile, so its
                // top-left neighbour lies in the 9x9 cell grid
                const int cx = nb.xi - x0t + 1, cy = nb.yi - y0t + 1;
                const bool inside = cx >= 0 && cx < kCellsW && cy >= 0 && cy < kCellsW;
                const int cell = inside ? cx + cy * kCellsW : 0;
                s_cell[i] = (uint16_t)cell;
                s_w[i] = inside ? make_float4(A * nb.w.x, A * nb.w.y, A * nb.w.z, A * nb.w.w)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
                s_item[i] = p / (uint32_t)LK;
                atomicAdd(&s_cnt[cell], 1u);
            }
            __syncthreads();
            for (int i = tid; i < ns * kQuads; i += kTileThreads) {
                const int pt = i / kQuads, q = i - pt * kQuads;
                s_g[i] = reinterpret_cast<const float4 *>(grad_out + (size_t)s_item[pt] * D)[q];
            }
            if (tid < 64) {  // exclusive scan of the 81 cell counts by one wave, 2 cells a lane
                const int c0 = 2 * tid, c1 = 2 * tid + 1;
                const uint32_t v0 = c0 < kCells ? s_cnt[c0] : 0u;
                const uint32_t v1 = c1 < kCells ? s_cnt[c1] : 0u;
                uint32_t incl = v0 + v1;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const uint32_t t = __shfl_up(incl, off, 64);
                    if (tid >= off) incl += t;
                }
                const uint32_t ex = incl - v0 - v1;
                if (c0 < kCells) {
                    s_cnt[c0] = ex;
                    s_cur[c0] = ex;
                }
                if (c1 < kCells) {
                    s_cnt[c1] = ex + v0;
                    s_cur[c1] = ex + v0;
                }
                if (tid == 63) s_cnt[kCells] = incl;
            }
            __syncthreads();
            for (int i = tid; i < ns; i += kTileThreads)
                s_ent[atomicAdd(&s_cur[s_cell[i]], 1u)] = (uint16_t)i;
            __syncthreads();
#pragma unroll
            for (int o = 0; o < kOwn; ++o) {
                const int pair = tid + o * kTileThreads;
                if (pair >= kTilePx * kQuads) break;
                const int px = pair / kQuads, q = pair - px * kQuads;
                const int x = px & (kTile - 1), y = px >> kTileShift;
#pragma unroll
                for (int role = 0; role < 4; ++role) {
                    const int cell = (x - (role & 1) + 1) + (y - (role >> 1) + 1) * kCellsW;
                    const int e0 = (int)s_cnt[cell], e1 = (int)s_cnt[cell + 1];
#pragma unroll 4
                    for (int e = e0; e < e1; ++e) {
                        const int pt = s_ent[e];
                        fma4(acc[o], pick(s_w[pt], role), s_g[pt * kQuads + q]);
                    }
                }
            }
            __syncthreads();  // the tables are rebuilt for the next sub-chunk
        }

        const size_t slice = (size_t)dm.Nv * M * D;
        float *gv = grad_value + (size_t)b * slice + (size_t)m * D;
#pragma unroll
        for (int o = 0; o < kOwn; ++o) {
            const int pair = tid + o * kTileThreads;
            if (pair >= kTilePx * kQuads) break;
            const int px = pair / kQuads, q = pair - px * kQuads;
            const int gx = x0t + (px & (kTile - 1)), gy = y0t + (px >> kTileShift);
            if (gy >= lvl.x || gx >= lvl.y) continue;
            float *dst = gv + (size_t)(lvl.z + gy * lvl.y + gx) * M * D + 4 * q;
            float4 a = acc[o];
            if (whole) {
                // this work item alone owns the pixel: plain read-add-write
                float4 *d4 = reinterpret_cast<float4 *>(dst);
                if (dm.accumulate) {
                    const float4 v = *d4;
                    a.x += v.x;
                    a.y += v.y;
                    a.z += v.z;
                    a.w += v.w;
                }
                *d4 = a;
            } else {
                atomicAdd(dst + 0, a.x);
                atomicAdd(dst + 1, a.y);
                atomicAdd(dst + 2, a.z);
                atomicAdd(dst + 3, a.w);
            }
        }
    }
}

__global__ void __launch_bounds__(kThreads) fill_zero_kernel(float4 *__restrict__ p, size_t n4) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride)
        p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
thread_local int g_last_hip_error = 0;

bool supported_d(int64_t D) {
    return D == 4 || D == 8 || D == 16 || D == 32 || D == 64 || D == 128 || D == 256;
}

msda_status check_sizes(int value_dtype, int64_t B, int64_t Nv, int64_t Nq, int64_t M,
                        int64_t D, int64_t L, int64_t K) {
    if (value_dtype != MSDA_F32 && value_dtype != MSDA_BF16) return MSDA_ERR_DTYPE;
    if (B < 0 || Nv < 0 || Nq < 0 || M < 1 || D < 1 || L < 1 || K < 1) return MSDA_ERR_SHAPE;
    if (L > kMaxLevels || !supported_d(D)) return MSDA_ERR_UNSUPPORTED;
    const int64_t lim = (int64_t)1 << 31;
    // the rows of one workgroup's queries stay 31-bit addressable
    if (M > ((int64_t)1 << 20) / D) return MSDA_ERR_UNSUPPORTED;
    // one batch slice of grad_value (fp32) and of the point arrays must be 31-bit addressable
    if (Nv > lim / (M * D * 4) || Nv * M * D * 4 >= lim) return MSDA_ERR_UNSUPPORTED;
    if (K > lim / L || Nq > lim / (M * L * K * 2) || Nq * M * L * K * 2 >= lim)
        return MSDA_ERR_UNSUPPORTED;
    // the backward stores point indices of the whole problem, four per point, in 32 bits
    if (B > 0 && Nq > 0 && B > (((int64_t)1 << 32) - 1) / (Nq * M * L * K * 4))
        return MSDA_ERR_UNSUPPORTED;
    // one launch covers Nq*M items with D/4 lanes each: keep the grid under 2^31 threads
    if (Nq * M > lim / (D / 4)) return MSDA_ERR_UNSUPPORTED;
    return MSDA_OK;
}

// Upper bound of the number of 8x8 tiles over all levels, from Nv and L only:
// sum ceil(H/8)*ceil(W/8) <= sum (HW + 7(H+W) + 49)/64 <= (15 Nv + 49 L)/64.
int64_t bins_bound(int64_t Nv, int64_t L) { return (15 * Nv + 49 * L) / 64 + 1; }

struct WorkLayout {
    int64_t nb_max, bm_bins, work_max, sorted_max;
    size_t off_counts, off_start, off_cursor, off_items, off_total, off_sorted, bytes;
};

WorkLayout work_layout(int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t L, int64_t K) {
    WorkLayout w;
    w.nb_max = bins_bound(Nv, L);
    w.bm_bins = B * M * w.nb_max;
    const int64_t pts = B * Nq * M * L * K;
    w.sorted_max = 4 * pts;
    w.work_max = w.bm_bins + (w.sorted_max + kChunk - 1) / kChunk;
    auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
    size_t o = 0;
    w.off_counts = o;
    o = align(o + 4 * (size_t)w.bm_bins);
    w.off_start = o;
    o = align(o + 4 * (size_t)w.bm_bins);
    w.off_cursor = o;
    o = align(o + 4 * (size_t)w.bm_bins);
    w.off_items = o;
    o = align(o + 8 * (size_t)w.work_max);
    w.off_total = o;
    o = align(o + 4);
    w.off_sorted = o;
    o = align(o + 4 * (size_t)w.sorted_max);
    w.bytes = o;
    return w;
}

struct Launch {
    int ipb, pc, ps;
    size_t lds;
};

Launch plan(int64_t D, int64_t L, int64_t K, int bytes_per_point) {
    Launch p;
    p.ipb = (int)(kThreads / (D / 4));
    const int lk = (int)(L * K);
    int pc = kSetupLdsBytes / (p.ipb * bytes_per_point) - 2;
    pc = pc < 1 ? 1 : pc;
    p.pc = pc < lk ? pc : lk;
    p.ps = p.pc + ((p.pc % 2 == 0) ? 1 : 2);
    p.lds = (size_t)p.ipb * p.ps * bytes_per_point;
    return p;
}

msda_status hip_status(hipError_t e) {
    if (e == hipSuccess) return MSDA_OK;
    g_last_hip_error = (int)e;
    return MSDA_ERR_HIP;
}

// Batches per launch so that a 1-D grid of per_batch workgroups per batch
// stays below 2^23 workgroups (2^31 threads).
int64_t batch_chunk(int64_t per_batch, int64_t B) {
    int64_t c = ((int64_t)1 << 23) / (per_batch > 0 ? per_batch : 1);
    c = c < 1 ? 1 : c;
    return c < B ? c : B;
}

template <int D, typename VT>
msda_status launch_fwd(const void *value, const int64_t *shapes, const int64_t *starts,
                       const float *loc, const float *attn, float *out, int64_t B, int64_t Nv,
                       int64_t Nq, int64_t M, int64_t L, int64_t K, hipStream_t s) {
    const Launch p = plan(D, L, K, 32);
    const int64_t items = Nq * M;
    const int64_t gx = (items + p.ipb - 1) / p.ipb;
    const int64_t bchunk = batch_chunk(gx, B);
    for (int64_t b0 = 0; b0 < B; b0 += bchunk) {
        const int64_t nb = (B - b0) < bchunk ? (B - b0) : bchunk;
        Dims dm{(int)Nv, (int)Nq, (int)M, (int)L, (int)K, p.pc, p.ps, (int)b0, (int)gx, 0, 0};
        hipLaunchKernelGGL((msda_fwd_kernel<D, VT>), dim3((unsigned)(gx * nb)), dim3(kThreads),
                           p.lds, s, static_cast<const VT *>(value), shapes, starts, loc, attn,
                           out, dm);
        msda_status st = hip_status(hipGetLastError());
        if (st != MSDA_OK) return st;
    }
    return MSDA_OK;
}

// Zero n4 float4s (16-byte units) at p.
msda_status fill_zero(void *p, size_t n4, hipStream_t s) {
    if (n4 == 0) return MSDA_OK;
    size_t blocks = (n4 + kThreads - 1) / kThreads;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       reinterpret_cast<float4 *>(p), n4);
    return hip_status(hipGetLastError());
}

template <int D, typename VT>
msda_status launch_bwd(const void *value, const int64_t *shapes, const int64_t *starts,
                       const float *loc, const float *attn, const float *gout, float *gval,
                       float *gloc, float *gattn, int64_t B, int64_t Nv, int64_t Nq, int64_t M,
                       int64_t L, int64_t K, const WorkLayout &wl, unsigned char *ws,
                       bool accumulate, hipStream_t s, hipEvent_t *ev) {
    // ev (optional): events recorded before each stage, for msda_backward_timed
    auto mark = [&](int i) {
        if (ev) (void)hipEventRecord(ev[i], s);
    };
    Work w;
    w.counts = reinterpret_cast<uint32_t *>(ws + wl.off_counts);
    w.start = reinterpret_cast<uint32_t *>(ws + wl.off_start);
    w.cursor = reinterpret_cast<uint32_t *>(ws + wl.off_cursor);
    w.items = reinterpret_cast<uint2 *>(ws + wl.off_items);
    w.work_total = reinterpret_cast<uint32_t *>(ws + wl.off_total);
    w.sorted = reinterpret_cast<uint32_t *>(ws + wl.off_sorted);
    // the counts region is padded to 256 bytes, so whole float4s can be cleared
    mark(1);
    msda_status st = fill_zero(w.counts, (wl.off_start - wl.off_counts) / 16, s);
    if (st != MSDA_OK) return st;

    const int hist_cap = (int)(wl.nb_max < kHistLds ? wl.nb_max : kHistLds);
    const Launch p = plan(D, L, K, 64);
    const int64_t gq = (Nq + p.ipb - 1) / p.ipb;
    const int64_t gs = (Nq + kScatterQueries - 1) / kScatterQueries;
    int64_t bchunk = batch_chunk(gq * M, B);
    mark(2);
    for (int64_t b0 = 0; b0 < B; b0 += bchunk) {
        const int64_t nb = (B - b0) < bchunk ? (B - b0) : bchunk;
        Dims dm{(int)Nv, (int)Nq, (int)M, (int)L, (int)K, p.pc, p.ps, (int)b0, (int)gq,
                (int)wl.nb_max, 0};
        hipLaunchKernelGGL((bwd_dots_kernel<D, VT>), dim3((unsigned)(gq * M * nb)),
                           dim3(kThreads), p.lds + 4 * (size_t)hist_cap, s,
                           static_cast<const VT *>(value), shapes, starts, loc, attn, gout, gloc,
                           gattn, w.counts, hist_cap, dm);
        st = hip_status(hipGetLastError());
        if (st != MSDA_OK) return st;
    }
    Dims dm{(int)Nv, (int)Nq, (int)M, (int)L, (int)K, 0, 0, 0, 0, (int)wl.nb_max,
            accumulate ? 1 : 0};
    mark(3);
    hipLaunchKernelGGL(bin_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, shapes, starts,
                       w.counts, w.start, w.cursor, w.items, w.work_total, (int)B, dm);
    st = hip_status(hipGetLastError());
    if (st != MSDA_OK) return st;
    bchunk = batch_chunk(gs * M, B);
    mark(4);
    for (int64_t b0 = 0; b0 < B; b0 += bchunk) {
        const int64_t nb = (B - b0) < bchunk ? (B - b0) : bchunk;
        Dims d2 = dm;
        d2.b0 = (int)b0;
        d2.nblk = (int)gs;
        hipLaunchKernelGGL(bin_scatter_kernel, dim3((unsigned)(gs * M * nb)), dim3(kThreads),
                           8 * (size_t)hist_cap, s, shapes, starts, loc, w.cursor, w.sorted,
                           hist_cap, d2);
        st = hip_status(hipGetLastError());
        if (st != MSDA_OK) return st;
    }
    const int64_t grid = wl.work_max < kTileGrid ? wl.work_max : kTileGrid;
    mark(5);
    hipLaunchKernelGGL((grad_value_tile_kernel<D>), dim3((unsigned)grid), dim3(kTileThreads), 0, s,
                       shapes, starts, loc, attn, gout, w.counts, w.start, w.items,
                       w.work_total, w.sorted, gval, dm);
    st = hip_status(hipGetLastError());
    mark(6);
    return st;
}

template <typename VT>
msda_status dispatch_fwd(int64_t D, const void *value, const int64_t *shapes,
                         const int64_t *starts, const float *loc, const float *attn, float *out,
                         int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t L, int64_t K,
                         hipStream_t s) {
#define MSDA_FWD_CASE(DD)                                                                     \
    case DD:                                                                                  \
        return launch_fwd<DD, VT>(value, shapes, starts, loc, attn, out, B, Nv, Nq, M, L, K, s);
    switch (D) {
        MSDA_FWD_CASE(4)
        MSDA_FWD_CASE(8)
        MSDA_FWD_CASE(16)
        MSDA_FWD_CASE(32)
        MSDA_FWD_CASE(64)
        MSDA_FWD_CASE(128)
        MSDA_FWD_CASE(256)
    default: return MSDA_ERR_UNSUPPORTED;
    }
#undef MSDA_FWD_CASE
}

template <typename VT>
msda_status dispatch_bwd(int64_t D, const void *value, const int64_t *shapes,
                         const int64_t *starts, const float *loc, const float *attn,
                         const float *gout, float *gval, float *gloc, float *gattn, int64_t B,
                         int64_t Nv, int64_t Nq, int64_t M, int64_t L, int64_t K,
                         const WorkLayout &wl, unsigned char *ws, bool acc, hipStream_t s,
                         hipEvent_t *ev) {
#define MSDA_BWD_CASE(DD)                                                                      \
    case DD:                                                                                   \
        return launch_bwd<DD, VT>(value, shapes, starts, loc, attn, gout, gval, gloc, gattn, B, \
                                  Nv, Nq, M, L, K, wl, ws, acc, s, ev);
    switch (D) {
        MSDA_BWD_CASE(4)
        MSDA_BWD_CASE(8)
        MSDA_BWD_CASE(16)
        MSDA_BWD_CASE(32)
        MSDA_BWD_CASE(64)
        MSDA_BWD_CASE(128)
        MSDA_BWD_CASE(256)
    default: return MSDA_ERR_UNSUPPORTED;
    }
#undef MSDA_BWD_CASE
}

}  // namespace

extern "C" {

msda_status msda_forward(const void *value, int value_dtype, const int64_t *spatial_shapes,
                         const int64_t *level_start_index, const float *sampling_loc,
                         const float *attn_weight, float *out, int64_t B, int64_t Nv,
                         int64_t Nq, int64_t M, int64_t D, int64_t L, int64_t K, void *stream) {
    msda_status st = check_sizes(value_dtype, B, Nv, Nq, M, D, L, K);
    if (st != MSDA_OK) return st;
    if (B == 0 || Nq == 0) return MSDA_OK;
    if (Nv < 1) return MSDA_ERR_SHAPE;
    if (!value || !spatial_shapes || !level_start_index || !sampling_loc || !attn_weight || !out)
        return MSDA_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (value_dtype == MSDA_F32)
        return dispatch_fwd<float>(D, value, spatial_shapes, level_start_index, sampling_loc,
                                   attn_weight, out, B, Nv, Nq, M, L, K, s);
    return dispatch_fwd<uint16_t>(D, value, spatial_shapes, level_start_index, sampling_loc,
                                  attn_weight, out, B, Nv, Nq, M, L, K, s);
}

size_t msda_backward_workspace_size(int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                                    int64_t L, int64_t K) {
    if (check_sizes(MSDA_F32, B, Nv, Nq, M, D, L, K) != MSDA_OK) return 0;
    if (B == 0 || Nq == 0) return 0;
    return work_layout(B, Nv, Nq, M, L, K).bytes;
}

}  // extern "C"

namespace {

msda_status backward_impl(const void *value, int value_dtype, const int64_t *spatial_shapes,
                          const int64_t *level_start_index, const float *sampling_loc,
                          const float *attn_weight, const float *grad_out, float *grad_value,
                          float *grad_sampling_loc, float *grad_attn_weight, int64_t B,
                          int64_t Nv, int64_t Nq, int64_t M, int64_t D, int64_t L, int64_t K,
                          void *workspace, size_t workspace_bytes, uint32_t flags,
                          hipStream_t s, hipEvent_t *ev) {
    msda_status st = check_sizes(value_dtype, B, Nv, Nq, M, D, L, K);
    if (st != MSDA_OK) return st;
    if (flags & ~MSDA_BWD_ACCUMULATE) return MSDA_ERR_UNSUPPORTED;
    const int64_t nval = B * Nv * M * D;
    if (nval > 0 && !grad_value) return MSDA_ERR_NULL;
    const bool work = B > 0 && Nq > 0;
    WorkLayout wl{};
    if (work) {
        if (Nv < 1) return MSDA_ERR_SHAPE;
        if (!value || !spatial_shapes || !level_start_index || !sampling_loc || !attn_weight ||
            !grad_out || !grad_sampling_loc || !grad_attn_weight)
            return MSDA_ERR_NULL;
        wl = work_layout(B, Nv, Nq, M, L, K);
        if (!workspace) return MSDA_ERR_NULL;
        if (workspace_bytes < wl.bytes) return MSDA_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return MSDA_ERR_WORKSPACE;
    }
    if (ev) (void)hipEventRecord(ev[0], s);
    if (!(flags & MSDA_BWD_ACCUMULATE)) {
        st = fill_zero(grad_value, (size_t)nval / 4, s);  // D is a multiple of 4
        if (st != MSDA_OK) return st;
    }
    if (!work) {
        if (ev)
            for (int i = 1; i < 7; ++i) (void)hipEventRecord(ev[i], s);
        return MSDA_OK;
    }
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    const bool acc = (flags & MSDA_BWD_ACCUMULATE) != 0;
    if (value_dtype == MSDA_F32)
        return dispatch_bwd<float>(D, value, spatial_shapes, level_start_index, sampling_loc,
                                   attn_weight, grad_out, grad_value, grad_sampling_loc,
                                   grad_attn_weight, B, Nv, Nq, M, L, K, wl, ws, acc, s, ev);
    return dispatch_bwd<uint16_t>(D, value, spatial_shapes, level_start_index, sampling_loc,
                                  attn_weight, grad_out, grad_value, grad_sampling_loc,
                                  grad_attn_weight, B, Nv, Nq, M, L, K, wl, ws, acc, s, ev);
}

}  // namespace

extern "C" {

msda_status msda_backward(const void *value, int value_dtype, const int64_t *spatial_shapes,
                          const int64_t *level_start_index, const float *sampling_loc,
                          const float *attn_weight, const float *grad_out, float *grad_value,
                          float *grad_sampling_loc, float *grad_attn_weight, int64_t B,
                          int64_t Nv, int64_t Nq, int64_t M, int64_t D, int64_t L, int64_t K,
                          void *workspace, size_t workspace_bytes, uint32_t flags,
                          void *stream) {
    return backward_impl(value, value_dtype, spatial_shapes, level_start_index, sampling_loc,
                         attn_weight, grad_out, grad_value, grad_sampling_loc, grad_attn_weight,
                         B, Nv, Nq, M, D, L, K, workspace, workspace_bytes, flags,
                         static_cast<hipStream_t>(stream), nullptr);
}

msda_status msda_backward_timed(const void *value, int value_dtype,
                                const int64_t *spatial_shapes, const int64_t *level_start_index,
                                const float *sampling_loc, const float *attn_weight,
                                const float *grad_out, float *grad_value,
                                float *grad_sampling_loc, float *grad_attn_weight, int64_t B,
                                int64_t Nv, int64_t Nq, int64_t M, int64_t D, int64_t L,
                                int64_t K, void *workspace, size_t workspace_bytes,
                                uint32_t flags, void *stream, float *stage_us) {
    if (!stage_us) return MSDA_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t ev[7];
    int made = 0;
    msda_status st = MSDA_OK;
    for (; made < 7; ++made) {
        st = hip_status(hipEventCreate(&ev[made]));
        if (st != MSDA_OK) break;
    }
    if (st == MSDA_OK) {
        st = backward_impl(value, value_dtype, spatial_shapes, level_start_index, sampling_loc,
                           attn_weight, grad_out, grad_value, grad_sampling_loc,
                           grad_attn_weight, B, Nv, Nq, M, D, L, K, workspace, workspace_bytes,
                           flags, s, ev);
        if (st == MSDA_OK) st = hip_status(hipEventSynchronize(ev[6]));
        for (int i = 0; i < MSDA_BWD_STAGES && st == MSDA_OK; ++i) {
            float ms = 0.f;
            st = hip_status(hipEventElapsedTime(&ms, ev[i], ev[i + 1]));
            stage_us[i] = 1000.f * ms;
        }
    }
    for (int i = 0; i < made; ++i) (void)hipEventDestroy(ev[i]);
    return st;
}

msda_status msda_validate_host(const int64_t *spatial_shapes_host, const int64_t *level_start_host,
                               int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D, int64_t L,
                               int64_t K) {
    msda_status st = check_sizes(MSDA_F32, B, Nv, Nq, M, D, L, K);
    if (st != MSDA_OK) return st;
    if (!spatial_shapes_host || !level_start_host) return MSDA_ERR_NULL;
    int64_t total = 0;
    for (int64_t l = 0; l < L; ++l) {
        const int64_t H = spatial_shapes_host[2 * l], W = spatial_shapes_host[2 * l + 1];
        if (H < 1 || W < 1) return MSDA_ERR_SHAPE;
        // pixel coordinates are formed in fp32: keep them exact integers
        if (H >= ((int64_t)1 << 24) || W >= ((int64_t)1 << 24)) return MSDA_ERR_UNSUPPORTED;
        if (level_start_host[l] != total) return MSDA_ERR_SHAPE;
        if (H > Nv / W) return MSDA_ERR_SHAPE;
        total += H * W;
        if (total > Nv) return MSDA_ERR_SHAPE;
    }
    if (total != Nv) return MSDA_ERR_SHAPE;
    return MSDA_OK;
}

const char *msda_status_string(int status) {
    switch (status) {
    case MSDA_OK: return "ok";
    case MSDA_ERR_NULL: return "a required pointer is NULL";
    case MSDA_ERR_SHAPE: return "sizes are negative or inconsistent with the level table";
    case MSDA_ERR_DTYPE: return "unknown value dtype";
    case MSDA_ERR_UNSUPPORTED:
        return "outside the supported limits (D in {4,8,...,256}, 1 <= L <= 16, 31-bit slices)";
    case MSDA_ERR_HIP: return "the HIP runtime refused a launch";
    case MSDA_ERR_WORKSPACE:
        return "workspace smaller than msda_backward_workspace_size or not 256-byte aligned";
    default: return "unknown msda status";
    }
}

int msda_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
