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
// Backward (msda_backward):
//   bwd_dots_kernel (on a side stream, concurrently with the rest): per
//      point the four <grad_out row, neighbour row> dot products, reduced
//      across the lane group with DPP, give grad_attn_weight and
//      grad_sampling_loc.
//   grad_value is a scatter (every point adds A * w * grad_out into four
//   pixels).  fp32 atomics run at a few hundred G lane-ops/s on this chip,
//   in LDS as in memory, so it is computed in gather form instead, per 8x8
//   pixel tile and head ("bin"):
//   bin_count_kernel: points per bin (LDS histogram, one global add per bin
//      and workgroup).
//   bin_scan_kernel: exclusive scan of the counts -> bin offsets, and a work
//      list of (bin, chunk of at most kChunk records).
//   bin_scatter_kernel: one 16-byte record per (point, bin) it touches,
//      written into its bin (LDS ranks, one global reservation per bin and
//      workgroup).
//   grad_value_tile_kernel: per work item, the records are counting-sorted
//      by the cell of their top-left neighbour and their grad_out rows are
//      staged in LDS in that order; a lane owns (pixel, channel quad) pairs
//      and sums over the four cells that feed its pixel, in registers.  Only
//      bins split over several chunks add into grad_value atomically.
//
// value and grad_value are addressed through raw buffer descriptors whose
// size is the batch slice.  A neighbour outside the map gets the offset
// kOOB, beyond every slice, so its fetch returns zeros without a branch; the
// same range check keeps an inconsistent level table from touching other
// memory.

#include <mutex>
#include <type_traits>

#include "common.h"

// hipError_t of the last MSDA_ERR_HIP on this thread, for every translation unit
thread_local int msda_internal_last_hip_error = 0;

namespace {

constexpr int kSetupLdsBytes = 36 * 1024;  // per-workgroup budget for the point tables
constexpr int kTileShift = 3;              // grad_value tiles of 8x8 pixels
constexpr int kTile = 1 << kTileShift;
constexpr int kTilePx = kTile * kTile;
constexpr int kChunk = 2048;               // points per grad_value work item, at most
constexpr int kHistLds = 4096;             // bins of one (batch, head) kept in an LDS histogram
constexpr int kScanThreads = 1024;
constexpr int kTileGrid = 16384;           // workgroups of the tile kernel, at most
constexpr int kDotsGrid = 512;             // workgroups of the dots kernel, at most

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    // lanes whose source is outside the row (or rows outside ROWS) receive 0
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts, then
// row broadcasts of the running totals of rows 0 and 0-1).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
    v += dpp_u32<0x111, 0xF>(v);  // row_shr:1
    v += dpp_u32<0x112, 0xF>(v);  // row_shr:2
    v += dpp_u32<0x114, 0xF>(v);  // row_shr:4
    v += dpp_u32<0x118, 0xF>(v);  // row_shr:8
    v += dpp_u32<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_u32<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
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

// Bilinear weights of the four neighbours from the fractional parts; 0 for a
// neighbour outside the map (bit c of `valid` clear).
__device__ __forceinline__ float4 tent_weights(float fx, float fy, uint32_t valid) {
    const float gx = 1.f - fx, gy = 1.f - fy;
    return make_float4((valid & 1u) ? gx * gy : 0.f, (valid & 2u) ? fx * gy : 0.f,
                       (valid & 4u) ? gx * fy : 0.f, (valid & 8u) ? fx * fy : 0.f);
}

// Pixel scale d x / d u along an axis of n pixels: n (x = u*n - 0.5, the
// default convention) or n - 1 (x = u*(n - 1), align_corners).
__device__ __forceinline__ float pixel_scale(int n, bool align) {
    return align ? (float)(n - 1) : (float)n;
}

__device__ __forceinline__ Neighbours neighbours(float u, float v, int4 lvl, uint32_t row_stride,
                                                 uint32_t head_off, bool align) {
    const int H = lvl.x, W = lvl.y, S = lvl.z;
    Neighbours n;
    // one rounding, the same as the CPU check: x = u*W - 0.5, y = v*H - 0.5, or
    // with align_corners x = u*(W-1), y = v*(H-1) (fma with a zero addend)
    const float off = align ? 0.f : -0.5f;
    const float x = __builtin_fmaf(u, pixel_scale(W, align), off);
    const float y = __builtin_fmaf(v, pixel_scale(H, align), off);
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
    n.valid = (vTL ? 1u : 0u) | (vTR ? 2u : 0u) | (vBL ? 4u : 0u) | (vBR ? 8u : 0u);
    n.w = tent_weights(n.fx, n.fy, n.valid);
    return n;
}

// The distinct grad_value tiles (bins) that hold at least one of the point's
// neighbours inside the map: tile (tx0 + (c & 1), ty0 + (c >> 1)) iff bit c
// of `mask` is set.  The neighbours span one or two tiles in each direction
// (sx, sy); x0 = -1 gives tx0 = -1, whose bits are then never set.
struct TileMask {
    int tx0, ty0;
    uint32_t mask;
};

__device__ __forceinline__ TileMask point_tile_mask(const Neighbours &n) {
    const int tx0 = n.xi >> kTileShift, ty0 = n.yi >> kTileShift;
    const uint32_t sx = ((n.xi + 1) >> kTileShift) != tx0 ? 1u : 0u;
    const uint32_t sy = ((n.yi + 1) >> kTileShift) != ty0 ? 1u : 0u;
    const uint32_t v = n.valid;
    const uint32_t tl = v & 1u, tr = (v >> 1) & 1u, bl = (v >> 2) & 1u, br = (v >> 3) & 1u;
    const uint32_t nsx = sx ^ 1u, nsy = sy ^ 1u;
    const uint32_t m0 = tl | (nsx & tr) | (nsy & bl) | (nsx & nsy & br);
    const uint32_t m1 = sx & (tr | (nsy & br));
    const uint32_t m2 = sy & (bl | (nsx & br));
    const uint32_t m3 = sx & sy & br;
    return TileMask{tx0, ty0, m0 | (m1 << 1) | (m2 << 2) | (m3 << 3)};
}

// Division by a divisor fixed at launch: n / d = (umulhi(n, mul) + n) >> shift
// with shift = ceil(log2 d) and mul = floor(2^32 (2^shift - d) / d) + 1
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994).  Exact for every n < 2^31, where the sum cannot
// overflow 32 bits.
struct FastDiv {
    uint32_t mul, shift;
};

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
    return (__umulhi(n, f.mul) + n) >> f.shift;
}

struct Dims {
    int Nv, Nq, M, L, K;
    int PC;      // points per chunk (point-table kernels)
    int PS;      // LDS stride per item (PC rounded to an odd count, for bank spread)
    int b0;      // first batch of this launch
    int nblk;    // workgroups per batch (forward) or per (batch, head) (backward)
    int nb_max;      // bin stride per (batch, head) in the workspace
    int accumulate;  // grad_value already holds a gradient to add to
    FastDiv div_lk;  // by L * K (count and scatter kernels)
    FastDiv div_k;   // by K
    int nblocks;     // query blocks of the launch (dots kernel)
    int align;       // pixel convention: x = u*(W-1) instead of u*W - 0.5
    int loc_div;     // dots kernel: location gradients divided by (W, H) (offset gradients)
    int softmax_run; // dots kernel: softmax backward over runs of this many points (0: none)
};

// Workspace of the backward pipeline (all 32-bit words).
struct Work {
    uint32_t *counts;      // [B][nb_max][M] points per bin
    uint32_t *start;       // [B][nb_max][M] first entry of each bin in `sorted`
    uint32_t *cursor;      // [B][nb_max][M] next free entry while scattering
    uint4 *items;          // [work_max] (bin, first record, records, whole bin)
    uint32_t *work_total;  // [1]
    uint4 *recs;           // [4 * points] records grouped by bin
};

// Raw inputs of the fused prologue, which computes the sampling location and
// the attention weight of each point from them:
//   loc = ref[b, q, l] + off[b, q, m, l, k] / (W_l, H_l)   (fp32: one IEEE
//         division and one addition per coordinate)
//   A   = softmax of the logits over the L*K points of (b, q, m), or over the
//         K points of each level when per_level is set.
struct Prologue {
    const float *ref;     // [B, Nq, L, 2]
    const float *off;     // [B, Nq, M, L, K, 2]
    const float *logits;  // [B, Nq, M, L * K]
    int per_level;
    // the softmax groups are runs of a power-of-two number (<= 64) of
    // consecutive points that the point loop hands to consecutive lanes of one
    // wave: the group max and sum are taken with lane shuffles
    int shfl;
    float *loc_out;   // forward: also store the locations [pts][2] and weights
    float *attn_out;  // [pts] it computed (for the backward), or nullptr
};

// Max / sum over aligned runs of n consecutive lanes (n a power of two <= 64);
// every lane of a run receives the result.  The whole run must be active.
// Within 16 lanes the partners come from DPP (lane ^ 1, lane ^ 2, then the
// mirrored quad and half-row, which pair the partial results the same way),
// beyond that from cross-row shuffles.
__device__ __forceinline__ float run_max(float v, int n) {
    if (n >= 2) v = fmaxf(v, dpp<0xB1>(v));
    if (n >= 4) v = fmaxf(v, dpp<0x4E>(v));
    if (n >= 8) v = fmaxf(v, dpp<0x141>(v));
    if (n >= 16) v = fmaxf(v, dpp<0x140>(v));
    if (n >= 32) v = fmaxf(v, __shfl_xor(v, 16, 64));
    if (n >= 64) v = fmaxf(v, __shfl_xor(v, 32, 64));
    return v;
}

__device__ __forceinline__ float run_sum(float v, int n) {
    if (n >= 2) v += dpp<0xB1>(v);
    if (n >= 4) v += dpp<0x4E>(v);
    if (n >= 8) v += dpp<0x141>(v);
    if (n >= 16) v += dpp<0x140>(v);
    if (n >= 32) v += __shfl_xor(v, 16, 64);
    if (n >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// Softmax weight of the point holding logit z inside its run of n lanes.
__device__ __forceinline__ float run_softmax(float z, int n) {
    const float e = expf(z - run_max(z, n));
    return e / run_sum(e, n);
}

// (max, 1 / sum exp(z - max)) over the n logits at z.
__device__ __forceinline__ float2 softmax_stats(const float *__restrict__ z, int n) {
    float mx = -INFINITY;
    for (int j = 0; j < n; ++j) mx = fmaxf(mx, z[j]);
    float sum = 0.f;
    for (int j = 0; j < n; ++j) sum += expf(z[j] - mx);
    return make_float2(mx, 1.f / sum);
}

// Location of a point from its level's reference point and pixel offset.  A
// level left out of the table (W = H = 0) gives a non-finite location, which
// samples nothing.
__device__ __forceinline__ float2 prologue_location(float2 r, float2 o, int4 lvl) {
    return make_float2(r.x + o.x / (float)lvl.y, r.y + o.y / (float)lvl.x);
}

// Softmax statistics of the groups of nitems consecutive items starting at
// point pt0 into s_st[item * groups + group].
__device__ __forceinline__ void stage_softmax_stats(float2 *s_st, const Prologue &pr, size_t pt0,
                                                    int nitems, int L, int K) {
    const int LK = L * K, ng = pr.per_level ? L : 1, gs = pr.per_level ? K : LK;
    for (int idx = threadIdx.x; idx < nitems * ng; idx += blockDim.x) {
        const int i1 = idx / ng, g = idx - i1 * ng;
        s_st[idx] = softmax_stats(pr.logits + pt0 + (size_t)i1 * LK + (size_t)g * gs, gs);
    }
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
// With FUSED the locations and weights come from the prologue inputs `pr`
// (loc and attn are unused): per item the softmax statistics of its logits
// are staged in LDS first, then each point's location and weight are formed
// where the plain kernel loads them.
template <int D, typename VT, bool FUSED>
__global__ void __launch_bounds__(kThreads)
msda_fwd_kernel(const VT *__restrict__ value, const int64_t *__restrict__ shapes,
                const int64_t *__restrict__ starts, const float *__restrict__ loc,
                const float *__restrict__ attn, Prologue pr, float *__restrict__ out, Dims dm) {
    constexpr int G = D / 4;
    constexpr int IPB = kThreads / G;
    __shared__ LevelLds s_lv;
    extern __shared__ __align__(16) unsigned char smem[];
    uint4 *s_off = reinterpret_cast<uint4 *>(smem);
    float4 *s_w = reinterpret_cast<float4 *>(s_off + IPB * dm.PS);
    float2 *s_st = reinterpret_cast<float2 *>(s_w + IPB * dm.PS);  // FUSED: softmax stats

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
    const int ng = pr.per_level ? dm.L : 1;
    if constexpr (FUSED) {
        if (!pr.shfl) {
            stage_softmax_stats(s_st, pr, pt0, nitems, dm.L, K);
            __syncthreads();
        }
    }

    const int it = threadIdx.x / G, c = threadIdx.x % G;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);

    for (int j0 = 0; j0 < LK; j0 += dm.PC) {
        const int pc = min(dm.PC, LK - j0);
        if (j0) __syncthreads();  // previous chunk consumed
        for (int idx = threadIdx.x; idx < nitems * pc; idx += kThreads) {
            const int i1 = idx / pc, jj = idx - i1 * pc, j = j0 + jj;
            const size_t p = pt0 + (size_t)i1 * LK + j;
            const int l = j / K;
            float2 uv;
            float A;
            if constexpr (FUSED) {
                const int q = (item0 + i1) / M;
                const float2 r =
                    reinterpret_cast<const float2 *>(pr.ref)[((size_t)b * dm.Nq + q) * dm.L + l];
                uv = prologue_location(r, reinterpret_cast<const float2 *>(pr.off)[p],
                                       s_lv.lvl[l]);
                const float z = pr.logits[p];
                if (pr.shfl) {  // one chunk holds whole items: runs never straddle waves
                    A = run_softmax(z, pr.per_level ? K : LK);
                } else {
                    const float2 st = s_st[i1 * ng + (pr.per_level ? l : 0)];
                    A = expf(z - st.x) * st.y;
                }
                if (pr.loc_out) {
                    reinterpret_cast<float2 *>(pr.loc_out)[p] = uv;
                    pr.attn_out[p] = A;
                }
            } else {
                uv = reinterpret_cast<const float2 *>(loc)[p];
                A = attn[p];
            }
            const int m = (item0 + i1) % M;
            Neighbours n = neighbours(uv.x, uv.y, s_lv.lvl[l], row_stride,
                                      (uint32_t)m * D * 4u, dm.align);
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
// backward: grad_attn_weight and grad_sampling_loc
// Workgroup = (batch b, head m, IPB consecutive queries).  Per point the
// table holds the four row offsets (later overwritten by the four dot
// products <grad_out row, value row>) and (fx, fy, A, valid bits).
// ---------------------------------------------------------------------------
template <int D, typename VT>
__global__ void __launch_bounds__(kThreads)
bwd_dots_kernel(const VT *__restrict__ value, const int64_t *__restrict__ shapes,
                const int64_t *__restrict__ starts, const float *__restrict__ loc,
                const float *__restrict__ attn, const float *__restrict__ grad_out,
                float *__restrict__ grad_loc, float *__restrict__ grad_attn,
                float *__restrict__ ref_part, Dims dm) {
    constexpr int G = D / 4;
    constexpr int IPB = kThreads / G;
    __shared__ LevelLds s_lv;
    extern __shared__ __align__(16) unsigned char smem[];
    uint4 *s_off = reinterpret_cast<uint4 *>(smem);  // row offsets, then the dots
    float4 *s_aux = reinterpret_cast<float4 *>(s_off + IPB * dm.PS);

    const int M = dm.M, K = dm.K, LK = dm.L * dm.K, Nq = dm.Nq;
    // per level, d pixel / d (location or offset): (W, H) or (W-1, H-1), over
    // (W, H) for offsets
    __shared__ float2 s_scale[kMaxLevels];
    stage_levels(&s_lv, shapes, starts, dm.L, dm.Nv, 0x7fffffff);
    if (threadIdx.x < dm.L) {
        const int4 lvl = s_lv.lvl[threadIdx.x];
        float sx = pixel_scale(lvl.y, dm.align), sy = pixel_scale(lvl.x, dm.align);
        if (dm.loc_div && lvl.y > 0) {  // d loc / d offset = 1 / (W, H)
            sx /= (float)lvl.y;
            sy /= (float)lvl.x;
        }
        s_scale[threadIdx.x] = make_float2(sx, sy);
    }
    __syncthreads();
    // blocks of IPB queries of one (batch, head), dm.nblk per (batch, head);
    // workgroup g takes blocks g, g + grid, ...
    const int total = dm.nblocks;
    for (int blk = blockIdx.x; blk < total; blk += gridDim.x) {
    if (blk != (int)blockIdx.x) __syncthreads();  // the point tables are reused
    const int wg = xcd_contiguous(blk, total);
    const int bm = wg / dm.nblk + dm.b0 * M;
    const int m = bm % M, b = bm / M;
    const int q0 = (wg % dm.nblk) * IPB;
    const int nitems = min(IPB, Nq - q0);
    const uint32_t row_stride = (uint32_t)M * D * 4u;
    const uint32_t head_off = (uint32_t)m * D * 4u;

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
        if (j0) __syncthreads();  // previous chunk consumed
        for (int idx = threadIdx.x; idx < nitems * pc; idx += kThreads) {
            const int i1 = idx / pc, jj = idx - i1 * pc, j = j0 + jj;
            const size_t p = pt0 + (size_t)i1 * M * LK + j;
            const float2 uv = reinterpret_cast<const float2 *>(loc)[p];
            const float A = attn[p];
            const Neighbours n =
                neighbours(uv.x, uv.y, s_lv.lvl[j / K], row_stride, head_off, dm.align);
            s_off[i1 * dm.PS + jj] = n.off;
            s_aux[i1 * dm.PS + jj] = make_float4(n.fx, n.fy, A, __uint_as_float(n.valid));
        }
        __syncthreads();
        if (it < nitems) {
            const int base = it * dm.PS;
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
                // the group's lanes are one wave: every lane has read the
                // offsets before lane 0 overwrites them
                if (c == 0)
                    s_off[base + jj] = make_uint4(__float_as_uint(d0), __float_as_uint(d1),
                                                  __float_as_uint(d2), __float_as_uint(d3));
            }
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < nitems * pc; idx += kThreads) {
            const int i1 = idx / pc, jj = idx - i1 * pc, j = j0 + jj;
            const size_t p = pt0 + (size_t)i1 * M * LK + j;
            const uint4 du = s_off[i1 * dm.PS + jj];
            const float4 ax = s_aux[i1 * dm.PS + jj];
            const int4 lvl = s_lv.lvl[j / K];
            float ga = 0.f, gx = 0.f, gy = 0.f;
            const uint32_t valid = __float_as_uint(ax.w);
            if (valid != 0u) {
                const float d0 = __uint_as_float(du.x), d1 = __uint_as_float(du.y);
                const float d2 = __uint_as_float(du.z), d3 = __uint_as_float(du.w);
                const float fx = ax.x, fy = ax.y, A = ax.z;
                const float4 w = tent_weights(fx, fy, valid);
                ga = w.x * d0 + w.y * d1 + w.z * d2 + w.w * d3;
                const float2 sc = s_scale[j / K];
                gx = A * sc.x * ((1.f - fy) * (d1 - d0) + fy * (d3 - d2));
                gy = A * sc.y * ((1.f - fx) * (d2 - d0) + fx * (d3 - d1));
            }
            // Fused prologue, when the chunk holds whole items (runs of
            // consecutive lanes are the items' softmax groups and levels):
            // the logit gradient A * (grad_A - sum over the group of A * grad_A)
            // replaces grad_A, and each level's sum of location gradients is
            // stored per item for the reference-point gradient.
            if (dm.softmax_run) {
                const float A = ax.z;
                ga = A * (ga - run_sum(A * ga, dm.softmax_run));
            }
            grad_attn[p] = ga;
            reinterpret_cast<float2 *>(grad_loc)[p] = make_float2(gx, gy);
            if (ref_part) {
                const float rx = run_sum(gx, K), ry = run_sum(gy, K);
                if (j % K == 0)  // offset gradients times (W, H): location gradients
                    reinterpret_cast<float2 *>(ref_part)[(row0 + (size_t)i1 * M) * dm.L + j / K] =
                        make_float2(rx * (float)lvl.y, ry * (float)lvl.x);
            }
        }
    }
    }
}

// ---------------------------------------------------------------------------
// backward: points per bin
// Workgroup = (batch b, head m, kBinPoints consecutive points of the
// (b, m) list in (query, level, point) order), kBinPPT points per thread,
// all of whose coordinates are loaded before any is used.
// ---------------------------------------------------------------------------
constexpr int kBinPPT = 16;
constexpr int kBinPoints = kBinPPT * kThreads;

__global__ void __launch_bounds__(kThreads)
bin_count_kernel(const int64_t *__restrict__ shapes, const int64_t *__restrict__ starts,
                 const float *__restrict__ loc, uint32_t *__restrict__ counts, int hist_cap,
                 Dims dm) {
    __shared__ LevelLds s_lv;
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *s_cnt = reinterpret_cast<uint32_t *>(smem);  // [hist_cap]

    const int M = dm.M, LK = dm.L * dm.K, Nq = dm.Nq;
    const int wg = xcd_contiguous(blockIdx.x, gridDim.x);
    const int bm = wg / dm.nblk + dm.b0 * M;
    const int m = bm % M, b = bm / M;
    const int f0 = (wg % dm.nblk) * kBinPoints;
    const int nf = Nq * LK;
    const size_t row0 = (size_t)b * Nq * M + m;  // item row of query 0

    float2 uv[kBinPPT];
#pragma unroll
    for (int r = 0; r < kBinPPT; ++r) {
        const int f = f0 + threadIdx.x + r * kThreads;
        uv[r] = make_float2(0.f, 0.f);
        if (f < nf) {
            const int q = (int)fdiv((uint32_t)f, dm.div_lk), j = f - q * LK;
            uv[r] = reinterpret_cast<const float2 *>(loc)[(row0 + (size_t)q * M) * LK + j];
        }
    }
    stage_levels(&s_lv, shapes, starts, dm.L, dm.Nv, dm.nb_max);
    const int nbins = s_lv.nbins;
    const bool lds = nbins <= hist_cap;
    uint32_t *gcount = counts + (size_t)b * dm.nb_max * M + m;  // tile i at gcount[i * M]
    if (lds) {
        for (int i = threadIdx.x; i < nbins; i += kThreads) s_cnt[i] = 0u;
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < kBinPPT; ++r) {
        const int f = f0 + threadIdx.x + r * kThreads;
        if (f < nf) {
            const int q = (int)fdiv((uint32_t)f, dm.div_lk), j = f - q * LK;
            const int l = (int)fdiv((uint32_t)j, dm.div_k);
            const Neighbours n = neighbours(uv[r].x, uv[r].y, s_lv.lvl[l], 0u, 0u, dm.align);
            const TileMask tm = point_tile_mask(n);
            const int tw = s_lv.tw[l];
            const int b00 = s_lv.lvl[l].w + tm.ty0 * tw + tm.tx0;
            if (lds) {
                if (tm.mask & 1u) atomicAdd(&s_cnt[b00], 1u);
                if (tm.mask & 2u) atomicAdd(&s_cnt[b00 + 1], 1u);
                if (tm.mask & 4u) atomicAdd(&s_cnt[b00 + tw], 1u);
                if (tm.mask & 8u) atomicAdd(&s_cnt[b00 + tw + 1], 1u);
            } else {
                if (tm.mask & 1u) atomicAdd(&gcount[(size_t)b00 * M], 1u);
                if (tm.mask & 2u) atomicAdd(&gcount[(size_t)(b00 + 1) * M], 1u);
                if (tm.mask & 4u) atomicAdd(&gcount[(size_t)(b00 + tw) * M], 1u);
                if (tm.mask & 8u) atomicAdd(&gcount[(size_t)(b00 + tw + 1) * M], 1u);
            }
        }
    }
    if (lds) {
        __syncthreads();
        for (int i = threadIdx.x; i < nbins; i += kThreads) {
            const uint32_t v = s_cnt[i];
            if (v) atomicAdd(&gcount[(size_t)i * M], v);
        }
    }
}

// ---------------------------------------------------------------------------
// backward: scan of the bin counts, work list
// One workgroup of kScanThreads.  Bins are visited in (batch, tile, head)
// order, which is also their order in memory: the bins of batch b are the
// nbins * M words from b * nb_max * M on; all batches form one flat scan.
// Each bin of n > 0 points becomes ceil(n / kChunk) work items (bin, first
// record, records, whole bin).
// ---------------------------------------------------------------------------
// Exclusive scan of (a, b) pairs over the kScanThreads threads of the block:
// wave-level scans with lane shuffles, then one scan of the wave totals.
// The block totals are returned in tot_a, tot_b.
__device__ __forceinline__ void block_exclusive_scan2(uint32_t &a, uint32_t &b, uint2 *s_wave,
                                                      uint32_t &tot_a, uint32_t &tot_b) {
    constexpr int kWaves = kScanThreads / 64;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const uint32_t ia = wave_inclusive_scan(a), ib = wave_inclusive_scan(b);
    if (lane == 63) s_wave[wave] = make_uint2(ia, ib);
    __syncthreads();
    if (wave == 0) {
        const uint2 v = lane < kWaves ? s_wave[lane] : make_uint2(0u, 0u);
        const uint32_t sa = wave_inclusive_scan(v.x), sb = wave_inclusive_scan(v.y);
        if (lane < kWaves) s_wave[lane] = make_uint2(sa - v.x, sb - v.y);  // exclusive
        if (lane == kWaves - 1) s_wave[kWaves] = make_uint2(sa, sb);
    }
    __syncthreads();
    const uint2 base = s_wave[wave];
    tot_a = s_wave[kWaves].x;
    tot_b = s_wave[kWaves].y;
    a = base.x + ia - a;
    b = base.y + ib - b;
    __syncthreads();  // s_wave is reused by the next call
}

__global__ void __launch_bounds__(kScanThreads)
bin_scan_kernel(const int64_t *__restrict__ shapes, const int64_t *__restrict__ starts,
                const uint32_t *__restrict__ counts, uint32_t *__restrict__ start,
                uint32_t *__restrict__ cursor, uint4 *__restrict__ items,
                uint32_t *__restrict__ work_total, int B, Dims dm) {
    constexpr int kPer = 8;
    __shared__ LevelLds s_lv;
    __shared__ uint2 s_wave[kScanThreads / 64 + 1];
    stage_levels(&s_lv, shapes, starts, dm.L, dm.Nv, dm.nb_max);
    // the used bins of every batch as one flat sequence f = b * per_b + (tile * M + m),
    // scanned in one pass (the bins of batch b start at b * nb_max * M in memory)
    const uint32_t per_b = (uint32_t)s_lv.nbins * (uint32_t)dm.M;
    const uint32_t stride_b = (uint32_t)dm.nb_max * (uint32_t)dm.M;
    const uint32_t nf = per_b * (uint32_t)B;
    uint32_t carry_e = 0, carry_c = 0;
    for (uint32_t base = 0; base < nf; base += kScanThreads * kPer) {
        const uint32_t g0 = base + threadIdx.x * kPer;
        uint32_t cnt[kPer], bin[kPer], e = 0, ch = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const uint32_t f = g0 + i;
            const uint32_t b = per_b ? f / per_b : 0u;
            bin[i] = b * stride_b + (f - b * per_b);
            cnt[i] = f < nf ? counts[bin[i]] : 0u;
            e += cnt[i];
            ch += (cnt[i] + kChunk - 1) / kChunk;
        }
        uint32_t tot_e, tot_c;
        block_exclusive_scan2(e, ch, s_wave, tot_e, tot_c);
        e += carry_e;
        ch += carry_c;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            if (g0 + i < nf) {
                start[bin[i]] = e;
                cursor[bin[i]] = e;
                const uint32_t nch = (cnt[i] + kChunk - 1) / kChunk;
                for (uint32_t k = 0; k < nch; ++k)
                    items[ch + k] = make_uint4(bin[i], e + k * kChunk,
                                               min((uint32_t)kChunk, cnt[i] - k * kChunk),
                                               nch == 1 ? 1u : 0u);
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
// backward: one record per (point, bin), scattered into the bins
// Same workgroups as bin_count_kernel.  A record holds what the tile kernel
// needs of the point: (q << 7 | cell, A * (1 - fx), A * fx, fy), where cell =
// (x0 - tile x + 1) + 9 * (y0 - tile y + 1) places the point's top-left
// neighbour in the 9x9 grid made of the tile and the column and row before it.
// ---------------------------------------------------------------------------
constexpr int kCellsW = kTile + 1;
constexpr int kCells = kCellsW * kCellsW;
constexpr int kRecQueryShift = 7;  // cells < 128

__global__ void __launch_bounds__(kThreads)
bin_scatter_kernel(const int64_t *__restrict__ shapes, const int64_t *__restrict__ starts,
                   const float *__restrict__ loc, const float *__restrict__ attn,
                   uint32_t *__restrict__ cursor, uint4 *__restrict__ recs, int hist_cap,
                   Dims dm) {
    __shared__ LevelLds s_lv;
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *s_cnt = reinterpret_cast<uint32_t *>(smem);  // [hist_cap] counts, then ranks
    uint32_t *s_base = s_cnt + hist_cap;                    // [hist_cap] reserved offsets

    const int M = dm.M, LK = dm.L * dm.K, Nq = dm.Nq;
    const int wg = xcd_contiguous(blockIdx.x, gridDim.x);
    const int bm = wg / dm.nblk + dm.b0 * M;
    const int m = bm % M, b = bm / M;
    const int f0 = (wg % dm.nblk) * kBinPoints;
    const int nf = Nq * LK;
    const size_t row0 = (size_t)b * Nq * M + m;  // item row of query 0

    // the thread's points: coordinates and weights, kept for both passes
    float2 uv[kBinPPT];
    float aw[kBinPPT];
#pragma unroll
    for (int r = 0; r < kBinPPT; ++r) {
        const int f = f0 + threadIdx.x + r * kThreads;
        uv[r] = make_float2(0.f, 0.f);
        aw[r] = 0.f;
        if (f < nf) {
            const int q = (int)fdiv((uint32_t)f, dm.div_lk), j = f - q * LK;
            const size_t p = (row0 + (size_t)q * M) * LK + j;
            uv[r] = reinterpret_cast<const float2 *>(loc)[p];
            aw[r] = attn[p];
        }
    }
    stage_levels(&s_lv, shapes, starts, dm.L, dm.Nv, dm.nb_max);
    const int nbins = s_lv.nbins;
    const bool lds = nbins <= hist_cap;
    uint32_t *gcur = cursor + (size_t)b * dm.nb_max * M + m;  // tile i at gcur[i * M]
    if (lds) {
        for (int i = threadIdx.x; i < nbins; i += kThreads) s_cnt[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kBinPPT; ++r) {
            const int f = f0 + threadIdx.x + r * kThreads;
            if (f < nf) {
                const int q = (int)fdiv((uint32_t)f, dm.div_lk), j = f - q * LK;
                const int l = (int)fdiv((uint32_t)j, dm.div_k);
                const Neighbours n = neighbours(uv[r].x, uv[r].y, s_lv.lvl[l], 0u, 0u, dm.align);
                const TileMask tm = point_tile_mask(n);
                const int tw = s_lv.tw[l];
                const int b00 = s_lv.lvl[l].w + tm.ty0 * tw + tm.tx0;
                if (tm.mask & 1u) atomicAdd(&s_cnt[b00], 1u);
                if (tm.mask & 2u) atomicAdd(&s_cnt[b00 + 1], 1u);
                if (tm.mask & 4u) atomicAdd(&s_cnt[b00 + tw], 1u);
                if (tm.mask & 8u) atomicAdd(&s_cnt[b00 + tw + 1], 1u);
            }
        }
        __syncthreads();
        for (int i = threadIdx.x; i < nbins; i += kThreads) {
            const uint32_t v = s_cnt[i];
            s_base[i] = v ? atomicAdd(&gcur[(size_t)i * M], v) : 0u;
            s_cnt[i] = 0u;
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < kBinPPT; ++r) {
        const int f = f0 + threadIdx.x + r * kThreads;
        if (f < nf) {
            const int q = (int)fdiv((uint32_t)f, dm.div_lk), j = f - q * LK;
            const int l = (int)fdiv((uint32_t)j, dm.div_k);
            const Neighbours n = neighbours(uv[r].x, uv[r].y, s_lv.lvl[l], 0u, 0u, dm.align);
            const TileMask tm = point_tile_mask(n);
            const int tw = s_lv.tw[l];
            const int b00 = s_lv.lvl[l].w + tm.ty0 * tw + tm.tx0;
            const uint32_t a0 = __float_as_uint(aw[r] * (1.f - n.fx));
            const uint32_t a1 = __float_as_uint(aw[r] * n.fx);
            const uint32_t fy = __float_as_uint(n.fy);
            // cell of the top-left neighbour relative to tile (tx0, ty0); one
            // tile to the right is 8 cells left, one tile down is 72 cells up
            const uint32_t key = ((uint32_t)q << kRecQueryShift);
            const int c00 = (n.xi - tm.tx0 * kTile + 1) + kCellsW * (n.yi - tm.ty0 * kTile + 1);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (tm.mask & (1u << c)) {
                    const int bin = b00 + (c & 1) + (c >> 1) * tw;
                    const uint32_t slot = lds ? s_base[bin] + atomicAdd(&s_cnt[bin], 1u)
                                              : atomicAdd(&gcur[(size_t)bin * M], 1u);
                    const int cell = c00 - (c & 1) * kTile - (c >> 1) * kTile * kCellsW;
                    recs[slot] = make_uint4(key | (uint32_t)cell, a0, a1, fy);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// backward: grad_value, one 8x8 tile (and chunk of its records) per work item
//
// A workgroup walks its work items in sub-chunks of kSub records as a
// two-stage pipeline over two LDS buffers: while it sums sub-chunk k out of
// one buffer, it counting-sorts sub-chunk k+1 by cell, loads that
// sub-chunk's grad_out rows straight into the other buffer in sorted order
// (global_load_lds, no registers held), and loads the records of sub-chunk
// k+2 into registers.
//
// Pixel (x, y) of the tile receives from the points of four cells, in four
// roles: top-right from cell (x, y+1), top-left from (x+1, y+1), bottom-right
// from (x, y), bottom-left from (x+1, y).  After the sort, cells (x, y+1) and
// (x+1, y+1) are one contiguous range of the buffer, and so are (x, y) and
// (x+1, y).  A lane owns (pixel, 4-channel quad) pairs and sums
// A * w * grad_out over those two ranges in registers across all sub-chunks
// of the item, so no two lanes ever add into the same value.  Each pixel is
// written once per work item.
// ---------------------------------------------------------------------------
constexpr int kTileThreads = 512;
constexpr int kStageBytes = 16 * 1024;  // grad_out rows per LDS buffer

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void global_void_t;

// A sub-chunk: records [it.y + off, it.y + off + kSub) of work item w.
struct SubChunk {
    uint32_t w, off;
    uint4 it;  // the work item: (bin, first record, records, whole bin)
    bool valid;
};

// acc += w[4e + role] * g[e * kQuads] over e in [e0, e2), role r0 below e1 and
// r1 from e1 on; four entries per round, all eight LDS reads issued first.
template <int kQuads>
__device__ __forceinline__ void pull_range(float4 &acc, const float *__restrict__ w,
                                           const float4 *__restrict__ g, int e0, int e1, int e2,
                                           int r0, int r1) {
    int e = e0;
    for (; e + 4 <= e2; e += 4) {
        const float w0 = w[4 * e + (e < e1 ? r0 : r1)];
        const float w1 = w[4 * e + 4 + (e + 1 < e1 ? r0 : r1)];
        const float w2 = w[4 * e + 8 + (e + 2 < e1 ? r0 : r1)];
        const float w3 = w[4 * e + 12 + (e + 3 < e1 ? r0 : r1)];
        const float4 g0 = g[e * kQuads];
        const float4 g1 = g[(e + 1) * kQuads];
        const float4 g2 = g[(e + 2) * kQuads];
        const float4 g3 = g[(e + 3) * kQuads];
        fma4(acc, w0, g0);
        fma4(acc, w1, g1);
        fma4(acc, w2, g2);
        fma4(acc, w3, g3);
    }
    for (; e < e2; ++e) fma4(acc, w[4 * e + (e < e1 ? r0 : r1)], g[e * kQuads]);
}

template <int D>
__global__ void __launch_bounds__(kTileThreads)
grad_value_tile_kernel(const int64_t *__restrict__ shapes, const int64_t *__restrict__ starts,
                       const float *__restrict__ grad_out, const uint4 *__restrict__ items,
                       const uint32_t *__restrict__ work_total, const uint4 *__restrict__ recs,
                       float *__restrict__ grad_value, Dims dm) {
    constexpr int kQuads = D / 4;
    constexpr int kSub = kStageBytes / (D * 4) < kTileThreads ? kStageBytes / (D * 4)
                                                              : kTileThreads;
    constexpr int kOwn = (kTilePx * kQuads + kTileThreads - 1) / kTileThreads;  // pairs per lane
    __shared__ LevelLds s_lv;
    __shared__ float4 s_g0[kSub * kQuads];  // grad_out rows in sorted order, buffer 0
    __shared__ float4 s_g1[kSub * kQuads];  // buffer 1
    __shared__ float4 s_w0[kSub];           // A * bilinear weights (TL, TR, BL, BR), sorted
    __shared__ float4 s_w1[kSub];
    __shared__ uint32_t s_st0[kCells + 1];  // first sorted slot of each cell, and the total
    __shared__ uint32_t s_st1[kCells + 1];
    __shared__ uint32_t s_tmp[kCells];      // cell counts, then placement cursors
    __shared__ uint32_t s_q[kSub];          // query of the record in each sorted slot

    const int M = dm.M, Nq = dm.Nq;
    const int tid = threadIdx.x;
    const uint32_t total = *work_total;
    const uint32_t grid = gridDim.x;
    if (blockIdx.x >= total) return;  // the grid is sized for the largest possible list
    stage_levels(&s_lv, shapes, starts, dm.L, dm.Nv, dm.nb_max);
    if (tid < kCells) s_tmp[tid] = 0u;

    // Sub-chunk k (summed), k+1 (sorted, rows loading), k+2 (records loading),
    // and the work item after the one of k+2.  Workgroup g takes items g,
    // g + grid, ... counted from the end of the list: the grid is normally
    // larger than the list, so each workgroup has one item and the hardware
    // dispatcher balances the load, starting with the last items (the bins of
    // the coarse levels, the largest).  The list is in (batch, level, tile,
    // head) order, so with 8 heads workgroup g (dispatched to XCD g % 8) and
    // its XCD mostly see one head, whose grad_out rows then stay in that L2.
    auto item_at = [&](uint32_t w) { return items[total - 1u - w]; };
    SubChunk A{0, 0, make_uint4(0, 0, 0, 0), false};
    SubChunk Bn{0, 0, make_uint4(0, 0, 0, 0), false};
    SubChunk C{blockIdx.x, 0, item_at(blockIdx.x), true};
    uint4 next_item = make_uint4(0, 0, 0, 0);
    if (C.w + grid < total) next_item = item_at(C.w + grid);
    auto advance = [&](SubChunk &c) {
        if (!c.valid) return;
        if (c.off + kSub < c.it.z) {
            c.off += kSub;
            return;
        }
        c.w += grid;
        c.off = 0;
        c.valid = c.w < total;
        c.it = next_item;
        if (c.valid && c.w + grid < total) next_item = item_at(c.w + grid);
    };
    auto count_of = [&](const SubChunk &c) {
        return c.valid ? (int)min((uint32_t)kSub, c.it.z - c.off) : 0;
    };

    uint4 rec = make_uint4(0, 0, 0, 0);  // record `tid` of sub-chunk k+1
    float4 acc[kOwn];
#pragma unroll
    for (int o = 0; o < kOwn; ++o) acc[o] = make_float4(0.f, 0.f, 0.f, 0.f);

    // sum sub-chunk A out of buffer P while preparing Bn in buffer P ^ 1
    auto step = [&](auto pc) {
        constexpr int P = decltype(pc)::value;
        float4 *gP = P ? s_g1 : s_g0;
        float4 *gF = P ? s_g0 : s_g1;
        const float *wP = reinterpret_cast<const float *>(P ? s_w1 : s_w0);
        float4 *wF = P ? s_w0 : s_w1;
        const uint32_t *stP = P ? s_st1 : s_st0;
        uint32_t *stF = P ? s_st0 : s_st1;

        // 1. count the cells of Bn
        const int nb = count_of(Bn);
        const int cell = (int)(rec.x & ((1u << kRecQueryShift) - 1u));
        if (tid < nb) atomicAdd(&s_tmp[cell], 1u);
        __syncthreads();
        // 2. exclusive scan of the 81 counts by one wave, 2 cells a lane
        if (tid < 64) {
            const int c0 = 2 * tid, c1 = 2 * tid + 1;
            const uint32_t v0 = c0 < kCells ? s_tmp[c0] : 0u;
            const uint32_t v1 = c1 < kCells ? s_tmp[c1] : 0u;
            const uint32_t incl = wave_inclusive_scan(v0 + v1);
            const uint32_t ex = incl - v0 - v1;
            if (c0 < kCells) {
                stF[c0] = ex;
                s_tmp[c0] = ex;
            }
            if (c1 < kCells) {
                stF[c1] = ex + v0;
                s_tmp[c1] = ex + v0;
            }
            if (tid == 63) stF[kCells] = incl;
        }
        __syncthreads();
        // 3. place the records of Bn in cell order
        if (tid < nb) {
            // the scan makes every slot < nb <= kSub; the clamp keeps LDS safe regardless
            const uint32_t slot = min(atomicAdd(&s_tmp[cell], 1u), (uint32_t)kSub - 1u);
            const float a0 = __uint_as_float(rec.y), a1 = __uint_as_float(rec.z);
            const float fy = __uint_as_float(rec.w), gy = 1.f - fy;
            wF[slot] = make_float4(a0 * gy, a1 * gy, a0 * fy, a1 * fy);
            s_q[slot] = rec.x >> kRecQueryShift;
        }
        __syncthreads();
        // 4. start the loads of Bn's rows (into gF) and of C's records
        if (tid < kCells) s_tmp[tid] = 0u;
        if (nb) {
            const uint32_t bm = Bn.it.x;  // (b * nb_max + tile) * M + m
            const int m = (int)(bm % (uint32_t)M);
            const int b = (int)(bm / (uint32_t)M / (uint32_t)dm.nb_max);
            const float *gob = grad_out + ((size_t)b * Nq * M + m) * D;
            for (int i = tid; i < nb * kQuads; i += kTileThreads) {
                const int slot = i / kQuads, qd = i - slot * kQuads;
                const uint32_t qy = min(s_q[slot], (uint32_t)Nq - 1u);  // a query of this batch
                const float *src = gob + (size_t)qy * M * D + 4 * qd;
                // each wave fills 64 consecutive float4 slots: lane l writes slot base + l
                __builtin_amdgcn_global_load_lds((global_void_t *)src,
                                                 (lds_void_t *)(gF + (i & ~63)), 16, 0, 0);
            }
        }
        const int ncn = count_of(C);
        if (tid < ncn) rec = recs[C.it.y + C.off + tid];
        // 5. sum A out of buffer P
        if (A.valid) {
#pragma unroll
            for (int o = 0; o < kOwn; ++o) {
                const int pair = tid + o * kTileThreads;
                if (pair >= kTilePx * kQuads) break;
                const int px = pair / kQuads, q = pair - px * kQuads;
                const int x = px & (kTile - 1), y = px >> kTileShift;
                const int cT = (y + 1) * kCellsW + x, cB = y * kCellsW + x;
                // cells (x, y+1) then (x+1, y+1): top-right, then top-left roles;
                // cells (x, y) then (x+1, y): bottom-right, then bottom-left roles
                pull_range<kQuads>(acc[o], wP, gP + q, (int)stP[cT], (int)stP[cT + 1], (int)stP[cT + 2],
                           1, 0);
                pull_range<kQuads>(acc[o], wP, gP + q, (int)stP[cB], (int)stP[cB + 1], (int)stP[cB + 2],
                           3, 2);
            }
            // 6. the item ends with A: write its tile
            if (A.off + kSub >= A.it.z) {
                const uint32_t bin = A.it.x;
                const int m = (int)(bin % (uint32_t)M);
                const uint32_t bt = bin / (uint32_t)M;
                const int b = (int)(bt / (uint32_t)dm.nb_max);
                const int lb = (int)(bt - (uint32_t)b * dm.nb_max);
                int l = 0;
                while (l + 1 < dm.L && s_lv.lvl[l + 1].w <= lb) ++l;
                const int4 lvl = s_lv.lvl[l];
                const int tw = s_lv.tw[l];
                const int ty = (lb - lvl.w) / tw, tx = (lb - lvl.w) - ty * tw;
                const size_t slice = (size_t)dm.Nv * M * D;
                float *gv = grad_value + (size_t)b * slice + (size_t)m * D;
#pragma unroll
                for (int o = 0; o < kOwn; ++o) {
                    const int pair = tid + o * kTileThreads;
                    if (pair >= kTilePx * kQuads) break;
                    const int px = pair / kQuads, q = pair - px * kQuads;
                    const int gx = tx * kTile + (px & (kTile - 1));
                    const int gy = ty * kTile + (px >> kTileShift);
                    float4 a = acc[o];
                    acc[o] = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (gy >= lvl.x || gx >= lvl.y) continue;
                    float *dst = gv + (size_t)(lvl.z + gy * lvl.y + gx) * M * D + 4 * q;
                    if (A.it.w) {
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
        // 7. rows of Bn and records of C have landed; buffer P is free
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
        A = Bn;
        Bn = C;
        advance(C);
    };

    // prologue: records of the first sub-chunk
    {
        const int n0 = count_of(C);
        if (tid < n0) rec = recs[C.it.y + C.off + tid];
        Bn = C;
        advance(C);
        __syncthreads();  // s_tmp cleared
    }
    while (A.valid || Bn.valid) {
        step(std::integral_constant<int, 0>());
        if (!(A.valid || Bn.valid)) break;
        step(std::integral_constant<int, 1>());
    }
}


// ---------------------------------------------------------------------------
// fused prologue, backward side
// fused_prologue_kernel: the locations and weights of every point, written
//    to the workspace for the backward pipeline (the same arithmetic as the
//    fused forward).  Workgroup = kProItems consecutive items (b, q, m).
// fused_epilogue_kernel: grad_logits = A * (grad_A - sum over the softmax
//    group of A * grad_A), in place over grad_A; and, when asked for,
//    grad_ref[b, q, l] = sum over heads and points of the location gradient
//    (the offset gradient times (W_l, H_l)).
// ---------------------------------------------------------------------------
constexpr int kProItems = 64;

__global__ void __launch_bounds__(kThreads)
fused_prologue_kernel(const int64_t *__restrict__ shapes, const int64_t *__restrict__ starts,
                      Prologue pr, float *__restrict__ loc, float *__restrict__ attn,
                      int64_t items, Dims dm) {
    __shared__ LevelLds s_lv;
    extern __shared__ __align__(16) unsigned char smem[];
    float2 *s_st = reinterpret_cast<float2 *>(smem);  // [kProItems * groups]
    stage_levels(&s_lv, shapes, starts, dm.L, dm.Nv, 0x7fffffff);
    const int M = dm.M, K = dm.K, L = dm.L, LK = L * K;
    const int ng = pr.per_level ? L : 1;
    const int64_t blocks = (items + kProItems - 1) / kProItems;
    for (int64_t blk = blockIdx.x; blk < blocks; blk += gridDim.x) {
        const int64_t item0 = blk * kProItems;
        const int nitems = (int)min((int64_t)kProItems, items - item0);
        const size_t pt0 = (size_t)item0 * LK;
        if (!pr.shfl) {
            if (blk != (int64_t)blockIdx.x) __syncthreads();  // s_st is reused
            stage_softmax_stats(s_st, pr, pt0, nitems, L, K);
            __syncthreads();
        }
        // idx runs over whole items, 256 at a time: with shfl every softmax run
        // lies inside one wave and is active or inactive as a whole
        for (int idx = threadIdx.x; idx < nitems * LK; idx += kThreads) {
            const int i1 = idx / LK, j = idx - i1 * LK, l = j / K;
            const size_t p = pt0 + idx;
            const size_t bq = (size_t)(item0 + i1) / M;
            const float2 r = reinterpret_cast<const float2 *>(pr.ref)[bq * L + l];
            reinterpret_cast<float2 *>(loc)[p] =
                prologue_location(r, reinterpret_cast<const float2 *>(pr.off)[p], s_lv.lvl[l]);
            const float z = pr.logits[p];
            if (pr.shfl) {
                attn[p] = run_softmax(z, pr.per_level ? K : LK);
            } else {
                const float2 st = s_st[i1 * ng + (pr.per_level ? l : 0)];
                attn[p] = expf(z - st.x) * st.y;
            }
        }
    }
}

__global__ void __launch_bounds__(kThreads)
fused_epilogue_kernel(const int64_t *__restrict__ shapes, const int64_t *__restrict__ starts,
                      const float *__restrict__ attn, float *__restrict__ grad_logits,
                      const float *__restrict__ grad_off, const float *__restrict__ ref_part,
                      float *__restrict__ grad_ref, int per_level, int shfl, int64_t groups,
                      int64_t refs, Dims dm) {
    __shared__ LevelLds s_lv;
    stage_levels(&s_lv, shapes, starts, dm.L, dm.Nv, 0x7fffffff);
    const int M = dm.M, K = dm.K, L = dm.L, LK = L * K;
    const int gs = per_level ? K : LK;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t t0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (ref_part) {
        // the dots kernel did the softmax backward and the per-(item, level)
        // sums: only the sum over heads is left
        const float2 *g = reinterpret_cast<const float2 *>(ref_part);
        for (int64_t u = t0; u < refs; u += stride) {
            const int64_t bq = u / L;
            const int l = (int)(u - bq * L);
            float gx = 0.f, gy = 0.f;
            for (int m = 0; m < M; ++m) {
                const float2 v = g[((size_t)bq * M + m) * L + l];
                gx += v.x;
                gy += v.y;
            }
            reinterpret_cast<float2 *>(grad_ref)[u] = make_float2(gx, gy);
        }
        return;
    }
    if (shfl) {
        // one point per lane, in order; a run of gs lanes is one softmax group
        // (gs divides 64 and the stride, so runs never straddle waves)
        const int64_t n = groups * gs;
        for (int64_t p = t0; p < n; p += stride) {
            const float a = attn[p], ga = grad_logits[p];
            const float s = run_sum(a * ga, gs);
            grad_logits[p] = a * (ga - s);
        }
    } else {
        for (int64_t u = t0; u < groups; u += stride) {
            const size_t p0 = (size_t)u * gs;  // the groups tile the points in order
            float s = 0.f;
            for (int j = 0; j < gs; ++j) s = __builtin_fmaf(attn[p0 + j], grad_logits[p0 + j], s);
            for (int j = 0; j < gs; ++j)
                grad_logits[p0 + j] = attn[p0 + j] * (grad_logits[p0 + j] - s);
        }
    }
    if (!grad_ref) return;
    const float2 *g2 = reinterpret_cast<const float2 *>(grad_off);
    if (shfl && (K & (K - 1)) == 0 && K <= 64) {
        // lane per (b, q, l, k): the sum over heads in a register, then over
        // the K lanes of the level
        const int64_t n = refs * K;
        for (int64_t u = t0; u < n; u += stride) {
            const int64_t bq = u / LK;
            const int r = (int)(u - bq * LK), l = r / K;
            const float2 *g = g2 + (size_t)bq * M * LK + r;
            float gx = 0.f, gy = 0.f;
            for (int m = 0; m < M; ++m) {
                const float2 v = g[(size_t)m * LK];
                gx += v.x;
                gy += v.y;
            }
            gx = run_sum(gx, K);
            gy = run_sum(gy, K);
            if (r == l * K) {
                const int4 lvl = s_lv.lvl[l];
                reinterpret_cast<float2 *>(grad_ref)[bq * L + l] =
                    make_float2(gx * (float)lvl.y, gy * (float)lvl.x);
            }
        }
        return;
    }
    for (int64_t u = t0; u < refs; u += stride) {
        const int64_t bq = u / L;
        const int l = (int)(u - bq * L);
        const int4 lvl = s_lv.lvl[l];
        const float2 *g = g2 + ((size_t)bq * M * L + l) * K;
        float gx = 0.f, gy = 0.f;
        for (int m = 0; m < M; ++m)
            for (int k = 0; k < K; ++k) {
                const float2 v = g[(size_t)m * LK + k];
                gx += v.x;
                gy += v.y;
            }
        reinterpret_cast<float2 *>(grad_ref)[u] = make_float2(gx * (float)lvl.y, gy * (float)lvl.x);
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
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
    o = align(o + 16 * (size_t)w.work_max);
    w.off_total = o;
    o = align(o + 4);
    w.off_sorted = o;
    o = align(o + 16 * (size_t)w.sorted_max);
    w.bytes = o;
    return w;
}

struct Launch {
    int ipb, pc, ps;
    size_t lds;
};

// `reserve`: LDS bytes taken from the point-table budget for other uses.
Launch plan(int64_t D, int64_t L, int64_t K, int bytes_per_point, int reserve = 0) {
    Launch p;
    p.ipb = (int)(kThreads / (D / 4));
    const int lk = (int)(L * K);
    int pc = (kSetupLdsBytes - reserve) / (p.ipb * bytes_per_point) - 2;
    pc = pc < 1 ? 1 : pc;
    p.pc = pc < lk ? pc : lk;
    p.ps = p.pc + ((p.pc % 2 == 0) ? 1 : 2);
    p.lds = (size_t)p.ipb * p.ps * bytes_per_point;
    return p;
}

// A softmax group that lane shuffles can reduce: a power of two <= 64.
bool pow2_run(int64_t n) { return n >= 1 && n <= 64 && (n & (n - 1)) == 0; }

FastDiv make_fastdiv(uint32_t d) {  // d >= 1
    uint32_t shift = 0;
    while (shift < 31 && (1u << shift) < d) ++shift;
    const uint64_t mul = ((uint64_t)1 << 32) * (((uint64_t)1 << shift) - d) / d + 1;
    return FastDiv{(uint32_t)mul, shift};
}

// pr == nullptr: locations and weights from loc / attn; otherwise from the
// prologue inputs (loc and attn unused).
template <int D, typename VT>
msda_status launch_fwd(const void *value, const int64_t *shapes, const int64_t *starts,
                       const float *loc, const float *attn, const Prologue *pr, float *out,
                       int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t L, int64_t K,
                       bool align, hipStream_t s) {
    const int ipb = (int)(kThreads / (D / 4));
    Prologue prv = pr ? *pr : Prologue{nullptr, nullptr, nullptr, 0, 0, nullptr, nullptr};
    int st_bytes = 0;
    Launch p = plan(D, L, K, 32);
    if (pr) {
        // softmax by lane shuffles when the items' points come in one chunk and
        // the groups are power-of-two runs of at most 64; else statistics in LDS
        prv.shfl = (p.pc == L * K && pow2_run(pr->per_level ? K : L * K)) ? 1 : 0;
        if (!prv.shfl) {
            st_bytes = ipb * (pr->per_level ? (int)L : 1) * (int)sizeof(float2);
            p = plan(D, L, K, 32, st_bytes);
        }
    }
    const size_t lds = p.lds + (size_t)st_bytes;
    const int64_t items = Nq * M;
    const int64_t gx = (items + p.ipb - 1) / p.ipb;
    const int64_t bchunk = batch_chunk(gx, B);
    for (int64_t b0 = 0; b0 < B; b0 += bchunk) {
        const int64_t nb = (B - b0) < bchunk ? (B - b0) : bchunk;
        Dims dm{(int)Nv, (int)Nq, (int)M, (int)L, (int)K, p.pc, p.ps, (int)b0, (int)gx, 0, 0};
        dm.align = align ? 1 : 0;
        const dim3 grid((unsigned)(gx * nb));
        if (pr)
            hipLaunchKernelGGL((msda_fwd_kernel<D, VT, true>), grid, dim3(kThreads), lds, s,
                               static_cast<const VT *>(value), shapes, starts, loc, attn, prv,
                               out, dm);
        else
            hipLaunchKernelGGL((msda_fwd_kernel<D, VT, false>), grid, dim3(kThreads), lds, s,
                               static_cast<const VT *>(value), shapes, starts, loc, attn, prv,
                               out, dm);
        msda_status st = hip_status(hipGetLastError());
        if (st != MSDA_OK) return st;
    }
    return MSDA_OK;
}

// Where the backward enqueues: the caller's stream, an optional side stream
// (with its fork / join events) and optional per-stage timing events.
struct Exec {
    hipStream_t s;
    hipStream_t side;
    hipEvent_t fork, filled, join;  // fork from s; grad_value zeroed; side work done
    hipEvent_t *ev;                 // optional: 2 * MSDA_BWD_STAGES caller events (start, end)
    bool fill_on_side;              // the grad_value zero-fill was enqueued on `side`
    // record the start (end = false) or end event of stage i on stream `on`
    void stamp(int i, bool end, hipStream_t on) const {
        if (ev && ev[2 * i + (end ? 1 : 0)]) (void)hipEventRecord(ev[2 * i + (end ? 1 : 0)], on);
    }
};

// The fused prologue's backward, as far as the dots kernel takes it: it
// writes offset gradients (location gradients / (W, H)) always; with in_dots
// also the logit gradients (softmax runs of softmax_run points) and, given
// ref_part, the per-(item, level) location-gradient sums [B][Nq][M][L][2].
struct FusedBwd {
    int softmax_run;  // requested run length (0: the runs do not fit lane shuffles)
    float *ref_part;  // nullptr: no reference-point gradient wanted
    bool in_dots;     // set by the launch: the dots kernel did both
};

// One side stream per device, created on first use (default priority,
// non-blocking with respect to the null stream).  The mutex is held while a
// backward enqueues, so the fork / join events are never shared between two
// calls in flight on the host.
constexpr int kMaxDevices = 64;
struct SideStream {
    bool tried = false;
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, filled = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

// Call with g_side_mu held.  nullptr when no side stream can be had.
SideStream *side_stream() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    SideStream &ss = g_side[dev];
    if (!ss.tried) {
        ss.tried = true;
        bool ok = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) == hipSuccess;
        ok = ok && hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) == hipSuccess;
        ok = ok && hipEventCreateWithFlags(&ss.filled, hipEventDisableTiming) == hipSuccess;
        ok = ok && hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) == hipSuccess;
        if (!ok) {
            if (ss.join) (void)hipEventDestroy(ss.join);
            if (ss.filled) (void)hipEventDestroy(ss.filled);
            if (ss.fork) (void)hipEventDestroy(ss.fork);
            if (ss.s) (void)hipStreamDestroy(ss.s);
            ss.s = nullptr;
            ss.fork = ss.filled = ss.join = nullptr;
            (void)hipGetLastError();
        }
    }
    return ss.s ? &ss : nullptr;
}

template <int D, typename VT>
msda_status launch_bwd(const void *value, const int64_t *shapes, const int64_t *starts,
                       const float *loc, const float *attn, const float *gout, float *gval,
                       float *gloc, float *gattn, int64_t B, int64_t Nv, int64_t Nq, int64_t M,
                       int64_t L, int64_t K, const WorkLayout &wl, unsigned char *ws,
                       bool accumulate, bool align, FusedBwd *fz, const Exec &ex) {
    const hipStream_t s = ex.s;
    Work w;
    w.counts = reinterpret_cast<uint32_t *>(ws + wl.off_counts);
    w.start = reinterpret_cast<uint32_t *>(ws + wl.off_start);
    w.cursor = reinterpret_cast<uint32_t *>(ws + wl.off_cursor);
    w.items = reinterpret_cast<uint4 *>(ws + wl.off_items);
    w.work_total = reinterpret_cast<uint32_t *>(ws + wl.off_total);
    w.recs = reinterpret_cast<uint4 *>(ws + wl.off_sorted);
    // grad_attn_weight and grad_sampling_loc do not depend on the bin
    // pipeline: with a side stream (forked from the caller's stream before
    // anything else) they are computed there, concurrently, and the caller's
    // stream waits for them at the end
    const hipStream_t ds = ex.side ? ex.side : s;
    const Launch p = plan(D, L, K, 32);
    const int64_t gq = (Nq + p.ipb - 1) / p.ipb;
    // the dots kernel finishes the fused prologue's backward itself when its
    // point table holds whole items and the softmax runs fit a wave
    if (fz) fz->in_dots = fz->softmax_run > 0 && p.pc == L * K;
    float *ref_part = fz && fz->in_dots ? fz->ref_part : nullptr;
    auto per_batch = [&](int64_t per_b, auto &&launch) -> msda_status {
        const int64_t bchunk = batch_chunk(per_b, B);
        for (int64_t b0 = 0; b0 < B; b0 += bchunk) {
            const int64_t nb = (B - b0) < bchunk ? (B - b0) : bchunk;
            launch(b0, (unsigned)(per_b * nb));
            const msda_status e = hip_status(hipGetLastError());
            if (e != MSDA_OK) return e;
        }
        return MSDA_OK;
    };
    ex.stamp(1, false, ds);
    msda_status st = per_batch(gq * M, [&](int64_t b0, unsigned grid) {
        Dims d2{(int)Nv, (int)Nq, (int)M, (int)L, (int)K, p.pc, p.ps, (int)b0, (int)gq, 0, 0};
        d2.nblocks = (int)grid;
        d2.align = align ? 1 : 0;
        d2.loc_div = fz ? 1 : 0;
        d2.softmax_run = fz && fz->in_dots ? fz->softmax_run : 0;
        // a few workgroups per CU suffice for this gather-bound kernel, and leave
        // room for the grad_value kernels running beside it
        const unsigned g = grid > (unsigned)kDotsGrid ? (unsigned)kDotsGrid : grid;
        hipLaunchKernelGGL((bwd_dots_kernel<D, VT>), dim3(g), dim3(kThreads), p.lds, ds,
                           static_cast<const VT *>(value), shapes, starts, loc, attn, gout, gloc,
                           gattn, ref_part, d2);
    });
    if (st != MSDA_OK) return st;
    ex.stamp(1, true, ds);
    if (ex.side) {
        st = hip_status(hipEventRecord(ex.join, ex.side));
        if (st != MSDA_OK) return st;
    }

    // the counts region is padded to 256 bytes, so whole float4s can be cleared
    ex.stamp(2, false, s);
    st = fill_zero(w.counts, (wl.off_start - wl.off_counts) / 16, s);
    if (st != MSDA_OK) return st;
    ex.stamp(2, true, s);

    const int hist_cap = (int)(wl.nb_max < kHistLds ? wl.nb_max : kHistLds);
    const int64_t gb = (Nq * L * K + kBinPoints - 1) / kBinPoints;  // per (batch, head)
    Dims dm{(int)Nv, (int)Nq, (int)M, (int)L, (int)K, 0, 0, 0, (int)gb, (int)wl.nb_max,
            accumulate ? 1 : 0, make_fastdiv((uint32_t)(L * K)), make_fastdiv((uint32_t)K)};
    dm.align = align ? 1 : 0;
    ex.stamp(3, false, s);
    st = per_batch(gb * M, [&](int64_t b0, unsigned grid) {
        Dims d2 = dm;
        d2.b0 = (int)b0;
        hipLaunchKernelGGL(bin_count_kernel, dim3(grid), dim3(kThreads), 4 * (size_t)hist_cap, s,
                           shapes, starts, loc, w.counts, hist_cap, d2);
    });
    if (st != MSDA_OK) return st;
    ex.stamp(3, true, s);

    ex.stamp(4, false, s);
    hipLaunchKernelGGL(bin_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, shapes, starts,
                       w.counts, w.start, w.cursor, w.items, w.work_total, (int)B, dm);
    st = hip_status(hipGetLastError());
    if (st != MSDA_OK) return st;
    ex.stamp(4, true, s);

    ex.stamp(5, false, s);
    st = per_batch(gb * M, [&](int64_t b0, unsigned grid) {
        Dims d2 = dm;
        d2.b0 = (int)b0;
        hipLaunchKernelGGL(bin_scatter_kernel, dim3(grid), dim3(kThreads), 8 * (size_t)hist_cap,
                           s, shapes, starts, loc, attn, w.cursor, w.recs, hist_cap, d2);
    });
    if (st != MSDA_OK) return st;
    ex.stamp(5, true, s);

    const int64_t grid = wl.work_max < kTileGrid ? wl.work_max : kTileGrid;
    if (ex.fill_on_side) {
        st = hip_status(hipStreamWaitEvent(s, ex.filled, 0));
        if (st != MSDA_OK) return st;
    }
    ex.stamp(6, false, s);
    hipLaunchKernelGGL((grad_value_tile_kernel<D>), dim3((unsigned)grid), dim3(kTileThreads), 0, s,
                       shapes, starts, gout, w.items, w.work_total, w.recs, gval, dm);
    st = hip_status(hipGetLastError());
    ex.stamp(6, true, s);
    if (st == MSDA_OK && ex.side) st = hip_status(hipStreamWaitEvent(s, ex.join, 0));
    return st;
}

template <typename VT>
msda_status dispatch_fwd(int64_t D, const void *value, const int64_t *shapes,
                         const int64_t *starts, const float *loc, const float *attn,
                         const Prologue *pr, float *out, int64_t B, int64_t Nv, int64_t Nq,
                         int64_t M, int64_t L, int64_t K, bool align, hipStream_t s) {
#define MSDA_FWD_CASE(DD)                                                                     \
    case DD:                                                                                  \
        return launch_fwd<DD, VT>(value, shapes, starts, loc, attn, pr, out, B, Nv, Nq, M, L,  \
                                  K, align, s);
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
                         const WorkLayout &wl, unsigned char *ws, bool acc, bool align,
                         FusedBwd *fz, const Exec &ex) {
#define MSDA_BWD_CASE(DD)                                                                      \
    case DD:                                                                                   \
        return launch_bwd<DD, VT>(value, shapes, starts, loc, attn, gout, gval, gloc, gattn, B, \
                                  Nv, Nq, M, L, K, wl, ws, acc, align, fz, ex);
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
                         int64_t Nq, int64_t M, int64_t D, int64_t L, int64_t K, uint32_t flags,
                         void *stream) {
    msda_status st = check_sizes(value_dtype, B, Nv, Nq, M, D, L, K);
    if (st != MSDA_OK) return st;
    if (flags & ~MSDA_ALIGN_CORNERS) return MSDA_ERR_UNSUPPORTED;
    const bool align = (flags & MSDA_ALIGN_CORNERS) != 0;
    if (B == 0 || Nq == 0) return MSDA_OK;
    if (Nv < 1) return MSDA_ERR_SHAPE;
    if (!value || !spatial_shapes || !level_start_index || !sampling_loc || !attn_weight || !out)
        return MSDA_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (value_dtype == MSDA_F32)
        return dispatch_fwd<float>(D, value, spatial_shapes, level_start_index, sampling_loc,
                                   attn_weight, nullptr, out, B, Nv, Nq, M, L, K, align, s);
    return dispatch_fwd<uint16_t>(D, value, spatial_shapes, level_start_index, sampling_loc,
                                  attn_weight, nullptr, out, B, Nv, Nq, M, L, K, align, s);
}

msda_status msda_forward_fused(const void *value, int value_dtype,
                               const int64_t *spatial_shapes, const int64_t *level_start_index,
                               const float *reference_points, const float *sampling_offsets,
                               const float *attn_logits, float *out, float *sampling_loc_out,
                               float *attn_weight_out, int64_t B, int64_t Nv, int64_t Nq,
                               int64_t M, int64_t D, int64_t L, int64_t K, uint32_t flags,
                               void *stream) {
    msda_status st = check_sizes(value_dtype, B, Nv, Nq, M, D, L, K);
    if (st != MSDA_OK) return st;
    if (flags & ~(MSDA_ALIGN_CORNERS | MSDA_SOFTMAX_PER_LEVEL)) return MSDA_ERR_UNSUPPORTED;
    const bool align = (flags & MSDA_ALIGN_CORNERS) != 0;
    if (B == 0 || Nq == 0) return MSDA_OK;
    if (Nv < 1) return MSDA_ERR_SHAPE;
    if (!value || !spatial_shapes || !level_start_index || !reference_points ||
        !sampling_offsets || !attn_logits || !out)
        return MSDA_ERR_NULL;
    if ((sampling_loc_out == nullptr) != (attn_weight_out == nullptr)) return MSDA_ERR_NULL;
    const Prologue pr{reference_points, sampling_offsets, attn_logits,
                      (flags & MSDA_SOFTMAX_PER_LEVEL) ? 1 : 0, 0, sampling_loc_out,
                      attn_weight_out};
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (value_dtype == MSDA_F32)
        return dispatch_fwd<float>(D, value, spatial_shapes, level_start_index, nullptr, nullptr,
                                   &pr, out, B, Nv, Nq, M, L, K, align, s);
    return dispatch_fwd<uint16_t>(D, value, spatial_shapes, level_start_index, nullptr, nullptr,
                                  &pr, out, B, Nv, Nq, M, L, K, align, s);
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
                          FusedBwd *fz, hipStream_t s, hipEvent_t *ev) {
    msda_status st = check_sizes(value_dtype, B, Nv, Nq, M, D, L, K);
    if (st != MSDA_OK) return st;
    if (flags & ~(MSDA_BWD_ACCUMULATE | MSDA_ALIGN_CORNERS)) return MSDA_ERR_UNSUPPORTED;
    // a grad_value record stores the query index in 25 bits
    if (Nq > ((int64_t)1 << (32 - kRecQueryShift))) return MSDA_ERR_UNSUPPORTED;
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
        // bin counters and work items are indexed with 31-bit integers
        if (wl.bm_bins >= ((int64_t)1 << 31) || wl.work_max >= ((int64_t)1 << 31))
            return MSDA_ERR_UNSUPPORTED;
        if (!workspace) return MSDA_ERR_NULL;
        if (workspace_bytes < wl.bytes) return MSDA_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return MSDA_ERR_WORKSPACE;
    }
    Exec ex{s, nullptr, nullptr, nullptr, nullptr, ev, false};
    std::unique_lock<std::mutex> lock(g_side_mu, std::defer_lock);
    if (work) {
        lock.lock();
        if (SideStream *ss = side_stream()) {
            ex.side = ss->s;
            ex.fork = ss->fork;
            ex.filled = ss->filled;
            ex.join = ss->join;
        }
    }
    if (ex.side) {
        st = hip_status(hipEventRecord(ex.fork, s));
        if (st == MSDA_OK) st = hip_status(hipStreamWaitEvent(ex.side, ex.fork, 0));
        if (st != MSDA_OK) return st;
    }
    if (!(flags & MSDA_BWD_ACCUMULATE)) {
        // with a side stream the fill runs there, ahead of the dots kernel, and
        // the tile kernel waits for it
        const hipStream_t fs = ex.side ? ex.side : s;
        ex.stamp(0, false, fs);
        st = fill_zero(grad_value, (size_t)nval / 4, fs);  // D % 4 == 0
        ex.stamp(0, true, fs);
        if (st == MSDA_OK && ex.side) {
            st = hip_status(hipEventRecord(ex.filled, ex.side));
            ex.fill_on_side = true;
        }
        if (st != MSDA_OK) return st;
    }
    if (flags & MSDA_BWD_ACCUMULATE) {  // no fill: an empty stage
        ex.stamp(0, false, s);
        ex.stamp(0, true, s);
    }
    if (!work) {
        for (int i = 1; i < MSDA_BWD_STAGES; ++i) {
            ex.stamp(i, false, s);
            ex.stamp(i, true, s);
        }
        return MSDA_OK;
    }
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    const bool acc = (flags & MSDA_BWD_ACCUMULATE) != 0;
    const bool align = (flags & MSDA_ALIGN_CORNERS) != 0;
    if (value_dtype == MSDA_F32)
        return dispatch_bwd<float>(D, value, spatial_shapes, level_start_index, sampling_loc,
                                   attn_weight, grad_out, grad_value, grad_sampling_loc,
                                   grad_attn_weight, B, Nv, Nq, M, L, K, wl, ws, acc, align,
                                   fz, ex);
    return dispatch_bwd<uint16_t>(D, value, spatial_shapes, level_start_index, sampling_loc,
                                  attn_weight, grad_out, grad_value, grad_sampling_loc,
                                  grad_attn_weight, B, Nv, Nq, M, L, K, wl, ws, acc, align,
                                  fz, ex);
}

// Workspace of the fused backward: the core's, then the locations [pts][2]
// and weights [pts] the prologue writes.
struct FusedLayout {
    size_t core, off_loc, off_attn, off_part, bytes;
};

FusedLayout fused_layout(int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t L, int64_t K) {
    auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t pts = (size_t)(B * Nq * M * L * K);
    FusedLayout f;
    f.core = work_layout(B, Nv, Nq, M, L, K).bytes;
    f.off_loc = f.core;
    f.off_attn = align(f.off_loc + 8 * pts);
    f.off_part = align(f.off_attn + 4 * pts);
    f.bytes = align(f.off_part + 8 * (size_t)(B * Nq * M * L));
    return f;
}

msda_status backward_fused_impl(const void *value, int value_dtype, const int64_t *shapes,
                                const int64_t *starts, const float *ref, const float *off,
                                const float *logits, const float *saved_loc,
                                const float *saved_attn, const float *grad_out, float *grad_value,
                                float *grad_off, float *grad_logits, float *grad_ref, int64_t B,
                                int64_t Nv, int64_t Nq, int64_t M, int64_t D, int64_t L,
                                int64_t K, void *workspace, size_t workspace_bytes,
                                uint32_t flags, hipStream_t s, hipEvent_t *ev) {
    msda_status st = check_sizes(value_dtype, B, Nv, Nq, M, D, L, K);
    if (st != MSDA_OK) return st;
    if (flags & ~(MSDA_BWD_ACCUMULATE | MSDA_ALIGN_CORNERS | MSDA_SOFTMAX_PER_LEVEL))
        return MSDA_ERR_UNSUPPORTED;
    const bool per_level = (flags & MSDA_SOFTMAX_PER_LEVEL) != 0;
    const uint32_t core_flags = flags & ~MSDA_SOFTMAX_PER_LEVEL;
    const bool work = B > 0 && Nq > 0;
    auto stamp = [&](int i, bool end) {
        if (ev && ev[2 * i + (end ? 1 : 0)]) (void)hipEventRecord(ev[2 * i + (end ? 1 : 0)], s);
    };
    if (!work) {
        stamp(MSDA_BWD_STAGES, false);
        stamp(MSDA_BWD_STAGES, true);
        FusedBwd none{0, nullptr, false};
        st = backward_impl(value, value_dtype, shapes, starts, nullptr, nullptr, grad_out,
                           grad_value, nullptr, nullptr, B, Nv, Nq, M, D, L, K, workspace,
                           workspace_bytes, core_flags, &none, s, ev);
        stamp(MSDA_BWD_STAGES + 1, false);
        stamp(MSDA_BWD_STAGES + 1, true);
        return st;
    }
    if (Nv < 1) return MSDA_ERR_SHAPE;
    if (!value || !shapes || !starts || !ref || !off || !logits || !grad_out || !grad_value ||
        !grad_off || !grad_logits)
        return MSDA_ERR_NULL;
    if ((saved_loc == nullptr) != (saved_attn == nullptr)) return MSDA_ERR_NULL;
    if (!workspace) return MSDA_ERR_NULL;
    const FusedLayout fl = fused_layout(B, Nv, Nq, M, L, K);
    if (workspace_bytes < fl.bytes) return MSDA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return MSDA_ERR_WORKSPACE;
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    const bool saved = saved_loc != nullptr;
    float *loc = reinterpret_cast<float *>(ws + fl.off_loc);
    float *attn = reinterpret_cast<float *>(ws + fl.off_attn);
    const int shfl = pow2_run(per_level ? K : L * K) ? 1 : 0;
    const Prologue pr{ref, off, logits, per_level ? 1 : 0, shfl, nullptr, nullptr};
    Dims dm{(int)Nv, (int)Nq, (int)M, (int)L, (int)K, 0, 0, 0, 0, 0, 0};
    const int64_t items = B * Nq * M;

    stamp(MSDA_BWD_STAGES, false);
    if (!saved) {
        const int64_t blocks = (items + kProItems - 1) / kProItems;
        const unsigned grid = (unsigned)(blocks < (1 << 20) ? blocks : (1 << 20));
        const size_t lds = shfl ? 0 : (size_t)kProItems * (per_level ? L : 1) * sizeof(float2);
        hipLaunchKernelGGL(fused_prologue_kernel, dim3(grid), dim3(kThreads), lds, s, shapes,
                           starts, pr, loc, attn, items, dm);
        st = hip_status(hipGetLastError());
        if (st != MSDA_OK) return st;
    }
    stamp(MSDA_BWD_STAGES, true);

    FusedBwd fz{shfl ? (int)(per_level ? K : L * K) : 0,
                grad_ref ? reinterpret_cast<float *>(ws + fl.off_part) : nullptr, false};
    const float *use_loc = saved ? saved_loc : loc, *use_attn = saved ? saved_attn : attn;
    st = backward_impl(value, value_dtype, shapes, starts, use_loc, use_attn, grad_out,
                       grad_value, grad_off, grad_logits, B, Nv, Nq, M, D, L, K, ws, fl.core,
                       core_flags, &fz, s, ev);
    if (st != MSDA_OK) return st;

    stamp(MSDA_BWD_STAGES + 1, false);
    if (fz.in_dots) {
        if (grad_ref) {
            const int64_t refs = B * Nq * L;
            int64_t blocks = (refs + kThreads - 1) / kThreads;
            blocks = blocks < (1 << 16) ? blocks : (1 << 16);
            hipLaunchKernelGGL(fused_epilogue_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                               s, shapes, starts, use_attn, grad_logits, grad_off, fz.ref_part,
                               grad_ref, per_level ? 1 : 0, shfl, (int64_t)0, refs, dm);
            st = hip_status(hipGetLastError());
        }
    } else {
        const int64_t groups = items * (per_level ? L : 1);
        const int64_t refs = grad_ref ? B * Nq * L : 0;
        // lanes per unit of work: a point (shuffle path) or a group / reference
        const int64_t gl = shfl ? (per_level ? K : L * K) : 1, rl = shfl ? K : 1;
        const int64_t units = groups * gl > refs * rl ? groups * gl : refs * rl;
        int64_t blocks = (units + kThreads - 1) / kThreads;
        blocks = blocks < (1 << 16) ? blocks : (1 << 16);
        hipLaunchKernelGGL(fused_epilogue_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                           shapes, starts, use_attn, grad_logits, grad_off, nullptr, grad_ref,
                           per_level ? 1 : 0, shfl, groups, refs, dm);
        st = hip_status(hipGetLastError());
    }
    stamp(MSDA_BWD_STAGES + 1, true);
    return st;
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
                         B, Nv, Nq, M, D, L, K, workspace, workspace_bytes, flags, nullptr,
                         static_cast<hipStream_t>(stream), nullptr);
}

msda_status msda_backward_events(const void *value, int value_dtype,
                                 const int64_t *spatial_shapes, const int64_t *level_start_index,
                                 const float *sampling_loc, const float *attn_weight,
                                 const float *grad_out, float *grad_value,
                                 float *grad_sampling_loc, float *grad_attn_weight, int64_t B,
                                 int64_t Nv, int64_t Nq, int64_t M, int64_t D, int64_t L,
                                 int64_t K, void *workspace, size_t workspace_bytes,
                                 uint32_t flags, void *stream, void *const *events) {
    if (!events) return MSDA_ERR_NULL;
    hipEvent_t ev[2 * MSDA_BWD_STAGES];
    for (int i = 0; i < 2 * MSDA_BWD_STAGES; ++i) ev[i] = static_cast<hipEvent_t>(events[i]);
    return backward_impl(value, value_dtype, spatial_shapes, level_start_index, sampling_loc,
                         attn_weight, grad_out, grad_value, grad_sampling_loc, grad_attn_weight,
                         B, Nv, Nq, M, D, L, K, workspace, workspace_bytes, flags, nullptr,
                         static_cast<hipStream_t>(stream), ev);
}

size_t msda_backward_fused_workspace_size(int64_t B, int64_t Nv, int64_t Nq, int64_t M,
                                          int64_t D, int64_t L, int64_t K) {
    if (check_sizes(MSDA_F32, B, Nv, Nq, M, D, L, K) != MSDA_OK) return 0;
    if (B == 0 || Nq == 0) return 0;
    return fused_layout(B, Nv, Nq, M, L, K).bytes;
}

msda_status msda_backward_fused(const void *value, int value_dtype,
                                const int64_t *spatial_shapes, const int64_t *level_start_index,
                                const float *reference_points, const float *sampling_offsets,
                                const float *attn_logits, const float *sampling_loc,
                                const float *attn_weight, const float *grad_out,
                                float *grad_value, float *grad_sampling_offsets,
                                float *grad_attn_logits, float *grad_reference_points, int64_t B,
                                int64_t Nv, int64_t Nq, int64_t M, int64_t D, int64_t L,
                                int64_t K, void *workspace, size_t workspace_bytes,
                                uint32_t flags, void *stream, void *const *events) {
    hipEvent_t ev[2 * MSDA_BWD_FUSED_STAGES];
    if (events)
        for (int i = 0; i < 2 * MSDA_BWD_FUSED_STAGES; ++i)
            ev[i] = static_cast<hipEvent_t>(events[i]);
    return backward_fused_impl(value, value_dtype, spatial_shapes, level_start_index,
                               reference_points, sampling_offsets, attn_logits, sampling_loc,
                               attn_weight, grad_out,
                               grad_value, grad_sampling_offsets, grad_attn_logits,
                               grad_reference_points, B, Nv, Nq, M, D, L, K, workspace,
                               workspace_bytes, flags, static_cast<hipStream_t>(stream),
                               events ? ev : nullptr);
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

int msda_last_hip_error(void) { return msda_internal_last_hip_error; }

}  // extern "C"
