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
// sample, accumulated in registers, one store per item.  A workgroup takes
// consecutive queries of one (batch, head).
//
// Backward (msda_backward):
//   bwd_dots_kernel (on a side stream, concurrently with the rest, for
//      problems of at least 2^18 points; otherwise first on the caller's
//      stream, where it also clears the bin counters): per point the four
//      <grad_out row, neighbour row> dot products, reduced across the lane
//      group with DPP, give grad_attn_weight and grad_sampling_loc.
//   grad_value is a scatter (every point adds A * w * grad_out into four
//   pixels).  fp32 atomics run at a few hundred G lane-ops/s on this chip,
//   in LDS as in memory, so it is computed in gather form instead, per 8x8
//   pixel tile and head ("bin"):
//   bin_count_kernel: points per bin (LDS histogram, one global add per bin
//      and workgroup).
//   bin_scan_kernel: exclusive scan of the counts -> bin offsets, and a work
//      list of (bin, chunk of at most kChunk records); a workgroup per block
//      of bins.
//   bin_scatter_kernel: one 16-byte record per (point, bin) it touches,
//      written into its bin (LDS ranks, one global reservation per bin and
//      workgroup).
//   grad_value_gather_kernel (heads of up to 32 channels): per work item,
//      the records are counting-sorted once by the cell of their top-left
//      neighbour; a lane owns a (cell, channel quad) pair, gathers the
//      grad_out row of each of its cell's records from memory and keeps one
//      sum per neighbour role; the role sums meet in LDS, each pixel
//      written once.
//   grad_value_tile_kernel (wider heads): the records are sorted per
//      sub-chunk and their grad_out rows staged in LDS in that order; a lane
//      owns (pixel, channel quad) pairs and sums over the four cells that
//      feed its pixel.  In both, only bins split over several chunks add
//      into grad_value atomically.
//
// value and grad_value are addressed through raw buffer descriptors whose
// size is the batch slice.  A neighbour outside the map gets the offset
// kOOB, beyond every slice, so its fetch returns zeros without a branch; the
// same range check keeps an inconsistent level table from touching other
// memory.

#include <mutex>
#include <type_traits>

#include "bins.h"

// hipError_t of the last MSDA_ERR_HIP on this thread, for every translation unit
thread_local int msda_internal_last_hip_error = 0;

namespace {

constexpr int kSetupLdsBytes = 36 * 1024;  // per-workgroup budget for the point tables
// the forward's budget when an item has more than 16 points: half, so that
// 8 workgroups fit a CU's LDS, with the points in chunks of at least 16 (the
// dots kernel, capped at 2 workgroups per CU, keeps whole items instead)
constexpr int kFwdLdsBytes = 18 * 1024;
constexpr int kDotsBatch = 4;              // points whose row loads the dots kernel overlaps
// the one-kernel backward of heads with few points: at most kSmallPoints
// points per (batch, head), workgroups of kSmallPixels pixels
constexpr int kSmallPoints = 256;
constexpr int kSmallPixels = 256;
static_assert(kSmallPoints <= kThreads, "one thread per point builds the point table");
static_assert(kSmallPixels % kThreads == 0, "each thread scans kSmallPixels / kThreads counts");

// Raw inputs of the fused prologue, which computes the sampling location and
// the attention weight of each point from them:
//   loc = ref[b, q, l] + off[b, q, m, l, k] / (W_l, H_l)   (fp32: one IEEE
//         division and one addition per coordinate)
//   A   = softmax of the logits over the L*K points of (b, q, m), or over the
//         K points of each level when per_level is set, times the scale
//         attention S of the point when one is given.
struct Prologue {
    const float *ref;     // [B, Nq, L, 2]
    const float *off;     // [B, Nq, M, L, K, 2]
    const float *logits;  // [B, Nq, M, L * K]
    const float *scale;   // [B, Nq, M, L, K] or nullptr (S = 1)
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

// Softmax statistics of the groups of nitems items, the first at point pt0
// and the others istride points apart, into s_st[item * groups + group].
__device__ __forceinline__ void stage_softmax_stats(float2 *s_st, const Prologue &pr, size_t pt0,
                                                    size_t istride, int nitems, int L, int K) {
    const int LK = L * K, ng = pr.per_level ? L : 1, gs = pr.per_level ? K : LK;
    for (int idx = threadIdx.x; idx < nitems * ng; idx += blockDim.x) {
        const int i1 = idx / ng, g = idx - i1 * ng;
        s_st[idx] = softmax_stats(pr.logits + pt0 + (size_t)i1 * istride + (size_t)g * gs, gs);
    }
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
// With FUSED the locations and weights come from the prologue inputs `pr`
// (loc and attn are unused): per item the softmax statistics of its logits
// are staged in LDS first, then each point's location and weight are formed
// where the plain kernel loads them.
// SPLIT lane groups share an item, each taking every SPLIT-th point, and
// their sums are added across lanes at the end: for problems too small to
// fill the chip with one group per item (the decoder's 300 queries), it
// gives 4x the workgroups and a quarter of the dependent row loads per lane.
template <int D>
constexpr int fwd_split() {
    return D <= 64 ? 4 : (D == 128 ? 2 : 1);  // SPLIT * D / 4 lanes stay within a wave
}

template <int D, typename VT, bool FUSED, int SPLIT>
__global__ void __launch_bounds__(kThreads)
msda_fwd_kernel(const VT *__restrict__ value, const int64_t *__restrict__ shapes,
                const int64_t *__restrict__ starts, const float *__restrict__ loc,
                const float *__restrict__ attn, Prologue pr, float *__restrict__ out, Dims dm) {
    constexpr int G = D / 4;
    constexpr int IPB = kThreads / (G * SPLIT);
    static_assert(G * SPLIT <= 64, "an item's lanes lie in one wave");
    __shared__ LevelLds s_lv;
    extern __shared__ __align__(16) unsigned char smem[];
    uint4 *s_off = reinterpret_cast<uint4 *>(smem);
    float4 *s_w = reinterpret_cast<float4 *>(s_off + IPB * dm.PS);
    float2 *s_st = reinterpret_cast<float2 *>(s_w + IPB * dm.PS);  // FUSED: softmax stats

    const int M = dm.M, K = dm.K, LK = dm.L * dm.K;
    // blocks of IPB queries of one (batch, head), dm.nblk per (batch, head),
    // in (batch, head, block) order, taken in launch order: consecutive
    // workgroups, spread over the XCDs by the dispatcher, gather from the same
    // stretch of the value rows at the same time.  (A mapping that gives each
    // XCD one contiguous range of blocks was measured slower: 105 vs 102 us
    // here, 150 vs 132 us for the dots kernel, at the encoder shape.)
    const int wg = blockIdx.x;
    const int bm = wg / dm.nblk + dm.b0 * M;
    const int m = bm % M, b = bm / M;
    const int q0 = (wg % dm.nblk) * IPB;
    const int nitems = min(IPB, dm.Nq - q0);
    const uint32_t row_stride = (uint32_t)M * D * 4u;
    const uint32_t head_off = (uint32_t)m * D * 4u;

    stage_levels(&s_lv, shapes, starts, dm.L, dm.Nv, 0x7fffffff);

    const size_t slice = (size_t)dm.Nv * M * D;
    const rsrc_t vr = make_rsrc(value + (size_t)b * slice, (uint32_t)(slice * sizeof(VT)));
    const size_t row0 = ((size_t)b * dm.Nq + q0) * M + m;  // item row of query q0
    const size_t pt0 = row0 * LK;
    const size_t istride = (size_t)M * LK;  // points between consecutive queries' items
    const int ng = pr.per_level ? dm.L : 1;
    if constexpr (FUSED) {
        if (!pr.shfl) {
            stage_softmax_stats(s_st, pr, pt0, istride, nitems, dm.L, K);
            __syncthreads();
        }
    }

    const int it = threadIdx.x / (G * SPLIT), sub = (threadIdx.x / G) % SPLIT, c = threadIdx.x % G;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);

    for (int j0 = 0; j0 < LK; j0 += dm.PC) {
        const int pc = min(dm.PC, LK - j0);
        if (j0) __syncthreads();  // previous chunk consumed
        for (int idx = threadIdx.x; idx < nitems * pc; idx += kThreads) {
            const int i1 = idx / pc, jj = idx - i1 * pc, j = j0 + jj;
            const size_t p = pt0 + (size_t)i1 * istride + j;
            const int l = j / K;
            float2 uv;
            float A;
            if constexpr (FUSED) {
                const int q = q0 + i1;
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
                if (pr.scale) A *= pr.scale[p];
                if (pr.loc_out) {
                    reinterpret_cast<float2 *>(pr.loc_out)[p] = uv;
                    pr.attn_out[p] = A;
                }
            } else {
                uv = reinterpret_cast<const float2 *>(loc)[p];
                A = attn[p];
            }
            Neighbours n = neighbours(uv.x, uv.y, s_lv.lvl[l], row_stride, head_off, dm.align);
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
            // two points (eight rows) per step: measured against 1, 3 and 4 at
            // the encoder shape (98 us vs 102) and the bf16 training shape (406 vs 425-461)
#pragma unroll 2
            for (int jj = sub; jj < pc; jj += SPLIT) {
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
    if constexpr (SPLIT > 1) {  // the item's groups are lanes G apart in one wave
#pragma unroll
        for (int o = G; o < G * SPLIT; o <<= 1) {
            acc.x += __shfl_xor(acc.x, o, 64);
            acc.y += __shfl_xor(acc.y, o, 64);
            acc.z += __shfl_xor(acc.z, o, 64);
            acc.w += __shfl_xor(acc.w, o, 64);
        }
    }
    if (it < nitems && sub == 0) {
        float4 *o = reinterpret_cast<float4 *>(out + (row0 + (size_t)it * M) * D) + c;
        *o = acc;
    }
}

// ---------------------------------------------------------------------------
// backward: grad_attn_weight and grad_sampling_loc
// Workgroup = (batch b, head m, IPB consecutive queries).  Per point the
// table holds the four row offsets (later overwritten by the four dot
// products <grad_out row, value row>) and (fx, fy, A, valid bits).
// ---------------------------------------------------------------------------
// The fused prologue's scale attention in the softmax backward: the weight
// the core used is A = S * P with P the softmax of the logits, so with
// g = d/dA, d/dS = P g and d/dlogit = P (S g - sum over the group of P S g)
// = A g - P sum(A g).  P is formed again from the logits.
struct ScaleBwd {
    const float *logits;  // [pts]
    const float *scale;   // [pts], or nullptr: no scale attention
    float *grad_scale;    // [pts]
};

template <int D, typename VT>
__global__ void __launch_bounds__(kThreads)
bwd_dots_kernel(const VT *__restrict__ value, const int64_t *__restrict__ shapes,
                const int64_t *__restrict__ starts, const float *__restrict__ loc,
                const float *__restrict__ attn, const float *__restrict__ grad_out,
                float *__restrict__ grad_loc, float *__restrict__ grad_attn,
                float *__restrict__ ref_part, ScaleBwd sb, float4 *__restrict__ clear,
                uint32_t clear_n4, Dims dm) {
    constexpr int G = D / 4;
    constexpr int IPB = kThreads / G;
    __shared__ LevelLds s_lv;
    extern __shared__ __align__(16) unsigned char smem[];
    uint4 *s_off = reinterpret_cast<uint4 *>(smem);  // row offsets, then the dots
    float4 *s_aux = reinterpret_cast<float4 *>(s_off + IPB * dm.PS);

    // on one stream, the bin counters of the grad_value pipeline that follows
    // (clear_n4 float4s, none otherwise)
    for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < clear_n4; i += gridDim.x * kThreads)
        clear[i] = make_float4(0.f, 0.f, 0.f, 0.f);

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
    // blocks of IPB queries of one (batch, head), dm.nblk per (batch, head),
    // in launch order as in the forward; workgroup g takes blocks g, g + grid, ...
    const int total = dm.nblocks;
    for (int blk = blockIdx.x; blk < total; blk += gridDim.x) {
    if (blk != (int)blockIdx.x) __syncthreads();  // the point tables are reused
    const int wg = blk;
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
            // kDotsBatch points at a time: their 4 * kDotsBatch row loads are in
            // flight together (this kernel shares the CUs with the grad_value
            // kernels, so one point's four loads would leave the wave waiting
            // on each point's latency)
            int jj = 0;
            for (; jj + kDotsBatch <= pc; jj += kDotsBatch) {
                uint4 o[kDotsBatch];
                float4 v[kDotsBatch][4];
#pragma unroll
                for (int u = 0; u < kDotsBatch; ++u) o[u] = s_off[base + jj + u];
#pragma unroll
                for (int u = 0; u < kDotsBatch; ++u) {
                    v[u][0] = Row4<VT>::load(vr, o[u].x, 4 * c);
                    v[u][1] = Row4<VT>::load(vr, o[u].y, 4 * c);
                    v[u][2] = Row4<VT>::load(vr, o[u].z, 4 * c);
                    v[u][3] = Row4<VT>::load(vr, o[u].w, 4 * c);
                }
                uint4 d[kDotsBatch];
#pragma unroll
                for (int u = 0; u < kDotsBatch; ++u)
                    d[u] = make_uint4(__float_as_uint(group_sum<G>(dot4(g4, v[u][0]))),
                                      __float_as_uint(group_sum<G>(dot4(g4, v[u][1]))),
                                      __float_as_uint(group_sum<G>(dot4(g4, v[u][2]))),
                                      __float_as_uint(group_sum<G>(dot4(g4, v[u][3]))));
                // the group's lanes are one wave: every lane has read the
                // offsets before lane 0 overwrites them
                if (c == 0) {
#pragma unroll
                    for (int u = 0; u < kDotsBatch; ++u) s_off[base + jj + u] = d[u];
                }
            }
            for (; jj < pc; ++jj) {
                const uint4 o = s_off[base + jj];
                const float4 v0 = Row4<VT>::load(vr, o.x, 4 * c);
                const float4 v1 = Row4<VT>::load(vr, o.y, 4 * c);
                const float4 v2 = Row4<VT>::load(vr, o.z, 4 * c);
                const float4 v3 = Row4<VT>::load(vr, o.w, 4 * c);
                const float d0 = group_sum<G>(dot4(g4, v0));
                const float d1 = group_sum<G>(dot4(g4, v1));
                const float d2 = group_sum<G>(dot4(g4, v2));
                const float d3 = group_sum<G>(dot4(g4, v3));
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
            // replaces grad_A (with a scale attention, see ScaleBwd), and each
            // level's sum of location gradients is stored per item for the
            // reference-point gradient.
            if (dm.softmax_run) {
                const float A = ax.z;
                const float t = run_sum(A * ga, dm.softmax_run);
                if (sb.scale) {
                    const float P = run_softmax(sb.logits[p], dm.softmax_run);
                    sb.grad_scale[p] = P * ga;
                    ga = A * ga - P * t;
                } else {
                    ga = A * (ga - t);
                }
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
// backward of heads with few points, in one kernel
// Workgroup = (batch b, head m, range of kSmallPixels pixels).  Every point of
// the head (at most kSmallPoints) is tabled once (neighbours, weights); its
// neighbours inside the range are counting-sorted by pixel in LDS, and a lane
// owning (pixel, 4-channel quad) sums A * w * grad_out over its pixel's
// entries in registers and writes the pixel once -- the binned pipeline's
// gather form with one bin per range, no float atomics (which run at a few
// hundred G lane-ops/s on this chip, in LDS too).  The range's workgroup also
// computes grad_attn_weight and grad_sampling_loc for every nsplit-th point,
// as the dots kernel does.  For DAT's sampling step and other small problems
// the binned pipeline's seven launches would cost more than the work.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *s_w,
                                                         uint32_t &total) {
    constexpr int kWaves = kThreads / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t inc = wave_inclusive_scan(v);
    if (lane == 63) s_w[wave] = inc;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const uint32_t x = s_w[w];
        base += w < wave ? x : 0u;
        tot += x;
    }
    total = tot;
    __syncthreads();  // s_w is free again
    return base + inc - v;
}

template <int D, typename VT>
__global__ void __launch_bounds__(kThreads)
bwd_small_kernel(const VT *__restrict__ value, const int64_t *__restrict__ shapes,
                 const int64_t *__restrict__ starts, const float *__restrict__ loc,
                 const float *__restrict__ attn, const float *__restrict__ grad_out,
                 float *__restrict__ grad_value, float *__restrict__ grad_loc,
                 float *__restrict__ grad_attn, Dims dm) {
    constexpr int G = D / 4;
    constexpr int NG = kThreads / G;      // lane groups
    constexpr int CPT = kSmallPixels / kThreads;  // pixel counts per thread in the scan
    __shared__ LevelLds s_lv;
    __shared__ float2 s_scale[kMaxLevels];
    __shared__ uint4 s_off[kSmallPoints];      // neighbour row offsets
    __shared__ float4 s_aux[kSmallPoints];     // fx, fy, A, valid bits
    __shared__ uint32_t s_cnt[kSmallPixels + 1];  // entries per pixel, then first entry
    __shared__ uint32_t s_ent[4 * kSmallPoints];  // point << 2 | neighbour, by pixel
    __shared__ uint32_t s_w[kThreads / 64];

    const int M = dm.M, LK = dm.L * dm.K, Nq = dm.Nq, Nv = dm.Nv;
    const int nsplit = dm.nblk;  // pixel ranges per (batch, head)
    const int bm = (int)blockIdx.x / nsplit + dm.b0 * M, sp = (int)blockIdx.x % nsplit;
    const int m = bm % M, b = bm / M;
    const int px0 = sp * kSmallPixels, npx = min(kSmallPixels, Nv - px0);
    const int npts = Nq * LK;
    const uint32_t row_stride = (uint32_t)M * D * 4u;
    const uint32_t head_off = (uint32_t)m * D * 4u;
    stage_levels(&s_lv, shapes, starts, dm.L, Nv, 0x7fffffff);
    if (threadIdx.x < dm.L) {
        const int4 lvl = s_lv.lvl[threadIdx.x];
        s_scale[threadIdx.x] =
            make_float2(pixel_scale(lvl.y, dm.align), pixel_scale(lvl.x, dm.align));
    }
    for (int i = threadIdx.x; i <= kSmallPixels; i += kThreads) s_cnt[i] = 0u;
    __syncthreads();

    // 1. the point table, and slots for the neighbours inside the range
    const size_t row0 = (size_t)b * Nq * M + m;  // item row of query 0
    int pix[4] = {-1, -1, -1, -1};
    uint32_t slot[4] = {0u, 0u, 0u, 0u};
    if ((int)threadIdx.x < npts) {
        const int qq = threadIdx.x / LK, j = threadIdx.x - qq * LK;
        const size_t p = (row0 + (size_t)qq * M) * LK + j;
        const float2 uv = reinterpret_cast<const float2 *>(loc)[p];
        const float A = attn[p];
        const int4 lvl = s_lv.lvl[j / dm.K];
        const Neighbours n = neighbours(uv.x, uv.y, lvl, row_stride, head_off, dm.align);
        s_off[threadIdx.x] = n.off;
        s_aux[threadIdx.x] = make_float4(n.fx, n.fy, A, __uint_as_float(n.valid));
        const int pTL = lvl.z + n.yi * lvl.y + n.xi;
        const int nb[4] = {pTL, pTL + 1, pTL + lvl.y, pTL + lvl.y + 1};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = nb[k] - px0;
            if ((n.valid & (1u << k)) && r >= 0 && r < npx) {
                pix[k] = r;
                slot[k] = atomicAdd(&s_cnt[r], 1u);
            }
        }
    }
    __syncthreads();
    // 2. first entry of each pixel (exclusive scan of the counts)
    {
        uint32_t c[CPT], sum = 0;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            c[i] = s_cnt[threadIdx.x * CPT + i];
            sum += c[i];
        }
        uint32_t total;
        uint32_t e = block_exclusive_scan(sum, s_w, total);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            s_cnt[threadIdx.x * CPT + i] = e;
            e += c[i];
        }
        if (threadIdx.x == 0) s_cnt[kSmallPixels] = total;
    }
    __syncthreads();
    if ((int)threadIdx.x < npts) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (pix[k] >= 0) s_ent[s_cnt[pix[k]] + slot[k]] = (threadIdx.x << 2) | (uint32_t)k;
    }
    __syncthreads();

    // 3. grad_attn_weight and grad_sampling_loc of every nsplit-th point
    const size_t slice = (size_t)Nv * M * D;
    const rsrc_t vr = make_rsrc(value + (size_t)b * slice, (uint32_t)(slice * sizeof(VT)));
    // the grad_out rows of the head, read through a buffer (see the dots kernel)
    const rsrc_t go =
        make_rsrc(grad_out + row0 * D, (uint32_t)(((size_t)(Nq - 1) * M + 1) * D * 4));
    auto g_row = [&](int qq, int c) {
        auto u = __builtin_amdgcn_raw_buffer_load_b128(
            go, (int)((uint32_t)qq * M * D * 4u + 16u * c), 0, 0);
        return make_float4(__uint_as_float(u[0]), __uint_as_float(u[1]), __uint_as_float(u[2]),
                           __uint_as_float(u[3]));
    };
    {
        const int grp = threadIdx.x / G, c = threadIdx.x % G;
        for (int pt = sp + grp * nsplit; pt < npts; pt += NG * nsplit) {
            const int qq = pt / LK, j = pt - qq * LK;
            const float4 g4 = g_row(qq, c);
            const uint4 o = s_off[pt];
            const float4 v0 = Row4<VT>::load(vr, o.x, 4 * c);
            const float4 v1 = Row4<VT>::load(vr, o.y, 4 * c);
            const float4 v2 = Row4<VT>::load(vr, o.z, 4 * c);
            const float4 v3 = Row4<VT>::load(vr, o.w, 4 * c);
            const float d0 = group_sum<G>(dot4(g4, v0));
            const float d1 = group_sum<G>(dot4(g4, v1));
            const float d2 = group_sum<G>(dot4(g4, v2));
            const float d3 = group_sum<G>(dot4(g4, v3));
            if (c == 0) {
                const float4 ax = s_aux[pt];
                const uint32_t valid = __float_as_uint(ax.w);
                const float fx = ax.x, fy = ax.y, A = ax.z;
                float ga = 0.f, gx = 0.f, gy = 0.f;
                if (valid != 0u) {
                    const float4 w = tent_weights(fx, fy, valid);
                    ga = w.x * d0 + w.y * d1 + w.z * d2 + w.w * d3;
                    const float2 sc = s_scale[j / dm.K];
                    gx = A * sc.x * ((1.f - fy) * (d1 - d0) + fy * (d3 - d2));
                    gy = A * sc.y * ((1.f - fx) * (d2 - d0) + fx * (d3 - d1));
                }
                const size_t p = (row0 + (size_t)qq * M) * LK + j;
                grad_attn[p] = ga;
                reinterpret_cast<float2 *>(grad_loc)[p] = make_float2(gx, gy);
            }
        }
    }

    // 4. grad_value of the range: lane = (pixel, quad), its entries summed
    float *gvb = grad_value + (size_t)b * slice + (size_t)m * D;
    for (int i = threadIdx.x; i < npx * G; i += kThreads) {
        const int px = i / G, c = i - px * G;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        const uint32_t e1 = s_cnt[px + 1];
        for (uint32_t e = s_cnt[px]; e < e1; ++e) {
            const uint32_t ent = s_ent[e];
            const int pt = (int)(ent >> 2), k = (int)(ent & 3u);
            const float4 ax = s_aux[pt];
            const float gx = 1.f - ax.x, gy = 1.f - ax.y;
            const float wk = (k & 1 ? ax.x : gx) * (k & 2 ? ax.y : gy);
            fma4(acc, ax.z * wk, g_row(pt / LK, c));
        }
        float4 *d4 = reinterpret_cast<float4 *>(gvb + (size_t)(px0 + px) * M * D) + c;
        if (dm.accumulate) {
            const float4 v = *d4;
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        *d4 = acc;
    }
}

// ---------------------------------------------------------------------------
// fused prologue, backward side
// fused_prologue_kernel: the locations and weights of every point, written
//    to the workspace for the backward pipeline (the same arithmetic as the
//    fused forward).  Workgroup = kProItems consecutive items (b, q, m).
// fused_epilogue_kernel: grad_logits = A * (grad_A - sum over the softmax
//    group of A * grad_A), in place over grad_A (with a scale attention, see
//    ScaleBwd: A g - P sum(A g), and grad_scale = P g); and, when asked for,
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
            stage_softmax_stats(s_st, pr, pt0, (size_t)LK, nitems, L, K);
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
            float A;
            if (pr.shfl) {
                A = run_softmax(z, pr.per_level ? K : LK);
            } else {
                const float2 st = s_st[i1 * ng + (pr.per_level ? l : 0)];
                A = expf(z - st.x) * st.y;
            }
            attn[p] = pr.scale ? A * pr.scale[p] : A;
        }
    }
}

__global__ void __launch_bounds__(kThreads)
fused_epilogue_kernel(const int64_t *__restrict__ shapes, const int64_t *__restrict__ starts,
                      const float *__restrict__ attn, float *__restrict__ grad_logits,
                      const float *__restrict__ grad_off, const float *__restrict__ ref_part,
                      float *__restrict__ grad_ref, int per_level, int shfl, int64_t groups,
                      int64_t refs, ScaleBwd sb, Dims dm) {
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
            if (sb.scale) {
                const float P = run_softmax(sb.logits[p], gs);
                sb.grad_scale[p] = P * ga;
                grad_logits[p] = a * ga - P * s;
            } else {
                grad_logits[p] = a * (ga - s);
            }
        }
    } else {
        for (int64_t u = t0; u < groups; u += stride) {
            const size_t p0 = (size_t)u * gs;  // the groups tile the points in order
            float s = 0.f;
            for (int j = 0; j < gs; ++j) s = __builtin_fmaf(attn[p0 + j], grad_logits[p0 + j], s);
            if (sb.scale) {
                const float2 st = softmax_stats(sb.logits + p0, gs);
                for (int j = 0; j < gs; ++j) {
                    const float P = expf(sb.logits[p0 + j] - st.x) * st.y;
                    const float ga = grad_logits[p0 + j];
                    sb.grad_scale[p0 + j] = P * ga;
                    grad_logits[p0 + j] = attn[p0 + j] * ga - P * s;
                }
            } else {
                for (int j = 0; j < gs; ++j)
                    grad_logits[p0 + j] = attn[p0 + j] * (grad_logits[p0 + j] - s);
            }
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
using msda_host::check_sizes;
using msda_host::fused_layout;
using msda_host::FusedLayout;

struct Launch {
    int ipb, pc, ps;
    size_t lds;
};

// `reserve`: LDS bytes taken from the point-table budget for other uses.
Launch plan(int64_t D, int64_t L, int64_t K, int bytes_per_point, int reserve = 0,
            int budget = kSetupLdsBytes, int split = 1) {
    Launch p;
    p.ipb = (int)(kThreads / (D / 4 * split));
    const int lk = (int)(L * K);
    int pc = (budget - reserve) / (p.ipb * bytes_per_point) - 2;
    pc = pc < 1 ? 1 : pc;
    p.pc = pc < lk ? pc : lk;
    p.ps = p.pc + ((p.pc % 2 == 0) ? 1 : 2);
    p.lds = (size_t)p.ipb * p.ps * bytes_per_point;
    return p;
}

Launch fwd_plan(int64_t D, int64_t L, int64_t K, int reserve = 0, int split = 1) {
    Launch p = plan(D, L, K, 32, reserve, kSetupLdsBytes, split);
    if (L * K > 16) {
        const Launch half = plan(D, L, K, 32, reserve, kFwdLdsBytes, split);
        if (half.pc >= 16) p = half;
    }
    return p;
}

// A softmax group that lane shuffles can reduce: a power of two <= 64.
bool pow2_run(int64_t n) { return n >= 1 && n <= 64 && (n & (n - 1)) == 0; }


// pr == nullptr: locations and weights from loc / attn; otherwise from the
// prologue inputs (loc and attn unused).
template <int D, typename VT>
msda_status launch_fwd(const void *value, const int64_t *shapes, const int64_t *starts,
                       const float *loc, const float *attn, const Prologue *pr, float *out,
                       int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t L, int64_t K,
                       bool align, hipStream_t s) {
    // one lane group per item, or fwd_split of them when one per item would
    // leave fewer than two workgroups per CU
    constexpr int kSplit = fwd_split<D>();
    const int64_t ipb1 = kThreads / (D / 4);
    const int split = (kSplit > 1 && B * M * ((Nq + ipb1 - 1) / ipb1) < 512) ? kSplit : 1;
    const int ipb = (int)(ipb1 / split);
    Prologue prv = pr ? *pr : Prologue{nullptr, nullptr, nullptr, nullptr, 0, 0, nullptr, nullptr};
    int st_bytes = 0;
    Launch p = fwd_plan(D, L, K, 0, split);
    if (pr) {
        // softmax by lane shuffles when the items' points come in one chunk and
        // the groups are power-of-two runs of at most 64; else statistics in LDS
        prv.shfl = (p.pc == L * K && pow2_run(pr->per_level ? K : L * K)) ? 1 : 0;
        if (!prv.shfl) {
            st_bytes = ipb * (pr->per_level ? (int)L : 1) * (int)sizeof(float2);
            p = fwd_plan(D, L, K, st_bytes, split);
        }
    }
    const size_t lds = p.lds + (size_t)st_bytes;
    const int64_t gx = (Nq + p.ipb - 1) / p.ipb;  // query blocks per (batch, head)
    const int64_t bchunk = batch_chunk(gx * M, B);
    for (int64_t b0 = 0; b0 < B; b0 += bchunk) {
        const int64_t nb = (B - b0) < bchunk ? (B - b0) : bchunk;
        Dims dm{(int)Nv, (int)Nq, (int)M, (int)L, (int)K, p.pc, p.ps, (int)b0, (int)gx, 0, 0};
        dm.align = align ? 1 : 0;
        const dim3 grid((unsigned)(gx * M * nb));
        const VT *vp = static_cast<const VT *>(value);
        if (pr && split > 1)
            hipLaunchKernelGGL((msda_fwd_kernel<D, VT, true, kSplit>), grid, dim3(kThreads), lds,
                               s, vp, shapes, starts, loc, attn, prv, out, dm);
        else if (pr)
            hipLaunchKernelGGL((msda_fwd_kernel<D, VT, true, 1>), grid, dim3(kThreads), lds, s,
                               vp, shapes, starts, loc, attn, prv, out, dm);
        else if (split > 1)
            hipLaunchKernelGGL((msda_fwd_kernel<D, VT, false, kSplit>), grid, dim3(kThreads),
                               lds, s, vp, shapes, starts, loc, attn, prv, out, dm);
        else
            hipLaunchKernelGGL((msda_fwd_kernel<D, VT, false, 1>), grid, dim3(kThreads), lds, s,
                               vp, shapes, starts, loc, attn, prv, out, dm);
        msda_status st = hip_status(hipGetLastError());
        if (st != MSDA_OK) return st;
    }
    return MSDA_OK;
}


// The fused prologue's backward, as far as the dots kernel takes it: it
// writes offset gradients (location gradients / (W, H)) always; with in_dots
// also the logit gradients (softmax runs of softmax_run points) and, given
// ref_part, the per-(item, level) location-gradient sums [B][Nq][M][L][2].
struct FusedBwd {
    int softmax_run;  // requested run length (0: the runs do not fit lane shuffles)
    float *ref_part;  // nullptr: no reference-point gradient wanted
    bool in_dots;     // set by the launch: the dots kernel did both
    ScaleBwd scale;   // the scale attention (scale.scale == nullptr: none)
};


template <int D, typename VT>
msda_status launch_bwd(const void *value, const int64_t *shapes, const int64_t *starts,
                       const float *loc, const float *attn, const float *gout, float *gval,
                       float *gloc, float *gattn, int64_t B, int64_t Nv, int64_t Nq, int64_t M,
                       int64_t L, int64_t K, const PassPlan &pp, unsigned char *ws,
                       bool accumulate, bool align, FusedBwd *fz, const Exec &ex) {
    // grad_attn_weight and grad_sampling_loc do not depend on the bin
    // pipeline: with a side stream they are computed there, concurrently
    const hipStream_t ds = ex.dots_stream();
    const Launch p = plan(D, L, K, 32);
    const int64_t gq = (Nq + p.ipb - 1) / p.ipb;
    // the dots kernel finishes the fused prologue's backward itself when its
    // point table holds whole items and the softmax runs fit a wave
    if (fz) fz->in_dots = fz->softmax_run > 0 && p.pc == L * K;
    float *ref_part = fz && fz->in_dots ? fz->ref_part : nullptr;
    const ScaleBwd sb = fz && fz->in_dots ? fz->scale : ScaleBwd{nullptr, nullptr, nullptr};
    // on one stream this kernel runs just before the grad_value pipeline and
    // also clears the bin counters of its first pass, which saves that pass a
    // launch (latency-bound small problems such as the decoder's gain ~5 us)
    const bool clear_here = ds == ex.s;
    float4 *clear = reinterpret_cast<float4 *>(ws + pp.wl.off_counts);
    const uint32_t clear_n4 = (uint32_t)((pp.wl.off_start - pp.wl.off_counts) / 16);
    ex.stamp(kStageDots, false, ds);
    msda_status st = per_batch(B, gq * M, [&](int64_t b0, unsigned grid) {
        Dims d2{(int)Nv, (int)Nq, (int)M, (int)L, (int)K, p.pc, p.ps, (int)b0, (int)gq, 0, 0};
        d2.nblocks = (int)grid;
        d2.align = align ? 1 : 0;
        d2.loc_div = fz ? 1 : 0;
        d2.softmax_run = fz && fz->in_dots ? fz->softmax_run : 0;
        // one workgroup per block of queries: beside the grad_value kernels the
        // backward takes the same time with a capped persistent grid (measured:
        // 512 workgroups), and this kernel finishes sooner uncapped
        const bool c = clear_here && b0 == 0;
        hipLaunchKernelGGL((bwd_dots_kernel<D, VT>), dim3(grid), dim3(kThreads), p.lds, ds,
                           static_cast<const VT *>(value), shapes, starts, loc, attn, gout, gloc,
                           gattn, ref_part, sb, c ? clear : nullptr, c ? clear_n4 : 0u, d2);
    });
    if (st != MSDA_OK) return st;
    ex.stamp(kStageDots, true, ds);
    return run_bins_passes<D, false>(shapes, starts, loc, attn, gout, gval, B, Nv, Nq, M, L, K,
                                     pp, ws, accumulate, align, ex, clear_here);
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

template <int D, typename VT>
msda_status launch_bwd_small(const void *value, const int64_t *shapes, const int64_t *starts,
                             const float *loc, const float *attn, const float *gout, float *gval,
                             float *gloc, float *gattn, int64_t B, int64_t Nv, int64_t Nq,
                             int64_t M, int64_t L, int64_t K, bool acc, bool align,
                             hipStream_t s) {
    const int64_t nsplit = (Nv + kSmallPixels - 1) / kSmallPixels;
    const int64_t bchunk = batch_chunk(M * nsplit, B);
    for (int64_t b0 = 0; b0 < B; b0 += bchunk) {
        const int64_t nb = (B - b0) < bchunk ? (B - b0) : bchunk;
        Dims dm{(int)Nv, (int)Nq, (int)M, (int)L, (int)K, 0, 0, (int)b0, (int)nsplit, 0,
                acc ? 1 : 0};
        dm.align = align ? 1 : 0;
        hipLaunchKernelGGL((bwd_small_kernel<D, VT>), dim3((unsigned)(nb * M * nsplit)),
                           dim3(kThreads), 0, s, static_cast<const VT *>(value), shapes, starts,
                           loc, attn, gout, gval, gloc, gattn, dm);
        const msda_status st = hip_status(hipGetLastError());
        if (st != MSDA_OK) return st;
    }
    return MSDA_OK;
}

template <typename VT>
msda_status dispatch_small(int64_t D, const void *value, const int64_t *shapes,
                           const int64_t *starts, const float *loc, const float *attn,
                           const float *gout, float *gval, float *gloc, float *gattn, int64_t B,
                           int64_t Nv, int64_t Nq, int64_t M, int64_t L, int64_t K, bool acc,
                           bool align, hipStream_t s) {
#define MSDA_SMALL_CASE(DD)                                                                   \
    case DD:                                                                                  \
        return launch_bwd_small<DD, VT>(value, shapes, starts, loc, attn, gout, gval, gloc,   \
                                        gattn, B, Nv, Nq, M, L, K, acc, align, s);
    switch (D) {
        MSDA_SMALL_CASE(4)
        MSDA_SMALL_CASE(8)
        MSDA_SMALL_CASE(16)
        MSDA_SMALL_CASE(32)
        MSDA_SMALL_CASE(64)
        MSDA_SMALL_CASE(128)
        MSDA_SMALL_CASE(256)
    default: return MSDA_ERR_UNSUPPORTED;
    }
#undef MSDA_SMALL_CASE
}

template <typename VT>
msda_status dispatch_bwd(int64_t D, const void *value, const int64_t *shapes,
                         const int64_t *starts, const float *loc, const float *attn,
                         const float *gout, float *gval, float *gloc, float *gattn, int64_t B,
                         int64_t Nv, int64_t Nq, int64_t M, int64_t L, int64_t K,
                         const PassPlan &pp, unsigned char *ws, bool acc, bool align,
                         FusedBwd *fz, const Exec &ex) {
#define MSDA_BWD_CASE(DD)                                                                      \
    case DD:                                                                                   \
        return launch_bwd<DD, VT>(value, shapes, starts, loc, attn, gout, gval, gloc, gattn, B, \
                                  Nv, Nq, M, L, K, pp, ws, acc, align, fz, ex);
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
                               const float *attn_logits, const float *attn_scale, float *out,
                               float *sampling_loc_out,
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
    const Prologue pr{reference_points, sampling_offsets, attn_logits, attn_scale,
                      (flags & MSDA_SOFTMAX_PER_LEVEL) ? 1 : 0, 0, sampling_loc_out,
                      attn_weight_out};
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (value_dtype == MSDA_F32)
        return dispatch_fwd<float>(D, value, spatial_shapes, level_start_index, nullptr, nullptr,
                                   &pr, out, B, Nv, Nq, M, L, K, align, s);
    return dispatch_fwd<uint16_t>(D, value, spatial_shapes, level_start_index, nullptr, nullptr,
                                  &pr, out, B, Nv, Nq, M, L, K, align, s);
}


}  // extern "C"

namespace {

msda_status backward_impl(const void *value, int value_dtype, const int64_t *spatial_shapes,
                          const int64_t *level_start_index, const float *sampling_loc,
                          const float *attn_weight, const float *grad_out, float *grad_value,
                          float *grad_sampling_loc, float *grad_attn_weight, int64_t B,
                          int64_t Nv, int64_t Nq, int64_t M, int64_t D, int64_t L, int64_t K,
                          void *workspace, size_t workspace_bytes, uint32_t flags,
                          FusedBwd *fz, hipStream_t s, void *side_stream,
                          void *const *side_events, hipEvent_t *ev) {
    msda_status st = check_sizes(value_dtype, B, Nv, Nq, M, D, L, K);
    if (st != MSDA_OK) return st;
    if (flags & ~(MSDA_BWD_ACCUMULATE | MSDA_ALIGN_CORNERS | MSDA_BWD_BINNED))
        return MSDA_ERR_UNSUPPORTED;
    // a grad_value record stores the query index in 25 bits
    if (Nq > ((int64_t)1 << (32 - kRecQueryShift))) return MSDA_ERR_UNSUPPORTED;
    const int64_t nval = B * Nv * M * D;
    if (nval > 0 && !grad_value) return MSDA_ERR_NULL;
    const bool work = B > 0 && Nq > 0;
    Exec ex{s, nullptr, nullptr, nullptr, ev};
    st = exec_side(ex, side_stream, side_events);
    if (st != MSDA_OK) return st;
    PassPlan pp{};
    if (work) {
        if (Nv < 1) return MSDA_ERR_SHAPE;
        if (!value || !spatial_shapes || !level_start_index || !sampling_loc || !attn_weight ||
            !grad_out || !grad_sampling_loc || !grad_attn_weight)
            return MSDA_ERR_NULL;
        if (!workspace) return MSDA_ERR_NULL;
        // the grad_value pipeline in as few passes as the workspace allows
        pp = pass_plan(B, Nv, Nq, M, L, K, false, workspace_bytes);
        if (pp.nb == 0) return MSDA_ERR_WORKSPACE;
        // bin counters and work items are indexed with 31-bit integers
        if (pp.wl.bm_bins >= ((int64_t)1 << 31) || pp.wl.work_max >= ((int64_t)1 << 31))
            return MSDA_ERR_UNSUPPORTED;
        if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return MSDA_ERR_WORKSPACE;
    }
    const bool acc = (flags & MSDA_BWD_ACCUMULATE) != 0;
    const bool align = (flags & MSDA_ALIGN_CORNERS) != 0;
    if (!work) {
        // no point: the gradient of value is zero
        for (int i = 0; i < MSDA_BWD_STAGES; ++i) {
            ex.stamp(i, false, s);
            ex.stamp(i, true, s);
        }
        return acc ? MSDA_OK : fill_zero(grad_value, (size_t)nval / 4, s);  // D % 4 == 0
    }
    // heads of few points: the whole backward in one kernel on the caller's
    // stream, recorded as the first stage (the other stages are empty)
    if (!fz && !(flags & MSDA_BWD_BINNED) && Nq * L * K <= kSmallPoints) {
        ex.stamp(kStageDots, false, s);
        st = value_dtype == MSDA_F32
                 ? dispatch_small<float>(D, value, spatial_shapes, level_start_index,
                                         sampling_loc, attn_weight, grad_out, grad_value,
                                         grad_sampling_loc, grad_attn_weight, B, Nv, Nq, M, L, K,
                                         acc, align, s)
                 : dispatch_small<uint16_t>(D, value, spatial_shapes, level_start_index,
                                            sampling_loc, attn_weight, grad_out, grad_value,
                                            grad_sampling_loc, grad_attn_weight, B, Nv, Nq, M, L,
                                            K, acc, align, s);
        ex.stamp(kStageDots, true, s);
        for (int i = kStageDots + 1; i < MSDA_BWD_STAGES; ++i) {
            ex.stamp(i, false, s);
            ex.stamp(i, true, s);
        }
        return st;
    }
    st = exec_fork(ex, B * Nq * M * L * K);
    if (st != MSDA_OK) return st;
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    if (value_dtype == MSDA_F32)
        st = dispatch_bwd<float>(D, value, spatial_shapes, level_start_index, sampling_loc,
                                 attn_weight, grad_out, grad_value, grad_sampling_loc,
                                 grad_attn_weight, B, Nv, Nq, M, L, K, pp, ws, acc, align, fz,
                                 ex);
    else
        st = dispatch_bwd<uint16_t>(D, value, spatial_shapes, level_start_index, sampling_loc,
                                    attn_weight, grad_out, grad_value, grad_sampling_loc,
                                    grad_attn_weight, B, Nv, Nq, M, L, K, pp, ws, acc, align, fz,
                                    ex);
    const msda_status js = exec_join(ex);
    return st != MSDA_OK ? st : js;
}

msda_status backward_fused_impl(const void *value, int value_dtype, const int64_t *shapes,
                                const int64_t *starts, const float *ref, const float *off,
                                const float *logits, const float *scale, const float *saved_loc,
                                const float *saved_attn, const float *grad_out, float *grad_value,
                                float *grad_off, float *grad_logits, float *grad_scale,
                                float *grad_ref, int64_t B,
                                int64_t Nv, int64_t Nq, int64_t M, int64_t D, int64_t L,
                                int64_t K, void *workspace, size_t workspace_bytes,
                                uint32_t flags, hipStream_t s, void *side_stream,
                                void *const *side_events, hipEvent_t *ev) {
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
        FusedBwd none{0, nullptr, false, ScaleBwd{nullptr, nullptr, nullptr}};
        st = backward_impl(value, value_dtype, shapes, starts, nullptr, nullptr, grad_out,
                           grad_value, nullptr, nullptr, B, Nv, Nq, M, D, L, K, workspace,
                           workspace_bytes, core_flags, &none, s, side_stream, side_events, ev);
        stamp(MSDA_BWD_STAGES + 1, false);
        stamp(MSDA_BWD_STAGES + 1, true);
        return st;
    }
    if (Nv < 1) return MSDA_ERR_SHAPE;
    if (!value || !shapes || !starts || !ref || !off || !logits || !grad_out || !grad_value ||
        !grad_off || !grad_logits)
        return MSDA_ERR_NULL;
    if ((saved_loc == nullptr) != (saved_attn == nullptr)) return MSDA_ERR_NULL;
    if ((scale == nullptr) != (grad_scale == nullptr)) return MSDA_ERR_NULL;
    if (!workspace) return MSDA_ERR_NULL;
    const FusedLayout fl = fused_layout(B, Nv, Nq, M, L, K);
    if (workspace_bytes < fl.off_core + fl.core_min) return MSDA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return MSDA_ERR_WORKSPACE;
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    const bool saved = saved_loc != nullptr;
    float *loc = reinterpret_cast<float *>(ws + fl.off_loc);
    float *attn = reinterpret_cast<float *>(ws + fl.off_attn);
    const int shfl = pow2_run(per_level ? K : L * K) ? 1 : 0;
    const Prologue pr{ref, off, logits, scale, per_level ? 1 : 0, shfl, nullptr, nullptr};
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
                grad_ref ? reinterpret_cast<float *>(ws + fl.off_part) : nullptr, false,
                ScaleBwd{logits, scale, grad_scale}};
    const float *use_loc = saved ? saved_loc : loc, *use_attn = saved ? saved_attn : attn;
    st = backward_impl(value, value_dtype, shapes, starts, use_loc, use_attn, grad_out,
                       grad_value, grad_off, grad_logits, B, Nv, Nq, M, D, L, K,
                       ws + fl.off_core, workspace_bytes - fl.off_core,
                       core_flags, &fz, s, side_stream, side_events, ev);
    if (st != MSDA_OK) return st;

    stamp(MSDA_BWD_STAGES + 1, false);
    if (fz.in_dots) {
        if (grad_ref) {
            const int64_t refs = B * Nq * L;
            int64_t blocks = (refs + kThreads - 1) / kThreads;
            blocks = blocks < (1 << 16) ? blocks : (1 << 16);
            hipLaunchKernelGGL(fused_epilogue_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                               s, shapes, starts, use_attn, grad_logits, grad_off, fz.ref_part,
                               grad_ref, per_level ? 1 : 0, shfl, (int64_t)0, refs,
                               ScaleBwd{nullptr, nullptr, nullptr}, dm);
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
                           per_level ? 1 : 0, shfl, groups, refs, fz.scale, dm);
        st = hip_status(hipGetLastError());
    }
    stamp(MSDA_BWD_STAGES + 1, true);
    return st;
}

}  // namespace

// ---------------------------------------------------------------------------
// msda_backward_noalloc: msda_backward with its workspace in a static device
// array instead of a caller buffer, for callers that cannot allocate.  Each
// GPU holds its own copy of the array; its address is looked up once per
// device, with that device current, and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[MSDA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The current device's copy of `scratch`.  In host code the array's name is
// only a stand-in for the symbol: kernels and copies get this address.
msda_status scratch_of_current_device(void **ptr) {
    int dev = -1;
    msda_status st = hip_status(hipGetDevice(&dev));
    if (st != MSDA_OK) return st;
    if (dev < 0 || dev >= kMaxDevices) return MSDA_ERR_UNSUPPORTED;
    std::call_once(g_scratch_once[dev], [dev] {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_err[dev] = e;
        g_scratch_ptr[dev] = e == hipSuccess ? p : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess) return hip_status(g_scratch_err[dev]);
    *ptr = g_scratch_ptr[dev];
    return MSDA_OK;
}

}  // namespace

extern "C" {

msda_status msda_backward(const void *value, int value_dtype, const int64_t *spatial_shapes,
                          const int64_t *level_start_index, const float *sampling_loc,
                          const float *attn_weight, const float *grad_out, float *grad_value,
                          float *grad_sampling_loc, float *grad_attn_weight, int64_t B,
                          int64_t Nv, int64_t Nq, int64_t M, int64_t D, int64_t L, int64_t K,
                          void *workspace, size_t workspace_bytes, uint32_t flags,
                          void *stream, void *side_stream, void *const *side_events) {
    return backward_impl(value, value_dtype, spatial_shapes, level_start_index, sampling_loc,
                         attn_weight, grad_out, grad_value, grad_sampling_loc, grad_attn_weight,
                         B, Nv, Nq, M, D, L, K, workspace, workspace_bytes, flags, nullptr,
                         static_cast<hipStream_t>(stream), side_stream, side_events, nullptr);
}

msda_status msda_backward_events(const void *value, int value_dtype,
                                 const int64_t *spatial_shapes, const int64_t *level_start_index,
                                 const float *sampling_loc, const float *attn_weight,
                                 const float *grad_out, float *grad_value,
                                 float *grad_sampling_loc, float *grad_attn_weight, int64_t B,
                                 int64_t Nv, int64_t Nq, int64_t M, int64_t D, int64_t L,
                                 int64_t K, void *workspace, size_t workspace_bytes,
                                 uint32_t flags, void *stream, void *side_stream,
                                 void *const *side_events, void *const *events) {
    if (!events) return MSDA_ERR_NULL;
    hipEvent_t ev[2 * MSDA_BWD_STAGES];
    for (int i = 0; i < 2 * MSDA_BWD_STAGES; ++i) ev[i] = static_cast<hipEvent_t>(events[i]);
    return backward_impl(value, value_dtype, spatial_shapes, level_start_index, sampling_loc,
                         attn_weight, grad_out, grad_value, grad_sampling_loc, grad_attn_weight,
                         B, Nv, Nq, M, D, L, K, workspace, workspace_bytes, flags, nullptr,
                         static_cast<hipStream_t>(stream), side_stream, side_events, ev);
}


msda_status msda_backward_fused(const void *value, int value_dtype,
                                const int64_t *spatial_shapes, const int64_t *level_start_index,
                                const float *reference_points, const float *sampling_offsets,
                                const float *attn_logits, const float *attn_scale,
                                const float *sampling_loc, const float *attn_weight,
                                const float *grad_out, float *grad_value,
                                float *grad_sampling_offsets, float *grad_attn_logits,
                                float *grad_attn_scale, float *grad_reference_points, int64_t B,
                                int64_t Nv, int64_t Nq, int64_t M, int64_t D, int64_t L,
                                int64_t K, void *workspace, size_t workspace_bytes,
                                uint32_t flags, void *stream, void *side_stream,
                                void *const *side_events, void *const *events) {
    hipEvent_t ev[2 * MSDA_BWD_FUSED_STAGES];
    if (events)
        for (int i = 0; i < 2 * MSDA_BWD_FUSED_STAGES; ++i)
            ev[i] = static_cast<hipEvent_t>(events[i]);
    return backward_fused_impl(value, value_dtype, spatial_shapes, level_start_index,
                               reference_points, sampling_offsets, attn_logits, attn_scale,
                               sampling_loc, attn_weight, grad_out, grad_value,
                               grad_sampling_offsets, grad_attn_logits, grad_attn_scale,
                               grad_reference_points, B, Nv, Nq, M, D, L, K, workspace,
                               workspace_bytes, flags, static_cast<hipStream_t>(stream),
                               side_stream, side_events, events ? ev : nullptr);
}

msda_status msda_backward_noalloc(const void *value, int value_dtype,
                                  const int64_t *spatial_shapes, const int64_t *level_start_index,
                                  const float *sampling_loc, const float *attn_weight,
                                  const float *grad_out, float *grad_value,
                                  float *grad_sampling_loc, float *grad_attn_weight, int64_t B,
                                  int64_t Nv, int64_t Nq, int64_t M, int64_t D, int64_t L,
                                  int64_t K, uint32_t flags, void *stream, void *side_stream,
                                  void *const *side_events) {
    msda_status st = check_sizes(value_dtype, B, Nv, Nq, M, D, L, K);
    if (st != MSDA_OK) return st;
    const bool work = B > 0 && Nq > 0;
    const size_t need = work ? min_workspace(Nv, Nq, L, K, false) : 0;
    if (need > MSDA_NOALLOC_SCRATCH_BYTES) return MSDA_ERR_SCRATCH;
    // the pointer checks of msda_backward, before the one-time symbol lookup
    if (B * Nv * M * D > 0 && !grad_value) return MSDA_ERR_NULL;
    if (work && (!value || !spatial_shapes || !level_start_index || !sampling_loc ||
                 !attn_weight || !grad_out || !grad_sampling_loc || !grad_attn_weight))
        return MSDA_ERR_NULL;
    void *ws = nullptr;
    if (work) {
        st = scratch_of_current_device(&ws);
        if (st != MSDA_OK) return st;
    }
    return backward_impl(value, value_dtype, spatial_shapes, level_start_index, sampling_loc,
                         attn_weight, grad_out, grad_value, grad_sampling_loc, grad_attn_weight,
                         B, Nv, Nq, M, D, L, K, ws, work ? (size_t)MSDA_NOALLOC_SCRATCH_BYTES : 0,
                         flags, nullptr, static_cast<hipStream_t>(stream), side_stream,
                         side_events, nullptr);
}

int msda_last_hip_error(void) { return msda_internal_last_hip_error; }

}  // extern "C"
