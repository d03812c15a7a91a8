// bins.h -- the binned, atomic-free grad_value pipeline of the backward
// (count -> scan -> scatter -> tile kernels) and the point geometry it shares
// with the sampling kernels: level tables in LDS, the bilinear neighbours of
// a point, the tiles they touch.  Included by the translation units of
// libmsda.so; everything has internal linkage.
#ifndef MSDA_CSRC_BINS_H
#define MSDA_CSRC_BINS_H

#include <type_traits>

#include "common.h"

namespace {

constexpr int kTileShift = 3;              // grad_value tiles of 8x8 pixels
constexpr int kTile = 1 << kTileShift;
constexpr int kTilePx = kTile * kTile;
using msda_host::kChunk;                   // records per grad_value work item, at most
constexpr int kHistLds = 4096;             // bins of one (batch, head) kept in an LDS histogram
constexpr int kScanThreads = 512;           // placed sooner beside the dots kernel than 1024
constexpr int kScanBlock = 8 * kScanThreads;  // bins scanned by one workgroup
constexpr int kTileGrid = 16384;           // workgroups of the tile kernel, at most

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
// For volumes (the 3-D variant) a level is zp[l] planes of H x W voxels, the
// plane z starting at row start + z*H*W, and its bins are the tiles of its
// planes, plane-major (tpp[l] tiles per plane).
struct LevelLds {
    int4 lvl[kMaxLevels];
    int tw[kMaxLevels];   // tiles along W
    int zp[kMaxLevels];   // planes (volumes only)
    int tpp[kMaxLevels];  // tiles per plane (volumes only)
    int nbins;            // bins of one (batch, head)
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

// The same for a volume level table [L, 3] with rows (Z, H, W).
__device__ __forceinline__ void stage_volume_levels(LevelLds *s, const int64_t *shapes,
                                                    const int64_t *starts, int L, int Nv,
                                                    int nb_max) {
    const int t = threadIdx.x;
    if (t < L) {
        const int64_t Z = shapes[3 * t], H = shapes[3 * t + 1], W = shapes[3 * t + 2];
        const int64_t S = starts[t];
        const bool dims_ok = Z >= 1 && H >= 1 && W >= 1 && Z <= Nv && H <= Nv && W <= Nv;
        const bool ok = dims_ok && S >= 0 && S <= Nv && H * W <= Nv && Z * (H * W) <= Nv - S;
        s->lvl[t] = ok ? make_int4((int)H, (int)W, (int)S, 0) : make_int4(0, 0, 0, 0);
        s->zp[t] = ok ? (int)Z : 0;
    }
    __syncthreads();
    if (t == 0) {
        int tb = 0;
        for (int l = 0; l < L; ++l) {
            int4 v = s->lvl[l];
            const int tw = (v.y + kTile - 1) >> kTileShift, th = (v.x + kTile - 1) >> kTileShift;
            const int tpp = tw * th;
            // every tile holds a voxel, so a level has at most as many bins as voxels (< 2^31)
            int n = tpp * s->zp[l];
            if (n > nb_max - tb) {  // keep every bin inside the caller's workspace
                v = make_int4(0, 0, 0, 0);
                n = 0;
            }
            v.w = tb;
            s->lvl[l] = v;
            s->tw[l] = n ? tw : 0;
            s->tpp[l] = n ? tpp : 0;
            s->zp[l] = n ? s->zp[l] : 0;
            tb += n;
        }
        s->nbins = tb;
    }
    __syncthreads();
}

template <bool VOL>
__device__ __forceinline__ void stage_bin_levels(LevelLds *s, const int64_t *shapes,
                                                 const int64_t *starts, int L, int Nv, int nb_max) {
    if constexpr (VOL)
        stage_volume_levels(s, shapes, starts, L, Nv, nb_max);
    else
        stage_levels(s, shapes, starts, L, Nv, nb_max);
}

// The two planes a volume point's neighbours lie in: z0 (bit 0 of the mask)
// and z0 + 1 (bit 1), those inside [0, Z); fz is the fractional part of the
// voxel coordinate z = w*Z - 0.5 (or w*(Z - 1) with align_corners), formed
// like x and y.
struct Planes {
    int z0;          // clamped to [-1, Z]
    uint32_t mask;
    float fz;
};

__device__ __forceinline__ Planes point_planes(float w, int Z, bool align) {
    const float zc = __builtin_fmaf(w, align ? (float)(Z - 1) : (float)Z, align ? 0.f : -0.5f);
    const float z0 = floorf(zc);
    Planes p;
    p.fz = zc - z0;
    const bool v0 = z0 >= 0.f && z0 <= (float)(Z - 1), v1 = z0 >= -1.f && z0 <= (float)(Z - 2);
    p.mask = (v0 ? 1u : 0u) | (v1 ? 2u : 0u);
    p.z0 = (int)fminf(fmaxf(z0, -1.f), (float)Z);
    return p;
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
    int zero_list;   // scan: list the bins to zero (overwrite mode, grad_value not filled)
    int combine;     // split bins: partial tiles added up by the combine kernel
    // bin pipeline: the tensors' head count and queries per batch (strides
    // of loc, attn, grad_out and grad_value) when M and Nq are those of a
    // pass over some of them
    int Ms, Nqs;
};

// Workspace of the backward pipeline (all 32-bit words).
struct Work {
    uint32_t *counts;      // [B][nb_max][M] points per bin
    uint32_t *start;       // [B][nb_max][M] first entry of each bin in `sorted`
    uint32_t *cursor;      // [B][nb_max][M] next free entry while scattering
    uint4 *items;          // [work_max] (bin, first record, records, whole bin)
    uint32_t *work_total;  // [3]: work items, bins on the zero list, split bins listed
    uint32_t *zero;        // [B * nb_max * M] bins whose tiles no work item writes
                           // outright (overwrite mode): empty bins, and split bins when
                           // their items add into grad_value atomically
    uint32_t *split;       // [B * nb_max * M] split bins whose items leave partial
                           // tiles, added up by the combine kernel
    uint4 *recs;           // [4 * points] records grouped by bin
};

// The tile of a bin (b * nb_max + tile) * M + m: its batch and head, its
// level's map and the tile's origin.  For volumes the tile lies in one
// plane of its level, whose first row is row0.
struct BinTile {
    int b, m;
    int H, W;    // the level's map
    int row0;    // first row of the map (volumes: of the tile's plane) in a batch slice
    int x0, y0;  // pixel of the tile's top-left corner
};

template <bool VOL>
__device__ __forceinline__ BinTile bin_tile(uint32_t bin, const LevelLds &lv, int M, int nb_max,
                                            int L) {
    BinTile t;
    t.m = (int)(bin % (uint32_t)M);
    const uint32_t bt = bin / (uint32_t)M;
    t.b = (int)(bt / (uint32_t)nb_max);
    const int lb = (int)(bt - (uint32_t)t.b * nb_max);
    // levels left out of the table own no bins; their first-bin entry equals the next one's
    int l = 0;
    while (l + 1 < L && lv.lvl[l + 1].w <= lb) ++l;
    const int4 lvl = lv.lvl[l];
    int rel = lb - lvl.w;
    t.row0 = lvl.z;
    if constexpr (VOL) {
        const int zpl = rel / lv.tpp[l];
        rel -= zpl * lv.tpp[l];
        t.row0 += zpl * lvl.x * lvl.y;
    }
    const int tw = lv.tw[l];
    const int ty = rel / tw;
    t.x0 = (rel - ty * tw) * kTile;
    t.y0 = ty * kTile;
    t.H = lvl.x;
    t.W = lvl.y;
    return t;
}

// Zero the channels of head t.m of the tile's pixels inside the map, with
// NT threads (thread index tid); D channels per head, M heads per row
// (the tensor's head stride).
template <int NT>
__device__ __forceinline__ void zero_tile(float *__restrict__ grad_value, const BinTile &t,
                                          size_t slice_v, int M, int D, int tid) {
    const int quads = D >> 2;
    float *gv = grad_value + (size_t)t.b * slice_v + (size_t)t.m * D;
    for (int i = tid; i < kTilePx * quads; i += NT) {
        const int px = i / quads, q = i - px * quads;
        const int gx = t.x0 + (px & (kTile - 1)), gy = t.y0 + (px >> kTileShift);
        if (gy < t.H && gx < t.W)
            reinterpret_cast<float4 *>(gv + (size_t)(t.row0 + gy * t.W + gx) * M * D)[q] =
                make_float4(0.f, 0.f, 0.f, 0.f);
    }
}
// ---------------------------------------------------------------------------
// backward: points per bin
// Workgroup = (batch b, head m, PPT * kThreads consecutive points of the
// (b, m) list in (query, level, point) order), PPT points per thread,
// all of whose coordinates are loaded before any is used.
// ---------------------------------------------------------------------------
// Points per thread: kBinPPT, or kBinPPTSmall where that would leave fewer
// than kBinMinGrid workgroups (small problems such as the decoder's 300
// queries, 32 workgroups: more workgroups, each with fewer points in flight;
// the voxel workload's 384 measured slower with more).
constexpr int kBinPPT = 16;
constexpr int kBinPPTSmall = 1;
constexpr int kBinMinGrid = 128;

// VOL: volume levels; a location is (u, v, w) and a point feeds the tiles of
// its two planes.
template <bool VOL, int PPT>
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
    const int f0 = (wg % dm.nblk) * (PPT * kThreads);
    const int nf = Nq * LK;
    const size_t row0 = (size_t)b * dm.Nqs * dm.Ms + m;  // item row of query 0

    float2 uv[PPT];
    float wz[PPT];  // VOL: the z coordinate
#pragma unroll
    for (int r = 0; r < PPT; ++r) {
        const int f = f0 + threadIdx.x + r * kThreads;
        uv[r] = make_float2(0.f, 0.f);
        wz[r] = 0.f;
        if (f < nf) {
            const int q = (int)fdiv((uint32_t)f, dm.div_lk), j = f - q * LK;
            const size_t p = (row0 + (size_t)q * dm.Ms) * LK + j;
            if constexpr (VOL) {
                uv[r] = make_float2(loc[3 * p], loc[3 * p + 1]);
                wz[r] = loc[3 * p + 2];
            } else {
                uv[r] = reinterpret_cast<const float2 *>(loc)[p];
            }
        }
    }
    stage_bin_levels<VOL>(&s_lv, shapes, starts, dm.L, dm.Nv, dm.nb_max);
    const int nbins = s_lv.nbins;
    const bool lds = nbins <= hist_cap;
    uint32_t *gcount = counts + (size_t)b * dm.nb_max * M + m;  // tile i at gcount[i * M]
    if (lds) {
        for (int i = threadIdx.x; i < nbins; i += kThreads) s_cnt[i] = 0u;
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < PPT; ++r) {
        const int f = f0 + threadIdx.x + r * kThreads;
        if (f < nf) {
            const int q = (int)fdiv((uint32_t)f, dm.div_lk), j = f - q * LK;
            const int l = (int)fdiv((uint32_t)j, dm.div_k);
            const Neighbours n = neighbours(uv[r].x, uv[r].y, s_lv.lvl[l], 0u, 0u, dm.align);
            const TileMask tm = point_tile_mask(n);
            const int tw = s_lv.tw[l];
            const int b00 = s_lv.lvl[l].w + tm.ty0 * tw + tm.tx0;
            auto add = [&](int bb) {
                if (lds) {
                    if (tm.mask & 1u) atomicAdd(&s_cnt[bb], 1u);
                    if (tm.mask & 2u) atomicAdd(&s_cnt[bb + 1], 1u);
                    if (tm.mask & 4u) atomicAdd(&s_cnt[bb + tw], 1u);
                    if (tm.mask & 8u) atomicAdd(&s_cnt[bb + tw + 1], 1u);
                } else {
                    if (tm.mask & 1u) atomicAdd(&gcount[(size_t)bb * M], 1u);
                    if (tm.mask & 2u) atomicAdd(&gcount[(size_t)(bb + 1) * M], 1u);
                    if (tm.mask & 4u) atomicAdd(&gcount[(size_t)(bb + tw) * M], 1u);
                    if (tm.mask & 8u) atomicAdd(&gcount[(size_t)(bb + tw + 1) * M], 1u);
                }
            };
            if constexpr (VOL) {
                const Planes pl = point_planes(wz[r], s_lv.zp[l], dm.align);
                const int tpp = s_lv.tpp[l];
                if (pl.mask & 1u) add(b00 + pl.z0 * tpp);
                if (pl.mask & 2u) add(b00 + (pl.z0 + 1) * tpp);
            } else {
                add(b00);
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
// backward: scan of the bin counts, work list, zero list
// One workgroup of kScanThreads per block of kScanBlock bins.  Bins are
// visited in (batch, tile, head) order, which is also their order in memory:
// bin (b * nb_max + tile) * M + m; all batches form one flat scan.  Each
// workgroup first sums the counts of every bin before its block (a
// redundant reduction, coalesced: the blocks are few -- two at the encoder
// shape -- and no workgroup waits for another), then scans its block.
// Each bin of n > 0 points becomes ceil(n / kChunk) work items (bin, first
// record, records, whole bin).  In overwrite mode the bins whose pixels no
// single work item writes outright -- empty bins, and bins split over several
// items that add into grad_value atomically -- go on the zero list, and their
// tiles are zeroed (by the gather kernel after its items, or by the scatter
// kernel before the tile kernel adds into them).  When the items of split
// bins leave partial tiles instead (dm.combine), those bins go on the split
// list of the combine kernel.
// ---------------------------------------------------------------------------
// Exclusive scan of (a, b, c) over the kScanThreads threads of the block:
// wave-level scans with DPP, then one scan of the wave totals.  The block
// totals are returned in tot.
__device__ __forceinline__ void block_exclusive_scan3(uint32_t &a, uint32_t &b, uint32_t &c,
                                                      uint4 *s_wave, uint3 &tot) {
    constexpr int kWaves = kScanThreads / 64;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const uint32_t ia = wave_inclusive_scan(a), ib = wave_inclusive_scan(b);
    const uint32_t ic = wave_inclusive_scan(c);
    if (lane == 63) s_wave[wave] = make_uint4(ia, ib, ic, 0u);
    __syncthreads();
    if (wave == 0) {
        const uint4 v = lane < kWaves ? s_wave[lane] : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t sa = wave_inclusive_scan(v.x), sb = wave_inclusive_scan(v.y);
        const uint32_t sc = wave_inclusive_scan(v.z);
        if (lane < kWaves) s_wave[lane] = make_uint4(sa - v.x, sb - v.y, sc - v.z, 0u);
        if (lane == kWaves - 1) s_wave[kWaves] = make_uint4(sa, sb, sc, 0u);
    }
    __syncthreads();
    const uint4 base = s_wave[wave];
    tot = make_uint3(s_wave[kWaves].x, s_wave[kWaves].y, s_wave[kWaves].z);
    a = base.x + ia - a;
    b = base.y + ib - b;
    c = base.z + ic - c;
    __syncthreads();  // s_wave is reused by the next call
}

// Sum of (a, b, c, d) over the kScanThreads threads of the block, returned
// to every thread.
__device__ __forceinline__ uint4 block_sum4(uint4 v, uint4 *s_wave) {
    constexpr int kWaves = kScanThreads / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v.x = wave_inclusive_scan(v.x);
    v.y = wave_inclusive_scan(v.y);
    v.z = wave_inclusive_scan(v.z);
    v.w = wave_inclusive_scan(v.w);
    if (lane == 63) s_wave[wave] = v;  // the wave's totals
    __syncthreads();
    uint4 t = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        t.x += s_wave[i].x;
        t.y += s_wave[i].y;
        t.z += s_wave[i].z;
        t.w += s_wave[i].w;
    }
    __syncthreads();  // s_wave is reused
    return t;
}

// The items of a bin of cnt > kChunk records: nch = ceil(cnt / kChunk) of
// them, item k taking records [floor(k cnt / nch), floor((k+1) cnt / nch)),
// so that each holds between kChunk / 2 and kChunk records.  The bounds are
// stepped through as k cq + floor(k cr / nch), cnt = cq nch + cr, without
// 64-bit products.
struct ChunkStep {
    uint32_t nch, cq, cr, first, rem;
    __device__ __forceinline__ ChunkStep(uint32_t cnt, uint32_t s0)
        : nch((cnt + kChunk - 1) / kChunk), cq(0), cr(0), first(s0), rem(0) {
        cq = cnt / nch;
        cr = cnt - cq * nch;
    }
    // first record of the next item
    __device__ __forceinline__ void next() {
        rem += cr;
        first += cq + (rem >= nch ? 1u : 0u);
        rem -= rem >= nch ? nch : 0u;
    }
};

template <bool VOL>
__global__ void __launch_bounds__(kScanThreads)
bin_scan_kernel(const int64_t *__restrict__ shapes, const int64_t *__restrict__ starts,
                const uint32_t *__restrict__ counts, uint32_t *__restrict__ start,
                uint32_t *__restrict__ cursor, uint4 *__restrict__ items,
                uint32_t *__restrict__ work_total, uint32_t *__restrict__ zero,
                uint32_t *__restrict__ split, int B, Dims dm) {
    constexpr int kPer = kScanBlock / kScanThreads;
    constexpr uint32_t kPass = kScanBlock;  // bins of the workgroup
    static_assert(kPass < (1 << 16), "list counts of one block fit 16 bits");
    __shared__ LevelLds s_lv;
    __shared__ uint4 s_wave[kScanThreads / 64 + 1];
    // the block's bins in flat order: their counts; for each thread's kPer
    // bins, the first record, first item, and zero- and split-list positions
    // (16 bits each) of the first.  Little LDS, so that the workgroup finds a
    // place beside the kernel on the other stream.
    __shared__ uint32_t s_cnt[kPass], s_e[kScanThreads], s_ch[kScanThreads], s_zs[kScanThreads];
    stage_bin_levels<VOL>(&s_lv, shapes, starts, dm.L, dm.Nv, dm.nb_max);
    // The used bins of every batch as one flat sequence f = (b * nbins + tile) * M + m;
    // this workgroup scans f in [base, base + kPass).  Bin f is at f + b * gap in
    // memory (the bins of batch b start at b * nb_max * M).  Counts are loaded and
    // the results stored with consecutive lanes on consecutive bins; in between,
    // each thread sums kPer consecutive bins, through LDS.
    const uint32_t nbins = (uint32_t)s_lv.nbins, Mu = (uint32_t)dm.M;
    const uint32_t per_b = nbins * Mu, gap = ((uint32_t)dm.nb_max - nbins) * Mu;
    const uint32_t nf = per_b * (uint32_t)B;
    const uint32_t base = blockIdx.x * kPass;
    if (base >= nf) {  // past the used bins (the grid is sized for the bound)
        if (blockIdx.x == 0 && threadIdx.x == 0) {  // no bins at all
            work_total[0] = 0u;
            work_total[1] = 0u;
            work_total[2] = 0u;
        }
        return;
    }
    const bool zeroing = dm.zero_list != 0, combine = dm.combine != 0;
    // split bins need zeroed tiles only when their items add atomically
    const uint32_t zero_above = combine ? 0xffffffffu : (uint32_t)kChunk;
    auto listed = [&](uint32_t c) {  // zero-list entry | split-list entry << 16
        return ((zeroing && (c == 0u || c > zero_above)) ? 1u : 0u) |
               ((combine && c > (uint32_t)kChunk) ? 1u << 16 : 0u);
    };
    // 0. records, items, zero-list and split-list entries of the bins before
    // the block (the list counts summed apart: they may pass 16 bits)
    uint32_t carry_e, carry_c, carry_z, carry_s;
    {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        for (uint32_t f = threadIdx.x; f < base; f += kScanThreads) {
            const uint32_t c = counts[f + f / per_b * gap];
            const uint32_t l = listed(c);
            v.x += c;
            v.y += (c + kChunk - 1) / kChunk;
            v.z += l & 0xffffu;
            v.w += l >> 16;
        }
        v = block_sum4(v, s_wave);
        carry_e = v.x;
        carry_c = v.y;
        carry_z = v.z;
        carry_s = v.w;
    }
    {
        // 1. the block's counts, coalesced, into LDS (zero past the end)
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const uint32_t f = base + threadIdx.x + i * kScanThreads;
            s_cnt[f - base] = f < nf ? counts[f + f / per_b * gap] : 0u;
        }
        __syncthreads();
        // 2. thread t: bins t * kPer ... of the block
        const uint32_t j0 = threadIdx.x * kPer;
        uint32_t cnt[kPer], e = 0, ch = 0, zs = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            cnt[i] = s_cnt[j0 + i];
            e += cnt[i];
            ch += (cnt[i] + kChunk - 1) / kChunk;
            zs += base + j0 + i < nf ? listed(cnt[i]) : 0u;
        }
        uint3 tot;
        block_exclusive_scan3(e, ch, zs, s_wave, tot);
        s_e[threadIdx.x] = e;
        s_ch[threadIdx.x] = ch;
        s_zs[threadIdx.x] = zs;
        __syncthreads();
        // 3. bin starts, cursors, work items and list entries, coalesced
        {
#pragma unroll 1
            for (uint32_t f = base + threadIdx.x; f < nf && f < base + kPass; f += kScanThreads) {
                const uint32_t j = f - base, bin = f + f / per_b * gap, c = s_cnt[j];
                // this bin's offsets: its group's, plus the bins before it in the
                // group (all below nf)
                const uint32_t g = j / kPer, o = j - g * kPer;
                uint32_t e0 = s_e[g] + carry_e, c0 = s_ch[g] + carry_c, zs0 = s_zs[g];
#pragma unroll
                for (uint32_t i = 0; i < kPer - 1; ++i) {
                    const uint32_t ci = i < o ? s_cnt[g * kPer + i] : 0u;
                    e0 += ci;
                    c0 += (ci + kChunk - 1) / kChunk;
                    zs0 += i < o ? listed(ci) : 0u;
                }
                start[bin] = e0;
                cursor[bin] = e0;
                // nch balanced items: item k takes records [k c / nch, (k+1) c / nch)
                const uint32_t nch = (c + kChunk - 1) / kChunk;
                if (nch == 1u) {
                    items[c0] = make_uint4(bin, e0, c, 1u);
                } else if (nch > 1u) {
                    ChunkStep cs(c, e0);
                    for (uint32_t k = 0; k < nch; ++k) {
                        const uint32_t r0 = cs.first;
                        cs.next();
                        items[c0 + k] = make_uint4(bin, r0, cs.first - r0, 0u);
                    }
                }
                const uint32_t l = listed(c);
                if (l & 1u) zero[carry_z + (zs0 & 0xffffu)] = bin;
                if (l >> 16) split[carry_s + (zs0 >> 16)] = bin;
            }
        }
        carry_e += tot.x;
        carry_c += tot.y;
        carry_z += tot.z & 0xffffu;
        carry_s += tot.z >> 16;
    }
    // the block holding the last bin writes the totals
    if (base + kPass >= nf && threadIdx.x == 0) {
        work_total[0] = carry_c;
        work_total[1] = carry_z;
        work_total[2] = carry_s;
    }
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
using msda_host::kRecQueryShift;   // cells < 128

// Zeroing (zero != nullptr, one launch per call): before its own points,
// workgroup g zeroes the tiles of zero-list entries g, g + grid, ... -- the
// grad_value kernel, launched after this one, then adds into them.
struct ZeroList {
    const uint32_t *zero;        // bins, or nullptr: nothing to zero
    const uint32_t *work_total;  // [3]: work items, entries on the list, split bins
    float *grad_value;
    int D;
};

template <bool VOL, int PPT>
__global__ void __launch_bounds__(kThreads)
bin_scatter_kernel(const int64_t *__restrict__ shapes, const int64_t *__restrict__ starts,
                   const float *__restrict__ loc, const float *__restrict__ attn,
                   uint32_t *__restrict__ cursor, uint4 *__restrict__ recs, int hist_cap,
                   ZeroList zl, Dims dm) {
    __shared__ LevelLds s_lv;
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *s_cnt = reinterpret_cast<uint32_t *>(smem);  // [hist_cap] counts, then ranks
    uint32_t *s_base = s_cnt + hist_cap;                    // [hist_cap] reserved offsets

    const int M = dm.M, LK = dm.L * dm.K, Nq = dm.Nq;
    const int wg = xcd_contiguous(blockIdx.x, gridDim.x);
    const int bm = wg / dm.nblk + dm.b0 * M;
    const int m = bm % M, b = bm / M;
    const int f0 = (wg % dm.nblk) * (PPT * kThreads);
    const int nf = Nq * LK;
    const size_t row0 = (size_t)b * dm.Nqs * dm.Ms + m;  // item row of query 0

    // the thread's points: coordinates and weights, kept for both passes
    float2 uv[PPT];
    float aw[PPT];
    float wz[PPT];  // VOL: the z coordinate
#pragma unroll
    for (int r = 0; r < PPT; ++r) {
        const int f = f0 + threadIdx.x + r * kThreads;
        uv[r] = make_float2(0.f, 0.f);
        aw[r] = 0.f;
        wz[r] = 0.f;
        if (f < nf) {
            const int q = (int)fdiv((uint32_t)f, dm.div_lk), j = f - q * LK;
            const size_t p = (row0 + (size_t)q * dm.Ms) * LK + j;
            if constexpr (VOL) {
                uv[r] = make_float2(loc[3 * p], loc[3 * p + 1]);
                wz[r] = loc[3 * p + 2];
            } else {
                uv[r] = reinterpret_cast<const float2 *>(loc)[p];
            }
            aw[r] = attn[p];
        }
    }
    stage_bin_levels<VOL>(&s_lv, shapes, starts, dm.L, dm.Nv, dm.nb_max);
    if (zl.zero) {
        const uint32_t nz = zl.work_total[1];
        const size_t slice_v = (size_t)dm.Nv * dm.Ms * zl.D;
        for (uint32_t zi = blockIdx.x; zi < nz; zi += gridDim.x)
            zero_tile<kThreads>(zl.grad_value, bin_tile<VOL>(zl.zero[zi], s_lv, M, dm.nb_max, dm.L),
                                slice_v, dm.Ms, zl.D, threadIdx.x);
    }
    const int nbins = s_lv.nbins;
    const bool lds = nbins <= hist_cap;
    uint32_t *gcur = cursor + (size_t)b * dm.nb_max * M + m;  // tile i at gcur[i * M]
    if (lds) {
        for (int i = threadIdx.x; i < nbins; i += kThreads) s_cnt[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < PPT; ++r) {
            const int f = f0 + threadIdx.x + r * kThreads;
            if (f < nf) {
                const int q = (int)fdiv((uint32_t)f, dm.div_lk), j = f - q * LK;
                const int l = (int)fdiv((uint32_t)j, dm.div_k);
                const Neighbours n = neighbours(uv[r].x, uv[r].y, s_lv.lvl[l], 0u, 0u, dm.align);
                const TileMask tm = point_tile_mask(n);
                const int tw = s_lv.tw[l];
                const int b00 = s_lv.lvl[l].w + tm.ty0 * tw + tm.tx0;
                auto add = [&](int bb) {
                    if (tm.mask & 1u) atomicAdd(&s_cnt[bb], 1u);
                    if (tm.mask & 2u) atomicAdd(&s_cnt[bb + 1], 1u);
                    if (tm.mask & 4u) atomicAdd(&s_cnt[bb + tw], 1u);
                    if (tm.mask & 8u) atomicAdd(&s_cnt[bb + tw + 1], 1u);
                };
                if constexpr (VOL) {
                    const Planes pl = point_planes(wz[r], s_lv.zp[l], dm.align);
                    const int tpp = s_lv.tpp[l];
                    if (pl.mask & 1u) add(b00 + pl.z0 * tpp);
                    if (pl.mask & 2u) add(b00 + (pl.z0 + 1) * tpp);
                } else {
                    add(b00);
                }
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
    for (int r = 0; r < PPT; ++r) {
        const int f = f0 + threadIdx.x + r * kThreads;
        if (f < nf) {
            const int q = (int)fdiv((uint32_t)f, dm.div_lk), j = f - q * LK;
            const int l = (int)fdiv((uint32_t)j, dm.div_k);
            const Neighbours n = neighbours(uv[r].x, uv[r].y, s_lv.lvl[l], 0u, 0u, dm.align);
            const TileMask tm = point_tile_mask(n);
            const int tw = s_lv.tw[l];
            const int b00 = s_lv.lvl[l].w + tm.ty0 * tw + tm.tx0;
            const uint32_t fy = __float_as_uint(n.fy);
            // cell of the top-left neighbour relative to tile (tx0, ty0); one
            // tile to the right is 8 cells left, one tile down is 72 cells up
            const uint32_t key = ((uint32_t)q << kRecQueryShift);
            const int c00 = (n.xi - tm.tx0 * kTile + 1) + kCellsW * (n.yi - tm.ty0 * kTile + 1);
            // the records of one plane: bins from bb, weight a = A (times the
            // plane's z tent for volumes)
            auto put = [&](int bb, float a) {
                const uint32_t a0 = __float_as_uint(a * (1.f - n.fx));
                const uint32_t a1 = __float_as_uint(a * n.fx);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (tm.mask & (1u << c)) {
                        const int bin = bb + (c & 1) + (c >> 1) * tw;
                        const uint32_t slot = lds ? s_base[bin] + atomicAdd(&s_cnt[bin], 1u)
                                                  : atomicAdd(&gcur[(size_t)bin * M], 1u);
                        const int cell = c00 - (c & 1) * kTile - (c >> 1) * kTile * kCellsW;
                        recs[slot] = make_uint4(key | (uint32_t)cell, a0, a1, fy);
                    }
                }
            };
            if constexpr (VOL) {
                const Planes pl = point_planes(wz[r], s_lv.zp[l], dm.align);
                const int tpp = s_lv.tpp[l];
                if (pl.mask & 1u) put(b00 + pl.z0 * tpp, aw[r] * (1.f - pl.fz));
                if (pl.mask & 2u) put(b00 + (pl.z0 + 1) * tpp, aw[r] * pl.fz);
            } else {
                put(b00, aw[r]);
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

template <int D, bool VOL>
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
    stage_bin_levels<VOL>(&s_lv, shapes, starts, dm.L, dm.Nv, dm.nb_max);
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
            const float *gob = grad_out + ((size_t)b * dm.Nqs * dm.Ms + m) * D;
            for (int i = tid; i < nb * kQuads; i += kTileThreads) {
                const int slot = i / kQuads, qd = i - slot * kQuads;
                const uint32_t qy = min(s_q[slot], (uint32_t)Nq - 1u);  // a query of this batch
                const float *src = gob + (size_t)qy * dm.Ms * D + 4 * qd;
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
                pull_range<kQuads>(acc[o], wP, gP + q, (int)stP[cT], (int)stP[cT + 1],
                                   (int)stP[cT + 2], 1, 0);
                pull_range<kQuads>(acc[o], wP, gP + q, (int)stP[cB], (int)stP[cB + 1],
                                   (int)stP[cB + 2], 3, 2);
            }
            // 6. the item ends with A: write its tile
            if (A.off + kSub >= A.it.z) {
                const BinTile t = bin_tile<VOL>(A.it.x, s_lv, M, dm.nb_max, dm.L);
                const size_t slice = (size_t)dm.Nv * dm.Ms * D;
                float *gv = grad_value + (size_t)t.b * slice + (size_t)t.m * D;
#pragma unroll
                for (int o = 0; o < kOwn; ++o) {
                    const int pair = tid + o * kTileThreads;
                    if (pair >= kTilePx * kQuads) break;
                    const int px = pair / kQuads, q = pair - px * kQuads;
                    const int gx = t.x0 + (px & (kTile - 1));
                    const int gy = t.y0 + (px >> kTileShift);
                    float4 a = acc[o];
                    acc[o] = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (gy >= t.H || gx >= t.W) continue;
                    float *dst = gv + (size_t)(t.row0 + gy * t.W + gx) * dm.Ms * D + 4 * q;
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
// backward: grad_value by gathering, one 8x8 tile (and chunk of its records)
// per work item, for heads of up to kGatherMaxD channels
//
// The item's records are counting-sorted by cell once, into LDS.  A lane
// owns one (cell, group of kGatherCPL channels) pair and walks the records
// of its cell, loading its channels of each record's grad_out row straight
// from global memory: the cell's lanes (two at D = 32) read the row together,
// so every record's row is fetched once, and kGatherBatch records per lane
// are in flight.  For
// cell (x, y) -- top-left neighbour at tile pixel (x-1, y-1) -- the lane keeps
// one sum per neighbour role:
//   top-left     (weight A (1-fx)(1-fy)) for pixel (x-1, y-1),
//   top-right    (A fx (1-fy))           for pixel (x,   y-1),
//   bottom-left  (A (1-fx) fy)           for pixel (x-1, y),
//   bottom-right (A fx fy)               for pixel (x,   y),
// and drops the roles whose pixel lies outside the tile.  Every pixel of the
// tile receives exactly one sum of each role, so the sums are exchanged
// through LDS without conflicts and each pixel is written once.
// ---------------------------------------------------------------------------
constexpr int kGatherMaxD = 32;
constexpr int kGatherCPL = 16;  // channels per lane (four quads): 81 cells x 2 lanes at D = 32
constexpr int kGatherBatch = 2;  // records whose rows a lane loads together
constexpr int kCombineGrid = 1024;  // combine kernel: workgroups, at most
constexpr int kCombineBatch = 4;    // combine kernel: partial tiles loaded together

template <int CPL> constexpr int gather_threads() { return kCells * (kGatherMaxD / CPL); }

template <int D, bool VOL, int CPL>
__global__ void __launch_bounds__(gather_threads<CPL>())
grad_value_gather_kernel(const int64_t *__restrict__ shapes, const int64_t *__restrict__ starts,
                         const float *__restrict__ grad_out, const uint4 *__restrict__ items,
                         const uint32_t *__restrict__ work_total, uint4 *__restrict__ recs,
                         const uint32_t *__restrict__ zero, float *__restrict__ grad_value,
                         Dims dm) {
    static_assert(D <= kGatherMaxD && D % 4 == 0, "one (cell, channel group) pair per lane");
    constexpr int kT = gather_threads<CPL>();
    constexpr int kQuads = D / 4;
    constexpr int kQPL = (CPL < D ? CPL : D) / 4;  // quads per lane
    constexpr int kGroups = kQuads / kQPL;          // lanes per cell
    constexpr int kPairs = kCells * kGroups;
    constexpr int kPer = (kChunk + kT - 1) / kT;     // records per thread in the sort
    static_assert(kPairs <= kT, "every (cell, channel group) pair has a lane");
    static_assert(4 * kTilePx * kQuads <= kChunk, "the role sums fit the record table");
    static_assert(kTilePx * kQuads <= kChunk / 2, "a partial tile fits an item's records");
    __shared__ LevelLds s_lv;
    __shared__ uint32_t s_cnt[kCells];     // records per cell
    __shared__ uint32_t s_st[kCells + 1];  // first sorted slot of each cell, and the total
    __shared__ uint4 s_tab[kChunk];        // the item's records in cell order
    // after the gather, the role sums: [role][pixel][quad], the quads of pixel
    // p rotated by p (quad q at slot q ^ (p mod kQuads)), so that the lanes
    // writing one quad of consecutive pixels hit different banks
    float4 *s_red = reinterpret_cast<float4 *>(s_tab);
    auto red_slot = [](int i) { return i ^ ((i / kQuads) & (kQuads - 1)); };  // i = p * kQuads + q

    const int M = dm.M, Nq = dm.Nq;
    const int tid = threadIdx.x;
    // the work items, then (overwrite mode) the tiles of the zero list
    const uint32_t total = work_total[0];
    const uint32_t nz = zero ? work_total[1] : 0u;
    if (blockIdx.x >= total + nz) return;  // the grid is sized for the largest possible list
    stage_bin_levels<VOL>(&s_lv, shapes, starts, dm.L, dm.Nv, dm.nb_max);
    if (tid < kCells) s_cnt[tid] = 0u;

    const bool owner = tid < kPairs;
    const int cell = tid / kGroups, grp = tid - cell * kGroups;
    const int cx = cell % kCellsW, cy = cell / kCellsW;
    const uint32_t row_stride = (uint32_t)dm.Ms * D * 4u;
    // the rows of one batch's queries; the host keeps them below 2^32 bytes,
    // and an offset of `slice` reads zeros (outside the descriptor's range)
    const uint32_t slice = (uint32_t)((size_t)Nq * dm.Ms * D * 4);
    __syncthreads();

    // Workgroup g takes items g, g + grid, ... counted from the end of the
    // list (the coarse levels' bins, the largest, first): the whole chip
    // works through one stretch of the list, and of the records, at a time.
    // (Cutting the list into one contiguous stretch per XCD, by head or by
    // tile range, was measured slower.)
    for (uint32_t w = blockIdx.x; w < total + nz; w += gridDim.x) {
        if (w >= total) {
            // an empty bin: no item writes its tile
            zero_tile<kT>(grad_value, bin_tile<VOL>(zero[w - total], s_lv, M, dm.nb_max, dm.L),
                          (size_t)dm.Nv * dm.Ms * D, dm.Ms, D, tid);
            continue;
        }
        const uint4 it = items[total - 1u - w];  // (bin, first record, records, whole bin)
        const int n = (int)min(it.z, (uint32_t)kChunk);
        // 1. the records, and each one's rank within its cell
        uint4 rec[kPer];
        uint32_t rank[kPer];
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int i = tid + r * kT;
            rec[r] = i < n ? recs[it.y + i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int i = tid + r * kT;
            rank[r] = i < n ? atomicAdd(&s_cnt[rec[r].x & ((1u << kRecQueryShift) - 1u)], 1u) : 0u;
        }
        __syncthreads();
        // 2. exclusive scan of the 81 counts by one wave, 2 cells a lane
        if (tid < 64) {
            const int c0 = 2 * tid, c1 = 2 * tid + 1;
            const uint32_t v0 = c0 < kCells ? s_cnt[c0] : 0u;
            const uint32_t v1 = c1 < kCells ? s_cnt[c1] : 0u;
            const uint32_t incl = wave_inclusive_scan(v0 + v1);
            const uint32_t ex = incl - v0 - v1;
            if (c0 < kCells) s_st[c0] = ex;
            if (c1 < kCells) s_st[c1] = ex + v0;
            if (tid == 63) s_st[kCells] = incl;
        }
        __syncthreads();
        // 3. the records in cell order (ranks are below their cell's count,
        // so every slot is below n); the counts are free for the next item
        if (tid < kCells) s_cnt[tid] = 0u;
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int i = tid + r * kT;
            if (i < n) {
                const uint32_t c = rec[r].x & ((1u << kRecQueryShift) - 1u);
                s_tab[min(s_st[c] + rank[r], (uint32_t)kChunk - 1u)] = rec[r];
            }
        }
        __syncthreads();

        // 4. the lane's cell: four role sums of A * w * grad_out
        const uint32_t bin = it.x;  // (b * nb_max + tile) * M + m
        const int m = (int)(bin % (uint32_t)M);
        const uint32_t bt = bin / (uint32_t)M;
        const int b = (int)(bt / (uint32_t)dm.nb_max);
        float4 acc[4][kQPL];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int k = 0; k < kQPL; ++k) acc[r][k] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (owner) {
            const rsrc_t go = make_rsrc(grad_out + (size_t)b * dm.Nqs * dm.Ms * D, slice);
            const uint32_t lane_off = (uint32_t)m * D * 4u + 16u * (uint32_t)(grp * kQPL);
            const int e0 = (int)s_st[cell], e1 = (int)s_st[cell + 1];
            for (int e = e0; e < e1; e += kGatherBatch) {
                uint4 t[kGatherBatch];
                float4 g[kGatherBatch][kQPL];
#pragma unroll
                for (int u = 0; u < kGatherBatch; ++u) t[u] = s_tab[min(e + u, e1 - 1)];
#pragma unroll
                for (int u = 0; u < kGatherBatch; ++u) {
                    const uint32_t q = min(t[u].x >> kRecQueryShift, (uint32_t)Nq - 1u);
                    const uint32_t off = e + u < e1 ? q * row_stride + lane_off : slice;
#pragma unroll
                    for (int k = 0; k < kQPL; ++k) {
                        auto v = __builtin_amdgcn_raw_buffer_load_b128(
                            go, (int)(off + 16u * k), 0, 0);
                        g[u][k] = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]),
                                              __uint_as_float(v[2]), __uint_as_float(v[3]));
                    }
                }
#pragma unroll
                for (int u = 0; u < kGatherBatch; ++u) {
                    const float a0 = __uint_as_float(t[u].y), a1 = __uint_as_float(t[u].z);
                    const float fy = __uint_as_float(t[u].w), gy = 1.f - fy;
                    const float w0 = a0 * gy, w1 = a1 * gy, w2 = a0 * fy, w3 = a1 * fy;
#pragma unroll
                    for (int k = 0; k < kQPL; ++k) {
                        fma4(acc[0][k], w0, g[u][k]);
                        fma4(acc[1][k], w1, g[u][k]);
                        fma4(acc[2][k], w2, g[u][k]);
                        fma4(acc[3][k], w3, g[u][k]);
                    }
                }
            }
        }
        __syncthreads();  // the record table is free: it takes the role sums
        if (owner) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int px = cx - 1 + (r & 1), py = cy - 1 + (r >> 1);
                if (px >= 0 && px < kTile && py >= 0 && py < kTile) {
#pragma unroll
                    for (int k = 0; k < kQPL; ++k)
                        s_red[r * kTilePx * kQuads +
                              red_slot((py * kTile + px) * kQuads + grp * kQPL + k)] = acc[r][k];
                }
            }
        }
        __syncthreads();
        // 5. the tile: pixel = the four roles' sums
        const BinTile tile = bin_tile<VOL>(bin, s_lv, M, dm.nb_max, dm.L);
        const size_t slice_v = (size_t)dm.Nv * dm.Ms * D;
        float *gv = grad_value + (size_t)b * slice_v + (size_t)m * D;
        auto tile_sum = [&](int i) {  // i = pixel * kQuads + quad
            const int j = red_slot(i);
            float4 a = s_red[j];
#pragma unroll
            for (int r = 1; r < 4; ++r) add4(a, s_red[r * kTilePx * kQuads + j]);
            return a;
        };
        auto write_px = [&](int i, float4 a) {
            const int px = i / kQuads, q = i - px * kQuads;
            const int gx = tile.x0 + (px & (kTile - 1));
            const int gy = tile.y0 + (px >> kTileShift);
            if (gy >= tile.H || gx >= tile.W) return;
            float4 *d4 = reinterpret_cast<float4 *>(
                gv + (size_t)(tile.row0 + gy * tile.W + gx) * dm.Ms * D + 4 * q);
            if (dm.accumulate) add4(a, *d4);
            *d4 = a;
        };
        if (it.w) {
            // this work item alone owns the tile
            for (int i = tid; i < kTilePx * kQuads; i += kT) write_px(i, tile_sum(i));
        } else {
            // one item of a split bin: the partial tile goes into the item's
            // own records, read already, for the combine kernel
            float4 *part = reinterpret_cast<float4 *>(recs + it.y);
            for (int i = tid; i < kTilePx * kQuads; i += kT) part[i] = tile_sum(i);
        }
        // the next item's first barrier orders these reads of s_red before
        // its records overwrite the table
    }
}

using msda_host::min_workspace;
using msda_host::pass_plan;
using msda_host::PassPlan;
using msda_host::WorkLayout;
using msda_host::work_layout;

// The tiles of split bins after the gather kernel: one workgroup per listed
// bin adds up, in item order, the partial tiles its items left at the start
// of their records, and writes the tile (adding to grad_value in accumulate
// mode).  Every pixel of the tile is written by one thread, once.
template <int D, bool VOL>
__global__ void __launch_bounds__(kThreads)
split_combine_kernel(const int64_t *__restrict__ shapes, const int64_t *__restrict__ starts,
                     const uint32_t *__restrict__ split, const uint32_t *__restrict__ work_total,
                     const uint32_t *__restrict__ counts, const uint32_t *__restrict__ start,
                     const uint4 *__restrict__ recs, float *__restrict__ grad_value, Dims dm) {
    constexpr int kQuads = D / 4;
    constexpr int kPerT = (kTilePx * kQuads + kThreads - 1) / kThreads;
    __shared__ LevelLds s_lv;
    const uint32_t total = work_total[2];
    if (blockIdx.x >= total) return;  // the grid is sized for the largest possible list
    stage_bin_levels<VOL>(&s_lv, shapes, starts, dm.L, dm.Nv, dm.nb_max);
    const int M = dm.M;
    for (uint32_t w = blockIdx.x; w < total; w += gridDim.x) {
        const uint32_t bin = split[w];
        ChunkStep cs(counts[bin], start[bin]);
        const uint32_t nch = cs.nch;
        float4 a[kPerT];
#pragma unroll
        for (int u = 0; u < kPerT; ++u) a[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        for (uint32_t k = 0; k < nch; k += kCombineBatch) {
            float4 v[kCombineBatch][kPerT];
#pragma unroll
            for (int c = 0; c < kCombineBatch; ++c) {
                const bool in = k + c < nch;
                const float4 *part = reinterpret_cast<const float4 *>(recs + cs.first);
#pragma unroll
                for (int u = 0; u < kPerT; ++u) {
                    const int i = threadIdx.x + u * kThreads;
                    v[c][u] = in && i < kTilePx * kQuads ? part[i]
                                                         : make_float4(0.f, 0.f, 0.f, 0.f);
                }
                cs.next();
            }
#pragma unroll
            for (int c = 0; c < kCombineBatch; ++c)
#pragma unroll
                for (int u = 0; u < kPerT; ++u) add4(a[u], v[c][u]);
        }
        const BinTile tile = bin_tile<VOL>(bin, s_lv, M, dm.nb_max, dm.L);
        float *gv = grad_value + (size_t)tile.b * dm.Nv * dm.Ms * D + (size_t)tile.m * D;
#pragma unroll
        for (int u = 0; u < kPerT; ++u) {
            const int i = threadIdx.x + u * kThreads;
            const int px = i / kQuads, q = i - px * kQuads;
            const int gx = tile.x0 + (px & (kTile - 1));
            const int gy = tile.y0 + (px >> kTileShift);
            if (i >= kTilePx * kQuads || gy >= tile.H || gx >= tile.W) continue;
            float4 *d4 = reinterpret_cast<float4 *>(
                gv + (size_t)(tile.row0 + gy * tile.W + gx) * dm.Ms * D + 4 * q);
            if (dm.accumulate) add4(a[u], *d4);
            *d4 = a[u];
        }
    }
}

// The grad_value stage: the gather kernel for heads of up to kGatherMaxD
// channels whose grad_out batch is 32-bit addressable (then the combine
// kernel writes the tiles of split bins), else the tile kernel (whose
// split-bin items add into zeroed tiles atomically).
// Nq queries of rows of Ms heads.
template <int D>
bool uses_gather(int64_t Nq, int64_t Ms) {
    return D <= kGatherMaxD && Nq * Ms * D * 4 < ((int64_t)1 << 32) - 64;
}

template <int D, bool VOL>
hipError_t launch_grad_value(const WorkLayout &wl, int64_t Nq, int64_t Ms, const int64_t *shapes,
                             const int64_t *starts, const float *gout, const Work &w,
                             float *gval, const Dims &dm, hipStream_t s) {
    const int64_t grid = wl.work_max < kTileGrid ? wl.work_max : kTileGrid;
    const uint4 *items = w.items, *recs = w.recs;
    const uint32_t *work_total = w.work_total;
    if constexpr (D <= kGatherMaxD) {
        if (uses_gather<D>(Nq, Ms)) {
            hipLaunchKernelGGL((grad_value_gather_kernel<D, VOL, kGatherCPL>),
                               dim3((unsigned)grid), dim3(gather_threads<kGatherCPL>()), 0, s,
                               shapes, starts, gout, items, work_total, w.recs,
                               dm.zero_list ? w.zero : nullptr, gval, dm);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            // split bins: more than kChunk records each, and at most one per bin
            int64_t nsplit = wl.sorted_max / (kChunk + 1) + 1;
            nsplit = nsplit < wl.bm_bins ? nsplit : wl.bm_bins;
            const unsigned cgrid = (unsigned)(nsplit < kCombineGrid ? nsplit : kCombineGrid);
            hipLaunchKernelGGL((split_combine_kernel<D, VOL>), dim3(cgrid), dim3(kThreads), 0, s,
                               shapes, starts, w.split, work_total, w.counts, w.start, recs,
                               gval, dm);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((grad_value_tile_kernel<D, VOL>), dim3((unsigned)grid),
                       dim3(kTileThreads), 0, s, shapes, starts, gout, items, work_total, recs,
                       gval, dm);
    return hipGetLastError();
}


// ---------------------------------------------------------------------------
// host side of the pipeline
// ---------------------------------------------------------------------------

Work work_at(const WorkLayout &wl, unsigned char *ws) {
    Work w;
    w.counts = reinterpret_cast<uint32_t *>(ws + wl.off_counts);
    w.start = reinterpret_cast<uint32_t *>(ws + wl.off_start);
    w.cursor = reinterpret_cast<uint32_t *>(ws + wl.off_cursor);
    w.items = reinterpret_cast<uint4 *>(ws + wl.off_items);
    w.work_total = reinterpret_cast<uint32_t *>(ws + wl.off_total);
    w.zero = reinterpret_cast<uint32_t *>(ws + wl.off_zero);
    w.split = reinterpret_cast<uint32_t *>(ws + wl.off_split);
    w.recs = reinterpret_cast<uint4 *>(ws + wl.off_sorted);
    return w;
}

FastDiv make_fastdiv(uint32_t d) {  // d >= 1
    uint32_t shift = 0;
    while (shift < 31 && (1u << shift) < d) ++shift;
    const uint64_t mul = ((uint64_t)1 << 32) * (((uint64_t)1 << shift) - d) / d + 1;
    return FastDiv{(uint32_t)mul, shift};
}

// Stages of the backward, for the caller's timing events (msda.h).
constexpr int kStageDots = 0, kStageClear = 1, kStageCount = 2, kStageScan = 3,
              kStageScatter = 4, kStageGather = 5;
static_assert(kStageGather + 1 == MSDA_BWD_STAGES, "stage numbering matches msda.h");

// Where the backward enqueues: the caller's stream s and, optionally, a
// second caller-owned stream for the grad_attn / grad_loc kernel, forked
// from s and joined back into it with the caller's two events; optional
// per-stage timing events.
struct Exec {
    hipStream_t s;
    hipStream_t side;         // nullptr: everything on s
    hipEvent_t fork, join;
    hipEvent_t *ev;           // optional: 2 * stages caller events (start, end)
    // in a pipeline of several passes: whether this is the first / last one
    // (a stage's start is recorded in the first pass, its end in the last)
    bool first = true, last = true;
    // record the start (end = false) or end event of stage i on stream `on`
    void stamp(int i, bool end, hipStream_t on) const {
        if (end ? !last : !first) return;
        if (ev && ev[2 * i + (end ? 1 : 0)]) (void)hipEventRecord(ev[2 * i + (end ? 1 : 0)], on);
    }
    hipStream_t dots_stream() const { return side ? side : s; }
};

// Check and take the caller's side stream and its two events.  A NULL
// side_stream, or one equal to the caller's stream, means one stream.
inline msda_status exec_side(Exec &ex, void *side_stream, void *const *side_events) {
    ex.side = nullptr;
    ex.fork = ex.join = nullptr;
    hipStream_t side = static_cast<hipStream_t>(side_stream);
    if (!side || side == ex.s) return MSDA_OK;
    if (!side_events || !side_events[0] || !side_events[1]) return MSDA_ERR_NULL;
    ex.side = side;
    ex.fork = static_cast<hipEvent_t>(side_events[0]);
    ex.join = static_cast<hipEvent_t>(side_events[1]);
    return MSDA_OK;
}

// Below this many sampling points (B * Nq * M * L * K) the backward runs on
// s alone: the fork and join cost more host time (two cross-stream waits,
// about 8 us each to enqueue) than running the grad_attn / grad_loc kernel
// beside the grad_value kernels saves.  Measured with the encoder's levels,
// B = 2, M = 8, L = K = 4: one stream 5 us faster at 300 queries (77k
// points), even at 1000, the side stream 5 us faster from 2000 on.
constexpr int64_t kSideMinPoints = (int64_t)1 << 18;

// The side stream, if the problem is large enough to use it, waits for
// everything enqueued on s so far; otherwise the side stream is dropped.
inline msda_status exec_fork(Exec &ex, int64_t points) {
    if (points < kSideMinPoints) ex.side = nullptr;
    if (!ex.side) return MSDA_OK;
    msda_status st = hip_status(hipEventRecord(ex.fork, ex.s));
    if (st == MSDA_OK) st = hip_status(hipStreamWaitEvent(ex.side, ex.fork, 0));
    return st;
}

// s waits for everything enqueued on the side stream so far.  Called after a
// successful fork on every path, failures included, so the side stream never
// runs ahead of work the caller enqueues on s later.
inline msda_status exec_join(const Exec &ex) {
    if (!ex.side) return MSDA_OK;
    msda_status st = hip_status(hipEventRecord(ex.join, ex.side));
    if (st == MSDA_OK) st = hip_status(hipStreamWaitEvent(ex.s, ex.join, 0));
    return st;
}

// Launches of per_b workgroups per batch, in chunks of batches that keep a
// grid below 2^23 workgroups; launch(b0, grid) enqueues one chunk.
template <typename F>
msda_status per_batch(int64_t B, int64_t per_b, F &&launch) {
    const int64_t bchunk = batch_chunk(per_b, B);
    for (int64_t b0 = 0; b0 < B; b0 += bchunk) {
        const int64_t nb = (B - b0) < bchunk ? (B - b0) : bchunk;
        launch(b0, (unsigned)(per_b * nb));
        const msda_status e = hip_status(hipGetLastError());
        if (e != MSDA_OK) return e;
    }
    return MSDA_OK;
}

// The grad_value pipeline on the caller's stream: clear the bin counters,
// count, scan (work list, zero list, split list), scatter the records, and
// the grad_value kernel(s).  In overwrite mode the tiles no work item writes
// outright must be zeroed: the scan lists them (empty bins; with the tile
// kernel also split bins, whose items add atomically).  The gather kernel
// zeroes the listed tiles itself, after its work items, with workgroups the
// items leave free; for the tile kernel the scatter kernel zeroes them first
// when the problem has at least two points per pixel and head, and sparser
// problems are zero-filled whole, by many workgroups at streaming speed (the
// scatter kernel's few workgroups would be slow to zero most of the tiles).
// The tensors hold Ms heads and Nqs queries per batch; this call covers
// heads [0, M) and queries [0, Nq) from the pointers given (a pass of
// run_bins_passes), and grad_value's slice of those heads.
template <int D, bool VOL>
msda_status run_bins(const int64_t *shapes, const int64_t *starts, const float *loc,
                     const float *attn, const float *gout, float *gval, int64_t B, int64_t Nv,
                     int64_t Nq, int64_t M, int64_t L, int64_t K, int64_t Ms, int64_t Nqs,
                     const WorkLayout &wl, unsigned char *ws, bool accumulate, bool align,
                     const Exec &ex, bool counts_clear) {
    const hipStream_t s = ex.s;
    const Work w = work_at(wl, ws);
    const bool gather = uses_gather<D>(Nq, Ms);
    // a pass over some of the heads cannot fill grad_value whole: its
    // untouched tiles are zeroed from the list
    const bool zero_list = !accumulate && (gather || Nq * L * K >= 2 * Nv || M != Ms);
    // the counts region is padded to 256 bytes, so whole float4s can be cleared
    // (unless the caller has: counts_clear)
    ex.stamp(kStageClear, false, s);
    msda_status st =
        counts_clear ? MSDA_OK : fill_zero(w.counts, (wl.off_start - wl.off_counts) / 16, s);
    if (st == MSDA_OK && !accumulate && !zero_list)
        st = fill_zero(gval, (size_t)(B * Nv * M * D) / 4, s);
    if (st != MSDA_OK) return st;
    ex.stamp(kStageClear, true, s);

    const int hist_cap = (int)(wl.nb_max < kHistLds ? wl.nb_max : kHistLds);
    const int64_t pts_bm = Nq * L * K;  // points per (batch, head)
    const int64_t big = kBinPPT * kThreads, small = kBinPPTSmall * kThreads;
    const bool few = B * M * ((pts_bm + big - 1) / big) < kBinMinGrid;
    const int64_t gb = (pts_bm + (few ? small : big) - 1) / (few ? small : big);  // per (b, m)
    Dims dm{(int)Nv, (int)Nq, (int)M, (int)L, (int)K, 0, 0, 0, (int)gb, (int)wl.nb_max,
            accumulate ? 1 : 0, make_fastdiv((uint32_t)(L * K)), make_fastdiv((uint32_t)K)};
    dm.align = align ? 1 : 0;
    dm.zero_list = zero_list ? 1 : 0;
    dm.combine = gather ? 1 : 0;
    dm.Ms = (int)Ms;
    dm.Nqs = (int)Nqs;
    ex.stamp(kStageCount, false, s);
    st = per_batch(B, gb * M, [&](int64_t b0, unsigned grid) {
        Dims d2 = dm;
        d2.b0 = (int)b0;
        if (few)
            hipLaunchKernelGGL((bin_count_kernel<VOL, kBinPPTSmall>), dim3(grid), dim3(kThreads),
                               4 * (size_t)hist_cap, s, shapes, starts, loc, w.counts, hist_cap,
                               d2);
        else
            hipLaunchKernelGGL((bin_count_kernel<VOL, kBinPPT>), dim3(grid), dim3(kThreads),
                               4 * (size_t)hist_cap, s, shapes, starts, loc, w.counts, hist_cap,
                               d2);
    });
    if (st != MSDA_OK) return st;
    ex.stamp(kStageCount, true, s);

    ex.stamp(kStageScan, false, s);
    // a workgroup per block of bins the bound allows; those past the used bins exit
    const unsigned scan_grid = (unsigned)((wl.bm_bins + kScanBlock - 1) / kScanBlock);
    hipLaunchKernelGGL(bin_scan_kernel<VOL>, dim3(scan_grid), dim3(kScanThreads), 0, s, shapes, starts,
                       w.counts, w.start, w.cursor, w.items, w.work_total, w.zero, w.split,
                       (int)B, dm);
    st = hip_status(hipGetLastError());
    if (st != MSDA_OK) return st;
    ex.stamp(kStageScan, true, s);

    ex.stamp(kStageScatter, false, s);
    st = per_batch(B, gb * M, [&](int64_t b0, unsigned grid) {
        Dims d2 = dm;
        d2.b0 = (int)b0;
        // the first launch zeroes every listed tile of the whole problem
        const ZeroList zl{(zero_list && !gather && b0 == 0) ? w.zero : nullptr, w.work_total,
                          gval, (int)D};
        if (few)
            hipLaunchKernelGGL((bin_scatter_kernel<VOL, kBinPPTSmall>), dim3(grid),
                               dim3(kThreads), 8 * (size_t)hist_cap, s, shapes, starts, loc, attn,
                               w.cursor, w.recs, hist_cap, zl, d2);
        else
            hipLaunchKernelGGL((bin_scatter_kernel<VOL, kBinPPT>), dim3(grid), dim3(kThreads),
                               8 * (size_t)hist_cap, s, shapes, starts, loc, attn, w.cursor,
                               w.recs, hist_cap, zl, d2);
    });
    if (st != MSDA_OK) return st;
    ex.stamp(kStageScatter, true, s);

    ex.stamp(kStageGather, false, s);
    st = hip_status(launch_grad_value<D, VOL>(wl, Nq, Ms, shapes, starts, gout, w, gval, dm, s));
    ex.stamp(kStageGather, true, s);
    return st;
}

// The grad_value pipeline over the whole problem in the passes of `pp`
// (pass_plan): boxes of pp.nb batches x pp.nm heads x pp.nq queries.  A pass
// is the problem restricted to its box -- the kernels address the tensors
// with the whole problem's strides (M heads, Nq queries per batch) from
// pointers to the box's first element, and the pass's bins are those of its
// (batch, head) pairs -- so it runs as a call of its own, reusing the
// workspace.  Boxes of different batches or heads write disjoint parts of
// grad_value; the boxes after the first of a query range add to it.  Passes
// are enqueued in order on s, which orders their use of the workspace.
// counts_clear: the first pass's bin counters are zero already (cleared by
// the kernel enqueued before it on s).
template <int D, bool VOL>
msda_status run_bins_passes(const int64_t *shapes, const int64_t *starts, const float *loc,
                            const float *attn, const float *gout, float *gval, int64_t B,
                            int64_t Nv, int64_t Nq, int64_t M, int64_t L, int64_t K,
                            const PassPlan &pp, unsigned char *ws, bool accumulate, bool align,
                            const Exec &ex, bool counts_clear = false) {
    const int64_t coords = VOL ? 3 : 2, LK = L * K;
    auto part = [](int64_t from, int64_t step, int64_t n) { return n - from < step ? n - from : step; };
    for (int64_t b0 = 0; b0 < B; b0 += pp.nb) {
        const int64_t nb = part(b0, pp.nb, B);
        for (int64_t m0 = 0; m0 < M; m0 += pp.nm) {
            const int64_t nm = part(m0, pp.nm, M);
            for (int64_t q0 = 0; q0 < Nq; q0 += pp.nq) {
                const int64_t nq = part(q0, pp.nq, Nq);
                const int64_t row = (b0 * Nq + q0) * M + m0;  // the box's first (query, head) row
                Exec ep = ex;
                ep.first = b0 == 0 && m0 == 0 && q0 == 0;
                ep.last = b0 + nb == B && m0 + nm == M && q0 + nq == Nq;
                const WorkLayout wl = nb == pp.nb && nm == pp.nm && nq == pp.nq
                                          ? pp.wl
                                          : work_layout(nb, Nv, nq, nm, L, K, VOL);
                const msda_status st = run_bins<D, VOL>(
                    shapes, starts, loc + coords * row * LK, attn + row * LK, gout + row * D,
                    gval + (b0 * Nv * M + m0) * D, nb, Nv, nq, nm, L, K, M, Nq, wl, ws,
                    accumulate || q0 > 0, align, ep, counts_clear && ep.first);
                if (st != MSDA_OK) return st;
            }
        }
    }
    return MSDA_OK;
}

}  // namespace

#endif  // MSDA_CSRC_BINS_H
