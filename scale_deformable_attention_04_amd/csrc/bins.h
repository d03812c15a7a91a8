// bins.h -- the binned, atomic-free grad_value pipeline of the backward
// (count -> scan -> scatter -> tile kernels) and the point geometry it shares
// with the sampling kernels: level tables in LDS, the bilinear neighbours of
// a point, the tiles they touch.  Included by the translation units of
// libmsda.so; everything has internal linkage except the per-device side
// stream (msda_side), of which there is one per process.
#ifndef MSDA_CSRC_BINS_H
#define MSDA_CSRC_BINS_H

#include <mutex>
#include <type_traits>

#include "common.h"

// One side stream per device, created on first use (default priority,
// non-blocking with respect to the null stream), shared by every backward
// of the library.  The mutex is held while a backward enqueues, so the fork /
// join events are never shared between two calls in flight on the host.
namespace msda_side {
constexpr int kMaxDevices = 64;
struct SideStream {
    bool tried = false;
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, filled = nullptr, join = nullptr;
};
std::mutex &mutex();
// Call with mutex() held.  nullptr when no side stream can be had.
SideStream *get();
}  // namespace msda_side

namespace {

constexpr int kTileShift = 3;              // grad_value tiles of 8x8 pixels
constexpr int kTile = 1 << kTileShift;
constexpr int kTilePx = kTile * kTile;
constexpr int kChunk = 2048;               // points per grad_value work item, at most
constexpr int kHistLds = 4096;             // bins of one (batch, head) kept in an LDS histogram
constexpr int kScanThreads = 1024;
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
// ---------------------------------------------------------------------------
// backward: points per bin
// Workgroup = (batch b, head m, kBinPoints consecutive points of the
// (b, m) list in (query, level, point) order), kBinPPT points per thread,
// all of whose coordinates are loaded before any is used.
// ---------------------------------------------------------------------------
constexpr int kBinPPT = 16;
constexpr int kBinPoints = kBinPPT * kThreads;

// VOL: volume levels; a location is (u, v, w) and a point feeds the tiles of
// its two planes.
template <bool VOL>
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
    float wz[kBinPPT];  // VOL: the z coordinate
#pragma unroll
    for (int r = 0; r < kBinPPT; ++r) {
        const int f = f0 + threadIdx.x + r * kThreads;
        uv[r] = make_float2(0.f, 0.f);
        wz[r] = 0.f;
        if (f < nf) {
            const int q = (int)fdiv((uint32_t)f, dm.div_lk), j = f - q * LK;
            const size_t p = (row0 + (size_t)q * M) * LK + j;
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
    for (int r = 0; r < kBinPPT; ++r) {
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

template <bool VOL>
__global__ void __launch_bounds__(kScanThreads)
bin_scan_kernel(const int64_t *__restrict__ shapes, const int64_t *__restrict__ starts,
                const uint32_t *__restrict__ counts, uint32_t *__restrict__ start,
                uint32_t *__restrict__ cursor, uint4 *__restrict__ items,
                uint32_t *__restrict__ work_total, int B, Dims dm) {
    constexpr int kPer = 8;
    __shared__ LevelLds s_lv;
    __shared__ uint2 s_wave[kScanThreads / 64 + 1];
    stage_bin_levels<VOL>(&s_lv, shapes, starts, dm.L, dm.Nv, dm.nb_max);
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
        // a rolled loop: this kernel is one workgroup on the critical path,
        // and its instruction fetches are not hidden by other waves
#pragma unroll 1
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

template <bool VOL>
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
    float wz[kBinPPT];  // VOL: the z coordinate
#pragma unroll
    for (int r = 0; r < kBinPPT; ++r) {
        const int f = f0 + threadIdx.x + r * kThreads;
        uv[r] = make_float2(0.f, 0.f);
        aw[r] = 0.f;
        wz[r] = 0.f;
        if (f < nf) {
            const int q = (int)fdiv((uint32_t)f, dm.div_lk), j = f - q * LK;
            const size_t p = (row0 + (size_t)q * M) * LK + j;
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
    for (int r = 0; r < kBinPPT; ++r) {
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
                pull_range<kQuads>(acc[o], wP, gP + q, (int)stP[cT], (int)stP[cT + 1],
                                   (int)stP[cT + 2], 1, 0);
                pull_range<kQuads>(acc[o], wP, gP + q, (int)stP[cB], (int)stP[cB + 1],
                                   (int)stP[cB + 2], 3, 2);
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
                int rel = lb - lvl.w;
                int plane0 = lvl.z;  // first row of the tile's map (volumes: of its plane)
                if constexpr (VOL) {
                    const int zpl = rel / s_lv.tpp[l];
                    rel -= zpl * s_lv.tpp[l];
                    plane0 += zpl * lvl.x * lvl.y;
                }
                const int ty = rel / tw, tx = rel - ty * tw;
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
                    float *dst = gv + (size_t)(plane0 + gy * lvl.y + gx) * M * D + 4 * q;
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

template <int CPL> constexpr int gather_threads() { return kCells * (kGatherMaxD / CPL); }

template <int D, bool VOL, int CPL>
__global__ void __launch_bounds__(gather_threads<CPL>())
grad_value_gather_kernel(const int64_t *__restrict__ shapes, const int64_t *__restrict__ starts,
                         const float *__restrict__ grad_out, const uint4 *__restrict__ items,
                         const uint32_t *__restrict__ work_total, const uint4 *__restrict__ recs,
                         float *__restrict__ grad_value, Dims dm) {
    static_assert(D <= kGatherMaxD && D % 4 == 0, "one (cell, channel group) pair per lane");
    constexpr int kT = gather_threads<CPL>();
    constexpr int kQuads = D / 4;
    constexpr int kQPL = (CPL < D ? CPL : D) / 4;  // quads per lane
    constexpr int kGroups = kQuads / kQPL;          // lanes per cell
    constexpr int kPairs = kCells * kGroups;
    constexpr int kPer = (kChunk + kT - 1) / kT;     // records per thread in the sort
    static_assert(kPairs <= kT, "every (cell, channel group) pair has a lane");
    static_assert(4 * kTilePx * kQuads <= kChunk, "the role sums fit the record table");
    __shared__ LevelLds s_lv;
    __shared__ uint32_t s_cnt[kCells];     // records per cell
    __shared__ uint32_t s_st[kCells + 1];  // first sorted slot of each cell, and the total
    __shared__ uint4 s_tab[kChunk];        // the item's records in cell order
    // after the gather, the role sums: [role][pixel][quad]
    float4 *s_red = reinterpret_cast<float4 *>(s_tab);

    const int M = dm.M, Nq = dm.Nq;
    const int tid = threadIdx.x;
    const uint32_t total = *work_total;
    if (blockIdx.x >= total) return;  // the grid is sized for the largest possible list
    stage_bin_levels<VOL>(&s_lv, shapes, starts, dm.L, dm.Nv, dm.nb_max);
    if (tid < kCells) s_cnt[tid] = 0u;

    const bool owner = tid < kPairs;
    const int cell = tid / kGroups, grp = tid - cell * kGroups;
    const int cx = cell % kCellsW, cy = cell / kCellsW;
    const uint32_t row_stride = (uint32_t)M * D * 4u;
    // one batch of grad_out; the host keeps it below 2^32 bytes, and an
    // offset of `slice` reads zeros (outside the descriptor's range)
    const uint32_t slice = (uint32_t)((size_t)Nq * M * D * 4);
    __syncthreads();

    // Workgroup g takes items g, g + grid, ... counted from the end of the
    // list (the coarse levels' bins, the largest, first).  The list is in
    // (batch, level, tile, head) order, so with 8 heads the workgroups of
    // one XCD (g % 8) mostly see one head, whose grad_out rows stay in that L2.
    for (uint32_t w = blockIdx.x; w < total; w += gridDim.x) {
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
            const rsrc_t go = make_rsrc(grad_out + (size_t)b * Nq * M * D, slice);
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
                        s_red[(r * kTilePx + py * kTile + px) * kQuads + grp * kQPL + k] =
                            acc[r][k];
                }
            }
        }
        __syncthreads();
        // 5. write the tile: pixel = the four roles' sums
        const int lb = (int)(bt - (uint32_t)b * dm.nb_max);
        int l = 0;
        while (l + 1 < dm.L && s_lv.lvl[l + 1].w <= lb) ++l;
        const int4 lvl = s_lv.lvl[l];
        const int tw = s_lv.tw[l];
        int rel = lb - lvl.w;
        int plane0 = lvl.z;  // first row of the tile's map (volumes: of its plane)
        if constexpr (VOL) {
            const int zpl = rel / s_lv.tpp[l];
            rel -= zpl * s_lv.tpp[l];
            plane0 += zpl * lvl.x * lvl.y;
        }
        const int ty = rel / tw, tx = rel - ty * tw;
        const size_t slice_v = (size_t)dm.Nv * M * D;
        float *gv = grad_value + (size_t)b * slice_v + (size_t)m * D;
        for (int i = tid; i < kTilePx * kQuads; i += kT) {
            const int px = i / kQuads, q = i - px * kQuads;
            float4 a = s_red[px * kQuads + q];
#pragma unroll
            for (int r = 1; r < 4; ++r) {
                const float4 v = s_red[(r * kTilePx + px) * kQuads + q];
                a.x += v.x;
                a.y += v.y;
                a.z += v.z;
                a.w += v.w;
            }
            const int gx = tx * kTile + (px & (kTile - 1));
            const int gy = ty * kTile + (px >> kTileShift);
            if (gy >= lvl.x || gx >= lvl.y) continue;
            float *dst = gv + (size_t)(plane0 + gy * lvl.y + gx) * M * D + 4 * q;
            if (it.w) {
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
        // the next item's first barrier orders these reads of s_red before
        // its records overwrite the table
    }
}

// The grad_value stage: the gather kernel for heads of up to kGatherMaxD
// channels whose grad_out batch is 32-bit addressable, else the tile kernel.
template <int D, bool VOL>
hipError_t launch_grad_value(int64_t work_max, int64_t Nq, int64_t M, const int64_t *shapes,
                             const int64_t *starts, const float *gout, const uint4 *items,
                             const uint32_t *work_total, const uint4 *recs, float *gval,
                             const Dims &dm, hipStream_t s) {
    const int64_t grid = work_max < kTileGrid ? work_max : kTileGrid;
    if constexpr (D <= kGatherMaxD) {
        if (Nq * M * D * 4 < ((int64_t)1 << 32) - 64) {
            hipLaunchKernelGGL((grad_value_gather_kernel<D, VOL, kGatherCPL>),
                               dim3((unsigned)grid), dim3(gather_threads<kGatherCPL>()), 0, s,
                               shapes, starts, gout, items, work_total, recs, gval, dm);
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
// Upper bound of the number of 8x8 tiles over all levels, from Nv and L only:
// sum ceil(H/8)*ceil(W/8) <= sum (HW + 7(H+W) + 49)/64 <= (15 Nv + 49 L)/64.
int64_t bins_bound(int64_t Nv, int64_t L) { return (15 * Nv + 49 * L) / 64 + 1; }

struct WorkLayout {
    int64_t nb_max, bm_bins, work_max, sorted_max;
    size_t off_counts, off_start, off_cursor, off_items, off_total, off_sorted, bytes;
};

// The workspace of the pipeline.  2-D levels (vol = false): at most four
// records per point and bins_bound(Nv, L) bins per (batch, head).  Volumes:
// two planes of four tiles, so eight records per point, and at most one bin
// per voxel (every tile of a plane holds a voxel).
WorkLayout work_layout(int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t L, int64_t K,
                       bool vol = false) {
    WorkLayout w;
    w.nb_max = vol ? Nv + 1 : bins_bound(Nv, L);
    w.bm_bins = B * M * w.nb_max;
    const int64_t pts = B * Nq * M * L * K;
    w.sorted_max = (vol ? 8 : 4) * pts;
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

FastDiv make_fastdiv(uint32_t d) {  // d >= 1
    uint32_t shift = 0;
    while (shift < 31 && (1u << shift) < d) ++shift;
    const uint64_t mul = ((uint64_t)1 << 32) * (((uint64_t)1 << shift) - d) / d + 1;
    return FastDiv{(uint32_t)mul, shift};
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

}  // namespace

#endif  // MSDA_CSRC_BINS_H
