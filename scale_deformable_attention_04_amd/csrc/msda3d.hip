// msda3d.hip -- gfx950 kernels and C ABI of the 3-D (trilinear) variant of
// the sampling core: points on multi-level voxel volumes, eight neighbours
// per point ("Deformable attention: multi-scale sparse sampling and detection
// practice", section 5.3: the 2-D method with one more coordinate and
// trilinear instead of bilinear interpolation).  The operation, layouts and
// error behaviour are specified in include/msda.h.
//
// The kernels follow the 2-D ones: an item is one (batch, query, head) served
// by a group of D/4 lanes, each lane holding four channels of the head's row;
// per-point coordinate work is done once per point into LDS.
//
// Forward (msda3d_fwd_kernel): per item, the sum over its points of A times
// the trilinear sample, accumulated in registers, one store per item.
//
// Backward:
//   msda3d_dots_kernel (on the backward's side stream): per point, the eight
//      <grad_out row, neighbour row> dot products (DPP reductions over the
//      lane group) give grad_attn and the three location gradients.
//   grad_value, concurrently, by the binned pipeline of the 2-D core (bins.h)
//   with volume levels: a point's eight neighbours are the bilinear
//   neighbours of (x, y) in its two planes z0 and z0 + 1, so it becomes two
//   plane points of weights A (1 - fz) and A fz, whose records go to the 8x8
//   tiles of those planes; the tile kernel then sums every voxel in
//   registers, with no atomics except for tiles split over several work items.

#include "bins.h"

namespace {

constexpr int kVolTableBytes = 48 * 1024;  // per-workgroup budget for the point tables
constexpr int kDots3Grid = 512;            // workgroups of the dots kernel, at most

// Level table in LDS: lvl[l] = (Z, H, W, start); a level whose voxels do not
// fit inside value becomes (0, 0, 0, 0) and has no voxel.
struct VolumeLds {
    int4 lvl[kMaxLevels];
};

__device__ __forceinline__ void stage_volumes(VolumeLds *s, const int64_t *shapes,
                                              const int64_t *starts, int L, int Nv) {
    const int t = threadIdx.x;
    if (t < L) {
        const int64_t Z = shapes[3 * t], H = shapes[3 * t + 1], W = shapes[3 * t + 2];
        const int64_t S = starts[t];
        const bool dims_ok = Z >= 1 && H >= 1 && W >= 1 && Z <= Nv && H <= Nv && W <= Nv;
        const bool ok = dims_ok && S >= 0 && S <= Nv && H * W <= Nv && Z * (H * W) <= Nv - S;
        s->lvl[t] = ok ? make_int4((int)Z, (int)H, (int)W, (int)S) : make_int4(0, 0, 0, 0);
    }
    __syncthreads();
}

// d voxel / d normalized coordinate along an axis of n voxels.
__device__ __forceinline__ float voxel_scale(int n, bool align) {
    return align ? (float)(n - 1) : (float)n;
}

// The eight neighbours of a point, corner c = dx + 2 dy + 4 dz at
// (x0 + dx, y0 + dy, z0 + dz); rows outside the volume get the offset kOOB.
struct Corners {
    uint4 lo, hi;  // fp32-unit byte offsets of corners 0-3 and 4-7 in the batch slice
    float fx, fy, fz;
};

__device__ __forceinline__ Corners corners3(float u, float v, float w, int4 lvl,
                                            uint32_t row_stride, uint32_t head_off, bool align) {
    const int Z = lvl.x, H = lvl.y, W = lvl.z, S = lvl.w;
    const float off = align ? 0.f : -0.5f;
    // one rounding per coordinate, as the CPU check does
    const float x = __builtin_fmaf(u, voxel_scale(W, align), off);
    const float y = __builtin_fmaf(v, voxel_scale(H, align), off);
    const float z = __builtin_fmaf(w, voxel_scale(Z, align), off);
    const float x0 = floorf(x), y0 = floorf(y), z0 = floorf(z);
    Corners c;
    c.fx = x - x0;
    c.fy = y - y0;
    c.fz = z - z0;
    // NaN compares false: a non-finite coordinate leaves every corner out
    const bool vx0 = x0 >= 0.f && x0 <= (float)(W - 1), vx1 = x0 >= -1.f && x0 <= (float)(W - 2);
    const bool vy0 = y0 >= 0.f && y0 <= (float)(H - 1), vy1 = y0 >= -1.f && y0 <= (float)(H - 2);
    const bool vz0 = z0 >= 0.f && z0 <= (float)(Z - 1), vz1 = z0 >= -1.f && z0 <= (float)(Z - 2);
    // clamp before converting so that every input converts to a defined int
    const int xi = (int)fminf(fmaxf(x0, -1.f), (float)W);
    const int yi = (int)fminf(fmaxf(y0, -1.f), (float)H);
    const int zi = (int)fminf(fmaxf(z0, -1.f), (float)Z);
    const uint32_t o = (uint32_t)(S + (zi * H + yi) * W + xi) * row_stride + head_off;
    const uint32_t sx = row_stride, sy = (uint32_t)W * row_stride;
    const uint32_t sz = (uint32_t)(H * W) * row_stride;
    const bool z0v = vz0, z1v = vz1;
    c.lo.x = (vx0 && vy0 && z0v) ? o : kOOB;
    c.lo.y = (vx1 && vy0 && z0v) ? o + sx : kOOB;
    c.lo.z = (vx0 && vy1 && z0v) ? o + sy : kOOB;
    c.lo.w = (vx1 && vy1 && z0v) ? o + sx + sy : kOOB;
    c.hi.x = (vx0 && vy0 && z1v) ? o + sz : kOOB;
    c.hi.y = (vx1 && vy0 && z1v) ? o + sz + sx : kOOB;
    c.hi.z = (vx0 && vy1 && z1v) ? o + sz + sy : kOOB;
    c.hi.w = (vx1 && vy1 && z1v) ? o + sz + sx + sy : kOOB;
    return c;
}

// A times the trilinear weights of corners 0-3 (lo) and 4-7 (hi), exactly
// zero where the corner's offset is kOOB (so that a non-finite A or
// coordinate cannot leak through a corner outside the volume).
__device__ __forceinline__ void trilinear_weights(const Corners &c, float A, float4 &wlo,
                                                  float4 &whi) {
    const float gx = 1.f - c.fx, gy = 1.f - c.fy, gz = 1.f - c.fz;
    const float a = gx * gy, b = c.fx * gy, d = gx * c.fy, e = c.fx * c.fy;
    wlo = make_float4(c.lo.x != kOOB ? A * (a * gz) : 0.f, c.lo.y != kOOB ? A * (b * gz) : 0.f,
                      c.lo.z != kOOB ? A * (d * gz) : 0.f, c.lo.w != kOOB ? A * (e * gz) : 0.f);
    whi = make_float4(c.hi.x != kOOB ? A * (a * c.fz) : 0.f, c.hi.y != kOOB ? A * (b * c.fz) : 0.f,
                      c.hi.z != kOOB ? A * (d * c.fz) : 0.f, c.hi.w != kOOB ? A * (e * c.fz) : 0.f);
}

// True when at least one corner is inside (kOOB is the only offset with bit 31 set).
__device__ __forceinline__ bool any_corner(const Corners &c) {
    return ((c.lo.x & c.lo.y & c.lo.z & c.lo.w & c.hi.x & c.hi.y & c.hi.z & c.hi.w) & kOOB) == 0u;
}

struct Dims3 {
    int Nv, Nq, M, L, K;
    int PC;    // points per chunk of the point tables
    int PS;    // LDS stride per item (PC rounded to an odd count)
    int b0;    // first batch of this launch
    int nblk;  // workgroups per batch (forward) or per (batch, head) (backward)
    int align;
    int nblocks;  // query blocks of the launch (dots kernel, a persistent grid)
};

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <int D, typename VT>
__global__ void __launch_bounds__(kThreads)
msda3d_fwd_kernel(const VT *__restrict__ value, const int64_t *__restrict__ shapes,
                  const int64_t *__restrict__ starts, const float *__restrict__ loc,
                  const float *__restrict__ attn, float *__restrict__ out, Dims3 dm) {
    constexpr int G = D / 4;
    constexpr int IPB = kThreads / G;
    __shared__ VolumeLds s_lv;
    extern __shared__ __align__(16) unsigned char smem[];
    uint4 *s_off = reinterpret_cast<uint4 *>(smem);                  // [IPB][PS][2]
    float4 *s_w = reinterpret_cast<float4 *>(s_off + 2 * IPB * dm.PS);  // [IPB][PS][2]

    const int M = dm.M, K = dm.K, LK = dm.L * dm.K;
    const int NqM = dm.Nq * M;
    const int wg = xcd_contiguous(blockIdx.x, gridDim.x);
    const int b = wg / dm.nblk + dm.b0;
    const int item0 = (wg % dm.nblk) * IPB;
    const int nitems = min(IPB, NqM - item0);
    const uint32_t row_stride = (uint32_t)M * D * 4u;
    stage_volumes(&s_lv, shapes, starts, dm.L, dm.Nv);

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
            const float A = attn[p];
            const int m = (item0 + i1) % M;
            const Corners cn = corners3(loc[3 * p], loc[3 * p + 1], loc[3 * p + 2],
                                        s_lv.lvl[j / K], row_stride, (uint32_t)m * D * 4u,
                                        dm.align);
            float4 wlo, whi;
            trilinear_weights(cn, A, wlo, whi);
            const int e = 2 * (i1 * dm.PS + jj);
            s_off[e] = cn.lo;
            s_off[e + 1] = cn.hi;
            s_w[e] = wlo;
            s_w[e + 1] = whi;
        }
        __syncthreads();
        if (it < nitems) {
            const int base = 2 * it * dm.PS;
#pragma unroll 2
            for (int jj = 0; jj < pc; ++jj) {
                const uint4 lo = s_off[base + 2 * jj], hi = s_off[base + 2 * jj + 1];
                const float4 wl = s_w[base + 2 * jj], wh = s_w[base + 2 * jj + 1];
                const float4 v0 = Row4<VT>::load(vr, lo.x, 4 * c);
                const float4 v1 = Row4<VT>::load(vr, lo.y, 4 * c);
                const float4 v2 = Row4<VT>::load(vr, lo.z, 4 * c);
                const float4 v3 = Row4<VT>::load(vr, lo.w, 4 * c);
                const float4 v4 = Row4<VT>::load(vr, hi.x, 4 * c);
                const float4 v5 = Row4<VT>::load(vr, hi.y, 4 * c);
                const float4 v6 = Row4<VT>::load(vr, hi.z, 4 * c);
                const float4 v7 = Row4<VT>::load(vr, hi.w, 4 * c);
                fma4(acc, wl.x, v0);
                fma4(acc, wl.y, v1);
                fma4(acc, wl.z, v2);
                fma4(acc, wl.w, v3);
                fma4(acc, wh.x, v4);
                fma4(acc, wh.y, v5);
                fma4(acc, wh.z, v6);
                fma4(acc, wh.w, v7);
            }
        }
    }
    if (it < nitems) {
        float4 *o = reinterpret_cast<float4 *>(out + ((size_t)b * NqM + item0 + it) * D) + c;
        *o = acc;
    }
}

// ---------------------------------------------------------------------------
// backward: grad_attn_weight and grad_sampling_loc.  Workgroup = (batch b,
// head m, IPB consecutive queries).  Per point the table holds the eight row
// offsets (later overwritten by the eight dot products) and (fx, fy, fz, A).
// ---------------------------------------------------------------------------
template <int D, typename VT>
__global__ void __launch_bounds__(kThreads)
msda3d_dots_kernel(const VT *__restrict__ value, const int64_t *__restrict__ shapes,
                   const int64_t *__restrict__ starts, const float *__restrict__ loc,
                   const float *__restrict__ attn, const float *__restrict__ grad_out,
                   float *__restrict__ grad_loc, float *__restrict__ grad_attn, Dims3 dm) {
    constexpr int G = D / 4;
    constexpr int IPB = kThreads / G;
    __shared__ VolumeLds s_lv;
    extern __shared__ __align__(16) unsigned char smem[];
    uint4 *s_off = reinterpret_cast<uint4 *>(smem);                     // [IPB][PS][2]
    float4 *s_aux = reinterpret_cast<float4 *>(s_off + 2 * IPB * dm.PS);  // [IPB][PS]

    const int M = dm.M, K = dm.K, LK = dm.L * dm.K, Nq = dm.Nq;
    stage_volumes(&s_lv, shapes, starts, dm.L, dm.Nv);
    // blocks of IPB queries of one (batch, head); workgroup g takes blocks g,
    // g + grid, ... (a few workgroups per CU leave room for the grad_value
    // kernels running beside this one)
    for (int blk = blockIdx.x; blk < dm.nblocks; blk += gridDim.x) {
    if (blk != (int)blockIdx.x) __syncthreads();  // the point tables are reused
    const int wg = xcd_contiguous(blk, dm.nblocks);
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
    // the grad_out row through a buffer load (see the 2-D dots kernel)
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
            const Corners cn = corners3(loc[3 * p], loc[3 * p + 1], loc[3 * p + 2],
                                        s_lv.lvl[j / K], row_stride, head_off, dm.align);
            const int e = i1 * dm.PS + jj;
            s_off[2 * e] = cn.lo;
            s_off[2 * e + 1] = cn.hi;
            // a point with no corner inside gets zero gradients: keep its
            // (possibly non-finite) fractions out of the arithmetic
            s_aux[e] = any_corner(cn) ? make_float4(cn.fx, cn.fy, cn.fz, attn[p])
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        __syncthreads();
        if (it < nitems) {
            for (int jj = 0; jj < pc; ++jj) {
                const int e = it * dm.PS + jj;
                const uint4 lo = s_off[2 * e], hi = s_off[2 * e + 1];
                const float4 v0 = Row4<VT>::load(vr, lo.x, 4 * c);
                const float4 v1 = Row4<VT>::load(vr, lo.y, 4 * c);
                const float4 v2 = Row4<VT>::load(vr, lo.z, 4 * c);
                const float4 v3 = Row4<VT>::load(vr, lo.w, 4 * c);
                const float4 v4 = Row4<VT>::load(vr, hi.x, 4 * c);
                const float4 v5 = Row4<VT>::load(vr, hi.y, 4 * c);
                const float4 v6 = Row4<VT>::load(vr, hi.z, 4 * c);
                const float4 v7 = Row4<VT>::load(vr, hi.w, 4 * c);
                const float d0 = group_sum<G>(dot4(g4, v0)), d1 = group_sum<G>(dot4(g4, v1));
                const float d2 = group_sum<G>(dot4(g4, v2)), d3 = group_sum<G>(dot4(g4, v3));
                const float d4 = group_sum<G>(dot4(g4, v4)), d5 = group_sum<G>(dot4(g4, v5));
                const float d6 = group_sum<G>(dot4(g4, v6)), d7 = group_sum<G>(dot4(g4, v7));
                // the group's lanes are one wave: all have read the offsets
                if (c == 0) {
                    s_off[2 * e] = make_uint4(__float_as_uint(d0), __float_as_uint(d1),
                                              __float_as_uint(d2), __float_as_uint(d3));
                    s_off[2 * e + 1] = make_uint4(__float_as_uint(d4), __float_as_uint(d5),
                                                  __float_as_uint(d6), __float_as_uint(d7));
                }
            }
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < nitems * pc; idx += kThreads) {
            const int i1 = idx / pc, jj = idx - i1 * pc, j = j0 + jj;
            const size_t p = pt0 + (size_t)i1 * M * LK + j;
            const int e = i1 * dm.PS + jj;
            const uint4 dl = s_off[2 * e], dh = s_off[2 * e + 1];
            const float4 ax = s_aux[e];
            const int4 lvl = s_lv.lvl[j / K];
            // outside corners read zero rows, so their dot products are 0
            const float d0 = __uint_as_float(dl.x), d1 = __uint_as_float(dl.y);
            const float d2 = __uint_as_float(dl.z), d3 = __uint_as_float(dl.w);
            const float d4 = __uint_as_float(dh.x), d5 = __uint_as_float(dh.y);
            const float d6 = __uint_as_float(dh.z), d7 = __uint_as_float(dh.w);
            const float fx = ax.x, fy = ax.y, fz = ax.z, A = ax.w;
            const float gx = 1.f - fx, gy = 1.f - fy, gz = 1.f - fz;
            float ga = 0.f, lx = 0.f, ly = 0.f, lz = 0.f;
            if (lvl.z > 0) {
                ga = gz * (gy * (gx * d0 + fx * d1) + fy * (gx * d2 + fx * d3)) +
                     fz * (gy * (gx * d4 + fx * d5) + fy * (gx * d6 + fx * d7));
                lx = A * voxel_scale(lvl.z, dm.align) *
                     (gz * (gy * (d1 - d0) + fy * (d3 - d2)) +
                      fz * (gy * (d5 - d4) + fy * (d7 - d6)));
                ly = A * voxel_scale(lvl.y, dm.align) *
                     (gz * (gx * (d2 - d0) + fx * (d3 - d1)) +
                      fz * (gx * (d6 - d4) + fx * (d7 - d5)));
                lz = A * voxel_scale(lvl.x, dm.align) *
                     (gy * (gx * (d4 - d0) + fx * (d5 - d1)) +
                      fy * (gx * (d6 - d2) + fx * (d7 - d3)));
            }
            grad_attn[p] = ga;
            grad_loc[3 * p] = lx;
            grad_loc[3 * p + 1] = ly;
            grad_loc[3 * p + 2] = lz;
        }
    }
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
using msda_host::check_sizes3;

struct Plan3 {
    int ipb, pc, ps;
    size_t lds;
};

Plan3 plan3(int64_t D, int64_t L, int64_t K, int bytes_per_point) {
    Plan3 p;
    p.ipb = (int)(kThreads / (D / 4));
    const int lk = (int)(L * K);
    int pc = kVolTableBytes / (p.ipb * bytes_per_point) - 2;
    pc = pc < 1 ? 1 : pc;
    p.pc = pc < lk ? pc : lk;
    p.ps = p.pc + ((p.pc % 2 == 0) ? 1 : 2);
    p.lds = (size_t)p.ipb * p.ps * bytes_per_point;
    return p;
}

template <int D, typename VT>
msda_status launch3_fwd(const void *value, const int64_t *shapes, const int64_t *starts,
                        const float *loc, const float *attn, float *out, int64_t B, int64_t Nv,
                        int64_t Nq, int64_t M, int64_t L, int64_t K, bool align, hipStream_t s) {
    const Plan3 p = plan3(D, L, K, 64);
    const int64_t gx = (Nq * M + p.ipb - 1) / p.ipb;
    const int64_t bchunk = batch_chunk(gx, B);
    for (int64_t b0 = 0; b0 < B; b0 += bchunk) {
        const int64_t nb = (B - b0) < bchunk ? (B - b0) : bchunk;
        const Dims3 dm{(int)Nv, (int)Nq, (int)M, (int)L, (int)K, p.pc, p.ps, (int)b0, (int)gx,
                       align ? 1 : 0};
        hipLaunchKernelGGL((msda3d_fwd_kernel<D, VT>), dim3((unsigned)(gx * nb)), dim3(kThreads),
                           p.lds, s, static_cast<const VT *>(value), shapes, starts, loc, attn,
                           out, dm);
        const msda_status st = hip_status(hipGetLastError());
        if (st != MSDA_OK) return st;
    }
    return MSDA_OK;
}

template <int D, typename VT>
msda_status launch3_bwd(const void *value, const int64_t *shapes, const int64_t *starts,
                        const float *loc, const float *attn, const float *gout, float *gval,
                        float *gloc, float *gattn, int64_t B, int64_t Nv, int64_t Nq, int64_t M,
                        int64_t L, int64_t K, bool align, bool accumulate, const PassPlan &pp,
                        unsigned char *ws, const Exec &ex) {
    // grad_attn_weight and grad_sampling_loc on the side stream (when there is one)
    const hipStream_t ds = ex.dots_stream();
    const Plan3 p = plan3(D, L, K, 48);
    const int64_t gq = (Nq + p.ipb - 1) / p.ipb;
    msda_status st = per_batch(B, gq * M, [&](int64_t b0, unsigned grid) {
        const Dims3 dm{(int)Nv, (int)Nq, (int)M, (int)L, (int)K, p.pc, p.ps, (int)b0, (int)gq,
                       align ? 1 : 0, (int)grid};
        const unsigned g = grid > (unsigned)kDots3Grid ? (unsigned)kDots3Grid : grid;
        hipLaunchKernelGGL((msda3d_dots_kernel<D, VT>), dim3(g), dim3(kThreads), p.lds, ds,
                           static_cast<const VT *>(value), shapes, starts, loc, attn, gout, gloc,
                           gattn, dm);
    });
    if (st != MSDA_OK) return st;
    // grad_value: the binned pipeline over volume levels
    return run_bins_passes<D, true>(shapes, starts, loc, attn, gout, gval, B, Nv, Nq, M, L, K,
                                    pp, ws, accumulate, align, ex);
}

#define MSDA3D_DISPATCH(FN, VT, ...)                                                           \
    switch (D) {                                                                               \
    case 4: return FN<4, VT>(__VA_ARGS__);                                                     \
    case 8: return FN<8, VT>(__VA_ARGS__);                                                     \
    case 16: return FN<16, VT>(__VA_ARGS__);                                                   \
    case 32: return FN<32, VT>(__VA_ARGS__);                                                   \
    case 64: return FN<64, VT>(__VA_ARGS__);                                                   \
    case 128: return FN<128, VT>(__VA_ARGS__);                                                 \
    case 256: return FN<256, VT>(__VA_ARGS__);                                                 \
    default: return MSDA_ERR_UNSUPPORTED;                                                      \
    }

template <typename VT>
msda_status dispatch3_fwd(int64_t D, const void *value, const int64_t *shapes,
                          const int64_t *starts, const float *loc, const float *attn, float *out,
                          int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t L, int64_t K,
                          bool align, hipStream_t s) {
    MSDA3D_DISPATCH(launch3_fwd, VT, value, shapes, starts, loc, attn, out, B, Nv, Nq, M, L, K,
                    align, s)
}

template <typename VT>
msda_status dispatch3_bwd(int64_t D, const void *value, const int64_t *shapes,
                          const int64_t *starts, const float *loc, const float *attn,
                          const float *gout, float *gval, float *gloc, float *gattn, int64_t B,
                          int64_t Nv, int64_t Nq, int64_t M, int64_t L, int64_t K, bool align,
                          bool acc, const PassPlan &pp, unsigned char *ws, const Exec &ex) {
    MSDA3D_DISPATCH(launch3_bwd, VT, value, shapes, starts, loc, attn, gout, gval, gloc, gattn,
                    B, Nv, Nq, M, L, K, align, acc, pp, ws, ex)
}

#undef MSDA3D_DISPATCH

}  // namespace

extern "C" {

msda_status msda3d_forward(const void *value, int value_dtype, const int64_t *volume_shapes,
                           const int64_t *level_start_index, const float *sampling_loc,
                           const float *attn_weight, float *out, int64_t B, int64_t Nv,
                           int64_t Nq, int64_t M, int64_t D, int64_t L, int64_t K,
                           uint32_t flags, void *stream) {
    msda_status st = check_sizes3(value_dtype, B, Nv, Nq, M, D, L, K);
    if (st != MSDA_OK) return st;
    if (flags & ~MSDA_ALIGN_CORNERS) return MSDA_ERR_UNSUPPORTED;
    const bool align = (flags & MSDA_ALIGN_CORNERS) != 0;
    if (B == 0 || Nq == 0) return MSDA_OK;
    if (Nv < 1) return MSDA_ERR_SHAPE;
    if (!value || !volume_shapes || !level_start_index || !sampling_loc || !attn_weight || !out)
        return MSDA_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (value_dtype == MSDA_F32)
        return dispatch3_fwd<float>(D, value, volume_shapes, level_start_index, sampling_loc,
                                    attn_weight, out, B, Nv, Nq, M, L, K, align, s);
    return dispatch3_fwd<uint16_t>(D, value, volume_shapes, level_start_index, sampling_loc,
                                   attn_weight, out, B, Nv, Nq, M, L, K, align, s);
}


msda_status msda3d_backward(const void *value, int value_dtype, const int64_t *volume_shapes,
                            const int64_t *level_start_index, const float *sampling_loc,
                            const float *attn_weight, const float *grad_out, float *grad_value,
                            float *grad_sampling_loc, float *grad_attn_weight, int64_t B,
                            int64_t Nv, int64_t Nq, int64_t M, int64_t D, int64_t L, int64_t K,
                            void *workspace, size_t workspace_bytes, uint32_t flags,
                            void *stream, void *side_stream, void *const *side_events) {
    msda_status st = check_sizes3(value_dtype, B, Nv, Nq, M, D, L, K);
    if (st != MSDA_OK) return st;
    if (flags & ~(MSDA_BWD_ACCUMULATE | MSDA_ALIGN_CORNERS)) return MSDA_ERR_UNSUPPORTED;
    // a grad_value record stores the query index in 25 bits
    if (Nq > ((int64_t)1 << (32 - kRecQueryShift))) return MSDA_ERR_UNSUPPORTED;
    const int64_t nval = B * Nv * M * D;
    if (nval > 0 && !grad_value) return MSDA_ERR_NULL;
    const bool work = B > 0 && Nq > 0;
    PassPlan pp{};
    if (work) {
        if (Nv < 1) return MSDA_ERR_SHAPE;
        if (!value || !volume_shapes || !level_start_index || !sampling_loc || !attn_weight ||
            !grad_out || !grad_sampling_loc || !grad_attn_weight)
            return MSDA_ERR_NULL;
        if (!workspace) return MSDA_ERR_NULL;
        // the grad_value pipeline in as few passes as the workspace allows
        pp = pass_plan(B, Nv, Nq, M, L, K, true, workspace_bytes);
        if (pp.nb == 0) return MSDA_ERR_WORKSPACE;
        if (pp.wl.bm_bins >= ((int64_t)1 << 31) || pp.wl.work_max >= ((int64_t)1 << 31) ||
            pp.wl.sorted_max >= ((int64_t)1 << 32))
            return MSDA_ERR_UNSUPPORTED;
        if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return MSDA_ERR_WORKSPACE;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    Exec ex{s, nullptr, nullptr, nullptr, nullptr};
    st = exec_side(ex, side_stream, side_events);
    if (st != MSDA_OK) return st;
    const bool acc = (flags & MSDA_BWD_ACCUMULATE) != 0;
    if (!work) return acc ? MSDA_OK : fill_zero(grad_value, (size_t)nval / 4, s);  // D % 4 == 0
    st = exec_fork(ex, B * Nq * M * L * K);
    if (st != MSDA_OK) return st;
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    const bool align = (flags & MSDA_ALIGN_CORNERS) != 0;
    if (value_dtype == MSDA_F32)
        st = dispatch3_bwd<float>(D, value, volume_shapes, level_start_index, sampling_loc,
                                  attn_weight, grad_out, grad_value, grad_sampling_loc,
                                  grad_attn_weight, B, Nv, Nq, M, L, K, align, acc, pp, ws, ex);
    else
        st = dispatch3_bwd<uint16_t>(D, value, volume_shapes, level_start_index, sampling_loc,
                                     attn_weight, grad_out, grad_value, grad_sampling_loc,
                                     grad_attn_weight, B, Nv, Nq, M, L, K, align, acc, pp, ws,
                                     ex);
    const msda_status js = exec_join(ex);
    return st != MSDA_OK ? st : js;
}

}  // extern "C"
