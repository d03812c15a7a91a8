// msda.hip -- gfx950 (MI355X, CDNA4) kernels and C ABI of the multi-scale
// deformable attention (MSDeformAttn) sampling core.  The operation, layouts
// and error behaviour are specified in include/msda.h.
//
// Work decomposition (both passes).  An "item" is one (batch, query, head);
// it owns L*K sampling points and D output channels.  A group of G = D/4
// lanes serves one item, lane c holding channels 4c..4c+3, so every
// neighbour fetch of a point is one coalesced read of the head's row of D
// values (16 bytes per lane for fp32, 8 for bf16).  A 256-thread workgroup
// serves IPB = 256/G consecutive items of one batch and walks their points in
// chunks:
//   phase 1  one thread per point: pixel coordinate, floor, the four
//            neighbours' row offsets and bilinear weights, into LDS;
//   phase 2  one lane group per item: fetch the four rows of every point and
//            accumulate (forward), or form the four <grad_out, row> dot
//            products, reduce them across the group with DPP, and scatter
//            A*w*grad_out into grad_value with fp32 atomics (backward);
//   phase 3  (backward) one thread per point: grad_attn_weight and
//            grad_sampling_loc from the reduced dot products.
// so the per-point coordinate work is done once per point rather than once
// per lane.
//
// value and grad_value are addressed through raw buffer descriptors whose
// size is the batch slice.  A neighbour outside the map gets the offset
// kOOB, beyond every slice, so its fetch returns zeros and its atomic is
// dropped by the hardware range check instead of needing a branch.  The same
// check keeps an inconsistent level table from touching other memory.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msda.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxLevels = 16;
constexpr uint32_t kOOB = 0x80000000u;     // byte offset past every slice (slices < 2^31 B)
constexpr int kRsrcWord3 = 0x00020000;     // gfx9 buffer descriptor word 3 (raw, 32-bit data)
constexpr int kSetupLdsBytes = 36 * 1024;  // per-workgroup budget for the point tables

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

__device__ __forceinline__ void atomic_add(rsrc_t r, uint32_t off, float v) {
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(v, r, (int)off, 0, 0);
}

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

// Level table entry staged in LDS: (H, W, start, 0).  A level whose pixels do
// not fit inside value becomes (0, 0, 0, 0), which puts every neighbour
// outside the map.
__device__ __forceinline__ void stage_levels(int4 *s_lvl, const int64_t *shapes,
                                             const int64_t *starts, int L, int Nv) {
    const int t = threadIdx.x;
    if (t < L) {
        const int64_t H = shapes[2 * t], W = shapes[2 * t + 1], S = starts[t];
        const bool ok = H >= 1 && W >= 1 && H <= Nv && W <= Nv && S >= 0 && S <= Nv &&
                        H * W <= (int64_t)Nv - S;
        s_lvl[t] = ok ? make_int4((int)H, (int)W, (int)S, 0) : make_int4(0, 0, 0, 0);
    }
}

// Neighbours of one sampling point, in the order TL (x0,y0), TR (x0+1,y0),
// BL (x0,y0+1), BR (x0+1,y0+1).
struct Neighbours {
    uint4 off;       // fp32-unit byte offsets of the rows in the batch slice, or kOOB
    float4 w;        // bilinear weights, 0 outside the map
    float fx, fy;    // fractional parts of the pixel coordinate
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
    const int xi = (int)fminf(fmaxf(x0, -1.f), (float)W);
    const int yi = (int)fminf(fmaxf(y0, -1.f), (float)H);
    const int pTL = S + yi * W + xi;
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

__device__ __forceinline__ void fma4(float4 &acc, float w, const float4 &v) {
    acc.x = __builtin_fmaf(w, v.x, acc.x);
    acc.y = __builtin_fmaf(w, v.y, acc.y);
    acc.z = __builtin_fmaf(w, v.z, acc.z);
    acc.w = __builtin_fmaf(w, v.w, acc.w);
}

__device__ __forceinline__ float dot4(const float4 &a, const float4 &b) {
    return __builtin_fmaf(a.w, b.w, __builtin_fmaf(a.z, b.z, __builtin_fmaf(a.y, b.y, a.x * b.x)));
}

struct Dims {
    int Nv, Nq, M, L, K;
    int PC;   // points per chunk
    int PS;   // LDS stride per item (PC rounded to an odd count, for bank spread)
    int b0;   // first batch of this launch
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
    extern __shared__ __align__(16) unsigned char smem[];
    int4 *s_lvl = reinterpret_cast<int4 *>(smem);
    uint4 *s_off = reinterpret_cast<uint4 *>(smem + kMaxLevels * sizeof(int4));
    float4 *s_w = reinterpret_cast<float4 *>(s_off + IPB * dm.PS);

    const int M = dm.M, K = dm.K, LK = dm.L * dm.K;
    const int NqM = dm.Nq * M;
    const int b = blockIdx.y + dm.b0;
    const int item0 = blockIdx.x * IPB;
    const int nitems = min(IPB, NqM - item0);
    const uint32_t row_stride = (uint32_t)M * D * 4u;

    stage_levels(s_lvl, shapes, starts, dm.L, dm.Nv);

    const size_t slice = (size_t)dm.Nv * M * D;
    const rsrc_t vr = make_rsrc(value + (size_t)b * slice, (uint32_t)(slice * sizeof(VT)));
    const size_t pt0 = ((size_t)b * NqM + item0) * LK;

    const int it = threadIdx.x / G, c = threadIdx.x % G;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);

    for (int j0 = 0; j0 < LK; j0 += dm.PC) {
        const int pc = min(dm.PC, LK - j0);
        __syncthreads();  // level table staged / previous chunk consumed
        for (int idx = threadIdx.x; idx < nitems * pc; idx += kThreads) {
            const int i1 = idx / pc, jj = idx - i1 * pc, j = j0 + jj;
            const size_t p = pt0 + (size_t)i1 * LK + j;
            const float2 uv = reinterpret_cast<const float2 *>(loc)[p];
            const float A = attn[p];
            const int m = (item0 + i1) % M;
            Neighbours n = neighbours(uv.x, uv.y, s_lvl[j / K], row_stride, (uint32_t)m * D * 4u);
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
// backward
// ---------------------------------------------------------------------------
template <int D, typename VT>
__global__ void __launch_bounds__(kThreads)
msda_bwd_kernel(const VT *__restrict__ value, const int64_t *__restrict__ shapes,
                const int64_t *__restrict__ starts, const float *__restrict__ loc,
                const float *__restrict__ attn, const float *__restrict__ grad_out,
                float *__restrict__ grad_value, float *__restrict__ grad_loc,
                float *__restrict__ grad_attn, Dims dm) {
    constexpr int G = D / 4;
    constexpr int IPB = kThreads / G;
    extern __shared__ __align__(16) unsigned char smem[];
    int4 *s_lvl = reinterpret_cast<int4 *>(smem);
    uint4 *s_off = reinterpret_cast<uint4 *>(smem + kMaxLevels * sizeof(int4));
    float4 *s_w = reinterpret_cast<float4 *>(s_off + IPB * dm.PS);
    float4 *s_aux = s_w + IPB * dm.PS;   // (fx, fy, A, valid bits)
    float4 *s_dot = s_aux + IPB * dm.PS;  // <g, row> of the four neighbours

    const int M = dm.M, K = dm.K, LK = dm.L * dm.K;
    const int NqM = dm.Nq * M;
    const int b = blockIdx.y + dm.b0;
    const int item0 = blockIdx.x * IPB;
    const int nitems = min(IPB, NqM - item0);
    const uint32_t row_stride = (uint32_t)M * D * 4u;

    stage_levels(s_lvl, shapes, starts, dm.L, dm.Nv);

    const size_t slice = (size_t)dm.Nv * M * D;
    const rsrc_t vr = make_rsrc(value + (size_t)b * slice, (uint32_t)(slice * sizeof(VT)));
    const rsrc_t gr = make_rsrc(grad_value + (size_t)b * slice, (uint32_t)(slice * 4u));
    const size_t pt0 = ((size_t)b * NqM + item0) * LK;

    const int it = threadIdx.x / G, c = threadIdx.x % G;
    // The lane's grad_out row in two arrangements: channels 4c..4c+3 for the dot
    // products and channels c, c+G, c+2G, c+3G for the scatter.  Both are read
    // through buffer loads: with plain pointer loads the load/store vectorizer
    // of the ROCm 7.2 compiler merged the float4's last element into the strided
    // loads' address chain (reading channel c+3 instead of 4c+3 for G = 2).
    float4 g4 = make_float4(0.f, 0.f, 0.f, 0.f);
    float gs[4] = {0.f, 0.f, 0.f, 0.f};
    if (it < nitems) {
        const rsrc_t go = make_rsrc(grad_out + ((size_t)b * NqM + item0) * D,
                                    (uint32_t)(nitems * D * 4));
        const uint32_t row = (uint32_t)(it * D) * 4u;
        auto u = __builtin_amdgcn_raw_buffer_load_b128(go, (int)(row + 16u * c), 0, 0);
        g4 = make_float4(__uint_as_float(u[0]), __uint_as_float(u[1]), __uint_as_float(u[2]),
                         __uint_as_float(u[3]));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            gs[i] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(go, (int)(row + 4u * (c + i * G)), 0, 0));
    }

    for (int j0 = 0; j0 < LK; j0 += dm.PC) {
        const int pc = min(dm.PC, LK - j0);
        __syncthreads();
        for (int idx = threadIdx.x; idx < nitems * pc; idx += kThreads) {
            const int i1 = idx / pc, jj = idx - i1 * pc, j = j0 + jj;
            const size_t p = pt0 + (size_t)i1 * LK + j;
            const float2 uv = reinterpret_cast<const float2 *>(loc)[p];
            const float A = attn[p];
            const int m = (item0 + i1) % M;
            Neighbours n = neighbours(uv.x, uv.y, s_lvl[j / K], row_stride, (uint32_t)m * D * 4u);
            s_off[i1 * dm.PS + jj] = n.off;
            s_w[i1 * dm.PS + jj] = n.w;
            s_aux[i1 * dm.PS + jj] = make_float4(n.fx, n.fy, A, __uint_as_float(n.valid));
        }
        __syncthreads();
        if (it < nitems) {
            const int base = it * dm.PS;
#pragma unroll 2
            for (int jj = 0; jj < pc; ++jj) {
                const uint4 o = s_off[base + jj];
                const float4 w = s_w[base + jj];
                const float A = s_aux[base + jj].z;
                const float4 v0 = Row4<VT>::load(vr, o.x, 4 * c);
                const float4 v1 = Row4<VT>::load(vr, o.y, 4 * c);
                const float4 v2 = Row4<VT>::load(vr, o.z, 4 * c);
                const float4 v3 = Row4<VT>::load(vr, o.w, 4 * c);
                const float d0 = group_sum<G>(dot4(g4, v0));
                const float d1 = group_sum<G>(dot4(g4, v1));
                const float d2 = group_sum<G>(dot4(g4, v2));
                const float d3 = group_sum<G>(dot4(g4, v3));
                if (c == 0) s_dot[base + jj] = make_float4(d0, d1, d2, d3);
                const float a0 = A * w.x, a1 = A * w.y, a2 = A * w.z, a3 = A * w.w;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t ch = 4u * (uint32_t)(c + i * G);
                    atomic_add(gr, o.x + ch, a0 * gs[i]);
                    atomic_add(gr, o.y + ch, a1 * gs[i]);
                    atomic_add(gr, o.z + ch, a2 * gs[i]);
                    atomic_add(gr, o.w + ch, a3 * gs[i]);
                }
            }
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < nitems * pc; idx += kThreads) {
            const int i1 = idx / pc, jj = idx - i1 * pc, j = j0 + jj;
            const size_t p = pt0 + (size_t)i1 * LK + j;
            const float4 d = s_dot[i1 * dm.PS + jj];
            const float4 w = s_w[i1 * dm.PS + jj];
            const float4 ax = s_aux[i1 * dm.PS + jj];
            const int4 lvl = s_lvl[j / K];
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
    // one batch slice of grad_value (fp32) and of the point arrays must be 31-bit addressable
    const int64_t lim = (int64_t)1 << 31;
    if (Nv > lim / (M * D * 4) || Nv * M * D * 4 >= lim) return MSDA_ERR_UNSUPPORTED;
    if (K > lim / L || Nq > lim / (M * L * K * 2) || Nq * M * L * K * 2 >= lim)
        return MSDA_ERR_UNSUPPORTED;
    if (B > lim) return MSDA_ERR_UNSUPPORTED;
    // one launch covers Nq*M items with D/4 lanes each: keep the grid under 2^31 threads
    if (Nq * M > lim / (D / 4)) return MSDA_ERR_UNSUPPORTED;
    return MSDA_OK;
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
    p.lds = kMaxLevels * sizeof(int4) + (size_t)p.ipb * p.ps * bytes_per_point;
    return p;
}

msda_status hip_status(hipError_t e) {
    if (e == hipSuccess) return MSDA_OK;
    g_last_hip_error = (int)e;
    return MSDA_ERR_HIP;
}

template <int D, typename VT>
msda_status launch_fwd(const void *value, const int64_t *shapes, const int64_t *starts,
                       const float *loc, const float *attn, float *out, int64_t B, int64_t Nv,
                       int64_t Nq, int64_t M, int64_t L, int64_t K, hipStream_t s) {
    const Launch p = plan(D, L, K, 32);
    const int64_t items = Nq * M;
    const unsigned gx = (unsigned)((items + p.ipb - 1) / p.ipb);
    for (int64_t b0 = 0; b0 < B; b0 += 65535) {
        const unsigned gy = (unsigned)((B - b0) < 65535 ? (B - b0) : 65535);
        Dims dm{(int)Nv, (int)Nq, (int)M, (int)L, (int)K, p.pc, p.ps, (int)b0};
        hipLaunchKernelGGL((msda_fwd_kernel<D, VT>), dim3(gx, gy), dim3(kThreads), p.lds, s,
                           static_cast<const VT *>(value), shapes, starts, loc, attn, out, dm);
        msda_status st = hip_status(hipGetLastError());
        if (st != MSDA_OK) return st;
    }
    return MSDA_OK;
}

template <int D, typename VT>
msda_status launch_bwd(const void *value, const int64_t *shapes, const int64_t *starts,
                       const float *loc, const float *attn, const float *gout, float *gval,
                       float *gloc, float *gattn, int64_t B, int64_t Nv, int64_t Nq, int64_t M,
                       int64_t L, int64_t K, hipStream_t s) {
    const Launch p = plan(D, L, K, 64);
    const int64_t items = Nq * M;
    const unsigned gx = (unsigned)((items + p.ipb - 1) / p.ipb);
    for (int64_t b0 = 0; b0 < B; b0 += 65535) {
        const unsigned gy = (unsigned)((B - b0) < 65535 ? (B - b0) : 65535);
        Dims dm{(int)Nv, (int)Nq, (int)M, (int)L, (int)K, p.pc, p.ps, (int)b0};
        hipLaunchKernelGGL((msda_bwd_kernel<D, VT>), dim3(gx, gy), dim3(kThreads), p.lds, s,
                           static_cast<const VT *>(value), shapes, starts, loc, attn, gout, gval,
                           gloc, gattn, dm);
        msda_status st = hip_status(hipGetLastError());
        if (st != MSDA_OK) return st;
    }
    return MSDA_OK;
}

template <typename VT>
msda_status dispatch_fwd(int64_t D, const void *value, const int64_t *shapes,
                         const int64_t *starts, const float *loc, const float *attn, float *out,
                         int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t L, int64_t K,
                         hipStream_t s) {
    switch (D) {
    case 4: return launch_fwd<4, VT>(value, shapes, starts, loc, attn, out, B, Nv, Nq, M, L, K, s);
    case 8: return launch_fwd<8, VT>(value, shapes, starts, loc, attn, out, B, Nv, Nq, M, L, K, s);
    case 16: return launch_fwd<16, VT>(value, shapes, starts, loc, attn, out, B, Nv, Nq, M, L, K, s);
    case 32: return launch_fwd<32, VT>(value, shapes, starts, loc, attn, out, B, Nv, Nq, M, L, K, s);
    case 64: return launch_fwd<64, VT>(value, shapes, starts, loc, attn, out, B, Nv, Nq, M, L, K, s);
    case 128: return launch_fwd<128, VT>(value, shapes, starts, loc, attn, out, B, Nv, Nq, M, L, K, s);
    case 256: return launch_fwd<256, VT>(value, shapes, starts, loc, attn, out, B, Nv, Nq, M, L, K, s);
    default: return MSDA_ERR_UNSUPPORTED;
    }
}

template <typename VT>
msda_status dispatch_bwd(int64_t D, const void *value, const int64_t *shapes,
                         const int64_t *starts, const float *loc, const float *attn,
                         const float *gout, float *gval, float *gloc, float *gattn, int64_t B,
                         int64_t Nv, int64_t Nq, int64_t M, int64_t L, int64_t K, hipStream_t s) {
#define MSDA_BWD_CASE(DD)                                                                      \
    case DD:                                                                                   \
        return launch_bwd<DD, VT>(value, shapes, starts, loc, attn, gout, gval, gloc, gattn, B, \
                                  Nv, Nq, M, L, K, s);
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

msda_status fill_zero(float *p, int64_t n, hipStream_t s) {
    if (n <= 0) return MSDA_OK;
    const size_t n4 = (size_t)n / 4;  // n is a multiple of D, itself a multiple of 4
    size_t blocks = (n4 + kThreads - 1) / kThreads;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       reinterpret_cast<float4 *>(p), n4);
    return hip_status(hipGetLastError());
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

msda_status msda_backward(const void *value, int value_dtype, const int64_t *spatial_shapes,
                          const int64_t *level_start_index, const float *sampling_loc,
                          const float *attn_weight, const float *grad_out, float *grad_value,
                          float *grad_sampling_loc, float *grad_attn_weight, int64_t B,
                          int64_t Nv, int64_t Nq, int64_t M, int64_t D, int64_t L, int64_t K,
                          uint32_t flags, void *stream) {
    msda_status st = check_sizes(value_dtype, B, Nv, Nq, M, D, L, K);
    if (st != MSDA_OK) return st;
    if (flags & ~MSDA_BWD_ACCUMULATE) return MSDA_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t nval = B * Nv * M * D;
    if (nval > 0 && !grad_value) return MSDA_ERR_NULL;
    if (B > 0 && Nq > 0) {
        if (Nv < 1) return MSDA_ERR_SHAPE;
        if (!value || !spatial_shapes || !level_start_index || !sampling_loc || !attn_weight ||
            !grad_out || !grad_sampling_loc || !grad_attn_weight)
            return MSDA_ERR_NULL;
    }
    if (!(flags & MSDA_BWD_ACCUMULATE)) {
        st = fill_zero(grad_value, nval, s);
        if (st != MSDA_OK) return st;
    }
    if (B == 0 || Nq == 0) return MSDA_OK;
    if (value_dtype == MSDA_F32)
        return dispatch_bwd<float>(D, value, spatial_shapes, level_start_index, sampling_loc,
                                   attn_weight, grad_out, grad_value, grad_sampling_loc,
                                   grad_attn_weight, B, Nv, Nq, M, L, K, s);
    return dispatch_bwd<uint16_t>(D, value, spatial_shapes, level_start_index, sampling_loc,
                                  attn_weight, grad_out, grad_value, grad_sampling_loc,
                                  grad_attn_weight, B, Nv, Nq, M, L, K, s);
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
    default: return "unknown msda status";
    }
}

int msda_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
