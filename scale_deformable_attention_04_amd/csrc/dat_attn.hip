// dat_attn.hip -- gfx950 kernels and C ABI of the dense part of DAT's
// deformable attention: standard multi-head attention of every query token
// against the Ns keys/values sampled at the deformed reference points (the
// DAT integration page, section 2.3; the sampling itself is the core with one
// level, one point and align_corners, in msda.hip).  Per batch b and head h:
//
//     S = scale * Q K^T + bias,   P = softmax over the keys of S,   O = P V
//
// The products run on the matrix cores in fp32 (v_mfma_f32_16x16x4f32, one
// 16x16 tile of C per 64-lane wave; lane l supplies A[l%16][l/16] and
// B[l/16][l%16] and holds C[4*(l/16) + r][l%16] in register r).
//
// Forward (dat_attn_fwd_kernel): a wave owns 16 queries.  It computes the
// transposed scores S^T = K Q^T one 16-key block at a time (keys in LDS,
// its queries' rows in registers), so each lane holds four keys of one query
// for every block; the row max and sum are lane-local plus two cross-row
// shuffles.  O^T = V^T P^T then takes P^T straight from those registers: its
// k-step s covers keys {4g + s : g = 0..3} of the block, which lane group g
// already holds as its register s.
//
// Backward: dat_attn_dq_kernel (per query block, like the forward) forms
// delta = rowsum(dO * O), P from the saved log-sum-exp, dP^T = V dO^T,
// dS = P (dP - delta), dQ = scale dS K and, when asked for, dbias = dS.
// dat_attn_dkdv_kernel (per 64-key block, the four waves one 16-key block
// each, queries in chunks staged through LDS) computes S = Q K^T and dP =
// dO V^T with keys as columns, so that dV^T = dO^T P and dK^T = scale Q^T dS
// contract over the queries with the same register trick; chunks of the
// query range from several workgroups add into dK, dV with fp32 atomics.

#include <math.h>

#include "common.h"

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kAttnThreads = 256;  // four waves
constexpr int kMaxKeys = 256;      // keys per (batch, head), at most
constexpr int kMaxKeyBlocks = kMaxKeys / 16;
constexpr int kQueryChunk = 64;    // queries staged per step of the dK/dV kernel

__device__ __forceinline__ v4f mfma16x4(float a, float b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Rows of (b, h) from a [B, T, heads, DH] tensor into LDS rows of RS floats;
// rows n..npad-1 are zero-filled (their keys are masked, but a product with
// them must stay finite).
template <int DH, int RS>
__device__ __forceinline__ void stage_rows(float *s, const float *__restrict__ src, int b, int h,
                                           int T, int heads, int n0, int n, int npad) {
    for (int i = threadIdx.x; i < npad * (DH / 4); i += blockDim.x) {
        const int row = i / (DH / 4), c4 = i - row * (DH / 4);
        float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row < n)
            val = reinterpret_cast<const float4 *>(
                src + (((size_t)b * T + n0 + row) * heads + h) * DH)[c4];
        float *d = s + row * RS + 4 * c4;
        d[0] = val.x;
        d[1] = val.y;
        d[2] = val.z;
        d[3] = val.w;
    }
}

// Max and sum over the four lanes l, l^16, l^32, l^48 (the lane groups that
// hold the other keys of the same query).
__device__ __forceinline__ float cross_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    return fmaxf(v, __shfl_xor(v, 32, 64));
}

__device__ __forceinline__ float cross_sum(float v) {
    v += __shfl_xor(v, 16, 64);
    return v + __shfl_xor(v, 32, 64);
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <int DH>
__global__ void __launch_bounds__(kAttnThreads)
dat_attn_fwd_kernel(const float *__restrict__ q, const float *__restrict__ k,
                    const float *__restrict__ v, const float *__restrict__ bias,
                    float *__restrict__ out, float *__restrict__ lse, int N, int Ns, int heads,
                    float scale) {
    constexpr int RS = DH + 2;  // LDS row stride: conflict-free reads of A[l%16][4s + l/16]
    constexpr int KS = DH / 4;  // k-steps of the score product
    extern __shared__ float s_kv[];  // [nkb * 16][RS]: K, then V

    const int bh = blockIdx.y, b = bh / heads, h = bh % heads;
    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4, j = l & 15;
    const int qi = blockIdx.x * 64 + wave * 16 + j;  // this lane's query
    const bool qok = qi < N;
    const int nkb = (Ns + 15) >> 4;

    stage_rows<DH, RS>(s_kv, k, b, h, Ns, heads, 0, Ns, nkb * 16);
    float qr[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
        qr[s] = qok ? q[(((size_t)b * N + qi) * heads + h) * DH + 4 * s + g] : 0.f;
    __syncthreads();

    // scores: sc[kb][r] = S[query qi][key kb*16 + 4g + r]
    v4f sc[kMaxKeyBlocks];
    const float *brow = bias ? bias + ((size_t)bh * N + (qok ? qi : 0)) * Ns : nullptr;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kMaxKeyBlocks; ++kb) {
        if (kb < nkb) {
            v4f acc = {0.f, 0.f, 0.f, 0.f};
            const float *krow = s_kv + (kb * 16 + j) * RS + g;
#pragma unroll
            for (int s = 0; s < KS; ++s) acc = mfma16x4(krow[4 * s], qr[s], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = kb * 16 + 4 * g + r;
                float x = acc[r] * scale;
                if (brow && qok && key < Ns) x += brow[key];
                x = key < Ns ? x : -INFINITY;
                acc[r] = x;
                mx = fmaxf(mx, x);
            }
            sc[kb] = acc;
        }
    }
    mx = cross_max(mx);
    float sum = 0.f;
#pragma unroll
    for (int kb = 0; kb < kMaxKeyBlocks; ++kb) {
        if (kb < nkb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = expf(sc[kb][r] - mx);
                sc[kb][r] = p;
                sum += p;
            }
        }
    }
    sum = cross_sum(sum);
    if (qok && g == 0) lse[(size_t)bh * N + qi] = mx + logf(sum);
    const float inv = 1.f / sum;

    __syncthreads();  // every wave is done with K
    stage_rows<DH, RS>(s_kv, v, b, h, Ns, heads, 0, Ns, nkb * 16);
    __syncthreads();

    // O^T[dim db*16 + 4g + r][query] = sum over keys of V^T P^T
#pragma unroll
    for (int db = 0; db < DH / 16; ++db) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < kMaxKeyBlocks; ++kb) {
            if (kb < nkb) {
                const float *vcol = s_kv + (kb * 16 + 4 * g) * RS + db * 16 + j;
#pragma unroll
                for (int s = 0; s < 4; ++s) acc = mfma16x4(vcol[s * RS], sc[kb][s], acc);
            }
        }
        if (qok) {
            float4 o = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
            reinterpret_cast<float4 *>(out + (((size_t)b * N + qi) * heads + h) * DH +
                                       db * 16)[g] = o;
        }
    }
}

// ---------------------------------------------------------------------------
// backward, part 1: delta, dQ, dbias (query blocks, as the forward)
// ---------------------------------------------------------------------------
template <int DH>
__global__ void __launch_bounds__(kAttnThreads)
dat_attn_dq_kernel(const float *__restrict__ q, const float *__restrict__ k,
                   const float *__restrict__ v, const float *__restrict__ bias,
                   const float *__restrict__ out, const float *__restrict__ lse,
                   const float *__restrict__ gout, float *__restrict__ gq,
                   float *__restrict__ gbias, float *__restrict__ delta, int N, int Ns, int heads,
                   float scale) {
    constexpr int RS = DH + 2;
    constexpr int KS = DH / 4;
    extern __shared__ float s_kv[];

    const int bh = blockIdx.y, b = bh / heads, h = bh % heads;
    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4, j = l & 15;
    const int qi = blockIdx.x * 64 + wave * 16 + j;
    const bool qok = qi < N;
    const int nkb = (Ns + 15) >> 4;
    const size_t qrow = (((size_t)b * N + (qok ? qi : 0)) * heads + h) * DH;

    stage_rows<DH, RS>(s_kv, k, b, h, Ns, heads, 0, Ns, nkb * 16);
    float qr[KS], dr[KS];
    float dpart = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        qr[s] = qok ? q[qrow + 4 * s + g] : 0.f;
        dr[s] = qok ? gout[qrow + 4 * s + g] : 0.f;
        dpart += qok ? dr[s] * out[qrow + 4 * s + g] : 0.f;
    }
    const float dl = cross_sum(dpart);  // delta = rowsum(dO * O)
    if (qok && g == 0) delta[(size_t)bh * N + qi] = dl;
    const float lq = qok ? lse[(size_t)bh * N + qi] : 0.f;
    __syncthreads();

    const float *brow = bias ? bias + ((size_t)bh * N + (qok ? qi : 0)) * Ns : nullptr;
    v4f pt[kMaxKeyBlocks];  // P^T, then dS^T
#pragma unroll
    for (int kb = 0; kb < kMaxKeyBlocks; ++kb) {
        if (kb < nkb) {
            v4f acc = {0.f, 0.f, 0.f, 0.f};
            const float *krow = s_kv + (kb * 16 + j) * RS + g;
#pragma unroll
            for (int s = 0; s < KS; ++s) acc = mfma16x4(krow[4 * s], qr[s], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = kb * 16 + 4 * g + r;
                float x = acc[r] * scale;
                if (brow && qok && key < Ns) x += brow[key];
                acc[r] = (key < Ns && qok) ? expf(x - lq) : 0.f;
            }
            pt[kb] = acc;
        }
    }
    __syncthreads();
    stage_rows<DH, RS>(s_kv, v, b, h, Ns, heads, 0, Ns, nkb * 16);
    __syncthreads();
    // dP^T = V dO^T (same layout as S^T); dS = P (dP - delta)
#pragma unroll
    for (int kb = 0; kb < kMaxKeyBlocks; ++kb) {
        if (kb < nkb) {
            v4f acc = {0.f, 0.f, 0.f, 0.f};
            const float *vrow = s_kv + (kb * 16 + j) * RS + g;
#pragma unroll
            for (int s = 0; s < KS; ++s) acc = mfma16x4(vrow[4 * s], dr[s], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) pt[kb][r] = pt[kb][r] * (acc[r] - dl);
            if (gbias && qok) {
                float4 *dst = reinterpret_cast<float4 *>(gbias + ((size_t)bh * N + qi) * Ns +
                                                         kb * 16 + 4 * g);
                if (kb * 16 + 4 * g + 3 < Ns && (Ns & 3) == 0) {
                    *dst = make_float4(pt[kb][0], pt[kb][1], pt[kb][2], pt[kb][3]);
                } else {
                    float *d = gbias + ((size_t)bh * N + qi) * Ns;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (kb * 16 + 4 * g + r < Ns) d[kb * 16 + 4 * g + r] = pt[kb][r];
                }
            }
        }
    }
    __syncthreads();
    stage_rows<DH, RS>(s_kv, k, b, h, Ns, heads, 0, Ns, nkb * 16);
    __syncthreads();
    // dQ^T = scale K^T dS^T
#pragma unroll
    for (int db = 0; db < DH / 16; ++db) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < kMaxKeyBlocks; ++kb) {
            if (kb < nkb) {
                const float *kcol = s_kv + (kb * 16 + 4 * g) * RS + db * 16 + j;
#pragma unroll
                for (int s = 0; s < 4; ++s) acc = mfma16x4(kcol[s * RS], pt[kb][s], acc);
            }
        }
        if (qok) {
            float4 o = make_float4(acc[0] * scale, acc[1] * scale, acc[2] * scale, acc[3] * scale);
            reinterpret_cast<float4 *>(gq + qrow + db * 16)[g] = o;
        }
    }
}

// ---------------------------------------------------------------------------
// backward, part 2: dK, dV.  Workgroup = (b, h, 64 keys, one range of
// queries); wave w owns keys kb0 + 16w .. +15 and loops over the range in
// chunks of kQueryChunk queries staged through LDS (Q, dO, lse, delta).
// ---------------------------------------------------------------------------
template <int DH>
__global__ void __launch_bounds__(kAttnThreads)
dat_attn_dkdv_kernel(const float *__restrict__ q, const float *__restrict__ k,
                     const float *__restrict__ v, const float *__restrict__ bias,
                     const float *__restrict__ lse, const float *__restrict__ delta,
                     const float *__restrict__ gout, float *__restrict__ gk,
                     float *__restrict__ gv, int N, int Ns, int heads, float scale,
                     int queries_per_split) {
    constexpr int RS = DH + 2;
    constexpr int KS = DH / 4;
    __shared__ float s_q[kQueryChunk * RS];
    __shared__ float s_do[kQueryChunk * RS];
    __shared__ float s_lse[kQueryChunk];
    __shared__ float s_dl[kQueryChunk];

    const int bh = blockIdx.y, b = bh / heads, h = bh % heads;
    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4, j = l & 15;
    const int key = blockIdx.x * 64 + wave * 16 + j;  // this lane's key (column)
    const bool kok = key < Ns;
    const int q_begin = blockIdx.z * queries_per_split;
    const int q_end = min(N, q_begin + queries_per_split);

    // the wave's key block in registers: K[key][4s + g], V[key][4s + g]
    float kr[KS], vr[KS];
    const size_t krow = (((size_t)b * Ns + (kok ? key : 0)) * heads + h) * DH;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        kr[s] = kok ? k[krow + 4 * s + g] : 0.f;
        vr[s] = kok ? v[krow + 4 * s + g] : 0.f;
    }
    v4f dk[DH / 16], dv[DH / 16];  // dK^T, dV^T [dim db*16 + 4g + r][key]
#pragma unroll
    for (int db = 0; db < DH / 16; ++db) {
        dk[db] = v4f{0.f, 0.f, 0.f, 0.f};
        dv[db] = v4f{0.f, 0.f, 0.f, 0.f};
    }

    for (int c0 = q_begin; c0 < q_end; c0 += kQueryChunk) {
        const int nq = min(kQueryChunk, q_end - c0);
        __syncthreads();  // the previous chunk is consumed
        stage_rows<DH, RS>(s_q, q, b, h, N, heads, c0, nq, kQueryChunk);
        stage_rows<DH, RS>(s_do, gout, b, h, N, heads, c0, nq, kQueryChunk);
        if (threadIdx.x < kQueryChunk) {
            const bool ok = (int)threadIdx.x < nq;
            s_lse[threadIdx.x] = ok ? lse[(size_t)bh * N + c0 + threadIdx.x] : 0.f;
            s_dl[threadIdx.x] = ok ? delta[(size_t)bh * N + c0 + threadIdx.x] : 0.f;
        }
        __syncthreads();
        for (int t0 = 0; t0 < nq; t0 += 16) {
            // S[query t0 + 4g + r][key] and dP[query t0 + 4g + r][key]
            v4f sa = {0.f, 0.f, 0.f, 0.f}, pa = {0.f, 0.f, 0.f, 0.f};
            const float *qa = s_q + (t0 + j) * RS + g;
            const float *da = s_do + (t0 + j) * RS + g;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                sa = mfma16x4(qa[4 * s], kr[s], sa);
                pa = mfma16x4(da[4 * s], vr[s], pa);
            }
            float p[4], ds[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = t0 + 4 * g + r;
                const int qq = c0 + t;
                float x = sa[r] * scale;
                if (bias && kok && t < nq) x += bias[((size_t)bh * N + qq) * Ns + key];
                p[r] = (kok && t < nq) ? expf(x - s_lse[t]) : 0.f;
                ds[r] = p[r] * (pa[r] - s_dl[t]);
            }
            // dV^T += dO^T P, dK^T += Q^T dS over this tile's 16 queries
#pragma unroll
            for (int db = 0; db < DH / 16; ++db) {
                const float *dcol = s_do + (t0 + 4 * g) * RS + db * 16 + j;
                const float *qcol = s_q + (t0 + 4 * g) * RS + db * 16 + j;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    dv[db] = mfma16x4(dcol[s * RS], p[s], dv[db]);
                    dk[db] = mfma16x4(qcol[s * RS], ds[s], dk[db]);
                }
            }
        }
    }
    if (!kok) return;
    float *gkr = gk + krow, *gvr = gv + krow;
#pragma unroll
    for (int db = 0; db < DH / 16; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int dim = db * 16 + 4 * g + r;
            if (gridDim.z == 1) {
                gkr[dim] = dk[db][r] * scale;
                gvr[dim] = dv[db][r];
            } else {
                atomicAdd(gkr + dim, dk[db][r] * scale);
                atomicAdd(gvr + dim, dv[db][r]);
            }
        }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
msda_status check_attn(int64_t B, int64_t N, int64_t Ns, int64_t heads, int64_t DH) {
    if (B < 0 || N < 0 || Ns < 1 || heads < 1 || DH < 1) return MSDA_ERR_SHAPE;
    if (DH != 16 && DH != 32 && DH != 64) return MSDA_ERR_UNSUPPORTED;
    if (Ns > kMaxKeys) return MSDA_ERR_UNSUPPORTED;
    const int64_t lim = (int64_t)1 << 31;
    // every tensor of one launch is addressed with 64-bit offsets, but the
    // grid's y extent and the per-(b, h) row counts stay 32-bit
    if (B * heads >= 65536 || N >= lim / 64 || N > lim / (heads * DH)) return MSDA_ERR_UNSUPPORTED;
    if (N * Ns >= lim) return MSDA_ERR_UNSUPPORTED;
    // the keys (then values) of one (b, h) in LDS: at most 64 KB per workgroup
    if ((((Ns + 15) / 16) * 16) * (DH + 2) * (int64_t)sizeof(float) > 65536)
        return MSDA_ERR_UNSUPPORTED;
    return MSDA_OK;
}

template <int DH>
size_t attn_lds(int64_t Ns) {
    return (size_t)(((Ns + 15) / 16) * 16) * (DH + 2) * sizeof(float);
}

template <int DH>
msda_status attn_fwd(const float *q, const float *k, const float *v, const float *bias,
                     float *out, float *lse, int64_t B, int64_t N, int64_t Ns, int64_t heads,
                     float scale, hipStream_t s) {
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)(B * heads));
    hipLaunchKernelGGL((dat_attn_fwd_kernel<DH>), grid, dim3(kAttnThreads), attn_lds<DH>(Ns), s,
                       q, k, v, bias, out, lse, (int)N, (int)Ns, (int)heads, scale);
    return hip_status(hipGetLastError());
}

template <int DH>
msda_status attn_bwd(const float *q, const float *k, const float *v, const float *bias,
                     const float *out, const float *lse, const float *gout, float *gq, float *gk,
                     float *gv, float *gbias, float *delta, int64_t B, int64_t N, int64_t Ns,
                     int64_t heads, float scale, hipStream_t s) {
    const dim3 g1((unsigned)((N + 63) / 64), (unsigned)(B * heads));
    hipLaunchKernelGGL((dat_attn_dq_kernel<DH>), g1, dim3(kAttnThreads), attn_lds<DH>(Ns), s, q,
                       k, v, bias, out, lse, gout, gq, gbias, delta, (int)N, (int)Ns,
                       (int)heads, scale);
    msda_status st = hip_status(hipGetLastError());
    if (st != MSDA_OK) return st;
    // split the queries so that the grid holds about two workgroups per CU;
    // split ranges are whole chunks, and more than one split adds atomically
    const int64_t key_blocks = (Ns + 63) / 64, chunks = (N + kQueryChunk - 1) / kQueryChunk;
    int64_t splits = 512 / (B * heads * key_blocks);
    splits = splits < 1 ? 1 : (splits > chunks ? chunks : splits);
    const int64_t per = ((chunks + splits - 1) / splits) * kQueryChunk;
    splits = (N + per - 1) / per;
    if (splits > 1) {
        const size_t n4 = (size_t)(B * Ns * heads * DH) / 4;  // DH % 16 == 0
        st = fill_zero(gk, n4, s);
        if (st == MSDA_OK) st = fill_zero(gv, n4, s);
        if (st != MSDA_OK) return st;
    }
    const dim3 g2((unsigned)key_blocks, (unsigned)(B * heads), (unsigned)(splits < 1 ? 1 : splits));
    hipLaunchKernelGGL((dat_attn_dkdv_kernel<DH>), g2, dim3(kAttnThreads), 0, s, q, k, v, bias,
                       lse, delta, gout, gk, gv, (int)N, (int)Ns, (int)heads, scale, (int)per);
    return hip_status(hipGetLastError());
}

}  // namespace

extern "C" {

msda_status msda_dat_attention_forward(const float *q, const float *k, const float *v,
                                       const float *bias, float *out, float *lse, int64_t B,
                                       int64_t N, int64_t Ns, int64_t heads, int64_t head_dim,
                                       float scale, void *stream) {
    msda_status st = check_attn(B, N, Ns, heads, head_dim);
    if (st != MSDA_OK) return st;
    if (B == 0 || N == 0) return MSDA_OK;
    if (!q || !k || !v || !out || !lse) return MSDA_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (head_dim) {
    case 16: return attn_fwd<16>(q, k, v, bias, out, lse, B, N, Ns, heads, scale, s);
    case 32: return attn_fwd<32>(q, k, v, bias, out, lse, B, N, Ns, heads, scale, s);
    default: return attn_fwd<64>(q, k, v, bias, out, lse, B, N, Ns, heads, scale, s);
    }
}

size_t msda_dat_attention_workspace_size(int64_t B, int64_t N, int64_t Ns, int64_t heads,
                                         int64_t head_dim) {
    if (check_attn(B, N, Ns, heads, head_dim) != MSDA_OK) return 0;
    return (size_t)(B * heads * N) * sizeof(float);
}

msda_status msda_dat_attention_backward(const float *q, const float *k, const float *v,
                                        const float *bias, const float *out, const float *lse,
                                        const float *grad_out, float *grad_q, float *grad_k,
                                        float *grad_v, float *grad_bias, void *workspace,
                                        size_t workspace_bytes, int64_t B, int64_t N,
                                        int64_t Ns, int64_t heads, int64_t head_dim,
                                        float scale, void *stream) {
    msda_status st = check_attn(B, N, Ns, heads, head_dim);
    if (st != MSDA_OK) return st;
    if (B == 0) return MSDA_OK;
    if (!k || !v || !grad_k || !grad_v) return MSDA_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (N == 0) {  // no query: the key and value gradients are zero
        const size_t n4 = (size_t)(B * Ns * heads * head_dim) / 4;
        st = fill_zero(grad_k, n4, s);
        return st == MSDA_OK ? fill_zero(grad_v, n4, s) : st;
    }
    if (!q || !out || !lse || !grad_out || !grad_q) return MSDA_ERR_NULL;
    if (grad_bias && !bias) return MSDA_ERR_NULL;
    if (!workspace) return MSDA_ERR_NULL;
    if (workspace_bytes < (size_t)(B * heads * N) * sizeof(float)) return MSDA_ERR_WORKSPACE;
    float *delta = static_cast<float *>(workspace);
    switch (head_dim) {
    case 16:
        return attn_bwd<16>(q, k, v, bias, out, lse, grad_out, grad_q, grad_k, grad_v, grad_bias,
                            delta, B, N, Ns, heads, scale, s);
    case 32:
        return attn_bwd<32>(q, k, v, bias, out, lse, grad_out, grad_q, grad_k, grad_v, grad_bias,
                            delta, B, N, Ns, heads, scale, s);
    default:
        return attn_bwd<64>(q, k, v, bias, out, lse, grad_out, grad_q, grad_k, grad_v, grad_bias,
                            delta, B, N, Ns, heads, scale, s);
    }
}

}  // extern "C"
