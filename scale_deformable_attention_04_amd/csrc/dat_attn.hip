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
// Forward (dat_attn_fwd_kernel): a wave owns tiles of 16 queries.  It
// computes the transposed scores S^T = K Q^T one 16-key block at a time
// (keys in LDS, its queries' rows in registers), so each lane holds four keys
// of one query for every block; the row max and sum are lane-local plus two
// cross-row shuffles.  O^T = V^T P^T then takes P^T straight from those
// registers: its k-step s covers keys {4g + s : g = 0..3} of the block, which
// lane group g already holds as its register s.  The kernels are built per
// count of 16-key blocks (1, 2, 4, 8, 16), so the score registers are a fixed
// array; scores are kept in base-2 units (log2 e folded into the scale).
//
// Backward: dat_attn_dq_kernel (per query block, like the forward) forms
// delta = rowsum(dO * O), P from the saved log-sum-exp, dP^T = V dO^T,
// dS = P (dP - delta), dQ = scale dS K and, when asked for, dbias = dS.
// dat_attn_dkdv_kernel (per 64-key block, the four waves one 16-key block
// each, queries in double-buffered chunks staged through LDS) computes S = Q K^T and dP =
// dO V^T with keys as columns, so that dV^T = dO^T P and dK^T = scale Q^T dS
// contract over the queries with the same register trick; chunks of the
// query range from several workgroups add into dK, dV with fp32 atomics.

#include <math.h>

#include "common.h"

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kAttnThreads = 256;  // four waves
constexpr int kAttnMinWaves = 4;   // per SIMD: at most 128 VGPRs a lane
constexpr int kMaxKeys = 256;      // keys per (batch, head), at most
constexpr int kQueryChunk = 64;    // queries per split unit of the dK/dV kernel

__device__ __forceinline__ v4f mfma16x4(float a, float b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Rows n0 .. n0+npad-1 of (b, h) from a [B, T, heads, DH] tensor into LDS
// rows of RS floats; rows n..npad-1 are zero-filled (their keys are masked,
// but a product with them must stay finite).  npad <= MAXROWS.  Each thread
// issues up to BATCH float4 loads before it writes any, so a staging waits
// for memory once per batch rather than once per float4 (a smaller BATCH
// where many registers are live).
template <int DH, int RS, int MAXROWS, int BATCH = 8>
__device__ __forceinline__ void stage_rows(float *s, const float *__restrict__ src, int b, int h,
                                           int T, int heads, int n0, int n, int npad) {
    constexpr int C4 = DH / 4;
    constexpr int ITEMS = (MAXROWS * C4 + kAttnThreads - 1) / kAttnThreads;
#pragma unroll
    for (int i0 = 0; i0 < ITEMS; i0 += BATCH) {
        float4 val[BATCH];
#pragma unroll
        for (int it = 0; it < BATCH; ++it) {
            const int i = threadIdx.x + (i0 + it) * kAttnThreads;
            const int row = i / C4, c4 = i - row * C4;
            val[it] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (i0 + it < ITEMS && row < n)
                val[it] = reinterpret_cast<const float4 *>(
                    src + (((size_t)b * T + n0 + row) * heads + h) * DH)[c4];
        }
#pragma unroll
        for (int it = 0; it < BATCH; ++it) {
            const int i = threadIdx.x + (i0 + it) * kAttnThreads;
            const int row = i / C4, c4 = i - row * C4;
            if (i0 + it < ITEMS && row < npad) {
                float *d = s + row * RS + 4 * c4;
                d[0] = val[it].x;
                d[1] = val[it].y;
                d[2] = val[it].z;
                d[3] = val[it].w;
            }
        }
    }
}

// A chunk of ROWS rows of (b, h) held in registers between its loads and its
// LDS stores, so that a kernel can load the next chunk while it computes on
// the current one.  Rows n..ROWS-1 are stored as zeros.
template <int DH, int ROWS>
struct RowChunk {
    static constexpr int C4 = DH / 4;
    static constexpr int ITEMS = (ROWS * C4 + kAttnThreads - 1) / kAttnThreads;
    float4 val[ITEMS];

    __device__ __forceinline__ void load(const float *__restrict__ src, int b, int h, int T,
                                         int heads, int n0, int n) {
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int i = threadIdx.x + it * kAttnThreads;
            const int row = i / C4, c4 = i - row * C4;
            val[it] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (row < n)
                val[it] = reinterpret_cast<const float4 *>(
                    src + (((size_t)b * T + n0 + row) * heads + h) * DH)[c4];
        }
    }

    template <int RS>
    __device__ __forceinline__ void store(float *s) const {
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int i = threadIdx.x + it * kAttnThreads;
            const int row = i / C4, c4 = i - row * C4;
            if (row < ROWS) {
                float *d = s + row * RS + 4 * c4;
                d[0] = val[it].x;
                d[1] = val[it].y;
                d[2] = val[it].z;
                d[3] = val[it].w;
            }
        }
    }
};

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
// scores of one tile of 16 queries
// NKB: key blocks of 16 the kernel is built for (the host takes the smallest
// of 1, 2, 4, 8, 16 that covers ceil(Ns / 16)); blocks past the staged ones
// skip their products (a uniform branch) and score -inf.
// ---------------------------------------------------------------------------
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// sc[kb][r] = log2(e) * scale * q.k for key kb*16 + 4g + r of this lane's
// query (exp2 of a difference of these is exp of the natural one); -inf for
// keys >= Ns, added from s_mask (0 below Ns, -inf from Ns on) rather than
// by per-lane compares, whose masks the compiler would keep across tiles.
template <int DH, int RS, int NKB>
__device__ __forceinline__ void tile_scores(v4f (&sc)[NKB], const float *s_k, const float *s_mask,
                                            const float (&qr)[DH / 4], int nkb, float scale2,
                                            int g, int j) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        v4f acc = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        if (kb < nkb) {
            v4f c = {0.f, 0.f, 0.f, 0.f};
            const float *krow = s_k + (kb * 16 + j) * RS + g;
#pragma unroll
            for (int s = 0; s < DH / 4; ++s) c = mfma16x4(krow[4 * s], qr[s], c);
            const float4 m = reinterpret_cast<const float4 *>(s_mask + kb * 16)[g];
            acc = v4f{fmaf(c[0], scale2, m.x), fmaf(c[1], scale2, m.y), fmaf(c[2], scale2, m.z),
                      fmaf(c[3], scale2, m.w)};
        }
        sc[kb] = acc;
    }
}

// sc += log2(e) * bias.  brs: buffer over the (b, h)'s bias rows [N][Ns];
// roff: byte offset of this lane's query row.  The key's offset is an
// immediate of the load; keys past Ns read the next row (or nothing: past the
// buffer a load returns 0) and stay -inf.
template <int NKB>
__device__ __forceinline__ void add_bias(v4f (&sc)[NKB], rsrc_t brs, uint32_t roff, int nkb,
                                         int g) {
    const int base = (int)(roff + 16u * g);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        if (kb < nkb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float bv = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(brs, base + kb * 64 + 4 * r, 0, 0));
                sc[kb][r] = fmaf(bv, kLog2e, sc[kb][r]);
            }
        }
    }
}

// LDS of the forward and dQ kernels: the key mask, then K (and V)
__device__ __forceinline__ void stage_mask(float *s_mask, int Ns, int nkb) {
    for (int i = threadIdx.x; i < nkb * 16; i += blockDim.x) s_mask[i] = i < Ns ? 0.f : -INFINITY;
}

// ---------------------------------------------------------------------------
// forward
// RESIDENT: K and V of the (b, h) are staged once, side by side, and each
// wave walks `tiles` tiles of 16 queries (a workgroup covers 64 * tiles
// consecutive queries).  Otherwise (keys too many for both to fit the LDS
// budget) one buffer holds K, then V, and tiles == 1.  Lanes past the last
// query compute on a copy of the last query's row and store nothing.
// ---------------------------------------------------------------------------
template <int DH, int NKB, bool RESIDENT>
__global__ void __launch_bounds__(kAttnThreads, kAttnMinWaves)
dat_attn_fwd_kernel(const float *__restrict__ q, const float *__restrict__ k,
                    const float *__restrict__ v, const float *__restrict__ bias,
                    float *__restrict__ out, float *__restrict__ lse, int N, int Ns, int heads,
                    float scale, int tiles) {
    constexpr int RS = DH + 2;  // LDS row stride: conflict-free reads of A[l%16][4s + l/16]
    constexpr int KS = DH / 4;  // k-steps of the score product
    extern __shared__ float s_kv[];

    const int bh = blockIdx.y, b = bh / heads, h = bh % heads;
    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4, j = l & 15;
    const int nkb = (Ns + 15) >> 4;
    const float scale2 = scale * kLog2e;
    float *s_mask = s_kv;  // [nkb * 16]
    float *s_k = s_kv + nkb * 16;
    float *s_v = RESIDENT ? s_k + nkb * 16 * RS : s_k;
    stage_mask(s_mask, Ns, nkb);
    if constexpr (RESIDENT) {
        stage_rows<DH, RS, NKB * 16>(s_k, k, b, h, Ns, heads, 0, Ns, nkb * 16);
        stage_rows<DH, RS, NKB * 16>(s_v, v, b, h, Ns, heads, 0, Ns, nkb * 16);
        __syncthreads();
    }

    for (int t = 0; t < (RESIDENT ? tiles : 1); ++t) {  // one tile unless resident
        const int q0 = ((blockIdx.x * tiles + t) * 4 + wave) * 16;  // the tile's first query
        if constexpr (RESIDENT) {
            if (q0 >= N) break;  // wave-uniform; no barrier follows in this mode
        }
        const int qi = q0 + j;  // this lane's query
        const bool qok = qi < N;
        const int qc = qok ? qi : N - 1;
        const size_t qrow = (((size_t)b * N + qc) * heads + h) * DH;
        if constexpr (!RESIDENT)
            stage_rows<DH, RS, NKB * 16>(s_k, k, b, h, Ns, heads, 0, Ns, nkb * 16);
        float qr[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) qr[s] = q[qrow + 4 * s + g];
        if constexpr (!RESIDENT) __syncthreads();

        // scores: sc[kb][r] ~ S[query qi][key kb*16 + 4g + r]
        v4f sc[NKB];
        tile_scores<DH, RS, NKB>(sc, s_k, s_mask, qr, nkb, scale2, g, j);
        if (bias)
            add_bias<NKB>(sc, make_rsrc(bias + (size_t)bh * N * Ns, (uint32_t)N * Ns * 4),
                          (uint32_t)qc * Ns * 4, nkb, g);
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[kb][r]);
        mx = cross_max(mx);
        float sum = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = __builtin_amdgcn_exp2f(sc[kb][r] - mx);
                sc[kb][r] = p;
                sum += p;
            }
        }
        sum = cross_sum(sum);
        if (qok && g == 0) lse[(size_t)bh * N + qi] = (mx + log2f(sum)) * kLn2;
        const float inv = 1.f / sum;

        if constexpr (!RESIDENT) {
            __syncthreads();  // every wave is done with K
            stage_rows<DH, RS, NKB * 16, 4>(s_v, v, b, h, Ns, heads, 0, Ns, nkb * 16);
            __syncthreads();
        }

        // O^T[dim db*16 + 4g + r][query] = sum over keys of V^T P^T
#pragma unroll
        for (int db = 0; db < DH / 16; ++db) {
            v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                if (kb < nkb) {
                    const float *vcol = s_v + (kb * 16 + 4 * g) * RS + db * 16 + j;
#pragma unroll
                    for (int s = 0; s < 4; ++s) acc = mfma16x4(vcol[s * RS], sc[kb][s], acc);
                }
            }
            if (qok) {
                float4 o = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
                reinterpret_cast<float4 *>(out + qrow + db * 16)[g] = o;
            }
        }
        if constexpr (!RESIDENT) __syncthreads();  // V is replaced by the next tile's K
    }
}

// ---------------------------------------------------------------------------
// backward, part 1: delta, dQ, dbias (query tiles, as the forward; RESIDENT
// as there, otherwise K, V, then K again through one buffer)
// ---------------------------------------------------------------------------
template <int DH, int NKB, bool RESIDENT>
__global__ void __launch_bounds__(kAttnThreads, kAttnMinWaves)
dat_attn_dq_kernel(const float *__restrict__ q, const float *__restrict__ k,
                   const float *__restrict__ v, const float *__restrict__ bias,
                   const float *__restrict__ out, const float *__restrict__ lse,
                   const float *__restrict__ gout, float *__restrict__ gq,
                   float *__restrict__ gbias, float *__restrict__ delta, int N, int Ns, int heads,
                   float scale, int tiles) {
    constexpr int RS = DH + 2;
    constexpr int KS = DH / 4;
    extern __shared__ float s_kv[];

    const int bh = blockIdx.y, b = bh / heads, h = bh % heads;
    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4, j = l & 15;
    const int nkb = (Ns + 15) >> 4;
    const float scale2 = scale * kLog2e;
    float *s_mask = s_kv;  // [nkb * 16]
    float *s_k = s_kv + nkb * 16;
    float *s_v = RESIDENT ? s_k + nkb * 16 * RS : s_k;
    stage_mask(s_mask, Ns, nkb);
    if constexpr (RESIDENT) {
        stage_rows<DH, RS, NKB * 16>(s_k, k, b, h, Ns, heads, 0, Ns, nkb * 16);
        stage_rows<DH, RS, NKB * 16>(s_v, v, b, h, Ns, heads, 0, Ns, nkb * 16);
        __syncthreads();
    }

    for (int t = 0; t < (RESIDENT ? tiles : 1); ++t) {  // one tile unless resident
        const int q0 = ((blockIdx.x * tiles + t) * 4 + wave) * 16;
        if constexpr (RESIDENT) {
            if (q0 >= N) break;
        }
        const int qi = q0 + j;
        const bool qok = qi < N;
        const int qc = qok ? qi : N - 1;
        const size_t qrow = (((size_t)b * N + qc) * heads + h) * DH;

        if constexpr (!RESIDENT)
            stage_rows<DH, RS, NKB * 16>(s_k, k, b, h, Ns, heads, 0, Ns, nkb * 16);
        float qr[KS], dr[KS];
        float dpart = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qr[s] = q[qrow + 4 * s + g];
            dr[s] = gout[qrow + 4 * s + g];
            dpart += dr[s] * out[qrow + 4 * s + g];
        }
        const float dl = cross_sum(dpart);  // delta = rowsum(dO * O)
        if (qok && g == 0) delta[(size_t)bh * N + qi] = dl;
        const float lq2 = lse[(size_t)bh * N + qc] * kLog2e;
        if constexpr (!RESIDENT) __syncthreads();

        v4f pt[NKB];  // P^T, then dS^T
        tile_scores<DH, RS, NKB>(pt, s_k, s_mask, qr, nkb, scale2, g, j);
        if (bias)
            add_bias<NKB>(pt, make_rsrc(bias + (size_t)bh * N * Ns, (uint32_t)N * Ns * 4),
                          (uint32_t)qc * Ns * 4, nkb, g);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) pt[kb][r] = __builtin_amdgcn_exp2f(pt[kb][r] - lq2);
        if constexpr (!RESIDENT) {
            __syncthreads();
            stage_rows<DH, RS, NKB * 16, 4>(s_v, v, b, h, Ns, heads, 0, Ns, nkb * 16);
            __syncthreads();
        }
        // dP^T = V dO^T (same layout as S^T); dS = P (dP - delta)
        float *grow = gbias ? gbias + ((size_t)bh * N + qc) * Ns : nullptr;
        // keys of this lane's dbias row to store: kb*16 + 4g + r < lim (none
        // past the last query; a per-tile bound keeps the compares per tile)
        const int lim = qok ? Ns - 4 * g : -64;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            if (kb < nkb) {
                v4f acc = {0.f, 0.f, 0.f, 0.f};
                const float *vrow = s_v + (kb * 16 + j) * RS + g;
#pragma unroll
                for (int s = 0; s < KS; ++s) acc = mfma16x4(vrow[4 * s], dr[s], acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) pt[kb][r] = pt[kb][r] * (acc[r] - dl);
                if (gbias) {
                    const int k0 = kb * 16 + 4 * g;
                    if ((Ns & 3) == 0) {  // whole float4s: four keys in or out together
                        if (kb * 16 < lim)
                            *reinterpret_cast<float4 *>(grow + k0) =
                                make_float4(pt[kb][0], pt[kb][1], pt[kb][2], pt[kb][3]);
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (kb * 16 + r < lim) grow[k0 + r] = pt[kb][r];
                    }
                }
            }
        }
        if constexpr (!RESIDENT) {
            __syncthreads();
            stage_rows<DH, RS, NKB * 16, 4>(s_k, k, b, h, Ns, heads, 0, Ns, nkb * 16);
            __syncthreads();
        }
        // dQ^T = scale K^T dS^T
#pragma unroll
        for (int db = 0; db < DH / 16; ++db) {
            v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                if (kb < nkb) {
                    const float *kcol = s_k + (kb * 16 + 4 * g) * RS + db * 16 + j;
#pragma unroll
                    for (int s = 0; s < 4; ++s) acc = mfma16x4(kcol[s * RS], pt[kb][s], acc);
                }
            }
            if (qok) {
                float4 o = make_float4(acc[0] * scale, acc[1] * scale, acc[2] * scale,
                                       acc[3] * scale);
                reinterpret_cast<float4 *>(gq + qrow + db * 16)[g] = o;
            }
        }
        if constexpr (!RESIDENT) __syncthreads();  // K is replaced by the next tile's
    }
}

// ---------------------------------------------------------------------------
// backward, part 2: dK, dV.  Workgroup = (b, h, 64 keys, one range of
// queries); wave w owns keys kb0 + 16w .. +15 and loops over the range in
// chunks of kQueryChunk queries (half that at head_dim 64) staged through
// LDS (Q, dO, lse, delta), two buffers: the next chunk's loads are in flight
// while the current one is consumed, and one barrier per chunk hands the
// buffers over.
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
    constexpr int QC = DH == 64 ? kQueryChunk / 2 : kQueryChunk;  // two buffers within 64 KB
    __shared__ float s_q[2][QC * RS];
    __shared__ float s_do[2][QC * RS];
    __shared__ float s_lse[2][QC];
    __shared__ float s_dl[2][QC];

    const int bh = blockIdx.y, b = bh / heads, h = bh % heads;
    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4, j = l & 15;
    const int key = blockIdx.x * 64 + wave * 16 + j;  // this lane's key (column)
    const bool kok = key < Ns;
    const float scale2 = scale * kLog2e;
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

    RowChunk<DH, QC> cq, cd;
    float vl = 0.f, vd = 0.f;
    auto load_chunk = [&](int c0) {
        const int nq = min(QC, q_end - c0);
        cq.load(q, b, h, N, heads, c0, nq);
        cd.load(gout, b, h, N, heads, c0, nq);
        if (threadIdx.x < QC) {
            const bool ok = (int)threadIdx.x < nq;
            vl = ok ? lse[(size_t)bh * N + c0 + threadIdx.x] * kLog2e : 0.f;
            vd = ok ? delta[(size_t)bh * N + c0 + threadIdx.x] : 0.f;
        }
    };
    auto store_chunk = [&](int buf) {
        cq.template store<RS>(s_q[buf]);
        cd.template store<RS>(s_do[buf]);
        if (threadIdx.x < QC) {
            s_lse[buf][threadIdx.x] = vl;
            s_dl[buf][threadIdx.x] = vd;
        }
    };
    if (q_begin < q_end) {
        load_chunk(q_begin);
        store_chunk(0);
    }
    __syncthreads();

    int buf = 0;
    for (int c0 = q_begin; c0 < q_end; c0 += QC, buf ^= 1) {
        const int nq = min(QC, q_end - c0);
        const bool more = c0 + QC < q_end;
        if (more) load_chunk(c0 + QC);
        const float *sq = s_q[buf], *sd = s_do[buf], *sl = s_lse[buf], *sdl = s_dl[buf];
        for (int t0 = 0; t0 < nq; t0 += 16) {
            // S[query t0 + 4g + r][key] and dP[query t0 + 4g + r][key]
            v4f sa = {0.f, 0.f, 0.f, 0.f}, pa = {0.f, 0.f, 0.f, 0.f};
            const float *qa = sq + (t0 + j) * RS + g;
            const float *da = sd + (t0 + j) * RS + g;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                sa = mfma16x4(qa[4 * s], kr[s], sa);
                pa = mfma16x4(da[4 * s], vr[s], pa);
            }
            float p[4], ds[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = t0 + 4 * g + r;
                const bool ok = kok && t < nq;
                float x = sa[r] * scale2;
                if (bias) {
                    const int qq = c0 + (t < nq ? t : nq - 1);
                    x = fmaf(bias[((size_t)bh * N + qq) * Ns + (kok ? key : Ns - 1)], kLog2e, x);
                }
                p[r] = ok ? __builtin_amdgcn_exp2f(x - sl[t]) : 0.f;
                ds[r] = p[r] * (pa[r] - sdl[t]);
            }
            // dV^T += dO^T P, dK^T += Q^T dS over this tile's 16 queries
#pragma unroll
            for (int db = 0; db < DH / 16; ++db) {
                const float *dcol = sd + (t0 + 4 * g) * RS + db * 16 + j;
                const float *qcol = sq + (t0 + 4 * g) * RS + db * 16 + j;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    dv[db] = mfma16x4(dcol[s * RS], p[s], dv[db]);
                    dk[db] = mfma16x4(qcol[s * RS], ds[s], dk[db]);
                }
            }
        }
        // the other buffer was last read in the previous chunk, before the
        // barrier that ended it
        if (more) store_chunk(buf ^ 1);
        __syncthreads();
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
// backward in one kernel when a (b, h) has 49..64 keys (four 16-key blocks)
// Workgroup = (b, h); wave w owns key block w for every query, so dK and dV
// are complete in its registers at the end (no atomics, no second kernel).
// Per tile of 16 queries the workgroup stages Q, dO, lse and delta (loaded
// one tile ahead); each wave forms S, P, dP, dS for its block with keys as
// columns (the dK/dV kernel's layout), adds dV^T += dO^T P and
// dK^T += Q^T dS, and its part of dQ = dS K, for which dS goes through LDS
// transposed (16 x 16 per wave); the four parts are summed in LDS.  Five
// products per (tile, block) instead of the seven the dQ and dK/dV kernels
// make together.
// ---------------------------------------------------------------------------
template <int DH>
__global__ void __launch_bounds__(kAttnThreads)
dat_attn_bwd_fused_kernel(const float *__restrict__ q, const float *__restrict__ k,
                          const float *__restrict__ v, const float *__restrict__ bias,
                          const float *__restrict__ out, const float *__restrict__ lse,
                          const float *__restrict__ gout, float *__restrict__ gq,
                          float *__restrict__ gk, float *__restrict__ gv,
                          float *__restrict__ gbias, int N, int Ns, int heads, float scale) {
    constexpr int RS = DH + 2;
    constexpr int KS = DH / 4;
    constexpr int TS = 17;  // row stride of the transposed dS tiles
    __shared__ float s_k[64 * RS];      // the four key blocks' K rows
    __shared__ float s_q[16 * RS];      // the tile's Q rows
    __shared__ float s_do[16 * RS];     // the tile's dO rows
    __shared__ float s_l[16], s_d[16];  // log2(e) * lse and delta of the tile's queries
    __shared__ float s_dq[4][16 * RS];  // the waves' parts of the tile's dQ [query][dim]
    __shared__ float s_t[4][16 * TS];   // the waves' dS [query][key]

    const int bh = blockIdx.x, b = bh / heads, h = bh % heads;
    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4, j = l & 15;
    const float scale2 = scale * kLog2e;
    const int key = wave * 16 + j;  // this lane's key (column)
    const bool kok = key < Ns;
    const bool live = wave * 16 < Ns;  // the wave's block holds a key (uniform)

    stage_rows<DH, RS, 64>(s_k, k, b, h, Ns, heads, 0, Ns, 64);
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

    // the tile's rows are loaded into registers one tile ahead and stored
    // into LDS between the tiles: Q, dO, O (for delta = rowsum(dO * O)), lse
    RowChunk<DH, 16> cq, cd, co;
    float cl = 0.f;
    auto load_tile = [&](int t0) {
        const int nq = min(16, N - t0);
        cq.load(q, b, h, N, heads, t0, nq);
        cd.load(gout, b, h, N, heads, t0, nq);
        co.load(out, b, h, N, heads, t0, nq);
        if (threadIdx.x < 16)
            cl = (int)threadIdx.x < nq ? lse[(size_t)bh * N + t0 + threadIdx.x] * kLog2e : 0.f;
    };
    auto store_tile = [&]() {
        cq.template store<RS>(s_q);
        cd.template store<RS>(s_do);
        // delta: thread i holds quad i % (DH/4) of row i / (DH/4); the row's
        // quads are DH/4 consecutive lanes
        constexpr int C4 = DH / 4;
#pragma unroll
        for (int it = 0; it < RowChunk<DH, 16>::ITEMS; ++it) {
            const float4 a = cd.val[it], o = co.val[it];
            float dp = a.x * o.x + a.y * o.y + a.z * o.z + a.w * o.w;
#pragma unroll
            for (int m = C4 / 2; m >= 1; m >>= 1) dp += __shfl_xor(dp, m, C4);
            const int i = threadIdx.x + it * kAttnThreads;
            if (i % C4 == 0 && i / C4 < 16) s_d[i / C4] = dp;
        }
        if (threadIdx.x < 16) s_l[threadIdx.x] = cl;
    };
    load_tile(0);
    store_tile();
    __syncthreads();

    for (int t0 = 0; t0 < N; t0 += 16) {
        const int nq = min(16, N - t0);
        const bool more = t0 + 16 < N;
        if (more) load_tile(t0 + 16);  // in flight while this tile is computed
        if (live) {
            // 2. S and dP with keys as columns: lane (j, g) holds rows 4g + r
            v4f sa = {0.f, 0.f, 0.f, 0.f}, pa = {0.f, 0.f, 0.f, 0.f};
            const float *qa = s_q + j * RS + g;
            const float *da = s_do + j * RS + g;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                sa = mfma16x4(qa[4 * s], kr[s], sa);
                pa = mfma16x4(da[4 * s], vr[s], pa);
            }
            float p[4], ds[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tq = 4 * g + r;
                const bool ok = kok && tq < nq;
                float x = sa[r] * scale2;
                if (bias)
                    x = fmaf(bias[((size_t)bh * N + t0 + (tq < nq ? tq : nq - 1)) * Ns +
                                  (kok ? key : Ns - 1)],
                             kLog2e, x);
                p[r] = ok ? __builtin_amdgcn_exp2f(x - s_l[tq]) : 0.f;
                ds[r] = p[r] * (pa[r] - s_d[tq]);
                if (gbias && ok) gbias[((size_t)bh * N + t0 + tq) * Ns + key] = ds[r];
            }
            // 3. dV^T += dO^T P, dK^T += Q^T dS over the tile's queries
#pragma unroll
            for (int db = 0; db < DH / 16; ++db) {
                const float *dcol = s_do + (4 * g) * RS + db * 16 + j;
                const float *qcol = s_q + (4 * g) * RS + db * 16 + j;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    dv[db] = mfma16x4(dcol[s * RS], p[s], dv[db]);
                    dk[db] = mfma16x4(qcol[s * RS], ds[s], dk[db]);
                }
            }
            // 4. dS transposed (query-major) for this wave's part of dQ; the
            // wave reads back only what it wrote, in order
            float *st = s_t[wave];
#pragma unroll
            for (int r = 0; r < 4; ++r) st[(4 * g + r) * TS + j] = ds[r];
            // dQ^T[dim][query] = sum over the block's keys of K^T dS^T
            float *dq = s_dq[wave];
#pragma unroll
            for (int db = 0; db < DH / 16; ++db) {
                v4f acc = {0.f, 0.f, 0.f, 0.f};
                const float *kcol = s_k + (wave * 16 + 4 * g) * RS + db * 16 + j;
                // k-step s, lane group g: key 4g + s in both operands
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    acc = mfma16x4(kcol[s * RS], st[j * TS + 4 * g + s], acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) dq[j * RS + db * 16 + 4 * g + r] = acc[r];
            }
        }
        __syncthreads();
        // 5. dQ of the tile: the live waves' parts summed; then the next
        // tile's rows into the buffers every wave has finished reading
        for (int i = threadIdx.x; i < nq * DH; i += kAttnThreads) {
            const int qt = i / DH, d = i - qt * DH;
            float a = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                if (w * 16 < Ns) a += s_dq[w][qt * RS + d];
            gq[(((size_t)b * N + t0 + qt) * heads + h) * DH + d] = a * scale;
        }
        if (more) store_tile();
        __syncthreads();
    }
    if (!kok) return;
    float *gkr = gk + krow, *gvr = gv + krow;
#pragma unroll
    for (int db = 0; db < DH / 16; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int dim = db * 16 + 4 * g + r;
            gkr[dim] = dk[db][r] * scale;
            gvr[dim] = dv[db][r];
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
    // one (b, h)'s bias rows are read through a buffer of 32-bit byte offsets
    if (N * Ns >= lim / 4) return MSDA_ERR_UNSUPPORTED;
    // the keys (then values) of one (b, h) and their mask in LDS: at most 64 KB
    // per workgroup
    if ((((Ns + 15) / 16) * 16) * (DH + 3) * (int64_t)sizeof(float) > 65536)
        return MSDA_ERR_UNSUPPORTED;
    return MSDA_OK;
}

// LDS of one of K, V (rows padded to whole 16-key blocks) and of the key mask
template <int DH>
size_t attn_lds(int64_t Ns) {
    return (size_t)(((Ns + 15) / 16) * 16) * (DH + 2) * sizeof(float);
}

inline size_t mask_lds(int64_t Ns) { return (size_t)(((Ns + 15) / 16) * 16) * sizeof(float); }

// Query tiling of the forward and dQ kernels: K and V stay resident when both
// fit 64 KB of LDS, and then each wave may take several tiles of 16 queries
// (K and V are staged once per workgroup instead of once per 64 queries):
// the largest power of two that still leaves >= 1024 workgroups (four per
// CU), when there are at least 2048 workgroups of one tile.
struct AttnTiling {
    bool resident;
    int tiles;
    int nkb;  // key blocks the kernel is built for: 1, 2, 4, 8 or 16
    dim3 grid;
    size_t lds;
};

template <int DH>
AttnTiling attn_tiling(int64_t B, int64_t N, int64_t Ns, int64_t heads) {
    AttnTiling t;
    const size_t one = attn_lds<DH>(Ns), mask = mask_lds(Ns);
    t.resident = 2 * one + mask <= 65536;
    const int64_t qblocks = (N + 63) / 64;
    int64_t tiles = 1;
    if (t.resident && B * heads * qblocks >= 2048)
        while (tiles * 2 <= qblocks &&
               B * heads * ((qblocks + tiles * 2 - 1) / (tiles * 2)) >= 1024)
            tiles *= 2;
    t.tiles = (int)tiles;
    const int64_t nkb = (Ns + 15) / 16;
    t.nkb = nkb <= 1 ? 1 : nkb <= 2 ? 2 : nkb <= 4 ? 4 : nkb <= 8 ? 8 : 16;
    t.grid = dim3((unsigned)((N + 64 * tiles - 1) / (64 * tiles)), (unsigned)(B * heads));
    t.lds = (t.resident ? 2 * one : one) + mask;
    return t;
}

// whether every Ns that maps to NKB key blocks keeps K and V resident
template <int DH, int NKB>
constexpr bool always_resident() {
    return (2 * NKB * 16 * (DH + 2) + NKB * 16) * (int)sizeof(float) <= 65536;
}

template <int DH, int NKB>
msda_status attn_fwd_nkb(const AttnTiling &t, const float *q, const float *k, const float *v,
                         const float *bias, float *out, float *lse, int N, int Ns, int heads,
                         float scale, hipStream_t s) {
    if constexpr (always_resident<DH, NKB>()) {
        hipLaunchKernelGGL((dat_attn_fwd_kernel<DH, NKB, true>), t.grid, dim3(kAttnThreads), t.lds,
                           s, q, k, v, bias, out, lse, N, Ns, heads, scale, t.tiles);
    } else {
        if (t.resident)
            hipLaunchKernelGGL((dat_attn_fwd_kernel<DH, NKB, true>), t.grid, dim3(kAttnThreads),
                               t.lds, s, q, k, v, bias, out, lse, N, Ns, heads, scale, t.tiles);
        else
            hipLaunchKernelGGL((dat_attn_fwd_kernel<DH, NKB, false>), t.grid, dim3(kAttnThreads),
                               t.lds, s, q, k, v, bias, out, lse, N, Ns, heads, scale, t.tiles);
    }
    return hip_status(hipGetLastError());
}

template <int DH>
msda_status attn_fwd(const float *q, const float *k, const float *v, const float *bias,
                     float *out, float *lse, int64_t B, int64_t N, int64_t Ns, int64_t heads,
                     float scale, hipStream_t s) {
    const AttnTiling t = attn_tiling<DH>(B, N, Ns, heads);
    const int n = (int)N, ns = (int)Ns, hh = (int)heads;
    switch (t.nkb) {
    case 1: return attn_fwd_nkb<DH, 1>(t, q, k, v, bias, out, lse, n, ns, hh, scale, s);
    case 2: return attn_fwd_nkb<DH, 2>(t, q, k, v, bias, out, lse, n, ns, hh, scale, s);
    case 4: return attn_fwd_nkb<DH, 4>(t, q, k, v, bias, out, lse, n, ns, hh, scale, s);
    case 8: return attn_fwd_nkb<DH, 8>(t, q, k, v, bias, out, lse, n, ns, hh, scale, s);
    default: return attn_fwd_nkb<DH, 16>(t, q, k, v, bias, out, lse, n, ns, hh, scale, s);
    }
}

template <int DH, int NKB>
msda_status attn_dq_nkb(const AttnTiling &t, const float *q, const float *k, const float *v,
                        const float *bias, const float *out, const float *lse, const float *gout,
                        float *gq, float *gbias, float *delta, int N, int Ns, int heads,
                        float scale, hipStream_t s) {
    if constexpr (always_resident<DH, NKB>()) {
        hipLaunchKernelGGL((dat_attn_dq_kernel<DH, NKB, true>), t.grid, dim3(kAttnThreads), t.lds,
                           s, q, k, v, bias, out, lse, gout, gq, gbias, delta, N, Ns, heads,
                           scale, t.tiles);
    } else {
        if (t.resident)
            hipLaunchKernelGGL((dat_attn_dq_kernel<DH, NKB, true>), t.grid, dim3(kAttnThreads),
                               t.lds, s, q, k, v, bias, out, lse, gout, gq, gbias, delta, N, Ns,
                               heads, scale, t.tiles);
        else
            hipLaunchKernelGGL((dat_attn_dq_kernel<DH, NKB, false>), t.grid, dim3(kAttnThreads),
                               t.lds, s, q, k, v, bias, out, lse, gout, gq, gbias, delta, N, Ns,
                               heads, scale, t.tiles);
    }
    return hip_status(hipGetLastError());
}

template <int DH>
msda_status attn_bwd(const float *q, const float *k, const float *v, const float *bias,
                     const float *out, const float *lse, const float *gout, float *gq, float *gk,
                     float *gv, float *gbias, float *delta, int64_t B, int64_t N, int64_t Ns,
                     int64_t heads, float scale, hipStream_t s) {
    // 49..64 keys and enough (b, h) pairs to fill the chip with one workgroup
    // each over at most 1024 queries: the one-kernel backward
    if (Ns > 48 && Ns <= 64 && B * heads >= 256 && N <= 1024) {
        hipLaunchKernelGGL((dat_attn_bwd_fused_kernel<DH>), dim3((unsigned)(B * heads)),
                           dim3(kAttnThreads), 0, s, q, k, v, bias, out, lse, gout, gq, gk, gv,
                           gbias, (int)N, (int)Ns, (int)heads, scale);
        return hip_status(hipGetLastError());
    }
    const AttnTiling t = attn_tiling<DH>(B, N, Ns, heads);
    const int n = (int)N, ns = (int)Ns, hh = (int)heads;
    msda_status st;
    switch (t.nkb) {
    case 1:
        st = attn_dq_nkb<DH, 1>(t, q, k, v, bias, out, lse, gout, gq, gbias, delta, n, ns, hh,
                                 scale, s);
        break;
    case 2:
        st = attn_dq_nkb<DH, 2>(t, q, k, v, bias, out, lse, gout, gq, gbias, delta, n, ns, hh,
                                 scale, s);
        break;
    case 4:
        st = attn_dq_nkb<DH, 4>(t, q, k, v, bias, out, lse, gout, gq, gbias, delta, n, ns, hh,
                                 scale, s);
        break;
    case 8:
        st = attn_dq_nkb<DH, 8>(t, q, k, v, bias, out, lse, gout, gq, gbias, delta, n, ns, hh,
                                 scale, s);
        break;
    default:
        st = attn_dq_nkb<DH, 16>(t, q, k, v, bias, out, lse, gout, gq, gbias, delta, n, ns, hh,
                                 scale, s);
        break;
    }
    if (st != MSDA_OK) return st;
    // split the queries so that the grid holds about four workgroups per CU;
    // split ranges are whole chunks, and more than one split adds atomically
    const int64_t key_blocks = (Ns + 63) / 64, chunks = (N + kQueryChunk - 1) / kQueryChunk;
    int64_t splits = 1024 / (B * heads * key_blocks);
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
