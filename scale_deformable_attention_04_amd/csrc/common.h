// common.h -- device and host helpers shared by the translation units of
// libmsda.so (the 2-D sampling core in msda.hip, the 3-D variant in
// msda3d.hip).  Everything here has internal linkage except the error slot.
#ifndef MSDA_CSRC_COMMON_H
#define MSDA_CSRC_COMMON_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_checks.h"
#include "msda.h"

// hipError_t of the last MSDA_ERR_HIP returned on this thread (msda.hip)
extern thread_local int msda_internal_last_hip_error;

namespace {

using msda_host::kMaxLevels;
using msda_host::supported_d;

constexpr int kThreads = 256;
constexpr uint32_t kOOB = 0x80000000u;     // byte offset past every slice (slices < 2^31 B)
constexpr int kRsrcWord3 = 0x00020000;     // gfx9 buffer descriptor word 3 (raw, 32-bit data)

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


__device__ __forceinline__ void add4(float4 &acc, const float4 &v) {
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
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

// Workgroup ids are dispatched round-robin over the 8 XCDs (workgroup k runs
// on XCD k % 8), and each XCD has its own L2.  Mapping id k to the logical
// index below gives every XCD one contiguous range of the work.  The bin
// count and scatter kernels and the 3-D kernels use it; the 2-D forward and
// dots kernels measured faster in plain launch order.  The mapping is a
// permutation of [0, total): results never depend on it.
constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_contiguous(int k, int total) {
    const int per = total / kXcds, rem = total % kXcds;
    const int x = k % kXcds, j = k / kXcds;
    return x * per + min(x, rem) + j;
}


// ---------------------------------------------------------------------------
// host helpers
// ---------------------------------------------------------------------------
inline msda_status hip_status(hipError_t e) {
    if (e == hipSuccess) return MSDA_OK;
    msda_internal_last_hip_error = (int)e;
    return MSDA_ERR_HIP;
}

// Batches per launch so that a 1-D grid of per_batch workgroups per batch
// stays below 2^23 workgroups (2^31 threads).
inline int64_t batch_chunk(int64_t per_batch, int64_t B) {
    int64_t c = ((int64_t)1 << 23) / (per_batch > 0 ? per_batch : 1);
    c = c < 1 ? 1 : c;
    return c < B ? c : B;
}

__global__ void __launch_bounds__(kThreads) fill_zero_kernel(float4 *__restrict__ p, size_t n4) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride)
        p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Zero n4 float4s (16-byte units) at p.
inline msda_status fill_zero(void *p, size_t n4, hipStream_t s) {
    if (n4 == 0) return MSDA_OK;
    size_t blocks = (n4 + kThreads - 1) / kThreads;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       reinterpret_cast<float4 *>(p), n4);
    return hip_status(hipGetLastError());
}

}  // namespace

#endif  // MSDA_CSRC_COMMON_H
