// probe.hip -- measurement kernels for the roofline of the sampling core
// (libmsda_probe.so; not part of the core library, used by the benchmark).
//
// The sampling kernels gather whole value rows -- four per sampling point,
// D channels of one head each, a lane group of D/4 lanes reading 16 bytes
// per lane -- so besides HBM bandwidth their ceiling is the rate at which
// the vector memory path delivers such rows from cache.  row_gather_kernel
// measures that rate in isolation: lane groups of row_bytes / lane_bytes
// lanes each read pseudo-random whole rows of a buffer with the same
// buffer-load instructions the sampling kernels use, four rows in flight
// per group.  With a buffer that fits one XCD's L2 (a few MB) the result is
// the L2-resident row-gather ceiling; with 16 KB the L1-resident one; with a
// buffer larger than the 256 MB Infinity Cache it approaches HBM.
// copy_kernel is a plain streaming copy (16-byte loads and stores), the
// achievable-bandwidth reference for the HBM roofline.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 4;             // rows a lane group loads before using any
constexpr int kRsrcWord3 = 0x00020000;   // gfx9 buffer descriptor word 3 (raw, 32-bit data)

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ uint32_t next_row(uint32_t &h, uint32_t rows) {
    // xorshift32 (Marsaglia, "Xorshift RNGs", 2003), then a multiply-high
    // range reduction onto [0, rows)
    h ^= h << 13;
    h ^= h >> 17;
    h ^= h << 5;
    return (uint32_t)(((uint64_t)h * rows) >> 32);
}

template <int LANE_BYTES>
__global__ void __launch_bounds__(kThreads)
row_gather_kernel(const void *__restrict__ buf, uint32_t rows, uint32_t row_bytes, uint32_t iters,
                  uint32_t seed, uint32_t *__restrict__ sink) {
    const uint32_t lanes_per_row = row_bytes / LANE_BYTES;
    const uint32_t tid = blockIdx.x * kThreads + threadIdx.x;
    const uint32_t group = tid / lanes_per_row, lane = tid - group * lanes_per_row;
    const rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(buf), (short)0,
                                                       (int)(rows * row_bytes), kRsrcWord3);
    // one random stream per lane group: its lanes read the same rows
    uint32_t h = (group + 1u) * 0x9E3779B9u ^ seed;
    h = h ? h : 1u;
    uint32_t acc = 0u;
    for (uint32_t it = 0; it < iters; it += kInFlight) {
        uint32_t off[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
            off[u] = next_row(h, rows) * row_bytes + lane * LANE_BYTES;
        if constexpr (LANE_BYTES == 16) {
            decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)) v[kInFlight];
#pragma unroll
            for (int u = 0; u < kInFlight; ++u)
                v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off[u], 0, 0);
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) acc += v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
        } else {
            decltype(__builtin_amdgcn_raw_buffer_load_b64(r, 0, 0, 0)) v[kInFlight];
#pragma unroll
            for (int u = 0; u < kInFlight; ++u)
                v[u] = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off[u], 0, 0);
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) acc += v[u][0] ^ v[u][1];
        }
    }
    sink[tid] = acc;  // keeps the loads alive
}

__global__ void __launch_bounds__(kThreads)
copy_kernel(const float4 *__restrict__ src, float4 *__restrict__ dst, size_t n4) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride)
        dst[i] = src[i];
}

}  // namespace

extern "C" {

// Lane groups in one msda_probe_row_gather launch: grid_blocks workgroups
// of 256 lanes, row_bytes / lane_bytes lanes per group.  sink must hold
// grid_blocks * 256 uint32 (device memory).  buf (device) must hold
// rows * row_bytes bytes, below 2^31.  Returns a hipError_t (0 = success).
int msda_probe_row_gather(const void *buf, uint32_t rows, uint32_t row_bytes,
                          uint32_t lane_bytes, uint32_t iters, uint32_t grid_blocks,
                          uint32_t seed, uint32_t *sink, void *stream) {
    if (!buf || !sink || rows == 0 || grid_blocks == 0) return (int)hipErrorInvalidValue;
    if (lane_bytes != 16 && lane_bytes != 8) return (int)hipErrorInvalidValue;
    if (row_bytes % lane_bytes != 0 || kThreads % (row_bytes / lane_bytes) != 0)
        return (int)hipErrorInvalidValue;
    if ((uint64_t)rows * row_bytes >= ((uint64_t)1 << 31) || iters % kInFlight != 0)
        return (int)hipErrorInvalidValue;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (lane_bytes == 16)
        hipLaunchKernelGGL(row_gather_kernel<16>, dim3(grid_blocks), dim3(kThreads), 0, s, buf,
                           rows, row_bytes, iters, seed, sink);
    else
        hipLaunchKernelGGL(row_gather_kernel<8>, dim3(grid_blocks), dim3(kThreads), 0, s, buf,
                           rows, row_bytes, iters, seed, sink);
    return (int)hipGetLastError();
}

// dst[0, bytes) = src[0, bytes) with 16-byte loads and stores (bytes a
// multiple of 16, both device pointers, 16-byte aligned).
int msda_probe_copy(const void *src, void *dst, uint64_t bytes, void *stream) {
    if (!src || !dst || bytes % 16 != 0) return (int)hipErrorInvalidValue;
    const size_t n4 = bytes / 16;
    size_t blocks = (n4 + kThreads - 1) / kThreads;
    if (blocks > 16384) blocks = 16384;
    if (blocks == 0) return 0;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const float4 *>(src),
                       static_cast<float4 *>(dst), n4);
    return (int)hipGetLastError();
}

}  // extern "C"
