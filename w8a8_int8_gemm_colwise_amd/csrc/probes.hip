// probes.hip -- attainable-ceiling probes for the roofline report (libsqprobe.so).
//
// Not part of the SmoothQuant path: measurement kernels that bound what
// the path's kernels can reach on the machine they run on.
//  * sqp_mfma_i8: a loop of v_mfma_i32_32x32x32_i8 on operands loaded from a
//    caller buffer (so the matrix cores switch real data; the clock under
//    sustained int8 MFMA load depends on the operand bits).
//  * sqp_read: a streaming read of a device buffer, 16 bytes per lane.
//  * sqp_copy: a plain copy of known size, the reference that scales the
//    HBM byte counters (FETCH_SIZE / WRITE_SIZE) of a profiled run.
// All three are bounded loops over in-bounds data; see sq_probe.h for the ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sq_probe.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;

// Each lane cycles through 8 operand pairs loaded from src; 4 independent
// accumulators keep the matrix core pipeline full.
__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(const v4i* __restrict__ src, int iters,
                                                             int* __restrict__ out) {
    const size_t base = (static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x) * 16;
    v4i a[8], b[8];
    for (int u = 0; u < 8; ++u) {
        a[u] = src[base + u];
        b[u] = src[base + 8 + u];
    }
    v16i acc[4];
    for (int c = 0; c < 4; ++c)
        for (int r = 0; r < 16; ++r) acc[c][r] = 0;
    for (int it = 0; it < iters; it += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[u], b[(u * 3 + c) & 7], acc[c], 0, 0, 0);
    }
    int s = 0;
    for (int c = 0; c < 4; ++c)
        for (int r = 0; r < 16; ++r) s ^= acc[c][r];
    out[blockIdx.x * kThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                        int* __restrict__ out) {
    uint32_t s = 0;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n16;
         i += static_cast<int64_t>(gridDim.x) * kThreads) {
        const uint4 v = p[i];
        s ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    out[blockIdx.x * kThreads + threadIdx.x] = static_cast<int>(s);
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const uint4* __restrict__ src,
                                                        uint4* __restrict__ dst, int64_t n16) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n16;
         i += static_cast<int64_t>(gridDim.x) * kThreads)
        dst[i] = src[i];
}

}  // namespace

extern "C" {

int sqp_mfma_i8(const void* src, int blocks, int iters, int* out, sqp_stream_t stream) {
    if (src == nullptr || out == nullptr || blocks <= 0 || iters <= 0 || iters % 8 != 0)
        return 1;
    mfma_loop_kernel<<<blocks, kThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        static_cast<const v4i*>(src), iters, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int sqp_copy(const void* src, void* dst, int64_t bytes, int blocks, sqp_stream_t stream) {
    if (src == nullptr || dst == nullptr || bytes <= 0 || bytes % 16 != 0 || blocks <= 0 ||
        ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) != 0)
        return 1;
    copy_kernel<<<blocks, kThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        static_cast<const uint4*>(src), static_cast<uint4*>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int sqp_read(const void* src, int64_t bytes, int blocks, int* out, sqp_stream_t stream) {
    if (src == nullptr || out == nullptr || bytes <= 0 || bytes % 16 != 0 || blocks <= 0 ||
        (reinterpret_cast<uintptr_t>(src) & 15) != 0)
        return 1;
    read_kernel<<<blocks, kThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        static_cast<const uint4*>(src), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
