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
//  * sqp_check_rcp / sqp_check_div_narrow / sqp_check_div: exhaustive (or,
//    for the fp32-dividend division, seeded) checks that the library's short
//    reciprocal and division sequences (sq_device.hpp, the same functions the
//    quantizer kernels call) return the correctly rounded IEEE result.  The
//    criterion is exact and uses no division instruction: q = RN(a / b) iff
//    the residual a - b q, exact in fp64, is below half an ulp of q times b
//    (ties: q's significand even).
// All are bounded loops over in-bounds data; see sq_probe.h for the ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sq_device.hpp"
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

// ---- exactness checks of the short division sequences -------------------------

// Whether q is the correctly rounded quotient RN(a / b) for finite a, b > 0
// whose quotient is a normal float.  b*q is exact in fp64 (24 x 24 bits), and
// for q within a few ulps of a/b so is a - b*q (both are multiples of
// ulp(b) ulp(q) and the difference is below 2^30 of them): one fp64 fma gives
// the exact residual r.  q is right iff a/b = q + r/b lies within half an ulp
// of q on the side of r -- the ulp below q is half the ulp above when q is a
// power of two -- with a tie going to the even significand.
__device__ __forceinline__ bool is_rn_quotient(float a, float b, float q) {
    const uint32_t qb = __float_as_uint(q);
    const uint32_t E = (qb >> 23) & 0xffu;
    if (qb >> 31 || E == 0 || E == 0xffu) return false;  // not a positive normal
    const double bd = b;
    const double r = __builtin_fma(-bd, static_cast<double>(q), static_cast<double>(a));
    if (r == 0.0) return true;
    // ulp of q's binade, 2^(E - 150), as an fp64 bit pattern
    const double ulp = __longlong_as_double(static_cast<long long>(E + 1023 - 150) << 52);
    const bool pow2 = (qb & 0x7fffffu) == 0;
    const double half = 0.5 * bd * ((r < 0.0 && pow2) ? 0.5 * ulp : ulp);
    const double ar = r < 0.0 ? -r : r;
    if (ar < half) return true;
    return ar == half && (qb & 1u) == 0;
}

// Adds the wave's mismatch counts to counts[0..1] (one atomic per wave and
// counter) and lowers first_bad to the smallest failing key of the wave.
__device__ __forceinline__ void report(unsigned long long* counts, uint32_t* first_bad,
                                       uint32_t n_bad, uint32_t n_ieee, uint32_t key_bad) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        n_bad += __shfl_xor(n_bad, o, 64);
        n_ieee += __shfl_xor(n_ieee, o, 64);
        key_bad = min(key_bad, static_cast<uint32_t>(__shfl_xor(static_cast<int>(key_bad), o, 64)));
    }
    if ((threadIdx.x & 63) == 0) {
        if (n_bad) atomicAdd(counts, static_cast<unsigned long long>(n_bad));
        if (n_ieee) atomicAdd(counts + 1, static_cast<unsigned long long>(n_ieee));
        if (key_bad != 0xffffffffu) atomicMin(first_bad, key_bad);
    }
}

// Every float bit pattern in [lo, hi): rcp_rn(b) (raw != 0: the hardware
// estimate alone, the checker's negative control) against RN(1 / b), and
// against the compiler's IEEE division 1.0f / b.
__global__ __launch_bounds__(kThreads) void check_rcp_kernel(uint32_t lo, uint32_t hi, int raw,
                                                             unsigned long long* __restrict__ counts,
                                                             uint32_t* __restrict__ first_bad) {
    uint32_t n_bad = 0, n_ieee = 0, key_bad = 0xffffffffu;
    const uint32_t stride = gridDim.x * kThreads;
    // hi <= 0x7f800000, so i + stride never wraps
    for (uint32_t i = lo + blockIdx.x * kThreads + threadIdx.x; i < hi; i += stride) {
        const float b = __uint_as_float(i);
        const float r = raw ? __builtin_amdgcn_rcpf(b) : sq::rcp_rn(b);
        if (!is_rn_quotient(1.0f, b, r)) {
            ++n_bad;
            key_bad = min(key_bad, i);
        }
        if (__float_as_uint(r) != __float_as_uint(1.0f / b)) ++n_ieee;
    }
    report(counts, first_bad, n_bad, n_ieee, key_bad);
}

// Every pair (a, b) with a a bf16 value in [1, 2) (128 significands) and b a
// float in [1, 2) (2^23 significands): key = a_index << 23 | b_index.
// div_rn_narrow(a, b, rcp_rn(b)) (raw != 0: only its first product
// RN(a * RN(1/b)), the negative control) against RN(a / b) and 1.0f * a / b.
__global__ __launch_bounds__(kThreads) void check_div_narrow_kernel(
    int raw, unsigned long long* __restrict__ counts, uint32_t* __restrict__ first_bad) {
    uint32_t n_bad = 0, n_ieee = 0, key_bad = 0xffffffffu;
    const uint32_t stride = gridDim.x * kThreads;
    for (uint32_t key = blockIdx.x * kThreads + threadIdx.x; key < (1u << 30); key += stride) {
        const float a = __uint_as_float(0x3f800000u | ((key >> 23) << 16));
        const float b = __uint_as_float(0x3f800000u | (key & 0x7fffffu));
        const float rb = sq::rcp_rn(b);
        const float q = raw ? a * rb : sq::div_rn_narrow(a, b, rb);
        if (!is_rn_quotient(a, b, q)) {
            ++n_bad;
            key_bad = min(key_bad, key);
        }
        if (__float_as_uint(q) != __float_as_uint(a / b)) ++n_ieee;
    }
    report(counts, first_bad, n_bad, n_ieee, key_bad);
}

// 32-bit mix of a counter (the finalizer of MurmurHash3).
__device__ __forceinline__ uint32_t mix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

// `count` pairs: b runs over every float significand in [1, 2) (index & 2^23-1)
// and a over fp32 significands in [1, 2) drawn from the counter; key = index.
// div_rn(a, b, rcp_rn(b)) (raw != 0: only its first product RN(a * RN(1/b)),
// the negative control) against RN(a / b) and a / b.
__global__ __launch_bounds__(kThreads) void check_div_kernel(
    uint32_t seed, uint32_t count, int raw, unsigned long long* __restrict__ counts,
    uint32_t* __restrict__ first_bad) {
    uint32_t n_bad = 0, n_ieee = 0, key_bad = 0xffffffffu;
    const uint32_t stride = gridDim.x * kThreads;
    for (uint32_t key = blockIdx.x * kThreads + threadIdx.x; key < count; key += stride) {
        const float a = __uint_as_float(0x3f800000u | (mix32(key ^ mix32(seed)) & 0x7fffffu));
        const float b = __uint_as_float(0x3f800000u | (key & 0x7fffffu));
        const float rb = sq::rcp_rn(b);
        const float q = raw ? a * rb : sq::div_rn(a, b, rb);
        if (!is_rn_quotient(a, b, q)) {
            ++n_bad;
            key_bad = min(key_bad, key);
        }
        if (__float_as_uint(q) != __float_as_uint(a / b)) ++n_ieee;
    }
    report(counts, first_bad, n_bad, n_ieee, key_bad);
}

// `count` chunks of eight values: chunk_codes (the quantizers' code step)
// against the code of the IEEE quotient, code_bits<CLAMP>(x / d).  Per chunk
// an absolute maximum m = 2^(j - 30) (1 + f), j < 60, drawn from (seed, key),
// with d and RN(1/d) formed as the kernels form them (step_rcp); element e is
// RN((k + f) d) for an integer k (|k| <= 126; with CLAMP |k| <= 140 and the
// dividend then limited to +-128 d, as the static quantizer limits it) and a
// fraction f uniform in [-1/2, 1/2), or, for about half of the elements, the
// value RN((k + 1/2) d) moved by -4..4 ulps (exact ties and near-ties, where
// the short form must defer to the division).  raw != 0: the short form
// without that deferral (the negative control).  Key = chunk index.
template <bool CLAMP>
__global__ __launch_bounds__(kThreads) void check_codes_kernel(
    uint32_t seed, uint32_t count, int raw, unsigned long long* __restrict__ counts,
    uint32_t* __restrict__ first_bad) {
    constexpr float kM = 12582912.0f;  // 1.5 * 2^23
    constexpr int kSpan = CLAMP ? 281 : 253;
    uint32_t n_bad = 0, key_bad = 0xffffffffu;
    const uint32_t stride = gridDim.x * kThreads;
    for (uint32_t key = blockIdx.x * kThreads + threadIdx.x; key < count; key += stride) {
        const uint32_t h0 = mix32(key ^ mix32(seed));
        const uint32_t h1 = mix32(h0 ^ 0x68e31da4u);
        const float m = __uint_as_float(((97u + h0 % 60u) << 23) | (h1 & 0x7fffffu));
        float d, rd;
        sq::step_rcp(m, d, rd);
        const float lim = 128.0f * d;
        float x[sq::kChunk];
#pragma unroll
        for (int e = 0; e < sq::kChunk; ++e) {
            const uint32_t h = mix32(h1 + 0x9e3779b9u * static_cast<uint32_t>(e + 1));
            const float k = static_cast<float>(static_cast<int>(h % kSpan) - kSpan / 2);
            float v;
            if (h & 0x80000000u) {
                const float tie = (k + 0.5f) * d;
                v = __uint_as_float(__float_as_uint(tie) + ((h >> 24) % 9u) - 4u);
            } else {
                v = (k + (static_cast<float>((h >> 8) & 0xffffu) * 0x1p-16f - 0.5f)) * d;
            }
            x[e] = CLAMP ? fminf(fmaxf(v, -lim), lim) : v;
        }
        uint32_t q[sq::kChunk];
        sq::chunk_codes<CLAMP>(x, d, rd, q);
#pragma unroll
        for (int e = 0; e < sq::kChunk; ++e) {
            uint32_t got = q[e];
            if (raw) {
                const float c = __builtin_fmaf(x[e], rd, kM);
                got = __float_as_uint(CLAMP ? __builtin_amdgcn_fmed3f(c, kM - sq::kQmax, kM + sq::kQmax) : c);
            }
            if ((got & 0xffu) != (sq::code_bits<CLAMP>(x[e] / d) & 0xffu)) {
                ++n_bad;
                key_bad = min(key_bad, key);
            }
        }
    }
    report(counts, first_bad, n_bad, 0u, key_bad);
}

// Elementwise IEEE quotient a[i] / b[i] as the compiler emits it (the
// library's reference division; the host checks it against its own).
__global__ __launch_bounds__(kThreads) void div_ref_kernel(const float* __restrict__ a,
                                                           const float* __restrict__ b,
                                                           float* __restrict__ q, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * kThreads)
        q[i] = a[i] / b[i];
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

int sqp_check_rcp(uint32_t lo, uint32_t hi, int raw, unsigned long long* counts,
                  uint32_t* first_bad, sqp_stream_t stream) {
    if (counts == nullptr || first_bad == nullptr || lo >= hi || hi > 0x7f800000u ||
        lo < 0x00800000u)
        return 1;
    check_rcp_kernel<<<8192, kThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        lo, hi, raw, counts, first_bad);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int sqp_check_div_narrow(int raw, unsigned long long* counts, uint32_t* first_bad,
                         sqp_stream_t stream) {
    if (counts == nullptr || first_bad == nullptr) return 1;
    check_div_narrow_kernel<<<8192, kThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        raw, counts, first_bad);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int sqp_check_div(uint32_t seed, uint32_t count, int raw, unsigned long long* counts,
                  uint32_t* first_bad, sqp_stream_t stream) {
    if (counts == nullptr || first_bad == nullptr || count == 0) return 1;
    check_div_kernel<<<8192, kThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        seed, count, raw, counts, first_bad);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int sqp_check_codes(uint32_t seed, uint32_t count, int clamp, int raw, unsigned long long* counts,
                    uint32_t* first_bad, sqp_stream_t stream) {
    if (counts == nullptr || first_bad == nullptr || count == 0) return 1;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (clamp)
        check_codes_kernel<true><<<8192, kThreads, 0, st>>>(seed, count, raw, counts, first_bad);
    else
        check_codes_kernel<false><<<8192, kThreads, 0, st>>>(seed, count, raw, counts, first_bad);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int sqp_div_ref(const float* a, const float* b, float* q, int64_t n, sqp_stream_t stream) {
    if (a == nullptr || b == nullptr || q == nullptr || n <= 0) return 1;
    div_ref_kernel<<<1024, kThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(a, b, q, n);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
