// robust.hip -- calibration robustness: a robust per-channel activation
// statistic, and the search over candidate smoothing strengths alpha.
//
//   [Teach] "SmoothQuant 如何解决激活量化难题？为什么适合 W8A8？"
//   §四: the calibration records per-channel activation peaks or a robust
//   statistic, and alpha / s is searched together with the weight range;
//   §六: the clip rate per layer and the stability of channel peaks are to be
//   checked, so that no single sample dominates the scales; §八: candidate
//   alphas are compared on activation saturation, weight quantization error
//   and a task set, per layer if needed.
//
// Channel quantile.  The nearest-rank q-quantile of |x[:, j]| is found by a
// radix select on the magnitude bit pattern (non-negative floats order like
// their bit patterns): 15 bits for bf16, 31 for fp32, 8 bits per pass.  Each
// pass counts, per column, the elements whose higher bits equal the prefix
// chosen so far, in a histogram of the next digit (LDS per block, then added
// into a global [K][256] histogram); a per-column select step walks that
// histogram to the bin holding the remaining rank and extends the prefix.
//
// Alpha search.  The fp64 product Y = X W^T of the calibration tokens is the
// reference; for each alpha the existing launchers calibrate, quantize the
// calibration tokens as deployed and run the int8 GEMM with fp32 output;
// deterministic two-level fp64 reductions give sum (y_q - y)^2 / sum y^2 and
// the weight quantization error sum (W^ - dw q)^2 / sum W^^2, W^ = RN(W s).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "../../include/sq.h"
#include "sq_device.hpp"
#include "sq_internal.hpp"

namespace sq {
namespace {

// ---- channel quantile -------------------------------------------------------

template <typename T> struct Mag;
template <> struct Mag<uint16_t> {
    static constexpr int kBits = 15;
    __device__ static uint32_t of(uint16_t v) { return v & 0x7fffu; }
    __device__ static float value(uint32_t m) { return __uint_as_float(m << 16); }
};
template <> struct Mag<float> {
    static constexpr int kBits = 31;
    __device__ static uint32_t of(float v) { return __float_as_uint(v) & 0x7fffffffu; }
    __device__ static float value(uint32_t m) { return __uint_as_float(m); }
};

constexpr int kQCols = 64;       // columns per block, one per lane
constexpr int kQThreads = 512;   // 8 waves walk interleaved rows
constexpr int kQBins = 256;
constexpr int kQUnroll = 16;     // loads in flight per lane (2 or 4 bytes each)

template <typename T>
__global__ __launch_bounds__(kQThreads) void quantile_hist_kernel(
    const T* __restrict__ x, int64_t rows, int64_t K, int64_t rpb, int shift, int width,
    const uint32_t* __restrict__ prefix, uint32_t* __restrict__ hist) {
    // bin-major: h[bin * 64 + lane], so a lane's counters all sit in its own
    // bank and a wave's 64 increments never collide, whatever the bins
    __shared__ uint32_t h[kQBins * kQCols];
    for (int i = threadIdx.x; i < kQBins * kQCols; i += kQThreads) h[i] = 0u;
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t col = static_cast<int64_t>(blockIdx.x) * kQCols + lane;
    const int hi = shift + width;   // at most 31: magnitude bits above the digit
    const uint32_t mask = (1u << width) - 1u;
    const int64_t r0 = static_cast<int64_t>(blockIdx.y) * rpb;
    const int64_t r1 = std::min<int64_t>(rows, r0 + rpb);
    if (col < K) {
        const uint32_t pre = prefix[col];
        uint32_t* hl = h + lane;
        constexpr int kStride = kQThreads / 64;
        int64_t t = r0 + wave;
        for (; t + (kQUnroll - 1) * kStride < r1; t += kQUnroll * kStride) {
            T v[kQUnroll];
#pragma unroll
            for (int u = 0; u < kQUnroll; ++u) v[u] = x[(t + u * kStride) * K + col];
#pragma unroll
            for (int u = 0; u < kQUnroll; ++u) {
                const uint32_t m = Mag<T>::of(v[u]);
                if ((m >> hi) == pre) atomicAdd(hl + ((m >> shift) & mask) * kQCols, 1u);
            }
        }
        for (; t < r1; t += kStride) {
            const uint32_t m = Mag<T>::of(x[t * K + col]);
            if ((m >> hi) == pre) atomicAdd(hl + ((m >> shift) & mask) * kQCols, 1u);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kQCols * kQBins; i += kQThreads) {
        const int c = i % kQCols, b = i / kQCols;
        const int64_t gc = static_cast<int64_t>(blockIdx.x) * kQCols + c;
        const uint32_t n = h[i];
        if (gc < K && n) atomicAdd(hist + gc * kQBins + b, n);
    }
}

// One wave per column: lane l holds bins 4l..4l+3 of the column's histogram
// (one 16-byte read each); an inclusive scan over the lanes finds the lane,
// then the bin, where the cumulative count first reaches the remaining rank.
// That bin extends the prefix, the rank drops by the count before it, and the
// histogram row is cleared for the next pass.  After the last pass the prefix
// is the whole magnitude pattern of the quantile.
template <typename T>
__global__ __launch_bounds__(256) void quantile_select_kernel(
    int64_t K, int width, uint32_t* __restrict__ prefix, uint32_t* __restrict__ rank,
    uint32_t* __restrict__ hist, float* __restrict__ out, int last) {
    const int lane = threadIdx.x & 63;
    const int64_t col = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (col >= K) return;  // whole waves
    uint4* hc = reinterpret_cast<uint4*>(hist + col * kQBins);
    const uint4 h = hc[lane];
    const uint32_t lsum = h.x + h.y + h.z + h.w;
    uint32_t incl = lsum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = static_cast<uint32_t>(__shfl_up(static_cast<int>(incl), o, 64));
        if (lane >= o) incl += t;
    }
    const uint32_t r = rank[col];
    uint32_t cum = incl - lsum;
    const bool mine = cum < r && r <= incl;
    int b = 3;
    if (mine) {
        const uint32_t c[4] = {h.x, h.y, h.z, h.w};
        for (b = 0; b < 3; ++b) {
            if (cum + c[b] >= r) break;
            cum += c[b];
        }
    }
    const unsigned long long bal = __ballot(mine);
    hc[lane] = make_uint4(0u, 0u, 0u, 0u);
    int bin;
    uint32_t before;
    if (bal) {
        const int src = __ffsll(static_cast<long long>(bal)) - 1;
        bin = __shfl(4 * lane + b, src, 64);
        before = static_cast<uint32_t>(__shfl(static_cast<int>(cum), src, 64));
    } else {
        // counts short of the rank (not reached with consistent counts): the
        // last bin, where a sequential scan of the histogram would stop
        const int nb = 1 << width;  // 128 or 256: bin nb - 1 is component w of lane nb/4 - 1
        bin = nb - 1;
        const uint32_t last = static_cast<uint32_t>(__shfl(static_cast<int>(h.w), nb / 4 - 1, 64));
        before = static_cast<uint32_t>(__shfl(static_cast<int>(incl), 63, 64)) - last;
    }
    if (lane == 0) {
        const uint32_t p = (prefix[col] << width) | static_cast<uint32_t>(bin);
        prefix[col] = p;
        rank[col] = r - before;
        if (last) out[col] = fmaxf(Mag<T>::value(p), kFloor);
    }
}

__global__ __launch_bounds__(256) void quantile_init_kernel(int64_t K, uint32_t rank0,
                                                            uint32_t* __restrict__ prefix,
                                                            uint32_t* __restrict__ rank,
                                                            uint32_t* __restrict__ hist,
                                                            float* __restrict__ out, int empty) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < K * kQBins;
         i += stride) {
        hist[i] = 0u;
        if (i < K) {
            prefix[i] = 0u;
            rank[i] = rank0;
            if (empty) out[i] = kFloor;
        }
    }
}

template <typename T>
hipError_t run_quantile(const T* x, int64_t rows, int64_t K, int64_t rank0, float* out,
                        uint32_t* hist, uint32_t* prefix, uint32_t* rank, hipStream_t stream) {
    const unsigned igrid = static_cast<unsigned>(std::min<int64_t>((K * kQBins + 255) / 256, 2048));
    quantile_init_kernel<<<igrid, 256, 0, stream>>>(K, static_cast<uint32_t>(rank0), prefix, rank,
                                                    hist, out, rows == 0 ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || rows == 0) return e;
    // about two blocks per CU over the strips of 64 columns
    const int64_t strips = (K + kQCols - 1) / kQCols;
    const int64_t want = std::max<int64_t>(1, (512 + strips - 1) / strips);
    const int64_t splits = std::min<int64_t>({want, (rows + 255) / 256, 65535});
    const int64_t rpb = (rows + splits - 1) / splits;
    const dim3 hgrid(static_cast<unsigned>(strips), static_cast<unsigned>((rows + rpb - 1) / rpb));
    const unsigned sgrid = static_cast<unsigned>((K + 3) / 4);
    constexpr int NB = Mag<T>::kBits;
    const int passes = (NB + 7) / 8;
    for (int p = 0; p < passes; ++p) {
        const int shift = std::max(0, NB - 8 * (p + 1));
        const int width = NB - 8 * p - shift;
        quantile_hist_kernel<T><<<hgrid, kQThreads, 0, stream>>>(x, rows, K, rpb, shift, width,
                                                                  prefix, hist);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        quantile_select_kernel<T><<<sgrid, 256, 0, stream>>>(K, width, prefix, rank, hist, out,
                                                             p == passes - 1 ? 1 : 0);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ---- alpha search -----------------------------------------------------------

// Y[m, n] = sum_k X[m, k] W[n, k] in fp64 (the inputs' products are exact in
// fp64).  128 x 128 output tile per block, four waves of 64 x 64, each a 4 x 4
// grid of 16 x 16 v_mfma_f64_16x16x4f64 tiles; K in steps of 16 staged in LDS:
// each step's rows arrive as 16-byte loads (8 bf16 or 4 fp32 per lane), all
// issued before any is converted.  The matrix instruction adds its four
// products to the accumulator in increasing k, so each output is the same as
// one fma per k in increasing k (measured bit-identical to that loop on the
// MI355X, and 1.3x faster: 512 x 12288 x 4096 in 1.07 ms instead of 1.39).
constexpr int kRT = 128;
constexpr int kRK = 16;

// Elements of a 16-byte chunk of T, as doubles.
__device__ __forceinline__ void chunk_f64(const uint4& v, double (&d)[8], uint16_t) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        d[2 * e] = static_cast<double>(__uint_as_float(u[e] << 16));
        d[2 * e + 1] = static_cast<double>(__uint_as_float(u[e] & 0xffff0000u));
    }
}
__device__ __forceinline__ void chunk_f64(const uint4& v, double (&d)[8], float) {
    d[0] = static_cast<double>(__uint_as_float(v.x));
    d[1] = static_cast<double>(__uint_as_float(v.y));
    d[2] = static_cast<double>(__uint_as_float(v.z));
    d[3] = static_cast<double>(__uint_as_float(v.w));
}

// One operand's rows [r0, r0 + kRT) x columns [k0, k0 + kRK) of a row-major
// [rows, K] tensor: the 16-byte chunks this thread loads (zero past `rows`).
template <typename T>
struct RefStage {
    static constexpr int E = 16 / sizeof(T);        // elements per chunk
    static constexpr int CPR = kRK / E;             // chunks per row
    static constexpr int LOADS = kRT * CPR / 256;   // chunks per thread
    static_assert(LOADS * 256 == kRT * CPR, "whole chunks per thread");
    uint4 v[LOADS];
    __device__ void load(const T* __restrict__ p, int64_t r0, int64_t rows, int64_t K, int64_t k0) {
#pragma unroll
        for (int l = 0; l < LOADS; ++l) {
            const int q = threadIdx.x + 256 * l;
            const int64_t r = r0 + q / CPR;
            v[l] = r < rows ? *reinterpret_cast<const uint4*>(p + r * K + k0 + (q % CPR) * E)
                            : make_uint4(0, 0, 0, 0);
        }
    }
    __device__ void store(double (*S)[kRT + 1]) const {
#pragma unroll
        for (int l = 0; l < LOADS; ++l) {
            const int q = threadIdx.x + 256 * l;
            const int r = q / CPR, c = q % CPR;
            double d[8];
            chunk_f64(v[l], d, T{});
#pragma unroll
            for (int e = 0; e < E; ++e) S[c * E + e][r] = d[e];
        }
    }
};

typedef double ref_v4d __attribute__((ext_vector_type(4)));

template <typename TX, typename TW>
__global__ __launch_bounds__(256) void ref_gemm_f64_kernel(const TX* __restrict__ x,
                                                           const TW* __restrict__ w, int64_t M,
                                                           int64_t N, int64_t K,
                                                           double* __restrict__ y) {
    __shared__ double As[kRK][kRT + 1];
    __shared__ double Bs[kRK][kRT + 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;  // the wave's 64 x 64 quadrant
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kRT;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kRT;
    // operands: lane l holds A[i = l % 16][k = l / 16] and B[k = l / 16][j = l % 16];
    // result: lane l holds C[i = l / 16 + 4 r][j = l % 16] in element r
    const int fi = lane & 15, fk = lane >> 4;
    ref_v4d acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = ref_v4d{0.0, 0.0, 0.0, 0.0};
    RefStage<TX> sa;
    RefStage<TW> sb;
    for (int64_t k0 = 0; k0 < K; k0 += kRK) {
        sa.load(x, m0, M, K, k0);
        sb.load(w, n0, N, K, k0);
        sa.store(As);
        sb.store(Bs);
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < kRK / 4; ++ks) {
            double a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[4 * ks + fk][wm * 64 + i * 16 + fi];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[4 * ks + fk][wn * 64 + j * 16 + fi];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm * 64 + i * 16 + fk + 4 * r;
                const int64_t n = n0 + wn * 64 + j * 16 + fi;
                if (m < M && n < N) y[m * N + n] = acc[i][j][r];
            }
}

constexpr int kEBlocks = 1024;   // partial sums per reduction
constexpr int kEThreads = 256;

// Block sum of two fp64 values in a fixed order (every lane's sequential sum,
// then a fixed tree); thread 0 writes the block's pair.
__device__ __forceinline__ void block_pair_sum(double a, double b, double* __restrict__ out) {
    __shared__ double ra[kEThreads], rb[kEThreads];
    ra[threadIdx.x] = a;
    rb[threadIdx.x] = b;
    __syncthreads();
    for (int d = kEThreads / 2; d >= 1; d >>= 1) {
        if (static_cast<int>(threadIdx.x) < d) {
            ra[threadIdx.x] += ra[threadIdx.x + d];
            rb[threadIdx.x] += rb[threadIdx.x + d];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        out[2 * blockIdx.x] = ra[0];
        out[2 * blockIdx.x + 1] = rb[0];
    }
}

// sum (y_q - y)^2 and sum y^2 over n outputs.
__global__ __launch_bounds__(kEThreads) void out_err_kernel(const float* __restrict__ yq,
                                                           const double* __restrict__ y,
                                                           int64_t n, double* __restrict__ part) {
    double a = 0.0, b = 0.0;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kEThreads + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * kEThreads) {
        const double r = y[i];
        const double d = static_cast<double>(yq[i]) - r;
        a += d * d;
        b += r * r;
    }
    block_pair_sum(a, b, part);
}

// sum (W^ - dw q)^2 and sum W^^2 with W^ = RN(W s) in fp32 (as the weight
// quantizer forms it) and dw the row's step (or the tensor's); blocks walk
// rows, threads 8-element chunks of a row (K % 64 == 0).
template <typename TW>
__global__ __launch_bounds__(kEThreads) void w_err_kernel(
    const TW* __restrict__ w, const float* __restrict__ s, const int8_t* __restrict__ wq,
    const float* __restrict__ w_scale, int per_tensor, int64_t N, int64_t K,
    double* __restrict__ part) {
    double a = 0.0, b = 0.0;
    const int64_t chunks = K / kChunk;
    for (int64_t row = blockIdx.x; row < N; row += gridDim.x) {
        const double dw = static_cast<double>(w_scale[per_tensor ? 0 : row]);
        const TW* wr = w + row * K;
        const int8_t* qr = wq + row * K;
        for (int64_t c = threadIdx.x; c < chunks; c += kEThreads) {
            float v[kChunk], sv[kChunk];
            load_chunk(wr, c, v);
            load_chunk(s, c, sv);
            const uint2 q8 = *reinterpret_cast<const uint2*>(qr + c * kChunk);
            const uint32_t qw[2] = {q8.x, q8.y};
#pragma unroll
            for (int e = 0; e < kChunk; ++e) {
                const float what = v[e] * sv[e];
                const int q = static_cast<int8_t>((qw[e >> 2] >> (8 * (e & 3))) & 0xffu);
                const double d = static_cast<double>(what) - static_cast<double>(q) * dw;
                a += d * d;
                b += static_cast<double>(what) * static_cast<double>(what);
            }
        }
    }
    block_pair_sum(a, b, part);
}

// One block: the partial pairs summed in a fixed order; out = num / den, or
// num when den is 0.
__global__ __launch_bounds__(kEThreads) void finish_ratio_kernel(const double* __restrict__ part,
                                                                 int nparts,
                                                                 double* __restrict__ out) {
    __shared__ double ra[kEThreads], rb[kEThreads];
    double a = 0.0, b = 0.0;
    for (int i = threadIdx.x; i < nparts; i += kEThreads) {
        a += part[2 * i];
        b += part[2 * i + 1];
    }
    ra[threadIdx.x] = a;
    rb[threadIdx.x] = b;
    __syncthreads();
    for (int d = kEThreads / 2; d >= 1; d >>= 1) {
        if (static_cast<int>(threadIdx.x) < d) {
            ra[threadIdx.x] += ra[threadIdx.x + d];
            rb[threadIdx.x] += rb[threadIdx.x + d];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) *out = rb[0] > 0.0 ? ra[0] / rb[0] : ra[0];
}

// The first index of the least value.
__global__ void argmin_kernel(const double* __restrict__ v, int n, int32_t* __restrict__ best) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    int b = 0;
    for (int i = 1; i < n; ++i)
        if (v[i] < v[b]) b = i;
    *best = b;
}

template <typename TX, typename TW>
hipError_t run_ref_gemm(const void* x, const void* w, int64_t M, int64_t N, int64_t K, double* y,
                        hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>((N + kRT - 1) / kRT),
                    static_cast<unsigned>((M + kRT - 1) / kRT));
    ref_gemm_f64_kernel<TX, TW><<<grid, 256, 0, stream>>>(static_cast<const TX*>(x),
                                                          static_cast<const TW*>(w), M, N, K, y);
    return hipGetLastError();
}

// Workspace carving: 256-byte aligned sections.
struct AlphaWs {
    double* yref;
    float* yq;
    int8_t* xq;
    float* xs;
    float* s;
    int8_t* wq;
    float* ws;
    float* st;
    float* xa;
    float* wa;
    double* part;
    size_t bytes;
};

AlphaWs carve(void* base, int64_t T, int64_t N, int64_t K) {
    uintptr_t p = reinterpret_cast<uintptr_t>(base);
    const uintptr_t p0 = p;
    auto take = [&](size_t n) {
        const uintptr_t r = p;
        p += (n + 255) & ~static_cast<size_t>(255);
        return r;
    };
    AlphaWs a;
    a.yref = reinterpret_cast<double*>(take(static_cast<size_t>(T * N) * 8));
    a.yq = reinterpret_cast<float*>(take(static_cast<size_t>(T * N) * 4));
    a.xq = reinterpret_cast<int8_t*>(take(static_cast<size_t>(T * K)));
    a.xs = reinterpret_cast<float*>(take(static_cast<size_t>(std::max<int64_t>(T, 1)) * 4));
    a.s = reinterpret_cast<float*>(take(static_cast<size_t>(K) * 4));
    a.wq = reinterpret_cast<int8_t*>(take(static_cast<size_t>(N * K)));
    a.ws = reinterpret_cast<float*>(take(static_cast<size_t>(std::max<int64_t>(N, 1)) * 4));
    a.st = reinterpret_cast<float*>(take(16));
    a.xa = reinterpret_cast<float*>(take(static_cast<size_t>(K) * 4));
    a.wa = reinterpret_cast<float*>(take(static_cast<size_t>(K) * 4));
    a.part = reinterpret_cast<double*>(take(static_cast<size_t>(kEBlocks) * 16));
    a.bytes = p - p0;
    return a;
}

}  // namespace

constexpr size_t quantile_ws_bytes(int64_t K) {
    return static_cast<size_t>(K) * (kQBins * 4 + 8) + 256;
}

size_t quantile_workspace_bytes(int64_t K) { return quantile_ws_bytes(K); }

// ---- the channel quantile without a caller workspace ---------------------------
//
// For callers that cannot allocate device memory: the quantile's histogram,
// prefix and rank words live in this file-scope array instead of a caller
// workspace (every device the library runs on holds its own copy from module
// load until the process ends).  Its host-side name is not a device address:
// each device's address is looked up once, with that device current, and only
// that address is passed to the kernels.  quantile_init_kernel clears the
// words each call, so the previous call's contents never matter; calls that
// overlap on one device share the array and race.
constexpr size_t kNoAllocBytes = quantile_ws_bytes(SQ_NOALLOC_MAX_K);
static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};  // each device's address of `scratch`
}  // namespace

hipError_t launch_channel_quantile_noalloc(const void* x, Dt x_dt, int64_t T, int64_t K,
                                           int64_t rank, float* out, hipStream_t stream) {
    if (quantile_ws_bytes(K) > kNoAllocBytes) return hipErrorInvalidValue;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* ws = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (g_scratch[dev] == nullptr) {
            void* p = nullptr;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (p == nullptr) return hipErrorInvalidSymbol;
            g_scratch[dev] = p;
        }
        ws = g_scratch[dev];
    }
    return launch_channel_quantile(x, x_dt, T, K, rank, out, ws, stream);
}

hipError_t launch_channel_quantile(const void* x, Dt x_dt, int64_t T, int64_t K, int64_t rank,
                                   float* out, void* ws, hipStream_t stream) {
    uint32_t* hist = static_cast<uint32_t*>(ws);
    uint32_t* prefix = hist + K * kQBins;
    uint32_t* rk = prefix + K;
    return (x_dt == Dt::BF16)
               ? run_quantile(static_cast<const uint16_t*>(x), T, K, rank, out, hist, prefix, rk,
                              stream)
               : run_quantile(static_cast<const float*>(x), T, K, rank, out, hist, prefix, rk,
                              stream);
}

size_t alpha_workspace_bytes(int64_t T, int64_t N, int64_t K) {
    return carve(nullptr, T, N, K).bytes;
}

hipError_t launch_alpha_search(const void* x_cal, Dt x_dt, int64_t T, const void* w, Dt w_dt,
                               int64_t N, int64_t K, const float* alphas, int n_alpha,
                               ActMode mode, bool w_per_tensor, double* err, double* werr,
                               int32_t* best, void* ws, hipStream_t stream) {
    const AlphaWs a = carve(ws, T, N, K);
    hipError_t e;
    if (x_dt == Dt::BF16)
        e = (w_dt == Dt::BF16) ? run_ref_gemm<uint16_t, uint16_t>(x_cal, w, T, N, K, a.yref, stream)
                               : run_ref_gemm<uint16_t, float>(x_cal, w, T, N, K, a.yref, stream);
    else
        e = (w_dt == Dt::BF16) ? run_ref_gemm<float, uint16_t>(x_cal, w, T, N, K, a.yref, stream)
                               : run_ref_gemm<float, float>(x_cal, w, T, N, K, a.yref, stream);
    if (e != hipSuccess) return e;
    const bool st = mode == ActMode::Static;
    for (int i = 0; i < n_alpha; ++i) {
        e = launch_calibrate(x_cal, x_dt, T, w, w_dt, N, K, alphas[i], w_per_tensor, nullptr,
                             nullptr, a.s, a.wq, a.ws, a.st, nullptr, nullptr, a.xa, a.wa,
                             nullptr, stream);
        if (e != hipSuccess) return e;
        e = launch_act_quant(x_cal, x_dt, T, K, a.s, nullptr, nullptr, 1e-5f, mode,
                             st ? a.st : nullptr, a.xq, a.xs, stream);
        if (e != hipSuccess) return e;
        e = launch_gemm(a.xq, st ? a.st : a.xs, mode == ActMode::PerToken, a.wq, a.ws,
                        w_per_tensor, T, N, K, a.yq, 0, Epi{}, Batch{}, stream);
        if (e != hipSuccess) return e;
        out_err_kernel<<<kEBlocks, kEThreads, 0, stream>>>(a.yq, a.yref, T * N, a.part);
        finish_ratio_kernel<<<1, kEThreads, 0, stream>>>(a.part, kEBlocks, err + i);
        if (w_dt == Dt::BF16)
            w_err_kernel<uint16_t><<<kEBlocks, kEThreads, 0, stream>>>(
                static_cast<const uint16_t*>(w), a.s, a.wq, a.ws, w_per_tensor ? 1 : 0, N, K,
                a.part);
        else
            w_err_kernel<float><<<kEBlocks, kEThreads, 0, stream>>>(
                static_cast<const float*>(w), a.s, a.wq, a.ws, w_per_tensor ? 1 : 0, N, K, a.part);
        finish_ratio_kernel<<<1, kEThreads, 0, stream>>>(a.part, kEBlocks, werr + i);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    argmin_kernel<<<1, 64, 0, stream>>>(err, n_alpha, best);
    return hipGetLastError();
}

}  // namespace sq
