// calibrate.hip -- offline half of the smoothing rewrite on gfx950.
//
//   [Teach] "SmoothQuant 如何解决激活量化难题？为什么适合 W8A8？" §四: record the
//   per-input-channel activation peak on calibration data, compute the
//   smoothing scale, fold it into the weights offline.
//   [Review] "SmoothQuant：大型语言模型的精准高效训练后量化 — 深度技术评审"
//   §5.3 eq. (4): s_j = max|X_j|^alpha / max|W_j|^(1-alpha).
//   [Edge] "嵌入式 SLM 动态权重量化：SmoothQuant 激活异常值迁移与 INT8 部署实战"
//   §二/§三: gamma/s and beta/s fold; W*diag(s) quantized to int8 offline with
//   one scale per channel (per OUTPUT channel here, the axis an int8 GEMM can
//   dequantize after the contraction).
//
// Kernels (all HBM-streaming except the O(K) factor pass):
//   fill_maxima     a_j = w_j = FLOOR bits, static scale bits = 0
//   colmax          column |max| of a row-major [rows, K] tensor: 16-byte
//                   loads along K, rows split over the waves of a block and over
//                   blocks, per-block LDS combine, one uint atomicMax per column
//                   per block (non-negative floats order like their bits)
//   smooth_factor   s_j (fp64 pow, one rounding), gamma/beta fold, static scale
//   weight_quant    per output row: What = W*s, row |max|, dw_n, codes; the row
//                   stays in registers between the max and the quantize passes
#include <algorithm>

#include "sq_device.hpp"
#include "sq_internal.hpp"

namespace sq {
namespace {

constexpr uint32_t kFloorBits = 0x33d6bf95u;  // bit pattern of 1e-7f
static_assert(sizeof(float) == 4, "fp32");

__global__ void fill_maxima_kernel(uint32_t* __restrict__ xa, uint32_t* __restrict__ wa,
                                   int64_t K, uint32_t* __restrict__ static_bits) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < K) {
        xa[i] = kFloorBits;
        wa[i] = kFloorBits;
    }
    if (i == 0 && static_bits) *static_bits = 0u;
}

// ---- column absmax ----------------------------------------------------------

constexpr int kColmaxThreads = 512;  // 8 waves; each wave walks its own rows
constexpr int kColmaxWaves = kColmaxThreads / 64;

template <typename T>
struct ColmaxLane;

// bf16: one 16-byte load = 8 columns; keep |x| as 16-bit patterns in 32-bit words.
template <>
struct ColmaxLane<uint16_t> {
    static constexpr int kCols = 8;
    uint32_t m[8];
    __device__ void init() {
#pragma unroll
        for (int i = 0; i < 8; ++i) m[i] = 0u;
    }
    __device__ void add(const uint4& u) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m[2 * i] = max(m[2 * i], w[i] & 0x7fffu);
            m[2 * i + 1] = max(m[2 * i + 1], (w[i] >> 16) & 0x7fffu);
        }
    }
    __device__ uint32_t f32_bits(int i) const { return m[i] << 16; }
};

// fp32: one 16-byte load = 4 columns.
template <>
struct ColmaxLane<float> {
    static constexpr int kCols = 4;
    uint32_t m[4];
    __device__ void init() {
#pragma unroll
        for (int i = 0; i < 4; ++i) m[i] = 0u;
    }
    __device__ void add(const uint4& u) {
        m[0] = max(m[0], u.x & 0x7fffffffu);
        m[1] = max(m[1], u.y & 0x7fffffffu);
        m[2] = max(m[2], u.z & 0x7fffffffu);
        m[3] = max(m[3], u.w & 0x7fffffffu);
    }
    __device__ uint32_t f32_bits(int i) const { return m[i]; }
};

template <typename T>
__global__ __launch_bounds__(kColmaxThreads) void colmax_kernel(
    const T* __restrict__ x, int64_t rows, int64_t K, int64_t rows_per_block,
    uint32_t* __restrict__ out_bits) {
    using Lane = ColmaxLane<T>;
    constexpr int kSeg = 64 * Lane::kCols;  // columns covered by one block
    __shared__ uint32_t red[kColmaxWaves][kSeg];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t col = static_cast<int64_t>(blockIdx.x) * kSeg + lane * Lane::kCols;
    const int64_t r_begin = static_cast<int64_t>(blockIdx.y) * rows_per_block;
    const int64_t r_end = min(rows, r_begin + rows_per_block);

    Lane acc;
    acc.init();
    if (col < K) {
        const T* p = x + col;
        int64_t r = r_begin + wave;
        // four independent 16-byte loads in flight per lane
        for (; r + 3 * kColmaxWaves < r_end; r += 4 * kColmaxWaves) {
            const uint4 u0 = *reinterpret_cast<const uint4*>(p + r * K);
            const uint4 u1 = *reinterpret_cast<const uint4*>(p + (r + kColmaxWaves) * K);
            const uint4 u2 = *reinterpret_cast<const uint4*>(p + (r + 2 * kColmaxWaves) * K);
            const uint4 u3 = *reinterpret_cast<const uint4*>(p + (r + 3 * kColmaxWaves) * K);
            acc.add(u0);
            acc.add(u1);
            acc.add(u2);
            acc.add(u3);
        }
        for (; r < r_end; r += kColmaxWaves) acc.add(*reinterpret_cast<const uint4*>(p + r * K));
    }
#pragma unroll
    for (int i = 0; i < Lane::kCols; ++i) red[wave][lane * Lane::kCols + i] = acc.f32_bits(i);
    __syncthreads();
    for (int c = threadIdx.x; c < kSeg; c += kColmaxThreads) {
        uint32_t v = red[0][c];
#pragma unroll
        for (int w = 1; w < kColmaxWaves; ++w) v = max(v, red[w][c]);
        const int64_t gc = static_cast<int64_t>(blockIdx.x) * kSeg + c;
        if (gc < K && v > kFloorBits) atomicMax(out_bits + gc, v);
    }
}

template <typename T>
hipError_t launch_colmax(const T* x, int64_t rows, int64_t K, uint32_t* out_bits,
                         hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    constexpr int kSeg = 64 * ColmaxLane<T>::kCols;
    const int64_t bx = (K + kSeg - 1) / kSeg;
    // about 4 blocks of 8 waves per CU over 256 CUs, at least 64 rows a block
    const int64_t want = (1024 + bx - 1) / bx;
    const int64_t max_split = (rows + 63) / 64;
    const int64_t by = std::max<int64_t>(1, std::min(want, max_split));
    const int64_t rpb = (rows + by - 1) / by;
    const int64_t by2 = (rows + rpb - 1) / rpb;
    dim3 grid(static_cast<unsigned>(bx), static_cast<unsigned>(by2));
    colmax_kernel<T><<<grid, kColmaxThreads, 0, stream>>>(x, rows, K, rpb, out_bits);
    return hipGetLastError();
}

// ---- smoothing factor, fold, static scale ------------------------------------

constexpr int kFactorThreads = 256;

__global__ __launch_bounds__(kFactorThreads) void smooth_factor_kernel(
    const float* __restrict__ a, const float* __restrict__ w, int64_t K, float alpha,
    const float* __restrict__ gamma, const float* __restrict__ beta, float* __restrict__ s,
    float* __restrict__ gamma_s, float* __restrict__ beta_s, uint32_t* __restrict__ static_bits) {
    __shared__ float red[kFactorThreads / 64];
    const double al = static_cast<double>(alpha);
    const double be = 1.0 - al;
    float local = 0.0f;
    for (int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; j < K;
         j += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const float aj = a[j];
        // eq. (4) in fp64, rounded once to fp32
        const float sj = static_cast<float>(pow(static_cast<double>(aj), al) /
                                            pow(static_cast<double>(w[j]), be));
        s[j] = sj;
        if (gamma) {
            gamma_s[j] = gamma[j] / sj;
            beta_s[j] = beta[j] / sj;
        }
        // RN(max(FLOOR, x)/127) is monotone in x, so the max of the per-channel
        // steps is the step of the max smoothed calibration peak RN(a_j/s_j).
        local = fmaxf(local, step_from_absmax(aj / sj));
    }
    if (!static_bits) return;
    local = wave_max(local);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = local;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = red[0];
        for (int i = 1; i < kFactorThreads / 64; ++i) m = fmaxf(m, red[i]);
        atomicMax(static_bits, __float_as_uint(m));
    }
}

// ---- weight smoothing + per-output-channel quantization ------------------------

// One row per team; the team is the whole block (kWqThreads lanes), the row
// stays in registers (CPT chunks of 8 per lane) between the max and the
// quantize passes.
template <typename T, int CPT>
__global__ __launch_bounds__(1024) void weight_quant_kernel(
    const T* __restrict__ w, int64_t N, int64_t K, const float* __restrict__ s,
    int8_t* __restrict__ wq, float* __restrict__ w_scale) {
    __shared__ float red[16];
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int64_t chunks = K / kChunk;
    for (int64_t n = blockIdx.x; n < N; n += gridDim.x) {
        const T* row = w + n * K;
        RawChunk<T> raw[CPT];
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int64_t c = tid + static_cast<int64_t>(i) * nthr;
            if (c < chunks) raw[i] = load_raw(row, c);
        }
        float v[CPT][kChunk];
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int64_t c = tid + static_cast<int64_t>(i) * nthr;
            if (c < chunks) {
                float sv[kChunk];
                load_chunk(s, c, sv);
                unpack(raw[i], v[i]);
#pragma unroll
                for (int e = 0; e < kChunk; ++e) {
                    v[i][e] = v[i][e] * sv[e];
                    m = fmaxf(m, fabsf(v[i][e]));
                }
            }
        }
        m = wave_max(m);
        if ((tid & 63) == 0) red[tid >> 6] = m;
        __syncthreads();
        m = red[0];
        for (int i = 1; i < (nthr >> 6); ++i) m = fmaxf(m, red[i]);
        __syncthreads();  // red is reused by the next row
        const float d = step_from_absmax(m);
        const float rd = 1.0f / d;
        if (tid == 0) w_scale[n] = d;
        int8_t* orow = wq + n * K;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int64_t c = tid + static_cast<int64_t>(i) * nthr;
            if (c < chunks) {
                int q[kChunk];
#pragma unroll
                for (int e = 0; e < kChunk; ++e) q[e] = code_of(div_rn(v[i][e], d, rd));
                *reinterpret_cast<uint2*>(orow + c * kChunk) = pack8(q);
            }
        }
    }
}

// Any K: two sweeps over the row from memory (the second mostly hits L2).
template <typename T>
__global__ __launch_bounds__(256) void weight_quant_stream_kernel(
    const T* __restrict__ w, int64_t N, int64_t K, const float* __restrict__ s,
    int8_t* __restrict__ wq, float* __restrict__ w_scale) {
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int64_t chunks = K / kChunk;
    for (int64_t n = blockIdx.x; n < N; n += gridDim.x) {
        const T* row = w + n * K;
        float m = 0.0f;
        for (int64_t c = tid; c < chunks; c += 256) {
            float v[kChunk], sv[kChunk];
            load_chunk(row, c, v);
            load_chunk(s, c, sv);
#pragma unroll
            for (int e = 0; e < kChunk; ++e) m = fmaxf(m, fabsf(v[e] * sv[e]));
        }
        m = wave_max(m);
        if ((tid & 63) == 0) red[tid >> 6] = m;
        __syncthreads();
        m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        __syncthreads();
        const float d = step_from_absmax(m);
        const float rd = 1.0f / d;
        if (tid == 0) w_scale[n] = d;
        for (int64_t c = tid; c < chunks; c += 256) {
            float v[kChunk], sv[kChunk];
            load_chunk(row, c, v);
            load_chunk(s, c, sv);
            int q[kChunk];
#pragma unroll
            for (int e = 0; e < kChunk; ++e) q[e] = code_of(div_rn(v[e] * sv[e], d, rd));
            *reinterpret_cast<uint2*>(wq + n * K + c * kChunk) = pack8(q);
        }
    }
}

int round_up64(int64_t v) { return static_cast<int>(((v + 63) / 64) * 64); }

template <typename T>
hipError_t launch_weight_quant(const T* w, int64_t N, int64_t K, const float* s, int8_t* wq,
                               float* w_scale, hipStream_t stream) {
    if (N <= 0) return hipSuccess;
    const int64_t chunks = K / kChunk;
    int cpt = 1;
    while (cpt <= 8 && (chunks + cpt - 1) / cpt > 1024) cpt *= 2;
    if (cpt > 8) {
        const int64_t grid = std::min<int64_t>(N, 2048);
        weight_quant_stream_kernel<T><<<static_cast<unsigned>(grid), 256, 0, stream>>>(
            w, N, K, s, wq, w_scale);
        return hipGetLastError();
    }
    const int threads = std::max(64, round_up64((chunks + cpt - 1) / cpt));
    // enough resident blocks to keep ~16-32 waves per CU busy
    const int64_t per_cu = std::max(1, 2048 / threads);
    const int64_t grid = std::min<int64_t>(N, 256 * per_cu);
    const unsigned g = static_cast<unsigned>(grid);
    switch (cpt) {
        case 1: weight_quant_kernel<T, 1><<<g, threads, 0, stream>>>(w, N, K, s, wq, w_scale); break;
        case 2: weight_quant_kernel<T, 2><<<g, threads, 0, stream>>>(w, N, K, s, wq, w_scale); break;
        case 4: weight_quant_kernel<T, 4><<<g, threads, 0, stream>>>(w, N, K, s, wq, w_scale); break;
        default: weight_quant_kernel<T, 8><<<g, threads, 0, stream>>>(w, N, K, s, wq, w_scale); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_calibrate(const void* x_cal, Dt x_dt, int64_t T, const void* w, Dt w_dt,
                            int64_t N, int64_t K, float alpha, const float* gamma,
                            const float* beta, float* s, int8_t* wq, float* w_scale,
                            float* act_scale_static, float* gamma_s, float* beta_s,
                            float* x_absmax, float* w_absmax, hipStream_t stream) {
    uint32_t* xa = reinterpret_cast<uint32_t*>(x_absmax);
    uint32_t* wa = reinterpret_cast<uint32_t*>(w_absmax);
    uint32_t* sb = reinterpret_cast<uint32_t*>(act_scale_static);
    fill_maxima_kernel<<<static_cast<unsigned>((K + 255) / 256), 256, 0, stream>>>(xa, wa, K, sb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    e = (x_dt == Dt::BF16)
            ? launch_colmax(static_cast<const uint16_t*>(x_cal), T, K, xa, stream)
            : launch_colmax(static_cast<const float*>(x_cal), T, K, xa, stream);
    if (e != hipSuccess) return e;
    e = (w_dt == Dt::BF16) ? launch_colmax(static_cast<const uint16_t*>(w), N, K, wa, stream)
                           : launch_colmax(static_cast<const float*>(w), N, K, wa, stream);
    if (e != hipSuccess) return e;

    const int64_t fgrid = std::min<int64_t>((K + kFactorThreads - 1) / kFactorThreads, 1024);
    smooth_factor_kernel<<<static_cast<unsigned>(fgrid), kFactorThreads, 0, stream>>>(
        x_absmax, w_absmax, K, alpha, gamma, beta, s, gamma_s, beta_s, sb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    return (w_dt == Dt::BF16)
               ? launch_weight_quant(static_cast<const uint16_t*>(w), N, K, s, wq, w_scale, stream)
               : launch_weight_quant(static_cast<const float*>(w), N, K, s, wq, w_scale, stream);
}

}  // namespace sq
