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
//   colmax_partial  column |max| of X_cal and of W in one launch: 16-byte loads
//                   along K, rows split over the waves of a block and over
//                   blocks, per-block LDS combine, per-block maxima written to
//                   scratch rows (non-negative floats order like their bits)
//   smooth_factor   reduce the per-block maxima to a_j, w_j; s_j (fp64 powers,
//                   square roots at alpha = 1/2, one rounding), gamma/beta fold,
//                   static scale
//   (fallback when the scratch does not fit: fill_maxima + colmax with one
//   uint atomicMax per column per block)
//   weight_quant    per output row: What = W*s, row |max|, dw_n, codes; the row
//                   stays in registers between the max and the quantize passes
//   per-tensor weight step: max over n, k of |RN(W[n,k]*s_k)| equals
//                   max_k RN(max_n |W[n,k]| * s_k) (RN is monotone and s > 0), so
//                   the factor pass takes it from the raw column maxima and the
//                   codes need one pass over W, as per channel
#include <algorithm>

#include "sq_device.hpp"
#include "sq_internal.hpp"

namespace sq {
namespace {

constexpr uint32_t kFloorBits = 0x33d6bf95u;  // bit pattern of 1e-7f
static_assert(sizeof(float) == 4, "fp32");

// X_cal's maxima start at the floor; W's start at 0 (the raw maxima, floored by
// the factor pass, which also needs them unfloored for the per-tensor step).
__global__ void fill_maxima_kernel(uint32_t* __restrict__ xa, uint32_t* __restrict__ wa,
                                   int64_t K, uint32_t* __restrict__ static_bits,
                                   uint32_t* __restrict__ w_tensor_bits) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < K) {
        xa[i] = kFloorBits;
        wa[i] = 0u;
    }
    if (i == 0 && static_bits) *static_bits = 0u;
    if (i == 0 && w_tensor_bits) *w_tensor_bits = 0u;
}

// ---- column absmax ----------------------------------------------------------

constexpr int kColmaxThreads = 1024;  // 16 waves; each wave walks its own rows
constexpr int kColmaxWaves = kColmaxThreads / 64;

template <typename T>
struct ColmaxLane;

// bf16: one 16-byte load = 8 columns.  |x| is the 15-bit pattern with the sign
// cleared, kept two columns per 32-bit word and folded with one packed 16-bit
// unsigned maximum per word (two VALU operations per word instead of five;
// measured 8-11% faster for the pass on the OPT-6.7B shapes).
typedef unsigned short colmax_u16x2 __attribute__((ext_vector_type(2)));
template <>
struct ColmaxLane<uint16_t> {
    static constexpr int kCols = 8;
    colmax_u16x2 m[4];  // m[i] holds columns 2i (x) and 2i + 1 (y)
    __device__ void init() {
#pragma unroll
        for (int i = 0; i < 4; ++i) m[i] = colmax_u16x2{0, 0};
    }
    __device__ void add(const uint4& u) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            m[i] = __builtin_elementwise_max(m[i], __builtin_bit_cast(colmax_u16x2, w[i] & 0x7fff7fffu));
    }
    __device__ uint32_t f32_bits(int i) const {
        return static_cast<uint32_t>((i & 1) ? m[i >> 1].y : m[i >> 1].x) << 16;
    }
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

// Column |max| of rows [r_begin, r_end) of a row-major [rows, K] tensor over
// the kSeg columns of segment `seg`, combined over the block's waves in LDS.
// The block's result for column c is left in red[0][c] (as fp32 bit patterns,
// which order like the values since they are non-negative).
template <typename T>
__device__ __forceinline__ void colmax_block(const T* __restrict__ x, int64_t K, int64_t seg,
                                             int64_t r_begin, int64_t r_end,
                                             uint32_t (*red)[64 * ColmaxLane<uint16_t>::kCols]) {
    using Lane = ColmaxLane<T>;
    constexpr int kSeg = 64 * Lane::kCols;  // columns covered by one block
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t col = seg * kSeg + lane * Lane::kCols;

    Lane acc;
    acc.init();
    if (col < K) {
        const T* p = x + col;
        int64_t r = r_begin + wave;
        // batches of eight 16-byte loads per lane; the next batch is issued
        // before the current one is folded in (two batches in flight)
        constexpr int U = 8;
        constexpr int64_t kStep = U * kColmaxWaves;
        uint4 cur[U], nxt[U];
        auto load_batch = [&](int64_t r0, uint4 (&u)[U]) {
#pragma unroll
            for (int j = 0; j < U; ++j) {
                const int64_t rr = r0 + j * kColmaxWaves;
                u[j] = (rr < r_end) ? *reinterpret_cast<const uint4*>(p + rr * K) : make_uint4(0, 0, 0, 0);
            }
        };
        if (r < r_end) load_batch(r, cur);
        for (; r < r_end; r += kStep) {
            if (r + kStep < r_end) load_batch(r + kStep, nxt);
#pragma unroll
            for (int j = 0; j < U; ++j) acc.add(cur[j]);
#pragma unroll
            for (int j = 0; j < U; ++j) cur[j] = nxt[j];
        }
    }
#pragma unroll
    for (int i = 0; i < Lane::kCols; ++i) red[wave][lane * Lane::kCols + i] = acc.f32_bits(i);
    __syncthreads();
    for (int c = threadIdx.x; c < kSeg; c += kColmaxThreads) {
        uint32_t v = red[0][c];
#pragma unroll
        for (int w = 1; w < kColmaxWaves; ++w) v = max(v, red[w][c]);
        red[0][c] = v;
    }
    __syncthreads();
}

// Atomic variant: fold the block's maxima into out_bits (pre-filled with the
// floor) with one uint atomicMax per column.
template <typename T>
__global__ __launch_bounds__(kColmaxThreads) void colmax_kernel(
    const T* __restrict__ x, int64_t rows, int64_t K, int64_t rows_per_block,
    uint32_t* __restrict__ out_bits) {
    constexpr int kSeg = 64 * ColmaxLane<T>::kCols;
    __shared__ uint32_t red[kColmaxWaves][64 * ColmaxLane<uint16_t>::kCols];
    const int64_t r_begin = static_cast<int64_t>(blockIdx.y) * rows_per_block;
    const int64_t r_end = min(rows, r_begin + rows_per_block);
    colmax_block<T>(x, K, blockIdx.x, r_begin, r_end, red);
    for (int c = threadIdx.x; c < kSeg; c += kColmaxThreads) {
        const int64_t gc = static_cast<int64_t>(blockIdx.x) * kSeg + c;
        if (gc < K && red[0][c] > kFloorBits) atomicMax(out_bits + gc, red[0][c]);
    }
}

// Partial variant, X_cal and W in one launch: blocks [0, segs_x*splits_x) cover
// X_cal, the rest W; block (seg, split) writes its column maxima to row `split`
// of `partial` ([splits_x + splits_w, K] words), which the factor kernel
// reduces.  No fill and no atomics; block 0 also clears the static-scale word.
template <typename TX, typename TW>
__global__ __launch_bounds__(kColmaxThreads) void colmax_partial_kernel(
    const TX* __restrict__ x, int64_t T, const TW* __restrict__ w, int64_t N, int64_t K,
    int segs_x, int64_t rpb_x, int segs_w, int64_t rpb_w, int splits_x,
    uint32_t* __restrict__ partial, uint32_t* __restrict__ static_bits,
    uint32_t* __restrict__ w_tensor_bits) {
    __shared__ uint32_t red[kColmaxWaves][64 * ColmaxLane<uint16_t>::kCols];
    if (blockIdx.x == 0 && threadIdx.x == 0 && static_bits) *static_bits = 0u;
    if (blockIdx.x == 0 && threadIdx.x == 0 && w_tensor_bits) *w_tensor_bits = 0u;
    int64_t b = blockIdx.x;
    const int64_t nbx = static_cast<int64_t>(segs_x) * splits_x;
    if (b < nbx) {
        constexpr int kSeg = 64 * ColmaxLane<TX>::kCols;
        const int64_t seg = b % segs_x, split = b / segs_x;
        const int64_t r0 = split * rpb_x;
        colmax_block<TX>(x, K, seg, r0, min(T, r0 + rpb_x), red);
        uint32_t* out = partial + split * K;
        for (int c = threadIdx.x; c < kSeg; c += kColmaxThreads)
            if (seg * kSeg + c < K) out[seg * kSeg + c] = red[0][c];
    } else {
        b -= nbx;
        constexpr int kSeg = 64 * ColmaxLane<TW>::kCols;
        const int64_t seg = b % segs_w, split = b / segs_w;
        const int64_t r0 = split * rpb_w;
        colmax_block<TW>(w, K, seg, r0, min(N, r0 + rpb_w), red);
        uint32_t* out = partial + (splits_x + split) * K;
        for (int c = threadIdx.x; c < kSeg; c += kColmaxThreads)
            if (seg * kSeg + c < K) out[seg * kSeg + c] = red[0][c];
    }
}

template <typename T>
hipError_t launch_colmax(const T* x, int64_t rows, int64_t K, uint32_t* out_bits,
                         hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    constexpr int kSeg = 64 * ColmaxLane<T>::kCols;
    const int64_t bx = (K + kSeg - 1) / kSeg;
    // one resident block of 16 waves per CU over 256 CUs, at least 128 rows a
    // block (each wave keeps two batches of eight 16-byte loads in flight)
    const int64_t want = (256 + bx - 1) / bx;
    const int64_t max_split = (rows + 127) / 128;
    const int64_t by = std::max<int64_t>(1, std::min(want, max_split));
    const int64_t rpb = (rows + by - 1) / by;
    const int64_t by2 = (rows + rpb - 1) / rpb;
    dim3 grid(static_cast<unsigned>(bx), static_cast<unsigned>(by2));
    colmax_kernel<T><<<grid, kColmaxThreads, 0, stream>>>(x, rows, K, rpb, out_bits);
    return hipGetLastError();
}

// ---- smoothing factor, fold, static scale ------------------------------------

constexpr int kFactorCols = 64;   // columns per block, one per lane
constexpr int kFactorWaves = 4;   // waves that split a column's per-block maxima
constexpr int kFactorThreads = 64 * kFactorWaves;

// With `partial` set, first reduce the per-block column maxima of X_cal (rows
// [0, splits_x)) and W (rows [splits_x, splits_x + splits_w)) into a_j
// (floored) and W's raw column maximum; otherwise a holds a_j and w the raw
// maxima (atomic pass).  w_j = max(FLOOR, raw) is stored in w either way.  The
// pass is latency-bound: wave g of a block takes partial rows g, g + 4, ...
// of both matrices in the block's 64 columns (eight loads in flight per
// batch, so up to 32 partial rows cost one round trip), the four results meet
// in LDS, and wave 0 finishes the columns (eq. (4), fold, static scale, and
// with w_tensor_bits the largest smoothed weight RN(raw * s_j)).
__global__ __launch_bounds__(kFactorThreads) void smooth_factor_kernel(
    float* __restrict__ a, float* __restrict__ w, int64_t K, float alpha,
    const uint32_t* __restrict__ partial, int splits_x, int splits_w,
    const float* __restrict__ gamma, const float* __restrict__ beta, float* __restrict__ s,
    float* __restrict__ gamma_s, float* __restrict__ beta_s, uint32_t* __restrict__ static_bits,
    const float* __restrict__ act_stat, uint32_t* __restrict__ w_tensor_bits) {
    __shared__ uint32_t pm[2][kFactorWaves][kFactorCols];
    const int lane = threadIdx.x & 63;
    const int g = threadIdx.x >> 6;
    const double al = static_cast<double>(alpha);
    const double be = 1.0 - al;
    float local = 0.0f;
    float local_w = 0.0f;  // max of RN(raw w_j * s_j) over the block's columns
    for (int64_t j0 = static_cast<int64_t>(blockIdx.x) * kFactorCols; j0 < K;
         j0 += static_cast<int64_t>(gridDim.x) * kFactorCols) {
        const int64_t j = j0 + lane;
        if (partial) {
            // rows [0, splits_x) hold X_cal's maxima, the rest W's
            const int total = splits_x + splits_w;
            uint32_t mx = kFloorBits, mw = 0u;  // W's maximum raw here, floored below
            if (j < K) {
                for (int i = g; i < total; i += 8 * kFactorWaves) {
                    uint32_t v[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int r = i + u * kFactorWaves;
                        v[u] = (r < total) ? partial[static_cast<int64_t>(r) * K + j] : 0u;
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        if (i + u * kFactorWaves < splits_x) mx = max(mx, v[u]);
                        else mw = max(mw, v[u]);
                    }
                }
            }
            pm[0][g][lane] = mx;
            pm[1][g][lane] = mw;
        }
        __syncthreads();
        if (g == 0 && j < K) {
            float aj, wraw;
            if (partial) {
                uint32_t ab = pm[0][0][lane], wb = pm[1][0][lane];
#pragma unroll
                for (int q = 1; q < kFactorWaves; ++q) {
                    ab = max(ab, pm[0][q][lane]);
                    wb = max(wb, pm[1][q][lane]);
                }
                aj = __uint_as_float(ab);
                wraw = __uint_as_float(wb);
                a[j] = aj;
            } else {
                aj = a[j];
                wraw = w[j];
            }
            const float wj = fmaxf(wraw, kFloor);
            w[j] = wj;
            if (act_stat) {
                // a given per-channel activation statistic replaces the peak
                aj = fmaxf(act_stat[j], kFloor);
                a[j] = aj;
            }
            // eq. (4) in fp64, rounded once to fp32.  At alpha = 1/2 both powers
            // are square roots: the fp64 square root is the correctly rounded
            // x^(1/2), in a fraction of pow's instructions (0.6-0.8 us less per
            // call); pow itself may differ from it in the last fp64 bit, which
            // the rounding to fp32 absorbs unless the quotient lies within
            // 2^-52 of an fp32 rounding boundary
            const bool half = al == 0.5;
            const double pa = half ? __builtin_sqrt(static_cast<double>(aj))
                                   : pow(static_cast<double>(aj), al);
            const double pw = half ? __builtin_sqrt(static_cast<double>(wj))
                                   : pow(static_cast<double>(wj), be);
            const float sj = static_cast<float>(pa / pw);
            s[j] = sj;
            if (gamma) {
                gamma_s[j] = gamma[j] / sj;
                beta_s[j] = beta[j] / sj;
            }
            // RN(max(FLOOR, x)/127) is monotone in x, so the max of the per-channel
            // steps is the step of the max smoothed calibration peak RN(a_j/s_j).
            local = fmaxf(local, step_from_absmax(aj / sj));
            // the largest smoothed weight magnitude in column j is RN(raw w_j * s_j)
            local_w = fmaxf(local_w, wraw * sj);
        }
        __syncthreads();  // pm is refilled by the next columns
    }
    if (g != 0) return;
    // non-negative floats order like their bit patterns
    if (static_bits) {
        local = wave_max(local);
        if (lane == 0) atomicMax(static_bits, __float_as_uint(local));
    }
    if (w_tensor_bits) {
        local_w = wave_max(local_w);
        if (lane == 0) atomicMax(w_tensor_bits, __float_as_uint(local_w));
    }
}

// The per-tensor weight step from the maximum smoothed weight magnitude held
// as bits in the same word: RN(max(FLOOR, m) / 127).
__global__ void weight_tensor_step_kernel(uint32_t* word) {
    if (threadIdx.x == 0) {
        const float m = __uint_as_float(word[0]);
        reinterpret_cast<float*>(word)[0] = step_from_absmax(m);
    }
}

// ---- weight smoothing + per-output-channel quantization ------------------------


// One output row per block; lane t owns chunks t + i*blockDim (i < CPT).  With
// D > 0 the lane's slice of s is loaded once and kept in registers for every
// row the block walks, and the loads of the block's next D rows are in flight
// while the current row is reduced and quantized (a ring of D+1 rows).  The
// row stays in registers between the absmax and the quantize passes.
// What the weight kernels produce per row n (the argument `w_scale`):
//   kWChannel  step dw_n = RN(max(FLOOR, max_k |What|) / 127) into w_scale[n], codes
//   kWGiven    codes with the step read from w_scale[0] (per tensor), not written
enum WMode : int { kWChannel = 0, kWGiven = 2 };

template <typename T, int CPT, int D, int MAXT = 1024, int WM = kWChannel>
__global__ __launch_bounds__(MAXT) void weight_quant_kernel(
    const T* __restrict__ w, int64_t N, int64_t K, const float* __restrict__ s,
    int8_t* __restrict__ wq, float* __restrict__ w_scale) {
    __shared__ float red[2][16];  // alternate rows use alternate halves: one barrier per row
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int nw = nthr >> 6;
    const int64_t chunks = K / kChunk;
    const int64_t G = gridDim.x;
    constexpr bool CACHE = D > 0;
    const float d_given = (WM == kWGiven) ? w_scale[0] : 0.0f;
    const float rd_given = (WM == kWGiven) ? 1.0f / d_given : 0.0f;

    // Every load is issued unconditionally, so the compiler's waits count the
    // loads in flight exactly (a load skipped on some path makes it wait for
    // every load, which drained the prefetch at each row): a lane past the
    // row's end reads the row's last chunk (and the matching factors), which
    // leaves the row maximum unchanged and is never stored, and the last
    // row's prefetch re-reads the current row (an L2 hit).  The factors are
    // requested before the first row.  Measured on the MI355X against the
    // per-lane conditional loads, identical codes and steps, caches flushed
    // before each call: 12288 x 4096 bf16 27.7-28.6 us vs 29.3-29.8, 4096 x
    // 4096 13.8-14.2 vs 15.1-15.2, 4096 x 16384 36.5-36.7 vs 38.9-39.4,
    // 22016 x 8192 unchanged (88-92 us).
    auto lane_chunk = [&](int i) {
        return min(tid + static_cast<int64_t>(i) * nthr, chunks - 1);
    };
    float sv[CACHE ? CPT : 1][kChunk];
    if constexpr (CACHE) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) load_chunk(s, lane_chunk(i), sv[i]);
    }
    RawChunk<T> ring[D + 1][CPT];
    auto fetch = [&](int64_t n, RawChunk<T> (&r)[CPT]) {
        const T* row = w + n * K;
#pragma unroll
        for (int i = 0; i < CPT; ++i) r[i] = load_raw(row, lane_chunk(i));
    };
#pragma unroll
    for (int j = 0; j < D; ++j) fetch(min(blockIdx.x + j * G, N - 1), ring[j]);
    int parity = 0;
    for (int64_t n = blockIdx.x; n < N; n += G, parity ^= 1) {
        fetch(n + D * G < N ? n + D * G : n, ring[D]);
        float v[CPT][kChunk];
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            float sl[kChunk];
            if constexpr (CACHE) {
#pragma unroll
                for (int e = 0; e < kChunk; ++e) sl[e] = sv[i][e];
            } else {
                load_chunk(s, lane_chunk(i), sl);
            }
            unpack(ring[0][i], v[i]);
#pragma unroll
            for (int e = 0; e < kChunk; ++e) {
                v[i][e] = v[i][e] * sl[e];
                m = fmaxf(m, fabsf(v[i][e]));
            }
        }
        float d = d_given, rd = rd_given;
        if (WM != kWGiven) {
            m = wave_max(m);
            if (nw > 1) {
                // the next row writes the other half of red, and the row after
                // it passes this row's successor's barrier first, which every
                // wave reaches only after reading this half
                if ((tid & 63) == 0) red[parity][tid >> 6] = m;
                __syncthreads();
                m = red[parity][0];
                for (int i = 1; i < nw; ++i) m = fmaxf(m, red[parity][i]);
            }
            step_rcp(m, d, rd);
            if (tid == 0) w_scale[n] = d;
        }
        // the step comes from the row's maximum (or, given, from the tensor's,
        // which bounds every row): d = RN(max(FLOOR, m) / 127) >= m / 127 (1 - 2^-24),
        // so every quotient is at most 127.00001 in magnitude and the clamp of
        // the code cannot act: the code is taken without it (code_bits)
        int8_t* orow = wq + n * K;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int64_t c = tid + static_cast<int64_t>(i) * nthr;
            if (c < chunks) {
                uint32_t q[kChunk];
                chunk_codes<false>(v[i], d, rd, q);
                *reinterpret_cast<uint2*>(orow + c * kChunk) = pack8_bits(q);
            }
        }
#pragma unroll
        for (int j = 0; j < D; ++j)
#pragma unroll
            for (int i = 0; i < CPT; ++i) ring[j][i] = ring[j + 1][i];
    }
}

// Any K: two sweeps over the row from memory (the second mostly hits L2).
template <typename T, int WM = kWChannel>
__global__ __launch_bounds__(256) void weight_quant_stream_kernel(
    const T* __restrict__ w, int64_t N, int64_t K, const float* __restrict__ s,
    int8_t* __restrict__ wq, float* __restrict__ w_scale) {
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int64_t chunks = K / kChunk;
    const float d_given = (WM == kWGiven) ? w_scale[0] : 0.0f;
    for (int64_t n = blockIdx.x; n < N; n += gridDim.x) {
        const T* row = w + n * K;
        float d = d_given;
        if (WM != kWGiven) {
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
            d = step_from_absmax(m);
            if (tid == 0) w_scale[n] = d;
        }
        const float rd = 1.0f / d;
        for (int64_t c = tid; c < chunks; c += 256) {
            float v[kChunk], sv[kChunk];
            load_chunk(row, c, v);
            load_chunk(s, c, sv);
            uint32_t q[kChunk];  // no clamp needed, as in weight_quant_kernel
            float p[kChunk];
#pragma unroll
            for (int e = 0; e < kChunk; ++e) p[e] = v[e] * sv[e];
            chunk_codes<false>(p, d, rd, q);
            *reinterpret_cast<uint2*>(wq + n * K + c * kChunk) = pack8_bits(q);
        }
    }
}

// Per-channel step, bf16 rows of 4097-6144 chunks: the packed row stays in
// registers and RN(w s) is formed twice (for the row maximum, then for the
// codes) with s read from L2 both times, so only the packed row is held (115
// VGPRs, one block of 1024 lanes per CU).  Measured on the MI355X against the
// one-row kernel with the products held (12288 x 49152): 438 vs 534 us with
// flushed caches, 412 vs 502 us warm; identical codes and steps.  A form with
// the factors requested two chunks ahead, 32-bit offsets and every load and
// store issued was slower (12288 x 49152 431-455 us vs 380-402, 12288 x
// 36864 365-400 vs 287-302).
template <int CPT, int NT>
__global__ __launch_bounds__(NT, 2) void weight_quant_recompute_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, const float* __restrict__ s,
    int8_t* __restrict__ wq, float* __restrict__ w_scale) {
    __shared__ float red[2][NT / 64];  // alternate rows use alternate halves
    const int tid = threadIdx.x;
    const int64_t chunks = K / kChunk;
    int parity = 0;
    for (int64_t n = blockIdx.x; n < N; n += gridDim.x, parity ^= 1) {
        RawChunk<uint16_t> raw[CPT];
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int64_t c = tid + static_cast<int64_t>(i) * NT;
            if (c < chunks) raw[i] = load_raw(w + n * K, c);
        }
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int64_t c = tid + static_cast<int64_t>(i) * NT;
            if (c < chunks) {
                float v[kChunk], sv[kChunk];
                load_chunk(s, c, sv);
                unpack(raw[i], v);
#pragma unroll
                for (int e = 0; e < kChunk; ++e) m = fmaxf(m, fabsf(v[e] * sv[e]));
            }
        }
        m = wave_max(m);
        if ((tid & 63) == 0) red[parity][tid >> 6] = m;
        __syncthreads();
        m = red[parity][0];
#pragma unroll
        for (int i = 1; i < NT / 64; ++i) m = fmaxf(m, red[parity][i]);
        float d, rd;
        step_rcp(m, d, rd);
        if (tid == 0) w_scale[n] = d;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int64_t c = tid + static_cast<int64_t>(i) * NT;
            if (c < chunks) {
                float v[kChunk], sv[kChunk];
                load_chunk(s, c, sv);
                unpack(raw[i], v);
                uint32_t q[kChunk];  // the row's own step: no clamp (weight_quant_kernel)
                float p[kChunk];
#pragma unroll
                for (int e = 0; e < kChunk; ++e) p[e] = v[e] * sv[e];
                chunk_codes<false>(p, d, rd, q);
                *reinterpret_cast<uint2*>(wq + n * K + c * kChunk) = pack8_bits(q);
            }
        }
    }
}

// Given (per-tensor) step: each code depends only on W[n,k], s_k and the step,
// so long rows are mapped elementwise.  Block b covers column segment
// b % segs (NT chunks, one per lane, s in registers) over row group b / segs,
// RU rows' loads in flight per lane.  Same arithmetic as weight_quant_kernel.
template <typename T, int NT, int RU>
__global__ __launch_bounds__(NT) void weight_quant_given_stream_kernel(
    const T* __restrict__ w, int64_t N, int64_t K, const float* __restrict__ s,
    int8_t* __restrict__ wq, const float* __restrict__ w_scale, int segs, int64_t rpb) {
    const int64_t chunks = K / kChunk;
    const int64_t seg = blockIdx.x % segs, rg = blockIdx.x / segs;
    const int64_t c = seg * NT + threadIdx.x;
    const int64_t r0 = rg * rpb, r1 = min(N, r0 + rpb);
    if (c >= chunks || r0 >= N) return;
    float sv[kChunk];
    load_chunk(s, c, sv);
    const float d = w_scale[0];
    const float rd = 1.0f / d;
    for (int64_t n = r0; n < r1; n += RU) {
        RawChunk<T> raw[RU];
#pragma unroll
        for (int u = 0; u < RU; ++u)
            if (n + u < r1) raw[u] = load_raw(w + (n + u) * K, c);
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            if (n + u < r1) {
                float v[kChunk];
                unpack(raw[u], v);
                uint32_t q[kChunk];  // the tensor's step bounds every quotient (no clamp)
                float p[kChunk];
#pragma unroll
                for (int e = 0; e < kChunk; ++e) p[e] = v[e] * sv[e];
                chunk_codes<false>(p, d, rd, q);
                *reinterpret_cast<uint2*>(wq + (n + u) * K + c * kChunk) = pack8_bits(q);
            }
        }
    }
}

template <typename T, int WM>
hipError_t launch_weight_quant_mode(const T* w, int64_t N, int64_t K, const float* s, int8_t* wq,
                                    float* ws, hipStream_t stream) {
    if (N <= 0) return hipSuccess;
    const int64_t chunks = K / kChunk;
    if (WM == kWGiven && chunks >= 1024) {
        // rows of 8192 elements or more with the per-tensor step: elementwise,
        // about 4096 blocks of 256 lanes (as the activation side's per-tensor map).
        // Measured against the row kernel in its given-step mode, identical codes,
        // warm / flushed caches: 12288 x 12288 bf16 90 vs 107 / 126 vs 133 us,
        // 36864 x 12288 292 vs 312 / 330 vs 339 us; at 4096 columns mixed (-5% .. +5%)
        constexpr int NT = 256, RU = 4;
        const int segs = static_cast<int>((chunks + NT - 1) / NT);
        const int64_t groups = std::max<int64_t>(1, std::min<int64_t>((N + RU - 1) / RU, 4096 / segs));
        const int64_t rpb = (N + groups - 1) / groups;
        const int64_t nblk = static_cast<int64_t>(segs) * ((N + rpb - 1) / rpb);
        weight_quant_given_stream_kernel<T, NT, RU><<<static_cast<unsigned>(nblk), NT, 0, stream>>>(
            w, N, K, s, wq, ws, segs, rpb);
        return hipGetLastError();
    }
    // Measured on the MI355X: one prefetched row (D = 1) beats deeper rings, and
    // bf16 rows stream best with four 16-byte loads per lane (fp32 rows with
    // two, which keeps the prefetch ring within the register budget).  Rows
    // beyond 4096 chunks use eight loads per lane without prefetch (up to 768
    // lanes), longer ones the two-sweep kernel.
    if (chunks > 8 * 768) {
        const int64_t grid = std::min<int64_t>(N, 2048);
        weight_quant_stream_kernel<T, WM><<<static_cast<unsigned>(grid), 256, 0, stream>>>(
            w, N, K, s, wq, ws);
        return hipGetLastError();
    }
    constexpr bool kBf16 = sizeof(T) == 2;
    if (kBf16 && WM == kWChannel && chunks > 4096 && chunks <= 6 * 1024) {
        const unsigned g = static_cast<unsigned>(std::min<int64_t>(N, 512));
        weight_quant_recompute_kernel<6, 1024><<<g, 1024, 0, stream>>>(
            reinterpret_cast<const uint16_t*>(w), N, K, s, wq, ws);
        return hipGetLastError();
    }
    int cpt, d;
    if (chunks <= 64) { cpt = 1; d = 1; }
    else if (chunks <= (kBf16 ? 256 : 2048)) { cpt = 2; d = 1; }
    else if (chunks <= 4096) { cpt = 4; d = kBf16 ? 1 : 0; }
    else { cpt = 8; d = 0; }
    const int threads = std::max(64, round_up64((chunks + cpt - 1) / cpt));
    const int64_t per_cu = std::max(1, 1024 / threads);
    const unsigned g = static_cast<unsigned>(std::min<int64_t>(N, 256 * per_cu));
    if (cpt == 1) weight_quant_kernel<T, 1, 1, 1024, WM><<<g, threads, 0, stream>>>(w, N, K, s, wq, ws);
    else if (cpt == 2) weight_quant_kernel<T, 2, 1, 1024, WM><<<g, threads, 0, stream>>>(w, N, K, s, wq, ws);
    else if (cpt == 4 && d == 1) weight_quant_kernel<T, kBf16 ? 4 : 2, 1, 1024, WM><<<g, threads, 0, stream>>>(w, N, K, s, wq, ws);
    else if (cpt == 4) weight_quant_kernel<T, 4, 0, 1024, WM><<<g, threads, 0, stream>>>(w, N, K, s, wq, ws);
    else weight_quant_kernel<T, 8, 0, 768, WM><<<g, threads, 0, stream>>>(w, N, K, s, wq, ws);
    return hipGetLastError();
}

// One pass over W: per output channel the kernel finds each row's step; per
// tensor the step is already in w_scale[0] (from the factor pass).
template <typename T>
hipError_t launch_weight_quant(const T* w, int64_t N, int64_t K, const float* s, int8_t* wq,
                               float* w_scale, bool per_tensor, hipStream_t stream) {
    if (!per_tensor) return launch_weight_quant_mode<T, kWChannel>(w, N, K, s, wq, w_scale, stream);
    return launch_weight_quant_mode<T, kWGiven>(w, N, K, s, wq, w_scale, stream);
}

// One block: step[0] = RN(max(FLOOR, max_i m[i]) / 127) over non-negative maxima.
__global__ __launch_bounds__(1024) void tensor_step_kernel(const float* __restrict__ m, int64_t n,
                                                           float* __restrict__ step) {
    __shared__ float red[16];
    float v = 0.0f;
    for (int64_t i = threadIdx.x; i < n; i += 1024) v = fmaxf(v, m[i]);
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < 16; ++i) v = fmaxf(v, red[i]);
        step[0] = step_from_absmax(v);
    }
}


}  // namespace

namespace {

struct Split {
    int segs = 0;
    int splits = 0;
    int64_t rpb = 0;
};

// X_cal and W in one launch of equal blocks: every block covers one column
// segment (1 KB of a row for either dtype) over the same number of rows r, the
// least r >= 128 for which all blocks fit in one round of 256 (one 16-wave
// block per CU); separate splits of X_cal and W would leave a second round of
// blocks on some CUs.
void plan_joint(int64_t T, int64_t N, int64_t K, int seg_x, int seg_w, Split& px, Split& pw) {
    px = Split{};
    pw = Split{};
    const int sx = T > 0 ? static_cast<int>((K + seg_x - 1) / seg_x) : 0;
    const int sw = N > 0 ? static_cast<int>((K + seg_w - 1) / seg_w) : 0;
    if (sx + sw == 0) return;
    const int64_t rowsegs = T * sx + N * sw;
    int64_t r = std::max<int64_t>(128, (rowsegs + 255) / 256);
    const int64_t rmax = std::max<int64_t>(T, N);
    for (;;) {
        const int64_t blocks = sx * ((T + r - 1) / r) + sw * ((N + r - 1) / r);
        if (blocks <= 256 || r >= rmax) break;
        r += std::max<int64_t>(1, r / 32);
    }
    if (T > 0) {
        px.segs = sx;
        px.splits = static_cast<int>((T + r - 1) / r);
        px.rpb = (T + px.splits - 1) / px.splits;
    }
    if (N > 0) {
        pw.segs = sw;
        pw.splits = static_cast<int>((N + r - 1) / r);
        pw.rpb = (N + pw.splits - 1) / pw.splits;
    }
}

template <typename TX, typename TW>
hipError_t launch_partial(const TX* x, int64_t T, const TW* w, int64_t N, int64_t K,
                          const Split& px, const Split& pw, uint32_t* partial,
                          uint32_t* static_bits, uint32_t* w_tensor_bits, hipStream_t stream) {
    const int64_t blocks = static_cast<int64_t>(px.segs) * px.splits +
                           static_cast<int64_t>(pw.segs) * pw.splits;
    colmax_partial_kernel<TX, TW><<<static_cast<unsigned>(blocks), kColmaxThreads, 0, stream>>>(
        x, T, w, N, K, px.segs, px.rpb, pw.segs, pw.rpb, px.splits, partial, static_bits,
        w_tensor_bits);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_tensor_step(const float* maxima, int64_t n, float* step, hipStream_t stream) {
    tensor_step_kernel<<<1, 1024, 0, stream>>>(maxima, n, step);
    return hipGetLastError();
}

hipError_t launch_calibrate(const void* x_cal, Dt x_dt, int64_t T, const void* w, Dt w_dt,
                            int64_t N, int64_t K, float alpha, bool w_per_tensor, const float* gamma,
                            const float* beta, float* s, int8_t* wq, float* w_scale,
                            float* act_scale_static, float* gamma_s, float* beta_s,
                            float* x_absmax, float* w_absmax, const float* act_stat,
                            hipStream_t stream) {
    if (act_stat) T = 0;  // the calibration activations are not read
    uint32_t* xa = reinterpret_cast<uint32_t*>(x_absmax);
    uint32_t* wa = reinterpret_cast<uint32_t*>(w_absmax);
    uint32_t* sb = reinterpret_cast<uint32_t*>(act_scale_static);
    // per tensor: w_scale[0] first holds the bits of the largest smoothed weight
    // magnitude (zeroed by the first kernel, raised by the factor pass), then the step
    uint32_t* wt = w_per_tensor ? reinterpret_cast<uint32_t*>(w_scale) : nullptr;
    hipError_t e;

    // The per-block column maxima need (splits_x + splits_w) * K words of
    // scratch; the int8 weight output, written only by the last kernel, holds
    // them when it is large enough.  Otherwise: fill + atomic column maxima.
    Split px, pw;
    plan_joint(T, N, K, x_dt == Dt::BF16 ? 512 : 256, w_dt == Dt::BF16 ? 512 : 256, px, pw);
    const int64_t need = static_cast<int64_t>(px.splits + pw.splits) * K * 4;
    const bool use_partial = N > 0 && need <= N * K;
    uint32_t* partial = use_partial ? reinterpret_cast<uint32_t*>(wq) : nullptr;
    if (use_partial) {
        if (x_dt == Dt::BF16 && w_dt == Dt::BF16)
            e = launch_partial(static_cast<const uint16_t*>(x_cal), T, static_cast<const uint16_t*>(w), N, K, px, pw, partial, sb, wt, stream);
        else if (x_dt == Dt::BF16)
            e = launch_partial(static_cast<const uint16_t*>(x_cal), T, static_cast<const float*>(w), N, K, px, pw, partial, sb, wt, stream);
        else if (w_dt == Dt::BF16)
            e = launch_partial(static_cast<const float*>(x_cal), T, static_cast<const uint16_t*>(w), N, K, px, pw, partial, sb, wt, stream);
        else
            e = launch_partial(static_cast<const float*>(x_cal), T, static_cast<const float*>(w), N, K, px, pw, partial, sb, wt, stream);
        if (e != hipSuccess) return e;
    } else {
        fill_maxima_kernel<<<static_cast<unsigned>((K + 255) / 256), 256, 0, stream>>>(xa, wa, K, sb, wt);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = (x_dt == Dt::BF16)
                ? launch_colmax(static_cast<const uint16_t*>(x_cal), T, K, xa, stream)
                : launch_colmax(static_cast<const float*>(x_cal), T, K, xa, stream);
        if (e != hipSuccess) return e;
        e = (w_dt == Dt::BF16) ? launch_colmax(static_cast<const uint16_t*>(w), N, K, wa, stream)
                               : launch_colmax(static_cast<const float*>(w), N, K, wa, stream);
        if (e != hipSuccess) return e;
    }

    const int64_t fgrid = std::min<int64_t>((K + kFactorCols - 1) / kFactorCols, 1024);
    smooth_factor_kernel<<<static_cast<unsigned>(fgrid), kFactorThreads, 0, stream>>>(
        x_absmax, w_absmax, K, alpha, partial, px.splits, pw.splits, gamma, beta, s, gamma_s,
        beta_s, sb, act_stat, wt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (w_per_tensor) {
        // with no rows the maximum is 0 and the step FLOOR / 127
        weight_tensor_step_kernel<<<1, 64, 0, stream>>>(wt);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }

    if (N == 0) return hipSuccess;
    return (w_dt == Dt::BF16)
               ? launch_weight_quant(static_cast<const uint16_t*>(w), N, K, s, wq, w_scale,
                                     w_per_tensor, stream)
               : launch_weight_quant(static_cast<const float*>(w), N, K, s, wq, w_scale,
                                     w_per_tensor, stream);
}

}  // namespace sq
