// act_quant.hip -- runtime activation side: smooth, then int8-quantize, in one
// HBM pass.
//
//   [Review] "SmoothQuant：大型语言模型的精准高效训练后量化 — 深度技术评审"
//   §5.1 eq. (3): the activation is divided per input channel by s
//   (X diag(s)^-1); §2.2 the symmetric quantizer (step = max|X|/127, round to
//   nearest); §2.5 dynamic vs static scales; §2.6 / Fig. 3 per-token scales.
//   [Edge] "嵌入式 SLM 动态权重量化：SmoothQuant 激活异常值迁移与 INT8 部署实战"
//   §二: the LayerNorm with gamma/s and beta/s folded in emits the smoothed
//   activation directly, followed by int8 quantization.
//
// act_quant_kernel: one token row per block.  The block's lanes own fixed
// chunks of 8 elements (chunk c = tid + i*blockDim), so per-column data
// (1/s_k, rcp_rn) is computed once per block and reused across the rows the
// block walks.  The row stays in registers between the absmax reduction and
// the quantize pass.  Divisions by s_k and by the step use div_rn() (correctly
// rounded, five VALU ops; three for x / s_k when x is bf16, div_x).  LayerNorm
// mode uses exactly 256 lanes so that lane t owns partial t of the canonical
// fp32 reduction (chunk c -> partial c mod 256, increasing k within a partial,
// then the fixed halving tree).
// act_quant_rows_kernel packs several short rows (K <= 256) into a wave;
// act_quant_stream_kernel re-reads long rows per sweep.  All three share the
// per-element arithmetic and have a row-maximum pass (the first pass of the
// dynamic per-tensor step) and a count mode (the static quantizer's
// saturation count, no codes written).
#include <algorithm>

#include "sq_device.hpp"
#include "sq_internal.hpp"

namespace sq {
namespace {

constexpr int kLnThreads = 256;

// Block-wide max of non-negative values; every lane receives the result.
// `red` holds two slots of 16 floats used by alternate rows (parity), so one
// barrier separates a call's writes from its reads: the next call writes the
// other slot, and the call after it passes that call's barrier first, which
// every wave reaches only after reading this slot.
__device__ __forceinline__ float block_max(float v, float* red, int parity) {
    v = wave_max(v);
    const int nw = blockDim.x >> 6;
    if (nw == 1) return v;
    float* r = red + (parity & 1) * 16;
    if ((threadIdx.x & 63) == 0) r[threadIdx.x >> 6] = v;
    __syncthreads();
    float m = r[0];
    for (int i = 1; i < nw; ++i) m = fmaxf(m, r[i]);
    return m;
}

// Canonical halving tree over the 256 lane partials:
// p[i] = p[i] + p[i+d] for d = 128, 64, ..., 1.  Every lane gets p[0].  After
// one barrier each wave evaluates the whole tree itself from the partials in
// `part` (256 floats, one region per reduction of a row: the row's other
// barriers lie between a region's reads and its next writes): lane l forms
// (p[l] + p[l+128]) + (p[l+64] + p[l+192]), which is p[l] after d = 64, and
// the steps d = 32..1 run on the wave's lanes.
__device__ __forceinline__ float canonical_tree(float p, float* part) {
    const int tid = threadIdx.x;
    part[tid] = p;
    __syncthreads();
    const int l = tid & 63;
    const float a = part[l] + part[l + 128];
    const float b = part[l + 64] + part[l + 192];
    float v = a + b;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = v + __shfl_down(v, d, 64);
    return __shfl(v, 0, 64);
}

// RN(1/s) of a chunk's eight column factors (rcp_rn), with the range test taken
// once for the chunk: the short sequence when every factor lies in
// [2^-126, 2^126), the IEEE division otherwise.
__device__ __forceinline__ void rcp_chunk(const float (&sv)[kChunk], float (&rs)[kChunk]) {
    float lo = sv[0], hi = sv[0];
#pragma unroll
    for (int e = 1; e < kChunk; ++e) {
        lo = fminf(lo, sv[e]);
        hi = fmaxf(hi, sv[e]);
    }
    if (lo >= 0x1p-126f && hi < 0x1p126f) {
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
            const float r = __builtin_amdgcn_rcpf(sv[e]);
            rs[e] = __builtin_fmaf(__builtin_fmaf(-sv[e], r, 1.0f), r, r);
        }
    } else {
#pragma unroll
        for (int e = 0; e < kChunk; ++e) rs[e] = 1.0f / sv[e];
    }
}

// Quantize one smoothed value with step d (rd = RN(1/d)).  In static mode the
// dividend is first limited to +-128 d (exact scaling by a power of two), which
// keeps the quotient finite and leaves every code unchanged: a quotient beyond
// 127.5 saturates to +-127 either way.
template <bool STATIC>
__device__ __forceinline__ int quantize(float xh, float d, float rd) {
    if (STATIC) {
        const float lim = 128.0f * d;
        xh = fminf(fmaxf(xh, -lim), lim);
    }
    return code_of(div_rn(xh, d, rd));
}

// Whether the static quantizer saturates xh: its rounded quotient (after the
// same dividend limit as quantize) lies outside [-127, 127].
__device__ __forceinline__ bool saturates(float xh, float d, float rd) {
    const float lim = 128.0f * d;
    xh = fminf(fmaxf(xh, -lim), lim);
    return fabsf(__builtin_rintf(div_rn(xh, d, rd))) > kQmax;
}

// Count mode of the static kernels (clip != nullptr): element k of a row
// that saturates adds 1 to clip_ch[k] (if given) and to the lane's count; the
// counts of a wave are summed and added to *clip once at the end.
__device__ __forceinline__ void count_clips(const float (&v)[kChunk], float d, float rd,
                                            int64_t c, uint32_t* clip_ch, int& n) {
#pragma unroll
    for (int e = 0; e < kChunk; ++e) {
        if (saturates(v[e], d, rd)) {
            ++n;
            if (clip_ch) atomicAdd(clip_ch + c * kChunk + e, 1u);
        }
    }
}

__device__ __forceinline__ void flush_clips(int n, unsigned long long* clip) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) n += __shfl_xor(n, o, 64);
    if ((threadIdx.x & 63) == 0 && n > 0) atomicAdd(clip, static_cast<unsigned long long>(n));
}

// D > 0: the lane's per-column constants (s_k and RN(1/s_k) in plain mode,
// gamma'_k and beta'_k in LayerNorm mode) are loaded once per block and kept in
// registers, and the loads of the block's next D rows are in flight while the
// current row is reduced and quantized (a ring of D+1 rows of 16-byte chunks).
// D = 0: the constants are re-read per row (L2 hits), 1/s_k is an IEEE
// division, and nothing is prefetched.
// clip != nullptr (static mode only): count mode, see count_clips; no codes.
// rowmax != nullptr (dynamic modes only): the row pass that stores the raw
// maximum max_k |xh_k| of every row in rowmax[m] and writes neither codes nor
// x_scale -- the first pass of the dynamic per-tensor step.
template <typename T, bool LN, bool STATIC, int CPT, int D, int MAXT, bool CACHE_ = (D > 0)>
__global__ __launch_bounds__(MAXT) void act_quant_kernel(
    const T* __restrict__ x, int64_t M, int64_t K, const float* __restrict__ s,
    const float* __restrict__ gs, const float* __restrict__ bs, float eps,
    const float* __restrict__ static_scale, int8_t* __restrict__ xq,
    float* __restrict__ x_scale, float* __restrict__ rowmax, unsigned long long* __restrict__ clip,
    uint32_t* __restrict__ clip_ch) {
    // [0, 256): mean partials, [256, 512): variance partials, [512, 544): row maxima
    __shared__ float lds[2 * kLnThreads + 32];
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int64_t chunks = K / kChunk;
    const float kf = static_cast<float>(K);
    constexpr bool CACHE = CACHE_;
    constexpr int CC = CACHE ? CPT : 1;
    const int64_t G = gridDim.x;

    RawChunk<T> ring[D + 1][CPT];
    auto fetch = [&](int64_t m, RawChunk<T> (&r)[CPT]) {
        const T* row = x + m * K;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int64_t c = tid + static_cast<int64_t>(i) * nthr;
            if (c < chunks) r[i] = load_raw(row, c);
        }
    };
    // the first rows' loads go out before the per-column set-up below
#pragma unroll
    for (int j = 0; j < D; ++j)
        if (blockIdx.x + j * G < M) fetch(blockIdx.x + j * G, ring[j]);

    // per-column constants: c0 = s (plain) or gamma' (LN); c1 = 1/s or beta'
    float c0[CC][kChunk], c1[CC][kChunk];
    if (CACHE) {
#pragma unroll
        for (int i = 0; i < CC; ++i) {
            const int64_t c = tid + static_cast<int64_t>(i) * nthr;
            if (c < chunks) {
                if (LN) {
                    load_chunk(gs, c, c0[i]);
                    load_chunk(bs, c, c1[i]);
                } else {
                    load_chunk(s, c, c0[i]);
#pragma unroll
                    for (int e = 0; e < kChunk; ++e) c1[i][e] = rcp_rn(c0[i][e]);
                }
            }
        }
    }
    float d_static = 0.0f, rd_static = 0.0f;
    if (STATIC) {
        d_static = *static_scale;
        rd_static = 1.0f / d_static;
    }
    int nclip = 0;
    int parity = 0;
    for (int64_t m = blockIdx.x; m < M; m += G, parity ^= 1) {
        if (m + D * G < M) fetch(m + D * G, ring[D]);
        float v[CPT][kChunk];
#pragma unroll
        for (int i = 0; i < CPT; ++i) unpack(ring[0][i], v[i]);

        if (LN) {
            // mean: canonical sum of x
            float p = 0.0f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int64_t c = tid + static_cast<int64_t>(i) * nthr;
                if (c < chunks) {
#pragma unroll
                    for (int e = 0; e < kChunk; ++e) p = p + v[i][e];
                }
            }
            const float mu = canonical_tree(p, lds) / kf;
            // biased variance: canonical sum of RN(d*d)
            p = 0.0f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int64_t c = tid + static_cast<int64_t>(i) * nthr;
                if (c < chunks) {
#pragma unroll
                    for (int e = 0; e < kChunk; ++e) {
                        v[i][e] = v[i][e] - mu;
                        const float dd = v[i][e] * v[i][e];
                        p = p + dd;
                    }
                }
            }
            const float var = canonical_tree(p, lds + kLnThreads) / kf;
            const float rho = 1.0f / __builtin_sqrtf(var + eps);
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int64_t c = tid + static_cast<int64_t>(i) * nthr;
                if (c < chunks) {
                    float g[kChunk], b[kChunk];
                    if (CACHE) {
#pragma unroll
                        for (int e = 0; e < kChunk; ++e) {
                            g[e] = c0[CACHE ? i : 0][e];
                            b[e] = c1[CACHE ? i : 0][e];
                        }
                    } else {
                        load_chunk(gs, c, g);
                        load_chunk(bs, c, b);
                    }
#pragma unroll
                    for (int e = 0; e < kChunk; ++e) {
                        float t = v[i][e] * rho;
                        t = t * g[e];
                        v[i][e] = t + b[e];
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int64_t c = tid + static_cast<int64_t>(i) * nthr;
                if (c < chunks) {
                    if (CACHE) {
#pragma unroll
                        for (int e = 0; e < kChunk; ++e)
                            v[i][e] = div_x<T>(v[i][e], c0[CACHE ? i : 0][e], c1[CACHE ? i : 0][e]);
                    } else {
                        float sv[kChunk];
                        load_chunk(s, c, sv);
                        {
                            float rs[kChunk];
                            rcp_chunk(sv, rs);
#pragma unroll
                            for (int e = 0; e < kChunk; ++e) v[i][e] = div_x<T>(v[i][e], sv[e], rs[e]);
                        }
                    }
                }
            }
        }

        float d, rd;
        if (STATIC) {
            d = d_static;
            rd = rd_static;
        } else {
            float mx = 0.0f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int64_t c = tid + static_cast<int64_t>(i) * nthr;
                if (c < chunks) {
#pragma unroll
                    for (int e = 0; e < kChunk; ++e) mx = fmaxf(mx, fabsf(v[i][e]));
                }
            }
            mx = block_max(mx, lds + 2 * kLnThreads, parity);
            d = step_from_absmax(mx);
            rd = 1.0f / d;
            if (tid == 0) {
                if (rowmax) rowmax[m] = mx;
                else x_scale[m] = d;
            }
        }
        if (STATIC && clip) {
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int64_t c = tid + static_cast<int64_t>(i) * nthr;
                if (c < chunks) count_clips(v[i], d, rd, c, clip_ch, nclip);
            }
        } else if (STATIC || rowmax == nullptr) {
            int8_t* orow = xq + m * K;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int64_t c = tid + static_cast<int64_t>(i) * nthr;
                if (c < chunks) {
                    int q[kChunk];
#pragma unroll
                    for (int e = 0; e < kChunk; ++e) q[e] = quantize<STATIC>(v[i][e], d, rd);
                    *reinterpret_cast<uint2*>(orow + c * kChunk) = pack8(q);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < D; ++j)
#pragma unroll
            for (int i = 0; i < CPT; ++i) ring[j][i] = ring[j + 1][i];
    }
    if (STATIC && clip) flush_clips(nclip, clip);
}

// Short rows (plain mode, K <= 256: at most 32 chunks).  A wave quantizes
// 64 / SG rows at once, SG lanes per row (SG = the chunk count rounded up to a
// power of two): lane l owns chunk l % SG of row l / SG, so its s_k and
// RN(1/s_k) stay in registers, and the row maximum is reduced within the
// lane's SG-lane group.  The next group of rows is in flight while the current
// one is quantized.  Per element the arithmetic is that of act_quant_kernel.
template <typename T, bool STATIC, int SG>
__global__ __launch_bounds__(256) void act_quant_rows_kernel(
    const T* __restrict__ x, int64_t M, int64_t K, const float* __restrict__ s,
    const float* __restrict__ static_scale, int8_t* __restrict__ xq,
    float* __restrict__ x_scale, float* __restrict__ rowmax, unsigned long long* __restrict__ clip,
    uint32_t* __restrict__ clip_ch) {
    constexpr int R = 64 / SG;
    const int lane = threadIdx.x & 63;
    const int r = lane / SG, c = lane % SG;
    const int64_t chunks = K / kChunk;
    const bool act = c < chunks;
    const int64_t W = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 6);
    const int64_t groups = (M + R - 1) / R;
    int64_t g = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);

    RawChunk<T> cur{}, nxt{};
    auto fetch = [&](int64_t gg, RawChunk<T>& rc) {
        const int64_t m = gg * R + r;
        if (act && m < M) rc = load_raw(x + m * K, c);
    };
    if (g < groups) fetch(g, cur);
    float c0[kChunk], c1[kChunk];
    if (act) {
        load_chunk(s, c, c0);
#pragma unroll
        for (int e = 0; e < kChunk; ++e) c1[e] = rcp_rn(c0[e]);
    } else {
#pragma unroll
        for (int e = 0; e < kChunk; ++e) c0[e] = c1[e] = 1.0f;
    }
    float d_static = 0.0f, rd_static = 0.0f;
    if (STATIC) {
        d_static = *static_scale;
        rd_static = 1.0f / d_static;
    }
    int nclip = 0;
    for (; g < groups; g += W) {
        if (g + W < groups) fetch(g + W, nxt);
        const int64_t m = g * R + r;
        const bool live = act && m < M;
        float v[kChunk];
        unpack(cur, v);
#pragma unroll
        for (int e = 0; e < kChunk; ++e) v[e] = div_x<T>(v[e], c0[e], c1[e]);
        float d, rd;
        if (STATIC) {
            d = d_static;
            rd = rd_static;
        } else {
            float mx = 0.0f;
            if (live) {
#pragma unroll
                for (int e = 0; e < kChunk; ++e) mx = fmaxf(mx, fabsf(v[e]));
            }
#pragma unroll
            for (int o = SG / 2; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
            d = step_from_absmax(mx);
            rd = 1.0f / d;
            if (c == 0 && m < M) {
                if (rowmax) rowmax[m] = mx;
                else x_scale[m] = d;
            }
        }
        if (STATIC && clip) {
            if (live) count_clips(v, d, rd, c, clip_ch, nclip);
        } else if ((STATIC || rowmax == nullptr) && live) {
            int q[kChunk];
#pragma unroll
            for (int e = 0; e < kChunk; ++e) q[e] = quantize<STATIC>(v[e], d, rd);
            *reinterpret_cast<uint2*>(xq + m * K + c * kChunk) = pack8(q);
        }
        cur = nxt;
    }
    if (STATIC && clip) flush_clips(nclip, clip);
}

// Any K: the row is re-read from memory for each sweep (mostly L2 hits).
// 256 lanes, so LayerNorm partials are canonical here too.
template <typename T, bool LN>
__device__ __forceinline__ void smooth_chunk(const T* row, int64_t c, const float* s,
                                             const float* gs, const float* bs, float mu,
                                             float rho, float (&v)[kChunk]) {
    load_chunk(row, c, v);
    if (LN) {
        float g[kChunk], b[kChunk];
        load_chunk(gs, c, g);
        load_chunk(bs, c, b);
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
            const float dlt = v[e] - mu;
            float t = dlt * rho;
            t = t * g[e];
            v[e] = t + b[e];
        }
    } else {
        float sv[kChunk];
        load_chunk(s, c, sv);
        {
            float rs[kChunk];
            rcp_chunk(sv, rs);
#pragma unroll
            for (int e = 0; e < kChunk; ++e) v[e] = div_x<T>(v[e], sv[e], rs[e]);
        }
    }
}

template <typename T, bool LN, bool STATIC>
__global__ __launch_bounds__(kLnThreads) void act_quant_stream_kernel(
    const T* __restrict__ x, int64_t M, int64_t K, const float* __restrict__ s,
    const float* __restrict__ gs, const float* __restrict__ bs, float eps,
    const float* __restrict__ static_scale, int8_t* __restrict__ xq,
    float* __restrict__ x_scale, float* __restrict__ rowmax, unsigned long long* __restrict__ clip,
    uint32_t* __restrict__ clip_ch) {
    // [0, 256): mean partials, [256, 512): variance partials, [512, 544): row maxima
    __shared__ float lds[2 * kLnThreads + 32];
    const int tid = threadIdx.x;
    const int64_t chunks = K / kChunk;
    const float kf = static_cast<float>(K);
    int nclip = 0;
    int parity = 0;
    for (int64_t m = blockIdx.x; m < M; m += gridDim.x, parity ^= 1) {
        const T* row = x + m * K;
        float mu = 0.0f, rho = 0.0f;
        if (LN) {
            float p = 0.0f;
            for (int64_t c = tid; c < chunks; c += kLnThreads) {
                float v[kChunk];
                load_chunk(row, c, v);
#pragma unroll
                for (int e = 0; e < kChunk; ++e) p = p + v[e];
            }
            mu = canonical_tree(p, lds) / kf;
            p = 0.0f;
            for (int64_t c = tid; c < chunks; c += kLnThreads) {
                float v[kChunk];
                load_chunk(row, c, v);
#pragma unroll
                for (int e = 0; e < kChunk; ++e) {
                    const float dlt = v[e] - mu;
                    const float dd = dlt * dlt;
                    p = p + dd;
                }
            }
            const float var = canonical_tree(p, lds + kLnThreads) / kf;
            rho = 1.0f / __builtin_sqrtf(var + eps);
        }
        float d, rd;
        if (STATIC) {
            d = *static_scale;
        } else {
            float mx = 0.0f;
            for (int64_t c = tid; c < chunks; c += kLnThreads) {
                float v[kChunk];
                smooth_chunk<T, LN>(row, c, s, gs, bs, mu, rho, v);
#pragma unroll
                for (int e = 0; e < kChunk; ++e) mx = fmaxf(mx, fabsf(v[e]));
            }
            mx = block_max(mx, lds + 2 * kLnThreads, parity);
            d = step_from_absmax(mx);
            if (rowmax) {
                if (tid == 0) rowmax[m] = mx;
                continue;
            }
            if (tid == 0) x_scale[m] = d;
        }
        rd = 1.0f / d;
        for (int64_t c = tid; c < chunks; c += kLnThreads) {
            float v[kChunk];
            smooth_chunk<T, LN>(row, c, s, gs, bs, mu, rho, v);
            if (STATIC && clip) {
                count_clips(v, d, rd, c, clip_ch, nclip);
                continue;
            }
            int q[kChunk];
#pragma unroll
            for (int e = 0; e < kChunk; ++e) q[e] = quantize<STATIC>(v[e], d, rd);
            *reinterpret_cast<uint2*>(xq + m * K + c * kChunk) = pack8(q);
        }
    }
    if (STATIC && clip) flush_clips(nclip, clip);
}

struct ActArgs {
    const void* x;
    int64_t M, K;
    const float *s, *gs, *bs;
    float eps;
    const float* static_scale;
    int8_t* xq;
    float* x_scale;
    float* rowmax;  // non-null: row-maximum pass (dynamic per-tensor step)
    unsigned long long* clip = nullptr;  // non-null: count mode of the static quantizer
    uint32_t* clip_ch = nullptr;         // per-channel counts in count mode (optional)
};

template <typename T, bool LN, bool STATIC, int CPT, int D, int MAXT = 1024>
hipError_t run(const ActArgs& a, int threads, hipStream_t stream) {
    // resident blocks: about 16 waves per CU, each block walks several rows
    const int64_t per_cu = std::max(1, 1024 / threads);
    const unsigned grid = static_cast<unsigned>(std::min<int64_t>(a.M, 256 * per_cu));
    act_quant_kernel<T, LN, STATIC, CPT, D, MAXT><<<grid, threads, 0, stream>>>(
        static_cast<const T*>(a.x), a.M, a.K, a.s, a.gs, a.bs, a.eps, a.static_scale, a.xq,
        a.x_scale, a.rowmax, a.clip, a.clip_ch);
    return hipGetLastError();
}

template <typename T, bool LN, bool STATIC>
hipError_t run_stream(const ActArgs& a, hipStream_t stream) {
    const unsigned grid = static_cast<unsigned>(std::min<int64_t>(a.M, 2048));
    act_quant_stream_kernel<T, LN, STATIC><<<grid, kLnThreads, 0, stream>>>(
        static_cast<const T*>(a.x), a.M, a.K, a.s, a.gs, a.bs, a.eps, a.static_scale, a.xq,
        a.x_scale, a.rowmax, a.clip, a.clip_ch);
    return hipGetLastError();
}


template <typename T, bool STATIC, int SG>
hipError_t run_rows(const ActArgs& a, hipStream_t stream) {
    // four waves per block, at most eight blocks per CU; each wave walks
    // groups of 64 / SG rows
    const int64_t groups = (a.M + 64 / SG - 1) / (64 / SG);
    const unsigned grid = static_cast<unsigned>(std::min<int64_t>((groups + 3) / 4, 256 * 8));
    act_quant_rows_kernel<T, STATIC, SG><<<grid, 256, 0, stream>>>(
        static_cast<const T*>(a.x), a.M, a.K, a.s, a.static_scale, a.xq, a.x_scale, a.rowmax,
        a.clip, a.clip_ch);
    return hipGetLastError();
}

template <typename T, bool STATIC>
hipError_t dispatch_plain(const ActArgs& a, hipStream_t stream) {
    const int64_t chunks = a.K / kChunk;
    // short rows: several rows per wave
    if (chunks <= 8) return run_rows<T, STATIC, 8>(a, stream);
    if (chunks <= 16) return run_rows<T, STATIC, 16>(a, stream);
    if (chunks <= 32) return run_rows<T, STATIC, 32>(a, stream);
    // rows up to 2048 chunks: one or two 16-byte loads per lane and row with the
    // per-column constants cached and the next row prefetched (measured: one
    // prefetched row beats deeper rings on the MI355X); longer rows:
    // four (up to 1024 lanes) or eight (up to 768 lanes) loads per lane without
    // caching; past that the multi-sweep kernel
    if (chunks <= 64) return run<T, false, STATIC, 1, 1>(a, 64, stream);
    if (chunks <= 2048) return run<T, false, STATIC, 2, 1>(a, round_up64((chunks + 1) / 2), stream);
    if (chunks <= 4 * 1024) return run<T, false, STATIC, 4, 0>(a, round_up64((chunks + 3) / 4), stream);
    if (chunks <= 8 * 768)
        return run<T, false, STATIC, 8, 0, 768>(a, round_up64((chunks + 7) / 8), stream);
    return run_stream<T, false, STATIC>(a, stream);
}

template <typename T, bool STATIC>
hipError_t dispatch_ln(const ActArgs& a, hipStream_t stream) {
    const int64_t chunks = a.K / kChunk;
    const int64_t need = (chunks + kLnThreads - 1) / kLnThreads;
    if (need <= 1) return run<T, true, STATIC, 1, 1, kLnThreads>(a, kLnThreads, stream);
    if (need <= 2) return run<T, true, STATIC, 2, 1, kLnThreads>(a, kLnThreads, stream);
    if (need <= 4) return run<T, true, STATIC, 4, 1, kLnThreads>(a, kLnThreads, stream);
    if (need <= 8) return run<T, true, STATIC, 8, 0, kLnThreads>(a, kLnThreads, stream);
    return run_stream<T, true, STATIC>(a, stream);
}

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * 256)
        p[i] = 0u;
}

hipError_t zero_words(uint32_t* p, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const unsigned grid = static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 1024));
    zero_words_kernel<<<grid, 256, 0, stream>>>(p, n);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const ActArgs& a, bool ln, bool st, hipStream_t stream) {
    if (ln) return st ? dispatch_ln<T, true>(a, stream) : dispatch_ln<T, false>(a, stream);
    return st ? dispatch_plain<T, true>(a, stream) : dispatch_plain<T, false>(a, stream);
}

}  // namespace

hipError_t launch_clip_count(const void* x, Dt x_dt, int64_t M, int64_t K, const float* s,
                             const float* gamma_s, const float* beta_s, float eps,
                             const float* static_scale, unsigned long long* clip,
                             uint32_t* clip_ch, hipStream_t stream) {
    hipError_t e = zero_words(reinterpret_cast<uint32_t*>(clip), 2, stream);
    if (e == hipSuccess && clip_ch) e = zero_words(clip_ch, K, stream);
    if (e != hipSuccess || M <= 0) return e;
    const bool ln = (s == nullptr);
    ActArgs a{x, M, K, s, gamma_s, beta_s, eps, static_scale, nullptr, nullptr, nullptr, clip,
              clip_ch};
    return (x_dt == Dt::BF16) ? dispatch<uint16_t>(a, ln, true, stream)
                              : dispatch<float>(a, ln, true, stream);
}

hipError_t launch_act_quant(const void* x, Dt x_dt, int64_t M, int64_t K, const float* s,
                            const float* gamma_s, const float* beta_s, float eps,
                            ActMode mode, const float* static_scale, int8_t* xq,
                            float* x_scale, hipStream_t stream) {
    if (M <= 0) {
        // an empty batch: the dynamic per-tensor step is FLOOR / 127
        return mode == ActMode::DynamicTensor ? launch_tensor_step(nullptr, 0, x_scale, stream)
                                              : hipSuccess;
    }
    const bool ln = (s == nullptr);
    auto go = [&](const ActArgs& a, bool st) {
        return (x_dt == Dt::BF16) ? dispatch<uint16_t>(a, ln, st, stream)
                                  : dispatch<float>(a, ln, st, stream);
    };
    if (mode != ActMode::DynamicTensor)
        return go(ActArgs{x, M, K, s, gamma_s, beta_s, eps, static_scale, xq, x_scale, nullptr},
                  mode == ActMode::Static);
    // dynamic per tensor: row maxima (staged in xq, 4M <= M*K bytes), the
    // one-block reduction into x_scale[0], then the static quantizer with it
    float* rowmax = reinterpret_cast<float*>(xq);
    hipError_t e = go(ActArgs{x, M, K, s, gamma_s, beta_s, eps, nullptr, xq, nullptr, rowmax},
                      false);
    if (e != hipSuccess) return e;
    e = launch_tensor_step(rowmax, M, x_scale, stream);
    if (e != hipSuccess) return e;
    return go(ActArgs{x, M, K, s, gamma_s, beta_s, eps, x_scale, xq, nullptr, nullptr}, true);
}

}  // namespace sq
