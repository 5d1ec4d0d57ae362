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
// the quantize pass.  Divisions by s_k use div_rn() (correctly rounded, five
// VALU ops; three when x is bf16, div_x); the codes come from chunk_codes
// (rne of the correctly rounded quotient by the step, without the division
// except where a half-integer lies within its error bound).  LayerNorm
// mode uses exactly 256 lanes so that lane t owns partial t of the canonical
// fp32 reduction (chunk c -> partial c mod 256, increasing k within a partial,
// then the fixed halving tree).
// act_quant_rows_kernel packs several short rows (K <= 256) into a wave;
// act_quant_stream_kernel re-reads long rows per sweep.  All three share the
// per-element arithmetic and have a row-maximum pass (the first pass of the
// dynamic per-tensor step) and a count mode (the static quantizer's
// saturation count, no codes written).
// act_quant_multi_kernel (plain) and act_quant_ln2_kernel (LayerNorm) take two
// bf16 rows per block; act_quant_static_stream_kernel maps long rows
// elementwise when the step is per tensor; act_quant_long_kernel holds one
// long plain row per block for the per-token step, with the row's factors
// requested at the row's start and the next row's chunks during the codes;
// act_quant_ln_row_kernel is the LayerNorm-mode codes kernel for rows of
// 1025-2048 chunks.  Same arithmetic per element.
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

// Quantize a chunk of eight smoothed values with step d (rd = RN(1/d)); each
// code is the low byte of its word (chunk_codes: rne(RN(xh / d)), clamped in
// static mode).  In static mode the dividends are first limited to +-128 d
// (exact scaling by a power of two), which keeps the quotients finite and
// leaves every code unchanged: a quotient beyond 127.5 saturates to +-127
// either way.  With a step taken from the row's (or the batch's) own maximum
// m, d = RN(max(FLOOR, m) / 127) >= m / 127 (1 - 2^-24), so |xh / d| <=
// 127.00001 and the clamp cannot change a code: it is skipped.
template <bool STATIC>
__device__ __forceinline__ void quantize_chunk(const float (&xh)[kChunk], float d, float rd,
                                               uint32_t (&q)[kChunk]) {
    if constexpr (STATIC) {
        const float lim = 128.0f * d;
        float x[kChunk];
#pragma unroll
        for (int e = 0; e < kChunk; ++e) x[e] = fminf(fmaxf(xh[e], -lim), lim);
        chunk_codes<true>(x, d, rd, q);
    } else {
        chunk_codes<false>(xh, d, rd, q);
    }
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

    // Every row and constant load is issued, so the compiler's waits count the
    // loads in flight exactly (a load skipped on some path makes it wait for
    // all of them, the prefetch just issued included): a chunk past the row's
    // end reads the row's last chunk and every use of it is guarded, and a
    // prefetch past the batch re-reads the block's current row (an L2 hit).
    auto lane_chunk = [&](int i) { return min(tid + static_cast<int64_t>(i) * nthr, chunks - 1); };
    RawChunk<T> ring[D + 1][CPT];
    auto fetch = [&](int64_t m, RawChunk<T> (&r)[CPT]) {
        const T* row = x + m * K;
#pragma unroll
        for (int i = 0; i < CPT; ++i) r[i] = load_raw(row, lane_chunk(i));
    };
    // the first rows' loads go out before the per-column set-up below
#pragma unroll
    for (int j = 0; j < D; ++j) fetch(min(blockIdx.x + j * G, M - 1), ring[j]);

    // per-column constants: c0 = s (plain) or gamma' (LN); c1 = 1/s or beta'
    float c0[CC][kChunk], c1[CC][kChunk];
    if (CACHE) {
#pragma unroll
        for (int i = 0; i < CC; ++i) {
            if (LN) {
                load_chunk(gs, lane_chunk(i), c0[i]);
                load_chunk(bs, lane_chunk(i), c1[i]);
            } else {
                load_chunk(s, lane_chunk(i), c0[i]);
#pragma unroll
                for (int e = 0; e < kChunk; ++e) c1[i][e] = rcp_rn(c0[i][e]);
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
        fetch(m + D * G < M ? m + D * G : m, ring[D]);
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
            step_rcp(mx, d, rd);
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
                    uint32_t q[kChunk];
                    quantize_chunk<STATIC>(v[i], d, rd, q);
                    *reinterpret_cast<uint2*>(orow + c * kChunk) = pack8_bits(q);
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

// Per-token codes of long plain rows (2048 < chunks <= 6144 with 1024 lanes):
// one row per block in registers, CPT chunks per lane.  The lane's factors
// s_k are requested at the start of each row (L2 hits, one round trip per
// row), the row's own chunks having been requested while the previous row
// was quantized; each chunk is unpacked and divided once its data are in (a
// scheduling barrier per chunk keeps the compiler from holding every
// factor and reciprocal at once), one barrier forms the row maximum, and
// the next row's chunks are requested before this row's codes are formed
// and stored.  Whether every factor lies in [2^-126, 2^126), where
// RN(1/s_k) takes the two-fma sequence of rcp_rn, is decided once per block
// (FAST); otherwise the IEEE division forms it.  Addresses are uniform bases
// plus 32-bit byte offsets (rows and s stay far below 4 GiB: K <= SQ_MAX_K).
// Per element the arithmetic is that of act_quant_kernel.
template <typename T>
__device__ __forceinline__ RawChunk<T> gload_raw(g_cchar* row, uint32_t c);
template <>
__device__ __forceinline__ RawChunk<uint16_t> gload_raw<uint16_t>(g_cchar* row, uint32_t c) {
    return RawChunk<uint16_t>{gload16(row + c * 16u)};
}
template <>
__device__ __forceinline__ RawChunk<float> gload_raw<float>(g_cchar* row, uint32_t c) {
    return RawChunk<float>{gload16(row + c * 32u), gload16(row + c * 32u + 16u)};
}

template <typename T, int CPT, int SP, bool FAST>
__device__ __forceinline__ void long_rows(const T* __restrict__ x, int64_t M, int64_t K,
                                          const float* __restrict__ s, int8_t* __restrict__ xq,
                                          float* __restrict__ x_scale, float* red) {
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int chunks = static_cast<int>(K / kChunk);
    const int64_t G = gridDim.x;
    uint32_t off[CPT];  // the lane's chunk indices, clamped into the row
    bool ok[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int c = tid + i * nthr;
        ok[i] = c < chunks;
        off[i] = static_cast<uint32_t>(min(c, chunks - 1));
    }
    RawChunk<T> ring[CPT];
    int64_t m = blockIdx.x;
    if (m < M) {
        g_cchar* xr = (g_cchar*)(x + m * K);
#pragma unroll
        for (int i = 0; i < CPT; ++i) ring[i] = gload_raw<T>(xr, off[i]);
    }
    int parity = 0;
    for (; m < M; m += G, parity ^= 1) {
        // an opaque factor base and opaque copies of the offsets keep the
        // loads and their address arithmetic in the loop (hoisted, 64-bit
        // addresses would hold registers for the whole row)
        g_cchar* sb = (g_cchar*)s;
        asm volatile("" : "+s"(sb));
        uint32_t o[CPT];
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            o[i] = off[i];
            asm volatile("" : "+v"(o[i]));
        }
        // factors of SP chunks in flight: chunk i's turn requests chunk i + SP
        float sf[CPT][kChunk];
        auto load_sf = [&](int i) { gload8f(sb + o[i] * 32u, sf[i]); };
#pragma unroll
        for (int i = 0; i < SP; ++i) load_sf(i);
        __builtin_amdgcn_sched_barrier(0);
        float v[CPT][kChunk];
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            // no branch on ok[i]: a lane past the row's end holds a copy of the
            // row's last chunk, which leaves the row maximum unchanged, and
            // every lane then passes the same waits
            if (i + SP < CPT) load_sf(i + SP);
            unpack(ring[i], v[i]);
#pragma unroll
            for (int e = 0; e < kChunk; ++e) {
                const float b = sf[i][e];
                float rb;
                if constexpr (FAST) {
                    const float r = __builtin_amdgcn_rcpf(b);
                    rb = __builtin_fmaf(__builtin_fmaf(-b, r, 1.0f), r, r);
                } else {
                    rb = 1.0f / b;
                }
                v[i][e] = div_x<T>(v[i][e], b, rb);
                mx = fmaxf(mx, fabsf(v[i][e]));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        mx = block_max(mx, red, parity);
        float d, rd;
        step_rcp(mx, d, rd);
        if (tid == 0) x_scale[m] = d;
        if (m + G < M) {
            g_cchar* xr = (g_cchar*)(x + (m + G) * K);
#pragma unroll
            for (int i = 0; i < CPT; ++i) ring[i] = gload_raw<T>(xr, o[i]);
        }
        g_char* orow = (g_char*)(xq + m * K);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            uint32_t q[kChunk];
            quantize_chunk<false>(v[i], d, rd, q);
            const uint2 packed = pack8_bits(q);
            if (ok[i]) gstore8(orow + o[i] * 8u, packed);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

template <typename T, int CPT>
__global__ __launch_bounds__(1024) void act_quant_long_kernel(
    const T* __restrict__ x, int64_t M, int64_t K, const float* __restrict__ s,
    int8_t* __restrict__ xq, float* __restrict__ x_scale) {
    __shared__ float red[32];
    const int64_t chunks = K / kChunk;
    int in_range = 1;
    for (int64_t c = threadIdx.x; c < chunks; c += blockDim.x) {
        float sv[kChunk];
        load_chunk(s, c, sv);
#pragma unroll
        for (int e = 0; e < kChunk; ++e)
            in_range &= (sv[e] >= 0x1p-126f && sv[e] < 0x1p126f) ? 1 : 0;
    }
    constexpr int SP = CPT < 3 ? CPT : 3;
    if (__syncthreads_and(in_range))
        long_rows<T, CPT, SP, true>(x, M, K, s, xq, x_scale, red);
    else
        long_rows<T, CPT, SP, false>(x, M, K, s, xq, x_scale, red);
}

// R rows at once (plain mode, codes of the per-token or static quantizer):
// every thread holds its CPT chunks of each of R rows, so the factors s_k and
// RN(1/s_k) in its registers serve R rows, the R row maxima meet in one block
// reduction (one barrier for R rows), and the next R rows' loads are in flight
// while the current ones are reduced and quantized.  Per element the
// arithmetic is that of act_quant_kernel.
template <typename T, bool STATIC, int CPT, int R, int NT>
__global__ __launch_bounds__(NT) void act_quant_multi_kernel(
    const T* __restrict__ x, int64_t M, int64_t K, const float* __restrict__ s,
    const float* __restrict__ static_scale, int8_t* __restrict__ xq,
    float* __restrict__ x_scale) {
    constexpr int NW = NT / 64;
    __shared__ float red[2][R][NW];
    const int tid = threadIdx.x;
    const int64_t chunks = K / kChunk;
    const int64_t G = static_cast<int64_t>(gridDim.x) * R;
    RawChunk<T> raw[R][CPT];
    int64_t m0 = static_cast<int64_t>(blockIdx.x) * R;
    // the factors are requested before the first rows, so that their
    // reciprocals are formed while the rows are still in flight (loads
    // complete in order: requested after the rows, the factors would wait for
    // them); lanes past the row's end read its last chunk and use nothing.
    // Measured on the MI355X against the rows-first order, outputs identical,
    // caches flushed before each call: 2048 x 4096 11.5-11.7 us vs 12.4-12.7,
    // 2048 x 16384 24.8-25.2 vs 25.4-26.2, 4096 x 12288 34.9-35.8 vs 35.0-36.4
    float c0[CPT][kChunk], c1[CPT][kChunk];
#pragma unroll
    for (int i = 0; i < CPT; ++i)
        load_chunk(s, min(tid + static_cast<int64_t>(i) * NT, chunks - 1), c0[i]);
    __builtin_amdgcn_sched_barrier(0);
    // the block's first rows, without a branch per load (a skipped load would
    // make the compiler wait for every load before the first reciprocal): a
    // row past the batch (odd M) reads the last row and is never stored, a
    // chunk past the row's end reads its last chunk and is never used
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t m = min(m0 + r, M - 1);
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            raw[r][i] = load_raw(x + m * K, min(tid + static_cast<int64_t>(i) * NT, chunks - 1));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < CPT; ++i)
#pragma unroll
        for (int e = 0; e < kChunk; ++e) c1[i][e] = rcp_rn(c0[i][e]);
    float d_static = 0.0f, rd_static = 0.0f;
    if (STATIC) {
        d_static = *static_scale;
        rd_static = 1.0f / d_static;
    }
    int parity = 0;
    for (; m0 < M; m0 += G, parity ^= 1) {
        float v[R][CPT][kChunk];
        float mx[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            mx[r] = 0.0f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                // one chunk per lane: no branch (it made the compiler copy every
                // value back into place; 2048 x 4096 3-6% faster): a lane past
                // the row's end holds the row's last chunk and its factors,
                // which leave the maximum unchanged.  With two chunks per lane
                // the branch stays: without it the 1024-lane block needed
                // more than 128 VGPRs and spilled (6-9% slower)
                unpack(raw[r][i], v[r][i]);
                if (CPT == 1 || tid + static_cast<int64_t>(i) * NT < chunks) {
#pragma unroll
                    for (int e = 0; e < kChunk; ++e) {
                        v[r][i][e] = div_x<T>(v[r][i][e], c0[i][e], c1[i][e]);
                        mx[r] = fmaxf(mx[r], fabsf(v[r][i][e]));
                    }
                }
            }
        }
        {
            // the next rows, every load issued (the last group re-reads its
            // own rows from L2), so the compiler's wait for them at the top
            // of the loop counts exactly (conditional loads made it wait for
            // everything in flight): 2048 x 16384 24.5-25.2 us vs 24.9-26.2,
            // 4096 x 12288 34.1-36.3 vs 35.2-36.9 with flushed caches
            const int64_t mn = (m0 + G < M) ? m0 + G : m0;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int64_t m = min(mn + r, M - 1);
#pragma unroll
                for (int i = 0; i < CPT; ++i)
                    raw[r][i] = load_raw(x + m * K, min(tid + static_cast<int64_t>(i) * NT, chunks - 1));
            }
        }
        if (!STATIC) {
            // red[parity] is rewritten two row groups later, after the barrier
            // of the next group, which every wave passes only after this read
#pragma unroll
            for (int r = 0; r < R; ++r) mx[r] = wave_max(mx[r]);
            if ((tid & 63) == 0) {
#pragma unroll
                for (int r = 0; r < R; ++r) red[parity][r][tid >> 6] = mx[r];
            }
            __syncthreads();
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float m = red[parity][r][0];
#pragma unroll
                for (int w = 1; w < NW; ++w) m = fmaxf(m, red[parity][r][w]);
                mx[r] = m;
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = m0 + r;
            if (row >= M) continue;
            float d, rd;
            if (STATIC) {
                d = d_static;
                rd = rd_static;
            } else {
                step_rcp(mx[r], d, rd);
                if (tid == 0) x_scale[row] = d;
            }
            int8_t* orow = xq + row * K;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int64_t c = tid + static_cast<int64_t>(i) * NT;
                if (c < chunks) {
                    uint32_t q[kChunk];
                    quantize_chunk<STATIC>(v[r][i], d, rd, q);
                    *reinterpret_cast<uint2*>(orow + c * kChunk) = pack8_bits(q);
                }
            }
        }
    }
}

// Plain mode with a per-tensor step (static, or the second pass of the dynamic
// per-tensor step): each element's code depends only on x, s_k and the step,
// so the map is streamed with no row structure.  Block b covers column segment
// b % segs (NT chunks, one per lane) over row group b / segs; the lane's s and
// RN(1/s) stay in registers, and the loads of RU rows are in flight at once.
// Same per-element arithmetic as act_quant_kernel in static mode.
template <typename T, int NT, int RU>
__global__ __launch_bounds__(NT) void act_quant_static_stream_kernel(
    const T* __restrict__ x, int64_t M, int64_t K, const float* __restrict__ s,
    const float* __restrict__ static_scale, int8_t* __restrict__ xq, int segs, int64_t rpb) {
    const int64_t chunks = K / kChunk;
    const int64_t seg = blockIdx.x % segs, rg = blockIdx.x / segs;
    const int64_t c = seg * NT + threadIdx.x;
    const int64_t r0 = rg * rpb, r1 = min(M, r0 + rpb);
    if (c >= chunks || r0 >= M) return;
    float sv[kChunk], rs[kChunk];
    load_chunk(s, c, sv);
    rcp_chunk(sv, rs);
    const float d = *static_scale;
    const float rd = 1.0f / d;
    for (int64_t m = r0; m < r1; m += RU) {
        RawChunk<T> raw[RU];
#pragma unroll
        for (int u = 0; u < RU; ++u)
            if (m + u < r1) raw[u] = load_raw(x + (m + u) * K, c);
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            if (m + u < r1) {
                float v[kChunk];
                unpack(raw[u], v);
                uint32_t q[kChunk];
                float xh[kChunk];
#pragma unroll
                for (int e = 0; e < kChunk; ++e) xh[e] = div_x<T>(v[e], sv[e], rs[e]);
                quantize_chunk<true>(xh, d, rd, q);
                *reinterpret_cast<uint2*>(xq + (m + u) * K + c * kChunk) = pack8_bits(q);
            }
        }
    }
}

// Plain mode, the first pass of the dynamic per-tensor step on long rows: the
// largest |RN(x / s_k)| of the whole batch needs no row structure either.  The
// column-segment layout of act_quant_static_stream_kernel; each block leaves
// its maximum in partial[blockIdx.x] for the one-block reduction.
template <typename T, int NT, int RU>
__global__ __launch_bounds__(NT) void act_absmax_stream_kernel(
    const T* __restrict__ x, int64_t M, int64_t K, const float* __restrict__ s,
    float* __restrict__ partial, int segs, int64_t rpb) {
    __shared__ float red[NT / 64];
    const int tid = threadIdx.x;
    const int64_t chunks = K / kChunk;
    const int64_t seg = blockIdx.x % segs, rg = blockIdx.x / segs;
    const int64_t c = seg * NT + tid;
    const bool ok = c < chunks;
    const int64_t cc = ok ? c : chunks - 1;  // idle lanes read a valid chunk, count nothing
    const int64_t r0 = rg * rpb, r1 = min(M, r0 + rpb);
    float sv[kChunk], rs[kChunk];
    load_chunk(s, cc, sv);
    rcp_chunk(sv, rs);
    float mx = 0.0f;
    for (int64_t m = r0; m < r1; m += RU) {
        RawChunk<T> raw[RU];
#pragma unroll
        for (int u = 0; u < RU; ++u)
            if (m + u < r1) raw[u] = load_raw(x + (m + u) * K, cc);
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            if (ok && m + u < r1) {
                float v[kChunk];
                unpack(raw[u], v);
#pragma unroll
                for (int e = 0; e < kChunk; ++e) mx = fmaxf(mx, fabsf(div_x<T>(v[e], sv[e], rs[e])));
            }
        }
    }
    mx = wave_max(mx);
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    if (tid == 0) {
        float m = red[0];
#pragma unroll
        for (int w = 1; w < NT / 64; ++w) m = fmaxf(m, red[w]);
        partial[blockIdx.x] = m;
    }
}

// LayerNorm mode, two rows at once (codes of the per-token or static
// quantizer): exactly 256 lanes, so lane t owns canonical partial t of both
// rows; the cached gamma'_k and beta'_k serve both rows, each of the three
// reductions (mean, variance, row maximum) takes one barrier for the two
// rows, and the next two rows' loads are in flight during the reductions.
// Per element the arithmetic is that of act_quant_kernel in LayerNorm mode.
// LDS reuse: a row pair writes part[0] before its first barrier and reads it
// before its second, part[1] between the second and third (static mode: after
// the second), and red after the third; every later write of an array comes
// after a barrier that all of its readers have passed.
template <typename T, bool STATIC, int CPT>
__global__ __launch_bounds__(kLnThreads) void act_quant_ln2_kernel(
    const T* __restrict__ x, int64_t M, int64_t K, const float* __restrict__ gs,
    const float* __restrict__ bs, float eps, const float* __restrict__ static_scale,
    int8_t* __restrict__ xq, float* __restrict__ x_scale) {
    constexpr int R = 2;
    constexpr int NW = kLnThreads / 64;
    __shared__ float part[2][R][kLnThreads];
    __shared__ float red[R][NW];
    const int tid = threadIdx.x;
    const int64_t chunks = K / kChunk;
    const float kf = static_cast<float>(K);
    const int64_t G = static_cast<int64_t>(gridDim.x) * R;
    RawChunk<T> raw[R][CPT];
    auto fetch = [&](int64_t m0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t m = m0 + r;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int64_t c = tid + static_cast<int64_t>(i) * kLnThreads;
                if (m < M && c < chunks) raw[r][i] = load_raw(x + m * K, c);
            }
        }
    };
    int64_t m0 = static_cast<int64_t>(blockIdx.x) * R;
    fetch(m0);
    float g[CPT][kChunk], b[CPT][kChunk];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int64_t c = tid + static_cast<int64_t>(i) * kLnThreads;
        if (c < chunks) {
            load_chunk(gs, c, g[i]);
            load_chunk(bs, c, b[i]);
        }
    }
    float d_static = 0.0f, rd_static = 0.0f;
    if (STATIC) {
        d_static = *static_scale;
        rd_static = 1.0f / d_static;
    }
    // the canonical halving tree of canonical_tree() over one row's partials
    auto tree = [&](const float* pp) {
        const int l = tid & 63;
        const float a = pp[l] + pp[l + 128];
        const float bb = pp[l + 64] + pp[l + 192];
        float t = a + bb;
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) t = t + __shfl_down(t, d, 64);
        return __shfl(t, 0, 64);
    };
    for (; m0 < M; m0 += G) {
        float v[R][CPT][kChunk];
        float p[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            p[r] = 0.0f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                unpack(raw[r][i], v[r][i]);
                const int64_t c = tid + static_cast<int64_t>(i) * kLnThreads;
                if (c < chunks) {
#pragma unroll
                    for (int e = 0; e < kChunk; ++e) p[r] = p[r] + v[r][i][e];
                }
            }
        }
        fetch(m0 + G);
        // mean: canonical sum of x
#pragma unroll
        for (int r = 0; r < R; ++r) part[0][r][tid] = p[r];
        __syncthreads();
        float mu[R];
#pragma unroll
        for (int r = 0; r < R; ++r) mu[r] = tree(part[0][r]) / kf;
        // biased variance: canonical sum of RN(d * d)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            p[r] = 0.0f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int64_t c = tid + static_cast<int64_t>(i) * kLnThreads;
                if (c < chunks) {
#pragma unroll
                    for (int e = 0; e < kChunk; ++e) {
                        v[r][i][e] = v[r][i][e] - mu[r];
                        const float dd = v[r][i][e] * v[r][i][e];
                        p[r] = p[r] + dd;
                    }
                }
            }
            part[1][r][tid] = p[r];
        }
        __syncthreads();
        float mx[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float var = tree(part[1][r]) / kf;
            const float rho = 1.0f / __builtin_sqrtf(var + eps);
            mx[r] = 0.0f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int64_t c = tid + static_cast<int64_t>(i) * kLnThreads;
                if (c < chunks) {
#pragma unroll
                    for (int e = 0; e < kChunk; ++e) {
                        float t = v[r][i][e] * rho;
                        t = t * g[i][e];
                        v[r][i][e] = t + b[i][e];
                        mx[r] = fmaxf(mx[r], fabsf(v[r][i][e]));
                    }
                }
            }
        }
        if (!STATIC) {
#pragma unroll
            for (int r = 0; r < R; ++r) mx[r] = wave_max(mx[r]);
            if ((tid & 63) == 0) {
#pragma unroll
                for (int r = 0; r < R; ++r) red[r][tid >> 6] = mx[r];
            }
            __syncthreads();
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float m = red[r][0];
#pragma unroll
                for (int w = 1; w < NW; ++w) m = fmaxf(m, red[r][w]);
                mx[r] = m;
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = m0 + r;
            if (row >= M) continue;
            float d, rd;
            if (STATIC) {
                d = d_static;
                rd = rd_static;
            } else {
                step_rcp(mx[r], d, rd);
                if (tid == 0) x_scale[row] = d;
            }
            int8_t* orow = xq + row * K;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int64_t c = tid + static_cast<int64_t>(i) * kLnThreads;
                if (c < chunks) {
                    uint32_t q[kChunk];
                    quantize_chunk<STATIC>(v[r][i], d, rd, q);
                    *reinterpret_cast<uint2*>(orow + c * kChunk) = pack8_bits(q);
                }
            }
        }
    }
}

// LayerNorm mode, codes of bf16 rows of 1025-2048 chunks (K 8200-16384).
// Measured on the MI355X against act_quant_kernel in LayerNorm mode, codes and
// steps identical, caches flushed before each call: 4096 x 9216 38.7-39.4 us
// vs 47.7-49.1, 4096 x 12288 44.7-46.3 vs 53.8-55.7, 4096 x 16384 58.3-60.4 vs
// 63.7-67.8; a form with four rows per 1024-lane block and the factors staged
// in LDS was slower than either (4096 x 12288 81 us).  One row per block of
// exactly 256 lanes (lane t owns canonical partial t: chunks
// t + 256 i, increasing k within the partial, then the fixed halving tree), as
// in act_quant_kernel, without its count and row-maximum passes.  Every load
// is issued (clamped indices; a chunk past the row's end is never used), so
// the compiler's waits count exactly; gamma'_k and beta'_k of the first SP
// chunks are requested before the mean reduction and each chunk's turn
// requests those SP chunks ahead, instead of one L2 round trip per chunk after
// the variance; a scheduling barrier per chunk bounds the registers held.
template <bool STATIC, int CPT, int SP>
__global__ __launch_bounds__(kLnThreads) void act_quant_ln_row_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const float* __restrict__ gs,
    const float* __restrict__ bs, float eps, const float* __restrict__ static_scale,
    int8_t* __restrict__ xq, float* __restrict__ x_scale) {
    __shared__ float lds[2 * kLnThreads + 32];
    const int t = threadIdx.x;
    const int chunks = static_cast<int>(K / kChunk);
    const float kf = static_cast<float>(K);
    float d_static = 0.0f, rd_static = 0.0f;
    if (STATIC) {
        d_static = *static_scale;
        rd_static = 1.0f / d_static;
    }
    int parity = 0;
    for (int64_t m = blockIdx.x; m < M; m += gridDim.x, parity ^= 1) {
        // uniform bases plus 32-bit offsets (K <= SQ_MAX_K), formed in the row
        // loop from opaque copies: the compiler neither hoists the factor loads
        // to the top of the row nor holds 64-bit addresses across it
        g_cchar* gb = (g_cchar*)gs;
        g_cchar* bb = (g_cchar*)bs;
        asm volatile("" : "+s"(gb), "+s"(bb));
        uint32_t o[CPT];
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            o[i] = static_cast<uint32_t>(min(t + i * kLnThreads, chunks - 1));
            asm volatile("" : "+v"(o[i]));
        }
        g_cchar* xr = (g_cchar*)(x + m * K);
        RawChunk<uint16_t> raw[CPT];
#pragma unroll
        for (int i = 0; i < CPT; ++i) raw[i] = RawChunk<uint16_t>{gload16(xr + o[i] * 16u)};
        float ga[CPT][kChunk], be[CPT][kChunk];
#pragma unroll
        for (int i = 0; i < SP; ++i) {
            gload8f(gb + o[i] * 32u, ga[i]);
            gload8f(bb + o[i] * 32u, be[i]);
        }
        float v[CPT][kChunk];
        float p = 0.0f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            unpack(raw[i], v[i]);
            if (t + i * kLnThreads < chunks) {
#pragma unroll
                for (int e = 0; e < kChunk; ++e) p = p + v[i][e];
            }
        }
        const float mu = canonical_tree(p, lds) / kf;
        p = 0.0f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            if (t + i * kLnThreads < chunks) {
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
        asm volatile("" : "+s"(gb), "+s"(bb));
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            if (i + SP < CPT) {
                gload8f(gb + o[i + SP] * 32u, ga[i + SP]);
                gload8f(bb + o[i + SP] * 32u, be[i + SP]);
            }
            if (t + i * kLnThreads < chunks) {
#pragma unroll
                for (int e = 0; e < kChunk; ++e) {
                    float q = v[i][e] * rho;
                    q = q * ga[i][e];
                    v[i][e] = q + be[i][e];
                    mx = fmaxf(mx, fabsf(v[i][e]));
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        float d = d_static, rd = rd_static;
        if (!STATIC) {
            mx = block_max(mx, lds + 2 * kLnThreads, parity);
            step_rcp(mx, d, rd);
            if (t == 0) x_scale[m] = d;
        }
        g_char* orow = (g_char*)(xq + m * K);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            uint32_t q[kChunk];
            quantize_chunk<STATIC>(v[i], d, rd, q);
            const uint2 packed = pack8_bits(q);
            if (t + i * kLnThreads < chunks) gstore8(orow + o[i] * 8u, packed);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
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
            step_rcp(mx, d, rd);
            if (c == 0 && m < M) {
                if (rowmax) rowmax[m] = mx;
                else x_scale[m] = d;
            }
        }
        if (STATIC && clip) {
            if (live) count_clips(v, d, rd, c, clip_ch, nclip);
        } else if ((STATIC || rowmax == nullptr) && live) {
            uint32_t q[kChunk];
            quantize_chunk<STATIC>(v, d, rd, q);
            *reinterpret_cast<uint2*>(xq + m * K + c * kChunk) = pack8_bits(q);
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
            uint32_t q[kChunk];
            quantize_chunk<STATIC>(v, d, rd, q);
            *reinterpret_cast<uint2*>(xq + m * K + c * kChunk) = pack8_bits(q);
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

// Two rows at once per block (bf16 codes, 64 < chunks <= 2048): one lane per
// chunk for rows of up to 512 chunks (128, 256 or 512 lanes; at most 768, 1536
// or 2048 blocks), else up to 1024 lanes with two chunks each (one block per
// CU).  Measured on the MI355X against one row per block: 8-12%
// faster on 2048 x 4096 and 2048 x 16384, within 3% on 65536 x 2048, 5% faster on
// 8192 x 1024.
template <bool STATIC>
hipError_t run_multi(const ActArgs& a, hipStream_t stream) {
    const int64_t chunks = a.K / kChunk;
    const int64_t pairs = (a.M + 1) / 2;
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    if (chunks <= 512) {
        // at most the blocks one round holds (77 VGPRs: three blocks of 512
        // lanes per CU; 73: six of 256); the rest take further row pairs
        // with the next pair in flight.  Measured against 1024 / 2048 blocks,
        // outputs identical, caches flushed: 2048 x 4096 10.7 us vs 11.0,
        // 4096 x 4096 13.9 vs 14.7-15.0, 2048 x 3072 9.8 vs 10.5, 16384 x 2048
        // 21.2 vs 23.1 (1536 blocks of 256 lanes)
        const unsigned cap = chunks > 256 ? 768u : chunks > 128 ? 1536u : 2048u;
        const unsigned grid = static_cast<unsigned>(std::min<int64_t>(pairs, cap));
        if (chunks <= 128)
            act_quant_multi_kernel<uint16_t, STATIC, 1, 2, 128><<<grid, 128, 0, stream>>>(
                x, a.M, a.K, a.s, a.static_scale, a.xq, a.x_scale);
        else if (chunks <= 256)
            act_quant_multi_kernel<uint16_t, STATIC, 1, 2, 256><<<grid, 256, 0, stream>>>(
                x, a.M, a.K, a.s, a.static_scale, a.xq, a.x_scale);
        else
            act_quant_multi_kernel<uint16_t, STATIC, 1, 2, 512><<<grid, 512, 0, stream>>>(
                x, a.M, a.K, a.s, a.static_scale, a.xq, a.x_scale);
    } else {
        const unsigned grid = static_cast<unsigned>(std::min<int64_t>(pairs, 256));
        act_quant_multi_kernel<uint16_t, STATIC, 2, 2, 1024><<<grid, 1024, 0, stream>>>(
            x, a.M, a.K, a.s, a.static_scale, a.xq, a.x_scale);
    }
    return hipGetLastError();
}

// About 4096 blocks of 256 lanes, four rows in flight per lane.  Measured on
// the MI355X against the row kernels, outputs identical, caches flushed before
// each call / warm: 4096 x 49152 bf16 160 us vs 262 / 125 vs 235 (4.8 TB/s),
// 4097 x 36864 124 vs 239, 4096 x 24576 94 vs 109 / 50 vs 88, 2048 x 16384
// 34 vs 35 / 20-22 vs 22; rows of 12288 or fewer elements were within 5% either
// way and stay on the row kernels.
template <typename T>
hipError_t run_static_stream(const ActArgs& a, hipStream_t stream) {
    constexpr int NT = 256, RU = 4;
    const int64_t chunks = a.K / kChunk;
    const int segs = static_cast<int>((chunks + NT - 1) / NT);
    const int64_t groups =
        std::max<int64_t>(1, std::min<int64_t>((a.M + RU - 1) / RU, 4096 / segs));
    const int64_t rpb = (a.M + groups - 1) / groups;
    const int64_t nblk = static_cast<int64_t>(segs) * ((a.M + rpb - 1) / rpb);
    act_quant_static_stream_kernel<T, NT, RU><<<static_cast<unsigned>(nblk), NT, 0, stream>>>(
        static_cast<const T*>(a.x), a.M, a.K, a.s, a.static_scale, a.xq, segs, rpb);
    return hipGetLastError();
}

// Per-token codes of rows of 2049-6144 chunks: four chunks per lane up to
// 4096 chunks, six beyond, at most 1024 lanes, one block per CU.  Measured on
// the MI355X against act_quant_kernel (eight chunks per lane, factors loaded
// chunk by chunk after the row had landed), codes and steps identical, caches
// flushed before each call: 4096 x 49152 bf16 140-145 us vs 192-198 (4.2-4.3
// TB/s), 4096 x 36864 110-115 vs 154-160, 4096 x 24576 75-81 vs 90-93,
// 2048 x 32768 56-58 vs 62-64, 4096 x 16448 64-66 vs 74-76.  Requesting the
// next row's first factors before this row's stores (so that the first wait
// of a row does not also wait for them) was no faster.
template <typename T>
hipError_t run_long(const ActArgs& a, hipStream_t stream) {
    const int64_t chunks = a.K / kChunk;
    const unsigned grid = static_cast<unsigned>(std::min<int64_t>(a.M, 256));
    if (chunks <= 4 * 1024) {
        act_quant_long_kernel<T, 4><<<grid, round_up64((chunks + 3) / 4), 0, stream>>>(
            static_cast<const T*>(a.x), a.M, a.K, a.s, a.xq, a.x_scale);
    } else {
        act_quant_long_kernel<T, 6><<<grid, round_up64((chunks + 5) / 6), 0, stream>>>(
            static_cast<const T*>(a.x), a.M, a.K, a.s, a.xq, a.x_scale);
    }
    return hipGetLastError();
}

template <typename T, bool STATIC>
hipError_t dispatch_plain(const ActArgs& a, hipStream_t stream) {
    const int64_t chunks = a.K / kChunk;
    if (STATIC && a.rowmax == nullptr && a.clip == nullptr && chunks >= 2048)
        return run_static_stream<T>(a, stream);
    if (sizeof(T) == 2 && a.rowmax == nullptr && a.clip == nullptr && chunks > 64 &&
        chunks <= 2048)
        return run_multi<STATIC>(a, stream);
    // short rows: several rows per wave
    if (chunks <= 8) return run_rows<T, STATIC, 8>(a, stream);
    if (chunks <= 16) return run_rows<T, STATIC, 16>(a, stream);
    if (chunks <= 32) return run_rows<T, STATIC, 32>(a, stream);
    // rows up to 2048 chunks: one or two 16-byte loads per lane and row with the
    // per-column constants cached and the next row prefetched (measured: one
    // prefetched row beats deeper rings on the MI355X); longer rows: per-token
    // codes in act_quant_long_kernel, the count and row-maximum passes with
    // four (up to 1024 lanes) or eight (up to 768 lanes) loads per lane
    // without caching; past that the multi-sweep kernel
    if (chunks <= 64) return run<T, false, STATIC, 1, 1>(a, 64, stream);
    if (chunks <= 2048) return run<T, false, STATIC, 2, 1>(a, round_up64((chunks + 1) / 2), stream);
    if (!STATIC && a.rowmax == nullptr && a.clip == nullptr && chunks <= 6 * 1024)
        return run_long<T>(a, stream);
    if (chunks <= 4 * 1024) return run<T, false, STATIC, 4, 0>(a, round_up64((chunks + 3) / 4), stream);
    if (chunks <= 8 * 768)
        return run<T, false, STATIC, 8, 0, 768>(a, round_up64((chunks + 7) / 8), stream);
    return run_stream<T, false, STATIC>(a, stream);
}

// Two rows at once per block in LayerNorm mode (bf16 codes, rows of up to 1024
// chunks).  Measured on the MI355X against one row per block, with the caches
// flushed before each call / with the input re-read warm: 4096 x 8192 7-12% /
// 5-10% faster (38 us vs 41-43 / 31 vs 32-34), 16384 x 2048 13-17% / 8-12%,
// 4096 x 1024 12% / 0-8%, 2048 x 4096 within 4% either way; rows of 1536 chunks
// (six per lane, 276 VGPRs) were 5% slower, so longer rows stay on the one-row
// kernel.
template <bool STATIC>
hipError_t run_ln2(const ActArgs& a, int64_t need, hipStream_t stream) {
    const int64_t pairs = (a.M + 1) / 2;
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    if (need <= 1) {
        const unsigned grid = static_cast<unsigned>(std::min<int64_t>(pairs, 1024));
        act_quant_ln2_kernel<uint16_t, STATIC, 1><<<grid, kLnThreads, 0, stream>>>(
            x, a.M, a.K, a.gs, a.bs, a.eps, a.static_scale, a.xq, a.x_scale);
    } else if (need <= 2) {
        const unsigned grid = static_cast<unsigned>(std::min<int64_t>(pairs, 1024));
        act_quant_ln2_kernel<uint16_t, STATIC, 2><<<grid, kLnThreads, 0, stream>>>(
            x, a.M, a.K, a.gs, a.bs, a.eps, a.static_scale, a.xq, a.x_scale);
    } else {
        const unsigned grid = static_cast<unsigned>(std::min<int64_t>(pairs, 512));
        act_quant_ln2_kernel<uint16_t, STATIC, 4><<<grid, kLnThreads, 0, stream>>>(
            x, a.M, a.K, a.gs, a.bs, a.eps, a.static_scale, a.xq, a.x_scale);
    }
    return hipGetLastError();
}

// LayerNorm mode, codes of bf16 rows of 1025-2048 chunks: one row per block of
// 256 lanes, six or eight chunks per lane; the grid is the blocks that fit at
// once (126 VGPRs at six chunks per lane: four per CU; 146 at eight: three).
template <bool STATIC>
hipError_t run_ln_row(const ActArgs& a, int64_t need, hipStream_t stream) {
    const unsigned grid = static_cast<unsigned>(std::min<int64_t>(a.M, need <= 6 ? 1024 : 768));
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    if (need <= 6)
        act_quant_ln_row_kernel<STATIC, 6, 2><<<grid, kLnThreads, 0, stream>>>(
            x, a.M, a.K, a.gs, a.bs, a.eps, a.static_scale, a.xq, a.x_scale);
    else
        act_quant_ln_row_kernel<STATIC, 8, 2><<<grid, kLnThreads, 0, stream>>>(
            x, a.M, a.K, a.gs, a.bs, a.eps, a.static_scale, a.xq, a.x_scale);
    return hipGetLastError();
}

template <typename T, bool STATIC>
hipError_t dispatch_ln(const ActArgs& a, hipStream_t stream) {
    const int64_t chunks = a.K / kChunk;
    const int64_t need = (chunks + kLnThreads - 1) / kLnThreads;
    if (sizeof(T) == 2 && a.rowmax == nullptr && a.clip == nullptr && need <= 4)
        return run_ln2<STATIC>(a, need, stream);
    if (sizeof(T) == 2 && a.rowmax == nullptr && a.clip == nullptr && need <= 8)
        return run_ln_row<STATIC>(a, need, stream);
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
    // one-block reduction into x_scale[0], then the static quantizer with it.
    // Plain rows of 2048 elements or more: block maxima of the streaming pass
    // instead of row maxima (at most segs * M floats with segs = ceil(K / 2048),
    // so they fit in xq's M * K bytes as well)
    float* rowmax = reinterpret_cast<float*>(xq);
    const int64_t chunks = K / kChunk;
    hipError_t e;
    int64_t nmax = M;
    if (!ln && chunks >= 256) {
        constexpr int NT = 256, RU = 4;
        const int segs = static_cast<int>((chunks + NT - 1) / NT);
        const int64_t groups = std::max<int64_t>(1, std::min<int64_t>((M + RU - 1) / RU, 4096 / segs));
        const int64_t rpb = (M + groups - 1) / groups;
        nmax = static_cast<int64_t>(segs) * ((M + rpb - 1) / rpb);
        if (x_dt == Dt::BF16)
            act_absmax_stream_kernel<uint16_t, NT, RU><<<static_cast<unsigned>(nmax), NT, 0, stream>>>(
                static_cast<const uint16_t*>(x), M, K, s, rowmax, segs, rpb);
        else
            act_absmax_stream_kernel<float, NT, RU><<<static_cast<unsigned>(nmax), NT, 0, stream>>>(
                static_cast<const float*>(x), M, K, s, rowmax, segs, rpb);
        e = hipGetLastError();
    } else {
        e = go(ActArgs{x, M, K, s, gamma_s, beta_s, eps, nullptr, xq, nullptr, rowmax}, false);
    }
    if (e != hipSuccess) return e;
    e = launch_tensor_step(rowmax, nmax, x_scale, stream);
    if (e != hipSuccess) return e;
    return go(ActArgs{x, M, K, s, gamma_s, beta_s, eps, x_scale, xq, nullptr, nullptr}, true);
}

}  // namespace sq
