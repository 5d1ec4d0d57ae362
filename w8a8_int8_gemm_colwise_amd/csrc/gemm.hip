// gemm.hip -- int8 x int8 -> int32 GEMM on the gfx950 matrix cores with the
// dequantizing epilogue.
//
//   [Edge] "嵌入式 SLM 动态权重量化：SmoothQuant 激活异常值迁移与 INT8 部署实战"
//   §三 (GEMM listing): int32 accumulation of activation code x weight code,
//   weight stored [out][in]; output = (float)acc * (act_scale * w_scale[n]).
//   [Review] "SmoothQuant：大型语言模型的精准高效训练后量化 — 深度技术评审"
//   §2.6 / Fig. 3: scales live on the outer dimensions (token, output
//   channel) so they factor out of the contraction.
//
//   [Review] §5.6 / Fig. 6: the batched products of attention run in int8 as
//   well (every kernel takes a batch index on grid.y, see Batch).
//
// Y[M, N] = Xq[M, K] . Wq[N, K]^T: both operands are K-contiguous ("NT"), the
// layout the MFMA operand registers want (16 consecutive int8 of one row per
// lane); 32x32 v_mfma_i32_32x32x32_i8 tiles accumulate in int32 registers.
// Kernels, chosen by launch_gemm from the shape:
//   gemm_pp_kernel      M > 64, K % 128 == 0: 256x128 or 256x256 tiles, eight
//                       waves in two groups alternating memory and compute
//                       phases ("ping-pong"), LDS stages of 128 K-bytes
//                       (three for 256x128, two for 256x256) filled by
//                       direct-to-LDS transfers
//   gemm_pp_mixed_kernel  both ping-pong tiles in one launch: 256x256 over the
//                       first columns, 256x128 over the rest, when that fills
//                       the rounds of 256 CUs better than either tile alone
//   gemm_shortk_kernel  M > 64, K in {64, 128, 256}: the tile's whole K in LDS
//                       at once, several blocks per CU (store-bound shapes such
//                       as the attention scores)
//   gemm_skinny_kernel  M <= 64 (decode): a weight stream, K split over the
//                       waves of a block with per-wave LDS rings
//   gemm_kernel         the rest: register-staged, two LDS buffers
// The pipelined kernels dequantize through a transposed epilogue (store_tile_t)
// that leaves each tile as whole 16-byte chunks of 128-byte row segments; the
// optional fused epilogue (Epi) adds bias, ReLU, or writes the next linear's
// int8 codes.  LDS chunks are XOR-swizzled so operand fetches hit distinct
// banks, and blocks are remapped so that the tiles one XCD runs are neighbours
// (sharing A rows and B columns in that XCD's L2).
#include <algorithm>
#include <type_traits>

#include "sq_device.hpp"
#include "sq_internal.hpp"

namespace sq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;              // K bytes per LDS stage
constexpr int kChunksPerRow = kBK / 16;
constexpr int kXcds = 8;

// 16-byte chunk permutation of a 64-byte LDS row.  Chosen by measurement on
// gfx950 (SQ_LDS_BANK_CONFLICT): for the MFMA operand fetch -- lanes 0-31
// read 32 consecutive rows at one chunk, lanes 32-63 the next chunk -- this
// permutation is free of bank conflicts, while e.g. c ^ (row & 3) or
// c ^ ((row >> 1 ^ row >> 3) & 3) serialize every ds_read_b128 two or four ways.
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * kBK + ((chunk ^ swz(row)) << 4);
}

// Rows of BK bytes (64 or 128).  128-byte rows use c ^ ((row >> 1) & 7),
// likewise measured conflict-free for the operand fetch pattern.
template <int BK>
__device__ __forceinline__ int swz_k(int row) {
    static_assert(BK == 64 || BK == 128, "64- or 128-byte rows");
    return BK == 64 ? (row >> 2) & 3 : (row >> 1) & 7;
}
template <int BK>
__device__ __forceinline__ int lds_off_k(int row, int chunk) {
    return row * BK + ((chunk ^ swz_k<BK>(row)) << 4);
}

enum OutKind { kOutF32 = 0, kOutBF16 = 1, kOutI32 = 2, kOutI8 = 3 };

template <int OUT>
constexpr int out_bytes() { return OUT == kOutBF16 ? 2 : OUT == kOutI8 ? 1 : 4; }

// Batch entry blockIdx.y of a strided batch (see Batch): offsets of the kernel's
// operand, scale and output pointers, applied at kernel entry.
#define SQ_APPLY_BATCH(OUT_)                                                        \
    do {                                                                            \
        const int64_t bz_ = blockIdx.y;                                             \
        if (bz_ > 0) {                                                              \
            A += bz_ * bat.a;                                                       \
            B += bz_ * bat.b;                                                       \
            if (sx) sx += bz_ * bat.sx;                                             \
            if (sw) sw += bz_ * bat.sw;                                             \
            Y = static_cast<int8_t*>(Y) + bz_ * bat.y * out_bytes<OUT_>();          \
        }                                                                           \
    } while (0)

// Fused epilogue on a dequantized value y (see Epi): bias, then ReLU to +0.
__device__ __forceinline__ float bias_relu(float y, bool has_bias, float b, int relu) {
    if (has_bias) y = y + b;
    if (relu) y = (y > 0.0f) ? y : 0.0f;
    return y;
}

// int8 code of y for the next linear: RN(y / s') (skipped when s' = 1), then
// the static quantizer with step D: the dividend is limited to +-128 D (an
// exact power-of-two scaling that leaves every code unchanged), then
// clamp(rne(RN(. / D))).  rs = RN(1 / s'), rD = RN(1 / D) for the exact division.
__device__ __forceinline__ int requant_code(float y, bool has_s, float sv, float rs, float D,
                                            float rD) {
    float xh = has_s ? div_rn(y, sv, rs) : y;
    const float lim = 128.0f * D;
    xh = fminf(fmaxf(xh, -lim), lim);
    return code_of(div_rn(xh, D, rD));
}

// One output element of the plain epilogues (register-staged and skinny
// kernels): dequantize, fuse, store.  o = row * N + col.
template <int OUT>
__device__ __forceinline__ void store_elem(void* __restrict__ Y, int64_t o, int a, float dx,
                                           float dw, const Epi& e, int col, float D, float rD) {
    if (OUT == kOutI32) {
        static_cast<int32_t*>(Y)[o] = a;
        return;
    }
    const float f = dx * dw;
    float y = static_cast<float>(a) * f;
    y = bias_relu(y, e.bias != nullptr, e.bias ? e.bias[col] : 0.0f, e.relu);
    if (OUT == kOutF32) {
        static_cast<float*>(Y)[o] = y;
    } else if (OUT == kOutBF16) {
        static_cast<__bf16*>(Y)[o] = static_cast<__bf16>(y);
    } else {
        const bool hs = e.next_s != nullptr;
        const float sv = hs ? e.next_s[col] : 1.0f;
        static_cast<int8_t*>(Y)[o] = static_cast<int8_t>(requant_code(y, hs, sv, 1.0f / sv, D, rD));
    }
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct Tile {
    static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
    static constexpr int WM = BM / WAVES_M;
    static constexpr int WN = BN / WAVES_N;
    static constexpr int TM = WM / 32;
    static constexpr int TN = WN / 32;
    static constexpr int LA = BM * kChunksPerRow / kThreads;  // A chunks per thread
    static constexpr int LB = BN * kChunksPerRow / kThreads;
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile is a multiple of 32x32");
};

// Map the launch index to (tile_m, tile_n): undo the round-robin XCD dispatch
// so that consecutive logical tiles run on one XCD, then walk tiles in groups
// of GROUP_M rows so neighbours share operands.
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    const int q = total / kXcds, r = total % kXcds;
    const int xcd = pid % kXcds, slot = pid / kXcds;
    const int lin = xcd * q + min(xcd, r) + slot;
    constexpr int GROUP_M = 8;
    const int per_group = GROUP_M * tiles_n;
    const int g = lin / per_group;
    const int first_m = g * GROUP_M;
    const int gm = min(tiles_m - first_m, GROUP_M);
    const int in_g = lin - g * per_group;
    tm = first_m + in_g % gm;
    tn = in_g / gm;
}

// Dequantizing epilogue for a wave's TM x TN grid of 32x32 accumulator tiles
// whose top-left output element is (row0, col0).  In a 32x32 MFMA result,
// lane l holds rows 8*g + 4*(l/32) + r (g, r in 0..3) of column l%32.
// y = RN(RN_f32(acc) * RN(dx_row * dw_col)); bf16 output rounds that to
// nearest even; the int32 output stores acc.
template <int OUT, int TM, int TN>
__device__ __forceinline__ void store_tile(const v16i (&acc)[TM][TN], int row0, int col0, int lane,
                                           const float* __restrict__ sx, int sx_per_token,
                                           const float* __restrict__ sw, int sw_per_tensor,
                                           void* __restrict__ Y, int M, int N, const Epi& e) {
    const int frow = lane & 31;
    const int fhalf = lane >> 5;
    const float D = (OUT == kOutI8) ? *e.next_step : 1.0f;
    const float rD = 1.0f / D;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = row0 + i * 32 + 8 * g + 4 * fhalf + r;
                if (row >= M) continue;
                const float dx = (OUT == kOutI32) ? 0.0f : sx[sx_per_token ? row : 0];
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int col = col0 + j * 32 + frow;
                    if (col >= N) continue;
                    const int a = acc[i][j][4 * g + r];
                    const int64_t o = static_cast<int64_t>(row) * N + col;
                    const float dw = (OUT == kOutI32) ? 0.0f : sw[sw_per_tensor ? 0 : col];
                    store_elem<OUT>(Y, o, a, dx, dw, e, col, D, rD);
                }
            }
        }
    }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int OUT>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_kernel(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, const float* __restrict__ sx,
    int sx_per_token, const float* __restrict__ sw, int sw_per_tensor, void* __restrict__ Y,
    int M, int N, int K, Epi epi, Batch bat) {
    SQ_APPLY_BATCH(OUT);
    using T = Tile<BM, BN, WAVES_M, WAVES_N>;
    static_assert(T::LA * T::kThreads == BM * kChunksPerRow, "A tile divides over threads");
    static_assert(T::LB * T::kThreads == BN * kChunksPerRow, "B tile divides over threads");
    __shared__ __attribute__((aligned(16))) int8_t As[2][BM * kBK];
    __shared__ __attribute__((aligned(16))) int8_t Bs[2][BN * kBK];

    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    int tmi, tni;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tmi, tni);
    const int m0 = tmi * BM, n0 = tni * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    // global -> register staging descriptors
    const int8_t* a_src[T::LA];
    const int8_t* b_src[T::LB];
    int a_lds[T::LA], b_lds[T::LB];
#pragma unroll
    for (int j = 0; j < T::LA; ++j) {
        const int q = tid + j * T::kThreads;
        const int row = q / kChunksPerRow, c = q % kChunksPerRow;
        const int grow = min(m0 + row, M - 1);
        a_src[j] = A + static_cast<int64_t>(grow) * K + c * 16;
        a_lds[j] = lds_off(row, c);
    }
#pragma unroll
    for (int j = 0; j < T::LB; ++j) {
        const int q = tid + j * T::kThreads;
        const int row = q / kChunksPerRow, c = q % kChunksPerRow;
        const int grow = min(n0 + row, N - 1);
        b_src[j] = B + static_cast<int64_t>(grow) * K + c * 16;
        b_lds[j] = lds_off(row, c);
    }

    v4i ra[T::LA], rb[T::LB];
    auto gload = [&](int k0) {
#pragma unroll
        for (int j = 0; j < T::LA; ++j)
            ra[j] = *reinterpret_cast<const v4i*>(a_src[j] + k0);
#pragma unroll
        for (int j = 0; j < T::LB; ++j)
            rb[j] = *reinterpret_cast<const v4i*>(b_src[j] + k0);
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < T::LA; ++j) *reinterpret_cast<v4i*>(&As[buf][a_lds[j]]) = ra[j];
#pragma unroll
        for (int j = 0; j < T::LB; ++j) *reinterpret_cast<v4i*>(&Bs[buf][b_lds[j]]) = rb[j];
    };

    v16i acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    // fragment read offsets: lane reads row (lane % 32) of each 32-row block,
    // chunk 2*kk + lane/32 of the 64-byte stage
    const int frow = lane & 31;
    const int fhalf = lane >> 5;

    const int ktiles = (K + kBK - 1) / kBK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < ktiles; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < ktiles) gload((kt + 1) * kBK);
#pragma unroll
        for (int kk = 0; kk < kBK / 32; ++kk) {
            v4i fa[T::TM], fb[T::TN];
            const int chunk = 2 * kk + fhalf;
#pragma unroll
            for (int i = 0; i < T::TM; ++i) {
                const int row = wm * T::WM + i * 32 + frow;
                fa[i] = *reinterpret_cast<const v4i*>(&As[cur][lds_off(row, chunk)]);
            }
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                const int row = wn * T::WN + j * 32 + frow;
                fb[j] = *reinterpret_cast<const v4i*>(&Bs[cur][lds_off(row, chunk)]);
            }
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int j = 0; j < T::TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < ktiles) sstore(cur ^ 1);
        __syncthreads();
    }

    store_tile<OUT, T::TM, T::TN>(acc, m0 + wm * T::WM, n0 + wn * T::WN, lane, sx, sx_per_token,
                                  sw, sw_per_tensor, Y, M, N, epi);
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
hipError_t run(const int8_t* xq, const float* sx, bool per_token, const int8_t* wq,
               const float* sw, bool w_per_tensor, int M, int N, int K, void* y, int out, const Epi& epi,
                    const Batch& bat, hipStream_t stream) {
    using T = Tile<BM, BN, WAVES_M, WAVES_N>;
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const dim3 grid(tiles, static_cast<unsigned>(bat.count)), block(T::kThreads);
    const int pt = per_token ? 1 : 0;
    const int wpt = w_per_tensor ? 1 : 0;
    switch (out) {
        case kOutF32:
            gemm_kernel<BM, BN, WAVES_M, WAVES_N, kOutF32><<<grid, block, 0, stream>>>(
                xq, wq, sx, pt, sw, wpt, y, M, N, K, epi, bat);
            break;
        case kOutBF16:
            gemm_kernel<BM, BN, WAVES_M, WAVES_N, kOutBF16><<<grid, block, 0, stream>>>(
                xq, wq, sx, pt, sw, wpt, y, M, N, K, epi, bat);
            break;
        case kOutI8:
            gemm_kernel<BM, BN, WAVES_M, WAVES_N, kOutI8><<<grid, block, 0, stream>>>(
                xq, wq, sx, pt, sw, wpt, y, M, N, K, epi, bat);
            break;
        default:
            gemm_kernel<BM, BN, WAVES_M, WAVES_N, kOutI32><<<grid, block, 0, stream>>>(
                xq, wq, sx, pt, sw, wpt, y, M, N, K, epi, bat);
            break;
    }
    return hipGetLastError();
}


// Epilogue for accumulators computed as W x X^T (MFMA operands swapped): in a
// 32x32 tile lane l holds output row l % 32 and, in registers 4g..4g+3, the
// four consecutive output columns 8g + 4(l / 32) .. +3.  Per 32-row slice of
// the wave tile, the dequantized values go to a per-wave LDS scratch of padded
// rows (8-byte writes for bf16, 16-byte writes for f32 / int32; the padding
// keeps a write instruction free of bank conflicts) and leave as whole
// 16-byte chunks, several lanes per row, so each global store instruction
// covers complete 128-byte row segments.  sxs / sws: LDS copies of the scales
// of the wave tile's rows and columns; bcs / scs / rcs: LDS copies of the
// columns' bias, next-layer smoothing factor s' and RN(1/s') (fused epilogue).
// The dequantization is the library's fixed order: f = s_x * s_w, then
// y = float(acc) * f, then bias and ReLU, then the output type (bf16 rounding,
// or the next linear's int8 code).
template <int OUT, int TN>
constexpr int epi_pitch() { return TN * 32 * out_bytes<OUT>() + (out_bytes<OUT>() == 4 ? 16 : 8); }

// NT: the whole 16-byte chunks leave as non-temporal stores (streaming hint:
// the lines are written on towards memory during the GEMM instead of staying
// dirty in the caches until a later kernel's reads evict them).  Measured on
// the MI355X with the OPT-6.7B prefill step (four linears, two alternations,
// identical outputs): GEMMs 1.5-6% faster and the calibrations that follow
// them up to 11% faster, the step 3.9% faster; the same hint on the weight
// codes, which the next GEMM reads, made that GEMM slower.
typedef unsigned int v4u_nt __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ void store16(int8_t* out, const uint4& v) {
    if constexpr (NT) {
        const v4u_nt w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<v4u_nt*>(out));
    } else {
        *reinterpret_cast<uint4*>(out) = v;
    }
}

template <int OUT, int TM, int TN, bool FUSED, bool NT>
__device__ __forceinline__ void store_tile_t(const v16i (&acc)[TM][TN], int row0, int col0,
                                             int lane, const float* sxs, const float* sws,
                                             const float* bcs, const float* scs,
                                             const float* rcs, const Epi& e, float D, float rD,
                                             void* __restrict__ Y, int M, int N,
                                             int8_t* scratch) {
    constexpr int ES = out_bytes<OUT>();            // output element bytes
    constexpr int SEG = TN * 32 * ES;              // bytes of one row of the wave tile
    constexpr int PITCH = epi_pitch<OUT, TN>();
    constexpr int CPR = SEG / 16;                  // 16-byte chunks per row
    constexpr int EPC = 16 / ES;                   // elements per chunk
    constexpr int NQ = 32 * CPR / 64;              // chunks per lane per 32-row slice
    static_assert(NQ * 64 == 32 * CPR, "whole chunks per lane");
    const int fr = lane & 31;
    const int h = lane >> 5;
    const bool hb = FUSED && e.bias != nullptr;
    const int relu = FUSED ? e.relu : 0;
    // whole slices go out as 16-byte stores when rows and base are 16-byte
    // aligned (a batch entry may start anywhere) and the slice is in range
    const bool cols_in = ((static_cast<int64_t>(N) * ES) % 16) == 0 &&
                         (reinterpret_cast<uintptr_t>(Y) & 15) == 0 && col0 + TN * 32 <= N;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const float dx = (OUT == kOutI32) ? 0.0f : sxs[i * 32 + fr];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            // the lane's 16 columns of this 32-column block: c = j*32 + 8g + 4h + t,
            // taken GB groups g at a time; every LDS read of a batch is issued
            // before any of its values is used
            constexpr int GB = 2;
#pragma unroll
            for (int g0 = 0; g0 < 4; g0 += GB) {
            float4 w4[GB], b4[GB], s4[GB], r4[GB];
#pragma unroll
            for (int gg = 0; gg < GB; ++gg) {
                const int g = g0 + gg;
                const int c = j * 32 + 8 * g + 4 * h;
                if (OUT != kOutI32) w4[gg] = *reinterpret_cast<const float4*>(sws + c);
                if (OUT != kOutI32 && FUSED) b4[gg] = *reinterpret_cast<const float4*>(bcs + c);
                if (OUT == kOutI8) {
                    s4[gg] = *reinterpret_cast<const float4*>(scs + c);
                    r4[gg] = *reinterpret_cast<const float4*>(rcs + c);
                }
            }
#pragma unroll
            for (int gg = 0; gg < GB; ++gg) {
                const int g = g0 + gg;
                const int c = j * 32 + 8 * g + 4 * h;  // first of the lane's 4 columns
                int8_t* dst = scratch + fr * PITCH + c * ES;
                if (OUT == kOutI32) {
                    v4i v;
                    for (int t = 0; t < 4; ++t) v[t] = acc[i][j][4 * g + t];
                    *reinterpret_cast<v4i*>(dst) = v;
                    continue;
                }
                const float dw[4] = {w4[gg].x, w4[gg].y, w4[gg].z, w4[gg].w};
                float y[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float f = dx * dw[t];
                    y[t] = static_cast<float>(acc[i][j][4 * g + t]) * f;
                }
                if constexpr (FUSED) {
                    const float bb[4] = {b4[gg].x, b4[gg].y, b4[gg].z, b4[gg].w};
#pragma unroll
                    for (int t = 0; t < 4; ++t) y[t] = bias_relu(y[t], hb, bb[t], relu);
                }
                if (OUT == kOutF32) {
                    *reinterpret_cast<float4*>(dst) = make_float4(y[0], y[1], y[2], y[3]);
                } else if (OUT == kOutBF16) {
                    typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
                    bf4 bv;
                    for (int t = 0; t < 4; ++t) bv[t] = static_cast<__bf16>(y[t]);
                    *reinterpret_cast<bf4*>(dst) = bv;
                } else {
                    const bool hs = e.next_s != nullptr;
                    const float ss[4] = {s4[gg].x, s4[gg].y, s4[gg].z, s4[gg].w};
                    const float rr[4] = {r4[gg].x, r4[gg].y, r4[gg].z, r4[gg].w};
                    uint32_t packed = 0;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int q = requant_code(y[t], hs, ss[t], rr[t], D, rD);
                        packed |= (static_cast<uint32_t>(q) & 0xffu) << (8 * t);
                    }
                    *reinterpret_cast<uint32_t*>(dst) = packed;
                }
            }
            }
        }
        // LDS operations of one wave complete in order: the reads see the
        // writes, and the next slice's writes follow these reads
        uint4 v[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int idx = lane + 64 * q;
            v[q] = *reinterpret_cast<const uint4*>(scratch + (idx / CPR) * PITCH + (idx % CPR) * 16);
        }
        const int srow = row0 + i * 32;
        if (cols_in && srow + 32 <= M) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int idx = lane + 64 * q;
                int8_t* out = static_cast<int8_t*>(Y) +
                              (static_cast<int64_t>(srow + idx / CPR) * N + col0 + (idx % CPR) * EPC) * ES;
                store16<NT>(out, v[q]);
            }
        } else {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int idx = lane + 64 * q;
                const int grow = srow + idx / CPR;
                const int gcol = col0 + (idx % CPR) * EPC;
                if (grow >= M) continue;
                int8_t* out = static_cast<int8_t*>(Y) + (static_cast<int64_t>(grow) * N + gcol) * ES;
#pragma unroll
                for (int t = 0; t < EPC; ++t) {
                    if (gcol + t >= N) continue;
                    // element t of the chunk, taken from its 32-bit word by shift
                    const int wi = t * ES / 4;
                    const uint32_t wv = wi == 0 ? v[q].x : wi == 1 ? v[q].y : wi == 2 ? v[q].z : v[q].w;
                    const uint32_t ev = wv >> (8 * ((t * ES) & 3));
                    if (ES == 4) *reinterpret_cast<uint32_t*>(out + t * ES) = ev;
                    else if (ES == 2) *reinterpret_cast<uint16_t*>(out + t * ES) = static_cast<uint16_t>(ev);
                    else out[t] = static_cast<int8_t>(ev);
                }
            }
        }
    }
}

// ---- pipeline helpers ---------------------------------------------------------

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void wait_lgkmcnt0() {
    // vmcnt and expcnt at their maxima (no wait), lgkmcnt 0
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Ordering point for both the IR optimizers (memory clobber) and the machine
// scheduler (sched_barrier with an empty mask lets nothing cross it).
__device__ __forceinline__ void compiler_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)(p)));
}

// global_load_lds_dwordx4 in its scalar-base form: lane l copies the 16 bytes
// at base + voff(l) to LDS address lds + 16 l; base and lds are wave-uniform.
// Issued from inline asm, the transfer is invisible to the compiler's wait
// counter tracking, so the kernel's own vmcnt waits are the only ones: the
// compiler otherwise drains every transfer in flight at each loop back-edge.
// The compiler uses M0 for nothing else in these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const int8_t* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds), "v"(voff), "s"(base)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// ---- ping-pong pipelined kernel ---------------------------------------------
//
// Eight waves, two per SIMD, in two groups of four (one wave of each group on
// every SIMD).  Each wave alternates a memory phase -- issue its share of the
// global->LDS transfers for stage t+STAGES-1, read all MFMA fragments of
// stage t from LDS into registers -- and a compute phase of back-to-back
// MFMAs on those registers.  Group 1 starts one phase late, so on every SIMD
// one wave's MFMAs run while the other wave's memory phase is in flight, and
// each block-wide barrier closes a compute phase of one group and a memory
// phase of the other.  Ordering (barrier n closes phase n of group 0 and
// phase n-1 of group 1):
//  * a stage buffer is refilled only in the memory phase after the one in
//    which both groups finished reading it (each wave drains its LDS reads
//    before arriving at a barrier);
//  * every wave waits for its own transfers of stage t+1 before the barrier
//    that precedes either group's memory phase of stage t+1.
// LDS bytes of the operand stages of one configuration
template <int BM, int BN, int BK, int STAGES>
constexpr int pp_stage_lds() { return STAGES * (BM + BN) * BK; }
// With two stages (the 256x256 tile with 128-byte K stages, 128 KB of LDS)
// group 0 moves every stage: it issues all transfers of stage t+1 at the start
// of its memory phase of stage t -- into the buffer of stage t-1, which group 0
// read one phase and group 1 read in the phase just closed -- and waits for
// them at the end of its compute phase of stage t, so stage t+1 has landed
// before the barrier that precedes either group's memory phase of stage t+1
// (two phases of lookahead).  Group 1 issues no transfers.

// One BM x BN output tile at rows [tm * BM, ...) and columns
// [n_base + tn * BN, ...), where (tm, tn) is tile `pid` of a tiles_m x tiles_n
// grid (XCD-aware order).  lds holds the operand stages, scales BM + BN floats
// and epi_cols 3 * BN floats.
template <int BM, int BN, int WAVES_M, int WAVES_N, int BK, int STAGES, int OUT>
__device__ __forceinline__ void pp_tile(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, const float* __restrict__ sx,
    int sx_per_token, const float* __restrict__ sw, int sw_per_tensor, void* __restrict__ Y,
    int M, int N, int K, const Epi& epi, int pid, int tiles_m, int tiles_n, int n_base,
    int8_t* __restrict__ lds, float* __restrict__ scales, float* __restrict__ epi_cols) {
    using T = Tile<BM, BN, WAVES_M, WAVES_N>;
    static_assert(WAVES_M * WAVES_N == 8, "two groups of four waves");
    constexpr int kRows = BM + BN;
    constexpr int kStageBytes = kRows * BK;
    constexpr int kCPR = BK / 16;            // 16-byte chunks per row
    constexpr int kRowsPerXfer = 1024 / BK;  // 1 KB per wave-wide transfer
    constexpr bool TWO = STAGES == 2;                 // group 0 moves every stage
    constexpr int kIssuers = TWO ? 4 : 8;
    constexpr int IPW = kRows / kRowsPerXfer / kIssuers;
    constexpr int NKK = BK / 32;
    static_assert(IPW * kIssuers * kRowsPerXfer == kRows, "stage divides over the waves");
    static_assert(BM % kRowsPerXfer == 0, "a transfer never straddles A and B");
    static_assert(STAGES >= 2, "two stages at least");
    constexpr int kEpiPitch = epi_pitch<OUT, T::TN>();
    static_assert(8 * 32 * kEpiPitch <= STAGES * kStageBytes, "epilogue scratch fits");
    static_assert(BM + BN <= 512, "one scale per thread");
    // scales: row scales, then column scales; epi_cols: bias, s', RN(1/s') per column
    int tmi, tni;
    tile_coords(pid, tiles_m, tiles_n, tmi, tni);
    const int m0 = tmi * BM, n0 = n_base + tni * BN;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int group = wave >> 2;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    // lane q of transfer x lands at LDS byte 16 q of the transfer's 1 KB and
    // fetches the global chunk whose swizzled slot that is.  With three or
    // more stages the offsets are kept in registers; with two, group 0's 16
    // transfers per wave are addressed as they are issued (registers are short)
    constexpr int kOff = TWO ? 1 : IPW;
    int src_off[kOff];
    bool src_a[kOff];
    auto src = [&](int x, bool& is_a) {
        const int q = x * 64 + lane;
        const int row = q / kCPR;
        const int c = (q % kCPR) ^ swz_k<BK>(row);
        is_a = x * kRowsPerXfer < BM;
        return is_a ? min(m0 + row, M - 1) * K + c * 16 : min(n0 + row - BM, N - 1) * K + c * 16;
    };
    if constexpr (!TWO) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) src_off[i] = src(wave * IPW + i, src_a[i]);
    }
    const int KT = K / BK;
    auto issue = [&](int t) {
        int8_t* stage = lds + (t % STAGES) * kStageBytes;
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int x = wave * IPW + i;
            if constexpr (TWO) {
                bool a;
                const int off = src(x, a);
                dma16(a ? A : B, static_cast<uint32_t>(off + t * BK), lds_addr(stage + x * 1024));
            } else {
                dma16(src_a[i] ? A : B, static_cast<uint32_t>(src_off[i] + t * BK),
                      lds_addr(stage + x * 1024));
            }
        }
    };
    // wait for this wave's transfers of stage t; later stages may stay in flight
    auto wait_stage = [&](int t) {
        const int younger = min(KT - 1, t + STAGES - 2) - t;
        if (younger >= 2) wait_vmcnt<2 * IPW>();
        else if (younger == 1) wait_vmcnt<IPW>();
        else wait_vmcnt<0>();
    };
    auto bar = [&]() {
        compiler_fence();
        __builtin_amdgcn_s_barrier();
        compiler_fence();
    };

    v16i acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    const int frow = lane & 31;
    const int fhalf = lane >> 5;
    v4i fa[NKK][T::TM], fb[NKK][T::TN];

    // the tile's scales: loaded before the first transfers are issued, stored
    // to LDS after stage 0 has landed (the store waits for every load in
    // flight, stages 1.. included, once per tile)
    float scale = 0.0f, cb = 0.0f, cs = 1.0f;
    const int st = threadIdx.x;
    if (OUT != kOutI32 && st < BM + BN)
        scale = st < BM ? sx[sx_per_token ? min(m0 + st, M - 1) : 0]
                        : sw[sw_per_tensor ? 0 : min(n0 + st - BM, N - 1)];
    if (OUT != kOutI32 && st < BN) {
        const int col = min(n0 + st, N - 1);
        if (epi.bias) cb = epi.bias[col];
        if (OUT == kOutI8 && epi.next_s) cs = epi.next_s[col];
    }
    const float D = (OUT == kOutI8) ? *epi.next_step : 1.0f;
    const float rD = 1.0f / D;
    compiler_fence();
    if constexpr (TWO) {
        if (group == 0) {
            issue(0);
            if (KT > 1) {
                issue(1);
                wait_vmcnt<IPW>();
            } else {
                wait_vmcnt<0>();
            }
        }
    } else {
        for (int t = 0; t < STAGES - 1 && t < KT; ++t) issue(t);
        wait_stage(0);
    }
    if (OUT != kOutI32 && st < BM + BN) scales[st] = scale;
    if (OUT != kOutI32 && st < BN) {
        epi_cols[st] = cb;
        epi_cols[BN + st] = cs;
        epi_cols[2 * BN + st] = 1.0f / cs;
    }
    bar();
    if (group == 1) bar();
    for (int t = 0; t < KT; ++t) {
        // memory phase
        if constexpr (TWO) {
            if (group == 0 && t >= 1 && t + 1 < KT) issue(t + 1);
        } else {
            if (t + STAGES - 1 < KT) issue(t + STAGES - 1);
        }
        const int8_t* S = lds + (t % STAGES) * kStageBytes;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
                fa[kk][i] = *reinterpret_cast<const v4i*>(
                    S + lds_off_k<BK>(wm * T::WM + i * 32 + frow, 2 * kk + fhalf));
#pragma unroll
            for (int j = 0; j < T::TN; ++j)
                fb[kk][j] = *reinterpret_cast<const v4i*>(
                    S + BM * BK + lds_off_k<BK>(wn * T::WN + j * 32 + frow, 2 * kk + fhalf));
        }
        compiler_fence();
        wait_lgkmcnt0();
        if (!TWO && group == 1 && t + 1 < KT) wait_stage(t + 1);
        bar();
        // compute phase
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int j = 0; j < T::TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[kk][j], fa[kk][i],
                                                                      acc[i][j], 0, 0, 0);
        compiler_fence();
        if (group == 0 && t + 1 < KT) {
            if constexpr (TWO) wait_vmcnt<0>();
            else wait_stage(t + 1);
        }
        bar();
    }
    if (group == 0) bar();

    __syncthreads();
    const int cw = wn * T::WN;
    int8_t* const scr = lds + wave * (32 * kEpiPitch);
    if (epi.bias != nullptr || epi.relu)
        store_tile_t<OUT, T::TM, T::TN, true, true>(acc, m0 + wm * T::WM, n0 + cw, lane,
                                              scales + wm * T::WM, scales + BM + cw,
                                              epi_cols + cw, epi_cols + BN + cw,
                                              epi_cols + 2 * BN + cw, epi, D, rD, Y, M, N, scr);
    else
        store_tile_t<OUT, T::TM, T::TN, false, true>(acc, m0 + wm * T::WM, n0 + cw, lane,
                                               scales + wm * T::WM, scales + BM + cw,
                                               epi_cols + cw, epi_cols + BN + cw,
                                               epi_cols + 2 * BN + cw, epi, D, rD, Y, M, N, scr);
}


template <int BM, int BN, int WAVES_M, int WAVES_N, int BK, int STAGES, int OUT>
__global__ __launch_bounds__(512, 1) void gemm_pp_kernel(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, const float* __restrict__ sx,
    int sx_per_token, const float* __restrict__ sw, int sw_per_tensor, void* __restrict__ Y,
    int M, int N, int K, Epi epi, Batch bat) {
    SQ_APPLY_BATCH(OUT);
    __shared__ __attribute__((aligned(1024))) int8_t lds[pp_stage_lds<BM, BN, BK, STAGES>()];
    __shared__ __attribute__((aligned(16))) float scales[BM + BN];
    __shared__ __attribute__((aligned(16))) float epi_cols[3 * BN];
    pp_tile<BM, BN, WAVES_M, WAVES_N, BK, STAGES, OUT>(
        A, B, sx, sx_per_token, sw, sw_per_tensor, Y, M, N, K, epi, blockIdx.x, (M + BM - 1) / BM,
        (N + BN - 1) / BN, 0, lds, scales, epi_cols);
}

// Two tile sizes in one launch: blocks [0, tiles_m * nb_big) take 256x256
// tiles over the columns [0, 256 * nb_big), the rest 256x128 tiles over the
// remaining columns.  The large tiles come first, so the last round is made of
// small ones; shapes whose 256x256 tiles fill whole rounds of the 256 CUs
// only part of the way use it (launch_gemm's cost model).
template <int OUT>
__global__ __launch_bounds__(512, 1) void gemm_pp_mixed_kernel(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, const float* __restrict__ sx,
    int sx_per_token, const float* __restrict__ sw, int sw_per_tensor, void* __restrict__ Y,
    int M, int N, int K, Epi epi, Batch bat, int nb_big) {
    SQ_APPLY_BATCH(OUT);
    constexpr int kLds = pp_stage_lds<256, 256, 128, 2>() > pp_stage_lds<256, 128, 128, 3>()
                             ? pp_stage_lds<256, 256, 128, 2>()
                             : pp_stage_lds<256, 128, 128, 3>();
    __shared__ __attribute__((aligned(1024))) int8_t lds[kLds];
    __shared__ __attribute__((aligned(16))) float scales[512];
    __shared__ __attribute__((aligned(16))) float epi_cols[3 * 256];
    const int tiles_m = (M + 255) / 256;
    const int big = tiles_m * nb_big;
    const int pid = blockIdx.x;
    if (pid < big) {
        pp_tile<256, 256, 2, 4, 128, 2, OUT>(A, B, sx, sx_per_token, sw, sw_per_tensor, Y, M, N, K,
                                            epi, pid, tiles_m, nb_big, 0, lds, scales, epi_cols);
    } else {
        const int n_base = 256 * nb_big;
        pp_tile<256, 128, 4, 2, 128, 3, OUT>(A, B, sx, sx_per_token, sw, sw_per_tensor, Y, M, N, K,
                                             epi, pid - big, tiles_m, (N - n_base + 127) / 128,
                                             n_base, lds, scales, epi_cols);
    }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int BK, int STAGES>
hipError_t run_pp(const int8_t* xq, const float* sx, bool per_token, const int8_t* wq,
                  const float* sw, bool w_per_tensor, int M, int N, int K, void* y, int out, const Epi& epi,
                    const Batch& bat, hipStream_t stream) {
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const dim3 grid(tiles, static_cast<unsigned>(bat.count)), block(512);
    const int pt = per_token ? 1 : 0;
    const int wpt = w_per_tensor ? 1 : 0;
    switch (out) {
        case kOutF32:
            gemm_pp_kernel<BM, BN, WAVES_M, WAVES_N, BK, STAGES, kOutF32>
                <<<grid, block, 0, stream>>>(xq, wq, sx, pt, sw, wpt, y, M, N, K, epi, bat);
            break;
        case kOutBF16:
            gemm_pp_kernel<BM, BN, WAVES_M, WAVES_N, BK, STAGES, kOutBF16>
                <<<grid, block, 0, stream>>>(xq, wq, sx, pt, sw, wpt, y, M, N, K, epi, bat);
            break;
        case kOutI8:
            gemm_pp_kernel<BM, BN, WAVES_M, WAVES_N, BK, STAGES, kOutI8>
                <<<grid, block, 0, stream>>>(xq, wq, sx, pt, sw, wpt, y, M, N, K, epi, bat);
            break;
        default:
            gemm_pp_kernel<BM, BN, WAVES_M, WAVES_N, BK, STAGES, kOutI32>
                <<<grid, block, 0, stream>>>(xq, wq, sx, pt, sw, wpt, y, M, N, K, epi, bat);
            break;
    }
    return hipGetLastError();
}

hipError_t run_pp_mixed(const int8_t* xq, const float* sx, bool per_token, const int8_t* wq,
                        const float* sw, bool w_per_tensor, int M, int N, int K, void* y, int out,
                        const Epi& epi, const Batch& bat, int nb_big, hipStream_t stream) {
    const int tiles_m = (M + 255) / 256;
    const int tiles = tiles_m * nb_big + tiles_m * ((N - 256 * nb_big + 127) / 128);
    const dim3 grid(tiles, static_cast<unsigned>(bat.count)), block(512);
    const int pt = per_token ? 1 : 0;
    const int wpt = w_per_tensor ? 1 : 0;
    switch (out) {
        case kOutF32:
            gemm_pp_mixed_kernel<kOutF32><<<grid, block, 0, stream>>>(xq, wq, sx, pt, sw, wpt, y, M, N, K, epi, bat, nb_big);
            break;
        case kOutBF16:
            gemm_pp_mixed_kernel<kOutBF16><<<grid, block, 0, stream>>>(xq, wq, sx, pt, sw, wpt, y, M, N, K, epi, bat, nb_big);
            break;
        case kOutI8:
            gemm_pp_mixed_kernel<kOutI8><<<grid, block, 0, stream>>>(xq, wq, sx, pt, sw, wpt, y, M, N, K, epi, bat, nb_big);
            break;
        default:
            gemm_pp_mixed_kernel<kOutI32><<<grid, block, 0, stream>>>(xq, wq, sx, pt, sw, wpt, y, M, N, K, epi, bat, nb_big);
            break;
    }
    return hipGetLastError();
}

// ---- short-K kernel (K = 64, 128 or 256, e.g. the attention scores Q K^T) ----
//
// With K this short a tile does little MFMA work per output byte, so the
// kernel is bound by its output stores (and the operand loads of the next
// tiles).  Each block loads the tile's whole K into LDS with one burst of
// global_load_lds transfers (panels of 128- or 64-byte rows, swizzled as in
// the ping-pong kernel), runs the MFMAs, and leaves through the transposed
// 16-byte-store epilogue, whose scratch reuses the operand LDS.  Four waves
// and at most 64 KB of LDS per block let several blocks share a CU, so one
// block's stores overlap the loads and MFMAs of the others.
// Short-K outputs (attention scores) leave as non-temporal stores too: on
// the 32 x 2048 x 2048 x 128 products the quantizer that reads the scores next
// took 84 instead of 106 us, the attention step 12% less time.
constexpr bool SK_NT = true;

template <int BM, int BN, int WAVES_M, int WAVES_N, int KS, int OUT, bool FUSED>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N)
__attribute__((amdgpu_waves_per_eu(KS == 256 ? 2 : OUT == kOutI8 ? (FUSED ? 2 : 3) : (FUSED ? 3 : 4))))
void gemm_shortk_kernel(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, const float* __restrict__ sx,
    int sx_per_token, const float* __restrict__ sw, int sw_per_tensor, void* __restrict__ Y,
    int M, int N, int K, Epi epi, Batch bat) {
    SQ_APPLY_BATCH(OUT);
    using T = Tile<BM, BN, WAVES_M, WAVES_N>;
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int BKP = KS >= 128 ? 128 : 64;  // bytes per row of one LDS panel
    constexpr int NP = KS / BKP;
    constexpr int kRows = BM + BN;
    constexpr int kPanel = kRows * BKP;
    constexpr int kCPR = BKP / 16;
    constexpr int kRowsPerXfer = 1024 / BKP;
    constexpr int XPP = kRows / kRowsPerXfer;  // wave-wide transfers per panel
    constexpr int IPW = XPP * NP / NW;         // transfers per wave
    constexpr int NKK = BKP / 32;
    static_assert(NP * BKP == KS && IPW * NW == XPP * NP, "panels divide over the waves");
    static_assert(BM % kRowsPerXfer == 0, "a transfer never straddles A and B");
    static_assert(IPW < 64, "vmcnt range");
    constexpr int kEpiPitch = epi_pitch<OUT, T::TN>();
    constexpr int kLds = NW * 32 * kEpiPitch > NP * kPanel ? NW * 32 * kEpiPitch : NP * kPanel;
    static_assert(BM + BN <= 2 * T::kThreads && BN <= T::kThreads, "scale staging");
    __shared__ __attribute__((aligned(1024))) int8_t lds[kLds];
    __shared__ __attribute__((aligned(16))) float scales[BM + BN];
    __shared__ __attribute__((aligned(16))) float epi_cols[3 * BN];

    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    int tmi, tni;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tmi, tni);
    const int m0 = tmi * BM, n0 = tni * BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int st = threadIdx.x;

    // scales and epilogue columns first (their loads retire before the
    // transfers issued after them)
    float sc0 = 0.0f, sc1 = 0.0f, cb = 0.0f, cs = 1.0f;
    if (OUT != kOutI32) {
        auto scale_of = [&](int r) {
            return r < BM ? sx[sx_per_token ? min(m0 + r, M - 1) : 0]
                          : sw[sw_per_tensor ? 0 : min(n0 + r - BM, N - 1)];
        };
        sc0 = scale_of(st);
        if (st + T::kThreads < BM + BN) sc1 = scale_of(st + T::kThreads);
        if (st < BN) {
            const int col = min(n0 + st, N - 1);
            if (epi.bias) cb = epi.bias[col];
            if (OUT == kOutI8 && epi.next_s) cs = epi.next_s[col];
        }
    }
    const float D = (OUT == kOutI8) ? *epi.next_step : 1.0f;
    const float rD = 1.0f / D;
    compiler_fence();
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int x = wave * IPW + i;
        const int p = x / XPP, xi = x % XPP;
        const int q = xi * 64 + lane;
        const int row = q / kCPR;
        const int c = (q % kCPR) ^ swz_k<BKP>(row);
        const bool is_a = xi * kRowsPerXfer < BM;
        const int off = is_a ? min(m0 + row, M - 1) * K : min(n0 + row - BM, N - 1) * K;
        dma16(is_a ? A : B, static_cast<uint32_t>(off + p * BKP + c * 16),
              lds_addr(lds + p * kPanel + xi * 1024));
    }
    wait_vmcnt<0>();
    if (OUT != kOutI32) {
        scales[st] = sc0;
        if (st + T::kThreads < BM + BN) scales[st + T::kThreads] = sc1;
        if (st < BN) {
            epi_cols[st] = cb;
            epi_cols[BN + st] = cs;
            epi_cols[2 * BN + st] = 1.0f / cs;
        }
    }
    compiler_fence();
    __syncthreads();

    v16i acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;
    const int frow = lane & 31;
    const int fhalf = lane >> 5;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int8_t* S = lds + p * kPanel;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            v4i fa[T::TM], fb[T::TN];
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
                fa[i] = *reinterpret_cast<const v4i*>(
                    S + lds_off_k<BKP>(wm * T::WM + i * 32 + frow, 2 * kk + fhalf));
#pragma unroll
            for (int j = 0; j < T::TN; ++j)
                fb[j] = *reinterpret_cast<const v4i*>(
                    S + BM * BKP + lds_off_k<BKP>(wn * T::WN + j * 32 + frow, 2 * kk + fhalf));
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int j = 0; j < T::TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[j], fa[i], acc[i][j],
                                                                      0, 0, 0);
        }
    }
    __syncthreads();
    const int cw = wn * T::WN;
    // bias / ReLU chosen by the launch (one epilogue per kernel keeps the
    // register count within four waves per SIMD)
    store_tile_t<OUT, T::TM, T::TN, FUSED, SK_NT>(acc, m0 + wm * T::WM, n0 + cw, lane, scales + wm * T::WM,
                                           scales + BM + cw, epi_cols + cw, epi_cols + BN + cw,
                                           epi_cols + 2 * BN + cw, epi, D, rD, Y, M, N,
                                           lds + wave * (32 * kEpiPitch));
}

template <int KS>
hipError_t run_shortk(const int8_t* xq, const float* sx, bool per_token, const int8_t* wq,
                      const float* sw, bool w_per_tensor, int M, int N, int K, void* y, int out,
                      const Epi& epi, const Batch& bat, hipStream_t stream) {
    constexpr int BM = 128, BN = 128;
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const dim3 grid(tiles, static_cast<unsigned>(bat.count)), block(256);
    const int pt = per_token ? 1 : 0;
    const int wpt = w_per_tensor ? 1 : 0;
    const bool fused = epi.bias != nullptr || epi.relu != 0;
#define SQ_SK(OUT_, F_)                                                                      \
    gemm_shortk_kernel<BM, BN, 2, 2, KS, OUT_, F_>                                           \
        <<<grid, block, 0, stream>>>(xq, wq, sx, pt, sw, wpt, y, M, N, K, epi, bat)
    switch (out) {
        case kOutF32:
            if (fused) SQ_SK(kOutF32, true); else SQ_SK(kOutF32, false);
            break;
        case kOutBF16:
            if (fused) SQ_SK(kOutBF16, true); else SQ_SK(kOutBF16, false);
            break;
        case kOutI8:
            if (fused) SQ_SK(kOutI8, true); else SQ_SK(kOutI8, false);
            break;
        default:  // int32 accumulators take no epilogue
            SQ_SK(kOutI32, false);
            break;
    }
#undef SQ_SK
    return hipGetLastError();
}

// ---- skinny-M kernel (decode: M <= 64): streams W once from HBM ---------------
//
// Every W byte meets at most two 32-row MFMA tiles here, so the kernel is bound
// by the weight stream.  A block owns 32 output channels and its WPB waves
// split the K chunks (128 bytes each) into contiguous ranges.  Each wave runs
// its own ring of ST LDS stages with no block-level barrier: one stage holds
// the chunk's 32 W rows and MT x 32 X rows (128 bytes each), filled by
// global_load_lds transfers that each move eight whole 128-byte row segments,
// so every load instruction covers full cache lines.  16-byte slot c of row r
// is stored at slot c ^ ((r >> 1) & 7), which keeps the fragment reads free of
// bank conflicts.  The K-to-MFMA-slot assignment is free as long as both
// operands share it: lane l (row l % 32, half h = l / 32) takes bytes
// 64h + 16s .. 64h + 16s + 15 of the chunk in MFMA step s.  The waves' int32
// partial tiles are summed exactly with LDS integer atomics.
template <int MT, int WPB, int ST>
struct Skinny {
    static constexpr int kGroups = 1 + MT;                 // 32-row groups per stage
    static constexpr int kStage = kGroups * 4096;          // bytes per stage
    static constexpr int kXfers = 4 * kGroups;             // 1 KB transfers per stage
    static constexpr int kRing = WPB * ST * kStage;        // LDS ring bytes per block
};

// fill one stage with the 128-byte K chunk `chunk` of every row it holds:
// transfers 0..3 read W (B), the others X (A); off[q] is the lane's byte
// offset of its row segment at K = 0
template <int XFERS>
__device__ __forceinline__ void skinny_issue(const int8_t* A, const int8_t* B, const uint32_t* off,
                                             int8_t* stage, int chunk) {
    const uint32_t k0 = static_cast<uint32_t>(chunk) * 128u;
#pragma unroll
    for (int q = 0; q < XFERS; ++q)
        dma16(q < 4 ? B : A, off[q] + k0, lds_addr(stage + q * 1024));
}

template <int MT, int WPB, int ST, int OUT>
__global__ __launch_bounds__(64 * WPB) void gemm_skinny_kernel(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, const float* __restrict__ sx,
    int sx_per_token, const float* __restrict__ sw, int sw_per_tensor, void* __restrict__ Y,
    int M, int N, int K, Epi epi, Batch bat) {
    SQ_APPLY_BATCH(OUT);
    using S = Skinny<MT, WPB, ST>;
    static_assert(ST >= 2 && ST <= 3, "2 or 3 stages");
    __shared__ __attribute__((aligned(1024))) int8_t ring[S::kRing];
    __shared__ int32_t red[MT * 32 * 32];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * 32;
    const int frow = lane & 31;
    const int half = lane >> 5;
    const float D = (OUT == kOutI8) ? *epi.next_step : 1.0f;
    const float rD = 1.0f / D;

    for (int i = threadIdx.x; i < MT * 32 * 32; i += 64 * WPB) red[i] = 0;

    // transfer q of a stage: group g = q / 4 (0 = W, 1.. = X tiles), rows
    // 8 (q % 4) .. 8 (q % 4) + 7 of the group; lane -> row + lane / 8 and the
    // source slot whose swizzled position is lane % 8
    int8_t* my = ring + wave * ST * S::kStage;
    uint32_t off[4 * (1 + MT)];  // the caller guarantees N*K and M*K < 2^31
#pragma unroll
    for (int q = 0; q < S::kXfers; ++q) {
        const int g = q / 4;
        const int row = 8 * (q % 4) + (lane >> 3);
        const int slot = (lane & 7) ^ ((row >> 1) & 7);
        off[q] = static_cast<uint32_t>(g == 0 ? min(n0 + row, N - 1) * K + 16 * slot
                                              : min((g - 1) * 32 + row, M - 1) * K + 16 * slot);
    }
    const int chunks = K / 128;
    const int first = static_cast<int>(static_cast<int64_t>(wave) * chunks / WPB);
    const int cnt = static_cast<int>(static_cast<int64_t>(wave + 1) * chunks / WPB) - first;
    v16i acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0;

    for (int i = 0; i < ST - 1 && i < cnt; ++i)
        skinny_issue<S::kXfers>(A, B, off, my + (i % ST) * S::kStage, first + i);
    for (int i = 0; i < cnt; ++i) {
        compiler_fence();
        if (i + ST - 1 < cnt)
            skinny_issue<S::kXfers>(A, B, off, my + ((i + ST - 1) % ST) * S::kStage, first + i + ST - 1);
        // stages issued after stage i may stay in flight
        const int younger = min(cnt - 1, i + ST - 1) - i;
        if (younger >= 2) wait_vmcnt<2 * S::kXfers>();
        else if (younger == 1) wait_vmcnt<S::kXfers>();
        else wait_vmcnt<0>();
        compiler_fence();
        const int8_t* st = my + (i % ST) * S::kStage;
        v4i wb[4], ab[MT][4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int off = frow * 128 + 16 * ((4 * half + s) ^ ((frow >> 1) & 7));
            wb[s] = *reinterpret_cast<const v4i*>(st + off);
#pragma unroll
            for (int t = 0; t < MT; ++t) ab[t][s] = *reinterpret_cast<const v4i*>(st + (1 + t) * 4096 + off);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int t = 0; t < MT; ++t)
                acc[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ab[t][s], wb[s], acc[t], 0, 0, 0);
    }
    compiler_fence();
    __syncthreads();  // red is zeroed
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = t * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            atomicAdd(&red[row * 32 + frow], acc[t][r]);
        }
    __syncthreads();
    for (int i = threadIdx.x; i < MT * 32 * 32; i += 64 * WPB) {
        const int row = i >> 5, col = n0 + (i & 31);
        if (row >= M || col >= N) continue;
        const int a = red[i];
        const int64_t o = static_cast<int64_t>(row) * N + col;
        const float dx = (OUT == kOutI32) ? 0.0f : sx[sx_per_token ? row : 0];
        const float dw = (OUT == kOutI32) ? 0.0f : sw[sw_per_tensor ? 0 : col];
        store_elem<OUT>(Y, o, a, dx, dw, epi, col, D, rD);
    }
}

template <int MT, int WPB, int ST>
hipError_t run_skinny(const int8_t* xq, const float* sx, bool per_token, const int8_t* wq,
                      const float* sw, bool w_per_tensor, int M, int N, int K, void* y, int out, const Epi& epi,
                    const Batch& bat, hipStream_t stream) {
    const dim3 grid((N + 31) / 32, static_cast<unsigned>(bat.count)), block(64 * WPB);
    const int pt = per_token ? 1 : 0;
    const int wpt = w_per_tensor ? 1 : 0;
    switch (out) {
        case kOutF32:
            gemm_skinny_kernel<MT, WPB, ST, kOutF32><<<grid, block, 0, stream>>>(xq, wq, sx, pt, sw, wpt, y, M, N, K, epi, bat);
            break;
        case kOutBF16:
            gemm_skinny_kernel<MT, WPB, ST, kOutBF16><<<grid, block, 0, stream>>>(xq, wq, sx, pt, sw, wpt, y, M, N, K, epi, bat);
            break;
        case kOutI8:
            gemm_skinny_kernel<MT, WPB, ST, kOutI8><<<grid, block, 0, stream>>>(xq, wq, sx, pt, sw, wpt, y, M, N, K, epi, bat);
            break;
        default:
            gemm_skinny_kernel<MT, WPB, ST, kOutI32><<<grid, block, 0, stream>>>(xq, wq, sx, pt, sw, wpt, y, M, N, K, epi, bat);
            break;
    }
    return hipGetLastError();
}

// Configurations measured on cold 70B-class FFN weights, (K, N) = (8192, 28672)
// and (28672, 8192): four waves per block when there are many channel blocks,
// eight when there are few; two 32-row X tiles take three stages.
hipError_t launch_skinny(const int8_t* xq, const float* sx, bool per_token, const int8_t* wq,
                         const float* sw, bool w_per_tensor, int M, int N, int K, void* y, int out, const Epi& epi,
                    const Batch& bat, hipStream_t stream) {
    const int blocks = (N + 31) / 32;
    if (M <= 32) {
        if (blocks >= 512) return run_skinny<1, 4, 2>(xq, sx, per_token, wq, sw, w_per_tensor, M, N, K, y, out, epi, bat, stream);
        return run_skinny<1, 8, 2>(xq, sx, per_token, wq, sw, w_per_tensor, M, N, K, y, out, epi, bat, stream);
    }
    return run_skinny<2, 4, 3>(xq, sx, per_token, wq, sw, w_per_tensor, M, N, K, y, out, epi, bat, stream);
}

}  // namespace

hipError_t launch_gemm(const int8_t* xq, const float* x_scale, bool x_per_token,
                       const int8_t* wq, const float* w_scale, bool w_per_tensor, int64_t M,
                       int64_t N, int64_t K, void* y, int out_kind, const Epi& epi,
                       const Batch& bat, hipStream_t stream) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    if (M <= 64) {
        // decode shapes: stream W once, K split over the waves of a block
        if (K % 128 == 0 && N * K < (int64_t(1) << 31)) {
            return launch_skinny(xq, x_scale, x_per_token, wq, w_scale, w_per_tensor, m, n, k, y, out_kind, epi, bat, stream);
        }
        return run<64, 128, 1, 4>(xq, x_scale, x_per_token, wq, w_scale, w_per_tensor, m, n, k, y, out_kind, epi, bat, stream);
    }
    // short K: the whole K of a tile in LDS at once
    if ((K == 64 || K == 128 || K == 256) && M * K < (int64_t(1) << 31) &&
        N * K < (int64_t(1) << 31)) {
        if (K == 64)
            return run_shortk<64>(xq, x_scale, x_per_token, wq, w_scale, w_per_tensor, m, n, k, y,
                                  out_kind, epi, bat, stream);
        if (K == 128)
            return run_shortk<128>(xq, x_scale, x_per_token, wq, w_scale, w_per_tensor, m, n, k,
                                   y, out_kind, epi, bat, stream);
        return run_shortk<256>(xq, x_scale, x_per_token, wq, w_scale, w_per_tensor, m, n, k, y,
                               out_kind, epi, bat, stream);
    }
    // ping-pong kernels: K a multiple of the 128-byte stage of the 256x128
    // tile, operand offsets in int32
    const bool pp_ok = (K % 128 == 0) && M * K < (int64_t(1) << 31) && N * K < (int64_t(1) << 31);
    if (pp_ok) {
        // pick the tiles by whole rounds of 256 CUs: a round of 256x256 tiles
        // (twice the work of a 256x128 tile) takes about 180/105 of a round of
        // 256x128 tiles (measured at K = 4096).  The first nb 256-column
        // blocks may take 256x256 tiles and the rest 256x128 tiles, in one
        // launch, large ones first.
        const int64_t tm = ((M + 255) / 256) * bat.count;  // row tiles of every batch entry
        const int64_t nb_all = (N + 255) / 256;
        // with r rounds of large tiles the best split is the widest that fits
        const int64_t rounds_all = (tm * nb_all + 255) / 256;
        int64_t best_nb = 0, best_cost = -1;
        for (int64_t r = 0; r <= rounds_all; ++r) {
            const int64_t nb = std::min<int64_t>(nb_all, 256 * r / tm);
            const int64_t rest = std::max<int64_t>(0, N - 256 * nb);
            const int64_t cost = ((tm * nb + 255) / 256) * 180 + ((tm * ((rest + 127) / 128) + 255) / 256) * 105;
            if (best_cost < 0 || cost < best_cost || (cost == best_cost && nb == nb_all)) {
                best_cost = cost;
                best_nb = nb;
            }
        }
        if (best_nb == nb_all)
            return run_pp<256, 256, 2, 4, 128, 2>(xq, x_scale, x_per_token, wq, w_scale, w_per_tensor, m, n, k, y,
                                                 out_kind, epi, bat, stream);
        if (best_nb == 0)
            return run_pp<256, 128, 4, 2, 128, 3>(xq, x_scale, x_per_token, wq, w_scale, w_per_tensor, m, n, k, y,
                                                  out_kind, epi, bat, stream);
        return run_pp_mixed(xq, x_scale, x_per_token, wq, w_scale, w_per_tensor, m, n, k, y, out_kind, epi, bat,
                            static_cast<int>(best_nb), stream);
    }
    const int64_t big_tiles = ((M + 255) / 256) * ((N + 127) / 128);
    if (big_tiles >= 256)
        return run<256, 128, 2, 2>(xq, x_scale, x_per_token, wq, w_scale, w_per_tensor, m, n, k, y, out_kind, epi, bat, stream);
    return run<128, 128, 2, 2>(xq, x_scale, x_per_token, wq, w_scale, w_per_tensor, m, n, k, y, out_kind, epi, bat, stream);
}

}  // namespace sq
