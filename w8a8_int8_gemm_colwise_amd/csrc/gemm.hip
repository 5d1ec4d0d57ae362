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
// Y[M, N] = Xq[M, K] . Wq[N, K]^T: both operands are K-contiguous ("NT"), the
// layout the MFMA operand registers want (16 consecutive int8 of one row per
// lane).  Each block owns a BM x BN tile of Y; K advances in 64-byte tiles
// staged through LDS with two buffers (global loads for tile k+1 are in flight
// while the matrix cores work on tile k).  Each wave owns a WM x WN sub-tile
// made of 32x32 v_mfma_i32_32x32x32_i8 tiles accumulated in int32 registers.
// LDS rows are 64 bytes; the 16-byte chunk c of row r is stored at chunk
// c ^ f(r) so that the ds_read_b128 of 16 consecutive rows hit distinct banks.
// Blocks are remapped so that the tiles one XCD runs are neighbours (sharing
// A rows and B columns in that XCD's L2).
#include "sq_device.hpp"
#include "sq_internal.hpp"

namespace sq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;              // K bytes per LDS stage
constexpr int kChunksPerRow = kBK / 16;
constexpr int kXcds = 8;

__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * kBK + ((chunk ^ swz(row)) << 4);
}

enum OutKind { kOutF32 = 0, kOutBF16 = 1, kOutI32 = 2 };

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
    static_assert(LA * kThreads == BM * kChunksPerRow, "A tile divides over threads");
    static_assert(LB * kThreads == BN * kChunksPerRow, "B tile divides over threads");
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

template <int BM, int BN, int WAVES_M, int WAVES_N, int OUT>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_kernel(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, const float* __restrict__ sx,
    int sx_per_token, const float* __restrict__ sw, void* __restrict__ Y, int M, int N, int K) {
    using T = Tile<BM, BN, WAVES_M, WAVES_N>;
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
    int a_lds[T::LA], b_lds[T::LB], a_kc[T::LA], b_kc[T::LB];
#pragma unroll
    for (int j = 0; j < T::LA; ++j) {
        const int q = tid + j * T::kThreads;
        const int row = q / kChunksPerRow, c = q % kChunksPerRow;
        const int grow = min(m0 + row, M - 1);
        a_src[j] = A + static_cast<int64_t>(grow) * K + c * 16;
        a_lds[j] = lds_off(row, c);
        a_kc[j] = c * 16;
    }
#pragma unroll
    for (int j = 0; j < T::LB; ++j) {
        const int q = tid + j * T::kThreads;
        const int row = q / kChunksPerRow, c = q % kChunksPerRow;
        const int grow = min(n0 + row, N - 1);
        b_src[j] = B + static_cast<int64_t>(grow) * K + c * 16;
        b_lds[j] = lds_off(row, c);
        b_kc[j] = c * 16;
    }

    v4i ra[T::LA], rb[T::LB];
    auto gload = [&](int k0) {
#pragma unroll
        for (int j = 0; j < T::LA; ++j)
            ra[j] = (k0 + a_kc[j] < K) ? *reinterpret_cast<const v4i*>(a_src[j] + k0) : v4i{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < T::LB; ++j)
            rb[j] = (k0 + b_kc[j] < K) ? *reinterpret_cast<const v4i*>(b_src[j] + k0) : v4i{0, 0, 0, 0};
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

    // epilogue: lane holds rows 8*g + 4*(lane/32) + r (g, r in 0..3) of
    // column lane%32 of each 32x32 tile
#pragma unroll
    for (int i = 0; i < T::TM; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * T::WM + i * 32 + 8 * g + 4 * fhalf + r;
                if (row >= M) continue;
                const float dx = (OUT == kOutI32) ? 0.0f : sx[sx_per_token ? row : 0];
#pragma unroll
                for (int j = 0; j < T::TN; ++j) {
                    const int col = n0 + wn * T::WN + j * 32 + frow;
                    if (col >= N) continue;
                    const int a = acc[i][j][4 * g + r];
                    const int64_t o = static_cast<int64_t>(row) * N + col;
                    if (OUT == kOutI32) {
                        static_cast<int32_t*>(Y)[o] = a;
                    } else {
                        const float f = dx * sw[col];
                        const float y = static_cast<float>(a) * f;
                        if (OUT == kOutF32)
                            static_cast<float*>(Y)[o] = y;
                        else
                            static_cast<__bf16*>(Y)[o] = static_cast<__bf16>(y);
                    }
                }
            }
        }
    }
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
hipError_t run(const int8_t* xq, const float* sx, bool per_token, const int8_t* wq,
               const float* sw, int M, int N, int K, void* y, int out, hipStream_t stream) {
    using T = Tile<BM, BN, WAVES_M, WAVES_N>;
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const dim3 grid(tiles), block(T::kThreads);
    const int pt = per_token ? 1 : 0;
    switch (out) {
        case kOutF32:
            gemm_kernel<BM, BN, WAVES_M, WAVES_N, kOutF32><<<grid, block, 0, stream>>>(
                xq, wq, sx, pt, sw, y, M, N, K);
            break;
        case kOutBF16:
            gemm_kernel<BM, BN, WAVES_M, WAVES_N, kOutBF16><<<grid, block, 0, stream>>>(
                xq, wq, sx, pt, sw, y, M, N, K);
            break;
        default:
            gemm_kernel<BM, BN, WAVES_M, WAVES_N, kOutI32><<<grid, block, 0, stream>>>(
                xq, wq, sx, pt, sw, y, M, N, K);
            break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const int8_t* xq, const float* x_scale, bool x_per_token,
                       const int8_t* wq, const float* w_scale, int64_t M, int64_t N, int64_t K,
                       void* y, int out_kind, hipStream_t stream) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    if (M <= 64)
        return run<64, 128, 1, 4>(xq, x_scale, x_per_token, wq, w_scale, m, n, k, y, out_kind, stream);
    const int64_t big_tiles = ((M + 255) / 256) * ((N + 127) / 128);
    if (big_tiles >= 256)
        return run<256, 128, 2, 2>(xq, x_scale, x_per_token, wq, w_scale, m, n, k, y, out_kind, stream);
    return run<128, 128, 2, 2>(xq, x_scale, x_per_token, wq, w_scale, m, n, k, y, out_kind, stream);
}

}  // namespace sq
