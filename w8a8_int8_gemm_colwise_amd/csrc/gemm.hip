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
// c ^ swz(r) so that the operand fetches (ds_read_b128) hit distinct banks.
// Blocks are remapped so that the tiles one XCD runs are neighbours (sharing
// A rows and B columns in that XCD's L2).
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
                                           const float* __restrict__ sw, void* __restrict__ Y,
                                           int M, int N) {
    const int frow = lane & 31;
    const int fhalf = lane >> 5;
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

template <int BM, int BN, int WAVES_M, int WAVES_N, int OUT>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_kernel(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, const float* __restrict__ sx,
    int sx_per_token, const float* __restrict__ sw, void* __restrict__ Y, int M, int N, int K) {
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
                                  sw, Y, M, N);
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


// Dequantizing epilogue through a per-wave LDS scratch (5 KB: 32 rows of
// 128 output bytes, 160-byte pitch so the two half-waves' rows land on
// different banks).  For each 32-row band the wave writes its accumulators in
// the MFMA layout (2- or 4-byte LDS stores), then reads the band back as
// 16-byte row chunks and stores whole 128-byte row segments to global memory.
// Elements are produced exactly as in store_tile.  Chunks that cross the
// matrix edge, or a Y whose rows are not 16-byte aligned, fall back to
// element stores.
template <int OUT, int TM, int TN>
__device__ __forceinline__ void store_tile_lds(const v16i (&acc)[TM][TN], int row0, int col0,
                                               int lane, const float* __restrict__ sx,
                                               int sx_per_token, const float* __restrict__ sw,
                                               void* __restrict__ Y, int M, int N,
                                               int8_t* scratch) {
    constexpr int ES = (OUT == kOutBF16) ? 2 : 4;  // output element bytes
    constexpr int JW = 128 / (32 * ES);            // 32-column tiles per 128-byte segment
    constexpr int PITCH = 160;
    constexpr int EPC = 16 / ES;                   // elements per 16-byte chunk
    static_assert(TN % JW == 0, "segments cover whole tiles");
    const int frow = lane & 31;
    const int fhalf = lane >> 5;
    const bool vec_ok = ((static_cast<int64_t>(N) * ES) % 16) == 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int jp = 0; jp < TN; jp += JW) {
#pragma unroll
            for (int jj = 0; jj < JW; ++jj) {
                const int j = jp + jj;
                const int col = col0 + j * 32 + frow;
                const float dw = (OUT == kOutI32 || col >= N) ? 0.0f : sw[col];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int rin = 8 * g + 4 * fhalf + r;
                        const int a = acc[i][j][4 * g + r];
                        int8_t* dst = scratch + rin * PITCH + (jj * 32 + frow) * ES;
                        if (OUT == kOutI32) {
                            *reinterpret_cast<int32_t*>(dst) = a;
                        } else {
                            const int row = min(row0 + i * 32 + rin, M - 1);
                            const float dx = sx[sx_per_token ? row : 0];
                            const float f = dx * dw;
                            const float y = static_cast<float>(a) * f;
                            if (OUT == kOutF32)
                                *reinterpret_cast<float*>(dst) = y;
                            else
                                *reinterpret_cast<__bf16*>(dst) = static_cast<__bf16>(y);
                        }
                    }
                }
            }
            // 32 rows x 8 chunks of 16 bytes, four per lane; LDS operations of
            // one wave complete in order, so the reads see the writes above
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int idx = lane + 64 * q;
                const int rr = idx >> 3, ch = idx & 7;
                const uint4 v = *reinterpret_cast<const uint4*>(scratch + rr * PITCH + ch * 16);
                const int grow = row0 + i * 32 + rr;
                const int gcol = col0 + jp * 32 + ch * EPC;
                if (grow >= M) continue;
                int8_t* out = static_cast<int8_t*>(Y) + (static_cast<int64_t>(grow) * N + gcol) * ES;
                if (vec_ok && gcol + EPC <= N) {
                    *reinterpret_cast<uint4*>(out) = v;
                } else {
                    const int8_t* src = reinterpret_cast<const int8_t*>(&v);
                    for (int e = 0; e < EPC; ++e)
                        if (gcol + e < N)
                            for (int b = 0; b < ES; ++b) out[e * ES + b] = src[e * ES + b];
                }
            }
        }
    }
}

// ---- pipelined kernel: direct global->LDS loads, STAGES LDS stages -----------
//
// Each stage holds the A rows then the B rows of one BK-byte K slice (rows of
// BK bytes, 16-byte chunks permuted by swz_k).  A stage is filled with
// global_load_lds_dwordx4: one instruction moves 64 lanes x 16 bytes into 1 KB
// of consecutive LDS, so lane q of a transfer fetches the global chunk whose
// swizzled LDS slot is q.  No VGPRs hold tiles in flight, so STAGES-1 stages
// are in flight while the matrix cores work on another.  The stages are
// distinct LDS arrays so the compiler can see that reading one stage does not
// depend on the transfers into the others; the waits are explicit vmcnt
// counts followed by a plain s_barrier, fenced for both the IR optimizers and
// the machine scheduler.

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Ordering point for both the IR optimizers (memory clobber) and the machine
// scheduler (sched_barrier with an empty mask lets nothing cross it).
__device__ __forceinline__ void compiler_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int BM, int BN, int WAVES_M, int WAVES_N, int BK, int STAGES, int MIN_BLOCKS, int OUT,
          bool SCHED = false>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, MIN_BLOCKS) void gemm_pipe_kernel(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, const float* __restrict__ sx,
    int sx_per_token, const float* __restrict__ sw, void* __restrict__ Y, int M, int N, int K) {
    using T = Tile<BM, BN, WAVES_M, WAVES_N>;
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int kRows = BM + BN;
    constexpr int kStageBytes = kRows * BK;
    constexpr int kCPR = BK / 16;              // 16-byte chunks per row
    constexpr int kRowsPerXfer = 1024 / BK;    // 1 KB per wave-wide transfer
    constexpr int kIssues = kRows / kRowsPerXfer;
    constexpr int IPW = kIssues / NW;
    static_assert(IPW * NW == kIssues, "stage divides over the waves");
    static_assert(BM % kRowsPerXfer == 0, "a transfer never straddles A and B");
    static_assert(STAGES >= 3 && STAGES <= 4, "3 or 4 stages");
    __shared__ __attribute__((aligned(1024))) int8_t L0[kStageBytes];
    __shared__ __attribute__((aligned(1024))) int8_t L1[kStageBytes];
    __shared__ __attribute__((aligned(1024))) int8_t L2[kStageBytes];
    __shared__ __attribute__((aligned(1024))) int8_t L3[STAGES > 3 ? kStageBytes : 16];

    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    int tmi, tni;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tmi, tni);
    const int m0 = tmi * BM, n0 = tni * BN;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    // byte offset (from A or B) of the source chunk of every transfer this
    // lane takes part in; the caller guarantees M*K and N*K fit in int32
    int src_off[IPW];
    bool src_a[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int q = (wave * IPW + i) * 64 + lane;  // 16-byte slot within the stage
        const int row = q / kCPR;
        const int c = (q % kCPR) ^ swz_k<BK>(row);
        src_a[i] = row < BM;  // uniform per transfer: BM is a multiple of 16
        src_off[i] = src_a[i] ? min(m0 + row, M - 1) * K + c * 16
                              : min(n0 + row - BM, N - 1) * K + c * 16;
    }
    auto issue = [&](int8_t* stage, int k0) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int8_t* g = (src_a[i] ? A : B) + (src_off[i] + k0);
            __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)(stage + (wave * IPW + i) * 1024), 16, 0, 0);
        }
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
    // Fragments of K-substep kk+1 are read from LDS while the MFMAs of substep
    // kk run (two fragment register sets).  With SCHED the machine scheduler
    // is told to interleave one LDS read after each MFMA.
    auto load_frags = [&](const int8_t* S, int kk, v4i (&fa)[T::TM], v4i (&fb)[T::TN]) {
        const int chunk = 2 * kk + fhalf;
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
            fa[i] = *reinterpret_cast<const v4i*>(
                S + lds_off_k<BK>(wm * T::WM + i * 32 + frow, chunk));
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
            fb[j] = *reinterpret_cast<const v4i*>(
                S + BM * BK + lds_off_k<BK>(wn * T::WN + j * 32 + frow, chunk));
    };
    auto compute = [&](const int8_t* S) {
        constexpr int NKK = BK / 32;
        v4i fa[2][T::TM], fb[2][T::TN];
        load_frags(S, 0, fa[0], fb[0]);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const int cur = kk & 1;
            if (kk + 1 < NKK) load_frags(S, kk + 1, fa[cur ^ 1], fb[cur ^ 1]);
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int j = 0; j < T::TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[cur][i], fb[cur][j],
                                                                      acc[i][j], 0, 0, 0);
            if constexpr (SCHED) {
                if (kk + 1 < NKK) {
#pragma unroll
                    for (int q = 0; q < T::TM + T::TN; ++q) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, T::TM * T::TN - (T::TM + T::TN), 0);
                }
            }
        }
    };
    // Wait until this wave's transfers into the stage about to be read have
    // landed (`younger` later stages may stay in flight), then meet the other
    // waves: after the barrier every wave's part of the stage is in LDS and
    // every wave has finished reading the stage that the next issue reuses.
    auto sync_stage = [&](int younger) {
        if (younger >= 2) wait_vmcnt<2 * IPW>();
        else if (younger == 1) wait_vmcnt<IPW>();
        else wait_vmcnt<0>();
        compiler_fence();
        __builtin_amdgcn_s_barrier();
        compiler_fence();
    };
    // One pipeline step for stage t held in `cur`; the step then refills
    // `nxt` (the buffer read one step earlier) with stage t + STAGES - 1.  In
    // the steady state STAGES-2 younger stages are in flight and the refill is
    // unconditional, so the step is straight-line code.  The buffers are passed
    // as the LDS arrays themselves so the compiler keeps their identities.
    const int KT = K / BK;
    auto steady = [&](int t, const int8_t* cur, int8_t* nxt) {
        wait_vmcnt<(STAGES - 2) * IPW>();
        compiler_fence();
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        issue(nxt, (t + STAGES - 1) * BK);
        compute(cur);
    };
    auto drain = [&](int t, const int8_t* cur, int8_t* nxt) {
        sync_stage(min(KT - 1 - t, STAGES - 2));
        if (t + STAGES - 1 < KT) issue(nxt, (t + STAGES - 1) * BK);
        compute(cur);
    };

    issue(L0, 0);
    if (KT > 1) issue(L1, BK);
    if (STAGES > 3 && KT > 2) issue(L2, 2 * BK);
    // steady state in groups of STAGES steps (buffers rotate 0..STAGES-1)
    int t = 0;
    if constexpr (STAGES == 4) {
        for (; t + 2 * STAGES - 1 <= KT; t += STAGES) {
            steady(t, L0, L3);
            steady(t + 1, L1, L0);
            steady(t + 2, L2, L1);
            steady(t + 3, L3, L2);
        }
        for (int g = 0; g < 2; ++g, t += STAGES) {
            if (t < KT) drain(t, L0, L3);
            if (t + 1 < KT) drain(t + 1, L1, L0);
            if (t + 2 < KT) drain(t + 2, L2, L1);
            if (t + 3 < KT) drain(t + 3, L3, L2);
        }
    } else {
        for (; t + 2 * STAGES - 1 <= KT; t += STAGES) {
            steady(t, L0, L2);
            steady(t + 1, L1, L0);
            steady(t + 2, L2, L1);
        }
        for (int g = 0; g < 2; ++g, t += STAGES) {
            if (t < KT) drain(t, L0, L2);
            if (t + 1 < KT) drain(t + 1, L1, L0);
            if (t + 2 < KT) drain(t + 2, L2, L1);
        }
    }

    // epilogue through LDS: every wave has finished reading the stages
    __syncthreads();
    constexpr int kScratch = 32 * 160;  // per wave
    constexpr int kPerStage = kStageBytes / kScratch;
    static_assert(kPerStage * 2 >= NW, "two stages hold the per-wave scratch");
    int8_t* scratch = (wave < kPerStage) ? L0 + wave * kScratch : L1 + (wave - kPerStage) * kScratch;
    store_tile_lds<OUT, T::TM, T::TN>(acc, m0 + wm * T::WM, n0 + wn * T::WN, lane, sx,
                                      sx_per_token, sw, Y, M, N, scratch);
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int BK, int STAGES, int MIN_BLOCKS,
          bool SCHED = false>
hipError_t run_pipe(const int8_t* xq, const float* sx, bool per_token, const int8_t* wq,
                    const float* sw, int M, int N, int K, void* y, int out, hipStream_t stream) {
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const dim3 grid(tiles), block(64 * WAVES_M * WAVES_N);
    const int pt = per_token ? 1 : 0;
    switch (out) {
        case kOutF32:
            gemm_pipe_kernel<BM, BN, WAVES_M, WAVES_N, BK, STAGES, MIN_BLOCKS, kOutF32, SCHED>
                <<<grid, block, 0, stream>>>(xq, wq, sx, pt, sw, y, M, N, K);
            break;
        case kOutBF16:
            gemm_pipe_kernel<BM, BN, WAVES_M, WAVES_N, BK, STAGES, MIN_BLOCKS, kOutBF16, SCHED>
                <<<grid, block, 0, stream>>>(xq, wq, sx, pt, sw, y, M, N, K);
            break;
        default:
            gemm_pipe_kernel<BM, BN, WAVES_M, WAVES_N, BK, STAGES, MIN_BLOCKS, kOutI32, SCHED>
                <<<grid, block, 0, stream>>>(xq, wq, sx, pt, sw, y, M, N, K);
            break;
    }
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

// fill one stage with the 128-byte K chunk `chunk` of every row it holds
template <int XFERS>
__device__ __forceinline__ void skinny_issue(const int8_t* const* src, int8_t* stage, int chunk) {
    const int64_t k0 = static_cast<int64_t>(chunk) * 128;
#pragma unroll
    for (int q = 0; q < XFERS; ++q)
        __builtin_amdgcn_global_load_lds(src[q] + k0, (lds_ptr_t)(stage + q * 1024), 16, 0, 0);
}

template <int MT, int WPB, int ST, int OUT>
__global__ __launch_bounds__(64 * WPB) void gemm_skinny_kernel(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, const float* __restrict__ sx,
    int sx_per_token, const float* __restrict__ sw, void* __restrict__ Y, int M, int N, int K) {
    using S = Skinny<MT, WPB, ST>;
    static_assert(ST >= 2 && ST <= 3, "2 or 3 stages");
    __shared__ __attribute__((aligned(1024))) int8_t ring[S::kRing];
    __shared__ int32_t red[MT * 32 * 32];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * 32;
    const int frow = lane & 31;
    const int half = lane >> 5;

    for (int i = threadIdx.x; i < MT * 32 * 32; i += 64 * WPB) red[i] = 0;

    // transfer q of a stage: group g = q / 4 (0 = W, 1.. = X tiles), rows
    // 8 (q % 4) .. 8 (q % 4) + 7 of the group; lane -> row + lane / 8 and the
    // source slot whose swizzled position is lane % 8
    int8_t* my = ring + wave * ST * S::kStage;
    const int8_t* src[4 * (1 + MT)];
#pragma unroll
    for (int q = 0; q < S::kXfers; ++q) {
        const int g = q / 4;
        const int row = 8 * (q % 4) + (lane >> 3);
        const int slot = (lane & 7) ^ ((row >> 1) & 7);
        src[q] = g == 0 ? B + static_cast<int64_t>(min(n0 + row, N - 1)) * K + 16 * slot
                        : A + static_cast<int64_t>(min((g - 1) * 32 + row, M - 1)) * K + 16 * slot;
    }
    const int chunks = K / 128;
    const int first = static_cast<int>(static_cast<int64_t>(wave) * chunks / WPB);
    const int cnt = static_cast<int>(static_cast<int64_t>(wave + 1) * chunks / WPB) - first;
    v16i acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0;

    for (int i = 0; i < ST - 1 && i < cnt; ++i) skinny_issue<S::kXfers>(src, my + (i % ST) * S::kStage, first + i);
    for (int i = 0; i < cnt; ++i) {
        compiler_fence();
        if (i + ST - 1 < cnt)
            skinny_issue<S::kXfers>(src, my + ((i + ST - 1) % ST) * S::kStage, first + i + ST - 1);
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
        if (OUT == kOutI32) {
            static_cast<int32_t*>(Y)[o] = a;
        } else {
            const float f = sx[sx_per_token ? row : 0] * sw[col];
            const float y = static_cast<float>(a) * f;
            if (OUT == kOutF32)
                static_cast<float*>(Y)[o] = y;
            else
                static_cast<__bf16*>(Y)[o] = static_cast<__bf16>(y);
        }
    }
}

template <int MT, int WPB, int ST>
hipError_t run_skinny(const int8_t* xq, const float* sx, bool per_token, const int8_t* wq,
                      const float* sw, int M, int N, int K, void* y, int out, hipStream_t stream) {
    const dim3 grid((N + 31) / 32), block(64 * WPB);
    const int pt = per_token ? 1 : 0;
    switch (out) {
        case kOutF32:
            gemm_skinny_kernel<MT, WPB, ST, kOutF32><<<grid, block, 0, stream>>>(xq, wq, sx, pt, sw, y, M, N, K);
            break;
        case kOutBF16:
            gemm_skinny_kernel<MT, WPB, ST, kOutBF16><<<grid, block, 0, stream>>>(xq, wq, sx, pt, sw, y, M, N, K);
            break;
        default:
            gemm_skinny_kernel<MT, WPB, ST, kOutI32><<<grid, block, 0, stream>>>(xq, wq, sx, pt, sw, y, M, N, K);
            break;
    }
    return hipGetLastError();
}

// Configurations measured on cold 70B-class FFN weights, (K, N) = (8192, 28672)
// and (28672, 8192): four waves per block when there are many channel blocks,
// eight when there are few; two 32-row X tiles take three stages.
hipError_t launch_skinny(const int8_t* xq, const float* sx, bool per_token, const int8_t* wq,
                         const float* sw, int M, int N, int K, void* y, int out, hipStream_t stream) {
    const int blocks = (N + 31) / 32;
    if (M <= 32) {
        if (blocks >= 512) return run_skinny<1, 4, 2>(xq, sx, per_token, wq, sw, M, N, K, y, out, stream);
        return run_skinny<1, 8, 2>(xq, sx, per_token, wq, sw, M, N, K, y, out, stream);
    }
    return run_skinny<2, 4, 3>(xq, sx, per_token, wq, sw, M, N, K, y, out, stream);
}

}  // namespace

hipError_t launch_gemm(const int8_t* xq, const float* x_scale, bool x_per_token,
                       const int8_t* wq, const float* w_scale, int64_t M, int64_t N, int64_t K,
                       void* y, int out_kind, hipStream_t stream) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    if (M <= 64) {
        // decode shapes: stream W once, K split over the waves of a block
        if (K % 128 == 0) {
            return launch_skinny(xq, x_scale, x_per_token, wq, w_scale, m, n, k, y, out_kind, stream);
        }
        return run<64, 128, 1, 4>(xq, x_scale, x_per_token, wq, w_scale, m, n, k, y, out_kind, stream);
    }
    // pipelined kernels: 128-byte K stages, operand offsets in int32
    const bool pipe_ok = (K % 128 == 0) && M * K < (int64_t(1) << 31) && N * K < (int64_t(1) << 31);
    if (pipe_ok) {
        // pick the tile by whole waves of 256 CUs: a 256x256 tile does twice the
        // work of a 256x128 tile at slightly higher efficiency
        const int64_t t_big = ((M + 255) / 256) * ((N + 255) / 256);
        const int64_t t_mid = ((M + 255) / 256) * ((N + 127) / 128);
        const int64_t cost_big = ((t_big + 255) / 256) * 2 * 100;
        const int64_t cost_mid = ((t_mid + 255) / 256) * 105;
        if (cost_big <= cost_mid)
            return run_pipe<256, 256, 2, 4, 64, 4, 1>(xq, x_scale, x_per_token, wq, w_scale, m, n, k,
                                                      y, out_kind, stream);
        return run_pipe<256, 128, 4, 2, 128, 3, 1>(xq, x_scale, x_per_token, wq, w_scale, m, n, k,
                                                   y, out_kind, stream);
    }
    const int64_t big_tiles = ((M + 255) / 256) * ((N + 127) / 128);
    if (big_tiles >= 256)
        return run<256, 128, 2, 2>(xq, x_scale, x_per_token, wq, w_scale, m, n, k, y, out_kind, stream);
    return run<128, 128, 2, 2>(xq, x_scale, x_per_token, wq, w_scale, m, n, k, y, out_kind, stream);
}

}  // namespace sq
