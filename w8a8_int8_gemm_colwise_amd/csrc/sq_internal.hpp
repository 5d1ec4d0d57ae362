// sq_internal.hpp -- host-side launchers implemented by the library's HIP
// translation units and called by the C ABI layer.  All sizes are validated
// by the ABI layer before these run; each launcher only enqueues kernels and
// returns the HIP error of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sq {

enum class Dt : int { F32 = 0, BF16 = 1 };
enum class ActMode : int { PerToken = 0, Static = 1, DynamicTensor = 2 };

// v rounded up to a whole number of 64-lane waves.
inline int round_up64(int64_t v) { return static_cast<int>(((v + 63) / 64) * 64); }

// Calibration (offline half).
hipError_t launch_calibrate(const void* x_cal, Dt x_dt, int64_t T, const void* w, Dt w_dt,
                            int64_t N, int64_t K, float alpha, bool w_per_tensor, const float* gamma,
                            const float* beta, float* s, int8_t* wq, float* w_scale,
                            float* act_scale_static, float* gamma_s, float* beta_s,
                            float* x_absmax, float* w_absmax, const float* act_stat,
                            hipStream_t stream);

// Saturation count of the static quantizer (count mode: no codes written);
// *clip and clip_ch[K] (optional) are overwritten.
hipError_t launch_clip_count(const void* x, Dt x_dt, int64_t M, int64_t K, const float* s,
                             const float* gamma_s, const float* beta_s, float eps,
                             const float* static_scale, unsigned long long* clip,
                             uint32_t* clip_ch, hipStream_t stream);

// Robust calibration: the nearest-rank quantile (rank 1..T) of |x[:, j]| per
// channel into out[K] (floored); workspace of quantile_workspace_bytes(K).
size_t quantile_workspace_bytes(int64_t K);
hipError_t launch_channel_quantile(const void* x, Dt x_dt, int64_t T, int64_t K, int64_t rank,
                                   float* out, void* ws, hipStream_t stream);
// The same with the library's own per-device scratch (K <= SQ_NOALLOC_MAX_K;
// the current device must be the stream's): no allocation, no workspace.
hipError_t launch_channel_quantile_noalloc(const void* x, Dt x_dt, int64_t T, int64_t K,
                                           int64_t rank, float* out, hipStream_t stream);

// Activation smoothing + quantization (runtime).
hipError_t launch_act_quant(const void* x, Dt x_dt, int64_t M, int64_t K, const float* s,
                            const float* gamma_s, const float* beta_s, float eps,
                            ActMode mode, const float* static_scale, int8_t* xq,
                            float* x_scale, hipStream_t stream);

// step[0] = RN(max(FLOOR, max_i maxima[i]) / 127): the per-tensor step from n
// non-negative maxima (one block).
hipError_t launch_tensor_step(const float* maxima, int64_t n, float* step, hipStream_t stream);

// Fused GEMM epilogue after the dequantization: bias (one RN addition), ReLU
// (y > 0 ? y : +0), and for int8 output the next linear's smoothing division
// and static step, clamp(rne(RN(RN(y / s'_n) / D))).
struct Epi {
    const float* bias = nullptr;       // [N] or null
    const float* next_s = nullptr;     // [N] or null (s' = 1); int8 output only
    const float* next_step = nullptr;  // [1] device, D; required for int8 output
    int relu = 0;
};

// Strided batch of independent GEMMs (the attention products): entry z uses
// A + z*a, B + z*b, x_scale + z*sx, w_scale + z*sw and writes Y + z*y (all in
// elements).  count = 1 is the plain GEMM.
struct Batch {
    int64_t count = 1;
    int64_t a = 0, b = 0, sx = 0, sw = 0, y = 0;
};

// Int8 GEMM with dequantizing epilogue.  out_kind: 0 = f32, 1 = bf16, 2 = i32
// (raw accumulators, epilogue unused), 3 = i8 (requantized for the next linear).
// w_per_tensor: w_scale[0] is the step of every output channel.
hipError_t launch_gemm(const int8_t* xq, const float* x_scale, bool x_per_token,
                       const int8_t* wq, const float* w_scale, bool w_per_tensor, int64_t M,
                       int64_t N, int64_t K, void* y, int out_kind, const Epi& epi,
                       const Batch& bat, hipStream_t stream);

// Alpha search over candidate smoothing strengths (host array alphas[n]):
// err[i], werr[i] (device fp64) and best (device); workspace of
// alpha_workspace_bytes(T, N, K).
size_t alpha_workspace_bytes(int64_t T, int64_t N, int64_t K);
hipError_t launch_alpha_search(const void* x_cal, Dt x_dt, int64_t T, const void* w, Dt w_dt,
                               int64_t N, int64_t K, const float* alphas, int n_alpha,
                               ActMode mode, bool w_per_tensor, double* err, double* werr,
                               int32_t* best, void* ws, hipStream_t stream);

}  // namespace sq
