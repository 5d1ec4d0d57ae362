// abi.hip -- the C ABI of libsq.so: host-side validation, then the launchers.
// See include/sq.h for the contract of every entry point.
#include "../../include/sq.h"

#include <algorithm>
#include <cmath>

#include "sq_internal.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_k(int64_t K) { return K > 0 && K % 64 == 0 && K <= SQ_MAX_K; }

bool valid_rows(int64_t r) { return r >= 0 && r <= 0x7fffffffLL; }

bool float_dtype(sq_dtype d) { return d == SQ_F32 || d == SQ_BF16; }

sq::Dt to_dt(sq_dtype d) { return d == SQ_BF16 ? sq::Dt::BF16 : sq::Dt::F32; }

sq_status from_hip(hipError_t e) { return e == hipSuccess ? SQ_OK : SQ_ERR_HIP; }

}  // namespace

extern "C" {

sq_status sq_calibrate(const void* x_cal, sq_dtype x_dt, int64_t T, const void* w, sq_dtype w_dt,
                       int64_t N, int64_t K, float alpha, sq_weight_mode w_mode,
                       const float* ln_gamma, const float* ln_beta, float* s, int8_t* wq,
                       float* w_scale, float* act_scale_static, float* ln_gamma_s,
                       float* ln_beta_s, float* x_absmax, float* w_absmax, sq_stream_t stream) {
    if (!valid_k(K) || !valid_rows(T) || !valid_rows(N)) return SQ_ERR_BAD_SHAPE;
    if (!float_dtype(x_dt) || !float_dtype(w_dt)) return SQ_ERR_BAD_DTYPE;
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return SQ_ERR_BAD_ALPHA;
    if (w_mode != SQ_W_PER_CHANNEL && w_mode != SQ_W_PER_TENSOR) return SQ_ERR_BAD_MODE;
    if (!s || !x_absmax || !w_absmax) return SQ_ERR_NULL_ARG;
    if (T > 0 && !x_cal) return SQ_ERR_NULL_ARG;
    if (N > 0 && (!w || !wq)) return SQ_ERR_NULL_ARG;
    if ((N > 0 || w_mode == SQ_W_PER_TENSOR) && !w_scale) return SQ_ERR_NULL_ARG;
    if ((ln_gamma == nullptr) != (ln_beta == nullptr)) return SQ_ERR_BAD_MODE;
    if (ln_gamma && (!ln_gamma_s || !ln_beta_s)) return SQ_ERR_NULL_ARG;
    const void* ptrs[] = {x_cal, w, ln_gamma, ln_beta, s, wq, w_scale, act_scale_static,
                          ln_gamma_s, ln_beta_s, x_absmax, w_absmax};
    for (const void* p : ptrs)
        if (!aligned16(p)) return SQ_ERR_ALIGNMENT;
    return from_hip(sq::launch_calibrate(
        x_cal, to_dt(x_dt), T, w, to_dt(w_dt), N, K, alpha, w_mode == SQ_W_PER_TENSOR, ln_gamma,
        ln_beta, s, wq, w_scale,
        act_scale_static, ln_gamma ? ln_gamma_s : nullptr, ln_gamma ? ln_beta_s : nullptr,
        x_absmax, w_absmax, nullptr, reinterpret_cast<hipStream_t>(stream)));
}

sq_status sq_calibrate_stat(const float* act_stat, const void* w, sq_dtype w_dt, int64_t N,
                            int64_t K, float alpha, sq_weight_mode w_mode,
                            const float* ln_gamma, const float* ln_beta, float* s, int8_t* wq,
                            float* w_scale, float* act_scale_static, float* ln_gamma_s,
                            float* ln_beta_s, float* a_out, float* w_absmax,
                            sq_stream_t stream) {
    if (!valid_k(K) || !valid_rows(N)) return SQ_ERR_BAD_SHAPE;
    if (!float_dtype(w_dt)) return SQ_ERR_BAD_DTYPE;
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return SQ_ERR_BAD_ALPHA;
    if (w_mode != SQ_W_PER_CHANNEL && w_mode != SQ_W_PER_TENSOR) return SQ_ERR_BAD_MODE;
    if (!act_stat || !s || !a_out || !w_absmax) return SQ_ERR_NULL_ARG;
    if (N > 0 && (!w || !wq)) return SQ_ERR_NULL_ARG;
    if ((N > 0 || w_mode == SQ_W_PER_TENSOR) && !w_scale) return SQ_ERR_NULL_ARG;
    if ((ln_gamma == nullptr) != (ln_beta == nullptr)) return SQ_ERR_BAD_MODE;
    if (ln_gamma && (!ln_gamma_s || !ln_beta_s)) return SQ_ERR_NULL_ARG;
    const void* ptrs[] = {act_stat, w, ln_gamma, ln_beta, s, wq, w_scale, act_scale_static,
                          ln_gamma_s, ln_beta_s, a_out, w_absmax};
    for (const void* p : ptrs)
        if (!aligned16(p)) return SQ_ERR_ALIGNMENT;
    return from_hip(sq::launch_calibrate(
        nullptr, sq::Dt::F32, 0, w, to_dt(w_dt), N, K, alpha, w_mode == SQ_W_PER_TENSOR,
        ln_gamma, ln_beta, s, wq, w_scale, act_scale_static, ln_gamma ? ln_gamma_s : nullptr,
        ln_gamma ? ln_beta_s : nullptr, a_out, w_absmax, act_stat,
        reinterpret_cast<hipStream_t>(stream)));
}

sq_status sq_smooth_quantize_act(const void* x, sq_dtype x_dt, int64_t M, int64_t K,
                                 const float* s, const float* ln_gamma_s,
                                 const float* ln_beta_s, float ln_eps, sq_act_mode mode,
                                 const float* static_scale, int8_t* xq, float* x_scale,
                                 sq_stream_t stream) {
    if (!valid_k(K) || !valid_rows(M)) return SQ_ERR_BAD_SHAPE;
    if (!float_dtype(x_dt)) return SQ_ERR_BAD_DTYPE;
    if (mode != SQ_PER_TOKEN && mode != SQ_STATIC_PER_TENSOR && mode != SQ_DYNAMIC_PER_TENSOR)
        return SQ_ERR_BAD_MODE;
    const bool ln = (ln_gamma_s != nullptr) || (ln_beta_s != nullptr);
    if (ln) {
        if (s) return SQ_ERR_BAD_MODE;
        if (!ln_gamma_s || !ln_beta_s) return SQ_ERR_NULL_ARG;
        if (!(ln_eps > 0.0f) || !std::isfinite(ln_eps)) return SQ_ERR_BAD_MODE;
    } else if (!s) {
        return SQ_ERR_NULL_ARG;
    }
    if (mode == SQ_STATIC_PER_TENSOR && !static_scale) return SQ_ERR_NULL_ARG;
    if (M > 0 && (!x || !xq)) return SQ_ERR_NULL_ARG;
    // per-token steps are written only for rows that exist; the batch step of
    // the dynamic per-tensor mode is written even for an empty batch (FLOOR/127)
    if (mode == SQ_PER_TOKEN && M > 0 && !x_scale) return SQ_ERR_NULL_ARG;
    if (mode == SQ_DYNAMIC_PER_TENSOR && !x_scale) return SQ_ERR_NULL_ARG;
    const float* st = (mode == SQ_STATIC_PER_TENSOR) ? static_scale : nullptr;
    const void* ptrs[] = {x, s, ln_gamma_s, ln_beta_s, st, xq, x_scale};
    for (const void* p : ptrs)
        if (!aligned16(p)) return SQ_ERR_ALIGNMENT;
    const sq::ActMode am = mode == SQ_PER_TOKEN           ? sq::ActMode::PerToken
                           : mode == SQ_STATIC_PER_TENSOR ? sq::ActMode::Static
                                                          : sq::ActMode::DynamicTensor;
    return from_hip(sq::launch_act_quant(x, to_dt(x_dt), M, K, ln ? nullptr : s, ln_gamma_s,
                                         ln_beta_s, ln_eps, am, st, xq, x_scale,
                                         reinterpret_cast<hipStream_t>(stream)));
}

sq_status sq_gemm_w8a8_ex(const int8_t* xq, const float* x_scale, sq_act_mode x_mode,
                          const int8_t* wq, const float* w_scale, sq_weight_mode w_mode,
                          int64_t M, int64_t N, int64_t K, const sq_epilogue* epi, void* y,
                          sq_dtype y_dt, sq_stream_t stream) {
    if (!valid_k(K) || !valid_rows(M) || !valid_rows(N)) return SQ_ERR_BAD_SHAPE;
    if (M * N > (int64_t(1) << 40)) return SQ_ERR_BAD_SHAPE;
    if (y_dt != SQ_F32 && y_dt != SQ_BF16 && y_dt != SQ_I32 && y_dt != SQ_I8)
        return SQ_ERR_BAD_DTYPE;
    if (x_mode != SQ_PER_TOKEN && x_mode != SQ_STATIC_PER_TENSOR &&
        x_mode != SQ_DYNAMIC_PER_TENSOR)
        return SQ_ERR_BAD_MODE;
    if (w_mode != SQ_W_PER_CHANNEL && w_mode != SQ_W_PER_TENSOR) return SQ_ERR_BAD_MODE;
    sq::Epi e;
    if (epi) {
        e.bias = epi->bias;
        e.next_s = epi->next_s;
        e.next_step = epi->next_scale;
        e.relu = epi->relu != 0;
    }
    const bool any = e.bias || e.next_s || e.next_step || e.relu;
    if (y_dt == SQ_I32 && any) return SQ_ERR_BAD_MODE;
    if (y_dt != SQ_I8 && (e.next_s || e.next_step)) return SQ_ERR_BAD_MODE;
    if (y_dt == SQ_I8 && !e.next_step) return SQ_ERR_NULL_ARG;
    if (M > 0 && N > 0) {
        if (!xq || !wq || !y) return SQ_ERR_NULL_ARG;
        if (y_dt != SQ_I32 && (!x_scale || !w_scale)) return SQ_ERR_NULL_ARG;
    }
    const void* ptrs[] = {xq, x_scale, wq, w_scale, y, e.bias, e.next_s, e.next_step};
    for (const void* p : ptrs)
        if (!aligned16(p)) return SQ_ERR_ALIGNMENT;
    const int out = (y_dt == SQ_F32) ? 0 : (y_dt == SQ_BF16) ? 1 : (y_dt == SQ_I32) ? 2 : 3;
    return from_hip(sq::launch_gemm(xq, x_scale, x_mode == SQ_PER_TOKEN, wq, w_scale,
                                    w_mode == SQ_W_PER_TENSOR, M, N, K, y, out, e, sq::Batch{},
                                    reinterpret_cast<hipStream_t>(stream)));
}

sq_status sq_bmm_w8a8(const int8_t* xq, int64_t xq_stride, const float* x_scale,
                      int64_t xs_stride, sq_act_mode x_mode, const int8_t* wq,
                      int64_t wq_stride, const float* w_scale, int64_t ws_stride,
                      sq_weight_mode w_mode, int64_t batch, int64_t M, int64_t N, int64_t K,
                      void* y, int64_t y_stride, sq_dtype y_dt, sq_stream_t stream) {
    if (!valid_k(K) || !valid_rows(M) || !valid_rows(N)) return SQ_ERR_BAD_SHAPE;
    if (batch < 0 || batch > 65535 || M * N > (int64_t(1) << 40)) return SQ_ERR_BAD_SHAPE;
    if (xq_stride < 0 || xs_stride < 0 || wq_stride < 0 || ws_stride < 0 || y_stride < 0)
        return SQ_ERR_BAD_SHAPE;
    if (y_dt != SQ_F32 && y_dt != SQ_BF16 && y_dt != SQ_I32) return SQ_ERR_BAD_DTYPE;
    if (x_mode != SQ_PER_TOKEN && x_mode != SQ_STATIC_PER_TENSOR &&
        x_mode != SQ_DYNAMIC_PER_TENSOR)
        return SQ_ERR_BAD_MODE;
    if (w_mode != SQ_W_PER_CHANNEL && w_mode != SQ_W_PER_TENSOR) return SQ_ERR_BAD_MODE;
    if (batch > 0 && M > 0 && N > 0) {
        if (!xq || !wq || !y) return SQ_ERR_NULL_ARG;
        if (y_dt != SQ_I32 && (!x_scale || !w_scale)) return SQ_ERR_NULL_ARG;
    }
    if (xq_stride % 16 != 0 || wq_stride % 16 != 0) return SQ_ERR_ALIGNMENT;
    const void* ptrs[] = {xq, x_scale, wq, w_scale, y};
    for (const void* p : ptrs)
        if (!aligned16(p)) return SQ_ERR_ALIGNMENT;
    if (batch == 0) return SQ_OK;
    sq::Batch b;
    b.count = batch;
    b.a = xq_stride;
    b.b = wq_stride;
    b.sx = xs_stride;
    b.sw = ws_stride;
    b.y = y_stride;
    const int out = (y_dt == SQ_F32) ? 0 : (y_dt == SQ_BF16) ? 1 : 2;
    return from_hip(sq::launch_gemm(xq, x_scale, x_mode == SQ_PER_TOKEN, wq, w_scale,
                                    w_mode == SQ_W_PER_TENSOR, M, N, K, y, out, sq::Epi{}, b,
                                    reinterpret_cast<hipStream_t>(stream)));
}

sq_status sq_gemm_w8a8(const int8_t* xq, const float* x_scale, sq_act_mode x_mode,
                       const int8_t* wq, const float* w_scale, sq_weight_mode w_mode, int64_t M,
                       int64_t N, int64_t K, void* y, sq_dtype y_dt, sq_stream_t stream) {
    if (y_dt == SQ_I8) return SQ_ERR_BAD_DTYPE;  // int8 output needs the fused epilogue
    return sq_gemm_w8a8_ex(xq, x_scale, x_mode, wq, w_scale, w_mode, M, N, K, nullptr, y, y_dt,
                           stream);
}

size_t sq_channel_quantile_workspace_size(int64_t K) {
    return valid_k(K) ? sq::quantile_workspace_bytes(K) : 0;
}

sq_status sq_channel_quantile(const void* x, sq_dtype x_dt, int64_t T, int64_t K, float q,
                              float* out, void* workspace, size_t workspace_bytes,
                              sq_stream_t stream) {
    if (!valid_k(K) || !valid_rows(T)) return SQ_ERR_BAD_SHAPE;
    if (!float_dtype(x_dt)) return SQ_ERR_BAD_DTYPE;
    if (!(q > 0.0f && q <= 1.0f)) return SQ_ERR_BAD_MODE;
    if (!out || !workspace || (T > 0 && !x)) return SQ_ERR_NULL_ARG;
    if (!aligned16(x) || !aligned16(out) || !aligned16(workspace)) return SQ_ERR_ALIGNMENT;
    if (workspace_bytes < sq::quantile_workspace_bytes(K)) return SQ_ERR_WORKSPACE;
    const int64_t r = std::max<int64_t>(
        1, std::min<int64_t>(T, static_cast<int64_t>(std::ceil(static_cast<double>(q) *
                                                               static_cast<double>(T)))));
    return from_hip(sq::launch_channel_quantile(x, to_dt(x_dt), T, K, r, out, workspace,
                                                reinterpret_cast<hipStream_t>(stream)));
}

sq_status sq_channel_quantile_noalloc(const void* x, sq_dtype x_dt, int64_t T, int64_t K,
                                      float q, float* out, sq_stream_t stream) {
    if (!valid_k(K) || !valid_rows(T) || K > SQ_NOALLOC_MAX_K) return SQ_ERR_BAD_SHAPE;
    if (!float_dtype(x_dt)) return SQ_ERR_BAD_DTYPE;
    if (!(q > 0.0f && q <= 1.0f)) return SQ_ERR_BAD_MODE;
    if (!out || (T > 0 && !x)) return SQ_ERR_NULL_ARG;
    if (!aligned16(x) || !aligned16(out)) return SQ_ERR_ALIGNMENT;
    const int64_t r = std::max<int64_t>(
        1, std::min<int64_t>(T, static_cast<int64_t>(std::ceil(static_cast<double>(q) *
                                                               static_cast<double>(T)))));
    return from_hip(sq::launch_channel_quantile_noalloc(x, to_dt(x_dt), T, K, r, out,
                                                        reinterpret_cast<hipStream_t>(stream)));
}

sq_status sq_clip_count(const void* x, sq_dtype x_dt, int64_t M, int64_t K, const float* s,
                        const float* ln_gamma_s, const float* ln_beta_s, float ln_eps,
                        const float* static_scale, unsigned long long* count,
                        uint32_t* per_channel, sq_stream_t stream) {
    if (!valid_k(K) || !valid_rows(M)) return SQ_ERR_BAD_SHAPE;
    if (!float_dtype(x_dt)) return SQ_ERR_BAD_DTYPE;
    const bool ln = (ln_gamma_s != nullptr) || (ln_beta_s != nullptr);
    if (ln) {
        if (s) return SQ_ERR_BAD_MODE;
        if (!ln_gamma_s || !ln_beta_s) return SQ_ERR_NULL_ARG;
        if (!(ln_eps > 0.0f) || !std::isfinite(ln_eps)) return SQ_ERR_BAD_MODE;
    } else if (!s) {
        return SQ_ERR_NULL_ARG;
    }
    if (!static_scale || !count || (M > 0 && !x)) return SQ_ERR_NULL_ARG;
    const void* ptrs[] = {x, s, ln_gamma_s, ln_beta_s, static_scale, count, per_channel};
    for (const void* p : ptrs)
        if (!aligned16(p)) return SQ_ERR_ALIGNMENT;
    return from_hip(sq::launch_clip_count(x, to_dt(x_dt), M, K, ln ? nullptr : s, ln_gamma_s,
                                          ln_beta_s, ln_eps, static_scale, count, per_channel,
                                          reinterpret_cast<hipStream_t>(stream)));
}

size_t sq_alpha_search_workspace_size(int64_t T, int64_t N, int64_t K) {
    if (!valid_k(K) || !valid_rows(T) || !valid_rows(N)) return 0;
    return sq::alpha_workspace_bytes(T, N, K);
}

sq_status sq_alpha_search(const void* x_cal, sq_dtype x_dt, int64_t T, const void* w,
                          sq_dtype w_dt, int64_t N, int64_t K, const float* alphas, int n_alpha,
                          sq_act_mode x_mode, sq_weight_mode w_mode, double* err, double* werr,
                          int32_t* best, void* workspace, size_t workspace_bytes,
                          sq_stream_t stream) {
    if (!valid_k(K) || !valid_rows(T) || !valid_rows(N) || T < 1 || N < 1)
        return SQ_ERR_BAD_SHAPE;
    if (T * N > (int64_t(1) << 31)) return SQ_ERR_BAD_SHAPE;
    if (!float_dtype(x_dt) || !float_dtype(w_dt)) return SQ_ERR_BAD_DTYPE;
    if (x_mode != SQ_PER_TOKEN && x_mode != SQ_STATIC_PER_TENSOR &&
        x_mode != SQ_DYNAMIC_PER_TENSOR)
        return SQ_ERR_BAD_MODE;
    if (w_mode != SQ_W_PER_CHANNEL && w_mode != SQ_W_PER_TENSOR) return SQ_ERR_BAD_MODE;
    if (n_alpha < 1 || n_alpha > 1024) return SQ_ERR_BAD_SHAPE;
    if (!x_cal || !w || !alphas || !err || !werr || !best || !workspace) return SQ_ERR_NULL_ARG;
    for (int i = 0; i < n_alpha; ++i)
        if (!(alphas[i] >= 0.0f && alphas[i] <= 1.0f)) return SQ_ERR_BAD_ALPHA;
    const void* ptrs[] = {x_cal, w, err, werr, best, workspace};
    for (const void* p : ptrs)
        if (!aligned16(p)) return SQ_ERR_ALIGNMENT;
    if (workspace_bytes < sq::alpha_workspace_bytes(T, N, K)) return SQ_ERR_WORKSPACE;
    const sq::ActMode am = x_mode == SQ_PER_TOKEN           ? sq::ActMode::PerToken
                           : x_mode == SQ_STATIC_PER_TENSOR ? sq::ActMode::Static
                                                            : sq::ActMode::DynamicTensor;
    return from_hip(sq::launch_alpha_search(x_cal, to_dt(x_dt), T, w, to_dt(w_dt), N, K, alphas,
                                            n_alpha, am, w_mode == SQ_W_PER_TENSOR, err, werr,
                                            best, workspace,
                                            reinterpret_cast<hipStream_t>(stream)));
}

const char* sq_status_string(sq_status status) {
    switch (status) {
        case SQ_OK: return "SQ_OK";
        case SQ_ERR_NULL_ARG: return "SQ_ERR_NULL_ARG: a required pointer is NULL";
        case SQ_ERR_BAD_SHAPE: return "SQ_ERR_BAD_SHAPE: invalid size (K must be a positive multiple of 64 up to SQ_MAX_K; sizes non-negative)";
        case SQ_ERR_BAD_DTYPE: return "SQ_ERR_BAD_DTYPE: dtype not allowed for this operand";
        case SQ_ERR_BAD_ALPHA: return "SQ_ERR_BAD_ALPHA: alpha must lie in [0, 1]";
        case SQ_ERR_ALIGNMENT: return "SQ_ERR_ALIGNMENT: pointers must be 16-byte aligned";
        case SQ_ERR_HIP: return "SQ_ERR_HIP: the HIP runtime rejected a kernel launch";
        case SQ_ERR_BAD_MODE: return "SQ_ERR_BAD_MODE: invalid mode or mode/argument combination";
        case SQ_ERR_WORKSPACE: return "SQ_ERR_WORKSPACE: workspace smaller than its size query";
    }
    return "SQ_ERR_UNKNOWN";
}

int sq_abi_version(void) { return SQ_ABI_VERSION; }

}  // extern "C"
