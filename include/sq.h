/*
 * sq.h -- C ABI of the SmoothQuant W8A8 linear-layer library for MI355X
 * (gfx950).  libsq.so implements every call with hand-written HIP kernels.
 *
 * The calls follow the smoothing rewrite of a linear layer,
 *     Y = X W = (X diag(s)^-1) (diag(s) W)
 * ([Review] "SmoothQuant：大型语言模型的精准高效训练后量化 — 深度技术评审",
 * §5.1 eq. (3)), split into the offline half (calibrate, smooth and quantize
 * the weights; [Teach] "SmoothQuant 如何解决激活量化难题？为什么适合 W8A8？",
 * §四) and the runtime half (smooth + quantize the activation, then the int8
 * GEMM with a dequantizing epilogue; [Edge] "嵌入式 SLM 动态权重量化：
 * SmoothQuant 激活异常值迁移与 INT8 部署实战", §二 runtime graph).
 *
 * Conventions shared by every call
 *   - Layouts are row-major.  X is [tokens, K]; W is stored [N, K] (output
 *     channel x input channel, as in the edge article's GEMM listing), so the
 *     layer computes Y[m, n] = sum_k X[m, k] W[n, k].
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library allocates nothing and keeps no state between calls; calls are
 *     re-entrant.  Inputs are never written.
 *   - Every call validates its arguments on the host first and returns a
 *     status without touching the device when they are invalid.  Otherwise it
 *     enqueues its kernels on `stream` (0 = the null stream) and returns
 *     without waiting; a fault inside a kernel surfaces at the caller's next
 *     synchronisation.  SQ_ERR_HIP means a launch was rejected.
 *   - Pointers must be 16-byte aligned; K must be a multiple of 64 and at most
 *     SQ_MAX_K (so that 127*127*K fits in int32); other sizes may be 0 (the
 *     call then does nothing or writes only the size-K outputs).
 *   - Inputs are assumed finite; results for NaN/Inf inputs, or for inputs
 *     whose smoothed values overflow fp32, are unspecified.
 *
 * Numerical contract (RN = one IEEE binary32 operation, round to nearest
 * even; rne = round to nearest integer, ties to even; clamp = to [-127, 127];
 * FLOOR = SQ_ABSMAX_FLOOR).  Every listed value is produced bit for bit:
 *   a_j  = max(FLOOR, max_t |x_cal[t, j]|)          w_j = max(FLOOR, max_n |W[n, j]|)
 *   s_j  = RN32( pow64(a_j, alpha) / pow64(w_j, 1 - alpha) )   (fp64, one rounding)
 *   What = RN(W[n,k] * s_k);  dw_n = RN(max(FLOOR, max_k |What|) / 127)
 *   wq   = clamp(rne(RN(What / dw_n)))
 *   g'_k = RN(gamma_k / s_k), b'_k = RN(beta_k / s_k)
 *   dx_static = RN(max(FLOOR, max_k RN(a_k / s_k)) / 127)
 *   plain mode:  xh_k = RN(x_k / s_k)
 *   LN mode:     mu = RN(S(x)/K); d_k = RN(x_k - mu); var = RN(S(RN(d*d))/K);
 *                rho = RN(1 / RN(sqrt(RN(var + eps))));
 *                xh_k = RN(RN(RN(d_k * rho) * g'_k) + b'_k)
 *                where S(v) is the canonical sum: 256 fp32 partials, element k
 *                added to partial floor(k/8) mod 256 in increasing k from +0,
 *                then p[i] = RN(p[i] + p[i+d]) for d = 128, 64, ..., 1.
 *   per-token:   dx_t = RN(max(FLOOR, max_k |xh_k|) / 127);  static: dx_t = dx_static
 *   dynamic per-tensor: dx_t = dx = RN(max(FLOOR, max_{t,k} |xh|) / 127) over the batch
 *   per-tensor weight:  dw_n = dw = RN(max(FLOOR, max_{n,k} |What|) / 127)
 *   xq   = clamp(rne(RN(xh_k / dx_t)))
 *   acc  = sum_k xq[t,k] * wq[n,k]   (exact int32)
 *   y    = RN(RN_f32(acc) * RN(dx_t * dw_n));  bf16 output = y rounded to
 *          bf16 (nearest even).
 *   fused epilogue (sq_gemm_w8a8_ex):  y1 = bias ? RN(y + b_n) : y;
 *          y2 = relu ? (y1 > 0 ? y1 : +0) : y1;  fp32 / bf16 output = y2;
 *          int8 output = clamp(rne(RN(RN(y2 / s'_n) / D))) with the next
 *          linear's smoothing factor s' (1 when absent) and static step D.
 */
#ifndef SQ_H
#define SQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* sq_stream_t; /* a hipStream_t */

#define SQ_ABI_VERSION 4
#define SQ_MAX_K 133120          /* largest multiple of 64 with 127*127*K < 2^31 */
#define SQ_ABSMAX_FLOOR 1e-7f    /* floor of every absolute maximum */
#define SQ_NOALLOC_MAX_K 16384   /* largest K of sq_channel_quantile_noalloc */

typedef enum {
    SQ_OK = 0,
    SQ_ERR_NULL_ARG = 1,  /* a required pointer is NULL */
    SQ_ERR_BAD_SHAPE = 2, /* negative size, K % 64 != 0, K > SQ_MAX_K, ... */
    SQ_ERR_BAD_DTYPE = 3, /* dtype not allowed for that operand */
    SQ_ERR_BAD_ALPHA = 4, /* alpha outside [0, 1] or not finite */
    SQ_ERR_ALIGNMENT = 5, /* pointer not 16-byte aligned */
    SQ_ERR_HIP = 6,       /* the HIP runtime rejected a launch */
    SQ_ERR_BAD_MODE = 7,  /* unknown mode, or a mode/argument combination */
    SQ_ERR_WORKSPACE = 8  /* workspace smaller than the size its query returns */
} sq_status;

typedef enum { SQ_F32 = 0, SQ_BF16 = 1, SQ_I8 = 2, SQ_I32 = 3 } sq_dtype;

/* Activation step granularity ([Review] §2.5-§2.6 dynamic / static, per token
 * / per tensor; §6.3 uses all three). */
typedef enum {
    SQ_PER_TOKEN = 0,          /* dynamic, one step per token */
    SQ_STATIC_PER_TENSOR = 1,  /* one step from calibration (dx_static) */
    SQ_DYNAMIC_PER_TENSOR = 2  /* dynamic, one step for the whole batch */
} sq_act_mode;

/* Weight step granularity.  SQ_W_PER_CHANNEL: one step per output channel
 * (the column-wise scale of Y = XW).  SQ_W_PER_TENSOR: one step for the whole
 * weight, as in the SmoothQuant-O1/O2/O3 settings of [Review] §6.3:
 *   O1 = SQ_W_PER_TENSOR + SQ_PER_TOKEN
 *   O2 = SQ_W_PER_TENSOR + SQ_DYNAMIC_PER_TENSOR
 *   O3 = SQ_W_PER_TENSOR + SQ_STATIC_PER_TENSOR */
typedef enum { SQ_W_PER_CHANNEL = 0, SQ_W_PER_TENSOR = 1 } sq_weight_mode;

/*
 * sq_calibrate -- the offline half.
 *   [Teach] §四 (collect calibration peaks, compute the smoothing scale,
 *   adjust the weights offline); [Review] §5.3 eq. (4) (s_j); [Edge] §二-§三
 *   (fold 1/s into the LayerNorm's gamma/beta, fold s into W, quantize W to
 *   int8 offline with one scale per channel -- here per OUTPUT channel).
 *
 *   x_cal [T, K]  calibration activations (dtype x_dt: F32 or BF16), T >= 0
 *   w     [N, K]  weight, output channel x input channel (F32 or BF16), N >= 0
 *   alpha         migration strength in [0, 1]
 *   w_mode        SQ_W_PER_CHANNEL or SQ_W_PER_TENSOR ([Review] §6.3)
 *   ln_gamma, ln_beta [K] fp32: the LayerNorm in front of the layer, or both
 *                 NULL when there is none
 * Outputs (device, caller-owned):
 *   s [K] fp32            smoothing factor
 *   wq [N, K] int8        smoothed, quantized weight
 *   w_scale               [N] fp32 dw_n per output channel (SQ_W_PER_CHANNEL), or
 *                         [1] fp32 dw (SQ_W_PER_TENSOR)
 *   act_scale_static [1]  dx_static (may be NULL)
 *   ln_gamma_s, ln_beta_s [K] fp32: folded LayerNorm (required iff ln_gamma)
 *   x_absmax, w_absmax [K] fp32: a_j and w_j (required; they also serve as the
 *                 library's working memory for the two column maxima)
 * Kernels: the column-absmax pass over X_cal and W, the factor pass, one
 * weight smooth+quantize pass; reads X_cal once and W twice.  The column-absmax
 * pass stages its per-block maxima in wq (written last, by the quantize pass)
 * when wq has room for them, else it folds them with atomics into x_absmax and
 * w_absmax; wq's contents are defined only once the call has completed on the
 * stream.  SQ_W_PER_TENSOR: the largest smoothed weight magnitude is
 * max_j RN(max_n |W[n,j]| * s_j) (rounding and multiplying by s_j > 0 are
 * monotone), taken from the column maxima in the factor pass and held in
 * w_scale[0] until a one-thread kernel replaces it with the step; W is still
 * read twice, and the quantize pass uses the single step.
 */
sq_status sq_calibrate(const void* x_cal, sq_dtype x_dt, int64_t T,
                       const void* w, sq_dtype w_dt, int64_t N, int64_t K, float alpha,
                       sq_weight_mode w_mode,
                       const float* ln_gamma, const float* ln_beta,
                       float* s, int8_t* wq, float* w_scale, float* act_scale_static,
                       float* ln_gamma_s, float* ln_beta_s,
                       float* x_absmax, float* w_absmax, sq_stream_t stream);

/*
 * sq_smooth_quantize_act -- runtime activation side.
 *   [Review] §5.1 eq. (3) (X diag(s)^-1); [Edge] §二 (LayerNorm with gamma/s,
 *   beta/s emits the smoothed activation, then int8 quantization); [Review]
 *   §2.5-§2.6 (dynamic per-token or static per-tensor scale).
 *
 *   x [M, K]  activation (F32 or BF16).  Plain mode: the input of the linear.
 *             LayerNorm mode: the input of the LayerNorm.
 *   s [K]     plain mode (then ln_gamma_s and ln_beta_s are NULL), or NULL
 *   ln_gamma_s, ln_beta_s [K]  LayerNorm mode (then s is NULL); ln_eps > 0
 *   mode      SQ_PER_TOKEN: x_scale [M] receives dx_t.
 *             SQ_STATIC_PER_TENSOR: static_scale [1] (device) holds dx_static;
 *             x_scale may be NULL and is not written.
 *             SQ_DYNAMIC_PER_TENSOR ([Review] §6.3 O2): x_scale [1] receives
 *             the batch step dx (also when M = 0: FLOOR / 127, so x_scale is
 *             required for every M); static_scale is not read.
 *   xq [M, K] int8 output codes.
 * Per-token and static: one kernel that reads X once and writes xq (and
 * x_scale) once.  Dynamic per-tensor: a maximum pass (row maxima, or block
 * maxima for plain rows of 2048 elements or more, staged in xq), a one-block
 * reduction into x_scale[0], then the static quantizer with that step -- X is
 * read twice.
 */
sq_status sq_smooth_quantize_act(const void* x, sq_dtype x_dt, int64_t M, int64_t K,
                                 const float* s, const float* ln_gamma_s,
                                 const float* ln_beta_s, float ln_eps,
                                 sq_act_mode mode, const float* static_scale,
                                 int8_t* xq, float* x_scale, sq_stream_t stream);

/*
 * sq_gemm_w8a8 -- int8 x int8 GEMM with int32 accumulation and the
 * dequantizing epilogue.  [Edge] §三 (GEMM listing: int32 accumulator of
 * activation code times weight code with W stored [out][in]; output =
 * (float)acc * (act_scale * weight_scale[n])); [Review] §2.6 / Fig. 3 (scales
 * only on the outer dimensions: token and output channel).
 *
 *   xq [M, K] int8, x_scale: [M] when x_mode = SQ_PER_TOKEN, [1] for either
 *      per-tensor mode
 *   wq [N, K] int8, w_scale: [N] when w_mode = SQ_W_PER_CHANNEL, [1] when
 *      SQ_W_PER_TENSOR
 *   y  [M, N] of y_dt: SQ_F32, SQ_BF16, or SQ_I32 (the raw accumulators,
 *      x_scale and w_scale then unused and may be NULL)
 * Runs on the gfx950 int8 matrix cores (MFMA), LDS-staged K tiles.
 */
sq_status sq_gemm_w8a8(const int8_t* xq, const float* x_scale, sq_act_mode x_mode,
                       const int8_t* wq, const float* w_scale, sq_weight_mode w_mode,
                       int64_t M, int64_t N, int64_t K,
                       void* y, sq_dtype y_dt, sq_stream_t stream);

/*
 * Fused epilogue of sq_gemm_w8a8_ex.  [Edge] §二 (no separate floating-point
 * operator between one int8 GEMM and the next: the smoothing of the next layer
 * is fused, the graph runs quantize -> int8 GEMM -> dequantized output);
 * [Teach] §七 (the speed-up relies on fused quantize / dequantize nodes).
 * Bias and ReLU are the linear's own epilogue (the pages give no formula; one
 * RN addition, and ReLU maps non-positive values to +0).
 */
typedef struct sq_epilogue {
    const float* bias;       /* [N] fp32 added after the dequantization, or NULL */
    const float* next_s;     /* SQ_I8 output only: [N] smoothing factor s' of the next
                                linear (whose input channels are these outputs), or
                                NULL for s' = 1 */
    const float* next_scale; /* SQ_I8 output only (required): [1] device, the next
                                linear's static per-tensor step D */
    int relu;                /* nonzero: ReLU after the bias */
} sq_epilogue;

/*
 * sq_gemm_w8a8_ex -- sq_gemm_w8a8 with a fused epilogue.
 *   epi  NULL: exactly sq_gemm_w8a8.
 *   y_dt SQ_F32 / SQ_BF16: y2 of the contract above.
 *        SQ_I8: int8 codes [M, N] for the next linear (static per-tensor
 *        input step), written instead of the fp32 / bf16 activation -- the
 *        next layer's sq_smooth_quantize_act is fused away.  Equals, bit for
 *        bit, sq_smooth_quantize_act(SQ_STATIC_PER_TENSOR, s = next_s) applied
 *        to the SQ_F32 output with the same epilogue.
 *        SQ_I32: raw accumulators; epi must then be NULL or empty.
 * Errors: SQ_ERR_BAD_MODE for next_s with a non-int8 output or an epilogue
 * with int32 output; SQ_ERR_NULL_ARG for int8 output without next_scale.
 */
sq_status sq_gemm_w8a8_ex(const int8_t* xq, const float* x_scale, sq_act_mode x_mode,
                          const int8_t* wq, const float* w_scale, sq_weight_mode w_mode,
                          int64_t M, int64_t N, int64_t K, const sq_epilogue* epi,
                          void* y, sq_dtype y_dt, sq_stream_t stream);

/*
 * sq_bmm_w8a8 -- a strided batch of int8 GEMMs: the batched matrix products
 * of attention.  [Review] §5.6 / Fig. 6 (the compute-heavy operations of the
 * Transformer block run in INT8: the linear layers and the batched matrix
 * multiplications of attention; softmax, LayerNorm and the activation stay in
 * floating point).  Entry z, with the contract of sq_gemm_w8a8:
 *     y[z] = dequant( xq[z] [M, K] . wq[z]^T, x_scale[z], w_scale[z] )
 *   scores  S = Q K^T: xq = codes of Q [S_q, d], wq = codes of K [S_k, d];
 *           K's per-token steps play the per-output-channel role (w_mode
 *           SQ_W_PER_CHANNEL) or one step per head (SQ_W_PER_TENSOR).
 *   output  O = P V: xq = codes of P [S_q, S_k], wq = codes of V^T [d, S_k]
 *           (one row per channel of V).
 * Operand codes and steps come from sq_smooth_quantize_act with s = 1.
 *   batch     number of entries (0 <= batch <= 65535)
 *   *_stride  elements between consecutive entries; 0 repeats one tensor for
 *             every entry.  xq_stride, wq_stride: multiples of 16 (always true
 *             for contiguous operands, since K % 64 == 0).  y_stride and the
 *             scale strides are free (an output entry that does not start on a
 *             16-byte boundary is written element by element).
 *   y_dt      SQ_F32, SQ_BF16 or SQ_I32.  Entries of y must not overlap.
 */
sq_status sq_bmm_w8a8(const int8_t* xq, int64_t xq_stride, const float* x_scale,
                      int64_t xs_stride, sq_act_mode x_mode, const int8_t* wq,
                      int64_t wq_stride, const float* w_scale, int64_t ws_stride,
                      sq_weight_mode w_mode, int64_t batch, int64_t M, int64_t N, int64_t K,
                      void* y, int64_t y_stride, sq_dtype y_dt, sq_stream_t stream);

/*
 * Robust calibration ([Teach] §四: the calibration may record a robust
 * per-channel statistic instead of the peak, and alpha is searched together
 * with the weight range; §六: check the clip rate per layer and the stability
 * of channel peaks so that no single sample dominates; §八: compare candidate
 * alphas on activation saturation, weight quantization error and a task set).
 *
 * sq_channel_quantile -- for every channel j of x [T, K] (F32 or BF16) the
 *   nearest-rank q-quantile of |x[:, j]|: the r-th smallest magnitude with
 *   r = max(1, min(T, ceil(q * T))) computed in fp64, floored at
 *   SQ_ABSMAX_FLOOR; q in (0, 1]; q = 1 is the peak of sq_calibrate.  T = 0
 *   gives the floor.  out [K] fp32 (device).  workspace: device memory of at
 *   least sq_channel_quantile_workspace_size(K) bytes, 16-byte aligned,
 *   overwritten.  A radix select: ceil(bits / 8) passes over x (bits = 15 for
 *   BF16, 31 for F32).  Channel-peak stability is the ratio of this call at
 *   q = 1 to a lower q (a large ratio: few tokens set the peak).
 */
size_t sq_channel_quantile_workspace_size(int64_t K);
sq_status sq_channel_quantile(const void* x, sq_dtype x_dt, int64_t T, int64_t K, float q,
                              float* out, void* workspace, size_t workspace_bytes,
                              sq_stream_t stream);

/*
 * sq_channel_quantile_noalloc -- sq_channel_quantile for callers that cannot
 *   allocate device memory (code under HIP graph capture, tight serving loops,
 *   harnesses that forbid hipMalloc): no workspace argument, and the call
 *   allocates nothing.  The histogram and rank words live in a scratch array
 *   the library holds on every device it runs on, from module load until the
 *   process ends: SQ_NOALLOC_MAX_K * 1032 + 256 bytes (about 16 MiB), so K
 *   must not exceed SQ_NOALLOC_MAX_K (else SQ_ERR_BAD_SHAPE).  Every other
 *   argument, the result and the errors are those of sq_channel_quantile.  The
 *   stream must belong to the current device.  All calls on one device share
 *   its array (each call clears what it uses, so earlier contents never
 *   matter): calls that overlap on one device -- on different streams, or
 *   from different host threads -- race and give undefined results.
 */
sq_status sq_channel_quantile_noalloc(const void* x, sq_dtype x_dt, int64_t T, int64_t K,
                                      float q, float* out, sq_stream_t stream);

/*
 * sq_calibrate_stat -- sq_calibrate with a given per-channel activation
 *   statistic act_stat [K] (device fp32, e.g. sq_channel_quantile) in place of
 *   the calibration peak: a_j = max(SQ_ABSMAX_FLOOR, act_stat_j) enters
 *   eq. (4) and the static step exactly as the peak does; a_out [K] receives
 *   a_j.  Every other argument and output as in sq_calibrate.  A statistic
 *   below the peak lowers the static step, which then saturates the tokens
 *   above it (see sq_clip_count).
 */
sq_status sq_calibrate_stat(const float* act_stat, const void* w, sq_dtype w_dt, int64_t N,
                            int64_t K, float alpha, sq_weight_mode w_mode,
                            const float* ln_gamma, const float* ln_beta, float* s, int8_t* wq,
                            float* w_scale, float* act_scale_static, float* ln_gamma_s,
                            float* ln_beta_s, float* a_out, float* w_absmax,
                            sq_stream_t stream);

/*
 * sq_clip_count -- the clip rate of the static quantizer on activations x
 *   [M, K] (plain mode with s, or LayerNorm mode with ln_gamma_s / ln_beta_s,
 *   as in sq_smooth_quantize_act) with the step static_scale [1] (device):
 *   an element saturates when its rounded quotient rne(RN(x^ / dx_static))
 *   lies outside [-127, 127].  count [1] (device) receives the number of
 *   saturated elements; per_channel [K] (device, or NULL) the number per input
 *   channel.  Both are overwritten; no codes are written.
 */
sq_status sq_clip_count(const void* x, sq_dtype x_dt, int64_t M, int64_t K, const float* s,
                        const float* ln_gamma_s, const float* ln_beta_s, float ln_eps,
                        const float* static_scale, unsigned long long* count,
                        uint32_t* per_channel, sq_stream_t stream);

/*
 * sq_alpha_search -- candidate smoothing strengths for one linear layer.
 *   x_cal [T, K] calibration activations (the layer's input), w [N, K], both
 *   F32 or BF16 (device); alphas [n_alpha] (HOST array, each in [0, 1],
 *   1 <= n_alpha <= 1024); x_mode / w_mode: the step granularities as
 *   deployed.  For alpha_i the layer is calibrated (sq_calibrate), the
 *   calibration tokens quantized (sq_smooth_quantize_act) and multiplied
 *   (sq_gemm_w8a8, fp32 output y_q); then (device fp64 outputs)
 *     err[i]  = sum (y_q - y)^2 / sum y^2,  y = X W^T computed in fp64
 *     werr[i] = sum (W^ - dw q)^2 / sum W^^2 over W^ = RN(W s) and its codes
 *   (a ratio with a zero denominator is its numerator; sums in a fixed order),
 *   and best [1] (device int32) the first index of the least err.  err stands
 *   in for the pages' task-set check; the saturation check is sq_clip_count
 *   on held-out tokens with each candidate's static step.  workspace: at least
 *   sq_alpha_search_workspace_size(T, N, K) bytes (about 12 T N + T K + N K),
 *   16-byte aligned, overwritten.  Calls on one stream must not share it.
 */
size_t sq_alpha_search_workspace_size(int64_t T, int64_t N, int64_t K);
sq_status sq_alpha_search(const void* x_cal, sq_dtype x_dt, int64_t T, const void* w,
                          sq_dtype w_dt, int64_t N, int64_t K, const float* alphas, int n_alpha,
                          sq_act_mode x_mode, sq_weight_mode w_mode, double* err, double* werr,
                          int32_t* best, void* workspace, size_t workspace_bytes,
                          sq_stream_t stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* sq_status_string(sq_status status);

/* SQ_ABI_VERSION of the loaded library. */
int sq_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SQ_H */
