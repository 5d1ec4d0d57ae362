/*
 * oracle.h -- plain CPU oracle for the SmoothQuant W8A8 linear-layer path.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the checker the GPU path is
 * compared against; it is used by the tests, by the smoke check and by the
 * benchmark's CPU-baseline leg, never by the product path.  It shares no code,
 * header, constant or helper with the HIP library.
 *
 * Every routine is a direct transcription of a definition from the pages:
 *   [Teach]  "SmoothQuant 如何解决激活量化难题？为什么适合 W8A8？" (teaching page)
 *   [Review] "SmoothQuant：大型语言模型的精准高效训练后量化 — 深度技术评审"
 *            (technical review of the ICML 2023 paper)
 *   [Edge]   "嵌入式 SLM 动态权重量化：SmoothQuant 激活异常值迁移与 INT8 部署实战"
 *            (edge deployment article with a C reference of calibrate/fuse/GEMM)
 * Where the pages leave a step open, the reading taken is stated at the
 * routine.  Floating point: every fp32 operation is a single IEEE binary32
 * operation rounded to nearest-even, in the order written (the file is
 * compiled with -ffp-contract=off -fno-fast-math, no FMA).
 *
 * dtype codes for raw inputs: ORC_F32 = fp32, ORC_BF16 = bfloat16 bit
 * patterns stored as uint16 (upcast to fp32 exactly by a 16-bit shift).
 */
#ifndef SQ_ORACLE_H
#define SQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };

/* Floor on every absolute maximum (the edge article seeds its running
 * maxima with 1e-7; applied here to every max so no scale is zero). */
#define ORC_FLOOR 1e-7f
#define ORC_QMAX 127.0f

/* a[k] = max(FLOOR, max_r |x[r,k]|) over a row-major [rows, K] tensor. */
void orc_colmax(const void* x, int dt, int64_t rows, int64_t K, float* out);

/* Eq. (4): s_j = max|X_j|^alpha / max|W_j|^(1-alpha), fp64 then one rounding. */
void orc_smooth_factor(const float* a, const float* w, int64_t K, float alpha, float* s);

/* Quad-precision audit of orc_smooth_factor: counts channels whose exact
 * quotient lies within 2^-40 (relative) of an fp32 rounding boundary, and
 * channels where the fp64 route and the quad route round differently. */
void orc_smooth_factor_audit(const float* a, const float* w, int64_t K, float alpha,
                             int64_t* n_near_tie, int64_t* n_mismatch);

/* Weight smoothing + per-output-channel symmetric int8:
 * What[n,k] = RN(W[n,k]*s[k]); d_n = RN(max(FLOOR, max_k|What|)/127);
 * wq = clamp(rne(RN(What/d_n))).  W is [N,K] row-major (out x in).
 * rows: optional list of n_rows row indices (NULL = all N rows, n_rows = N);
 * outputs are packed [n_rows, K] and [n_rows]. */
void orc_weight_quant(const void* w, int dt, int64_t N, int64_t K, const float* s,
                      const int64_t* rows, int64_t n_rows, int8_t* wq, float* w_scale);

/* Variant quantizing with one scale per INPUT column (the axis the edge
 * article's listing takes its maxima over).  Exists only so a test can show
 * that reading is rejected: its scale cannot be factored out of the GEMM. */
void orc_weight_quant_per_input(const void* w, int dt, int64_t N, int64_t K, const float* s,
                                int8_t* wq, float* col_scale);

/* LayerNorm fold: g_s = RN(gamma/s), b_s = RN(beta/s). */
void orc_ln_fold(const float* gamma, const float* beta, const float* s, int64_t K,
                 float* g_s, float* b_s);

/* Static activation scale from calibration: RN(max(FLOOR, max_k RN(a_k/s_k))/127). */
float orc_static_scale(const float* a, const float* s, int64_t K);

/* Plain smoothing X*diag(s)^-1: xhat = RN(x/s_k).  rows as in orc_weight_quant. */
void orc_act_smooth(const void* x, int dt, int64_t M, int64_t K, const float* s,
                    const int64_t* rows, int64_t n_rows, float* xhat);

/* LayerNorm with the smoothing folded into gamma/beta (canonical fp32
 * reduction order, biased two-pass variance, eps). */
void orc_act_ln(const void* x, int dt, int64_t M, int64_t K, const float* g_s,
                const float* b_s, float eps, const int64_t* rows, int64_t n_rows, float* xhat);

/* The canonical fp32 sum used by the LayerNorm (256 strided partials of
 * 8-element chunks, then a fixed halving tree). */
float orc_canonical_sum(const float* v, int64_t K);

/* Per-token dynamic int8: d_t = RN(max(FLOOR, max_k|xhat|)/127). */
void orc_quant_per_token(const float* xhat, int64_t M, int64_t K, int8_t* q, float* scale);

/* Per-tensor weight step (SmoothQuant-O1..O3): one dw for the whole smoothed
 * weight; returns dw and writes the codes [N, K]. */
float orc_weight_quant_per_tensor(const void* w, int dt, int64_t N, int64_t K, const float* s,
                                  int8_t* wq);

/* Dynamic per-tensor activation step (SmoothQuant-O2): one step for every
 * token of the batch; returns it and writes the codes [M, K]. */
float orc_quant_dynamic_per_tensor(const float* xhat, int64_t M, int64_t K, int8_t* q);

/* Static per-tensor int8 with a given scale; returns the number of codes
 * that saturated (|RN(xhat/d)| rounded beyond 127). */
int64_t orc_quant_static(const float* xhat, int64_t M, int64_t K, float scale, int8_t* q);

/* Exact integer GEMM acc[m,n] = sum_k xq[m,k]*wq[n,k] (int64 accumulate).
 * Returns 0, or -1 if some result does not fit int32. */
int orc_gemm_i32(const int8_t* xq, const int8_t* wq, int64_t M, int64_t N, int64_t K,
                 int32_t* acc);

/* Dequant: y = RN((float)acc * RN(dx_t * dw_n)); x_per_token=0 reads dx[0],
 * w_per_tensor=1 reads dw[0]. */
void orc_dequant(const int32_t* acc, const float* x_scale, int x_per_token,
                 const float* w_scale, int w_per_tensor, int64_t M, int64_t N, float* y);

/* Epilogue after dequantization: optional bias (one RN addition), optional
 * ReLU (y > 0 ? y : +0). */
void orc_epilogue(const float* y, int64_t M, int64_t N, const float* bias, int relu, float* out);

/* int8 codes for the next linear: clamp(rne(RN(RN(y / s'_n) / D))), s' = 1 when
 * next_s is NULL; returns the saturation count. */
int64_t orc_requant(const float* y, int64_t M, int64_t N, const float* next_s, float D,
                    int8_t* q);

/* fp32 -> bf16 bit pattern, round to nearest even. */
void orc_f32_to_bf16(const float* y, int64_t n, uint16_t* out);

/* fp64 LayerNorm reference (textbook, for the tolerance check of the
 * canonical fp32 LayerNorm): out = (x-mean)/sqrt(var+eps)*g + b in fp64. */
void orc_ln_f64(const void* x, int dt, int64_t M, int64_t K, const double* g, const double* b,
                double eps, double* out);

/* Number of OpenMP threads the oracle runs with. */
int orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
