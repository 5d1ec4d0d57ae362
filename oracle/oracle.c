/*
 * oracle.c -- plain, slow, obviously correct CPU definition of the SmoothQuant
 * W8A8 linear-layer path.  TEST INFRASTRUCTURE ONLY (see oracle.h): only the
 * tests, the smoke check and the benchmark's CPU-baseline leg may load it.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp (x86-64
 * SSE arithmetic, default rounding mode = round to nearest even).  OpenMP
 * only splits independent rows/columns; it never changes an operation order.
 *
 * Page short names used in the citations below:
 *   [Teach]  "SmoothQuant 如何解决激活量化难题？为什么适合 W8A8？"
 *   [Review] "SmoothQuant：大型语言模型的精准高效训练后量化 — 深度技术评审"
 *   [Edge]   "嵌入式 SLM 动态权重量化：SmoothQuant 激活异常值迁移与 INT8 部署实战"
 */
#include "oracle.h"

#include <math.h>
#include <omp.h>
#include <quadmath.h>
#include <stdlib.h>
#include <string.h>

/* ---- raw element access ------------------------------------------------ */

/* bf16 is the top half of an fp32 bit pattern, so the upcast is exact. */
static float load_elem(const void* base, int dt, int64_t idx) {
    if (dt == ORC_BF16) {
        uint32_t u = (uint32_t)((const uint16_t*)base)[idx] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return f;
    }
    return ((const float*)base)[idx];
}

/* Round half to even, then saturate to the symmetric int8 range [-127, 127].
 * [Review] §2.2: the quantizer divides by the step and rounds to the nearest
 * integer; the step is max|X|/(2^(N-1)-1), so the code range is symmetric.
 * Reading: ties go to even (the page does not fix the tie rule), and the
 * clamp is +-127 (the edge listing's -128 lower bound would break symmetry). */
static int8_t quantize_code(float q) {
    float r = rintf(q); /* default rounding mode: nearest, ties to even */
    if (r > ORC_QMAX) r = ORC_QMAX;
    if (r < -ORC_QMAX) r = -ORC_QMAX;
    return (int8_t)r;
}

/* Step of the symmetric quantizer from an absolute maximum:
 * d = RN(max(FLOOR, m) / 127).  [Review] §2.2 (Delta = max|X| / (2^(N-1)-1)). */
static float step_from_absmax(float m) {
    if (m < ORC_FLOOR) m = ORC_FLOOR;
    return m / ORC_QMAX;
}

int orc_num_threads(void) { return omp_get_max_threads(); }

/* Threads of the OpenMP loops (the benchmark also times one thread). */
void orc_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* ---- calibration -------------------------------------------------------- */

/* [Teach] §四 and [Edge] §三: calibration records the absolute peak of every
 * input channel; [Review] §5.3 eq. (4) consumes max|X_j| and max|W_j|.
 * Column k of a row-major [rows, K] tensor is input channel k (for W stored
 * [out][in] as in the edge listing, column k is input channel k too). */
void orc_colmax(const void* x, int dt, int64_t rows, int64_t K, float* out) {
    /* columns are split into blocks across threads; each block is swept row
     * by row so the reads follow the row-major layout */
    const int64_t BLK = 256;
#pragma omp parallel for schedule(static)
    for (int64_t k0 = 0; k0 < K; k0 += BLK) {
        int64_t k1 = (k0 + BLK < K) ? k0 + BLK : K;
        for (int64_t k = k0; k < k1; ++k) out[k] = ORC_FLOOR;
        for (int64_t r = 0; r < rows; ++r) {
            for (int64_t k = k0; k < k1; ++k) {
                float v = fabsf(load_elem(x, dt, r * K + k));
                if (v > out[k]) out[k] = v;
            }
        }
    }
}

/* [Review] §5.3 eq. (4): s_j = max(|X_j|)^alpha / max(|W_j|)^(1-alpha).
 * Reading: evaluated in fp64 (pow, pow, divide) and rounded once to fp32;
 * no epsilon is added to the denominator (the floor on both maxima already
 * keeps it positive). */
void orc_smooth_factor(const float* a, const float* w, int64_t K, float alpha, float* s) {
    const double al = (double)alpha;
    const double be = 1.0 - al;
    for (int64_t j = 0; j < K; ++j) {
        double num = pow((double)a[j], al);
        double den = pow((double)w[j], be);
        s[j] = (float)(num / den);
    }
}

void orc_smooth_factor_audit(const float* a, const float* w, int64_t K, float alpha,
                             int64_t* n_near_tie, int64_t* n_mismatch) {
    const __float128 al = (__float128)alpha;
    const __float128 be = (__float128)1 - al;
    int64_t ties = 0, mism = 0;
    for (int64_t j = 0; j < K; ++j) {
        __float128 q = powq((__float128)a[j], al) / powq((__float128)w[j], be);
        float f = (float)q;
        float nb = (q > (__float128)f) ? nextafterf(f, INFINITY) : nextafterf(f, 0.0f);
        __float128 mid = ((__float128)f + (__float128)nb) / 2;
        __float128 dist = fabsq(q - mid);
        if (dist <= fabsq(q) * 0x1p-40Q) ++ties;
        double num = pow((double)a[j], (double)alpha);
        double den = pow((double)w[j], 1.0 - (double)alpha);
        if ((float)(num / den) != f) ++mism;
    }
    *n_near_tie = ties;
    *n_mismatch = mism;
}

/* [Review] §5.1 eq. (3) and §5.5: the weight side of the rewrite is
 * diag(s)W, i.e. input channel k of W is multiplied by s_k.  [Edge] §二/§三:
 * the smoothed weight is then quantized offline to int8 with a per-channel
 * scale max/127.  Reading: the scale is per OUTPUT channel n (one row of the
 * [out][in] storage), the only axis an int8 GEMM can dequantize after the
 * contraction ([Review] §2.6, Fig. 3). */
void orc_weight_quant(const void* w, int dt, int64_t N, int64_t K, const float* s,
                      const int64_t* rows, int64_t n_rows, int8_t* wq, float* w_scale) {
    if (rows == NULL) n_rows = N;
#pragma omp parallel
    {
        float* what = (float*)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < n_rows; ++i) {
            int64_t n = rows ? rows[i] : i;
            float m = 0.0f;
            for (int64_t k = 0; k < K; ++k) {
                what[k] = load_elem(w, dt, n * K + k) * s[k];
                float v = fabsf(what[k]);
                if (v > m) m = v;
            }
            float d = step_from_absmax(m);
            w_scale[i] = d;
            for (int64_t k = 0; k < K; ++k) wq[i * K + k] = quantize_code(what[k] / d);
        }
        free(what);
    }
}

/* [Review] §6.3: the SmoothQuant-O1/O2/O3 settings quantize the weight per
 * TENSOR -- one step for the whole smoothed weight:
 * dw = RN(max(FLOOR, max_{n,k} |What|) / 127), wq = clamp(rne(RN(What / dw))).
 * Two plain passes over W (the maximum, then the codes).  Returns dw. */
float orc_weight_quant_per_tensor(const void* w, int dt, int64_t N, int64_t K, const float* s,
                                  int8_t* wq) {
    float m = 0.0f;
#pragma omp parallel for schedule(static) reduction(max : m)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            float v = fabsf(load_elem(w, dt, n * K + k) * s[k]);
            if (v > m) m = v;
        }
    }
    const float d = step_from_absmax(m);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            wq[n * K + k] = quantize_code((load_elem(w, dt, n * K + k) * s[k]) / d);
    return d;
}

void orc_weight_quant_per_input(const void* w, int dt, int64_t N, int64_t K, const float* s,
                                int8_t* wq, float* col_scale) {
    for (int64_t k = 0; k < K; ++k) {
        float m = 0.0f;
        for (int64_t n = 0; n < N; ++n) {
            float v = fabsf(load_elem(w, dt, n * K + k) * s[k]);
            if (v > m) m = v;
        }
        col_scale[k] = step_from_absmax(m);
    }
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            wq[n * K + k] = quantize_code((load_elem(w, dt, n * K + k) * s[k]) / col_scale[k]);
}

/* [Edge] §二 (LayerNorm absorption): gamma_new = gamma/s, beta_new = beta/s;
 * [Review] §5.5: diag(s)^-1 is folded into the preceding LayerNorm. */
void orc_ln_fold(const float* gamma, const float* beta, const float* s, int64_t K,
                 float* g_s, float* b_s) {
    for (int64_t k = 0; k < K; ++k) {
        g_s[k] = gamma[k] / s[k];
        b_s[k] = beta[k] / s[k];
    }
}

/* [Review] §2.5 (static quantization: scale computed offline from
 * calibration and reused).  The smoothed calibration channel peak is
 * RN(a_k/s_k); since RN is monotone this equals the max over calibration
 * tokens of |RN(x/s_k)|, so one [K] pass gives the per-tensor static scale. */
float orc_static_scale(const float* a, const float* s, int64_t K) {
    float m = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        float v = a[k] / s[k];
        if (v > m) m = v;
    }
    return step_from_absmax(m);
}

/* ---- runtime activation side ------------------------------------------- */

/* [Review] §5.1 eq. (3): Xhat = X diag(s)^-1, i.e. divide input channel k by
 * s_k; [Edge] §二 names this runtime op a division.  One fp32 division. */
void orc_act_smooth(const void* x, int dt, int64_t M, int64_t K, const float* s,
                    const int64_t* rows, int64_t n_rows, float* xhat) {
    if (rows == NULL) n_rows = M;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t m = rows ? rows[i] : i;
        for (int64_t k = 0; k < K; ++k) xhat[i * K + k] = load_elem(x, dt, m * K + k) / s[k];
    }
}

/* Canonical fp32 sum (reading: the pages fix no reduction order).
 * 256 partials; element k belongs to partial floor(k/8) mod 256 and each
 * partial adds its elements in increasing k starting from +0.0f; then the
 * partials are combined by a halving tree p[i] = p[i] + p[i+d] for
 * d = 128, 64, ..., 1 and i < d. */
float orc_canonical_sum(const float* v, int64_t K) {
    float p[256];
    for (int i = 0; i < 256; ++i) p[i] = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        int part = (int)((k / 8) % 256);
        p[part] = p[part] + v[k];
    }
    for (int d = 128; d >= 1; d /= 2)
        for (int i = 0; i < d; ++i) p[i] = p[i] + p[i + d];
    return p[0];
}

/* [Edge] §二: the LayerNorm in front of the linear computes LN(x)*gamma+beta
 * and, after the fold, emits the smoothed Xhat directly.  Reading of the
 * unstated details: mean mu = RN(S1/K); d_k = RN(x_k - mu); biased variance
 * RN(S2/K) with S2 the canonical sum of RN(d_k*d_k); rho =
 * RN(1/RN(sqrt(RN(var + eps)))); Xhat_k = RN(RN(RN(d_k*rho)*g_k) + b_k). */
void orc_act_ln(const void* x, int dt, int64_t M, int64_t K, const float* g_s,
                const float* b_s, float eps, const int64_t* rows, int64_t n_rows, float* xhat) {
    if (rows == NULL) n_rows = M;
    const float kf = (float)K;
#pragma omp parallel
    {
        float* v = (float*)malloc((size_t)K * sizeof(float));
        float* dd = (float*)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < n_rows; ++i) {
            int64_t m = rows ? rows[i] : i;
            for (int64_t k = 0; k < K; ++k) v[k] = load_elem(x, dt, m * K + k);
            float mu = orc_canonical_sum(v, K) / kf;
            for (int64_t k = 0; k < K; ++k) {
                v[k] = v[k] - mu;     /* d_k */
                dd[k] = v[k] * v[k];
            }
            float var = orc_canonical_sum(dd, K) / kf;
            float rho = 1.0f / sqrtf(var + eps);
            for (int64_t k = 0; k < K; ++k) {
                float t = v[k] * rho;
                t = t * g_s[k];
                xhat[i * K + k] = t + b_s[k];
            }
        }
        free(v);
        free(dd);
    }
}

/* [Review] §2.5 (dynamic: scale from the current activation) and §2.6 Fig. 3
 * (per-token granularity: one scale per row, an outer GEMM dimension). */
void orc_quant_per_token(const float* xhat, int64_t M, int64_t K, int8_t* q, float* scale) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float mx = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = fabsf(xhat[m * K + k]);
            if (v > mx) mx = v;
        }
        float d = step_from_absmax(mx);
        scale[m] = d;
        for (int64_t k = 0; k < K; ++k) q[m * K + k] = quantize_code(xhat[m * K + k] / d);
    }
}

/* [Review] §6.3: SmoothQuant-O2 (and the naive W8A8 baseline of the same
 * section) quantizes the activation with one DYNAMIC per-tensor step, taken
 * over every token of the batch: d = RN(max(FLOOR, max_{t,k} |xhat|) / 127),
 * q = clamp(rne(RN(xhat / d))).  Returns d. */
float orc_quant_dynamic_per_tensor(const float* xhat, int64_t M, int64_t K, int8_t* q) {
    float mx = 0.0f;
#pragma omp parallel for schedule(static) reduction(max : mx)
    for (int64_t i = 0; i < M * K; ++i) {
        float v = fabsf(xhat[i]);
        if (v > mx) mx = v;
    }
    const float d = step_from_absmax(mx);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M * K; ++i) q[i] = quantize_code(xhat[i] / d);
    return d;
}

/* [Review] §2.5 (static) with one per-tensor scale; codes beyond the range
 * saturate at +-127 ([Edge] §三 clips to int8). */
int64_t orc_quant_static(const float* xhat, int64_t M, int64_t K, float scale, int8_t* q) {
    int64_t sat = 0;
#pragma omp parallel for schedule(static) reduction(+ : sat)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k) {
            float qq = xhat[m * K + k] / scale;
            if (fabsf(rintf(qq)) > ORC_QMAX) ++sat;
            q[m * K + k] = quantize_code(qq);
        }
    }
    return sat;
}

/* ---- integer GEMM and dequant ------------------------------------------ */

/* [Edge] §三 (int8 GEMM listing): int32 accumulator of a[i,k]*w[j,k] with the
 * weight stored [out][in]; [Review] §5.6: the linear runs as an INT8 GEMM.
 * Accumulated in int64 and checked to fit int32. */
int orc_gemm_i32(const int8_t* xq, const int8_t* wq, int64_t M, int64_t N, int64_t K,
                 int32_t* acc) {
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t t = 0;
            for (int64_t k = 0; k < K; ++k) t += (int64_t)xq[m * K + k] * (int64_t)wq[n * K + k];
            if (t > INT32_MAX || t < INT32_MIN) bad = 1;
            acc[m * N + n] = (int32_t)t;
        }
    }
    return bad ? -1 : 0;
}

/* [Edge] §三: the output is (float)acc times the product of the activation
 * scale and the weight scale of output channel n, in that order. */
void orc_dequant(const int32_t* acc, const float* x_scale, int x_per_token,
                 const float* w_scale, int w_per_tensor, int64_t M, int64_t N, float* y) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float dx = x_per_token ? x_scale[m] : x_scale[0];
        for (int64_t n = 0; n < N; ++n) {
            float f = dx * (w_per_tensor ? w_scale[0] : w_scale[n]);
            y[m * N + n] = (float)acc[m * N + n] * f;
        }
    }
}

/* Fused epilogue after the dequantization ([Edge] §二: no separate runtime
 * operator between this GEMM and the next int8 GEMM; [Teach] §七: fused
 * quantize / dequantize nodes).  Reading (the pages give no formula): the
 * bias is one more RN addition, ReLU keeps positive values and maps the rest
 * to +0:  y1 = bias ? RN(y + b_n) : y;  out = relu ? (y1 > 0 ? y1 : +0) : y1. */
void orc_epilogue(const float* y, int64_t M, int64_t N, const float* bias, int relu, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            float v = y[m * N + n];
            if (bias) v = v + bias[n];
            if (relu) v = (v > 0.0f) ? v : 0.0f;
            out[m * N + n] = v;
        }
    }
}

/* Requantize the layer output for the next linear: its smoothing X/s' (the
 * next layer's input channels are this layer's output channels, [Review]
 * §5.1 eq. (3)) and its static per-tensor step D ([Review] §2.5):
 * q = clamp(rne(RN(RN(y / s'_n) / D))); next_s NULL means s' = 1.  Returns
 * the number of codes that saturated. */
int64_t orc_requant(const float* y, int64_t M, int64_t N, const float* next_s, float D,
                    int8_t* q) {
    int64_t sat = 0;
#pragma omp parallel for schedule(static) reduction(+ : sat)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            float xh = next_s ? y[m * N + n] / next_s[n] : y[m * N + n];
            float qq = xh / D;
            if (fabsf(rintf(qq)) > ORC_QMAX) ++sat;
            q[m * N + n] = quantize_code(qq);
        }
    }
    return sat;
}

/* bf16 = the fp32 value rounded to 8 significand bits, ties to even
 * (inputs are finite). */
void orc_f32_to_bf16(const float* y, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &y[i], sizeof u);
        uint32_t lsb = (u >> 16) & 1u;
        out[i] = (uint16_t)((u + 0x7FFFu + lsb) >> 16);
    }
}

/* ---- fp64 references ---------------------------------------------------- */

/* The LayerNorm in front of a linear, LN(x) * gamma + beta ([Edge] §二), in
 * fp64 with the biased variance: the exact-arithmetic reference of the
 * LayerNorm workload's int8-vs-fp64 output error.  Not on the int8 path (that
 * is orc_act_ln, fp32 with the fused kernel's order). */
void orc_ln_f64(const void* x, int dt, int64_t M, int64_t K, const double* g, const double* b,
                double eps, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double s1 = 0.0;
        for (int64_t k = 0; k < K; ++k) s1 += (double)load_elem(x, dt, m * K + k);
        double mu = s1 / (double)K;
        double s2 = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double d = (double)load_elem(x, dt, m * K + k) - mu;
            s2 += d * d;
        }
        double inv = 1.0 / sqrt(s2 / (double)K + eps);
        for (int64_t k = 0; k < K; ++k)
            out[m * K + k] = ((double)load_elem(x, dt, m * K + k) - mu) * inv * g[k] + b[k];
    }
}
