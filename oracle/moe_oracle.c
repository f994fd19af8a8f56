/*
 * moe_oracle.c -- plain, slow, fp64 CPU oracle of the Flash-MoE expert layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or table with the GPU library and never calls it.
 *
 * Everything is computed from the definition, in double precision, on the
 * canonical tensors (one quantisation code per byte, bf16 bit patterns for
 * scales, biases, norm weight, router and shared-gate vectors):
 *
 *   - RMSNorm in two passes (sum of squares, then scaling):
 *       "48GB内存运行397B模型", section "Metal GPU管线" (RMS归一化);
 *       juejin post, "2. Metal 着色器——手写 GPU 内核".
 *   - router GEMV over the experts, softmax, top-K:
 *       juejin post, "3. 流水线设计" (GPU 路由 -> CPU topK);
 *       mxp.tw notes, "3. Pipeline 設計" (routing softmax 和 topK);
 *       flash-moe README translation, "Pipeline mỗi lớp".
 *     The K selected probabilities are renormalised to sum to one.
 *   - expert weights dequantised as  w = code * scale + bias, with one scale
 *     and one bias per group of 64 consecutive reduction-axis entries of a row:
 *       "48GB内存运行397B模型", sections "量化策略" and "Metal GPU管线"
 *       (4-bit dequant mat-vec, (nibble*scale+bias)*x).
 *   - SwiGLU, a = silu(gate) * up:  same page, "Metal GPU管线" (Fused SwiGLU).
 *   - combine: out = x + sum_k w_k y_k + sigmoid(g_s) y_shared:
 *       same page, "Metal GPU管线" (MoE combine + residual + sigmoid gate);
 *       juejin post, "2. Metal 着色器" (融合 MoE combine + 残差 + sigmoid 门控).
 *
 * No blocking, fusion or reordering beyond the definition: every dot product
 * is one serial sum in index order.  OpenMP only splits independent output
 * rows, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* bf16 bit pattern -> exact value (bf16 is the top half of an fp32). */
static double bf16_value(uint16_t v) {
    uint32_t u = (uint32_t)v << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* One dequantised weight, exact in fp64. */
double oracle_dequant(uint8_t code, uint16_t scale_bits, uint16_t bias_bits) {
    return (double)code * bf16_value(scale_bits) + bf16_value(bias_bits);
}

/* Pass 1: mean of squares; pass 2: h_i = x_i / sqrt(ms + eps) * gamma_i. */
void oracle_rmsnorm(int64_t n, const float *x, const uint16_t *gamma, double eps, double *h) {
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) ss += (double)x[i] * (double)x[i];
    double inv = 1.0 / sqrt(ss / (double)n + eps);
    for (int64_t i = 0; i < n; ++i) h[i] = (double)x[i] * inv * bf16_value(gamma[i]);
}

/* out_r = sum_c W[r][c] * v_c for a bf16 matrix W [rows][cols]. */
void oracle_gemv_bf16(int64_t rows, int64_t cols, const uint16_t *W, const double *v, double *out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *row = W + r * cols;
        double acc = 0.0;
        for (int64_t c = 0; c < cols; ++c) acc += bf16_value(row[c]) * v[c];
        out[r] = acc;
    }
}

/* out_r = sum_c (q[r][c] * s[r][c/G] + b[r][c/G]) * v_c  -- the quantised GEMV. */
void oracle_qgemv(int64_t rows, int64_t cols, int64_t group, const uint8_t *codes,
                  const uint16_t *scale, const uint16_t *bias, const double *v, double *out) {
    const int64_t ng = cols / group;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double acc = 0.0;
        for (int64_t c = 0; c < cols; ++c) {
            int64_t g = r * ng + c / group;
            acc += oracle_dequant(codes[r * cols + c], scale[g], bias[g]) * v[c];
        }
        out[r] = acc;
    }
}

static double sigmoid(double t) { return 1.0 / (1.0 + exp(-t)); }

/*
 * Softmax over all E logits, then the K largest by the key (logit descending,
 * expert index ascending), then renormalisation of the K probabilities.
 * Writes idx[K] in key order and w[K].  Returns 0, or -1 on bad arguments.
 */
int oracle_route(int64_t E, int64_t K, const double *z, int32_t *idx, double *w) {
    if (K < 1 || K > E) return -1;
    double zmax = z[0];
    for (int64_t e = 1; e < E; ++e) if (z[e] > zmax) zmax = z[e];
    double *p = (double *)malloc((size_t)E * sizeof(double));
    char *taken = (char *)calloc((size_t)E, 1);
    if (!p || !taken) { free(p); free(taken); return -1; }
    double denom = 0.0;
    for (int64_t e = 0; e < E; ++e) { p[e] = exp(z[e] - zmax); denom += p[e]; }
    for (int64_t e = 0; e < E; ++e) p[e] /= denom;
    /* selection by repeated scan: the first (lowest-index) maximum wins. */
    for (int64_t k = 0; k < K; ++k) {
        int64_t best = -1;
        for (int64_t e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || z[e] > z[best]) best = e;
        }
        taken[best] = 1;
        idx[k] = (int32_t)best;
    }
    double sel = 0.0;
    for (int64_t k = 0; k < K; ++k) sel += p[idx[k]];
    for (int64_t k = 0; k < K; ++k) w[k] = p[idx[k]] / sel;
    free(p);
    free(taken);
    return 0;
}

/*
 * One expert's FFN on a normalised token h[H]:
 *   g = W_gate h, u = W_up h  (W_gate, W_up: [F][H]),
 *   a_j = silu(g_j) * u_j,    silu(t) = t * sigmoid(t),
 *   y = W_down a              (W_down: [H][F]).
 * codes/scale/bias point at the three matrices in the order gate, up, down.
 */
void oracle_expert(int64_t H, int64_t F, int64_t group, const uint8_t *const codes[3],
                   const uint16_t *const scale[3], const uint16_t *const bias[3],
                   const double *h, double *y) {
    double *g = (double *)malloc((size_t)F * sizeof(double));
    double *u = (double *)malloc((size_t)F * sizeof(double));
    double *a = (double *)malloc((size_t)F * sizeof(double));
    oracle_qgemv(F, H, group, codes[0], scale[0], bias[0], h, g);
    oracle_qgemv(F, H, group, codes[1], scale[1], bias[1], h, u);
    for (int64_t j = 0; j < F; ++j) a[j] = g[j] * sigmoid(g[j]) * u[j];
    oracle_qgemv(H, F, group, codes[2], scale[2], bias[2], a, y);
    free(g);
    free(u);
    free(a);
}

/*
 * The whole expert layer for one token, given every expert the routing may
 * select.  experts_* hold E+1 entries of 3 pointers each (gate, up, down); entry
 * E is the shared expert.  Entries of experts that are not selected may be NULL.
 * Outputs: out[H], idx[K], w[K]; optional (NULL to skip) z_out[E], gs_out[1].
 */
int oracle_layer(int64_t H, int64_t F, int64_t E, int64_t K, int64_t group, double eps,
                 const float *x, const uint16_t *gamma, const uint16_t *router,
                 const uint16_t *shared_gate, const uint8_t *const *experts_codes,
                 const uint16_t *const *experts_scale, const uint16_t *const *experts_bias,
                 double *out, int32_t *idx, double *w, double *z_out, double *gs_out) {
    double *h = (double *)malloc((size_t)H * sizeof(double));
    double *z = (double *)malloc((size_t)E * sizeof(double));
    double *y = (double *)malloc((size_t)H * sizeof(double));
    int rc = 0;
    oracle_rmsnorm(H, x, gamma, eps, h);
    oracle_gemv_bf16(E, H, router, h, z);
    double gs = 0.0;
    oracle_gemv_bf16(1, H, shared_gate, h, &gs);
    if (oracle_route(E, K, z, idx, w) != 0) { rc = -1; goto done; }
    for (int64_t o = 0; o < H; ++o) out[o] = (double)x[o];
    for (int64_t k = 0; k <= K; ++k) {
        int64_t e = (k < K) ? idx[k] : E;
        double coef = (k < K) ? w[k] : sigmoid(gs);
        if (!experts_codes[3 * e] || !experts_codes[3 * e + 1] || !experts_codes[3 * e + 2]) {
            rc = -2;
            goto done;
        }
        oracle_expert(H, F, group, experts_codes + 3 * e, experts_scale + 3 * e,
                      experts_bias + 3 * e, h, y);
        for (int64_t o = 0; o < H; ++o) out[o] += coef * y[o];
    }
    if (z_out) memcpy(z_out, z, (size_t)E * sizeof(double));
    if (gs_out) *gs_out = gs;
done:
    free(h);
    free(z);
    free(y);
    return rc;
}
