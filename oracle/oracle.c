/*
 * CPU oracle: the MoE layer and the residual stack, in fp64 — TEST
 * INFRASTRUCTURE (only tests, the smoke check and the CPU-baseline leg of the
 * benchmark use it; it shares no code with the GPU library).
 *
 * What the method computes, and where it is stated:
 *  - Routing: "Luce Spark runs 35B MoE models on 16GB GPU without speed loss"
 *    (theneuralfeed.com), opening paragraph — each token is routed to about 8
 *    of 256 experts.  The evaluation workloads fix the rest: top-k of the
 *    router logits, the softmax renormalised over the chosen experts, RMSNorm
 *    before routing, a Zipf bias added to the logits, SwiGLU experts, Q4_0
 *    weights valued (q - 8) * scale, and the gate-weighted combine.
 *  - Same page, paragraph "The key components": where an expert's weights sit
 *    (pinned slot, ring slot, host memory) never changes what is computed —
 *    full residency is bit-identical to all-GPU execution.  This file
 *    therefore never looks at placement.
 *
 * Every step is the plain definition, in fp64, in natural index order.
 * OpenMP splits only independent output elements, so results do not depend on
 * the thread count.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* Threads the OpenMP loops of this library use (for reporting). */
int oracle_num_threads(void) { return omp_get_max_threads(); }

/* Threads for the OpenMP loops that follow (timing only: results do not depend on it). */
void oracle_set_num_threads(int n) {
    if (n > 0) omp_set_num_threads(n);
}

/* IEEE binary16 -> fp64, exact (sign, 5-bit exponent, 10-bit fraction). */
double oracle_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-14 * 2^-10 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* GGUF Q4_0 block: fp16 scale s (little-endian) then 16 bytes; weight j is
 * the low nibble of byte j and weight j+16 the high nibble; value (q-8)*s. */
void oracle_q4_0_block(const uint8_t* blk, double* w) {
    uint16_t sh = (uint16_t)(blk[0] | (blk[1] << 8));
    double s = oracle_f16_to_f64(sh);
    for (int j = 0; j < 16; ++j) {
        int lo = blk[2 + j] & 0x0f;
        int hi = blk[2 + j] >> 4;
        w[j] = (double)(lo - 8) * s;
        w[j + 16] = (double)(hi - 8) * s;
    }
}

/* u = x / sqrt(mean(x^2) + eps), unit gain. */
void oracle_rmsnorm(int d, const double* x, double eps, double* u) {
    double ss = 0.0;
    for (int i = 0; i < d; ++i) ss += x[i] * x[i];
    double r = sqrt(ss / (double)d + eps);
    for (int i = 0; i < d; ++i) u[i] = x[i] / r;
}

/* logits_e = sum_i wr[e][i] u_i + bias_e. */
void oracle_router(int E, int d, const float* wr, const double* u, const float* bias, double* logits) {
    #pragma omp parallel for schedule(static)
    for (int e = 0; e < E; ++e) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += (double)wr[(int64_t)e * d + i] * u[i];
        logits[e] = acc + (bias ? (double)bias[e] : 0.0);
    }
}

/* The K experts that come first under (logit descending, index ascending),
 * in that order: K passes, each taking the best expert not yet chosen. */
void oracle_topk(int E, int K, const double* logits, int32_t* idx) {
    char* taken = (char*)calloc((size_t)E, 1);
    for (int k = 0; k < K; ++k) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || logits[e] > logits[best]) best = e; /* ties keep the lower index */
        }
        taken[best] = 1;
        idx[k] = best;
    }
    free(taken);
}

/* Softmax over the chosen logits (the full softmax renormalised over the
 * chosen set); shifted by the first chosen logit. */
void oracle_gates(int K, const double* logits, const int32_t* idx, double* g) {
    double m = logits[idx[0]];
    double z = 0.0;
    for (int k = 0; k < K; ++k) {
        g[k] = exp(logits[idx[k]] - m);
        z += g[k];
    }
    for (int k = 0; k < K; ++k) g[k] /= z;
}

/* out = W v for W [rows][cols] in fp32 or Q4_0 (blocks along cols). */
void oracle_matvec(int rows, int cols, int wfmt, const void* w, const double* v, double* out) {
    #pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        double acc = 0.0;
        if (wfmt == ORACLE_W_F32) {
            const float* row = (const float*)w + (int64_t)r * cols;
            for (int i = 0; i < cols; ++i) acc += (double)row[i] * v[i];
        } else {
            int nb = cols / 32;
            const uint8_t* row = (const uint8_t*)w + (int64_t)r * nb * 18;
            double wb[32];
            for (int b = 0; b < nb; ++b) {
                oracle_q4_0_block(row + (int64_t)b * 18, wb);
                for (int j = 0; j < 32; ++j) acc += wb[j] * v[b * 32 + j];
            }
        }
        out[r] = acc;
    }
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* SwiGLU expert: h = silu(Wg u) * (Wu u), y = Wd h.  h may be NULL. */
void oracle_expert(int d, int f, int wfmt, const void* gate, const void* up, const void* down,
                   const double* u, double* h_out, double* y) {
    double* a = (double*)malloc(sizeof(double) * (size_t)f);
    double* b = (double*)malloc(sizeof(double) * (size_t)f);
    double* h = (double*)malloc(sizeof(double) * (size_t)f);
    oracle_matvec(f, d, wfmt, gate, u, a);
    oracle_matvec(f, d, wfmt, up, u, b);
    for (int j = 0; j < f; ++j) h[j] = silu(a[j]) * b[j];
    oracle_matvec(d, f, wfmt, down, h, y);
    if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)f);
    free(a);
    free(b);
    free(h);
}

int oracle_layer(const oracle_shape* s, int T, const double* x, const float* wr,
                 const float* bias, const int32_t* bias_row, const void* const* gate,
                 const void* const* up, const void* const* down, const int32_t* forced,
                 double* y, int32_t* idx_out, double* g_out, double* logits_out) {
    const int d = s->d, E = s->E, K = s->K, f = s->f;
    if (d <= 0 || E <= 0 || K <= 0 || K > E || f <= 0) return -1;
    if (s->wfmt == ORACLE_W_Q4_0 && (d % 32 || f % 32)) return -1;
    double* u = (double*)malloc(sizeof(double) * (size_t)d);
    double* lg = (double*)malloc(sizeof(double) * (size_t)E);
    double* ye = (double*)malloc(sizeof(double) * (size_t)d);
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    double* g = (double*)malloc(sizeof(double) * (size_t)K);
    for (int t = 0; t < T; ++t) {
        const double* xt = x + (int64_t)t * d;
        if (s->norm)
            oracle_rmsnorm(d, xt, s->eps, u);
        else
            memcpy(u, xt, sizeof(double) * (size_t)d);
        const float* brow = bias ? bias + (int64_t)(bias_row ? bias_row[t] : 0) * E : NULL;
        oracle_router(E, d, wr, u, brow, lg);
        if (forced && forced[(int64_t)t * K] >= 0)
            memcpy(sel, forced + (int64_t)t * K, sizeof(int32_t) * (size_t)K);
        else
            oracle_topk(E, K, lg, sel);
        oracle_gates(K, lg, sel, g);
        double* yt = y + (int64_t)t * d;
        for (int i = 0; i < d; ++i) yt[i] = 0.0;
        for (int k = 0; k < K; ++k) { /* rank order */
            int e = sel[k];
            oracle_expert(d, f, s->wfmt, gate[e], up[e], down[e], u, NULL, ye);
            for (int i = 0; i < d; ++i) yt[i] += g[k] * ye[i];
        }
        if (idx_out) memcpy(idx_out + (int64_t)t * K, sel, sizeof(int32_t) * (size_t)K);
        if (g_out) memcpy(g_out + (int64_t)t * K, g, sizeof(double) * (size_t)K);
        if (logits_out) memcpy(logits_out + (int64_t)t * E, lg, sizeof(double) * (size_t)E);
    }
    free(u);
    free(lg);
    free(ye);
    free(sel);
    free(g);
    return 0;
}

int oracle_stack(const oracle_shape* s, int L, int T, double* x, const float* const* wr,
                 const float* const* bias, const int32_t* bias_row, const void* const* gate,
                 const void* const* up, const void* const* down, int32_t* idx_trace,
                 double* x_trace) {
    const int d = s->d, E = s->E, K = s->K;
    double* y = (double*)malloc(sizeof(double) * (size_t)d);
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    int rc = 0;
    for (int t = 0; t < T && rc == 0; ++t) {
        double* xt = x + (int64_t)t * d;
        for (int l = 0; l < L && rc == 0; ++l) {
            if (x_trace) memcpy(x_trace + ((int64_t)t * L + l) * d, xt, sizeof(double) * (size_t)d);
            int32_t row = bias_row ? bias_row[t] : 0;
            rc = oracle_layer(s, 1, xt, wr[l], bias ? bias[l] : NULL, &row, gate + (int64_t)l * E,
                              up + (int64_t)l * E, down + (int64_t)l * E, NULL, y, sel, NULL, NULL);
            for (int i = 0; i < d; ++i) xt[i] += y[i];
            if (idx_trace) memcpy(idx_trace + ((int64_t)t * L + l) * K, sel, sizeof(int32_t) * (size_t)K);
        }
    }
    free(y);
    free(sel);
    return rc;
}
