/*
 * Seeded synthetic inputs for the resident-expert-caching MoE workloads.
 *
 * This module is shared by the CPU oracle and the GPU path.  It holds none of
 * the method's arithmetic: it only draws numbers (router weights, expert
 * weights, tokens, the Zipf routing bias) and encodes expert weights into the
 * GGUF Q4_0 block format that both sides then consume bit for bit.
 *
 * Random numbers: Philox4x64-10, the counter-based generator published by
 * Salmon, Moraes, Dror and Shaw ("Parallel random numbers: as easy as 1, 2, 3",
 * SC'11).  Every value is a pure function of (seed, tensor id, counter), so any
 * single expert can be regenerated on its own and the result never depends on
 * the thread count.
 *
 * Normals: Box-Muller on 24-bit uniforms, with series for ln, sin and cos
 * written out below so the result does not depend on the host libm.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "gen.h"

/* ---------------- Philox4x64-10 ---------------- */

static inline uint64_t mulhilo64(uint64_t a, uint64_t b, uint64_t* hi) {
    __uint128_t p = (__uint128_t)a * (__uint128_t)b;
    *hi = (uint64_t)(p >> 64);
    return (uint64_t)p;
}

void wl_philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4]) {
    /* Multipliers and Weyl increments from the Philox paper (4x64 variant). */
    const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
    const uint64_t W0 = 0x9E3779B97F4A7C15ULL, W1 = 0xBB67AE8584CAA73BULL;
    uint64_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += W0; k1 += W1; }
        uint64_t hi0, hi1;
        uint64_t lo0 = mulhilo64(M0, c0, &hi0);
        uint64_t lo1 = mulhilo64(M1, c2, &hi1);
        uint64_t n0 = hi1 ^ c1 ^ k0;
        uint64_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* ---------------- normals ---------------- */

/* Normals by Box-Muller.  ln, cos and sin are evaluated with short series in
 * single precision (their error is far below the 24-bit uniform spacing), in
 * branch-free loops over a batch so the compiler can vectorise them; every
 * operation is an IEEE basic operation, so the result is the same with or
 * without vectorisation. */
#define WL_BATCH 32 /* Philox blocks per batch -> 256 normals */

static void wl_box_muller(int npairs, const uint32_t* ua, const uint32_t* ub, float* z) {
    for (int p = 0; p < npairs; ++p) {
        /* u1 in (0, 1]: ln u1 = e ln2 + ln m, m in [sqrt(1/2), sqrt(2)) */
        float u1 = 1.0f - (float)(int32_t)(ua[p] >> 8) * (1.0f / 16777216.0f);
        uint32_t bits;
        memcpy(&bits, &u1, 4);
        int e = (int)(bits >> 23) - 127;
        uint32_t mb = (bits & 0x7fffffu) | 0x3f800000u;
        float m;
        memcpy(&m, &mb, 4);
        int big = m > 1.41421356f;
        m = m * (1.0f - 0.5f * (float)big); /* exact: 1 or 1/2 */
        e += big;
        float t = (m - 1.0f) / (m + 1.0f);
        float t2 = t * t;
        float ser = 1.0f + t2 * (1.0f / 3 + t2 * (1.0f / 5 + t2 * (1.0f / 7 + t2 * (1.0f / 9))));
        float ln = (float)e * 0.693147181f + 2.0f * t * ser;
        float rad = sqrtf(-2.0f * ln);
        /* angle 2 pi u2, quarter-turn reduction to |phi| <= pi/4 */
        float w = (float)(int32_t)(ub[p] >> 8) * (4.0f / 16777216.0f);
        float q = (float)(int)(w + 0.5f);
        float phi = (w - q) * 1.57079633f;
        float p2 = phi * phi;
        float sn = phi * (1.0f - p2 * (1.0f / 6) * (1.0f - p2 * (1.0f / 20) * (1.0f - p2 * (1.0f / 42) * (1.0f - p2 * (1.0f / 72)))));
        float cs = 1.0f - p2 * 0.5f * (1.0f - p2 * (1.0f / 12) * (1.0f - p2 * (1.0f / 30) * (1.0f - p2 * (1.0f / 56) * (1.0f - p2 * (1.0f / 90)))));
        /* rotate (cos, sin) of phi by qi quarter turns: swap for odd qi, then
         * flip signs; done with exact bit blends and +-1 products */
        int qi = ((int)q) & 3;
        uint32_t snb, csb;
        memcpy(&snb, &sn, 4);
        memcpy(&csb, &cs, 4);
        uint32_t mask = 0u - (uint32_t)(qi & 1);
        uint32_t cb = (snb & mask) | (csb & ~mask), sb = (csb & mask) | (snb & ~mask);
        float c0, s0;
        memcpy(&c0, &cb, 4);
        memcpy(&s0, &sb, 4);
        float c = c0 * (float)(1 - 2 * ((qi ^ (qi >> 1)) & 1));
        float s = s0 * (float)(1 - 2 * ((qi >> 1) & 1));
        z[2 * p] = rad * c;
        z[2 * p + 1] = rad * s;
    }
}

/* Normals for Philox blocks blk0 .. blk0+nblk-1 of stream (key, a, b):
 * block i gives normals 8i .. 8i+7. */
static void wl_normals_blocks(const uint64_t key[2], uint64_t a, uint64_t b, int64_t blk0, int nblk,
                              float sigma, float* out) {
    uint32_t ua[WL_BATCH * 4], ub[WL_BATCH * 4];
    float z[WL_BATCH * 8];
    for (int i = 0; i < nblk; ++i) {
        uint64_t ctr[4] = {(uint64_t)(blk0 + i), a, b, 0};
        uint64_t r[4];
        wl_philox4x64_10(ctr, key, r);
        for (int p = 0; p < 4; ++p) {
            ua[4 * i + p] = (uint32_t)(r[p] & 0xffffffffu);
            ub[4 * i + p] = (uint32_t)(r[p] >> 32);
        }
    }
    wl_box_muller(nblk * 4, ua, ub, z);
    for (int j = 0; j < nblk * 8; ++j) out[j] = z[j] * sigma;
}

void wl_normal_f32(uint64_t seed, uint64_t tensor, uint64_t a, uint64_t b,
                   int64_t n, float sigma, float* out) {
    const uint64_t key[2] = {seed, tensor};
    int64_t nblk = (n + 7) / 8;
    int64_t nbat = (nblk + WL_BATCH - 1) / WL_BATCH;
    #pragma omp parallel for schedule(static) if (nbat > 64)
    for (int64_t bt = 0; bt < nbat; ++bt) {
        float z[WL_BATCH * 8];
        int64_t blk0 = bt * WL_BATCH;
        int nb = (int)((nblk - blk0) < WL_BATCH ? (nblk - blk0) : WL_BATCH);
        wl_normals_blocks(key, a, b, blk0, nb, sigma, z);
        int64_t base = blk0 * 8;
        for (int j = 0; j < nb * 8 && base + j < n; ++j) out[base + j] = z[j];
    }
}

/* One uniform double in [0, 1) (53 bits) for draw i of stream (key, a, b). */
double wl_uniform(uint64_t seed, uint64_t tensor, uint64_t a, uint64_t b, uint64_t i) {
    const uint64_t key[2] = {seed, tensor};
    uint64_t ctr[4] = {i, a, b, 1};
    uint64_t r[4];
    wl_philox4x64_10(ctr, key, r);
    return (double)(r[0] >> 11) * (1.0 / 9007199254740992.0);
}

/* ---------------- fp16 encoding (round to nearest even) ---------------- */

uint16_t wl_f32_to_f16(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t ax = x & 0x7fffffffu;
    if (ax >= 0x7f800000u) /* inf / nan */
        return (uint16_t)(sign | 0x7c00u | (ax > 0x7f800000u ? 0x200u : 0u));
    if (ax >= 0x477ff000u) /* rounds to >= 65520: overflow to inf */
        return (uint16_t)(sign | 0x7c00u);
    if (ax < 0x33000001u) /* < 2^-25 (ties to zero) */
        return (uint16_t)sign;
    int e = (int)(ax >> 23);
    uint32_t mant = (ax & 0x7fffffu) | 0x800000u;
    if (e < 113) { /* subnormal half: value = mant * 2^(e-150); unit is 2^-24 */
        int shift = 126 - e; /* 14..24 */
        uint32_t q = mant >> shift;
        uint32_t rem = mant & ((1u << shift) - 1u);
        uint32_t half = 1u << (shift - 1);
        if (rem > half || (rem == half && (q & 1u))) q += 1u;
        return (uint16_t)(sign | q);
    }
    uint32_t q = ((uint32_t)(e - 112) << 10) | ((mant >> 13) & 0x3ffu);
    uint32_t rem = mant & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (q & 1u))) q += 1u;
    return (uint16_t)(sign | q);
}

float wl_f16_to_f32(uint16_t h) {
    uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
    float v;
    if (e == 0) {
        v = (float)m * (1.0f / 16777216.0f);
        if (sign) v = -v;
        return v;
    }
    uint32_t bits = sign | (e == 31 ? (0xffu << 23) | (m << 13) : ((e + 112u) << 23) | (m << 13));
    memcpy(&v, &bits, 4);
    return v;
}

/* ---------------- GGUF Q4_0 encoding ---------------- */

/* One block: 32 weights -> 18 bytes (fp16 scale, then 16 bytes; weight j in
 * the low nibble of byte j, weight j+16 in the high nibble).  The scale is the
 * largest-magnitude weight (first on ties, sign kept) divided by -8; codes are
 * round-half-up of w/scale + 8, clamped to [0, 15]; an all-zero block gets
 * scale 0 and every code 8. */
void wl_q4_0_encode_block(const float* w, uint8_t* out) {
    float amax = 0.0f, m = 0.0f;
    for (int j = 0; j < 32; ++j) {
        float a = fabsf(w[j]);
        if (a > amax) { amax = a; m = w[j]; }
    }
    uint16_t sh = wl_f32_to_f16(amax > 0.0f ? m / -8.0f : 0.0f);
    float s = wl_f16_to_f32(sh);
    float inv = (s != 0.0f) ? 1.0f / s : 0.0f;
    out[0] = (uint8_t)(sh & 0xff);
    out[1] = (uint8_t)(sh >> 8);
    for (int j = 0; j < 16; ++j) {
        int q0 = (int)floorf(w[j] * inv + 8.5f);
        int q1 = (int)floorf(w[j + 16] * inv + 8.5f);
        q0 = q0 < 0 ? 0 : (q0 > 15 ? 15 : q0);
        q1 = q1 < 0 ? 0 : (q1 > 15 ? 15 : q1);
        out[2 + j] = (uint8_t)(q0 | (q1 << 4));
    }
}

void wl_q4_0_encode(int64_t rows, int64_t cols, const float* w, uint8_t* out) {
    int64_t nb = cols / 32;
    #pragma omp parallel for schedule(static) if (rows > 64)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b)
            wl_q4_0_encode_block(w + r * cols + b * 32, out + (r * nb + b) * 18);
}

/* ---------------- model tensors ---------------- */

/* Tensor ids keep the Philox streams of different tensors apart. */
enum { WL_T_ROUTER = 1, WL_T_GATE = 2, WL_T_UP = 3, WL_T_DOWN = 4, WL_T_PERM = 5, WL_T_TOKENS = 100 };

void wl_router(uint64_t seed, int layer, int E, int d, float sigma, float* wr) {
    wl_normal_f32(seed, WL_T_ROUTER, (uint64_t)layer, 0, (int64_t)E * d, sigma, wr);
}

/* Draw one matrix [rows][cols] N(0, sigma) with 8 normals per Philox block,
 * block index along the row-major order, then encode it if Q4_0. */
static void wl_matrix(uint64_t seed, uint64_t tensor, int layer, int expert, int rows, int cols,
                      int wfmt, float sigma, void* out, float* scratch) {
    float* w = (wfmt == WL_FMT_F32) ? (float*)out : scratch;
    int64_t n = (int64_t)rows * cols; /* a multiple of 32 */
    const uint64_t key[2] = {seed, tensor};
    int64_t nblk = n / 8;
    for (int64_t blk0 = 0; blk0 < nblk; blk0 += WL_BATCH) {
        int nb = (int)((nblk - blk0) < WL_BATCH ? (nblk - blk0) : WL_BATCH);
        wl_normals_blocks(key, (uint64_t)layer, (uint64_t)expert, blk0, nb, sigma, w + blk0 * 8);
    }
    if (wfmt == WL_FMT_Q4_0) {
        int64_t nb = cols / 32;
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t b = 0; b < nb; ++b)
                wl_q4_0_encode_block(w + r * (int64_t)cols + b * 32, (uint8_t*)out + (r * nb + b) * 18);
    }
}

int64_t wl_matrix_bytes(int rows, int cols, int wfmt) {
    return wfmt == WL_FMT_F32 ? (int64_t)rows * cols * 4 : (int64_t)rows * (cols / 32) * 18;
}

int wl_expert(uint64_t seed, int layer, int expert, int d, int f, int wfmt, float sigma,
              void* gate, void* up, void* down, float* scratch) {
    if (d % 32 || f % 32) return -1;
    wl_matrix(seed, WL_T_GATE, layer, expert, f, d, wfmt, sigma, gate, scratch);
    wl_matrix(seed, WL_T_UP, layer, expert, f, d, wfmt, sigma, up, scratch);
    wl_matrix(seed, WL_T_DOWN, layer, expert, d, f, wfmt, sigma, down, scratch);
    return 0;
}

/* Many experts into one contiguous buffer, expert-major (gate | up | down per
 * expert); experts are independent, so they are drawn in parallel. */
int wl_experts(uint64_t seed, int layer0, int n_layers, int E, int d, int f, int wfmt, float sigma,
               uint8_t* out) {
    if (d % 32 || f % 32) return -1;
    int64_t mb = wl_matrix_bytes(f, d, wfmt), db = wl_matrix_bytes(d, f, wfmt);
    int64_t per = 2 * mb + db;
    int64_t total = (int64_t)n_layers * E;
    #pragma omp parallel
    {
        float* scratch = (float*)malloc(sizeof(float) * (size_t)d * (size_t)f);
        #pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < total; ++i) {
            int l = layer0 + (int)(i / E), e = (int)(i % E);
            uint8_t* p = out + i * per;
            wl_expert(seed, l, e, d, f, wfmt, sigma, p, p + mb, p + 2 * mb, scratch);
        }
        free(scratch);
    }
    return 0;
}

void wl_tokens(uint64_t seed, uint64_t stream, int64_t t0, int64_t T, int d, float* x) {
    #pragma omp parallel for schedule(static) if (T > 16)
    for (int64_t t = 0; t < T; ++t)
        wl_normal_f32(seed, WL_T_TOKENS + stream, (uint64_t)(t0 + t), 0, d, 1.0f, x + t * (int64_t)d);
}

/* Zipf routing bias for one layer: a seeded permutation gives every expert a
 * popularity rank r (1-based); p_r is proportional to r^-alpha and the bias is
 * scale * ln p_r, computed in fp64 and rounded once to fp32. */
void wl_zipf_bias(uint64_t seed, int layer, int E, double alpha, double scale, float* bias,
                  int32_t* rank_out) {
    int32_t perm[4096];
    if (E > 4096) return;
    for (int i = 0; i < E; ++i) perm[i] = i;
    for (int i = E - 1; i >= 1; --i) { /* Fisher-Yates */
        double u = wl_uniform(seed, WL_T_PERM, (uint64_t)layer, 0, (uint64_t)i);
        int j = (int)(u * (double)(i + 1));
        if (j > i) j = i;
        int32_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
    }
    double z = 0.0;
    for (int r = 1; r <= E; ++r) z += pow((double)r, -alpha);
    for (int r = 1; r <= E; ++r) {
        int e = perm[r - 1];
        double p = pow((double)r, -alpha) / z;
        bias[e] = (float)(scale * log(p));
        if (rank_out) rank_out[e] = r;
    }
}
