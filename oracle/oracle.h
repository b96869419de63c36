/*
 * CPU oracle for the resident-expert-caching MoE layer — TEST INFRASTRUCTURE.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  The product path never links, loads or calls it, and it
 * shares no code with the GPU library.
 *
 * Sources for what is computed:
 *  - "Luce Spark runs 35B MoE models on 16GB GPU without speed loss"
 *    (theneuralfeed.com), opening paragraph: the router picks about 8 of 256
 *    experts per token; paragraph "The key components": (1) per-expert
 *    routing counts and a pinned most-used set, (2) a fixed ring of spare GPU
 *    slots filled from pinned host memory with LRU eviction, (3) one graph per
 *    token; full residency is bit-identical to all-GPU execution.
 *  - The evaluation workloads: Q4_0 weights valued (q - 8) * scale, a SwiGLU
 *    expert FFN, top-k with the softmax renormalised over the chosen experts,
 *    RMSNorm before the router, residual update x += MoE(RMSNorm(x)), and a
 *    Zipf logit bias added to the router output.
 *
 * All arithmetic is fp64; fp32 and Q4_0 inputs convert to fp64 exactly.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#define ORACLE_W_F32 0
#define ORACLE_W_Q4_0 1

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t d;     /* hidden size */
    int32_t E;     /* experts per layer */
    int32_t K;     /* experts chosen per token */
    int32_t f;     /* expert intermediate size */
    int32_t wfmt;  /* ORACLE_W_F32 or ORACLE_W_Q4_0 */
    int32_t norm;  /* 1: RMSNorm before the router and the experts */
    double eps;    /* RMSNorm epsilon */
} oracle_shape;

/* threads the OpenMP loops use (reporting only) */
int oracle_num_threads(void);
/* set the OpenMP thread count (timing only) */
void oracle_set_num_threads(int n);

/* ---- elementary steps ---- */
double oracle_f16_to_f64(uint16_t h);
void oracle_q4_0_block(const uint8_t* blk18, double* w32);
void oracle_rmsnorm(int d, const double* x, double eps, double* u);
void oracle_router(int E, int d, const float* wr, const double* u, const float* bias, double* logits);
void oracle_topk(int E, int K, const double* logits, int32_t* idx);
void oracle_gates(int K, const double* logits, const int32_t* idx, double* g);
void oracle_matvec(int rows, int cols, int wfmt, const void* w, const double* v, double* out);
void oracle_expert(int d, int f, int wfmt, const void* gate, const void* up, const void* down,
                   const double* u, double* h, double* y);

/* ---- one MoE layer over T independent tokens ----
 * x        [T][d]   layer input (before RMSNorm)
 * wr       [E][d]   router weights, fp32
 * bias     [rows][E] router logit bias, fp32, or NULL
 * bias_row [T]      row of `bias` used by each token, or NULL (row 0)
 * gate/up/down [E]  per-expert weights: gate, up [f][d]; down [d][f];
 *                   fp32 row-major or GGUF Q4_0 blocks along the input dim
 * forced   [T][K]   or NULL: when forced[t*K] >= 0 token t uses this selection
 *                   (in this order) instead of its own top-k
 * Outputs (each may be NULL except y):
 * y [T][d] MoE output (without the residual); idx [T][K]; g [T][K];
 * logits [T][E].
 */
int oracle_layer(const oracle_shape* s, int T, const double* x, const float* wr,
                 const float* bias, const int32_t* bias_row, const void* const* gate,
                 const void* const* up, const void* const* down, const int32_t* forced,
                 double* y, int32_t* idx, double* g, double* logits);

/* ---- the residual stack x_{l+1} = x_l + MoE_l(RMSNorm(x_l)) ----
 * wr[L], bias[L] (each may be NULL), experts [L*E] pointer arrays,
 * x [T][d] updated in place; idx_trace [T][L][K] and x_trace [T][L][d]
 * (layer inputs) may be NULL.  Tokens are independent. */
int oracle_stack(const oracle_shape* s, int L, int T, double* x, const float* const* wr,
                 const float* const* bias, const int32_t* bias_row, const void* const* gate,
                 const void* const* up, const void* const* down, int32_t* idx_trace,
                 double* x_trace);

/* ---- placement / LRU-ring simulator ---- */
typedef struct oracle_sim oracle_sim;

typedef struct {
    int64_t seq;      /* 1-based fill sequence number */
    int32_t layer, expert, slot;
    int32_t kind;     /* ORACLE_EV_FILL or ORACLE_EV_PREFETCH */
    int32_t victim;   /* evicted l*E+e, or -1 when an empty ring slot was used */
    int32_t pad;
} oracle_event;

#define ORACLE_EV_FILL 2
#define ORACLE_EV_PREFETCH 3

/* stats: accesses, pinned_hits, cold_hits, ring_hits, fills, evictions, h2d_bytes */
#define ORACLE_N_STATS 8 /* accesses, pinned, cold, ring, fills, evictions, h2d bytes, prefetches */

oracle_sim* oracle_sim_create(int L, int E, int64_t P, int R, int64_t slot_bytes);
void oracle_sim_destroy(oracle_sim* s);
void oracle_sim_place_uniform(oracle_sim* s);
void oracle_sim_calibrate(oracle_sim* s, int reset_counts);
/* one online self-tuning step (hysteresis in percent, counts >>= decay_shift); returns swaps */
int64_t oracle_sim_retune(oracle_sim* s, int hyst_pct, int decay_shift);
void oracle_sim_decode_token(oracle_sim* s, int K, const int32_t* idx /* [L][K] */);
void oracle_sim_decode_layer(oracle_sim* s, int layer, int K, const int32_t* idx /* [K] */);
/* B tokens decoded together: accesses in (layer, token, rank) order */
void oracle_sim_decode_batch(oracle_sim* s, int B, int K, const int32_t* idx /* [B][L][K] */);
void oracle_sim_prefill_layer(oracle_sim* s, int layer, int T, int K, const int32_t* idx /* [T][K] */);
/* after a prefill layer: prefetch the next layer's predicted experts (hist [E]) */
int64_t oracle_sim_prefetch(oracle_sim* s, int layer, const int32_t* hist);
void oracle_sim_stats(const oracle_sim* s, int64_t* out);
void oracle_sim_reset_stats(oracle_sim* s);
void oracle_sim_placement(const oracle_sim* s, int32_t* slot_of /* [L][E] */,
                          int32_t* ring_owner /* [R] */, int64_t* ring_stamp /* [R] */,
                          int64_t* counts /* [L][E] */);
int64_t oracle_sim_events(const oracle_sim* s, oracle_event* out, int64_t cap);
int64_t oracle_sim_quota(int L, int64_t P, int layer);

#ifdef __cplusplus
}
#endif
#endif
