/*
 * moe_spark — resident expert caching for MoE decode on one MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only; "device" pointers are HIP device
 * memory (e.g. a torch tensor's data_ptr on ROCm), "host" pointers are
 * ordinary CPU memory.  Streams are hipStream_t passed as void*.
 *
 * What the library implements, and where it is described (each entry point
 * below names its passage, with these short names):
 *  [Spark] "Luce Spark runs 35B MoE models on 16GB GPU without speed loss"
 *  (theneuralfeed.com):
 *   - opening paragraph: each token is routed to about 8 of 256 experts, so
 *     only a fraction of the experts needs to sit in GPU memory;
 *   - paragraph "The key components":
 *     (1) calibrated placement — per-expert routing counts are accumulated
 *         and the most-used set is pinned in GPU memory;
 *     (2) a bounded asynchronous cache — a fixed ring of spare GPU slots; on
 *         a cold expert the weights are copied asynchronously from pinned host
 *         memory into a spare slot, evicting the least recently used entry,
 *         which costs throughput but does not stall;
 *     (3) the whole token runs as one graph instead of one graph per layer;
 *     and full residency is bit-identical to all-GPU execution (here: outputs
 *     are bit-identical at every residency).
 *  [Bagua] "Luce Spark: Shattering the VRAM Ceiling for 35B MoEs on 16GB GPUs
 *  Without the Offload Tax" (baguaai.com), "Event Core" and "Actionable
 *  Advice": hot experts live in GPU memory, the long tail in system RAM, and
 *  the link between them becomes the bottleneck.
 *
 * Ownership: the context owns the HBM slot arena ((P + R) expert slots), the
 * pinned host arena (every expert, copied in by moe_spark_set_expert), all
 * device tables, the token graphs and the fill-agent thread.  The caller owns
 * activation buffers and the streams it passes in.
 *
 * Errors: every call returns a moe_spark_status; moe_spark_last_error()
 * describes the last failure.  Calls that launch work are asynchronous on the
 * compute stream; device-side faults of the method (a fill that never
 * arrives) surface at moe_spark_synchronize().
 *
 * Environment, read by moe_spark_create (all optional; results never depend
 * on them):
 *   MOE_SPARK_PULL_FILLS=0      cold experts are copied by the host fill agent
 *                               on copy streams, not pulled by the kernels
 *                               from the pinned arena's device address (Q4_0)
 *   MOE_SPARK_COPY_STREAMS=1|2  copy streams the agent spreads decode fills
 *                               over (default 2)
 *   MOE_SPARK_FILL_COLS=1..128  prefill: grid columns of fill work-groups in
 *                               each pinned-expert GEMM launch (default 8)
 *   MOE_SPARK_DECODE_STREAM=1   decode launches its kernels one by one instead
 *                               of replaying the token graph
 */
#ifndef MOE_SPARK_H
#define MOE_SPARK_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_SPARK_OK = 0,
    MOE_SPARK_E_INVALID = 1, /* bad argument or shape */
    MOE_SPARK_E_NOMEM = 2,   /* an arena could not be allocated */
    MOE_SPARK_E_HIP = 3,     /* a HIP call failed, or a device-side error */
    MOE_SPARK_E_STATE = 4    /* call out of order (e.g. forward before all weights set) */
} moe_spark_status;

/* Expert weight formats (router weights are always fp32). */
typedef enum {
    MOE_SPARK_W_F32 = 0,  /* fp32, row-major [out][in] */
    MOE_SPARK_W_Q4_0 = 1  /* GGUF Q4_0: per row, blocks of 32 along `in`, 18 bytes each:
                             fp16 scale s (little endian), 16 bytes of codes; weight j in
                             the low nibble of byte j, weight j+16 in the high nibble;
                             value (q - 8) * s.  The Q4_0 paths multiply the codes with
                             activations rounded to fp16 (the normalised input and the
                             SwiGLU output), so those must stay inside fp16's range
                             (|v| <= 65504); fp32 contexts have no such limit. */
} moe_spark_wfmt;

/* Flags of moe_spark_layer_forward. */
#define MOE_SPARK_PRE_RMSNORM 1u /* u = x / sqrt(mean(x^2) + eps) before router and experts */
#define MOE_SPARK_RESIDUAL 2u    /* y = x + MoE(u) instead of y = MoE(u) */

typedef struct {
    int32_t n_layers;     /* L */
    int32_t d_model;      /* d: multiple of 256, <= 8192 */
    int32_t n_experts;    /* E: <= 1024 */
    int32_t top_k;        /* K: 1 <= K <= min(E, 16) */
    int32_t d_ff;         /* f: multiple of 128, <= 4096 */
    int32_t wfmt;         /* moe_spark_wfmt */
    float rms_eps;        /* RMSNorm epsilon (1e-6) */
    int32_t n_bias_rows;  /* router-bias rows per layer (0 = no bias) */
    int64_t resident_cap; /* P: pinned slots, global over layers, 0 <= P <= L*E */
    int32_t ring_slots;   /* R: spare ring slots; R >= K unless P == L*E; R <= 1024 */
    int32_t max_tokens;   /* largest n_tokens of moe_spark_prefill (0: no prefill) */
    int64_t event_cap;    /* capacity of the fill-event log (0: default 1<<20) */
} moe_spark_config;

typedef struct {
    int64_t accesses;      /* expert accesses (decode: per token, layer, rank;
                              prefill: per layer, distinct expert) */
    int64_t pinned_hits;   /* accesses served by a pinned slot */
    int64_t cold_hits;     /* accesses to a non-pinned expert (= ring_hits + fills) */
    int64_t ring_hits;     /* cold hits already in the ring */
    int64_t fills;         /* cold hits copied host -> ring slot */
    int64_t evictions;     /* fills that evicted a ring entry */
    int64_t h2d_bytes;     /* fills * slot bytes */
    int64_t fill_ns_sum;   /* host-observed latency of fills: request seen -> data ready */
    int64_t fill_ns_max;
    int64_t calib_uploads; /* experts copied into pinned slots by calibration */
    int64_t tokens;        /* tokens run by the decode graph */
    int64_t retunes;       /* online self-tuning steps taken (moe_spark_set_autotune) */
    int64_t retune_swaps;  /* experts those steps swapped into the pinned set */
    int64_t prefetches;    /* speculative copies of predicted experts into ring slots (prefill);
                              counted in h2d_bytes and, when they evict, in evictions */
} moe_spark_stats;

typedef struct {
    int64_t seq;     /* 1-based fill number */
    int32_t layer, expert;
    int32_t slot;    /* global slot id: pinned 0..P-1, ring P..P+R-1 */
    int32_t kind;    /* MOE_SPARK_EV_FILL or MOE_SPARK_EV_PREFETCH */
    int32_t victim;  /* evicted layer*E+expert, or -1 (slot was empty) */
    int32_t pad;
} moe_spark_event;

#define MOE_SPARK_EV_FILL 2
#define MOE_SPARK_EV_PREFETCH 3  /* a speculative copy of a predicted expert (prefill) */

typedef struct moe_spark_ctx moe_spark_ctx;

/* Create a context: allocates the HBM slot arena ((P+R) slots), the pinned
 * host arena (L*E slots) and all tables, and starts the fill agent.
 * compute_stream / copy_stream: hipStream_t, or NULL to let the context make
 * its own.  Q4_0 fills are pulled by the kernels themselves, through the
 * pinned host arena's device address: in decode the cold expert's
 * work-groups read it, compute from it and write it into the ring slot; in
 * prefill extra work-groups of the pinned experts' GEMM launches copy each
 * chunk's fills into their ring slots before the cold experts' GEMMs run.
 * Set MOE_SPARK_PULL_FILLS=0 in the environment to hand them to the fill
 * agent instead.  The fill agent issues the other ring fills on copy_stream;
 * while a prefill runs it also uses one more stream of the context's own
 * whenever copy_stream is busy (fills of one ring slot in flight together
 * share a stream).  moe_spark_synchronize waits for both.  Kernels wait for fills, so
 * neither copy stream may share a hardware queue with the compute stream:
 * keep the process's streams within GPU_MAX_HW_QUEUES (a fill that never
 * starts ends the wait with E_HIP "fill did not arrive in time").
 * Errors: E_INVALID (bad config; for Q4_0 also any shape other than
 * d_model = 2048, d_ff = 512, top_k <= 8, which the hand-tiled Q4_0 kernels
 * are built for; fp32 contexts take other shapes), E_NOMEM (arena), E_HIP.
 * Passage: [Spark] "The key components" (1) and (2): the pinned set and the
 * fixed ring of spare GPU slots are the slot arena's P and R slots; [Bagua]
 * "Event Core": the long tail lives in system RAM (the pinned host arena).
 */
moe_spark_status moe_spark_create(const moe_spark_config* cfg, void* compute_stream,
                                  void* copy_stream, moe_spark_ctx** out);

/* Stop the fill agent, free everything.  NULL is allowed.
 * Passage: none of its own (releases what moe_spark_create made).
 */
void moe_spark_destroy(moe_spark_ctx* ctx);

/* Text of the last error on this context (never NULL; "" when none).
 * Passage: none of its own (error reporting of every entry point).
 */
const char* moe_spark_last_error(const moe_spark_ctx* ctx);

/* Bytes of one expert slot (gate + up + down) in the configured format.
 * Passage: [Spark] "The key components" (2): the unit a cold-expert copy moves.
 */
int64_t moe_spark_slot_bytes(const moe_spark_ctx* ctx);

/* Router of one layer, host memory: w [E][d] fp32; bias [n_bias_rows][E]
 * fp32 (added to the logits before top-k and softmax), or NULL when
 * n_bias_rows == 0.  Copied; synchronous.
 * Passage: [Spark] opening paragraph: the router picks about 8 of 256 experts
 * per token.  Synchronises both streams first (queued work may read it).
 */
moe_spark_status moe_spark_set_router(moe_spark_ctx* ctx, int32_t layer, const float* w,
                                      const float* bias);

/* One expert, host memory: gate, up [f][d]; down [d][f]; in the configured
 * format (row-major fp32, or GGUF Q4_0 blocks along the input dimension).
 * Repacked into the pinned host arena; the caller may free its buffers.
 * If the expert sits in a pinned slot its slot is refreshed.
 * Passage: [Bagua] "Event Core" and [Spark] opening paragraph: every expert's
 * weights live in system RAM (the pinned host arena); the resident ones are
 * copies.  Synchronises both streams first; every resident copy (pinned slot
 * or ring slot) is refreshed, so outputs stay independent of residency.
 */
moe_spark_status moe_spark_set_expert(moe_spark_ctx* ctx, int32_t layer, int32_t expert,
                                      const void* gate, const void* up, const void* down);

/* n experts with flat ids first .. first+n-1 (id = layer*E + expert) from one
 * host buffer, each expert gate | up | down back to back (same formats as
 * moe_spark_set_expert).  Repacks on host threads.
 * Passage: as moe_spark_set_expert.
 */
moe_spark_status moe_spark_set_experts(moe_spark_ctx* ctx, int64_t first, int64_t n,
                                       const void* blob);

/* Initial placement: layer l pins experts 0..q_l-1, q_l = floor(P/L) + [l < P mod L];
 * pinned slots 0..P-1 in (layer, expert) order; the ring is emptied.
 * Uploads the pinned experts; synchronous.  E_STATE before all weights are set.
 * Passage: [Spark] "The key components": the "naive uniform offload" the
 * calibrated placement is measured against (here it keeps the same ring).
 */
moe_spark_status moe_spark_place_uniform(moe_spark_ctx* ctx);

/* Calibrated placement: each layer pins its q_l most-counted experts (count
 * descending, expert ascending).  Experts that stay keep their slot; freed
 * slots (ascending) go to newly pinned experts in (layer, expert) order; a
 * newly pinned expert's ring entry is emptied.  reset_counts != 0 zeroes the
 * counts afterwards.  Synchronises both streams (call between tokens).
 * Passage: [Spark] "The key components" (1): accumulate per-expert routing
 * frequencies and pin the most-used set; [Bagua] "Dynamic Expert
 * Calibration".
 */
moe_spark_status moe_spark_calibrate(moe_spark_ctx* ctx, int32_t reset_counts);

/* Online self-tuning of the placement during decode.  The pages' "The key
 * components" paragraph has the engine profile live traffic and keep
 * re-deciding which experts stay resident; this is that loop made explicit.
 * Once interval_tokens decode tokens have run since the placement last
 * changed (calibration, uniform placement or the previous step), the next
 * decode token is preceded by one step, taken on the host between tokens:
 *  - per layer, experts are ordered by (count desc, expert asc); the
 *    strongest unpinned expert x displaces the weakest pinned expert y while
 *    100*count[x] > (100 + hysteresis_pct)*count[y] (the next strongest and
 *    next weakest are then compared; the first failing pair ends the layer);
 *  - slots move as in moe_spark_calibrate (freed slots, ascending, to the
 *    entering experts in (layer, expert) order; their ring entries emptied);
 *  - every count is then shifted right by decay_shift bits.
 * interval_tokens = 0 turns it off (the default).  Only decode tokens count;
 * a step synchronises both streams and uploads the entering experts.
 * Errors: E_INVALID for interval < 0, hysteresis_pct outside [0, 100000] or
 * decay_shift outside [0, 62].
 * Passage: [Spark] opening paragraph ("self-tunes over time") and [Bagua]
 * "Dynamic Expert Calibration" (profiles real-time traffic).
 */
moe_spark_status moe_spark_set_autotune(moe_spark_ctx* ctx, int32_t interval_tokens, int32_t hysteresis_pct,
                                        int32_t decay_shift);

/* One MoE layer for n_tokens tokens, each run as a separate batch-1 decode
 * step in order (route, then experts, then combine).  Device pointers:
 * x [T][d] fp32 input, y [T][d] fp32 output (y may equal x),
 * bias_row [T] int32 row of the router bias per token (NULL: row 0),
 * topk_out [T][K] int32 and gates_out [T][K] fp32 (either may be NULL).
 * flags: MOE_SPARK_PRE_RMSNORM | MOE_SPARK_RESIDUAL.  Counts, placement and
 * stats are updated exactly as in a decode step of that layer.
 * Passage: [Spark] opening paragraph (one MoE layer: about 8 of 256 experts
 * per token) and "The key components" (1)-(2) for the counts and the cache.
 */
moe_spark_status moe_spark_layer_forward(moe_spark_ctx* ctx, int32_t layer, const float* x,
                                         float* y, int32_t n_tokens, const int32_t* bias_row,
                                         uint32_t flags, int32_t* topk_out, float* gates_out);

/* moe_spark_layer_forward without any allocation, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, kernels and results as
 * moe_spark_layer_forward (bit for bit), Q4_0 contexts only.  The per-token
 * scratch (router partial logits and squares, the layer's selection and
 * publish flag, the SwiGLU output) lives in a file-scope device array of
 * 576 KiB per GPU, held until the process ends, instead of the context's
 * buffers.  Every call on a GPU shares that GPU's array: calls that overlap
 * on one GPU (two streams, or two contexts) race and must be serialised by
 * the caller.  The call allocates nothing and calls no allocating routine.
 * Errors: E_INVALID for a non-Q4_0 context or a shape beyond the scratch
 * (more than 1024 experts, top_k > 8, d_ff > 512) and for the arguments
 * moe_spark_layer_forward rejects; E_STATE as moe_spark_layer_forward. */
moe_spark_status moe_spark_layer_forward_noalloc(moe_spark_ctx* ctx, int32_t layer, const float* x,
                                                 float* y, int32_t n_tokens, const int32_t* bias_row,
                                                 uint32_t flags, int32_t* topk_out, float* gates_out);

/* Decode n_tokens independent tokens through all L layers, one graph launch
 * per token: x_{l+1} = x_l + MoE_l(RMSNorm(x_l)).  x [T][d] fp32 device,
 * updated in place; bias_row [T] int32 device or NULL.  The graph for a given
 * (x, bias_row) pair is built once and replayed; n_tokens = 0 only builds it.
 * Passage: [Spark] "The key components" (3): the entire token as one graph
 * instead of one per layer; (2) for cold experts inside it.
 */
moe_spark_status moe_spark_decode(moe_spark_ctx* ctx, float* x, int32_t n_tokens,
                                  const int32_t* bias_row);

/* Batched decode: n_tokens independent tokens advance through all L layers
 * in steps of `batch` consecutive tokens (1 <= batch <= 16; the last step
 * takes what is left), one graph launch per step.  Each token computes
 * x_{l+1} = x_l + MoE_l(RMSNorm(x_l)) exactly as in moe_spark_decode, so its
 * outputs are bit-identical to batch-1 decode of the same token.  Serving
 * several requests at once is the use the pages' "The key components"
 * paragraph names for the engine; the expert cache is unchanged: within a
 * step the layer's accesses are made in (token, rank) order, token by token,
 * before the next layer's, and every counter, the fill log and the ring
 * follow from that order.  Each distinct expert of a layer-step is read once
 * for all the tokens that chose it.
 * With moe_spark_set_prefetch on, the next layer's predicted experts are
 * copied into ring entries the layer no longer needs, beside its GEMMs.
 * x [T][d] fp32 device, updated in place; bias_row [T] int32 device or NULL.
 * Q4_0 contexts only.  Below full residency the ring must hold a whole
 * step's accesses (ring_slots >= batch * top_k), so no expert a step uses is
 * evicted before the step has read it.  The graph for a given (x, bias_row,
 * batch) is built once and replayed; n_tokens = 0 only builds it.  Online
 * self-tuning (moe_spark_set_autotune) runs between steps.
 * Errors: E_INVALID (format, batch, ring size, n_tokens, x), E_STATE.
 * Passage: [Spark] "The key components" (3) and the engine's server use
 * (opening paragraph); the cache is (1)-(2) unchanged.
 */
moe_spark_status moe_spark_decode_batched(moe_spark_ctx* ctx, float* x, int32_t n_tokens, int32_t batch,
                                          const int32_t* bias_row);

/* moe_spark_decode with n_tokens = 1.
 * Passage: [Spark] "The key components" (3), one token.
 */
moe_spark_status moe_spark_token_forward(moe_spark_ctx* ctx, float* x, const int32_t* bias_row);

/* Batched prefill of n_tokens (1 <= n_tokens <= max_tokens) through all L
 * layers, Q4_0 contexts only.  Per layer: RMSNorm, router GEMM (fp32), exact
 * top-K with the softmax renormalised over the chosen experts, routing counts,
 * a deterministic sort of the (token, rank) assignments by expert, then a
 * grouped expert GEMM on the matrix cores: the Q4_0 codes as exact fp16
 * values q - 8, activations rounded once to fp16, fp32 accumulation, each
 * block's fp16 scale applied to the block's sum in fp32 (gate/up with SwiGLU,
 * then down); the rank-order combine adds the result to x.  The layer's distinct experts are
 * accessed once each in ascending id; non-pinned ones stream through the
 * spare-slot ring in chunks of at most R, filled as in moe_spark_create
 * describes (pulled during the pinned experts' GEMMs, or agent copies).
 * With moe_spark_set_prefetch on, the next layer's predicted experts are
 * copied into ring entries the layer no longer needs, beside its GEMMs.
 * x [T][d] fp32 device, updated in place; bias_row [T] int32 device or NULL.
 * Synchronises the compute stream once per layer (the host plans each layer
 * from its expert histogram).  Errors: E_INVALID (format, n_tokens, x),
 * E_STATE (max_tokens was 0 at create, weights or placement missing).
 * Passage: [Spark] opening paragraph (routing) and "The key components"
 * (1)-(2): the counts that calibration reads and the ring that streams the
 * cold experts.
 */
moe_spark_status moe_spark_prefill(moe_spark_ctx* ctx, float* x, int32_t n_tokens,
                                   const int32_t* bias_row);

/* Trace buffers (device, or NULL to stop tracing) filled by decode,
 * token_forward and prefill: x_layers [cap][L][d] fp32 (input of each layer),
 * topk [cap][L][K] int32, gates [cap][L][K] fp32.  Rows follow a trace cursor
 * that starts at 0 at this call and advances by one per decoded token and by
 * n_tokens per prefill batch; rows at or past cap are not written.
 * layer_forward traces token t of its call at row t, layer `layer`.
 * Passage: none of its own (observability for parity checks).
 */
moe_spark_status moe_spark_set_trace(moe_spark_ctx* ctx, float* x_layers, int32_t* topk,
                                     float* gates, int64_t cap_tokens);

/* Speculative prefetch in moe_spark_prefill (off at create; enable != 0
 * turns it on).  After layer l's routing, layer l+1's router applied to
 * layer l's input predicts layer l+1's top-K for every token; the predicted
 * experts that are neither pinned nor in the ring go, in ascending id, into
 * ring slots: at most R - (the layer's last chunk's non-pinned experts)
 * copies, chosen after that chunk's policy, so that no slot the chunk reads
 * or fills is taken.  The host hands these copies to the DMA engine on the
 * copy stream once layer l is queued; they run beside the rest of layer l
 * and layer l+1's routing, and layer l+1's first launch that touches slot
 * data waits for them.  A prefetch is not an access: routing counts and
 * the access counters do not change; it is counted in stats.prefetches and
 * logged with kind MOE_SPARK_EV_PREFETCH.  Outputs do not change.
 * Errors: E_STATE when fills are copied by the host agent
 * (MOE_SPARK_PULL_FILLS=0) or max_tokens was 0 at create.
 * Passage: none describes a prefetch; [Bagua] "Actionable Advice" names the
 * swap latency between system RAM and the GPU as the bottleneck, and this
 * moves part of it under the matrix-core work.
 */
moe_spark_status moe_spark_set_prefetch(moe_spark_ctx* ctx, int32_t enable);

/* The prediction histograms of the last moe_spark_prefill with prefetch on:
 * out [L][E] int32 host, row l = predicted assignments per expert of layer l
 * (row 0 and rows of a prefill without prefetch are zero).
 * Passage: as moe_spark_set_prefetch.
 */
moe_spark_status moe_spark_get_prefetch_hist(moe_spark_ctx* ctx, int32_t* out);

/* Copy the counters (see moe_spark_stats) to host memory after waiting for
 * the compute stream; reset_stats zeroes them.
 * Passage: [Spark] "The key components" (1): the cold-hit rate ("36% to ~7%")
 * is cold_hits / accesses; [Bagua] "Actionable Advice": fills and their
 * bytes are the swap traffic between system RAM and the GPU.
 */
moe_spark_status moe_spark_get_stats(moe_spark_ctx* ctx, moe_spark_stats* out);
/* Passage: as moe_spark_get_stats. */
moe_spark_status moe_spark_reset_stats(moe_spark_ctx* ctx);

/* Host outputs (each may be NULL): slot_of [L][E] (pinned slot or -1),
 * ring_owner [R] (layer*E+expert or -1), ring_stamp [R] (LRU clock),
 * counts [L][E].
 * Passage: [Spark] "The key components" (1)-(2): the pinned set, the ring
 * and the routing frequencies.
 */
moe_spark_status moe_spark_get_placement(moe_spark_ctx* ctx, int32_t* slot_of,
                                         int32_t* ring_owner, int64_t* ring_stamp,
                                         int64_t* counts);

/* Copy up to cap fill events (oldest first) to host memory; *n_total gets
 * the number logged (events past event_cap are counted, not stored).
 * Passage: [Spark] "The key components" (2): every copy into a spare slot
 * and the LRU entry it evicted.
 */
moe_spark_status moe_spark_get_events(moe_spark_ctx* ctx, moe_spark_event* out, int64_t cap,
                                      int64_t* n_total);

/* Wait for all work of the context; report device-side errors.
 * Passage: [Spark] "The key components" (2): a fill costs throughput but
 * never stalls; one that never lands is reported here, not waited for.
 */
moe_spark_status moe_spark_synchronize(moe_spark_ctx* ctx);

/* Time the decode kernels in isolation: replays the gate/up and down kernels
 * of every layer with each layer's last published selection (no placement
 * policy, no fills), round-robin over layers, `iters` passes, bracketed by
 * HIP events on the compute stream.  Outputs microseconds per launch:
 * us_gateup (for Q4_0: router-partial reduce + top-k + gate/up GEMV + SwiGLU),
 * us_down (down GEMV + combine + residual + next layer's router partials) and
 * us_route (Q4_0: the first layer's router-partial kernel; fp32: -1).
 * Writes only context scratch buffers.  Call between tokens.
 * Passage: none of its own (measures the expert kernels against HBM
 * bandwidth).
 */
moe_spark_status moe_spark_time_expert_kernels(moe_spark_ctx* ctx, int32_t iters,
                                               float* us_gateup, float* us_down,
                                               float* us_route);

/* Time a bare streaming read shaped like one batch-1 gate/up launch: the same
 * grid and the same non-temporal 16-byte loads, over the gate and up rows of
 * slots 0..top_k-1 (top_k x 1,179,648 B for the target shape), with no
 * routing and no arithmetic beyond folding the words together; `iters`
 * back-to-back launches bracketed by HIP events on the compute stream.
 * Output: microseconds per launch (*us).  This is the ceiling that the
 * gate/up launch's weight phase runs against on this chip.  Q4_0 only
 * (E_INVALID otherwise); E_STATE if the context has fewer than top_k slots.
 * Writes only context scratch.  Call between tokens.
 * Passage: none of its own (a measurement of the chip, not of the method).
 */
moe_spark_status moe_spark_time_stream_probe(moe_spark_ctx* ctx, int32_t iters, float* us);

#ifdef __cplusplus
}
#endif
#endif
