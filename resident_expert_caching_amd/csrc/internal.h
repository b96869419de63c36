// Internal definitions shared by the host runtime and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_spark.h"

namespace moe {

constexpr int kMaxK = 16;        // largest top-k
constexpr int kMaxE = 1024;      // largest expert count
constexpr int kMaxR = 1024;      // largest ring
constexpr int kQ4MaxK = 8;       // Q4_0 down kernel covers up to 8 experts per pass
constexpr uint32_t kFifoCap = 4096;

// Q4_0 target shape of the repacked GEMV kernels.
constexpr int kQD = 2048;        // d
constexpr int kQF = 512;         // f
constexpr int kQNBD = kQD / 32;  // 64 blocks along d (one per lane)
constexpr int kQNBF = kQF / 32;  // 16 blocks along f
// Gate/up: a work-group owns 16 rows of gate and the same 16 rows of up.
constexpr int kGURows = 16;
constexpr int64_t kGUChunk = 4 * 8 * 64 * 16 + 4 * 64 * 16;        // 36,864 B
constexpr int64_t kGURegion = (kQF / kGURows) * kGUChunk;          // 1,179,648 B
constexpr int64_t kDownCodes = (int64_t)kQD * kQNBF * 16;          // 524,288 B
constexpr int64_t kDownScales = (int64_t)kQD * kQNBF * 2;          // 65,536 B
constexpr int64_t kQ4SlotBytes = kGURegion + kDownCodes + kDownScales;  // 1,769,472 B
constexpr int kDownRowsPerWG = 8;
// Router partial logits: a work-group owns kRW consecutive rows of x and
// writes the router dot products restricted to those rows for every expert.
// Streams the fill agent spreads ring fills over (the caller's copy stream and
// kCopyStreams - 1 of the context's own).
constexpr int kCopyStreams = 2;

constexpr int kRW = 16;
constexpr int kNP = kQD / kRW;   // 128 partial rows

// Device statistics counters (int64 each).
enum DevStat { DS_ACC = 0, DS_PIN, DS_COLD, DS_RING, DS_FILL, DS_EVICT, DS_H2D, DS_TOKENS, DS_PREF, DS_N };

// Error bits.
enum DevError { ERR_FILL_TIMEOUT = 1, ERR_FIFO_OVERRUN = 2, ERR_BAD_SLOT = 4 };

// One fill request, written by the route kernel into host-mapped memory.
// A copy request for the host fill agent.  Requests are numbered on their own
// (fills the decode kernels copy themselves post none), and each carries the
// fill number that the slot's ready flag must reach.
struct FifoEntry {
    uint64_t seq;   // request number, written last; 0 = empty
    int32_t key;    // layer*E + expert (index into the host arena)
    int32_t ring;   // ring slot index 0..R-1
    uint64_t fill;  // fill number: ready[ring] is set to it once the copy has landed
};

// Routing decision of one layer for the current token.
struct LayerSel {
    int32_t idx[kMaxK];
    int32_t slot[kMaxK];
    float gate[kMaxK];
    uint64_t wait[kMaxK];  // fill sequence number to wait for (0: data already resident)
    float inv_rms;
    int32_t pad[3];
};

// Token index: base + *ptr (ptr may be null).
struct TokRef {
    const int32_t* ptr;
    int32_t base;
};

struct PolicyTables {
    int32_t* slot_of;      // [L*E]
    int32_t* ring_owner;   // [R]
    uint64_t* ring_stamp;  // [R]
    uint64_t* ring_seq;    // [R] fill number of the current content
    uint64_t* clock;       // LRU clock
    uint64_t* fill_seq;    // fills issued
    uint64_t* req_seq;     // copy requests posted to the host fill agent
    int64_t* counts;       // [L*E]
    int64_t* stats;        // [DS_N]
    moe_spark_event* events;
    int64_t* n_events;
    int64_t event_cap;
    FifoEntry* fifo;       // host-mapped, device address
    int32_t* error;
    int64_t P;
    int32_t R;
    int32_t E;
    int64_t slot_bytes;
    int32_t pull;          // 1: decode kernels copy their fills from the host arena themselves
};

struct RouteArgs {
    const float* x_base;   // [T][d]
    TokRef tok;            // selects x and bias row
    TokRef trace_tok;      // selects the trace row
    int32_t d, E, K, layer, L, norm;
    float eps;
    const float* wr;       // [E][d]
    const float* bias;     // [rows][E] or null
    const int32_t* bias_row;  // [T] or null
    int32_t n_bias_rows;
    float* logits;         // scratch [E]
    uint32_t* done;        // last-block counter
    LayerSel* sel;
    float* u;              // [d] normalised input
    float* ut;             // Q4_0 path: [8][64] float4, ut[j*64+b] = u[32b+4j .. +3]
    PolicyTables pt;
    float* tr_x;           // [cap][L][d] or null
    int32_t* tr_topk;      // [cap][L][K] or null
    float* tr_gates;
    int64_t tr_cap;
    int32_t* topk_out;     // [T][K] or null (indexed by tok)
    float* gates_out;
    int32_t q4;            // write ut
};

struct ExpertArgs {
    const uint8_t* slots;  // slot arena
    int64_t slot_bytes;
    const LayerSel* sel;
    const uint64_t* ready; // host-mapped [R] ready flags (device address)
    int64_t P;
    int64_t n_slots;       // P + R: slot ids outside [0, n_slots) are refused
    int32_t R;
    int32_t d, f, K;
    const float* u;        // [d]
    const float* ut;       // transposed u (Q4_0)
    float* h;              // [K][f]; Q4_0: transposed per expert, see kernels
    // down only
    const float* x_base;   // residual input [T][d]
    float* y_base;         // output [T][d]
    TokRef tok;
    int32_t residual;
    int32_t advance;       // last layer of a decode token: bump the cursors
    int32_t* cursors;      // [2]: x cursor, trace cursor
    uint32_t* done;        // last-block counter (advance only)
    int64_t* stats;
    int32_t* error;
    uint64_t spin_limit_ticks;  // fill wait limit, in wall-clock ticks (100 MHz)
};

// Arguments of the Q4_0 decode kernels (q4_decode.hip).  Per token-layer:
// gate/up (reduce router partials, top-k, policy, gate/up GEMV + SwiGLU),
// then down (down GEMV, gate-weighted combine, residual, router partials of
// the next layer).  The first layer's partials come from the router-partial
// kernel.
struct Q4Args {
    const float* x_base;     // [T][d] layer input (residual)
    float* y_base;           // [T][d] layer output (may equal x_base)
    TokRef tok;
    TokRef trace_tok;
    int32_t layer, L, E, K;
    int32_t norm;            // RMSNorm before router and experts
    int32_t residual;        // y = x + MoE
    int32_t replay;          // timing replay: reuse the published selection, no policy
    float eps;
    float* pl;               // [kNP][E] router partial logits
    float* ps;               // [kNP] partial sums of squares
    const float* wr_part;    // packed router [kNP][E][kRW] whose partials this kernel writes, or null
    const float* bias;       // this layer's router bias [n_bias_rows][E] or null
    const int32_t* bias_row; // [T] or null
    int32_t n_bias_rows;
    uint8_t* slots;          // slot arena (written by pulled fills)
    const uint8_t* arena;    // pinned host arena (device address): the source of pulled fills
    int64_t slot_bytes, P, n_slots;
    const uint64_t* ready;   // host-mapped ring ready flags (device address)
    LayerSel* sel;           // this layer's published selection
    uint32_t* pub;           // this layer's publish flag
    float* h;                // [K][f] in the down kernel's transposed layout
    PolicyTables pt;
    float* tr_x;
    int32_t* tr_topk;
    float* tr_gates;
    int64_t tr_cap;
    int32_t* topk_out;
    float* gates_out;
    uint64_t spin_limit_ticks;
};

// Token staging of the Q4_0 decode graph (q4_decode.hip).
struct TokenIO {
    float* x;                  // caller's [T][d] tokens
    const int32_t* bias_row;   // caller's [T] router-bias rows or null
    float* xbuf;               // [d] the current token
    int32_t* tokrow;           // [1] its bias row
    int32_t* cursors;          // [2] token cursor, trace cursor
    int32_t* ntok;             // [1] tokens of this decode call
    int64_t* stats;
};
hipError_t launch_token_begin(const TokenIO& io, int32_t n_tokens, hipStream_t s);
hipError_t launch_token_end(const TokenIO& io, hipStream_t s);

hipError_t launch_q4_router_partial(const Q4Args& a, hipStream_t s);
hipError_t launch_q4_gateup(const Q4Args& a, hipStream_t s);
hipError_t launch_q4_down(const Q4Args& a, hipStream_t s);
// slots 0..K-1 read as one gate/up launch reads its experts; out[(f/16) * K]
hipError_t launch_q4_stream_probe(const uint8_t* slots, int64_t slot_bytes, int32_t K, uint32_t* out, hipStream_t s);
hipError_t launch_advance(int32_t* cursors, int64_t* stats, hipStream_t s);

// Batched decode (qb_decode.hip): B tokens advance through the stack together,
// one step at a time.  Per layer: a route launch (router, top-k and gates per
// token), then gate/up and down launches that stream each distinct expert once
// for all the tokens that chose it (matrix-core skinny GEMMs).  Gate/up groups
// the accesses by distinct expert, and its work-group (0,0) runs the placement
// policy over them in (token, rank) order; down also does the rank-order
// combine, the residual and the next layer's router partials.
constexpr int kMaxB = 16;                 // tokens per step
constexpr int kMaxBK = kMaxB * kQ4MaxK;   // accesses per layer-step

// Routing and placement of one layer for the current step.  Accesses are
// numbered i = b*K + k; distinct experts j = 0..D-1 ascend by expert id and
// own the accesses dent[doff[j] .. doff[j+1]) in ascending i.
struct BatchSel {
    int32_t idx[kMaxBK];
    float gate[kMaxBK];
    int32_t slot[kMaxBK];    // route: the expert's pinned slot or -1; gate/up (0,0): the slot the access reads
    int32_t D;
    int32_t pad0;
    int32_t dexp[kMaxBK];
    int32_t dslot[kMaxBK];
    uint64_t dwait[kMaxBK];  // fill number to wait for or pull (0: resident)
    int32_t doff[kMaxBK + 1];
    int32_t dent[kMaxBK];
};

struct QBArgs {
    int32_t layer, L, E, K;
    int32_t B;                // step capacity: the grid's token dimension
    const int32_t* nb;        // tokens in the current step (device, 1..B)
    float* xb;                // [B][d] the step's tokens: layer input, updated in place
    const int32_t* rows;      // [B] their router-bias rows
    int32_t norm;
    float eps;
    float* pl;                // [B][kNP][E] router partial logits
    float* ps;                // [B][kNP] partial sums of squares
    const float* wr_part;     // packed router [kNP][E][kRW] whose partials the launch writes, or null
    const float* bias;        // this layer's router bias [n_bias_rows][E] or null
    int32_t n_bias_rows;
    uint16_t* u16;            // [B][d] normalised input, fp16 bits
    uint8_t* slots;
    const uint8_t* arena;
    int64_t slot_bytes, P, n_slots;
    const uint64_t* ready;
    BatchSel* sel;            // this layer's routing and placement
    uint32_t* pub;            // this layer's flag: slots of cold experts published
    uint16_t* h16;            // [B*K][f] SwiGLU output, fp16 bits: row doff[j] + m is distinct expert j's m-th access
    PolicyTables pt;
    float* tr_x;              // traces: token b of the step goes to row *trace_base + b
    int32_t* tr_topk;
    float* tr_gates;
    int64_t tr_cap;
    const int32_t* trace_base;
    uint64_t spin_limit_ticks;
};

// Token staging of the batched decode graph.
struct BatchIO {
    float* x;                 // caller's [T][d] tokens
    const int32_t* bias_row;  // caller's [T] router-bias rows or null
    float* xb;                // [B][d] the step's tokens
    int32_t* rows;            // [B] their bias rows
    int32_t* nb;              // [1] tokens in the step
    int32_t* cursors;         // [2] first token of the step, trace cursor
    int32_t* ntok;            // [1] tokens of this decode call
    int64_t* stats;
    int32_t B;
};

hipError_t launch_qb_begin(const BatchIO& io, int32_t n_tokens, hipStream_t s);
hipError_t launch_qb_end(const BatchIO& io, hipStream_t s);
hipError_t launch_qb_router_partial(const QBArgs& a, hipStream_t s);
hipError_t launch_qb_route(const QBArgs& a, hipStream_t s);
hipError_t launch_qb_gateup(const QBArgs& a, hipStream_t s);
hipError_t launch_qb_down(const QBArgs& a, hipStream_t s);

// Arguments of the batched-prefill kernels (prefill.hip), one layer.
struct PfArgs {
    float* x;                 // [T][d] residual stream, updated in place
    int32_t T, layer, L, E, K;
    int32_t norm;
    float eps;
    const float* wr;          // this layer's packed router [kNP][E][kRW]
    const float* bias;        // this layer's router bias [n_bias_rows][E] or null
    const int32_t* bias_row;  // [T] or null
    int32_t n_bias_rows;
    uint16_t* u;              // [T][d/32][32] normalised input per Q4_0 block, fp16 in operand order
    float* inv;               // [T] 1 / rms
    float* logits;            // [T][E]
    int32_t* topk;            // [T][K]
    float* gates;             // [T][K]
    int32_t* hist;            // [E] assignments per expert (zeroed before the routing launches)
    // prediction for the prefetch (all null without it): the next layer's
    // router applied to this layer's input, its top-K counted per expert
    const float* wr2;         // the next layer's packed router
    const float* bias2;       // the next layer's router bias or null
    float* logits2;           // [T][E]
    int32_t* topk2;           // [T][K] the predicted top-K
    int32_t* hist2;           // [E] predicted assignments per expert of the next layer
    int32_t* pfill2;          // [1 + 2 kMaxR] the prefetch copies: count, then (arena key, slot) pairs
    int32_t pf_budget;        // prefetch launch after the last chunk: copies at most this many
    // mapped host mirror that the first-chunk policy fills for the host
    // (device address, or null): [0] histogram flag, [1] lists flag, then
    // hist [E], the fill list [1 + 2 kMaxR], the prefetch list [1 + 2 kMaxR];
    // a flag takes the value `seq` once what it covers is written
    int32_t* host_state;
    int32_t seq;
    const int32_t* goff;      // [E+1] first sorted position of each expert's group
    // the host's plan (goff | experts | items, n_meta ints) in mapped host
    // memory: the scatter launch reads goff there and copies the whole plan
    // to the device buffer that goff points into (or null: already there)
    const int32_t* meta_host;
    int32_t n_meta;
    int32_t* perm;            // [T*K] token of each sorted position
    int32_t* apos;            // [T][K] sorted position of assignment (t, k)
    const int32_t* items;     // [n_items][2] GEMM work items: (expert, first row of the tile)
    int32_t n_items;
    const int32_t* pf_experts;  // the chunk's experts, ascending, for the policy
    int32_t n_pf_experts;
    int32_t* pslot;           // [E] slot chosen for each expert this layer
    uint64_t* pwait;          // [E] fill number to wait for (0: resident, or pulled)
    const uint8_t* arena;     // pinned host arena (device address) when the fill kernel pulls fills, else null
    int32_t* pfill;           // [1 + 2 kMaxR]: the last policy run's fill count, then (arena key, slot) pairs
    int32_t n_fill_x;         // gate/up and down launches: leading grid columns that pull those fills (0: none)
    uint16_t* h;              // [T*K][f/32][32] SwiGLU output per Q4_0 block, fp16 in operand order
    float* y;                 // [T*K][d] expert outputs
    uint8_t* slots;           // slot arena (written by pulled fills)
    int64_t slot_bytes, P, n_slots;
    const uint64_t* ready;
    PolicyTables pt;
    float* tr_x;              // traces: token t goes to row *tr_base + t
    int32_t* tr_topk;
    float* tr_gates;
    int64_t tr_cap;
    const int32_t* tr_base;   // the context's trace cursor
    uint64_t spin_limit_ticks;
};

// norm, router, top-k + counts + histogram (with a.hist2: also the
// prediction of the next layer's top-K)
hipError_t launch_pf_front(const PfArgs& a, hipStream_t s);
// the first chunk's policy (with a.hist2 and a one-chunk layer: then the
// prefetch rule)
hipError_t launch_pf_policy_first(const PfArgs& a, hipStream_t s);
hipError_t launch_pf_scatter(const PfArgs& a, hipStream_t s);  // sort assignments by (expert, token)
hipError_t launch_pf_policy(const PfArgs& a, hipStream_t s);   // a chunk's experts through the placement policy
// gate/up GEMM and down GEMM over a list of work items, each launch with
// n_fill_x leading grid columns of work-groups pulling a share of the last
// policy run's fills
hipError_t launch_pf_gemms(const PfArgs& a, hipStream_t s);
hipError_t launch_pf_combine(const PfArgs& a, hipStream_t s);  // rank-order combine + residual
// after a layer's last chunk: the experts of layer a.layer + 1 with
// a.hist2 > 0 (ascending) through the prefetch rule, at most a.pf_budget
// copies, listed in a.pfill2
hipError_t launch_pf_prefetch(const PfArgs& a, hipStream_t s);
hipError_t launch_cursor_add(int32_t* cursor, int32_t n, hipStream_t s);
hipError_t prepare_pf_kernels();  // resolve the prefill kernels before their first launch

// Launchers (kernels.hip).
hipError_t launch_route(const RouteArgs& a, hipStream_t s);
hipError_t launch_gateup(const ExpertArgs& a, int wfmt, hipStream_t s);
hipError_t launch_down(const ExpertArgs& a, int wfmt, hipStream_t s);

}  // namespace moe
