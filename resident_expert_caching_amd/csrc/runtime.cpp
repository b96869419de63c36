// Host runtime of the moe_spark C ABI: arenas, weight repacking, placement
// (uniform and calibrated), the fill agent that serves cold-expert copies,
// eager layer forward, and the whole-token decode graph.
//
// Method: "Luce Spark runs 35B MoE models on 16GB GPU without speed loss"
// (theneuralfeed.com), paragraph "The key components":
//  (1) calibrated placement pins the most-used experts — moe_spark_calibrate;
//  (2) a fixed ring of spare GPU slots, filled on a cold hit by an
//      asynchronous copy from pinned host memory while the LRU entry is
//      evicted — the route kernel decides (device tables), the fill agent
//      thread below issues hipMemcpyAsync on the copy stream and publishes a
//      ready flag that only the work-groups needing that slot wait for;
//  (3) the entire token runs as one graph — moe_spark_decode captures all
//      layers' kernels once per (x, bias_row) and replays the graph per token;
//      placement lives in device tables, so the graph never needs recapture.
#include <hip/hip_runtime.h>
#include <immintrin.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <cstdlib>
#include <deque>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "internal.h"
#include "moe_spark.h"

using namespace moe;

namespace {

constexpr int kThrottle = 8;  // decode tokens in flight at most
constexpr int kPfFillCols = 8;  // prefill: grid columns of fill work-groups in a gate/up launch (x 8 rows)

struct GraphEntry {
    float* x = nullptr;
    const int32_t* bias_row = nullptr;
    int32_t batch = 0;  // 0: batch-1 token graph; B: batched step graph
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

int64_t now_ns() {
    return std::chrono::duration_cast<std::chrono::nanoseconds>(
               std::chrono::steady_clock::now().time_since_epoch())
        .count();
}

}  // namespace

// Device scratch of moe_spark_layer_forward_noalloc: the per-token buffers of
// the Q4_0 layer kernels (router partial logits and squares, the layer's
// selection and publish flag, the SwiGLU output), in a file-scope device
// array so that the call allocates nothing.  Each GPU holds its own copy until
// the process ends; host code uses the per-device address that
// hipGetSymbolAddress returns (the array's name is only a host-side stand-in).
namespace {
constexpr size_t kNoAllocPL = 0;                                          // float [kNP][kMaxE]
constexpr size_t kNoAllocPS = kNoAllocPL + sizeof(float) * kNP * kMaxE;     // float [kNP]
constexpr size_t kNoAllocSel = kNoAllocPS + sizeof(float) * kNP;           // LayerSel
constexpr size_t kNoAllocPub = kNoAllocSel + 512;                          // uint32_t
constexpr size_t kNoAllocH = kNoAllocPub + 256;                            // float [kQ4MaxK][kQF]
constexpr size_t kNoAllocUsed = kNoAllocH + sizeof(float) * kQ4MaxK * kQF;
constexpr size_t kNoAllocScratchBytes = 576 * 1024;
static_assert(sizeof(LayerSel) <= 512, "selection fits its scratch slot");
static_assert(kNoAllocUsed <= kNoAllocScratchBytes, "no-alloc scratch layout fits the array");
constexpr int kMaxDevices = 64;
uint8_t* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;
}  // namespace

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
// Once per device, with that device current: the device address of this
// GPU's copy of the scratch array.
hipError_t scratch_init(int device) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[device]) return hipSuccess;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[device] = static_cast<uint8_t*>(ptr);
    return hipSuccess;
}

uint8_t* scratch_of(int device) {
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    return g_scratch[device];
}

// Zero a flag with a kernel (a memset node would not replay reliably inside
// a captured graph).
__global__ void noalloc_clear_kernel(uint32_t* flag) {
    if (threadIdx.x == 0) *flag = 0u;
}
}  // namespace

struct moe_spark_ctx {
    moe_spark_config cfg{};
    int device = 0;
    int64_t slot_bytes = 0;
    int64_t n_slots = 0;  // P + R
    int64_t n_experts_total = 0;
    hipStream_t compute = nullptr, copy = nullptr;
    bool own_compute = false, own_copy = false;
    // fills of ring slot r go to copy_streams[r % kCopyStreams]: copies into one
    // slot stay ordered, copies into different slots use several DMA engines
    hipStream_t copy_x[kCopyStreams - 1] = {};

    uint8_t* d_slots = nullptr;
    uint8_t* h_arena = nullptr;
    const uint8_t* d_arena = nullptr;  // the host arena's device address (pulled decode fills)
    bool pull_fills = false;           // Q4_0 decode kernels copy their own fills
    float* d_router = nullptr;
    float* d_bias = nullptr;

    // device tables
    int32_t* d_slot_of = nullptr;
    int32_t* d_ring_owner = nullptr;
    uint64_t* d_ring_stamp = nullptr;
    uint64_t* d_ring_seq = nullptr;
    uint64_t* d_clock = nullptr;  // [3]: clock, fill_seq, req_seq
    int64_t* d_counts = nullptr;
    int64_t* d_stats = nullptr;
    moe_spark_event* d_events = nullptr;
    int64_t* d_n_events = nullptr;
    int32_t* d_error = nullptr;
    int32_t* d_cursors = nullptr;   // [2]
    uint32_t* d_done = nullptr;     // [2*L + 4] last-block counters
    LayerSel* d_sel = nullptr;      // [L] + 1 scratch
    float* d_logits = nullptr;      // [E]
    float* d_u = nullptr;           // [d]
    float* d_ut = nullptr;          // [d]
    float* d_h = nullptr;           // [kMaxK * f]
    float* d_xscratch = nullptr;    // [d]
    float* d_pl = nullptr;          // [kNP][E] router partial logits (Q4_0)
    float* d_ps = nullptr;          // [kNP] partial sums of squares (Q4_0)
    uint32_t* d_pub = nullptr;      // [L] selection-published flags (Q4_0)
    float* d_xbuf = nullptr;        // [d] token staged for the Q4_0 decode graph
    int32_t* d_tokrow = nullptr;    // [1] its router-bias row
    int32_t* d_ntok = nullptr;      // [1] tokens of the current decode call

    // batched decode (Q4_0): the step's tokens and their routing
    float* d_bx = nullptr;          // [kMaxB][d]
    int32_t* d_brows = nullptr;     // [kMaxB]
    int32_t* d_bn = nullptr;        // [1] tokens in the current step
    float* d_bpl = nullptr;         // [kMaxB][kNP][E]
    float* d_bps = nullptr;         // [kMaxB][kNP]
    uint16_t* d_bu16 = nullptr;     // [kMaxB][d] fp16
    BatchSel* d_bsel = nullptr;     // [L]
    uint32_t* d_bpub = nullptr;     // [L] cold-slot publish flags
    uint16_t* d_bh16 = nullptr;     // [kMaxBK][f] fp16

    // batched prefill (allocated when max_tokens > 0)
    uint16_t* d_pu = nullptr;       // [Tmax][d/32][32] fp16 per Q4_0 block
    float* d_pinv = nullptr;        // [Tmax]
    float* d_plog = nullptr;        // [Tmax][E]
    bool pf_prefetch = false;         // prefill: speculative prefetch of the next layer's predicted experts
    hipEvent_t pf_q_ev = nullptr;     // prefetch list written (compute stream)
    hipEvent_t pf_done_ev = nullptr;  // prefetch copies landed (side stream)
    int32_t* d_ptopk = nullptr;     // [Tmax][K]
    float* d_pgate = nullptr;       // [Tmax][K]
    int32_t* d_phist = nullptr;     // [E]
    float* d_plog2 = nullptr;       // [T][E] the next layer's router logits (prefetch prediction)
    int32_t* d_ptopk2 = nullptr;    // [T][K] the next layer's predicted top-K
    int32_t* d_ppred = nullptr;     // [L][E] predicted assignments of layer l (row 0 stays zero), last prefill
    int32_t* d_pperm = nullptr;     // [Tmax*K]
    int32_t* d_papos = nullptr;     // [Tmax][K]
    int32_t* d_pslot = nullptr;     // [E]
    uint64_t* d_pwait = nullptr;    // [E]
    int32_t* d_pfill = nullptr;     // [1 + 2 kMaxR] the prefill policy's pulled fills
    int32_t* d_pfill2 = nullptr;    // [1 + 2 kMaxR] the prefetch copies
    uint16_t* d_ph = nullptr;       // [Tmax*K][f/32][32] fp16 per Q4_0 block
    float* d_py = nullptr;          // [Tmax*K][d]
    int32_t* d_pmeta = nullptr;     // goff [E+1] | experts [E] | items [2*max_items]
    int32_t* h_pmeta = nullptr;     // the host's plan, mapped coherent (the scatter launch copies it over)
    int32_t* dm_pmeta = nullptr;    // its device address
    int32_t* h_pfill2 = nullptr;    // pinned copy of d_pfill2 (prefetch list of a layer of several chunks)
    // mapped coherent host mirror the first-chunk policy writes (PfArgs::host_state):
    // [0] histogram flag, [1] lists flag, hist [E], fill list, prefetch list
    int32_t* h_pstate = nullptr;
    int32_t* d_pstate = nullptr;    // its device address
    int32_t pf_seq = 0;             // last flag value
    int64_t pf_max_items = 0;

    // host-mapped
    FifoEntry* h_fifo = nullptr;
    FifoEntry* d_fifo = nullptr;
    uint64_t* h_ready = nullptr;
    uint64_t* d_ready = nullptr;

    // host mirrors / state
    std::vector<uint8_t> router_set, expert_set;
    int64_t n_router_set = 0, n_expert_set = 0;
    bool placed = false;
    std::vector<int32_t> slot_of;  // host copy of the placement

    float* tr_x = nullptr;
    int32_t* tr_topk = nullptr;
    float* tr_gates = nullptr;
    int64_t tr_cap = 0;

    std::vector<GraphEntry> graphs;
    hipEvent_t tok_ev[kThrottle] = {};
    int64_t tok_launched = 0;
    uint64_t spin_ticks = 0;
    bool stream_decode = false;  // MOE_SPARK_DECODE_STREAM=1: per-kernel launches instead of the token graph
    // Streams the fill agent may spread a burst of fills over in decode: all
    // kCopyStreams (a lone fill still takes the first; the calibrated decode
    // runs the same with one or two, a fill-heavy one 30% faster with two).
    // Prefill always uses all of them.  MOE_SPARK_COPY_STREAMS=1..kCopyStreams
    // sets the decode figure.
    int n_copy = kCopyStreams;
    std::atomic<int> burst_fills{0};
    // prefill with pulled fills: grid columns of fill work-groups in a gate/up
    // launch (x 8 rows); MOE_SPARK_FILL_COLS=1..128 at creation
    int pf_fill_cols = kPfFillCols;

    // fill agent
    std::thread agent;
    std::atomic<bool> stop{false};
    std::atomic<int64_t> fill_ns_sum{0}, fill_ns_max{0};
    std::atomic<int> agent_error{0};
    std::string agent_msg;
    int64_t calib_uploads = 0;
    // online self-tuning (moe_spark_set_autotune)
    int32_t at_interval = 0, at_hyst = 0, at_shift = 0;
    int64_t at_since = 0;  // decoded tokens since the placement last changed
    int64_t retunes = 0, retune_swaps = 0;

    std::string err;

    moe_spark_status fail(moe_spark_status st, const char* fmt, ...) {
        char buf[512];
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(buf, sizeof buf, fmt, ap);
        va_end(ap);
        err = buf;
        return st;
    }
};

#define HIPCHK(call)                                                                           \
    do {                                                                                       \
        hipError_t e_ = (call);                                                                \
        if (e_ != hipSuccess)                                                                  \
            return ctx->fail(MOE_SPARK_E_HIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
    } while (0)

namespace {

thread_local std::string g_create_err;

// ---------------------------------------------------------------- repacking

// GGUF Q4_0 (gate, up [f][d/32][18]; down [d][f/32][18]) -> slot layout read
// by the Q4_0 kernels (values unchanged, only moved).
void repack_q4(const uint8_t* gate, const uint8_t* up, const uint8_t* down, uint8_t* dst) {
    for (int g = 0; g < kQF / kGURows; ++g) {
        uint8_t* chunk = dst + (int64_t)g * kGUChunk;
        for (int w = 0; w < 4; ++w) {
            const uint8_t* mat = (w >> 1) ? up : gate;
            for (int i = 0; i < 8; ++i) {
                const int row = g * kGURows + (w & 1) * 8 + i;
                for (int b = 0; b < kQNBD; ++b) {
                    const uint8_t* blk = mat + ((int64_t)row * kQNBD + b) * 18;
                    memcpy(chunk + ((int64_t)(w * 8 + i) * 64 + b) * 16, blk + 2, 16);
                    memcpy(chunk + 32768 + (int64_t)(w * 64 + b) * 16 + i * 2, blk, 2);
                }
            }
        }
    }
    uint8_t* dc = dst + kGURegion;
    uint8_t* ds = dc + kDownCodes;
    for (int r = 0; r < kQD; ++r) {
        for (int b = 0; b < kQNBF; ++b) {
            const uint8_t* blk = down + ((int64_t)r * kQNBF + b) * 18;
            memcpy(dc + (int64_t)r * 256 + b * 16, blk + 2, 16);
            memcpy(ds + ((int64_t)(r >> 2) * 16 + b) * 8 + (r & 3) * 2, blk, 2);
        }
    }
}

int64_t matrix_bytes(int rows, int cols, int wfmt) {
    return wfmt == MOE_SPARK_W_F32 ? (int64_t)rows * cols * 4 : (int64_t)rows * (cols / 32) * 18;
}

void pack_expert(const moe_spark_ctx* ctx, const void* gate, const void* up, const void* down,
                 uint8_t* dst) {
    const int d = ctx->cfg.d_model, f = ctx->cfg.d_ff;
    if (ctx->cfg.wfmt == MOE_SPARK_W_Q4_0) {
        repack_q4((const uint8_t*)gate, (const uint8_t*)up, (const uint8_t*)down, dst);
    } else {
        const int64_t mb = (int64_t)f * d * 4;
        memcpy(dst, gate, mb);
        memcpy(dst + mb, up, mb);
        memcpy(dst + 2 * mb, down, (int64_t)d * f * 4);
    }
}

int64_t quota(int L, int64_t P, int l) { return P / L + ((int64_t)l < P % L ? 1 : 0); }

// ---------------------------------------------------------------- fill agent

hipStream_t copy_stream_at(const moe_spark_ctx* ctx, int i) { return i == 0 ? ctx->copy : ctx->copy_x[i - 1]; }

hipError_t sync_copies(const moe_spark_ctx* ctx) {
    hipError_t e = ctx->copy ? hipStreamSynchronize(ctx->copy) : hipSuccess;
    for (hipStream_t st : ctx->copy_x)
        if (st) {
            const hipError_t f = hipStreamSynchronize(st);
            if (e == hipSuccess) e = f;
        }
    return e;
}

void agent_loop(moe_spark_ctx* ctx) {
    hipSetDevice(ctx->device);
    struct Pending {
        uint64_t seq;
        int ring;
        hipEvent_t ev;
        int stream;
        int64_t t0;
        bool flagged;  // the copy stream itself writes the ready flag after the copy
    };
    std::deque<Pending> pend;
    // Stream choice: a ring slot with a copy in flight keeps that copy's
    // stream, so one slot's fills finish in order; otherwise the first stream
    // unless it is busy, then the least busy one.  A lone fill therefore
    // always takes the first stream; only bursts spread over the others.
    std::vector<int> ring_stream(std::max(ctx->cfg.ring_slots, 1), -1), ring_pending(ring_stream.size(), 0);
    int stream_pending[kCopyStreams] = {};
    auto pick = [&](int ring) {
        if (ring_pending[ring] > 0) return ring_stream[ring];
        int best = 0;
        const int nc = !ctx->copy_x[0] ? 1  // the extra streams exist only without pulled fills
                       : ctx->burst_fills.load(std::memory_order_relaxed) ? kCopyStreams
                                                                           : ctx->n_copy;
        for (int i = 1; i < nc && stream_pending[best] > 0; ++i)
            if (stream_pending[i] < stream_pending[best]) best = i;
        return best;
    };
    std::vector<hipEvent_t> pool;
    uint64_t next = 1;
    int idle = 0;
    const int64_t P = ctx->cfg.resident_cap, SB = ctx->slot_bytes;
    while (!ctx->stop.load(std::memory_order_relaxed)) {
        bool did = false;
        for (;;) {
            FifoEntry* fe = ctx->h_fifo + ((next - 1) % kFifoCap);
            const uint64_t s = __atomic_load_n(&fe->seq, __ATOMIC_ACQUIRE);
            if (s != next) break;
            const int key = fe->key, ring = fe->ring;
            const uint64_t fill = fe->fill;
            const int64_t t0 = now_ns();
            hipEvent_t ev;
            if (pool.empty()) {
                if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) ev = nullptr;
            } else {
                ev = pool.back();
                pool.pop_back();
            }
            bool ok = key >= 0 && key < ctx->n_experts_total && ring >= 0 && ring < ctx->cfg.ring_slots;
            const int si = ok ? pick(ring) : 0;
            const hipStream_t st = copy_stream_at(ctx, si);
            if (ok)
                ok = hipMemcpyAsync(ctx->d_slots + (P + ring) * SB, ctx->h_arena + (int64_t)key * SB, SB,
                                    hipMemcpyHostToDevice, st) == hipSuccess;
            // The ready flag is written by the copy stream right behind the
            // copy, so the waiting work-groups need not wait for this thread
            // to see the copy finish; the host writes it only if that fails.
            const bool flagged = ok && hipStreamWriteValue64(st, ctx->d_ready + ring, fill, 0) == hipSuccess;
            if (ok && ev) ok = hipEventRecord(ev, st) == hipSuccess;
            if (!ok) {
                ctx->agent_error.store(1);
                if (ev) pool.push_back(ev);
                // publish anyway: the data is wrong but nothing waits forever
                __atomic_store_n(ctx->h_ready + (ring >= 0 && ring < ctx->cfg.ring_slots ? ring : 0), fill,
                                 __ATOMIC_RELEASE);
            } else {
                pend.push_back({fill, ring, ev, si, t0, flagged});
                ring_stream[ring] = si;
                ++ring_pending[ring];
                ++stream_pending[si];
            }
            ++next;
            did = true;
        }
        // Publish every finished copy.  Copies into one ring slot in flight at
        // once share a stream, so a later fill of a slot never finishes first.
        for (auto it = pend.begin(); it != pend.end();) {
            const hipError_t q = it->ev ? hipEventQuery(it->ev) : hipStreamQuery(copy_stream_at(ctx, it->stream));
            if (q == hipErrorNotReady) {
                ++it;
                continue;
            }
            if (q != hipSuccess) ctx->agent_error.store(1);
            if (!it->flagged || q != hipSuccess) __atomic_store_n(ctx->h_ready + it->ring, it->seq, __ATOMIC_RELEASE);
            const int64_t dt = now_ns() - it->t0;
            ctx->fill_ns_sum.fetch_add(dt);
            int64_t m = ctx->fill_ns_max.load();
            while (dt > m && !ctx->fill_ns_max.compare_exchange_weak(m, dt)) {
            }
            if (it->ev) pool.push_back(it->ev);
            --ring_pending[it->ring];
            --stream_pending[it->stream];
            it = pend.erase(it);
            did = true;
        }
        if (did) {
            idle = 0;
        } else if (++idle > 20000) {
            std::this_thread::sleep_for(std::chrono::microseconds(20));
        } else {
            __builtin_ia32_pause();
        }
    }
    for (auto& p : pend)
        if (p.ev) hipEventDestroy(p.ev);
    for (auto ev : pool) hipEventDestroy(ev);
}

moe_spark_status check_config(const moe_spark_config* c, std::string& why) {
    char buf[256];
    auto bad = [&](const char* m) {
        why = m;
        return MOE_SPARK_E_INVALID;
    };
    if (!c) return bad("config is NULL");
    if (c->n_layers <= 0) return bad("n_layers must be > 0");
    if (c->n_experts <= 0 || c->n_experts > kMaxE || c->n_experts % 4)
        return bad("n_experts must be a multiple of 4 in [4, 1024]");
    if (c->top_k <= 0 || c->top_k > c->n_experts || c->top_k > kMaxK)
        return bad("top_k must be in [1, min(n_experts, 16)]");
    if (c->d_model <= 0 || c->d_model % 256 || c->d_model > 8192)
        return bad("d_model must be a multiple of 256 up to 8192");
    if (c->d_ff <= 0 || c->d_ff % 4 || c->d_ff > 8192) return bad("d_ff must be a multiple of 4 up to 8192");
    if (c->wfmt != MOE_SPARK_W_F32 && c->wfmt != MOE_SPARK_W_Q4_0) return bad("unknown weight format");
    if (c->wfmt == MOE_SPARK_W_Q4_0 && (c->d_model != kQD || c->d_ff != kQF || c->top_k > kQ4MaxK)) {
        snprintf(buf, sizeof buf, "Q4_0 kernels are built for d_model=%d, d_ff=%d, top_k<=%d", kQD, kQF,
                 kQ4MaxK);
        why = buf;
        return MOE_SPARK_E_INVALID;
    }
    const int64_t LE = (int64_t)c->n_layers * c->n_experts;
    if (c->resident_cap < 0 || c->resident_cap > LE) return bad("resident_cap must be in [0, L*E]");
    if (c->ring_slots < 0 || c->ring_slots > kMaxR) return bad("ring_slots must be in [0, 1024]");
    if (c->resident_cap < LE && c->ring_slots < c->top_k)
        return bad("ring_slots must be >= top_k when not every expert is pinned");
    if (c->n_bias_rows < 0) return bad("n_bias_rows must be >= 0");
    if (c->max_tokens < 0) return bad("max_tokens must be >= 0");
    if (c->event_cap < 0) return bad("event_cap must be >= 0");
    if (!(c->rms_eps >= 0.0f)) return bad("rms_eps must be >= 0");
    return MOE_SPARK_OK;
}

void free_all(moe_spark_ctx* ctx) {
    if (ctx->agent.joinable()) {
        ctx->stop.store(true);
        ctx->agent.join();
    }
    for (auto& g : ctx->graphs) {
        if (g.exec) hipGraphExecDestroy(g.exec);
        if (g.graph) hipGraphDestroy(g.graph);
    }
    ctx->graphs.clear();
    for (auto& e : ctx->tok_ev)
        if (e) hipEventDestroy(e);
    void* dptrs[] = {ctx->d_slots,  ctx->d_router,   ctx->d_bias,   ctx->d_slot_of, ctx->d_ring_owner,
                     ctx->d_ring_stamp, ctx->d_ring_seq, ctx->d_clock, ctx->d_counts, ctx->d_stats,
                     ctx->d_events, ctx->d_n_events, ctx->d_error,  ctx->d_cursors, ctx->d_done,
                     ctx->d_sel,    ctx->d_logits,   ctx->d_u,      ctx->d_ut,      ctx->d_h,
                     ctx->d_xscratch, ctx->d_pl,     ctx->d_ps,     ctx->d_pub,     ctx->d_pu,
                     ctx->d_pinv,     ctx->d_plog,   ctx->d_ptopk,  ctx->d_pgate,   ctx->d_phist,
                     ctx->d_pperm,    ctx->d_papos,  ctx->d_pslot,  ctx->d_pwait,   ctx->d_pfill,  ctx->d_ph,
                     ctx->d_py,       ctx->d_pmeta,  ctx->d_xbuf,   ctx->d_tokrow,  ctx->d_ntok,
                     ctx->d_bx,       ctx->d_brows,  ctx->d_bn,     ctx->d_bpl,     ctx->d_bps,
                     ctx->d_bu16,     ctx->d_bsel,   ctx->d_bpub,   ctx->d_bh16,   ctx->d_ppred,
                     ctx->d_pfill2,   ctx->d_plog2,  ctx->d_ptopk2};
    for (void* p : dptrs)
        if (p) hipFree(p);
    if (ctx->h_arena) hipHostFree(ctx->h_arena);
    if (ctx->h_fifo) hipHostFree(ctx->h_fifo);
    if (ctx->h_ready) hipHostFree(ctx->h_ready);
    if (ctx->h_pmeta) hipHostFree(ctx->h_pmeta);
    if (ctx->h_pfill2) hipHostFree(ctx->h_pfill2);
    if (ctx->h_pstate) hipHostFree(ctx->h_pstate);
    if (ctx->pf_q_ev) hipEventDestroy(ctx->pf_q_ev);
    if (ctx->pf_done_ev) hipEventDestroy(ctx->pf_done_ev);
    if (ctx->own_compute && ctx->compute) hipStreamDestroy(ctx->compute);
    if (ctx->own_copy && ctx->copy) hipStreamDestroy(ctx->copy);
    for (hipStream_t st : ctx->copy_x)
        if (st) hipStreamDestroy(st);
}

template <typename T>
hipError_t dalloc(T** p, size_t n) {
    return hipMalloc((void**)p, n * sizeof(T) > 0 ? n * sizeof(T) : 16);
}

PolicyTables tables(const moe_spark_ctx* ctx, bool pull = false) {
    PolicyTables t;
    t.pull = pull ? 1 : 0;
    t.slot_of = ctx->d_slot_of;
    t.ring_owner = ctx->d_ring_owner;
    t.ring_stamp = ctx->d_ring_stamp;
    t.ring_seq = ctx->d_ring_seq;
    t.clock = ctx->d_clock;
    t.fill_seq = ctx->d_clock + 1;
    t.req_seq = ctx->d_clock + 2;
    t.counts = ctx->d_counts;
    t.stats = ctx->d_stats;
    t.events = ctx->d_events;
    t.n_events = ctx->d_n_events;
    t.event_cap = ctx->cfg.event_cap;
    t.fifo = ctx->d_fifo;
    t.error = ctx->d_error;
    t.P = ctx->cfg.resident_cap;
    t.R = ctx->cfg.ring_slots;
    t.E = ctx->cfg.n_experts;
    t.slot_bytes = ctx->slot_bytes;
    return t;
}

RouteArgs route_args(const moe_spark_ctx* ctx, int layer, const float* x, TokRef tok, TokRef ttok,
                     const int32_t* bias_row, int norm, int32_t* topk_out, float* gates_out) {
    const auto& c = ctx->cfg;
    RouteArgs a{};
    a.x_base = x;
    a.tok = tok;
    a.trace_tok = ttok;
    a.d = c.d_model;
    a.E = c.n_experts;
    a.K = c.top_k;
    a.layer = layer;
    a.L = c.n_layers;
    a.norm = norm;
    a.eps = c.rms_eps;
    a.wr = ctx->d_router + (int64_t)layer * c.n_experts * c.d_model;
    a.bias = c.n_bias_rows > 0 ? ctx->d_bias + (int64_t)layer * c.n_bias_rows * c.n_experts : nullptr;
    a.bias_row = bias_row;
    a.n_bias_rows = c.n_bias_rows;
    a.logits = ctx->d_logits;
    a.done = ctx->d_done + 2 * layer;
    a.sel = ctx->d_sel + layer;
    a.u = ctx->d_u;
    a.ut = ctx->d_ut;
    a.pt = tables(ctx);
    a.tr_x = ctx->tr_x;
    a.tr_topk = ctx->tr_topk;
    a.tr_gates = ctx->tr_gates;
    a.tr_cap = ctx->tr_cap;
    a.topk_out = topk_out;
    a.gates_out = gates_out;
    a.q4 = c.wfmt == MOE_SPARK_W_Q4_0;
    return a;
}

ExpertArgs expert_args(const moe_spark_ctx* ctx, int layer, const float* x, float* y, TokRef tok,
                       int residual, int advance) {
    const auto& c = ctx->cfg;
    ExpertArgs a{};
    a.slots = ctx->d_slots;
    a.slot_bytes = ctx->slot_bytes;
    a.sel = ctx->d_sel + layer;
    a.ready = ctx->d_ready;
    a.P = c.resident_cap;
    a.n_slots = ctx->n_slots;
    a.R = c.ring_slots;
    a.d = c.d_model;
    a.f = c.d_ff;
    a.K = c.top_k;
    a.u = ctx->d_u;
    a.ut = ctx->d_ut;
    a.h = ctx->d_h;
    a.x_base = x;
    a.y_base = y;
    a.tok = tok;
    a.residual = residual;
    a.advance = advance;
    a.cursors = ctx->d_cursors;
    a.done = ctx->d_done + 2 * layer + 1;
    a.stats = ctx->d_stats;
    a.error = ctx->d_error;
    a.spin_limit_ticks = ctx->spin_ticks;
    return a;
}

// Arguments of the Q4_0 decode kernels of one token-layer.  wr_layer: the
// layer whose packed router the launch turns into partial logits (-1: none).
Q4Args q4_args(const moe_spark_ctx* ctx, int layer, const float* x, float* y, TokRef tok, TokRef ttok,
               const int32_t* bias_row, int norm, int residual, int wr_layer, int32_t* topk_out,
               float* gates_out, int replay) {
    const auto& c = ctx->cfg;
    Q4Args a{};
    a.x_base = x;
    a.y_base = y;
    a.tok = tok;
    a.trace_tok = ttok;
    a.layer = layer;
    a.L = c.n_layers;
    a.E = c.n_experts;
    a.K = c.top_k;
    a.norm = norm;
    a.residual = residual;
    a.replay = replay;
    a.eps = c.rms_eps;
    a.pl = ctx->d_pl;
    a.ps = ctx->d_ps;
    a.wr_part = wr_layer >= 0 ? ctx->d_router + (int64_t)wr_layer * c.n_experts * c.d_model : nullptr;
    a.bias = c.n_bias_rows > 0 ? ctx->d_bias + (int64_t)layer * c.n_bias_rows * c.n_experts : nullptr;
    a.bias_row = bias_row;
    a.n_bias_rows = c.n_bias_rows;
    a.slots = ctx->d_slots;
    a.slot_bytes = ctx->slot_bytes;
    a.P = c.resident_cap;
    a.n_slots = ctx->n_slots;
    a.ready = ctx->d_ready;
    a.arena = ctx->d_arena;
    a.sel = ctx->d_sel + layer;
    a.pub = ctx->d_pub + layer;
    a.h = ctx->d_h;
    a.pt = tables(ctx, ctx->pull_fills);
    a.tr_x = replay ? nullptr : ctx->tr_x;
    a.tr_topk = replay ? nullptr : ctx->tr_topk;
    a.tr_gates = replay ? nullptr : ctx->tr_gates;
    a.tr_cap = ctx->tr_cap;
    a.topk_out = topk_out;
    a.gates_out = gates_out;
    a.spin_limit_ticks = ctx->spin_ticks;
    return a;
}

moe_spark_status ready_check(moe_spark_ctx* ctx) {
    if (ctx->n_router_set != ctx->cfg.n_layers || ctx->n_expert_set != ctx->n_experts_total)
        return ctx->fail(MOE_SPARK_E_STATE, "every router and expert must be set first (%lld/%d routers, %lld/%lld experts)",
                         (long long)ctx->n_router_set, ctx->cfg.n_layers, (long long)ctx->n_expert_set,
                         (long long)ctx->n_experts_total);
    if (!ctx->placed) return ctx->fail(MOE_SPARK_E_STATE, "no placement yet: call moe_spark_place_uniform");
    return MOE_SPARK_OK;
}

// Upload experts into pinned slots: (slot, key) pairs, coalescing runs that are
// contiguous in both arenas.
moe_spark_status upload_pinned(moe_spark_ctx* ctx, std::vector<std::pair<int32_t, int32_t>> moves) {
    std::sort(moves.begin(), moves.end(), [](auto a, auto b) { return a.first < b.first; });
    const int64_t SB = ctx->slot_bytes;
    size_t i = 0;
    while (i < moves.size()) {
        size_t j = i + 1;
        while (j < moves.size() && moves[j].first == moves[j - 1].first + 1 &&
               moves[j].second == moves[j - 1].second + 1)
            ++j;
        const int64_t n = (int64_t)(j - i);
        HIPCHK(hipMemcpyAsync(ctx->d_slots + (int64_t)moves[i].first * SB,
                              ctx->h_arena + (int64_t)moves[i].second * SB, n * SB, hipMemcpyHostToDevice,
                              ctx->copy));
        i = j;
    }
    HIPCHK(sync_copies(ctx));
    return MOE_SPARK_OK;
}

void drop_graphs(moe_spark_ctx* ctx) {
    hipStreamSynchronize(ctx->compute);
    for (auto& g : ctx->graphs) {
        if (g.exec) hipGraphExecDestroy(g.exec);
        if (g.graph) hipGraphDestroy(g.graph);
    }
    ctx->graphs.clear();
}

TokenIO token_io(const moe_spark_ctx* ctx, float* x, const int32_t* bias_row) {
    TokenIO io;
    io.x = x;
    io.bias_row = bias_row;
    io.xbuf = ctx->d_xbuf;
    io.tokrow = ctx->d_tokrow;
    io.cursors = ctx->d_cursors;
    io.ntok = ctx->d_ntok;
    io.stats = ctx->d_stats;
    return io;
}

// Reset the token cursor for a decode call of n tokens (Q4_0: also stage the
// first token).
moe_spark_status begin_decode(moe_spark_ctx* ctx, float* x, const int32_t* bias_row, int32_t n) {
    if (ctx->cfg.wfmt == MOE_SPARK_W_Q4_0) {
        HIPCHK(launch_token_begin(token_io(ctx, x, bias_row), n, ctx->compute));
    } else {
        HIPCHK(hipMemsetAsync(ctx->d_cursors, 0, sizeof(int32_t), ctx->compute));
    }
    return MOE_SPARK_OK;
}

moe_spark_status launch_token_kernels(moe_spark_ctx* ctx, float* x, const int32_t* bias_row) {
    const int L = ctx->cfg.n_layers, wfmt = ctx->cfg.wfmt;
    const TokRef tok{ctx->d_cursors, 0}, ttok{ctx->d_cursors + 1, 0};
    if (wfmt == MOE_SPARK_W_Q4_0) {
        // the token sits in xbuf, its bias row in tokrow (fixed addresses)
        float* xb = ctx->d_xbuf;
        const TokRef t0{nullptr, 0};
        HIPCHK(launch_q4_router_partial(q4_args(ctx, 0, xb, xb, t0, ttok, ctx->d_tokrow, 1, 1, 0, nullptr, nullptr, 0),
                                        ctx->compute));
        for (int l = 0; l < L; ++l) {
            const Q4Args a = q4_args(ctx, l, xb, xb, t0, ttok, ctx->d_tokrow, 1, 1, l + 1 < L ? l + 1 : -1, nullptr,
                                     nullptr, 0);
            HIPCHK(launch_q4_gateup(a, ctx->compute));
            HIPCHK(launch_q4_down(a, ctx->compute));
        }
        HIPCHK(launch_token_end(token_io(ctx, x, bias_row), ctx->compute));
        return MOE_SPARK_OK;
    }
    for (int l = 0; l < L; ++l) {
        const RouteArgs ra = route_args(ctx, l, x, tok, ttok, bias_row, 1, nullptr, nullptr);
        HIPCHK(launch_route(ra, ctx->compute));
        const ExpertArgs ea = expert_args(ctx, l, x, x, tok, 1, l == L - 1);
        HIPCHK(launch_gateup(ea, wfmt, ctx->compute));
        HIPCHK(launch_down(ea, wfmt, ctx->compute));
    }
    return MOE_SPARK_OK;
}

BatchIO batch_io(const moe_spark_ctx* ctx, float* x, const int32_t* bias_row, int32_t batch) {
    BatchIO io;
    io.x = x;
    io.bias_row = bias_row;
    io.xb = ctx->d_bx;
    io.rows = ctx->d_brows;
    io.nb = ctx->d_bn;
    io.cursors = ctx->d_cursors;
    io.ntok = ctx->d_ntok;
    io.stats = ctx->d_stats;
    io.B = batch;
    return io;
}

// Arguments of the batched decode kernels of one layer.  wr_layer: the layer
// whose packed router the launch turns into partial logits (-1: none).
QBArgs qb_args(const moe_spark_ctx* ctx, int layer, int wr_layer, int32_t batch) {
    const auto& c = ctx->cfg;
    QBArgs a{};
    a.layer = layer;
    a.L = c.n_layers;
    a.E = c.n_experts;
    a.K = c.top_k;
    a.B = batch;
    a.nb = ctx->d_bn;
    a.xb = ctx->d_bx;
    a.rows = ctx->d_brows;
    a.norm = 1;
    a.eps = c.rms_eps;
    a.pl = ctx->d_bpl;
    a.ps = ctx->d_bps;
    a.wr_part = wr_layer >= 0 ? ctx->d_router + (int64_t)wr_layer * c.n_experts * c.d_model : nullptr;
    a.bias = c.n_bias_rows > 0 ? ctx->d_bias + (int64_t)layer * c.n_bias_rows * c.n_experts : nullptr;
    a.n_bias_rows = c.n_bias_rows;
    a.u16 = ctx->d_bu16;
    a.slots = ctx->d_slots;
    a.arena = ctx->d_arena;
    a.slot_bytes = ctx->slot_bytes;
    a.P = c.resident_cap;
    a.n_slots = ctx->n_slots;
    a.ready = ctx->d_ready;
    a.sel = ctx->d_bsel + layer;
    a.pub = ctx->d_bpub + layer;
    a.h16 = ctx->d_bh16;
    a.pt = tables(ctx, ctx->pull_fills);
    a.tr_x = ctx->tr_x;
    a.tr_topk = ctx->tr_topk;
    a.tr_gates = ctx->tr_gates;
    a.tr_cap = ctx->tr_cap;
    a.trace_base = ctx->d_cursors + 1;
    a.spin_limit_ticks = ctx->spin_ticks;
    return a;
}

// One step of batched decode: the first layer's router partials, then route,
// gate/up and down per layer, then the step's write-back and staging.
moe_spark_status launch_step_kernels(moe_spark_ctx* ctx, float* x, const int32_t* bias_row, int32_t batch) {
    const int L = ctx->cfg.n_layers;
    HIPCHK(launch_qb_router_partial(qb_args(ctx, 0, 0, batch), ctx->compute));
    for (int l = 0; l < L; ++l) {
        const QBArgs a = qb_args(ctx, l, l + 1 < L ? l + 1 : -1, batch);
        HIPCHK(launch_qb_route(a, ctx->compute));
        HIPCHK(launch_qb_gateup(a, ctx->compute));
        HIPCHK(launch_qb_down(a, ctx->compute));
    }
    HIPCHK(launch_qb_end(batch_io(ctx, x, bias_row, batch), ctx->compute));
    return MOE_SPARK_OK;
}

moe_spark_status get_graph(moe_spark_ctx* ctx, float* x, const int32_t* bias_row, int32_t batch,
                           hipGraphExec_t* out) {
    for (auto& g : ctx->graphs)
        if (g.x == x && g.bias_row == bias_row && g.batch == batch) {
            *out = g.exec;
            return MOE_SPARK_OK;
        }
    if (ctx->graphs.size() >= 4) {
        HIPCHK(hipStreamSynchronize(ctx->compute));
        auto& g = ctx->graphs.front();
        hipGraphExecDestroy(g.exec);
        hipGraphDestroy(g.graph);
        ctx->graphs.erase(ctx->graphs.begin());
    }
    GraphEntry ge;
    ge.x = x;
    ge.bias_row = bias_row;
    ge.batch = batch;
    HIPCHK(hipStreamBeginCapture(ctx->compute, hipStreamCaptureModeThreadLocal));
    moe_spark_status st = batch ? launch_step_kernels(ctx, x, bias_row, batch) : launch_token_kernels(ctx, x, bias_row);
    hipGraph_t graph = nullptr;
    const hipError_t ec = hipStreamEndCapture(ctx->compute, &graph);
    if (st != MOE_SPARK_OK) {
        if (graph) hipGraphDestroy(graph);
        return st;
    }
    if (ec != hipSuccess) return ctx->fail(MOE_SPARK_E_HIP, "graph capture failed: %s", hipGetErrorString(ec));
    ge.graph = graph;
    const hipError_t ei = hipGraphInstantiate(&ge.exec, graph, nullptr, nullptr, 0);
    if (ei != hipSuccess) {
        hipGraphDestroy(graph);
        return ctx->fail(MOE_SPARK_E_HIP, "graph instantiate failed: %s", hipGetErrorString(ei));
    }
    ctx->graphs.push_back(ge);
    *out = ge.exec;
    return MOE_SPARK_OK;
}

}  // namespace

// ====================================================================== C ABI

extern "C" {

moe_spark_status moe_spark_create(const moe_spark_config* cfg, void* compute_stream, void* copy_stream,
                                  moe_spark_ctx** out) {
    if (!out) return MOE_SPARK_E_INVALID;
    *out = nullptr;
    std::string why;
    moe_spark_status st = check_config(cfg, why);
    if (st != MOE_SPARK_OK) {
        g_create_err = why;
        return st;
    }
    auto* ctx = new moe_spark_ctx();
    ctx->cfg = *cfg;
    if (ctx->cfg.event_cap == 0) ctx->cfg.event_cap = 1 << 20;
    const auto& c = ctx->cfg;
    const int d = c.d_model, f = c.d_ff, E = c.n_experts, L = c.n_layers;
    ctx->slot_bytes = c.wfmt == MOE_SPARK_W_Q4_0 ? kQ4SlotBytes : (int64_t)3 * f * d * 4;
    ctx->n_experts_total = (int64_t)L * E;
    ctx->n_slots = c.resident_cap + c.ring_slots;
    ctx->router_set.assign(L, 0);
    ctx->expert_set.assign(ctx->n_experts_total, 0);
    ctx->slot_of.assign(ctx->n_experts_total, -1);

    auto fail_create = [&](moe_spark_status s, const std::string& m) {
        g_create_err = m;
        free_all(ctx);
        delete ctx;
        return s;
    };
    hipError_t e = hipGetDevice(&ctx->device);
    if (e != hipSuccess) return fail_create(MOE_SPARK_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    e = scratch_init(ctx->device);  // this GPU's no-alloc scratch (moe_spark_layer_forward_noalloc)
    if (e != hipSuccess)
        return fail_create(MOE_SPARK_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    int rate_khz = 0;
    if (hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, ctx->device) != hipSuccess || rate_khz <= 0)
        rate_khz = 100000;
    ctx->spin_ticks = (uint64_t)rate_khz * 1000ull * 2ull;  // 2 s
    if (const char* ev = getenv("MOE_SPARK_DECODE_STREAM")) ctx->stream_decode = ev[0] == '1';
    if (const char* ev = getenv("MOE_SPARK_COPY_STREAMS")) {
        const int n = atoi(ev);
        if (n >= 1 && n <= kCopyStreams) ctx->n_copy = n;
    }
    if (const char* ev = getenv("MOE_SPARK_FILL_COLS")) {
        const int n = atoi(ev);
        if (n >= 1 && n <= 128) ctx->pf_fill_cols = n;
    }
    if (compute_stream) {
        ctx->compute = (hipStream_t)compute_stream;
    } else {
        if (hipStreamCreateWithFlags(&ctx->compute, hipStreamNonBlocking) != hipSuccess)
            return fail_create(MOE_SPARK_E_HIP, "hipStreamCreate failed");
        ctx->own_compute = true;
    }
    if (copy_stream) {
        ctx->copy = (hipStream_t)copy_stream;
    } else {
        if (hipStreamCreateWithFlags(&ctx->copy, hipStreamNonBlocking) != hipSuccess)
            return fail_create(MOE_SPARK_E_HIP, "hipStreamCreate failed");
        ctx->own_copy = true;
    }
    if (hipMalloc((void**)&ctx->d_slots, (size_t)std::max<int64_t>(ctx->n_slots, 1) * ctx->slot_bytes) != hipSuccess) {
        ctx->d_slots = nullptr;
        return fail_create(MOE_SPARK_E_NOMEM, "slot arena allocation failed");
    }
    if (hipHostMalloc((void**)&ctx->h_arena, (size_t)ctx->n_experts_total * ctx->slot_bytes, hipHostMallocDefault) !=
        hipSuccess) {
        ctx->h_arena = nullptr;
        return fail_create(MOE_SPARK_E_NOMEM, "pinned host arena allocation failed");
    }
    {   // decode pulls its own fills from the arena through its device address
        void* dp = nullptr;
        const char* ev = getenv("MOE_SPARK_PULL_FILLS");
        const bool want = !(ev && ev[0] == '0');
        if (want && c.wfmt == MOE_SPARK_W_Q4_0 && hipHostGetDevicePointer(&dp, ctx->h_arena, 0) == hipSuccess && dp) {
            ctx->d_arena = (const uint8_t*)dp;
            ctx->pull_fills = true;
        }
    }
    // The host agent's extra copy streams exist only when it copies fills:
    // fewer streams leave the copy stream a hardware queue of its own, so
    // that prefill's prefetch copies on it run beside the compute stream.
    if (!ctx->pull_fills)
        for (hipStream_t& st : ctx->copy_x)
            if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess)
                return fail_create(MOE_SPARK_E_HIP, "hipStreamCreate failed");
    const int R = c.ring_slots;
    bool ok = true;
    ok &= dalloc(&ctx->d_router, (size_t)L * E * d) == hipSuccess;
    ok &= dalloc(&ctx->d_bias, (size_t)L * std::max(c.n_bias_rows, 1) * E) == hipSuccess;
    ok &= dalloc(&ctx->d_slot_of, (size_t)L * E) == hipSuccess;
    ok &= dalloc(&ctx->d_ring_owner, (size_t)std::max(R, 1)) == hipSuccess;
    ok &= dalloc(&ctx->d_ring_stamp, (size_t)std::max(R, 1)) == hipSuccess;
    ok &= dalloc(&ctx->d_ring_seq, (size_t)std::max(R, 1)) == hipSuccess;
    ok &= dalloc(&ctx->d_clock, 3) == hipSuccess;
    ok &= dalloc(&ctx->d_counts, (size_t)L * E) == hipSuccess;
    ok &= dalloc(&ctx->d_stats, DS_N) == hipSuccess;
    ok &= dalloc(&ctx->d_events, (size_t)c.event_cap) == hipSuccess;
    ok &= dalloc(&ctx->d_n_events, 1) == hipSuccess;
    ok &= dalloc(&ctx->d_error, 1) == hipSuccess;
    ok &= dalloc(&ctx->d_cursors, 2) == hipSuccess;
    ok &= dalloc(&ctx->d_done, (size_t)2 * L + 4) == hipSuccess;
    ok &= dalloc(&ctx->d_sel, (size_t)L + 1) == hipSuccess;
    ok &= dalloc(&ctx->d_logits, (size_t)E) == hipSuccess;
    ok &= dalloc(&ctx->d_u, (size_t)d) == hipSuccess;
    ok &= dalloc(&ctx->d_ut, (size_t)d) == hipSuccess;
    ok &= dalloc(&ctx->d_h, (size_t)kMaxK * f) == hipSuccess;
    ok &= dalloc(&ctx->d_xscratch, (size_t)d) == hipSuccess;
    ok &= dalloc(&ctx->d_pl, (size_t)kNP * E) == hipSuccess;
    ok &= dalloc(&ctx->d_ps, (size_t)kNP) == hipSuccess;
    ok &= dalloc(&ctx->d_pub, (size_t)L) == hipSuccess;
    ok &= dalloc(&ctx->d_xbuf, (size_t)d) == hipSuccess;
    ok &= dalloc(&ctx->d_tokrow, 1) == hipSuccess;
    ok &= dalloc(&ctx->d_ntok, 1) == hipSuccess;
    if (c.wfmt == MOE_SPARK_W_Q4_0) {
        ok &= dalloc(&ctx->d_bx, (size_t)kMaxB * d) == hipSuccess;
        ok &= dalloc(&ctx->d_brows, (size_t)kMaxB) == hipSuccess;
        ok &= dalloc(&ctx->d_bn, 1) == hipSuccess;
        ok &= dalloc(&ctx->d_bpl, (size_t)kMaxB * kNP * E) == hipSuccess;
        ok &= dalloc(&ctx->d_bps, (size_t)kMaxB * kNP) == hipSuccess;
        ok &= dalloc(&ctx->d_bu16, (size_t)kMaxB * d) == hipSuccess;
        ok &= dalloc(&ctx->d_bsel, (size_t)L) == hipSuccess;
        ok &= dalloc(&ctx->d_bpub, (size_t)L) == hipSuccess;
        ok &= dalloc(&ctx->d_bh16, (size_t)kMaxBK * f) == hipSuccess;
    }
    if (!ok) return fail_create(MOE_SPARK_E_NOMEM, "device table allocation failed");
    if (c.max_tokens > 0) {
        const size_t T = (size_t)c.max_tokens, K = (size_t)c.top_k;
        ctx->pf_max_items = (int64_t)(T * K / 128 + E + 1);
        ok &= dalloc(&ctx->d_pu, T * d) == hipSuccess;
        ok &= dalloc(&ctx->d_pinv, T) == hipSuccess;
        ok &= dalloc(&ctx->d_plog, T * E) == hipSuccess;
        ok &= dalloc(&ctx->d_plog2, T * E) == hipSuccess;
        ok &= dalloc(&ctx->d_ptopk2, T * K) == hipSuccess;
        ok &= hipEventCreateWithFlags(&ctx->pf_q_ev, hipEventDisableTiming) == hipSuccess;
        ok &= hipEventCreateWithFlags(&ctx->pf_done_ev, hipEventDisableTiming) == hipSuccess;
        ok &= dalloc(&ctx->d_pfill2, (size_t)(1 + 2 * kMaxR)) == hipSuccess;
        ok &= dalloc(&ctx->d_ptopk, T * K) == hipSuccess;
        ok &= dalloc(&ctx->d_pgate, T * K) == hipSuccess;
        ok &= dalloc(&ctx->d_phist, (size_t)E) == hipSuccess;
        ok &= dalloc(&ctx->d_ppred, (size_t)L * E) == hipSuccess;
        ok &= dalloc(&ctx->d_pperm, T * K) == hipSuccess;
        ok &= dalloc(&ctx->d_papos, T * K) == hipSuccess;
        ok &= dalloc(&ctx->d_pslot, (size_t)E) == hipSuccess;
        ok &= dalloc(&ctx->d_pwait, (size_t)E) == hipSuccess;
        ok &= dalloc(&ctx->d_pfill, (size_t)(1 + 2 * kMaxR)) == hipSuccess;
        ok &= dalloc(&ctx->d_ph, T * K * f) == hipSuccess;
        ok &= dalloc(&ctx->d_py, T * K * d) == hipSuccess;
        const size_t meta = (size_t)(2 * E + 1 + 2 * ctx->pf_max_items);
        ok &= dalloc(&ctx->d_pmeta, meta) == hipSuccess;
        if (!ok) return fail_create(MOE_SPARK_E_NOMEM, "prefill buffer allocation failed");
        if (c.wfmt == MOE_SPARK_W_Q4_0 && prepare_pf_kernels() != hipSuccess)
            return fail_create(MOE_SPARK_E_HIP, "prefill kernels could not be prepared");
        const size_t pstate = (size_t)(2 + E + 2 * (1 + 2 * kMaxR));
        if (hipHostMalloc((void**)&ctx->h_pmeta, meta * sizeof(int32_t), hipHostMallocMapped | hipHostMallocCoherent) !=
                hipSuccess ||
            hipHostMalloc((void**)&ctx->h_pfill2, (size_t)(1 + 2 * kMaxR) * sizeof(int32_t), hipHostMallocDefault) !=
                hipSuccess ||
            hipHostMalloc((void**)&ctx->h_pstate, pstate * sizeof(int32_t),
                          hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess)
            return fail_create(MOE_SPARK_E_NOMEM, "prefill staging allocation failed");
        memset(ctx->h_pstate, 0, pstate * sizeof(int32_t));
        if (hipHostGetDevicePointer((void**)&ctx->d_pstate, ctx->h_pstate, 0) != hipSuccess || !ctx->d_pstate ||
            hipHostGetDevicePointer((void**)&ctx->dm_pmeta, ctx->h_pmeta, 0) != hipSuccess || !ctx->dm_pmeta)
            return fail_create(MOE_SPARK_E_HIP, "hipHostGetDevicePointer(prefill host buffers) failed");
    }
    if (hipHostMalloc((void**)&ctx->h_fifo, sizeof(FifoEntry) * kFifoCap, hipHostMallocMapped | hipHostMallocCoherent) !=
            hipSuccess ||
        hipHostMalloc((void**)&ctx->h_ready, sizeof(uint64_t) * std::max(R, 1),
                      hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess)
        return fail_create(MOE_SPARK_E_NOMEM, "mapped host allocation failed");
    memset(ctx->h_fifo, 0, sizeof(FifoEntry) * kFifoCap);
    memset(ctx->h_ready, 0, sizeof(uint64_t) * std::max(R, 1));
    if (hipHostGetDevicePointer((void**)&ctx->d_fifo, ctx->h_fifo, 0) != hipSuccess ||
        hipHostGetDevicePointer((void**)&ctx->d_ready, ctx->h_ready, 0) != hipSuccess)
        return fail_create(MOE_SPARK_E_HIP, "hipHostGetDevicePointer failed");
    // zero every table
    ok &= hipMemset(ctx->d_slot_of, 0xff, sizeof(int32_t) * L * E) == hipSuccess;
    ok &= hipMemset(ctx->d_ring_owner, 0xff, sizeof(int32_t) * std::max(R, 1)) == hipSuccess;
    ok &= hipMemset(ctx->d_ring_stamp, 0, sizeof(uint64_t) * std::max(R, 1)) == hipSuccess;
    ok &= hipMemset(ctx->d_ring_seq, 0, sizeof(uint64_t) * std::max(R, 1)) == hipSuccess;
    ok &= hipMemset(ctx->d_clock, 0, sizeof(uint64_t) * 3) == hipSuccess;
    ok &= hipMemset(ctx->d_counts, 0, sizeof(int64_t) * L * E) == hipSuccess;
    ok &= hipMemset(ctx->d_stats, 0, sizeof(int64_t) * DS_N) == hipSuccess;
    ok &= hipMemset(ctx->d_n_events, 0, sizeof(int64_t)) == hipSuccess;
    ok &= hipMemset(ctx->d_error, 0, sizeof(int32_t)) == hipSuccess;
    ok &= hipMemset(ctx->d_cursors, 0, sizeof(int32_t) * 2) == hipSuccess;
    ok &= hipMemset(ctx->d_done, 0, sizeof(uint32_t) * (2 * L + 4)) == hipSuccess;
    ok &= hipMemset(ctx->d_sel, 0, sizeof(LayerSel) * (L + 1)) == hipSuccess;
    ok &= hipMemset(ctx->d_bias, 0, sizeof(float) * L * std::max(c.n_bias_rows, 1) * E) == hipSuccess;
    ok &= hipMemset(ctx->d_xscratch, 0, sizeof(float) * d) == hipSuccess;
    ok &= hipMemset(ctx->d_u, 0, sizeof(float) * d) == hipSuccess;
    ok &= hipMemset(ctx->d_ut, 0, sizeof(float) * d) == hipSuccess;
    ok &= hipMemset(ctx->d_h, 0, sizeof(float) * kMaxK * f) == hipSuccess;
    ok &= hipMemset(ctx->d_pl, 0, sizeof(float) * kNP * E) == hipSuccess;
    ok &= hipMemset(ctx->d_ps, 0, sizeof(float) * kNP) == hipSuccess;
    ok &= hipMemset(ctx->d_pub, 0, sizeof(uint32_t) * L) == hipSuccess;
    ok &= hipMemset(ctx->d_xbuf, 0, sizeof(float) * d) == hipSuccess;
    ok &= hipMemset(ctx->d_tokrow, 0, sizeof(int32_t)) == hipSuccess;
    ok &= hipMemset(ctx->d_ntok, 0, sizeof(int32_t)) == hipSuccess;
    if (c.wfmt == MOE_SPARK_W_Q4_0) {
        ok &= hipMemset(ctx->d_bx, 0, sizeof(float) * kMaxB * d) == hipSuccess;
        ok &= hipMemset(ctx->d_brows, 0, sizeof(int32_t) * kMaxB) == hipSuccess;
        ok &= hipMemset(ctx->d_bn, 0, sizeof(int32_t)) == hipSuccess;
        ok &= hipMemset(ctx->d_bsel, 0, sizeof(BatchSel) * L) == hipSuccess;
        ok &= hipMemset(ctx->d_bpub, 0, sizeof(uint32_t) * L) == hipSuccess;
        ok &= hipMemset(ctx->d_bh16, 0, sizeof(uint16_t) * kMaxBK * f) == hipSuccess;
        ok &= hipMemset(ctx->d_bu16, 0, sizeof(uint16_t) * kMaxB * d) == hipSuccess;
    }
    for (auto& ev : ctx->tok_ev) ok &= hipEventCreateWithFlags(&ev, hipEventDisableTiming) == hipSuccess;
    ok &= hipDeviceSynchronize() == hipSuccess;
    if (!ok) return fail_create(MOE_SPARK_E_HIP, "table initialisation failed");
    if (R > 0) ctx->agent = std::thread(agent_loop, ctx);
    *out = ctx;
    return MOE_SPARK_OK;
}

void moe_spark_destroy(moe_spark_ctx* ctx) {
    if (!ctx) return;
    if (ctx->compute) hipStreamSynchronize(ctx->compute);
    sync_copies(ctx);
    free_all(ctx);
    delete ctx;
}

const char* moe_spark_last_error(const moe_spark_ctx* ctx) {
    return ctx ? ctx->err.c_str() : g_create_err.c_str();
}

int64_t moe_spark_slot_bytes(const moe_spark_ctx* ctx) { return ctx ? ctx->slot_bytes : 0; }

// Before weights or the router change: nothing queued may still read them
// (kernels, pulled or agent fills in flight, uploads).
static moe_spark_status quiesce(moe_spark_ctx* ctx) {
    HIPCHK(hipStreamSynchronize(ctx->compute));
    HIPCHK(sync_copies(ctx));
    return MOE_SPARK_OK;
}

moe_spark_status moe_spark_set_router(moe_spark_ctx* ctx, int32_t layer, const float* w, const float* bias) {
    if (!ctx) return MOE_SPARK_E_INVALID;
    const auto& c = ctx->cfg;
    if (layer < 0 || layer >= c.n_layers || !w) return ctx->fail(MOE_SPARK_E_INVALID, "bad layer or NULL weights");
    if ((c.n_bias_rows > 0) != (bias != nullptr))
        return ctx->fail(MOE_SPARK_E_INVALID, "bias must be given iff n_bias_rows > 0");
    moe_spark_status st = quiesce(ctx);  // kernels still queued may read this layer's router
    if (st != MOE_SPARK_OK) return st;
    const int64_t ED = (int64_t)c.n_experts * c.d_model;
    if (c.wfmt == MOE_SPARK_W_Q4_0) {
        // [p][e][i] = w[e][16p + i]: one 16-row slice of every router row per partial work-group
        std::vector<float> packed((size_t)ED);
        const int E = c.n_experts;
        for (int p = 0; p < kNP; ++p)
            for (int e = 0; e < E; ++e)
                memcpy(&packed[((size_t)p * E + e) * kRW], w + (int64_t)e * c.d_model + p * kRW, kRW * sizeof(float));
        HIPCHK(hipMemcpy(ctx->d_router + layer * ED, packed.data(), ED * sizeof(float), hipMemcpyHostToDevice));
    } else {
        HIPCHK(hipMemcpy(ctx->d_router + layer * ED, w, ED * sizeof(float), hipMemcpyHostToDevice));
    }
    if (bias) {
        const int64_t RE = (int64_t)c.n_bias_rows * c.n_experts;
        HIPCHK(hipMemcpy(ctx->d_bias + layer * RE, bias, RE * sizeof(float), hipMemcpyHostToDevice));
    }
    if (!ctx->router_set[layer]) {
        ctx->router_set[layer] = 1;
        ++ctx->n_router_set;
    }
    return MOE_SPARK_OK;
}

// After experts first .. first+n-1 were repacked into the host arena: copy
// every resident copy of them again, in pinned slots and in ring slots, so no
// slot keeps old weights (outputs stay independent of residency).  The ring
// tables are unchanged, so the placement state is too.
static moe_spark_status refresh_resident(moe_spark_ctx* ctx, int64_t first, int64_t n) {
    if (!ctx->placed) return MOE_SPARK_OK;
    std::vector<std::pair<int32_t, int32_t>> moves;
    for (int64_t i = first; i < first + n; ++i)
        if (ctx->slot_of[i] >= 0) moves.push_back({ctx->slot_of[i], (int32_t)i});
    const int R = ctx->cfg.ring_slots;
    if (R > 0) {
        std::vector<int32_t> owner(R);
        HIPCHK(hipMemcpy(owner.data(), ctx->d_ring_owner, sizeof(int32_t) * R, hipMemcpyDeviceToHost));
        for (int r = 0; r < R; ++r)
            if (owner[r] >= first && owner[r] < first + n)
                moves.push_back({(int32_t)(ctx->cfg.resident_cap + r), owner[r]});
    }
    if (moves.empty()) return MOE_SPARK_OK;
    return upload_pinned(ctx, moves);
}

moe_spark_status moe_spark_set_expert(moe_spark_ctx* ctx, int32_t layer, int32_t expert, const void* gate,
                                      const void* up, const void* down) {
    if (!ctx) return MOE_SPARK_E_INVALID;
    const auto& c = ctx->cfg;
    if (layer < 0 || layer >= c.n_layers || expert < 0 || expert >= c.n_experts || !gate || !up || !down)
        return ctx->fail(MOE_SPARK_E_INVALID, "bad layer/expert or NULL weights");
    const int64_t key = (int64_t)layer * c.n_experts + expert;
    moe_spark_status st = quiesce(ctx);
    if (st != MOE_SPARK_OK) return st;
    pack_expert(ctx, gate, up, down, ctx->h_arena + key * ctx->slot_bytes);
    if (!ctx->expert_set[key]) {
        ctx->expert_set[key] = 1;
        ++ctx->n_expert_set;
    }
    return refresh_resident(ctx, key, 1);
}

moe_spark_status moe_spark_set_experts(moe_spark_ctx* ctx, int64_t first, int64_t n, const void* blob) {
    if (!ctx) return MOE_SPARK_E_INVALID;
    const auto& c = ctx->cfg;
    if (first < 0 || n < 0 || first + n > ctx->n_experts_total || (!blob && n > 0))
        return ctx->fail(MOE_SPARK_E_INVALID, "expert range out of bounds");
    const int d = c.d_model, f = c.d_ff;
    const int64_t mb = matrix_bytes(f, d, c.wfmt), db = matrix_bytes(d, f, c.wfmt);
    const int64_t per = 2 * mb + db;
    const uint8_t* src = (const uint8_t*)blob;
    moe_spark_status st = quiesce(ctx);
    if (st != MOE_SPARK_OK) return st;
    unsigned nt = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    std::vector<std::thread> th;
    for (unsigned t = 0; t < nt; ++t)
        th.emplace_back([&, t] {
            for (int64_t i = t; i < n; i += nt) {
                const uint8_t* p = src + i * per;
                pack_expert(ctx, p, p + mb, p + 2 * mb, ctx->h_arena + (first + i) * ctx->slot_bytes);
            }
        });
    for (auto& x : th) x.join();
    for (int64_t i = first; i < first + n; ++i)
        if (!ctx->expert_set[i]) {
            ctx->expert_set[i] = 1;
            ++ctx->n_expert_set;
        }
    return refresh_resident(ctx, first, n);
}

moe_spark_status moe_spark_place_uniform(moe_spark_ctx* ctx) {
    if (!ctx) return MOE_SPARK_E_INVALID;
    if (ctx->n_expert_set != ctx->n_experts_total || ctx->n_router_set != ctx->cfg.n_layers)
        return ctx->fail(MOE_SPARK_E_STATE, "set every router and expert before placing");
    const auto& c = ctx->cfg;
    const int L = c.n_layers, E = c.n_experts, R = c.ring_slots;
    HIPCHK(hipStreamSynchronize(ctx->compute));
    std::vector<std::pair<int32_t, int32_t>> moves;
    int32_t next = 0;
    for (int l = 0; l < L; ++l) {
        const int64_t q = quota(L, c.resident_cap, l);
        for (int e = 0; e < E; ++e) {
            const int32_t key = l * E + e;
            ctx->slot_of[key] = e < q ? next++ : -1;
            if (e < q) moves.push_back({ctx->slot_of[key], key});
        }
    }
    HIPCHK(hipMemcpy(ctx->d_slot_of, ctx->slot_of.data(), sizeof(int32_t) * L * E, hipMemcpyHostToDevice));
    HIPCHK(hipMemset(ctx->d_ring_owner, 0xff, sizeof(int32_t) * std::max(R, 1)));
    HIPCHK(hipMemset(ctx->d_ring_stamp, 0, sizeof(uint64_t) * std::max(R, 1)));
    moe_spark_status st = upload_pinned(ctx, moves);
    if (st != MOE_SPARK_OK) return st;
    ctx->placed = true;
    ctx->at_since = 0;
    return MOE_SPARK_OK;
}

// Move the pinned set to `want`: experts leaving it free their slots; the
// freed slots, ascending, go to the experts entering it in (layer, expert)
// order, and an entering expert's ring entry is emptied.  owner / stamp are
// host copies of the ring; tables are uploaded, the moved experts copied in.
moe_spark_status repin(moe_spark_ctx* ctx, const std::vector<uint8_t>& want, std::vector<int32_t>& owner,
                       std::vector<uint64_t>& stamp) {
    const auto& c = ctx->cfg;
    const int L = c.n_layers, E = c.n_experts, R = c.ring_slots;
    std::vector<int32_t> freed;
    for (int64_t key = 0; key < (int64_t)L * E; ++key)
        if (ctx->slot_of[key] >= 0 && !want[key]) {
            freed.push_back(ctx->slot_of[key]);
            ctx->slot_of[key] = -1;
        }
    std::sort(freed.begin(), freed.end());
    std::vector<std::pair<int32_t, int32_t>> moves;
    size_t nf = 0;
    for (int64_t key = 0; key < (int64_t)L * E; ++key) {
        if (!want[key] || ctx->slot_of[key] >= 0) continue;
        if (nf >= freed.size()) return ctx->fail(MOE_SPARK_E_STATE, "placement: more experts to pin than slots");
        ctx->slot_of[key] = freed[nf++];
        moves.push_back({ctx->slot_of[key], (int32_t)key});
        for (int r = 0; r < R; ++r)
            if (owner[r] == (int32_t)key) {
                owner[r] = -1;
                stamp[r] = 0;
            }
    }
    moe_spark_status st = upload_pinned(ctx, moves);
    if (st != MOE_SPARK_OK) return st;
    ctx->calib_uploads += (int64_t)moves.size();
    HIPCHK(hipMemcpy(ctx->d_slot_of, ctx->slot_of.data(), sizeof(int32_t) * L * E, hipMemcpyHostToDevice));
    HIPCHK(hipMemcpy(ctx->d_ring_owner, owner.data(), sizeof(int32_t) * std::max(R, 1), hipMemcpyHostToDevice));
    HIPCHK(hipMemcpy(ctx->d_ring_stamp, stamp.data(), sizeof(uint64_t) * std::max(R, 1), hipMemcpyHostToDevice));
    return MOE_SPARK_OK;
}

// Host copies of the routing counts and the ring, after all queued work.
moe_spark_status read_tables(moe_spark_ctx* ctx, std::vector<int64_t>& counts, std::vector<int32_t>& owner,
                             std::vector<uint64_t>& stamp) {
    const auto& c = ctx->cfg;
    const int64_t LE = (int64_t)c.n_layers * c.n_experts;
    const int R1 = std::max(c.ring_slots, 1);
    HIPCHK(hipStreamSynchronize(ctx->compute));
    HIPCHK(sync_copies(ctx));
    counts.resize(LE);
    owner.resize(R1);
    stamp.resize(R1);
    HIPCHK(hipMemcpy(counts.data(), ctx->d_counts, sizeof(int64_t) * LE, hipMemcpyDeviceToHost));
    HIPCHK(hipMemcpy(owner.data(), ctx->d_ring_owner, sizeof(int32_t) * R1, hipMemcpyDeviceToHost));
    HIPCHK(hipMemcpy(stamp.data(), ctx->d_ring_stamp, sizeof(uint64_t) * R1, hipMemcpyDeviceToHost));
    return MOE_SPARK_OK;
}

moe_spark_status moe_spark_calibrate(moe_spark_ctx* ctx, int32_t reset_counts) {
    if (!ctx) return MOE_SPARK_E_INVALID;
    moe_spark_status st = ready_check(ctx);
    if (st != MOE_SPARK_OK) return st;
    const auto& c = ctx->cfg;
    const int L = c.n_layers, E = c.n_experts;
    std::vector<int64_t> counts;
    std::vector<int32_t> owner;
    std::vector<uint64_t> stamp;
    st = read_tables(ctx, counts, owner, stamp);
    if (st != MOE_SPARK_OK) return st;
    // target pinned set: per layer, the q_l most-counted experts (count desc, id asc)
    std::vector<uint8_t> want((size_t)L * E, 0);
    std::vector<int> order(E);
    for (int l = 0; l < L; ++l) {
        for (int e = 0; e < E; ++e) order[e] = e;
        const int64_t* cl = counts.data() + (int64_t)l * E;
        std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return cl[a] > cl[b]; });
        const int64_t q = quota(L, c.resident_cap, l);
        for (int64_t i = 0; i < q; ++i) want[(int64_t)l * E + order[i]] = 1;
    }
    st = repin(ctx, want, owner, stamp);
    if (st != MOE_SPARK_OK) return st;
    if (reset_counts) HIPCHK(hipMemset(ctx->d_counts, 0, sizeof(int64_t) * L * E));
    HIPCHK(hipDeviceSynchronize());
    ctx->at_since = 0;
    return MOE_SPARK_OK;
}

// One step of online self-tuning, between two decode tokens.  Per layer, in
// the order (count desc, id asc), the strongest unpinned expert x displaces
// the weakest pinned expert y while 100*count[x] > (100 + hysteresis)*count[y];
// the first pair that fails ends the layer.  Then every count is shifted
// right by decay_shift, so older traffic fades.
moe_spark_status retune(moe_spark_ctx* ctx) {
    const auto& c = ctx->cfg;
    const int L = c.n_layers, E = c.n_experts;
    std::vector<int64_t> counts;
    std::vector<int32_t> owner;
    std::vector<uint64_t> stamp;
    moe_spark_status st = read_tables(ctx, counts, owner, stamp);
    if (st != MOE_SPARK_OK) return st;
    std::vector<uint8_t> want((size_t)L * E);
    for (int64_t key = 0; key < (int64_t)L * E; ++key) want[key] = ctx->slot_of[key] >= 0;
    std::vector<int> order(E), outs, ins;
    int64_t swaps = 0;
    for (int l = 0; l < L; ++l) {
        const int64_t base = (int64_t)l * E;
        for (int e = 0; e < E; ++e) order[e] = e;
        const int64_t* cl = counts.data() + base;
        std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return cl[a] > cl[b]; });
        outs.clear();
        ins.clear();
        for (int i = 0; i < E; ++i)
            if (!want[base + order[i]]) outs.push_back(order[i]);
        for (int i = E - 1; i >= 0; --i)
            if (want[base + order[i]]) ins.push_back(order[i]);
        for (size_t i = 0; i < outs.size() && i < ins.size(); ++i) {
            const int x = outs[i], y = ins[i];
            if (!(100 * cl[x] > (int64_t)(100 + ctx->at_hyst) * cl[y])) break;
            want[base + x] = 1;
            want[base + y] = 0;
            ++swaps;
        }
    }
    if (swaps) {
        st = repin(ctx, want, owner, stamp);
        if (st != MOE_SPARK_OK) return st;
    }
    if (ctx->at_shift) {
        for (auto& v : counts) v >>= ctx->at_shift;
        HIPCHK(hipMemcpy(ctx->d_counts, counts.data(), sizeof(int64_t) * L * E, hipMemcpyHostToDevice));
    }
    HIPCHK(hipDeviceSynchronize());
    ++ctx->retunes;
    ctx->retune_swaps += swaps;
    ctx->at_since = 0;
    return MOE_SPARK_OK;
}

// Before a decode token: retune once `interval` tokens have run since the
// placement last changed.
moe_spark_status maybe_retune(moe_spark_ctx* ctx) {
    if (ctx->at_interval <= 0 || ctx->at_since < ctx->at_interval) return MOE_SPARK_OK;
    return retune(ctx);
}

moe_spark_status moe_spark_set_autotune(moe_spark_ctx* ctx, int32_t interval_tokens, int32_t hysteresis_pct,
                                        int32_t decay_shift) {
    if (!ctx) return MOE_SPARK_E_INVALID;
    if (interval_tokens < 0 || hysteresis_pct < 0 || hysteresis_pct > 100000 || decay_shift < 0 || decay_shift > 62)
        return ctx->fail(MOE_SPARK_E_INVALID, "interval >= 0, hysteresis in [0, 100000] %, decay shift in [0, 62]");
    ctx->at_interval = interval_tokens;
    ctx->at_hyst = hysteresis_pct;
    ctx->at_shift = decay_shift;
    ctx->at_since = 0;
    return MOE_SPARK_OK;
}

moe_spark_status moe_spark_layer_forward(moe_spark_ctx* ctx, int32_t layer, const float* x, float* y,
                                         int32_t n_tokens, const int32_t* bias_row, uint32_t flags,
                                         int32_t* topk_out, float* gates_out) {
    if (!ctx) return MOE_SPARK_E_INVALID;
    const auto& c = ctx->cfg;
    if (layer < 0 || layer >= c.n_layers || n_tokens < 0 || (n_tokens > 0 && (!x || !y)))
        return ctx->fail(MOE_SPARK_E_INVALID, "bad layer, token count or NULL buffer");
    if (flags & ~(MOE_SPARK_PRE_RMSNORM | MOE_SPARK_RESIDUAL)) return ctx->fail(MOE_SPARK_E_INVALID, "unknown flags");
    if ((topk_out == nullptr) != (gates_out == nullptr))
        return ctx->fail(MOE_SPARK_E_INVALID, "topk_out and gates_out go together");
    moe_spark_status st = ready_check(ctx);
    if (st != MOE_SPARK_OK) return st;
    const int norm = (flags & MOE_SPARK_PRE_RMSNORM) != 0, res = (flags & MOE_SPARK_RESIDUAL) != 0;
    if (c.wfmt == MOE_SPARK_W_Q4_0) {
        for (int t = 0; t < n_tokens; ++t) {
            const TokRef tok{nullptr, t};
            const Q4Args a = q4_args(ctx, layer, x, y, tok, tok, bias_row, norm, res, -1, topk_out, gates_out, 0);
            Q4Args ap = a;
            ap.wr_part = ctx->d_router + (int64_t)layer * c.n_experts * c.d_model;
            HIPCHK(launch_q4_router_partial(ap, ctx->compute));
            HIPCHK(launch_q4_gateup(a, ctx->compute));
            HIPCHK(launch_q4_down(a, ctx->compute));
        }
        return MOE_SPARK_OK;
    }
    for (int t = 0; t < n_tokens; ++t) {
        const TokRef tok{nullptr, t};
        const RouteArgs ra = route_args(ctx, layer, x, tok, tok, bias_row, norm, topk_out, gates_out);
        HIPCHK(launch_route(ra, ctx->compute));
        const ExpertArgs ea = expert_args(ctx, layer, x, y, tok, res, 0);
        HIPCHK(launch_gateup(ea, c.wfmt, ctx->compute));
        HIPCHK(launch_down(ea, c.wfmt, ctx->compute));
    }
    return MOE_SPARK_OK;
}

moe_spark_status moe_spark_layer_forward_noalloc(moe_spark_ctx* ctx, int32_t layer, const float* x, float* y,
                                                 int32_t n_tokens, const int32_t* bias_row, uint32_t flags,
                                                 int32_t* topk_out, float* gates_out) {
    if (!ctx) return MOE_SPARK_E_INVALID;
    const auto& c = ctx->cfg;
    if (c.wfmt != MOE_SPARK_W_Q4_0)
        return ctx->fail(MOE_SPARK_E_INVALID, "layer_forward_noalloc runs Q4_0 contexts only");
    if (c.n_experts > kMaxE || c.top_k > kQ4MaxK || c.d_ff > kQF)
        return ctx->fail(MOE_SPARK_E_INVALID, "shape exceeds the no-alloc scratch (%zu bytes)",
                         (size_t)kNoAllocScratchBytes);
    if (layer < 0 || layer >= c.n_layers || n_tokens < 0 || (n_tokens > 0 && (!x || !y)))
        return ctx->fail(MOE_SPARK_E_INVALID, "bad layer, token count or NULL buffer");
    if (flags & ~(MOE_SPARK_PRE_RMSNORM | MOE_SPARK_RESIDUAL)) return ctx->fail(MOE_SPARK_E_INVALID, "unknown flags");
    if ((topk_out == nullptr) != (gates_out == nullptr))
        return ctx->fail(MOE_SPARK_E_INVALID, "topk_out and gates_out go together");
    moe_spark_status st = ready_check(ctx);
    if (st != MOE_SPARK_OK) return st;
    uint8_t* scr = scratch_of(ctx->device);
    if (!scr) return ctx->fail(MOE_SPARK_E_STATE, "no-alloc scratch was not set up on device %d", ctx->device);
    float* pl = reinterpret_cast<float*>(scr + kNoAllocPL);
    float* ps = reinterpret_cast<float*>(scr + kNoAllocPS);
    LayerSel* sel = reinterpret_cast<LayerSel*>(scr + kNoAllocSel);
    uint32_t* pub = reinterpret_cast<uint32_t*>(scr + kNoAllocPub);
    float* h = reinterpret_cast<float*>(scr + kNoAllocH);
    // the publish flag starts at zero (every down launch leaves it zero; this
    // covers the first call on the GPU and a call after an aborted one)
    hipLaunchKernelGGL(noalloc_clear_kernel, dim3(1), dim3(64), 0, ctx->compute, pub);
    HIPCHK(hipGetLastError());
    const int norm = (flags & MOE_SPARK_PRE_RMSNORM) != 0, res = (flags & MOE_SPARK_RESIDUAL) != 0;
    for (int t = 0; t < n_tokens; ++t) {
        const TokRef tok{nullptr, t};
        Q4Args a = q4_args(ctx, layer, x, y, tok, tok, bias_row, norm, res, -1, topk_out, gates_out, 0);
        a.pl = pl;
        a.ps = ps;
        a.sel = sel;
        a.pub = pub;
        a.h = h;
        Q4Args ap = a;
        ap.wr_part = ctx->d_router + (int64_t)layer * c.n_experts * c.d_model;
        HIPCHK(launch_q4_router_partial(ap, ctx->compute));
        HIPCHK(launch_q4_gateup(a, ctx->compute));
        HIPCHK(launch_q4_down(a, ctx->compute));
    }
    return MOE_SPARK_OK;
}

moe_spark_status moe_spark_decode(moe_spark_ctx* ctx, float* x, int32_t n_tokens, const int32_t* bias_row) {
    if (!ctx) return MOE_SPARK_E_INVALID;
    if (n_tokens < 0 || (n_tokens > 0 && !x)) return ctx->fail(MOE_SPARK_E_INVALID, "bad token count or NULL x");
    moe_spark_status st = ready_check(ctx);
    if (st != MOE_SPARK_OK) return st;
    if (!x) return MOE_SPARK_OK;
    if (ctx->stream_decode) {
        if (n_tokens == 0) return MOE_SPARK_OK;
        st = begin_decode(ctx, x, bias_row, n_tokens);
        if (st != MOE_SPARK_OK) return st;
        for (int t = 0; t < n_tokens; ++t) {
            st = maybe_retune(ctx);
            if (st != MOE_SPARK_OK) return st;
            st = launch_token_kernels(ctx, x, bias_row);
            if (st != MOE_SPARK_OK) return st;
            ++ctx->at_since;
        }
        return MOE_SPARK_OK;
    }
    hipGraphExec_t exec;
    st = get_graph(ctx, x, bias_row, 0, &exec);  // n_tokens == 0 only prepares the graph
    if (st != MOE_SPARK_OK || n_tokens == 0) return st;
    st = begin_decode(ctx, x, bias_row, n_tokens);
    if (st != MOE_SPARK_OK) return st;
    for (int t = 0; t < n_tokens; ++t) {
        st = maybe_retune(ctx);
        if (st != MOE_SPARK_OK) return st;
        hipEvent_t& ev = ctx->tok_ev[ctx->tok_launched % kThrottle];
        if (ctx->tok_launched >= kThrottle) HIPCHK(hipEventSynchronize(ev));
        HIPCHK(hipGraphLaunch(exec, ctx->compute));
        HIPCHK(hipEventRecord(ev, ctx->compute));
        ++ctx->tok_launched;
        ++ctx->at_since;
    }
    return MOE_SPARK_OK;
}

moe_spark_status moe_spark_token_forward(moe_spark_ctx* ctx, float* x, const int32_t* bias_row) {
    return moe_spark_decode(ctx, x, 1, bias_row);
}

moe_spark_status moe_spark_decode_batched(moe_spark_ctx* ctx, float* x, int32_t n_tokens, int32_t batch,
                                          const int32_t* bias_row) {
    if (!ctx) return MOE_SPARK_E_INVALID;
    const auto& c = ctx->cfg;
    if (c.wfmt != MOE_SPARK_W_Q4_0) return ctx->fail(MOE_SPARK_E_INVALID, "batched decode needs Q4_0 experts");
    if (batch < 1 || batch > kMaxB) return ctx->fail(MOE_SPARK_E_INVALID, "batch %d outside [1, %d]", batch, kMaxB);
    if (c.resident_cap < (int64_t)c.n_layers * c.n_experts && c.ring_slots < batch * c.top_k)
        return ctx->fail(MOE_SPARK_E_INVALID,
                         "batch %d needs a ring of at least batch * top_k = %d slots below full residency (have %d)",
                         batch, batch * c.top_k, c.ring_slots);
    if (n_tokens < 0 || (n_tokens > 0 && !x)) return ctx->fail(MOE_SPARK_E_INVALID, "bad token count or NULL x");
    moe_spark_status st = ready_check(ctx);
    if (st != MOE_SPARK_OK) return st;
    if (!x) return MOE_SPARK_OK;
    hipGraphExec_t exec = nullptr;
    if (!ctx->stream_decode) {
        st = get_graph(ctx, x, bias_row, batch, &exec);  // n_tokens == 0 only prepares the graph
        if (st != MOE_SPARK_OK) return st;
    }
    if (n_tokens == 0) return MOE_SPARK_OK;
    HIPCHK(launch_qb_begin(batch_io(ctx, x, bias_row, batch), n_tokens, ctx->compute));
    for (int t0 = 0; t0 < n_tokens; t0 += batch) {
        st = maybe_retune(ctx);
        if (st != MOE_SPARK_OK) return st;
        if (exec) {
            hipEvent_t& ev = ctx->tok_ev[ctx->tok_launched % kThrottle];
            if (ctx->tok_launched >= kThrottle) HIPCHK(hipEventSynchronize(ev));
            HIPCHK(hipGraphLaunch(exec, ctx->compute));
            HIPCHK(hipEventRecord(ev, ctx->compute));
            ++ctx->tok_launched;
        } else {
            st = launch_step_kernels(ctx, x, bias_row, batch);
            if (st != MOE_SPARK_OK) return st;
        }
        ctx->at_since += std::min(batch, n_tokens - t0);
    }
    return MOE_SPARK_OK;
}

struct BurstFills {  // lets the fill agent use every copy stream while a prefill runs
    moe_spark_ctx* ctx;
    explicit BurstFills(moe_spark_ctx* c) : ctx(c) { ctx->burst_fills.store(1); }
    ~BurstFills() { ctx->burst_fills.store(0); }
};

// Wait until the prefill host mirror's flag f holds seq (written by the
// first-chunk policy kernel); a device error or 10 s without it fails.
static moe_spark_status wait_host_flag(moe_spark_ctx* ctx, int f, int32_t seq) {
    const int64_t t0 = now_ns();
    for (int polls = 0;; ++polls) {
        if (__atomic_load_n(ctx->h_pstate + f, __ATOMIC_ACQUIRE) == seq) return MOE_SPARK_OK;
        if ((polls & 1023) == 1023) {
            const hipError_t q = hipStreamQuery(ctx->compute);
            if (q != hipSuccess && q != hipErrorNotReady)
                return ctx->fail(MOE_SPARK_E_HIP, "prefill: %s", hipGetErrorString(q));
            if (q == hipSuccess && __atomic_load_n(ctx->h_pstate + f, __ATOMIC_ACQUIRE) != seq)
                return ctx->fail(MOE_SPARK_E_HIP, "prefill: the policy kernel finished without publishing");
            if (now_ns() - t0 > 10000000000ll) return ctx->fail(MOE_SPARK_E_HIP, "prefill: policy results timed out");
        }
        _mm_pause();
    }
}

// Copy the slots of a fill list (count, then (layer*E + expert, global slot)
// pairs, as the prefill policy and prefetch kernels write it) from the host
// arena by the copy stream's DMA engine.
static moe_spark_status dma_fill_list(moe_spark_ctx* ctx, const int32_t* list) {
    const auto& c = ctx->cfg;
    const int nf = std::min(list[0], c.ring_slots);
    const int64_t SB = ctx->slot_bytes;
    for (int j = 0; j < nf; ++j) {
        const int key = list[1 + 2 * j], slot = list[2 + 2 * j];
        if (key < 0 || key >= ctx->n_experts_total || slot < c.resident_cap || slot >= ctx->n_slots)
            return ctx->fail(MOE_SPARK_E_HIP, "a prefill fill list holds an invalid entry");
        HIPCHK(hipMemcpyAsync(ctx->d_slots + (int64_t)slot * SB, ctx->h_arena + (int64_t)key * SB, SB,
                              hipMemcpyHostToDevice, ctx->copy));
    }
    return MOE_SPARK_OK;
}

moe_spark_status moe_spark_prefill(moe_spark_ctx* ctx, float* x, int32_t n_tokens, const int32_t* bias_row) {
    if (!ctx) return MOE_SPARK_E_INVALID;
    const auto& c = ctx->cfg;
    if (c.wfmt != MOE_SPARK_W_Q4_0) return ctx->fail(MOE_SPARK_E_INVALID, "prefill runs the Q4_0 expert format");
    if (c.max_tokens <= 0) return ctx->fail(MOE_SPARK_E_STATE, "prefill needs max_tokens > 0 at create");
    if (n_tokens < 1 || n_tokens > c.max_tokens || !x)
        return ctx->fail(MOE_SPARK_E_INVALID, "n_tokens must be in [1, max_tokens] and x non-NULL");
    moe_spark_status st = ready_check(ctx);
    if (st != MOE_SPARK_OK) return st;
    const BurstFills burst(ctx);
    const int L = c.n_layers, E = c.n_experts, K = c.top_k, R = c.ring_slots;
    const int32_t T = n_tokens;
    int32_t* goff = ctx->h_pmeta;
    int32_t* experts = goff + E + 1;
    int32_t* items = experts + E;
    int32_t* d_goff = ctx->d_pmeta;
    int32_t* d_experts = d_goff + E + 1;
    int32_t* d_items = d_experts + E;
    const bool prefetch = ctx->pf_prefetch && ctx->pull_fills && R > 0;
    HIPCHK(hipMemsetAsync(ctx->d_ppred, 0, sizeof(int32_t) * L * E, ctx->compute));
    if (prefetch) {  // copies of an earlier call that stopped on an error
        HIPCHK(hipEventRecord(ctx->pf_done_ev, ctx->copy));
        HIPCHK(hipStreamWaitEvent(ctx->compute, ctx->pf_done_ev, 0));
    }
    for (int l = 0; l < L; ++l) {
        PfArgs a{};
        a.x = x;
        a.T = T;
        a.layer = l;
        a.L = L;
        a.E = E;
        a.K = K;
        a.norm = 1;
        a.eps = c.rms_eps;
        a.wr = ctx->d_router + (int64_t)l * E * c.d_model;
        a.bias = c.n_bias_rows > 0 ? ctx->d_bias + (int64_t)l * c.n_bias_rows * E : nullptr;
        a.bias_row = bias_row;
        a.n_bias_rows = c.n_bias_rows;
        a.u = ctx->d_pu;
        a.inv = ctx->d_pinv;
        a.logits = ctx->d_plog;
        a.topk = ctx->d_ptopk;
        a.gates = ctx->d_pgate;
        a.hist = ctx->d_phist;
        a.goff = d_goff;
        a.perm = ctx->d_pperm;
        a.apos = ctx->d_papos;
        a.pslot = ctx->d_pslot;
        a.pwait = ctx->d_pwait;
        a.arena = ctx->pull_fills ? ctx->d_arena : nullptr;  // fills pulled by a kernel, else agent copies
        a.pfill = ctx->d_pfill;
        a.h = ctx->d_ph;
        a.y = ctx->d_py;
        a.slots = ctx->d_slots;
        a.slot_bytes = ctx->slot_bytes;
        a.P = c.resident_cap;
        a.n_slots = ctx->n_slots;
        a.ready = ctx->d_ready;
        a.pt = tables(ctx, ctx->pull_fills);
        a.tr_x = ctx->tr_x;
        a.tr_topk = ctx->tr_topk;
        a.tr_gates = ctx->tr_gates;
        a.tr_cap = ctx->tr_cap;
        a.tr_base = ctx->d_cursors + 1;
        a.spin_limit_ticks = ctx->spin_ticks;
        // with prefetch, the routing also predicts the next layer's top-K
        const bool predict = prefetch && l + 1 < L;
        if (predict) {
            a.wr2 = ctx->d_router + (int64_t)(l + 1) * E * c.d_model;
            a.bias2 = c.n_bias_rows > 0 ? ctx->d_bias + (int64_t)(l + 1) * c.n_bias_rows * E : nullptr;
            a.logits2 = ctx->d_plog2;
            a.topk2 = ctx->d_ptopk2;
            a.hist2 = ctx->d_ppred + (int64_t)(l + 1) * E;
            a.pfill2 = ctx->d_pfill2;
        }
        // 1. routing of all tokens; the assignment histogram comes back to
        //    plan the layer while the first chunk's policy runs (and so its
        //    fills start).  With prefetch the policy's fill list and the
        //    prefetch list (when the layer is one chunk) follow, for the
        //    host to hand to the DMA engine.
        HIPCHK(hipMemsetAsync(ctx->d_phist, 0, sizeof(int32_t) * E, ctx->compute));
        HIPCHK(launch_pf_front(a, ctx->compute));
        // the first-chunk policy writes the histogram, then its fill list and
        // the prefetch list, into the mapped host mirror, raising a flag after
        // each; the host reads them there (no copy on the compute stream)
        const int32_t seq = ++ctx->pf_seq;
        a.host_state = ctx->d_pstate;
        a.seq = seq;
        HIPCHK(launch_pf_policy_first(a, ctx->compute));
        a.host_state = nullptr;  // no other kernel writes the mirror
        const int32_t* hist_h = ctx->h_pstate + 2;
        const int32_t* fills_h = hist_h + E;
        const int32_t* pref_h = fills_h + 1 + 2 * kMaxR;
        st = wait_host_flag(ctx, 0, seq);
        if (st != MOE_SPARK_OK) return st;
        // 2. plan: groups in expert order; distinct experts ascending, cut into
        //    chunks of at most R cold (non-pinned) experts, so that every
        //    expert of a chunk sits in the ring while the chunk computes
        goff[0] = 0;
        for (int e = 0; e < E; ++e) goff[e + 1] = goff[e] + hist_h[e];
        struct Chunk {
            int e_begin, e_end, i_begin, i_cold, i_end;  // items [i_begin, i_cold): pinned experts
            int n_cold;                                  // non-pinned experts
        };
        // Within a chunk the GEMM tiles of pinned experts come first and those
        // of cold experts (in fill order) last, so the matrix cores work while
        // the fills cross PCIe.
        std::vector<Chunk> chunks;
        std::vector<int> chunk_experts;
        int ne = 0, ni = 0, cold = 0;
        Chunk cur{0, 0, 0, 0, 0, 0};
        auto close_chunk = [&]() -> bool {
            for (int pass = 0; pass < 2; ++pass) {
                if (pass == 1) cur.i_cold = ni;
                for (int e : chunk_experts) {
                    const bool is_cold = ctx->slot_of[(int64_t)l * E + e] < 0;
                    if (is_cold != (pass == 1)) continue;
                    for (int m0 = 0; m0 < hist_h[e]; m0 += 128) {
                        if (ni >= ctx->pf_max_items) return false;
                        items[2 * ni] = e;
                        items[2 * ni + 1] = m0;
                        ++ni;
                    }
                }
            }
            cur.e_end = ne;
            cur.i_end = ni;
            cur.n_cold = cold;
            if (cur.e_end > cur.e_begin) chunks.push_back(cur);
            cur = Chunk{ne, ne, ni, ni, ni, 0};
            chunk_experts.clear();
            cold = 0;
            return true;
        };
        for (int e = 0; e < E; ++e) {
            if (hist_h[e] == 0) continue;
            const bool is_cold = ctx->slot_of[(int64_t)l * E + e] < 0;
            if (is_cold && cold == R && !close_chunk())
                return ctx->fail(MOE_SPARK_E_STATE, "prefill work list overflow");
            cold += is_cold;
            experts[ne++] = e;
            chunk_experts.push_back(e);
        }
        if (!close_chunk()) return ctx->fail(MOE_SPARK_E_STATE, "prefill work list overflow");
        const size_t meta = (size_t)(2 * E + 1) + 2 * (size_t)ni;
        // 3. sort assignments (the launch also copies the plan to the
        //    device), run each chunk, combine
        {
            PfArgs sa = a;
            sa.meta_host = ctx->dm_pmeta;
            sa.n_meta = (int32_t)meta;
            HIPCHK(launch_pf_scatter(sa, ctx->compute));
        }
        // Prefetch: the layer's ring data (this layer's prefetched experts,
        // copied during the layer before, and the first chunk's fills) come
        // by DMA on the copy stream; the first launch that touches slot data
        // waits for them.  After the first layer, the first chunk's fills are
        // mispredictions (few), so the chunk's pinned and cold experts run in
        // one launch; the first layer pulls its fills during its pinned
        // experts' GEMMs.
        const bool dma_first = prefetch && l > 0;
        if (prefetch) {  // the lists are on the host
            st = wait_host_flag(ctx, 1, seq);
            if (st != MOE_SPARK_OK) return st;
        }
        if (dma_first) {
            st = dma_fill_list(ctx, fills_h);
            if (st != MOE_SPARK_OK) return st;
            HIPCHK(hipEventRecord(ctx->pf_done_ev, ctx->copy));
            HIPCHK(hipStreamWaitEvent(ctx->compute, ctx->pf_done_ev, 0));
        }
        // Per chunk: its policy (the first chunk's ran already); the GEMMs of
        // its pinned experts, whose gate/up launch also pulls the chunk's
        // fills; then the GEMMs of its cold experts.  With agent copies the
        // cold experts' work-groups wait for each fill's ready flag.
        // With prefetch, the next layer's predicted experts go through the
        // prefetch rule after the layer's last policy run (in the first
        // policy kernel when the layer is one chunk), taking at most the
        // R - n_cold ring entries that the last chunk does not use (the least
        // recently used), so no slot that this layer still reads or fills is
        // overwritten; the host hands their copies to the DMA engine, which
        // runs them beside the rest of this layer and the next one's routing.
        bool late_list = false;
        for (const Chunk& ch : chunks) {
            PfArgs b = a;
            if (&ch != &chunks[0]) {
                b.pf_experts = d_experts + ch.e_begin;
                b.n_pf_experts = ch.e_end - ch.e_begin;
                HIPCHK(launch_pf_policy(b, ctx->compute));
                const int pf_budget = R - ch.n_cold;
                if (predict && &ch == &chunks.back() && pf_budget > 0) {
                    PfArgs q = a;
                    q.pf_budget = pf_budget;
                    HIPCHK(launch_pf_prefetch(q, ctx->compute));
                    HIPCHK(hipMemcpyAsync(ctx->h_pfill2, ctx->d_pfill2, sizeof(int32_t) * (1 + 2 * kMaxR),
                                          hipMemcpyDeviceToHost, ctx->compute));
                    HIPCHK(hipEventRecord(ctx->pf_q_ev, ctx->compute));
                    late_list = true;
                }
            }
            b.items = d_items + 2 * ch.i_begin;
            if (dma_first && &ch == &chunks[0]) {
                b.n_items = ch.i_end - ch.i_begin;
                b.n_fill_x = 0;
                HIPCHK(launch_pf_gemms(b, ctx->compute));
                continue;
            }
            b.n_items = ch.i_cold - ch.i_begin;
            b.n_fill_x = b.arena ? ctx->pf_fill_cols : 0;
            HIPCHK(launch_pf_gemms(b, ctx->compute));
            b.items = d_items + 2 * ch.i_cold;
            b.n_items = ch.i_end - ch.i_cold;
            b.n_fill_x = 0;
            HIPCHK(launch_pf_gemms(b, ctx->compute));
        }
        HIPCHK(launch_pf_combine(a, ctx->compute));
        if (predict) {
            // the layer is queued: the prefetch copies go to the DMA engine
            if (late_list) HIPCHK(hipEventSynchronize(ctx->pf_q_ev));
            if (late_list || chunks.size() == 1) {
                st = dma_fill_list(ctx, late_list ? ctx->h_pfill2 : pref_h);
                if (st != MOE_SPARK_OK) return st;
            }
        }
    }
    HIPCHK(launch_cursor_add(ctx->d_cursors + 1, T, ctx->compute));  // trace rows continue after the batch
    return MOE_SPARK_OK;
}

moe_spark_status moe_spark_set_trace(moe_spark_ctx* ctx, float* x_layers, int32_t* topk, float* gates,
                                     int64_t cap_tokens) {
    if (!ctx) return MOE_SPARK_E_INVALID;
    if (cap_tokens < 0 || ((topk == nullptr) != (gates == nullptr)))
        return ctx->fail(MOE_SPARK_E_INVALID, "bad trace buffers");
    drop_graphs(ctx);
    ctx->tr_x = x_layers;
    ctx->tr_topk = topk;
    ctx->tr_gates = gates;
    ctx->tr_cap = (x_layers || topk) ? cap_tokens : 0;
    HIPCHK(hipMemset(ctx->d_cursors + 1, 0, sizeof(int32_t)));
    return MOE_SPARK_OK;
}

moe_spark_status moe_spark_set_prefetch(moe_spark_ctx* ctx, int32_t enable) {
    if (!ctx) return MOE_SPARK_E_INVALID;
    if (enable && !ctx->pull_fills)
        return ctx->fail(MOE_SPARK_E_STATE, "prefetch needs fills pulled from the host arena by the kernels");
    if (enable && ctx->cfg.max_tokens <= 0) return ctx->fail(MOE_SPARK_E_STATE, "prefetch needs max_tokens > 0");
    ctx->pf_prefetch = enable != 0;
    return MOE_SPARK_OK;
}

moe_spark_status moe_spark_get_prefetch_hist(moe_spark_ctx* ctx, int32_t* out) {
    if (!ctx || !out) return MOE_SPARK_E_INVALID;
    if (!ctx->d_ppred) return ctx->fail(MOE_SPARK_E_STATE, "prefill is not enabled (max_tokens = 0)");
    HIPCHK(hipStreamSynchronize(ctx->compute));
    HIPCHK(hipMemcpy(out, ctx->d_ppred, sizeof(int32_t) * ctx->cfg.n_layers * ctx->cfg.n_experts,
                     hipMemcpyDeviceToHost));
    return MOE_SPARK_OK;
}

moe_spark_status moe_spark_get_stats(moe_spark_ctx* ctx, moe_spark_stats* out) {
    if (!ctx || !out) return MOE_SPARK_E_INVALID;
    HIPCHK(hipStreamSynchronize(ctx->compute));
    int64_t s[DS_N];
    HIPCHK(hipMemcpy(s, ctx->d_stats, sizeof s, hipMemcpyDeviceToHost));
    out->accesses = s[DS_ACC];
    out->pinned_hits = s[DS_PIN];
    out->cold_hits = s[DS_COLD];
    out->ring_hits = s[DS_RING];
    out->fills = s[DS_FILL];
    out->evictions = s[DS_EVICT];
    out->prefetches = s[DS_PREF];
    out->h2d_bytes = s[DS_H2D];
    out->fill_ns_sum = ctx->fill_ns_sum.load();
    out->fill_ns_max = ctx->fill_ns_max.load();
    out->calib_uploads = ctx->calib_uploads;
    out->retunes = ctx->retunes;
    out->retune_swaps = ctx->retune_swaps;
    out->tokens = s[DS_TOKENS];
    return MOE_SPARK_OK;
}

moe_spark_status moe_spark_reset_stats(moe_spark_ctx* ctx) {
    if (!ctx) return MOE_SPARK_E_INVALID;
    HIPCHK(hipStreamSynchronize(ctx->compute));
    HIPCHK(hipMemset(ctx->d_stats, 0, sizeof(int64_t) * DS_N));
    HIPCHK(hipDeviceSynchronize());
    ctx->fill_ns_sum.store(0);
    ctx->fill_ns_max.store(0);
    ctx->calib_uploads = 0;
    ctx->retunes = 0;
    ctx->retune_swaps = 0;
    return MOE_SPARK_OK;
}

moe_spark_status moe_spark_get_placement(moe_spark_ctx* ctx, int32_t* slot_of, int32_t* ring_owner,
                                         int64_t* ring_stamp, int64_t* counts) {
    if (!ctx) return MOE_SPARK_E_INVALID;
    const auto& c = ctx->cfg;
    const int64_t LE = (int64_t)c.n_layers * c.n_experts;
    HIPCHK(hipStreamSynchronize(ctx->compute));
    if (slot_of) HIPCHK(hipMemcpy(slot_of, ctx->d_slot_of, sizeof(int32_t) * LE, hipMemcpyDeviceToHost));
    if (ring_owner && c.ring_slots > 0)
        HIPCHK(hipMemcpy(ring_owner, ctx->d_ring_owner, sizeof(int32_t) * c.ring_slots, hipMemcpyDeviceToHost));
    if (ring_stamp && c.ring_slots > 0)
        HIPCHK(hipMemcpy(ring_stamp, ctx->d_ring_stamp, sizeof(int64_t) * c.ring_slots, hipMemcpyDeviceToHost));
    if (counts) HIPCHK(hipMemcpy(counts, ctx->d_counts, sizeof(int64_t) * LE, hipMemcpyDeviceToHost));
    return MOE_SPARK_OK;
}

moe_spark_status moe_spark_get_events(moe_spark_ctx* ctx, moe_spark_event* out, int64_t cap, int64_t* n_total) {
    if (!ctx || cap < 0 || (cap > 0 && !out)) return MOE_SPARK_E_INVALID;
    HIPCHK(hipStreamSynchronize(ctx->compute));
    int64_t n = 0;
    HIPCHK(hipMemcpy(&n, ctx->d_n_events, sizeof n, hipMemcpyDeviceToHost));
    if (n_total) *n_total = n;
    const int64_t m = std::min(std::min(n, cap), ctx->cfg.event_cap);
    if (m > 0) HIPCHK(hipMemcpy(out, ctx->d_events, sizeof(moe_spark_event) * m, hipMemcpyDeviceToHost));
    return MOE_SPARK_OK;
}

moe_spark_status moe_spark_synchronize(moe_spark_ctx* ctx) {
    if (!ctx) return MOE_SPARK_E_INVALID;
    HIPCHK(hipStreamSynchronize(ctx->compute));
    HIPCHK(sync_copies(ctx));
    int32_t e = 0;
    HIPCHK(hipMemcpy(&e, ctx->d_error, sizeof e, hipMemcpyDeviceToHost));
    if (e & ERR_FILL_TIMEOUT) return ctx->fail(MOE_SPARK_E_HIP, "a cold-expert fill did not arrive in time");
    if (e & ERR_BAD_SLOT) return ctx->fail(MOE_SPARK_E_HIP, "an expert kernel was handed an invalid slot");
    if (e) return ctx->fail(MOE_SPARK_E_HIP, "device error flags 0x%x", e);
    if (ctx->agent_error.load()) return ctx->fail(MOE_SPARK_E_HIP, "fill agent: a host-to-device copy failed");
    return MOE_SPARK_OK;
}

moe_spark_status moe_spark_time_expert_kernels(moe_spark_ctx* ctx, int32_t iters, float* us_gateup, float* us_down,
                                               float* us_route) {
    if (!ctx || iters <= 0) return MOE_SPARK_E_INVALID;
    moe_spark_status st = ready_check(ctx);
    if (st != MOE_SPARK_OK) return st;
    const auto& c = ctx->cfg;
    const int L = c.n_layers;
    HIPCHK(hipStreamSynchronize(ctx->compute));
    hipEvent_t e0, e1, e2;
    HIPCHK(hipEventCreate(&e0));
    HIPCHK(hipEventCreate(&e1));
    HIPCHK(hipEventCreate(&e2));
    hipEvent_t e3;
    HIPCHK(hipEventCreate(&e3));
    const TokRef tok{nullptr, 0};
    const bool q4 = c.wfmt == MOE_SPARK_W_Q4_0;
    float* xs = ctx->d_xscratch;
    HIPCHK(hipEventRecord(e0, ctx->compute));
    for (int it = 0; it < iters; ++it)
        for (int l = 0; l < L; ++l) {
            if (q4) {
                HIPCHK(launch_q4_gateup(q4_args(ctx, l, xs, xs, tok, tok, nullptr, 1, 1, -1, nullptr, nullptr, 1),
                                        ctx->compute));
            } else {
                HIPCHK(launch_gateup(expert_args(ctx, l, xs, xs, tok, 1, 0), c.wfmt, ctx->compute));
            }
        }
    HIPCHK(hipEventRecord(e1, ctx->compute));
    for (int it = 0; it < iters; ++it)
        for (int l = 0; l < L; ++l) {
            if (q4) {
                HIPCHK(launch_q4_down(q4_args(ctx, l, xs, xs, tok, tok, nullptr, 1, 1, l + 1 < L ? l + 1 : -1,
                                              nullptr, nullptr, 1),
                                      ctx->compute));
            } else {
                HIPCHK(launch_down(expert_args(ctx, l, xs, xs, tok, 1, 0), c.wfmt, ctx->compute));
            }
        }
    HIPCHK(hipEventRecord(e2, ctx->compute));
    if (q4)
        for (int it = 0; it < iters; ++it)
            for (int l = 0; l < L; ++l)
                HIPCHK(launch_q4_router_partial(q4_args(ctx, l, xs, xs, tok, tok, nullptr, 1, 1, l, nullptr, nullptr, 1),
                                                ctx->compute));
    HIPCHK(hipEventRecord(e3, ctx->compute));
    HIPCHK(hipEventSynchronize(e3));
    float ms1 = 0, ms2 = 0, ms3 = 0;
    HIPCHK(hipEventElapsedTime(&ms1, e0, e1));
    HIPCHK(hipEventElapsedTime(&ms2, e1, e2));
    HIPCHK(hipEventElapsedTime(&ms3, e2, e3));
    hipEventDestroy(e0);
    hipEventDestroy(e1);
    hipEventDestroy(e2);
    hipEventDestroy(e3);
    const float n = (float)iters * L;
    if (us_gateup) *us_gateup = ms1 * 1000.0f / n;
    if (us_down) *us_down = ms2 * 1000.0f / n;
    if (us_route) *us_route = q4 ? ms3 * 1000.0f / n : -1.0f;
    return MOE_SPARK_OK;
}

moe_spark_status moe_spark_time_stream_probe(moe_spark_ctx* ctx, int32_t iters, float* us) {
    if (!ctx || iters <= 0 || !us) return MOE_SPARK_E_INVALID;
    moe_spark_status st = ready_check(ctx);
    if (st != MOE_SPARK_OK) return st;
    const auto& c = ctx->cfg;
    if (c.wfmt != MOE_SPARK_W_Q4_0) return ctx->fail(MOE_SPARK_E_INVALID, "the streaming probe reads Q4_0 slots");
    if (ctx->n_slots < c.top_k) return ctx->fail(MOE_SPARK_E_STATE, "the streaming probe reads top_k slots");
    static_assert(kQF / kGURows * kQ4MaxK <= kQD, "probe output fits the scratch row");
    HIPCHK(hipStreamSynchronize(ctx->compute));
    hipEvent_t e0, e1;
    HIPCHK(hipEventCreate(&e0));
    HIPCHK(hipEventCreate(&e1));
    uint32_t* out = reinterpret_cast<uint32_t*>(ctx->d_xscratch);
    HIPCHK(hipEventRecord(e0, ctx->compute));
    for (int it = 0; it < iters; ++it)
        HIPCHK(launch_q4_stream_probe(ctx->d_slots, ctx->slot_bytes, c.top_k, out, ctx->compute));
    HIPCHK(hipEventRecord(e1, ctx->compute));
    HIPCHK(hipEventSynchronize(e1));
    float ms = 0;
    HIPCHK(hipEventElapsedTime(&ms, e0, e1));
    hipEventDestroy(e0);
    hipEventDestroy(e1);
    *us = ms * 1000.0f / (float)iters;
    return MOE_SPARK_OK;
}

}  // extern "C"
