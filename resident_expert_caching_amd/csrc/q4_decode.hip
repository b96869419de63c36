// gfx950 Q4_0 decode kernels: one token-layer is two launches.
//
//   gateup  every work-group rebuilds the router logits from the partial
//           dot products the previous launch left behind, runs the top-k and
//           the renormalised softmax itself ("Luce Spark runs 35B MoE models
//           on 16GB GPU without speed loss", opening paragraph: each token
//           picks about 8 of 256 experts), looks its expert up in the slot
//           table, and computes h = silu(Wg u) * (Wu u) for 16 rows of one
//           expert.  Work-group (0,0) also runs the placement policy of the
//           same page's paragraph "The key components" — per-expert counts,
//           pinned set, the LRU spare-slot ring and the fill request — and
//           publishes the slot of every cold expert; only work-groups of cold
//           experts wait for that, and for the fill to land.
//   down    the down GEMV of all K experts for 16 output rows, the
//           gate-weighted combine in rank order, the residual, and the
//           router partial logits of the next layer over those 16 rows.
//
// A router logit l_e = inv_rms * sum_i Wr[e][i] x_i + b_e is assembled from
// kNP partial sums over 16-row slices of x, each written by the work-group
// that produced those rows, so the router never needs a launch of its own.
// Reductions have fixed trees and fixed orders; there are no floating-point
// atomics; the slot a weight is read from never changes the arithmetic, so
// outputs are bit-identical at every residency (same paragraph: full
// residency is bit-identical to all-GPU execution).
//
// Q4_0 inner product per row: sum_i s (q_i - 8) u_i = s (sum_i q_i u_i - 8 U_b)
// with U_b the block's activation sum, so the offset and the scale leave the
// inner loop.
#include <hip/hip_runtime.h>
#include <math.h>

#include "device_common.h"
#include "internal.h"
#include "policy.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
static_assert(kNP == 128, "the gate/up kernel sums the partial squares with two loads per lane");

__device__ __forceinline__ bool spin_expired(const Q4Args& a, uint64_t t0) {
    return wall_clock64() - t0 > a.spin_limit_ticks ||
           (__hip_atomic_load(a.pt.error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & ERR_FILL_TIMEOUT);
}

// Partial router logits over one 16-row slice: pl[p][e] = sum_i Wr[e][16p+i] xs[i]
// and ps[p] = sum_i xs[i]^2.  wpre holds this thread's first expert's weights.
__device__ __forceinline__ void router_partial(const Q4Args& a, int p, const float* xs, const f32x4* wpre) {
    const int t = threadIdx.x, E = a.E;
    for (int e = t; e < E; e += kThreads) {
        f32x4 w[4];
        if (e == t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = wpre[i];
        } else {
            const f32x4* w4 = reinterpret_cast<const f32x4*>(a.wr_part + ((int64_t)p * E + e) * kRW);
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = w4[i];
        }
        float q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            q[i] = (w[i].x * xs[4 * i] + w[i].y * xs[4 * i + 1]) + (w[i].z * xs[4 * i + 2] + w[i].w * xs[4 * i + 3]);
        a.pl[(int64_t)p * E + e] = (q[0] + q[1]) + (q[2] + q[3]);
    }
    if (t == 0) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < kRW; ++i) s += xs[i] * xs[i];
        a.ps[p] = s;
    }
}

__device__ __forceinline__ void load_wpre(const Q4Args& a, int p, f32x4* wpre) {
    const int t = threadIdx.x;
    if (a.wr_part && t < a.E) {
        const f32x4* w4 = reinterpret_cast<const f32x4*>(a.wr_part + ((int64_t)p * a.E + t) * kRW);
#pragma unroll
        for (int i = 0; i < 4; ++i) wpre[i] = w4[i];
    }
}

// ---------------------------------------------------------------- router partials (first layer)

// Grid kNP.  Work-group p reads rows 16p..16p+15 of the token's x.
__global__ __launch_bounds__(kThreads) void q4_router_partial_kernel(Q4Args a) {
    const int p = blockIdx.x, t = threadIdx.x;
    f32x4 wpre[4];
    load_wpre(a, p, wpre);
    __shared__ float xs[kRW];
    if (t < kRW) xs[t] = a.x_base[(int64_t)tok_value(a.tok) * kQD + p * kRW + t];
    __syncthreads();
    router_partial(a, p, xs, wpre);
}

// ---------------------------------------------------------------- placement policy

// Single wave of work-group (0,0): counts, slot lookup, the LRU ring and fill
// requests, in rank order; then the selection is published for the cold
// experts' work-groups and the down launch.  sel_e, gk and sof live in LDS.
__device__ void run_policy(const Q4Args& a, const int* sel_e, const float* gk, const int32_t* sof, int tok,
                           float inv, int32_t* r_owner, uint64_t* r_stamp, uint64_t* r_seq) {
    const int lane = threadIdx.x;
    const PolicyTables& pt = a.pt;
    const int K = a.K, E = a.E;
    const int32_t kbase = a.layer * E;
    int my_slot = -1;
    uint64_t my_wait = 0;
    int any_cold = 0;
    for (int k = 0; k < K; ++k) any_cold |= sof[sel_e[k]] < 0;
    RingState rs{};
    if (!any_cold) {
        if (lane < K) my_slot = sof[sel_e[lane]];
        rs.n_pin = K;
    } else {
        ring_load(pt, r_owner, r_stamp, r_seq, rs);
#pragma nounroll
        for (int k = 0; k < K; ++k) {
            int slot;
            uint64_t wseq;
            ring_access(pt, a.layer, sel_e[k], sof[sel_e[k]], r_owner, r_stamp, r_seq, rs, slot, wseq);
            if (lane == k) {
                my_slot = slot;
                my_wait = wseq;
            }
        }
        ring_store(pt, r_owner, r_stamp, r_seq, rs);
    }
    if (lane < K) {
        const int myk = sel_e[lane];
        const float myg = gk[lane];
        atomicAdd(reinterpret_cast<unsigned long long*>(pt.counts + kbase + myk), 1ull);
        a.sel->idx[lane] = myk;
        a.sel->slot[lane] = my_slot;
        a.sel->gate[lane] = myg;
        a.sel->wait[lane] = my_wait;
        if (a.tr_topk) {
            const int ttok = tok_value(a.trace_tok);
            if (ttok < a.tr_cap) {
                const int64_t o = ((int64_t)ttok * a.L + a.layer) * K + lane;
                a.tr_topk[o] = myk;
                a.tr_gates[o] = myg;
            }
        }
        if (a.topk_out) {
            a.topk_out[(int64_t)tok * K + lane] = myk;
            a.gates_out[(int64_t)tok * K + lane] = myg;
        }
    }
    if (lane == 0) a.sel->inv_rms = inv;
    stats_flush(pt, K, rs);
    if (any_cold) {
        // only work-groups of cold experts read the selection inside this
        // launch; the down launch sees it at the kernel boundary
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        if (lane == 0) __hip_atomic_store(a.pub, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------- gate/up

// pv[j] = partial-logit row rg + 4j, experts e4..e4+3, loads issued from j = S on
template <int S>
__device__ __forceinline__ void load_partials(f32x4* pv, const float* pl, int rg, int E, int e4) {
#pragma unroll
    for (int jj = 0; jj < kNP / 4; ++jj) {
        const int j = (jj + S) & (kNP / 4 - 1);
        pv[j] = *reinterpret_cast<const f32x4*>(pl + (int64_t)(rg + 4 * j) * E + e4);
    }
}

// Grid (f/16, K).  Work-group (g, k) owns rows 16g..16g+15 of the gate and up
// matrices of the rank-k expert: waves 0, 1 gate rows, waves 2, 3 up rows,
// 8 rows per wave, lane b = Q4_0 block b along d.  Slot chunk g (36,864 B):
// codes at ((w*8 + i)*64 + b)*16, scales at 32768 + (w*64 + b)*16 + 2i, so
// every load of a wave is one coalesced 1 KiB line.
__global__ __launch_bounds__(kThreads) void q4_gateup_kernel(Q4Args a) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int g = blockIdx.x, k = blockIdx.y;
    const int E = a.E, K = a.K;
    const int tok = tok_value(a.tok);

    __shared__ int32_t sof[kMaxE];
    __shared__ __align__(16) float xt[kQD / 32 * 36];
    __shared__ __align__(16) uint64_t kpad[kThreads];
    __shared__ __align__(16) uint64_t cand[kMaxE / 64 * kQ4MaxK + 16];
    __shared__ int s_e[kMaxK];
    __shared__ float s_l[kMaxK];
    __shared__ float s_g[kMaxK];
    __shared__ float s_z;
    __shared__ int s_slot;
    __shared__ unsigned long long s_wseq;
    __shared__ float red[32];
    __shared__ int32_t r_owner[kMaxR];
    __shared__ uint64_t r_stamp[kMaxR];
    __shared__ uint64_t r_seq[kMaxR];

    // Every global load the routing needs is issued before the first LDS
    // store, so their latencies overlap: x, the slot-table row, the partial
    // sums of squares, the partial logits of this wave's first 64-expert
    // chunk, and the bias row index, then the bias values that depend on it.
    // Wave w owns chunk w (and w+4, ... past 256 experts): lane l sums the
    // partial rows l/16, l/16 + 4, ... of experts 64c + 4(l%16) .. +3, the
    // four row groups meet in a butterfly, and the lane keeps the logit of
    // expert 64c + 4(l%16) + l/16.
    const f32x4* x4 = reinterpret_cast<const f32x4*>(a.x_base + (int64_t)tok * kQD);
    const f32x4 xv0 = x4[t], xv1 = x4[t + kThreads];
    const int32_t sof0 = t < E ? a.pt.slot_of[(int64_t)a.layer * E + t] : -1;
    const float ps0 = a.ps[lane], ps1 = a.ps[lane + 64];
    const int e4 = 64 * w + 4 * (lane & 15), rg = lane >> 4;
    f32x4 pv[kNP / 4];
    if (e4 < E) {
        // the 32 work-groups on one XCD start at 8 different rows, so they do
        // not all ask the XCD's L2 for the same lines at the same moment (the
        // sum below still runs in row order)
        switch (((g >> 3) + k) & 7) {
            case 0: load_partials<0>(pv, a.pl, rg, E, e4); break;
            case 1: load_partials<4>(pv, a.pl, rg, E, e4); break;
            case 2: load_partials<8>(pv, a.pl, rg, E, e4); break;
            case 3: load_partials<12>(pv, a.pl, rg, E, e4); break;
            case 4: load_partials<16>(pv, a.pl, rg, E, e4); break;
            case 5: load_partials<20>(pv, a.pl, rg, E, e4); break;
            case 6: load_partials<24>(pv, a.pl, rg, E, e4); break;
            default: load_partials<28>(pv, a.pl, rg, E, e4); break;
        }
    }
    const float* brow = nullptr;
    if (a.bias) {
        int row = a.bias_row ? a.bias_row[tok] : 0;
        row = row < 0 ? 0 : (row >= a.n_bias_rows ? a.n_bias_rows - 1 : row);
        brow = a.bias + (int64_t)row * E;
    }
    const float b0 = (brow && e4 + rg < E) ? brow[e4 + rg] : 0.0f;

    // x is transposed through LDS: Q4_0 block b (32 floats) sits at float
    // 36*b, so the per-lane 16-byte reads of a block are free of bank conflicts.
    *reinterpret_cast<f32x4*>(&xt[36 * (t >> 3) + 4 * (t & 7)]) = xv0;
    *reinterpret_cast<f32x4*>(&xt[36 * ((t + kThreads) >> 3) + 4 * (t & 7)]) = xv1;
    if (t < E) sof[t] = sof0;
    for (int e = t + kThreads; e < E; e += kThreads) sof[e] = a.pt.slot_of[(int64_t)a.layer * E + e];
    // 1 / rms, in every wave
    const float ss = wave_sum(ps0 + ps1);
    const float inv = a.norm ? 1.0f / sqrtf(ss / (float)kQD + a.eps) : 1.0f;
    // logit = inv * (sum of the 128 partials: 32 in row order per lane, then
    // the four row groups) + bias; every lane of a row-group quartet ends
    // with the same bits, since each butterfly step adds the same two values
    const int n_chunks = (E + 63) >> 6;
    for (int c = w; c < n_chunks; c += 4) {
        const int ec = 64 * c + 4 * (lane & 15);
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if (ec < E) {
            if (c != w) {  // chunks past the first 256 experts
#pragma unroll
                for (int j = 0; j < kNP / 4; ++j)
                    pv[j] = *reinterpret_cast<const f32x4*>(a.pl + (int64_t)(rg + 4 * j) * E + ec);
            }
#pragma unroll
            for (int j = 0; j < kNP / 4; ++j) acc += pv[j];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[q] += __shfl_xor(acc[q], 16, 64);
            acc[q] += __shfl_xor(acc[q], 32, 64);
        }
        const int e = ec + rg;
        const float bias = c == w ? b0 : ((brow && e < E) ? brow[e] : 0.0f);
        const float v = (rg == 0 ? acc.x : rg == 1 ? acc.y : rg == 2 ? acc.z : acc.w) * inv + bias;
        topk_rank_chunk(e < E ? topk_key(v, e) : 0ull, c, K, kpad, cand);
    }
    topk_merge(n_chunks, K, cand, s_e, s_l);
    f32x4 xx[8];  // this lane's Q4_0 block of x
#pragma unroll
    for (int j = 0; j < 8; ++j) xx[j] = *reinterpret_cast<const f32x4*>(&xt[36 * lane + 4 * j]);

    if (w == 0) {
        if (g == 0 && k == 0 && !a.replay) {
            // gates: softmax over the chosen logits, shifted by the largest
            if (lane < K) s_g[lane] = expf(s_l[lane] - s_l[0]);
            if (lane == 0) {
                float z = 0.0f;
                for (int kk = 0; kk < K; ++kk) z += s_g[kk];
                s_z = z;
            }
            if (lane < K) s_g[lane] = s_g[lane] / s_z;
            if (a.tr_x) {
                const int ttok = tok_value(a.trace_tok);
                if (ttok < a.tr_cap) {
                    f32x4* t4 = reinterpret_cast<f32x4*>(a.tr_x + ((int64_t)ttok * a.L + a.layer) * kQD);
#pragma unroll
                    for (int j = 0; j < 8; ++j) t4[lane * 8 + j] = xx[j];
                }
            }
            run_policy(a, s_e, s_g, sof, tok, inv, r_owner, r_stamp, r_seq);
        }
    }
    __syncthreads();

    int slot;
    uint64_t wseq = 0;
    if (a.replay) {
        slot = a.sel->slot[k];
    } else {
        slot = sof[s_e[k]];
        if (slot < 0) {  // cold expert: take the slot work-group (0,0) chose
            if (t == 0) {
                const uint64_t t0 = wall_clock64();
                while (__hip_atomic_load(a.pub, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
                    __builtin_amdgcn_s_sleep(1);
                    if (spin_expired(a, t0)) {
                        atomicOr(a.pt.error, (int)ERR_FILL_TIMEOUT);
                        break;
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                s_slot = a.sel->slot[k];
                s_wseq = a.sel->wait[k];
            }
            __syncthreads();
            slot = s_slot;
            wseq = s_wseq;
        }
    }
    if (slot < 0 || slot >= a.n_slots) {  // never expected: refuse rather than fault
        if (t == 0) atomicOr(a.pt.error, (int)ERR_BAD_SLOT);
        return;
    }
    // A fill issued for this token: in pull mode this expert's work-groups copy
    // it from the host arena themselves (below); otherwise wait for the host
    // agent's copy to land.
    const bool pull = a.pt.pull && wseq && slot >= a.P;
    if (wseq && slot >= a.P && !pull) {
        if (t == 0) {
            const uint64_t* flag = a.ready + (slot - a.P);
            const uint64_t t0 = wall_clock64();
            int polls = 0;
            while (__hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM) < wseq) {
                fill_poll_pause(polls);
                if (spin_expired(a, t0)) {
                    atomicOr(a.pt.error, (int)ERR_FILL_TIMEOUT);
                    break;
                }
            }
        }
        __syncthreads();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
    }

    const int64_t key = (int64_t)a.layer * E + s_e[k];
    const uint8_t* chunk = (pull ? a.arena + key * a.slot_bytes : a.slots + (int64_t)slot * a.slot_bytes) +
                           (int64_t)g * kGUChunk;
    const u32x4* cp = reinterpret_cast<const u32x4*>(chunk) + w * 8 * 64 + lane;
    u32x4 c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = __builtin_nontemporal_load(cp + i * 64);
    const u32x4 sc = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(chunk + 32768) + w * 64 + lane);
    if (pull) {
        // the fill: this chunk of gate/up rows as read, plus 1/32 of the down
        // region, into the ring slot (the down launch and later ring hits
        // read the slot; nothing else reads it during this launch)
        uint8_t* dst = a.slots + (int64_t)slot * a.slot_bytes;
        u32x4* dp = reinterpret_cast<u32x4*>(dst + (int64_t)g * kGUChunk) + w * 8 * 64 + lane;
#pragma unroll
        for (int i = 0; i < 8; ++i) __builtin_nontemporal_store(c[i], dp + i * 64);
        __builtin_nontemporal_store(sc, reinterpret_cast<u32x4*>(dst + (int64_t)g * kGUChunk + 32768) + w * 64 + lane);
        constexpr int kDownShare = (int)((kQ4SlotBytes - kGURegion) / (kQF / kGURows) / 16);  // 16-byte words
        const u32x4* hs = reinterpret_cast<const u32x4*>(a.arena + key * a.slot_bytes + kGURegion) + g * kDownShare;
        u32x4* ds = reinterpret_cast<u32x4*>(dst + kGURegion) + g * kDownShare;
        for (int i = t; i < kDownShare; i += kThreads) __builtin_nontemporal_store(__builtin_nontemporal_load(hs + i), ds + i);
    }

    f32x4 uu[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) uu[j] = xx[j] * inv;
    f16x2 ua[16];
    const float UO = kQ4Offset * q4_pairs(uu, ua);

    const uint32_t sw[4] = {sc.x, sc.y, sc.z, sc.w};
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float s = half_bits_to_float(sw[i >> 1] >> ((i & 1) * 16));
        v[i] = s * (q4_dot(c[i], ua) - UO);
    }
    // 8 rows x 64 lanes -> one row per group of 8 lanes (fixed tree)
    {
        const bool h32 = lane & 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float send = h32 ? v[q] : v[q + 4];
            const float keep = h32 ? v[q + 4] : v[q];
            v[q] = keep + __shfl_xor(send, 32, 64);
        }
        const bool h16 = lane & 16;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const float send = h16 ? v[q] : v[q + 2];
            const float keep = h16 ? v[q + 2] : v[q];
            v[q] = keep + __shfl_xor(send, 16, 64);
        }
        const bool h8 = lane & 8;
        const float send = h8 ? v[0] : v[1];
        const float keep = h8 ? v[1] : v[0];
        v[0] = keep + __shfl_xor(send, 8, 64);
        v[0] += __shfl_xor(v[0], 4, 64);
        v[0] += __shfl_xor(v[0], 2, 64);
        v[0] += __shfl_xor(v[0], 1, 64);
    }
    // lane group (lane >> 3) holds row (lane>>5)*4 + ((lane>>4)&1)*2 + ((lane>>3)&1) of the wave
    if ((lane & 7) == 0) red[w * 8 + (lane >> 3)] = v[0];
    __syncthreads();
    if (t < 16) {
        const int j = t;
        const float hv = silu(red[j]) * red[16 + j];
        // h layout for the down kernel: f32x4 (k*8 + jj)*16 + b holds h[32b + 4jj .. +3]
        const int n = g * 16 + j;
        const int b = n >> 5, jj = (n >> 2) & 7, cc = n & 3;
        a.h[(((int64_t)k * 8 + jj) * 16 + b) * 4 + cc] = hv;
    }
}

// ---------------------------------------------------------------- streaming probe

// A measurement of the chip, not part of the method: the gate/up launch's
// grid and weight loads with nothing around them.  Work-group (g, k) reads
// chunk g of slot k exactly as q4_gateup_kernel's weight phase reads its
// expert's chunk (eight 1 KiB code lines and one scale line per wave,
// non-temporal) and folds the words into one per work-group, written to
// out[k * gridDim.x + g] so that the loads are kept.
__global__ __launch_bounds__(kThreads) void q4_stream_probe_kernel(const uint8_t* slots, int64_t slot_bytes,
                                                                   uint32_t* out) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int g = blockIdx.x, k = blockIdx.y;
    const uint8_t* chunk = slots + (int64_t)k * slot_bytes + (int64_t)g * kGUChunk;
    const u32x4* cp = reinterpret_cast<const u32x4*>(chunk) + w * 8 * 64 + lane;
    u32x4 c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = __builtin_nontemporal_load(cp + i * 64);
    const u32x4 sc = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(chunk + 32768) + w * 64 + lane);
    uint32_t v = sc.x ^ sc.y ^ sc.z ^ sc.w;
#pragma unroll
    for (int i = 0; i < 8; ++i) v ^= c[i].x ^ c[i].y ^ c[i].z ^ c[i].w;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v ^= __shfl_xor(v, o, 64);
    __shared__ uint32_t red[kThreads / 64];
    if (lane == 0) red[w] = v;
    __syncthreads();
    if (t == 0) out[k * gridDim.x + g] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// ---------------------------------------------------------------- down + combine + next router partials

// Grid kNP.  Work-group p owns output rows 16p..16p+15.  Thread t: expert rank
// (t >> 5), row half ((t >> 4) & 1), Q4_0 block (t & 15) along f; 8 rows each.
// Slot down region: codes [r][b][16 B], scales [r/4][b][4] fp16.
__global__ __launch_bounds__(kThreads) void q4_down_kernel(Q4Args a) {
    const int t = threadIdx.x, lane = t & 63;
    const int p = blockIdx.x;
    const int kq = t >> 5, half = (lane >> 4) & 1, b = lane & 15;
    const int r0 = p * kRW + half * 8;
    const int tok = tok_value(a.tok);
    const int K = a.K;
    const bool act = kq < K;

    // Loads in dependency order, as straight-line code, so the wait before
    // the weight loads covers the slot and h loads only, not the router
    // weights and the residual issued after them (loads retire in order).
    // Lanes past rank K load rank 0's slot and h rows (in bounds, unused);
    // an invalid slot is reported and read as slot 0, never used.
    const int slot = a.sel->slot[act ? kq : 0];
    f32x4 hh[8];
    {
        const f32x4* h4 = reinterpret_cast<const f32x4*>(a.h) + (act ? kq : 0) * 8 * 16 + b;
#pragma unroll
        for (int j = 0; j < 8; ++j) hh[j] = h4[j * 16];
    }
    const bool valid = slot >= 0 && slot < a.n_slots;
    const uint8_t* base = a.slots + (int64_t)(valid ? slot : 0) * a.slot_bytes + kGURegion;
    u32x4 c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        c[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (int64_t)(r0 + i) * 256) + b);
    const u32x2 s0 = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(base + kDownCodes) + (r0 >> 2) * 16 + b);
    const u32x2 s1 = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(base + kDownCodes) + ((r0 >> 2) + 1) * 16 + b);

    f32x4 wpre[4];
    load_wpre(a, p, wpre);
    float xr = 0.0f;
    if (t < kRW && a.residual) xr = a.x_base[(int64_t)tok * kQD + p * kRW + t];
    float gk[kQ4MaxK];  // the combine's gates, in rank order
#pragma unroll
    for (int kk = 0; kk < kQ4MaxK; ++kk) gk[kk] = (t < kRW && kk < K) ? a.sel->gate[kk] : 0.0f;

    float z[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = 0.0f;
    if (act && !valid) {
        if (b == 0 && half == 0) atomicOr(a.pt.error, (int)ERR_BAD_SLOT);
    } else if (act) {
        f16x2 ha[16];
        const float HO = kQ4Offset * q4_pairs(hh, ha);
        const uint32_t sw[4] = {s0.x, s0.y, s1.x, s1.y};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float s = half_bits_to_float(sw[i >> 1] >> ((i & 1) * 16));
            z[i] = s * (q4_dot(c[i], ha) - HO);
        }
    }
    // 8 rows x 16 lanes -> one row per pair of lanes (fixed tree)
    {
        const bool h8 = lane & 8;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float send = h8 ? z[q] : z[q + 4];
            const float keep = h8 ? z[q + 4] : z[q];
            z[q] = keep + __shfl_xor(send, 8, 64);
        }
        const bool h4 = lane & 4;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const float send = h4 ? z[q] : z[q + 2];
            const float keep = h4 ? z[q + 2] : z[q];
            z[q] = keep + __shfl_xor(send, 4, 64);
        }
        const bool h2 = lane & 2;
        const float send = h2 ? z[0] : z[1];
        const float keep = h2 ? z[1] : z[0];
        z[0] = keep + __shfl_xor(send, 2, 64);
        z[0] += __shfl_xor(z[0], 1, 64);
    }
    __shared__ float zs[kQ4MaxK][kRW];
    __shared__ float xn[kRW];
    if ((lane & 1) == 0)
        zs[kq][half * 8 + ((lane >> 3) & 1) * 4 + ((lane >> 2) & 1) * 2 + ((lane >> 1) & 1)] = z[0];
    __syncthreads();
    if (t < kRW) {
        float y = 0.0f;
#pragma unroll
        for (int kk = 0; kk < kQ4MaxK; ++kk)
            if (kk < K) y += gk[kk] * zs[kk][t];  // rank order
        const float o = a.residual ? xr + y : y;
        a.y_base[(int64_t)tok * kQD + p * kRW + t] = o;
        xn[t] = o;
    }
    if (p == 0 && t == 0 && !a.replay) *a.pub = 0u;  // every gate/up work-group of this layer has finished
    if (a.wr_part) {
        __syncthreads();
        router_partial(a, p, xn, wpre);
    }
}

__global__ void advance_kernel(int32_t* cursors, int64_t* stats) {
    if (threadIdx.x == 0) {
        cursors[0] += 1;
        cursors[1] += 1;
        stats[DS_TOKENS] += 1;
    }
}

// Decode stages the current token in a fixed buffer so that every kernel of
// the token graph finds x (and the token's router-bias row) at a fixed
// address, with no dependent load of the token cursor.
// Before the first token of a decode call: cursor 0, token count, stage x[0].
__global__ __launch_bounds__(kThreads) void token_begin_kernel(TokenIO io, int32_t n_tokens) {
    const f32x4* src = reinterpret_cast<const f32x4*>(io.x);
    f32x4* dst = reinterpret_cast<f32x4*>(io.xbuf);
    for (int i = threadIdx.x; i < kQD / 4; i += kThreads) dst[i] = src[i];
    if (threadIdx.x == 0) {
        io.cursors[0] = 0;
        *io.ntok = n_tokens;
        *io.tokrow = io.bias_row ? io.bias_row[0] : 0;
    }
}

// Last node of a token graph: write the token's result back to x[t], stage
// x[t+1] and its bias row, advance the cursors.
__global__ __launch_bounds__(kThreads) void token_end_kernel(TokenIO io) {
    const int t = io.cursors[0];
    const int n = *io.ntok;
    f32x4* xb = reinterpret_cast<f32x4*>(io.xbuf);
    f32x4* xt = reinterpret_cast<f32x4*>(io.x + (int64_t)t * kQD);
    const bool more = t + 1 < n;
    for (int i = threadIdx.x; i < kQD / 4; i += kThreads) {
        xt[i] = xb[i];
        if (more) xb[i] = xt[i + kQD / 4];
    }
    if (threadIdx.x == 0 && more) *io.tokrow = io.bias_row ? io.bias_row[t + 1] : 0;
    __syncthreads();
    if (threadIdx.x == 0) {
        io.cursors[0] = t + 1;
        io.cursors[1] += 1;
        io.stats[DS_TOKENS] += 1;
    }
}

}  // namespace

hipError_t launch_q4_router_partial(const Q4Args& a, hipStream_t s) {
    if (!a.wr_part || a.E > kMaxE) return hipErrorInvalidValue;
    hipLaunchKernelGGL(q4_router_partial_kernel, dim3(kNP), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_q4_gateup(const Q4Args& a, hipStream_t s) {
    if (a.K < 1 || a.K > kQ4MaxK || a.E > kMaxE || a.E < a.K) return hipErrorInvalidValue;
    hipLaunchKernelGGL(q4_gateup_kernel, dim3(kQF / kGURows, a.K), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_q4_stream_probe(const uint8_t* slots, int64_t slot_bytes, int32_t K, uint32_t* out, hipStream_t s) {
    hipLaunchKernelGGL(q4_stream_probe_kernel, dim3(kQF / kGURows, K), dim3(kThreads), 0, s, slots, slot_bytes, out);
    return hipGetLastError();
}

hipError_t launch_q4_down(const Q4Args& a, hipStream_t s) {
    if (a.K < 1 || a.K > kQ4MaxK || a.E > kMaxE) return hipErrorInvalidValue;
    hipLaunchKernelGGL(q4_down_kernel, dim3(kNP), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_token_begin(const TokenIO& io, int32_t n_tokens, hipStream_t s) {
    hipLaunchKernelGGL(token_begin_kernel, dim3(1), dim3(kThreads), 0, s, io, n_tokens);
    return hipGetLastError();
}

hipError_t launch_token_end(const TokenIO& io, hipStream_t s) {
    hipLaunchKernelGGL(token_end_kernel, dim3(1), dim3(kThreads), 0, s, io);
    return hipGetLastError();
}

hipError_t launch_advance(int32_t* cursors, int64_t* stats, hipStream_t s) {
    hipLaunchKernelGGL(advance_kernel, dim3(1), dim3(64), 0, s, cursors, stats);
    return hipGetLastError();
}

}  // namespace moe
