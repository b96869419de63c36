// gfx950 Q4_0 batched decode: B tokens (B <= 16) go through the stack
// together, one step at a time, four launches per layer.
//
//   route   one work-group per token rebuilds its router logits from the
//           partial dot products of the previous launch, takes the top-k and
//           the softmax renormalised over it ("Luce Spark runs 35B MoE models
//           on 16GB GPU without speed loss", opening paragraph: about 8 of
//           256 experts per token), counts the choices and stores the
//           token's normalised input as fp16 pairs.  The last work-group to
//           finish runs the placement policy of the same page's paragraph
//           "The key components" over the step's accesses in (token, rank)
//           order, and groups the accesses by distinct expert.
//   gateup  work-group (g, y) streams rows 16g..16g+15 of the gate and up
//           matrices of a work item's expert (up to 4 of the tokens that
//           chose it) and applies them to each of those tokens; a popular
//           expert's items re-read its rows from L2.
//   down    work-group (p, s) computes output rows 16p..16p+15 of the down
//           GEMV of 16 accesses (an expert chosen by several tokens is
//           re-read from L2).
//   combine work-group p does the gate-weighted combine of those rows in rank
//           order, the residual, and the next layer's router partials of
//           every token over them.
//
// Per token, every value is formed by the same operations in the same order
// as in the batch-1 kernels, so a token's outputs do not depend on the batch
// it runs in nor on where its experts' weights sit.
#include <hip/hip_runtime.h>
#include <math.h>

#include "device_common.h"
#include "internal.h"
#include "policy.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kDownSlice = 16;  // accesses per down work-group
constexpr int kGURowsMax = 64;  // work-item rows of the gate/up grid (more items loop)
typedef __attribute__((address_space(4))) const BatchSel ConstSel;
static_assert(kNP == 128, "the route kernel sums the partial squares with two loads per lane");
static_assert(kMaxBK <= kThreads, "one thread per access in the route kernel's policy pass");

__device__ __forceinline__ bool qb_spin_expired(const QBArgs& a, uint64_t t0) {
    return wall_clock64() - t0 > a.spin_limit_ticks ||
           (__hip_atomic_load(a.pt.error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & ERR_FILL_TIMEOUT);
}

// Partial router logits of token b over one 16-row slice:
// pl[b][p][e] = sum_i Wr[e][16p+i] xs[i], ps[b][p] = sum_i xs[i]^2.
__device__ __forceinline__ void qb_router_partial(const QBArgs& a, int b, int p, const float* xs,
                                                  const f32x4* wpre) {
    const int t = threadIdx.x, E = a.E;
    float* pl = a.pl + ((int64_t)b * kNP + p) * E;
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
        pl[e] = (q[0] + q[1]) + (q[2] + q[3]);
    }
    if (t == 0) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < kRW; ++i) s += xs[i] * xs[i];
        a.ps[(int64_t)b * kNP + p] = s;
    }
}

__device__ __forceinline__ void qb_load_wpre(const QBArgs& a, int p, f32x4* wpre) {
    const int t = threadIdx.x;
    if (a.wr_part && t < a.E) {
        const f32x4* w4 = reinterpret_cast<const f32x4*>(a.wr_part + ((int64_t)p * a.E + t) * kRW);
#pragma unroll
        for (int i = 0; i < 4; ++i) wpre[i] = w4[i];
    }
}

// ---------------------------------------------------------------- router partials (first layer)

// Grid (kNP, B).  Work-group (p, b) reads rows 16p..16p+15 of token b.
__global__ __launch_bounds__(kThreads) void qb_router_partial_kernel(QBArgs a) {
    const int p = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    if (b >= *a.nb) return;
    f32x4 wpre[4];
    qb_load_wpre(a, p, wpre);
    __shared__ float xs[kRW];
    if (t < kRW) xs[t] = a.xb[(int64_t)b * kQD + p * kRW + t];
    __syncthreads();
    qb_router_partial(a, b, p, xs, wpre);
}

// ---------------------------------------------------------------- route + policy

// Grid B.  Work-group b routes token b; the last one to finish places the
// step's accesses.
__global__ __launch_bounds__(kThreads) void qb_route_kernel(QBArgs a) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int b = blockIdx.x;
    const int nb = *a.nb;
    if (b >= nb) return;
    const int E = a.E, K = a.K;
    BatchSel* sel = a.sel;

    __shared__ __align__(16) float xt[kQD / 32 * 36];
    __shared__ __align__(16) uint64_t kpad[kThreads];
    __shared__ __align__(16) uint64_t cand[kMaxE / 64 * kQ4MaxK + 16];
    __shared__ int s_e[kMaxK];
    __shared__ float s_l[kMaxK];
    __shared__ float s_g[kMaxK];
    __shared__ float s_z;
    __shared__ int s_last;
    __shared__ int32_t sof[kMaxE];

    // every routing load first (x, slot-table row, partial squares, partial
    // logits, bias)
    const f32x4* x4 = reinterpret_cast<const f32x4*>(a.xb + (int64_t)b * kQD);
    const f32x4 xv0 = x4[t], xv1 = x4[t + kThreads];
    const int32_t sof0 = t < E ? a.pt.slot_of[(int64_t)a.layer * E + t] : -1;
    const float* psb = a.ps + (int64_t)b * kNP;
    const float ps0 = psb[lane], ps1 = psb[lane + 64];
    const float* plb = a.pl + (int64_t)b * kNP * E;
    const int e4 = 64 * w + 4 * (lane & 15), rg = lane >> 4;
    f32x4 pv[kNP / 4];
    if (e4 < E) {
#pragma unroll
        for (int j = 0; j < kNP / 4; ++j) pv[j] = *reinterpret_cast<const f32x4*>(plb + (int64_t)(rg + 4 * j) * E + e4);
    }
    const float* brow = nullptr;
    if (a.bias) {
        int row = a.rows[b];
        row = row < 0 ? 0 : (row >= a.n_bias_rows ? a.n_bias_rows - 1 : row);
        brow = a.bias + (int64_t)row * E;
    }
    const float b0 = (brow && e4 + rg < E) ? brow[e4 + rg] : 0.0f;

    // x transposed through LDS: Q4_0 block q at float 36q
    *reinterpret_cast<f32x4*>(&xt[36 * (t >> 3) + 4 * (t & 7)]) = xv0;
    *reinterpret_cast<f32x4*>(&xt[36 * ((t + kThreads) >> 3) + 4 * (t & 7)]) = xv1;
    if (t < E) sof[t] = sof0;
    for (int e = t + kThreads; e < E; e += kThreads) sof[e] = a.pt.slot_of[(int64_t)a.layer * E + e];
    const float ss = wave_sum(ps0 + ps1);
    const float inv = a.norm ? 1.0f / sqrtf(ss / (float)kQD + a.eps) : 1.0f;
    // logit = inv * (the 128 partials: 32 in row order per lane, then the
    // four row groups) + bias
    const int n_chunks = (E + 63) >> 6;
    for (int c = w; c < n_chunks; c += 4) {
        const int ec = 64 * c + 4 * (lane & 15);
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if (ec < E) {
            if (c != w) {
#pragma unroll
                for (int j = 0; j < kNP / 4; ++j)
                    pv[j] = *reinterpret_cast<const f32x4*>(plb + (int64_t)(rg + 4 * j) * E + ec);
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

    if (w == 0) {
        // gates: softmax over the chosen logits, shifted by the largest
        if (lane < K) s_g[lane] = expf(s_l[lane] - s_l[0]);
        __builtin_amdgcn_wave_barrier();
        if (lane == 0) {
            float z = 0.0f;
            for (int kk = 0; kk < K; ++kk) z += s_g[kk];
            s_z = z;
        }
        __builtin_amdgcn_wave_barrier();
        if (lane < K) s_g[lane] = s_g[lane] / s_z;
        const int ttok = *a.trace_base + b;
        if (lane < K) {
            const int myk = s_e[lane];
            const float myg = s_g[lane];
            sel->idx[b * K + lane] = myk;
            sel->gate[b * K + lane] = myg;
            sel->slot[b * K + lane] = sof[myk];  // its pinned slot or -1, for the policy
            atomicAdd(reinterpret_cast<unsigned long long*>(a.pt.counts + (int64_t)a.layer * E + myk), 1ull);
            if (a.tr_topk && ttok < a.tr_cap) {
                const int64_t o = ((int64_t)ttok * a.L + a.layer) * K + lane;
                a.tr_topk[o] = myk;
                a.tr_gates[o] = myg;
            }
        }
        if (lane == 0) sel->inv_rms[b] = inv;
        // lane q: Q4_0 block q of x; the trace row, then the fp16 pairs of
        // the normalised block and their sum, for the gate/up kernel
        f32x4 xx[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) xx[j] = *reinterpret_cast<const f32x4*>(&xt[36 * lane + 4 * j]);
        if (a.tr_x && ttok < a.tr_cap) {
            f32x4* t4 = reinterpret_cast<f32x4*>(a.tr_x + ((int64_t)ttok * a.L + a.layer) * kQD);
#pragma unroll
            for (int j = 0; j < 8; ++j) t4[lane * 8 + j] = xx[j];
        }
        f32x4 uu[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) uu[j] = xx[j] * inv;
        f16x2 ua[16];
        const float U = q4_pairs(uu, ua);
        u32x4* dst = reinterpret_cast<u32x4*>(a.ua + ((int64_t)b * 64 + lane) * 16);
#pragma unroll
        for (int m = 0; m < 4; ++m)
            dst[m] = u32x4{__builtin_bit_cast(uint32_t, ua[4 * m]), __builtin_bit_cast(uint32_t, ua[4 * m + 1]),
                           __builtin_bit_cast(uint32_t, ua[4 * m + 2]), __builtin_bit_cast(uint32_t, ua[4 * m + 3])};
        a.ub[(int64_t)b * 64 + lane] = U;
    }

    // ---- the last work-group of the step places its accesses
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (t == 0) {
        const unsigned prev = __hip_atomic_fetch_add(a.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (unsigned)nb - 1;
    }
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

    __shared__ int32_t s_idx[kMaxBK];
    __shared__ int32_t s_pin[kMaxBK];
    __shared__ int32_t s_slot[kMaxBK];
    __shared__ unsigned long long s_wseq[kMaxBK];
    __shared__ uint32_t s_bits[kMaxE / 32];
    __shared__ int32_t s_pre[kMaxE / 32];
    __shared__ int32_t s_cnt[kMaxBK];
    __shared__ int32_t s_off[kMaxBK + 1];
    __shared__ int32_t s_ioff[kMaxBK + 1];
    __shared__ int s_D, s_cold;
    __shared__ int32_t r_owner[kMaxR];
    __shared__ uint64_t r_stamp[kMaxR];
    __shared__ uint64_t r_seq[kMaxR];

    const int n = nb * K;
    const int nw = (E + 31) >> 5;
    if (t == 0) {
        __hip_atomic_store(a.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_cold = 0;
    }
    for (int i = t; i < nw; i += kThreads) s_bits[i] = 0u;
    if (t < kMaxBK) s_cnt[t] = 0;
    int e_t = -1, pin_t = -1;
    if (t < n) {
        e_t = __hip_atomic_load(&sel->idx[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        pin_t = __hip_atomic_load(&sel->slot[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_idx[t] = e_t;
        s_pin[t] = pin_t;
    }
    __syncthreads();
    if (t < n) {
        atomicOr(&s_bits[e_t >> 5], 1u << (e_t & 31));
        if (pin_t < 0) s_cold = 1;
    }
    __syncthreads();
    if (w == 0) {  // exclusive prefix of the per-word popcounts: rank of an expert among the distinct
        const int c = lane < nw ? __popc(s_bits[lane]) : 0;
        int incl = c;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            const int o = __shfl_up(incl, m, 64);
            if (lane >= m) incl += o;
        }
        if (lane < nw) s_pre[lane] = incl - c;
        if (lane == 63) s_D = incl;
    }
    __syncthreads();
    int rank = 0, pos = 0;
    if (t < n) {
        rank = s_pre[e_t >> 5] + __popc(s_bits[e_t >> 5] & ((1u << (e_t & 31)) - 1u));
        for (int i = 0; i < t; ++i) pos += s_idx[i] == e_t;  // earlier accesses of the same expert
        atomicAdd(&s_cnt[rank], 1);
    }
    __syncthreads();
    if (w == 0) {  // group offsets: exclusive prefix over the distinct experts, two per lane
        const int c0 = s_cnt[2 * lane], c1 = s_cnt[2 * lane + 1];
        int incl = c0 + c1;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            const int o = __shfl_up(incl, m, 64);
            if (lane >= m) incl += o;
        }
        const int excl = incl - (c0 + c1);
        s_off[2 * lane] = excl;
        s_off[2 * lane + 1] = excl + c0;
        if (lane == 63) s_off[kMaxBK] = incl;
    }
    if (w == 2) {  // work-item offsets: the same prefix over ceil(count / kItemTok)
        const int c0 = (s_cnt[2 * lane] + kItemTok - 1) / kItemTok, c1 = (s_cnt[2 * lane + 1] + kItemTok - 1) / kItemTok;
        int incl = c0 + c1;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            const int o = __shfl_up(incl, m, 64);
            if (lane >= m) incl += o;
        }
        const int excl = incl - (c0 + c1);
        s_ioff[2 * lane] = excl;
        s_ioff[2 * lane + 1] = excl + c0;
        if (lane == 63) s_ioff[kMaxBK] = incl;
    }
    if (w == 1) {
        // the policy, one access at a time in (token, rank) order
        RingState rs{};
        if (!s_cold) {
            for (int i = lane; i < n; i += 64) {
                s_slot[i] = s_pin[i];
                s_wseq[i] = 0ull;
            }
            rs.n_pin = n;
        } else {
            ring_load(a.pt, r_owner, r_stamp, r_seq, rs);
#pragma nounroll
            for (int i = 0; i < n; ++i) {
                int slot;
                uint64_t wseq;
                ring_access(a.pt, a.layer, s_idx[i], s_pin[i], r_owner, r_stamp, r_seq, rs, slot, wseq);
                if (lane == 0) {
                    s_slot[i] = slot;
                    s_wseq[i] = wseq;
                }
            }
            ring_store(a.pt, r_owner, r_stamp, r_seq, rs);
        }
        stats_flush(a.pt, n, rs);
    }
    __syncthreads();
    const int D = s_D;
    if (t < n) {
        sel->slot[t] = s_slot[t];
        sel->dent[s_off[rank] + pos] = t;
        if (pos == 0) {  // the expert's first access: its slot, and the fill it made (if any)
            sel->dexp[rank] = e_t;
            sel->dslot[rank] = s_slot[t];
            sel->dwait[rank] = s_wseq[t];
        }
        const int item = s_ioff[rank] + pos / kItemTok;
        sel->item_acc[item][pos % kItemTok] = t;
        if (pos % kItemTok == 0) {
            const int left = s_cnt[rank] - pos;
            sel->item_j[item] = rank;
            sel->item_n[item] = left < kItemTok ? left : kItemTok;
        }
    }
    if (t <= D) sel->doff[t] = t < D ? s_off[t] : n;
    if (t == 0) {
        sel->D = D;
        sel->NI = s_ioff[kMaxBK];
    }
}

// ---------------------------------------------------------------- gate/up

// Rows 16g..16g+15 of the gate and up matrices of one work item's expert
// (waves 0, 1 gate rows, waves 2, 3 up rows, 8 rows per wave, lane q = Q4_0
// block q along d), applied to the item's tokens (at most kItemTok).
__device__ __forceinline__ void qb_gateup_item(const QBArgs& a, const ConstSel* sel, int g, int it,
                                               u32x4 (*s_ua)[kThreads], float (*s_ub)[64], float (*red)[32]) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int K = a.K;
    const int j = sel->item_j[it], cn = sel->item_n[it];
    const bool first_item = it == 0 || sel->item_j[it - 1] != j;
    const int e = sel->dexp[j], slot = sel->dslot[j];
    const uint64_t wseq = sel->dwait[j];
    int acc_i[kItemTok];
#pragma unroll
    for (int q = 0; q < kItemTok; ++q) acc_i[q] = sel->item_acc[it][q];  // entries past cn: not used

    if (slot < 0 || slot >= a.n_slots || cn < 1 || cn > kItemTok) {  // never expected: refuse rather than fault
        if (t == 0) atomicOr(a.pt.error, (int)ERR_BAD_SLOT);
        return;
    }
    // a fill made in this step: pulled from the host arena by every item of
    // the expert, written into the ring slot by the first item's work-groups
    const bool pull = a.pt.pull && wseq && slot >= a.P;
    if (wseq && slot >= a.P && !pull) {  // wait for the host agent's copy
        if (t == 0) {
            const uint64_t* flag = a.ready + (slot - a.P);
            const uint64_t t0 = wall_clock64();
            int polls = 0;
            while (__hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM) < wseq) {
                fill_poll_pause(polls);
                if (qb_spin_expired(a, t0)) {
                    atomicOr(a.pt.error, (int)ERR_FILL_TIMEOUT);
                    break;
                }
            }
        }
        __syncthreads();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
    }

    const int64_t key = (int64_t)a.layer * a.E + e;
    const uint8_t* chunk = (pull ? a.arena + key * a.slot_bytes : a.slots + (int64_t)slot * a.slot_bytes) +
                           (int64_t)g * kGUChunk;
    const u32x4* cp = reinterpret_cast<const u32x4*>(chunk) + w * 8 * 64 + lane;
    u32x4 c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = __builtin_nontemporal_load(cp + i * 64);
    const u32x4 sc = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(chunk + 32768) + w * 64 + lane);

    // the tokens' fp16 pairs and block sums, while the weights are in flight
    {
        u32x4 st[kItemTok];
        float su[kItemTok];
#pragma unroll
        for (int q = 0; q < kItemTok; ++q) {
            if (q < cn) {
                const int bq = acc_i[q] / K;
                st[q] = reinterpret_cast<const u32x4*>(a.ua + (int64_t)bq * 64 * 16)[t];
                if (t < 64) su[q] = a.ub[(int64_t)bq * 64 + t];
            }
        }
#pragma unroll
        for (int q = 0; q < kItemTok; ++q) {
            if (q < cn) {
                s_ua[q][t] = st[q];
                if (t < 64) s_ub[q][t] = su[q];
            }
        }
    }

    if (pull && first_item) {
        // the fill: this chunk of gate/up rows as read, plus 1/32 of the down
        // region, into the ring slot (read by the down launch and later hits)
        uint8_t* dst = a.slots + (int64_t)slot * a.slot_bytes;
        u32x4* dp = reinterpret_cast<u32x4*>(dst + (int64_t)g * kGUChunk) + w * 8 * 64 + lane;
#pragma unroll
        for (int i = 0; i < 8; ++i) __builtin_nontemporal_store(c[i], dp + i * 64);
        __builtin_nontemporal_store(sc, reinterpret_cast<u32x4*>(dst + (int64_t)g * kGUChunk + 32768) + w * 64 + lane);
        constexpr int kDownShare = (int)((kQ4SlotBytes - kGURegion) / (kQF / kGURows) / 16);
        const u32x4* hs = reinterpret_cast<const u32x4*>(a.arena + key * a.slot_bytes + kGURegion) + g * kDownShare;
        u32x4* ds = reinterpret_cast<u32x4*>(dst + kGURegion) + g * kDownShare;
        for (int i = t; i < kDownShare; i += kThreads) __builtin_nontemporal_store(__builtin_nontemporal_load(hs + i), ds + i);
    }

    // codes -> fp16 (1024 + q) pairs, in the order q4_dot consumes them
    f16x2 wq[8][16];
    float sv[8];
    {
        constexpr uint32_t kHi = 0x64646464u, kEven = 0x04020400u, kOdd = 0x04030401u;
        const uint32_t sw[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t wd[4] = {c[i].x, c[i].y, c[i].z, c[i].w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint32_t lo = wd[m] & 0x0F0F0F0Fu, hi = (wd[m] >> 4) & 0x0F0F0F0Fu;
                wq[i][4 * m + 0] = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(kHi, lo, kEven));
                wq[i][4 * m + 1] = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(kHi, lo, kOdd));
                wq[i][4 * m + 2] = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(kHi, hi, kEven));
                wq[i][4 * m + 3] = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(kHi, hi, kOdd));
            }
            sv[i] = half_bits_to_float(sw[i >> 1] >> ((i & 1) * 16));
        }
    }
    __syncthreads();

    // all the item's tokens at once, so their reduction trees' cross-lane
    // steps are in flight together
    float v[kItemTok][8];
#pragma unroll
    for (int u = 0; u < kItemTok; ++u) {
        const int q = u < cn ? u : cn - 1;  // past the item: recompute its last token, not stored
        // this lane's block: 16 fp16 pairs, read as words
        const uint32_t* up = reinterpret_cast<const uint32_t*>(&s_ua[q][lane * 4]);
        f16x2 ua[16];
#pragma unroll
        for (int pp = 0; pp < 16; ++pp) ua[pp] = __builtin_bit_cast(f16x2, up[pp]);
        const float UO = kQ4Offset * s_ub[q][lane];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float acc = 0.0f;
#pragma unroll
            for (int pp = 0; pp < 16; ++pp) acc = __builtin_amdgcn_fdot2(wq[i][pp], ua[pp], acc, false);
            v[u][i] = sv[i] * (acc - UO);
        }
    }
    // 8 rows x 64 lanes -> one row per group of 8 lanes (fixed tree), per token
    const bool h32 = lane & 32, h16 = lane & 16, h8 = lane & 8;
#pragma unroll
    for (int u = 0; u < kItemTok; ++u) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float send = h32 ? v[u][r] : v[u][r + 4];
            const float keep = h32 ? v[u][r + 4] : v[u][r];
            v[u][r] = keep + __shfl_xor(send, 32, 64);
        }
    }
#pragma unroll
    for (int u = 0; u < kItemTok; ++u) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const float send = h16 ? v[u][r] : v[u][r + 2];
            const float keep = h16 ? v[u][r + 2] : v[u][r];
            v[u][r] = keep + __shfl_xor(send, 16, 64);
        }
    }
#pragma unroll
    for (int u = 0; u < kItemTok; ++u) {
        const float send = h8 ? v[u][0] : v[u][1];
        const float keep = h8 ? v[u][1] : v[u][0];
        v[u][0] = keep + __shfl_xor(send, 8, 64);
    }
#pragma unroll
    for (int u = 0; u < kItemTok; ++u) v[u][0] += __shfl_xor(v[u][0], 4, 64);
#pragma unroll
    for (int u = 0; u < kItemTok; ++u) v[u][0] += __shfl_xor(v[u][0], 2, 64);
#pragma unroll
    for (int u = 0; u < kItemTok; ++u) v[u][0] += __shfl_xor(v[u][0], 1, 64);
#pragma unroll
    for (int u = 0; u < kItemTok; ++u)
        if (u < cn && (lane & 7) == 0) red[u][w * 8 + (lane >> 3)] = v[u][0];
    __syncthreads();
    if (t < 16 * cn) {
        const int q = t >> 4, jr = t & 15;
        const float hv = silu(red[q][jr]) * red[q][16 + jr];
        // h layout for the down kernel: f32x4 (i*8 + jj)*16 + blk holds h_i[32blk + 4jj .. +3]
        const int rn = g * 16 + jr;
        const int blk = rn >> 5, jj = (rn >> 2) & 7, cc = rn & 3;
        a.h[(((int64_t)acc_i[q] * 8 + jj) * 16 + blk) * 4 + cc] = hv;
    }
}

// Grid (f/16, min(B*K, 64)): work-group (g, y) takes work items y,
// y + gridDim.y, ... of the step.
__global__ __launch_bounds__(kThreads) void qb_gateup_kernel(QBArgs a) {
    __shared__ __align__(16) u32x4 s_ua[kItemTok][kThreads];
    __shared__ float s_ub[kItemTok][64];
    __shared__ float red[kItemTok][32];
    // read-only here (written by the route launch): through the constant
    // address space, so uniform reads go through the scalar cache
    const ConstSel* sel = (const ConstSel*)a.sel;
    const int NI = sel->NI;
    for (int it = blockIdx.y; it < NI; it += gridDim.y) {
        if (it != (int)blockIdx.y) __syncthreads();  // LDS reuse
        qb_gateup_item(a, sel, blockIdx.x, it, s_ua, s_ub, red);
    }
}

// ---------------------------------------------------------------- down + combine + next router partials

// Grid (kNP, ceil(B*K/16)).  Work-group (p, s) computes output rows
// 16p..16p+15 of accesses 16s..16s+15: thread t takes access 16s + (t >> 5)
// and access 16s + 8 + (t >> 5), row half ((t >> 4) & 1), Q4_0 block (t & 15)
// along f, 8 rows each; both accesses' codes, scales and h are loaded
// together.  The per-access rows go to zb for the combine launch (a kernel
// boundary is the cheaper hand-over here: a release fence at device scope in
// each of a thousand work-groups writes back L2 every time).
__global__ __launch_bounds__(kThreads) void qb_down_kernel(QBArgs a) {
    const int t = threadIdx.x, lane = t & 63;
    const int p = blockIdx.x, s = blockIdx.y;
    const int kq = t >> 5, half = (lane >> 4) & 1, blk = lane & 15;
    const int r0 = p * kRW + half * 8;
    const int nb = *a.nb;
    const int K = a.K, n = nb * K;
    const int n_slices = (n + kDownSlice - 1) / kDownSlice;
    if (s >= n_slices) return;
    const BatchSel* sel = a.sel;

    const f32x4* h4 = reinterpret_cast<const f32x4*>(a.h);
    u32x4 c[2][8];
    u32x2 sc[2][2];
    f32x4 hh[2][8];
    bool ok[2] = {false, false};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int i = s * kDownSlice + q * 8 + kq;
        if (i < n) {
            const int slot = sel->slot[i];
            ok[q] = slot >= 0 && slot < a.n_slots;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) hh[q][jj] = h4[((int64_t)i * 8 + jj) * 16 + blk];
            if (ok[q]) {
                const uint8_t* base = a.slots + (int64_t)slot * a.slot_bytes + kGURegion;
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    c[q][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (int64_t)(r0 + r) * 256) + blk);
                sc[q][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(base + kDownCodes) + (r0 >> 2) * 16 + blk);
                sc[q][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(base + kDownCodes) + ((r0 >> 2) + 1) * 16 + blk);
            } else if (blk == 0 && half == 0) {
                atomicOr(a.pt.error, (int)ERR_BAD_SLOT);
            }
        }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int i = s * kDownSlice + q * 8 + kq;
        if (i >= n) continue;
        float z[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) z[r] = 0.0f;
        if (ok[q]) {
            f16x2 ha[16];
            const float HO = kQ4Offset * q4_pairs(hh[q], ha);
            const uint32_t sw[4] = {sc[q][0].x, sc[q][0].y, sc[q][1].x, sc[q][1].y};
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float sv = half_bits_to_float(sw[r >> 1] >> ((r & 1) * 16));
                z[r] = sv * (q4_dot(c[q][r], ha) - HO);
            }
        }
        // 8 rows x 16 lanes -> one row per pair of lanes (fixed tree)
        {
            const bool h8 = lane & 8;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float send = h8 ? z[u] : z[u + 4];
                const float keep = h8 ? z[u + 4] : z[u];
                z[u] = keep + __shfl_xor(send, 8, 64);
            }
            const bool h4b = lane & 4;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const float send = h4b ? z[u] : z[u + 2];
                const float keep = h4b ? z[u + 2] : z[u];
                z[u] = keep + __shfl_xor(send, 4, 64);
            }
            const bool h2 = lane & 2;
            const float send = h2 ? z[0] : z[1];
            const float keep = h2 ? z[1] : z[0];
            z[0] = keep + __shfl_xor(send, 2, 64);
            z[0] += __shfl_xor(z[0], 1, 64);
        }
        if ((lane & 1) == 0)
            a.zb[(int64_t)i * kQD + p * kRW + half * 8 + ((lane >> 3) & 1) * 4 + ((lane >> 2) & 1) * 2 +
                 ((lane >> 1) & 1)] = z[0];
    }

}

// Grid kNP.  Work-group p adds up rows 16p..16p+15 of each token's accesses
// in rank order (the gate-weighted combine), adds the residual, and writes
// the next layer's router partials of every token over those rows.
__global__ __launch_bounds__(kThreads) void qb_combine_kernel(QBArgs a) {
    const int t = threadIdx.x, p = blockIdx.x;
    const int nb = *a.nb;
    const int K = a.K, n = nb * K;
    const BatchSel* sel = a.sel;
    __shared__ float xn[kMaxB][kRW];
    __shared__ float s_g[kMaxBK];

    f32x4 wpre[4];
    qb_load_wpre(a, p, wpre);
    const int tb = t >> 4, tr = t & 15;  // token tb, row tr
    float xr = 0.0f;
    float zk[kQ4MaxK];
    if (tb < nb) {
        xr = a.xb[(int64_t)tb * kQD + p * kRW + tr];
#pragma unroll
        for (int kk = 0; kk < kQ4MaxK; ++kk) zk[kk] = kk < K ? a.zb[(int64_t)(tb * K + kk) * kQD + p * kRW + tr] : 0.0f;
    }
    if (t < n) s_g[t] = sel->gate[t];
    __syncthreads();
    if (tb < nb) {
        float y = 0.0f;
#pragma unroll
        for (int kk = 0; kk < kQ4MaxK; ++kk)
            if (kk < K) y += s_g[tb * K + kk] * zk[kk];  // rank order
        const float o = xr + y;
        a.xb[(int64_t)tb * kQD + p * kRW + tr] = o;
        xn[tb][tr] = o;
    }
    if (a.wr_part) {
        __syncthreads();
        for (int b = 0; b < nb; ++b) qb_router_partial(a, b, p, xn[b], wpre);
    }
}

// ---------------------------------------------------------------- step staging

// Before the first step of a decode call: cursor 0, token count, stage the
// first step's tokens and bias rows.
__global__ __launch_bounds__(1024) void qb_begin_kernel(BatchIO io, int32_t n_tokens) {
    const int nb = n_tokens < io.B ? n_tokens : io.B;
    const f32x4* src = reinterpret_cast<const f32x4*>(io.x);
    f32x4* dst = reinterpret_cast<f32x4*>(io.xb);
    for (int i = threadIdx.x; i < nb * (kQD / 4); i += blockDim.x) dst[i] = src[i];
    if (threadIdx.x < (unsigned)nb) io.rows[threadIdx.x] = io.bias_row ? io.bias_row[threadIdx.x] : 0;
    if (threadIdx.x == 0) {
        io.cursors[0] = 0;
        *io.ntok = n_tokens;
        *io.nb = nb;
    }
}

// Last node of a step graph: write the step's tokens back, stage the next
// step's, advance the cursors.
__global__ __launch_bounds__(1024) void qb_end_kernel(BatchIO io) {
    const int c = io.cursors[0];
    const int n = *io.ntok;
    const int nb = *io.nb;
    f32x4* xb = reinterpret_cast<f32x4*>(io.xb);
    f32x4* x = reinterpret_cast<f32x4*>(io.x);
    for (int i = threadIdx.x; i < nb * (kQD / 4); i += blockDim.x) x[(int64_t)c * (kQD / 4) + i] = xb[i];
    const int c2 = c + nb;
    const int left = n - c2;
    const int nb2 = left < io.B ? left : io.B;
    __syncthreads();
    for (int i = threadIdx.x; i < nb2 * (kQD / 4); i += blockDim.x) xb[i] = x[(int64_t)c2 * (kQD / 4) + i];
    if ((int)threadIdx.x < nb2) io.rows[threadIdx.x] = io.bias_row ? io.bias_row[c2 + threadIdx.x] : 0;
    __syncthreads();
    if (threadIdx.x == 0) {
        io.cursors[0] = c2;
        io.cursors[1] += nb;
        io.stats[DS_TOKENS] += nb;
        if (nb2 > 0) *io.nb = nb2;
    }
}

}  // namespace

hipError_t launch_qb_begin(const BatchIO& io, int32_t n_tokens, hipStream_t s) {
    if (io.B < 1 || io.B > kMaxB || n_tokens < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(qb_begin_kernel, dim3(1), dim3(1024), 0, s, io, n_tokens);
    return hipGetLastError();
}

hipError_t launch_qb_end(const BatchIO& io, hipStream_t s) {
    if (io.B < 1 || io.B > kMaxB) return hipErrorInvalidValue;
    hipLaunchKernelGGL(qb_end_kernel, dim3(1), dim3(1024), 0, s, io);
    return hipGetLastError();
}

hipError_t launch_qb_router_partial(const QBArgs& a, hipStream_t s) {
    if (!a.wr_part || a.E > kMaxE || a.B < 1 || a.B > kMaxB) return hipErrorInvalidValue;
    hipLaunchKernelGGL(qb_router_partial_kernel, dim3(kNP, a.B), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_qb_route(const QBArgs& a, hipStream_t s) {
    if (a.K < 1 || a.K > kQ4MaxK || a.E > kMaxE || a.E < a.K || a.B < 1 || a.B > kMaxB) return hipErrorInvalidValue;
    hipLaunchKernelGGL(qb_route_kernel, dim3(a.B), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_qb_gateup(const QBArgs& a, hipStream_t s) {
    if (a.K < 1 || a.K > kQ4MaxK || a.E > kMaxE || a.B < 1 || a.B > kMaxB) return hipErrorInvalidValue;
    int rows = a.B * a.K < a.E ? a.B * a.K : a.E;
    rows = rows < kGURowsMax ? rows : kGURowsMax;
    hipLaunchKernelGGL(qb_gateup_kernel, dim3(kQF / kGURows, rows), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_qb_combine(const QBArgs& a, hipStream_t s) {
    if (a.K < 1 || a.K > kQ4MaxK || a.E > kMaxE || a.B < 1 || a.B > kMaxB) return hipErrorInvalidValue;
    hipLaunchKernelGGL(qb_combine_kernel, dim3(kNP), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_qb_down(const QBArgs& a, hipStream_t s) {
    if (a.K < 1 || a.K > kQ4MaxK || a.E > kMaxE || a.B < 1 || a.B > kMaxB) return hipErrorInvalidValue;
    hipLaunchKernelGGL(qb_down_kernel, dim3(kNP, (a.B * a.K + kDownSlice - 1) / kDownSlice), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
