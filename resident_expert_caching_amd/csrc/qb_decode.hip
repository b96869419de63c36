// gfx950 Q4_0 batched decode: B tokens (B <= 16) go through the stack
// together, one step at a time, three launches per layer.
//
//   route   one work-group per token rebuilds its router logits from the
//           partial dot products of the previous launch, takes the top-k and
//           the softmax renormalised over it ("Luce Spark runs 35B MoE models
//           on 16GB GPU without speed loss", opening paragraph: about 8 of
//           256 experts per token), counts the choices and stores the
//           token's normalised input in fp16.
//   gateup  every work-group groups the step's accesses by distinct expert;
//           work-group (0,0) also runs the placement policy of the same
//           page's paragraph "The key components" over them in (token, rank)
//           order.  Work-group (g, j) streams rows 16g..16g+15 of the gate and
//           up matrices of distinct expert j once, for all the tokens that
//           chose it: a skinny GEMM on the matrix cores (tokens x rows, the
//           Q4_0 codes decoded exactly to fp16, each block's scale applied in
//           fp32).
//   down    work-group p computes output rows 16p..16p+15 of every distinct
//           expert's down GEMV on the matrix cores the same way, then the
//           gate-weighted combine of each token in rank order, the residual,
//           and the next layer's router partials of every token over those rows.
//
// A token's result does not depend on which other tokens share its step nor
// on where its experts' weights sit: the matrix cores sum each output element
// in a fixed order, and the combine and the router partials are per token.
#include <hip/hip_runtime.h>
#include <math.h>

#include "device_common.h"
#include "internal.h"
#include "policy.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kGURowsMax = 24;  // distinct-expert rows of the gate/up grid (more experts loop)
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(unsigned short, (_Float16)lo) |
           ((uint32_t)__builtin_bit_cast(unsigned short, (_Float16)hi) << 16);
}
typedef __attribute__((address_space(4))) const BatchSel ConstSel;
static_assert(kNP == 128, "the route kernel sums the partial squares with two loads per lane");
static_assert(kMaxBK <= kThreads, "one thread per access in the gate/up kernel's grouping");

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
        // lane q: Q4_0 block q of x; the trace row, then the normalised block
        // rounded to fp16, for the gate/up kernel's matrix-core operand
        f32x4 xx[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) xx[j] = *reinterpret_cast<const f32x4*>(&xt[36 * lane + 4 * j]);
        if (a.tr_x && ttok < a.tr_cap) {
            f32x4* t4 = reinterpret_cast<f32x4*>(a.tr_x + ((int64_t)ttok * a.L + a.layer) * kQD);
#pragma unroll
            for (int j = 0; j < 8; ++j) t4[lane * 8 + j] = xx[j];
        }
        // matrix-core operand order: 16 bytes h = (u[4h..4h+3], u[16+4h..16+4h+3])
        u32x4* dst = reinterpret_cast<u32x4*>(a.u16 + ((int64_t)b * kQD + 32 * lane));
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const f32x4 u0 = xx[h] * inv, u1 = xx[4 + h] * inv;
            dst[h] = u32x4{pack_f16(u0.x, u0.y), pack_f16(u0.z, u0.w), pack_f16(u1.x, u1.y), pack_f16(u1.z, u1.w)};
        }
    }
}

// ---------------------------------------------------------------- gate/up

// Matrix-core operand order inside a Q4_0 block: position p = 8h + i (h = 0..3)
// holds weight 4h + i for i < 4 and weight 16 + 4h + (i - 4) for i >= 4, so that
// the four code bytes 4h..4h+3 of a row supply one lane's eight values (low
// nibbles, then high nibbles).  Activations are stored in the same order.
__device__ __forceinline__ int mfma_pos(int k) {  // position of weight k (0..31) of a block
    return (k & 16) ? 8 * ((k - 16) >> 2) + 4 + (k & 3) : 8 * (k >> 2) + (k & 3);
}

// One lane's eight weights of a block as fp16 (q - 8), exact: code word w
// (bytes 4h..4h+3 of the row's block).  A byte permute sets each code under
// the byte 0x64, so each fp16 is 1024 + q exactly; subtracting 1032 is exact.
__device__ __forceinline__ f16x8 q4_word_to_f16x8(uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    constexpr uint32_t kHi = 0x64646464u, k01 = 0x04010400u, k23 = 0x04030402u;
    const f16x2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
    const f16x2 p0 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(kHi, lo, k01)) - off;
    const f16x2 p1 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(kHi, lo, k23)) - off;
    const f16x2 p2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(kHi, hi, k01)) - off;
    const f16x2 p3 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(kHi, hi, k23)) - off;
    return f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

constexpr int kGUCodeStride = 260;  // words per chunk row in LDS (1 KiB + 16 B: rows fall on distinct banks)
constexpr int kGUScaleStride = 66;  // fp16 scales per chunk row in LDS

// Rows 16g..16g+15 of the gate (tile 0) and up (tile 1) matrices of distinct
// expert j, for the tokens that chose it.  The chunk's codes and scales are
// loaded with coalesced 16-byte loads and staged in LDS; then wave w runs Q4_0
// blocks 16w..16w+15 on the matrix cores: D[token m][row n] = sum over the
// block of u[m][k] (q[n][k] - 8), lane layout A[m = lane%16][p = 8(lane/16)+i],
// B[p][n = lane%16], D[m = 4(lane/16) + r][n], followed by the block's fp16
// scale of row n in fp32.  The four waves' sums are added in wave order.
__device__ __forceinline__ void qb_gateup_expert(const QBArgs& a, int e, int slot, uint64_t wseq, int c0, int cn,
                                                 const int32_t* dent, int g, uint32_t* s_code, unsigned short* s_sc,
                                                 float (*red)[2][16][17]) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int K = a.K;
    if (slot < 0 || slot >= a.n_slots || cn < 1 || cn > kMaxB) {  // never expected: refuse rather than fault
        if (t == 0) atomicOr(a.pt.error, (int)ERR_BAD_SLOT);
        return;
    }
    // a fill made in this step: read from the host arena and copied into the
    // ring slot by this expert's work-groups (chunk g and 1/32 of the down rows)
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
    // wave w loads chunk rows 8w..8w+7, lane = block (one coalesced 1 KiB line per row)
    const u32x4* cp = reinterpret_cast<const u32x4*>(chunk) + w * 8 * 64 + lane;
    u32x4 c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = __builtin_nontemporal_load(cp + i * 64);
    const u32x4 sc = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(chunk + 32768) + w * 64 + lane);
    // the tokens' activations of this wave's blocks, A rows = tokens
    const int l16 = lane & 15, kg = lane >> 4;
    const int tok = l16 < cn ? dent[l16] / K : -1;
    f16x8 A[16];
#pragma unroll
    for (int bb = 0; bb < 16; ++bb)
        A[bb] = tok >= 0 ? *reinterpret_cast<const f16x8*>(a.u16 + (int64_t)tok * kQD + (16 * w + bb) * 32 + 8 * kg)
                         : f16x8{};
    if (pull) {
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
    // stage: row r = 8w + i, block = lane
#pragma unroll
    for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x4*>(s_code + (8 * w + i) * kGUCodeStride + lane * 4) = c[i];
    {
        const uint32_t sw[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) s_sc[(8 * w + i) * kGUScaleStride + lane] = (unsigned short)(sw[i >> 1] >> ((i & 1) * 16));
    }
    __syncthreads();
    f32x4 acc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int bb = 0; bb < 16; ++bb) {
        const int b = 16 * w + bb;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int r = tt * 16 + l16;  // chunk row: gate rows 0..15, up rows 16..31
            const f16x8 B = q4_word_to_f16x8(s_code[r * kGUCodeStride + b * 4 + kg]);
            const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[bb], B, zero, 0, 0, 0);
            const float s = half_bits_to_float(s_sc[r * kGUScaleStride + b]);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[tt][q] += s * d[q];
        }
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int q = 0; q < 4; ++q) red[w][tt][4 * kg + q][l16] = acc[tt][q];
    __syncthreads();
    {
        const int m = t >> 4, n = t & 15;  // token m, row n
        if (m < cn) {
            const float gt = ((red[0][0][m][n] + red[1][0][m][n]) + red[2][0][m][n]) + red[3][0][m][n];
            const float ut = ((red[0][1][m][n] + red[1][1][m][n]) + red[2][1][m][n]) + red[3][1][m][n];
            const int f = g * 16 + n;  // h row c0 + m (grouped order), in the down launch's operand order
            a.h16[(int64_t)(c0 + m) * kQF + (f & ~31) + mfma_pos(f & 31)] =
                __builtin_bit_cast(unsigned short, (_Float16)(silu(gt) * ut));
        }
    }
}

// Grid (f/16, min(B*K, E, 24)).  Every work-group groups the step's accesses
// by distinct expert (ascending id; each expert's accesses in (token, rank)
// order) from the route launch's selections, then takes distinct experts
// y, y + gridDim.y, ...  Work-group (0,0) also runs the placement policy over
// the accesses in (token, rank) order — the paragraph "The key components":
// pinned set, LRU spare ring, fills — writes the grouping and the slots for
// the down launch, and publishes the slots only when some expert is cold;
// only cold experts' work-groups wait for that.
__global__ __launch_bounds__(kThreads) void qb_gateup_kernel(QBArgs a) {
    __shared__ __align__(16) uint32_t s_code[32 * kGUCodeStride];  // work-group (0,0): the ring tables first
    __shared__ unsigned short s_sc[32 * kGUScaleStride];
    __shared__ float red[4][2][16][17];
    __shared__ int32_t s_idx[kMaxBK], s_pin[kMaxBK], s_cnt[kMaxBK], s_off[kMaxBK + 1], s_dexp[kMaxBK],
        s_dent[kMaxBK], s_slot[kMaxBK];
    __shared__ unsigned long long s_wseq[kMaxBK];
    __shared__ uint32_t s_bits[kMaxE / 32];
    __shared__ uint32_t s_tbits[kMaxB][kMaxE / 32];  // experts chosen by each token
    __shared__ int32_t s_pre[kMaxE / 32];
    __shared__ int s_D, s_cold, s_jslot;
    __shared__ unsigned long long s_jwait;
    static_assert(sizeof(s_code) >= kMaxR * (4 + 8 + 8), "the ring tables fit in the code staging area");

    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    BatchSel* sel = a.sel;
    const int nb = *a.nb, K = a.K, E = a.E, n = nb * K;
    const bool leader = blockIdx.x == 0 && blockIdx.y == 0;
    const int nw = (E + 31) >> 5;

    // ---- the grouping: rank of an expert among the distinct ones from a
    // bitmap of the chosen experts; an access's place in its group from the
    // earlier tokens that chose the same expert (each token chooses an
    // expert at most once), read from per-token bitmaps
    if (t == 0) s_cold = 0;
    for (int i = t; i < nw; i += kThreads) s_bits[i] = 0u;
    for (int i = t; i < nb * nw; i += kThreads) s_tbits[i / nw][i % nw] = 0u;
    if (t < kMaxBK) s_cnt[t] = 0;
    int e_t = -1, pin_t = -1;
    if (t < n) {
        e_t = sel->idx[t];
        pin_t = sel->slot[t];  // pinned slot or -1, from the route launch
        s_idx[t] = e_t;
        s_pin[t] = pin_t;
    }
    __syncthreads();
    if (t < n) {
        atomicOr(&s_bits[e_t >> 5], 1u << (e_t & 31));
        atomicOr(&s_tbits[t / K][e_t >> 5], 1u << (e_t & 31));
        if (pin_t < 0) s_cold = 1;
    }
    __syncthreads();
    if (w == 0) {  // exclusive prefix of the per-word popcounts
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
        const int tb = t / K;
#pragma unroll
        for (int b2 = 0; b2 < kMaxB; ++b2)
            if (b2 < tb) pos += (s_tbits[b2][e_t >> 5] >> (e_t & 31)) & 1u;
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
    if (leader && w == 1) {
        // the policy, one access at a time in (token, rank) order
        RingState rs{};
        if (!s_cold) {
            for (int i = lane; i < n; i += 64) {
                s_slot[i] = s_pin[i];
                s_wseq[i] = 0ull;
            }
            rs.n_pin = n;
        } else {
            int32_t* r_owner = reinterpret_cast<int32_t*>(s_code);
            uint64_t* r_stamp = reinterpret_cast<uint64_t*>(s_code + kMaxR);
            uint64_t* r_seq = reinterpret_cast<uint64_t*>(s_code + 3 * kMaxR);
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
        s_dent[s_off[rank] + pos] = t;
        if (pos == 0) s_dexp[rank] = e_t;
    }
    if (leader) {
        // the grouping and the slots, for the down launch and the cold
        // experts' work-groups
        if (t < n) {
            sel->slot[t] = s_slot[t];
            sel->dent[s_off[rank] + pos] = t;
            if (pos == 0) {  // the expert's first access: its slot, and the fill it made (if any)
                sel->dexp[rank] = e_t;
                sel->dslot[rank] = s_slot[t];
                sel->dwait[rank] = s_wseq[t];
            }
        }
        if (t <= D) sel->doff[t] = t < D ? s_off[t] : n;
        if (t == 0) sel->D = D;
        if (s_cold) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __syncthreads();
            if (t == 0) __hip_atomic_store(a.pub, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();

    for (int j = blockIdx.y; j < D; j += gridDim.y) {
        if (j != (int)blockIdx.y) __syncthreads();  // LDS reuse
        const int c0 = s_off[j], cn = s_cnt[j];
        const int first = s_dent[c0];
        int slot = s_pin[first];
        uint64_t wseq = 0;
        if (slot < 0) {  // cold: the slot work-group (0,0) chose
            if (leader) {
                slot = s_slot[first];
                wseq = s_wseq[first];
            } else {
                if (t == 0) {
                    const uint64_t t0 = wall_clock64();
                    while (__hip_atomic_load(a.pub, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
                        __builtin_amdgcn_s_sleep(1);
                        if (qb_spin_expired(a, t0)) {
                            atomicOr(a.pt.error, (int)ERR_FILL_TIMEOUT);
                            break;
                        }
                    }
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                    s_jslot = __hip_atomic_load(&sel->dslot[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    s_jwait = __hip_atomic_load(&sel->dwait[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                __syncthreads();
                slot = s_jslot;
                wseq = s_jwait;
            }
        }
        qb_gateup_expert(a, s_dexp[j], slot, wseq, c0, cn, s_dent + c0, blockIdx.x, s_code, s_sc, red);
    }
}

// ---------------------------------------------------------------- down + combine + next router partials

constexpr int kDownThreads = 1024;
constexpr int kDCodeStride = 68;  // words per down row in a wave's LDS (256 B + 16 B)

// Grid kNP, 1024 threads.  Work-group p owns output rows 16p..16p+15.  Wave w
// takes distinct experts w, w + 16, ...: it stages the expert's 16 down rows
// (4 KiB of codes, 512 B of scales, coalesced) in its own LDS, then runs the
// 16 Q4_0 blocks along f on the matrix cores with the tokens that chose the
// expert as rows, as in gate/up.  Then the gate-weighted combine of each token
// in rank order, the residual, and the next layer's router partials of every
// token over the work-group's rows.
__global__ __launch_bounds__(kDownThreads) void qb_down_kernel(QBArgs a) {
    // the wave index as a uniform value, so the selection reads below are
    // scalar loads (counted apart from the vector loads)
    const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int p = blockIdx.x;
    const int nb = *a.nb;
    const int K = a.K, n = nb * K, E = a.E;
    const ConstSel* sel = (const ConstSel*)a.sel;
    const int D = sel->D;
    __shared__ __align__(16) uint32_t s_code[kDownThreads / 64][16 * kDCodeStride];
    __shared__ float s_sc[kDownThreads / 64][16][17];
    __shared__ float zs[kMaxBK][kRW + 1];
    __shared__ float xn[kMaxB][kRW];
    __shared__ float s_g[kMaxBK];

    // the combine's inputs are loaded now but stored to LDS after the experts
    // loop, so the loop's loads do not wait behind them
    const int tb = t >> 4, tr = t & 15;  // combine: token tb, row tr
    float xr = 0.0f, gt = 0.0f;
    if (tb < nb) xr = a.xb[(int64_t)tb * kQD + p * kRW + tr];
    if (t < n) gt = sel->gate[t];

    const int l16 = lane & 15, kg = lane >> 4;
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    uint32_t* wcode = s_code[w];
    // the wave's first expert record is read together with D (w < 16 <= kMaxBK
    // keeps it in bounds), so its weight loads wait for one round trip, not two
    static_assert(kDownThreads / 64 <= kMaxBK, "first records in bounds");
    int nslot = sel->dslot[w], nc0 = sel->doff[w], nc1 = sel->doff[w + 1];
    for (int j = w; j < D; j += kDownThreads / 64) {
        const int slot = nslot, c0 = nc0, cn = nc1 - nc0;
        if (j + kDownThreads / 64 < D) {
            nslot = sel->dslot[j + kDownThreads / 64];
            nc0 = sel->doff[j + kDownThreads / 64];
            nc1 = sel->doff[j + kDownThreads / 64 + 1];
        }
        if (slot < 0 || slot >= a.n_slots || cn < 1 || cn > kMaxB) {
            if (lane == 0) atomicOr(a.pt.error, (int)ERR_BAD_SLOT);
            continue;
        }
        const uint8_t* base = a.slots + (int64_t)slot * a.slot_bytes + kGURegion;
        // rows 16p..16p+15: 4 KiB of codes (lane: row 4q + lane/16, block lane%16) and
        // 512 B of scales (lane: rows 4(lane/16)..+3, block lane%16)
        const u32x4* cr = reinterpret_cast<const u32x4*>(base + (int64_t)p * kRW * 256) + lane;
        u32x4 cc[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) cc[q] = __builtin_nontemporal_load(cr + q * 64);
        const u32x2 sc = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(base + kDownCodes) + p * 64 + lane);
        // A row l16: h row c0 + l16 (the expert's tokens are rows c0 .. c0+cn-1);
        // the accesses of this lane's D rows, for the combine
        int dm[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) dm[q] = 4 * kg + q < cn ? sel->dent[c0 + 4 * kg + q] : 0;
        f16x8 A[16];
#pragma unroll
        for (int bb = 0; bb < 16; ++bb)
            A[bb] = l16 < cn ? *reinterpret_cast<const f16x8*>(a.h16 + (int64_t)(c0 + l16) * kQF + bb * 32 + 8 * kg)
                             : f16x8{};
        __builtin_amdgcn_wave_barrier();  // the wave's LDS region is free again
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<u32x4*>(wcode + (4 * q + kg) * kDCodeStride + l16 * 4) = cc[q];
        {
            const uint32_t sw[4] = {sc.x >> 0, sc.x >> 16, sc.y >> 0, sc.y >> 16};
#pragma unroll
            for (int i = 0; i < 4; ++i) s_sc[w][4 * kg + i][l16] = half_bits_to_float(sw[i]);
        }
        __builtin_amdgcn_wave_barrier();
        f32x4 acc = zero;
#pragma unroll
        for (int bb = 0; bb < 16; ++bb) {
            const f16x8 B = q4_word_to_f16x8(wcode[l16 * kDCodeStride + bb * 4 + kg]);
            const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[bb], B, zero, 0, 0, 0);
            const float s = s_sc[w][l16][bb];
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] += s * d[q];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int m = 4 * kg + q;
            if (m < cn) zs[dm[q]][l16] = acc[q];
        }
    }
    // the next layer's router rows of this work-group's slice, in flight during
    // the combine: thread t takes expert t % E (every expert when E divides
    // the thread count)
    if (t < n) s_g[t] = gt;
    const bool wfix = a.wr_part && (kDownThreads % E) == 0;
    f32x4 wpre[4];
    if (wfix) {
        const f32x4* w4 = reinterpret_cast<const f32x4*>(a.wr_part + ((int64_t)p * E + t % E) * kRW);
#pragma unroll
        for (int i = 0; i < 4; ++i) wpre[i] = w4[i];
    }
    __syncthreads();
    if (tb < nb) {
        float y = 0.0f;
#pragma unroll
        for (int kk = 0; kk < kQ4MaxK; ++kk)
            if (kk < K) y += s_g[tb * K + kk] * zs[tb * K + kk][tr];  // rank order
        const float o = xr + y;
        a.xb[(int64_t)tb * kQD + p * kRW + tr] = o;
        xn[tb][tr] = o;
    }
    if (a.wr_part) {
        __syncthreads();
        // pl[b][p][e] = sum_i Wr[e][16p+i] xn[b][i]; ps[b][p] = sum_i xn[b][i]^2
        for (int q = t; q < nb * E; q += kDownThreads) {
            const int b = q / E, e = q - b * E;
            f32x4 wv[4];
            if (wfix) {
#pragma unroll
                for (int i = 0; i < 4; ++i) wv[i] = wpre[i];
            } else {
                const f32x4* w4 = reinterpret_cast<const f32x4*>(a.wr_part + ((int64_t)p * E + e) * kRW);
#pragma unroll
                for (int i = 0; i < 4; ++i) wv[i] = w4[i];
            }
            const float* xs = xn[b];
            float s4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s4[i] = (wv[i].x * xs[4 * i] + wv[i].y * xs[4 * i + 1]) + (wv[i].z * xs[4 * i + 2] + wv[i].w * xs[4 * i + 3]);
            a.pl[((int64_t)b * kNP + p) * E + e] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        }
        if (t < nb) {
            float s2 = 0.0f;
#pragma unroll
            for (int i = 0; i < kRW; ++i) s2 += xn[t][i] * xn[t][i];
            a.ps[(int64_t)t * kNP + p] = s2;
        }
    }
    if (p == 0 && t == 0) *a.pub = 0u;  // every gate/up work-group of this layer has finished
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

hipError_t launch_qb_down(const QBArgs& a, hipStream_t s) {
    if (a.K < 1 || a.K > kQ4MaxK || a.E > kMaxE || a.B < 1 || a.B > kMaxB) return hipErrorInvalidValue;
    hipLaunchKernelGGL(qb_down_kernel, dim3(kNP), dim3(kDownThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
