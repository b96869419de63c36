// gfx950 batched prefill of the Q4_0 MoE stack: T tokens through one layer
// at a time.
//
//   norm     RMSNorm per token; the normalised input in bf16 for the expert
//            GEMMs, 1/rms kept in fp32 for the router.
//   router   logits[t][e] = inv_rms[t] * x[t]·Wr[e] + bias, fp32 MFMA.
//   topk     exact top-K per token and the softmax renormalised over the
//            chosen experts ("Luce Spark runs 35B MoE models on 16GB GPU
//            without speed loss", opening paragraph: about 8 of 256 experts
//            per token); per-expert routing counts (paragraph "The key
//            components", item 1) and the per-expert assignment histogram.
//   scatter  deterministic counting sort of the (token, rank) assignments by
//            (expert, token).
//   policy   one wave: the layer's distinct experts in ascending id, each
//            accessed once through the pinned set or the spare-slot ring
//            (same paragraph, item 2); the host runs it in chunks of at most
//            R cold experts, so every expert of a chunk is resident while the
//            chunk's GEMMs run.
//   fill     the policy run's fills pulled from the pinned host arena into
//            their ring slots (the same item's copy from host memory, done
//            by the GPU) by extra work-groups of the gate/up and down
//            launches over the chunk's pinned experts (three quarters of the
//            pieces, then the rest), so the copies cross PCIe while the
//            matrix cores work; the cold experts' GEMMs follow.  Without a
//            pull arena the host agent copies them and the GEMMs wait.
//   gateup   grouped GEMM on the matrix cores: H = silu(U Wg^T) * (U Wu^T)
//            per expert group; Q4_0 weights are dequantised to bf16 in LDS,
//            v_mfma_f32_16x16x32_bf16 accumulates in fp32.
//   down     grouped GEMM Y = H Wd^T, same scheme.
//   combine  x[t] += sum_k g[t][k] Y[pos(t,k)] in rank order.
//
// Every reduction order is fixed and no result depends on the slot a weight
// is read from, so prefill outputs are bit-identical at every residency.
#include <hip/hip_runtime.h>
#include <math.h>

#include "device_common.h"
#include "internal.h"
#include "policy.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kPfThreads = 256;
constexpr int kBM = 128;       // tokens per GEMM tile
constexpr int kBK = 64;        // K per pipeline step (two Q4_0 blocks)
constexpr int kLdsRow = 72;    // bf16 per LDS tile row (64 + 8 padding)

__device__ __forceinline__ uint16_t bf16_bits(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return (uint32_t)bf16_bits(lo) | ((uint32_t)bf16_bits(hi) << 16);
}

// 32 weights of one Q4_0 block (GGUF nibble order) as bf16 (q - 8) * s into
// dst[0..31] (LDS, 16-byte aligned).
__device__ __forceinline__ void dequant_block_bf16(const u32x4 c, float s, uint16_t* dst) {
    const uint32_t wd[4] = {c.x, c.y, c.z, c.w};
    uint32_t lo[8], hi[8];
    const float m8 = -8.0f * s;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t x = wd[m];
        // bytes 4m..4m+3: low nibbles are weights 4m..4m+3, high nibbles 4m+16..4m+19
        const float l0 = fmaf((float)(x & 0xfu), s, m8), l1 = fmaf((float)((x >> 8) & 0xfu), s, m8);
        const float l2 = fmaf((float)((x >> 16) & 0xfu), s, m8), l3 = fmaf((float)((x >> 24) & 0xfu), s, m8);
        const float h0 = fmaf((float)((x >> 4) & 0xfu), s, m8), h1 = fmaf((float)((x >> 12) & 0xfu), s, m8);
        const float h2 = fmaf((float)((x >> 20) & 0xfu), s, m8), h3 = fmaf((float)(x >> 28), s, m8);
        lo[2 * m] = pack_bf16(l0, l1);
        lo[2 * m + 1] = pack_bf16(l2, l3);
        hi[2 * m] = pack_bf16(h0, h1);
        hi[2 * m + 1] = pack_bf16(h2, h3);
    }
    u32x4* d4 = reinterpret_cast<u32x4*>(dst);
    d4[0] = u32x4{lo[0], lo[1], lo[2], lo[3]};
    d4[1] = u32x4{lo[4], lo[5], lo[6], lo[7]};
    d4[2] = u32x4{hi[0], hi[1], hi[2], hi[3]};
    d4[3] = u32x4{hi[4], hi[5], hi[6], hi[7]};
}

// ---------------------------------------------------------------- norm

// Grid T, 256 threads: one token per work-group.
__global__ __launch_bounds__(kPfThreads) void pf_norm_kernel(PfArgs a) {
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const f32x4* x4 = reinterpret_cast<const f32x4*>(a.x + (int64_t)t * kQD);
    const f32x4 v0 = x4[tid], v1 = x4[tid + kPfThreads];
    float ss = (v0.x * v0.x + v0.y * v0.y) + (v0.z * v0.z + v0.w * v0.w);
    ss += (v1.x * v1.x + v1.y * v1.y) + (v1.z * v1.z + v1.w * v1.w);
    ss = wave_sum(ss);
    __shared__ float part[4];
    if (lane == 0) part[w] = ss;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    const float inv = a.norm ? 1.0f / sqrtf(tot / (float)kQD + a.eps) : 1.0f;
    if (tid == 0) a.inv[t] = inv;
    uint32_t* u2 = reinterpret_cast<uint32_t*>(a.u + (int64_t)t * kQD);
    u2[2 * tid] = pack_bf16(v0.x * inv, v0.y * inv);
    u2[2 * tid + 1] = pack_bf16(v0.z * inv, v0.w * inv);
    u2[2 * (tid + kPfThreads)] = pack_bf16(v1.x * inv, v1.y * inv);
    u2[2 * (tid + kPfThreads) + 1] = pack_bf16(v1.z * inv, v1.w * inv);
    const int64_t tt = (int64_t)*a.tr_base + t;
    if (a.tr_x && tt < a.tr_cap) {
        f32x4* tr = reinterpret_cast<f32x4*>(a.tr_x + (tt * a.L + a.layer) * kQD);
        tr[tid] = v0;
        tr[tid + kPfThreads] = v1;
    }
}

// ---------------------------------------------------------------- router

// One work-group of 4 waves per 32 tokens x 32 experts, on the fp32 matrix
// cores (v_mfma_f32_16x16x4_f32: fp32 products, fp32 accumulation).  Wave w
// covers d in [512w, 512w + 512).  For a 16-wide slice k0..k0+15 of d, lane
// (i, g) = (lane % 16, lane / 16) loads the four consecutive values 4g..4g+3
// of token row i and of expert row i (the router is packed [d/16][E][16], so
// both are 16-byte loads); MFMA j then takes k = k0 + 4g + j from lane group g
// on both operands, which covers the slice.  The four waves' partial sums
// meet in LDS and are added in wave order.
// Output: logits[t][e] = inv_rms[t] * (x[t] . Wr[e]) + bias.
__global__ __launch_bounds__(256) void pf_router_kernel(PfArgs a) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, i = lane & 15, g = lane >> 4;
    const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
    const int E = a.E;
    const bool ta = t0 + i < a.T, tb = t0 + 16 + i < a.T;
    const bool ea = e0 + i < E, eb = e0 + 16 + i < E;
    const float* xa = a.x + (int64_t)(ta ? t0 + i : 0) * kQD + 4 * g;
    const float* xb = a.x + (int64_t)(tb ? t0 + 16 + i : 0) * kQD + 4 * g;
    const float* wa = a.wr + (int64_t)(ea ? e0 + i : 0) * kRW + 4 * g;
    const float* wb = a.wr + (int64_t)(eb ? e0 + 16 + i : 0) * kRW + 4 * g;
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 acc[2][2] = {{zero, zero}, {zero, zero}};
    constexpr int kSplit = kQD / 4;
#pragma unroll 4
    for (int k0 = w * kSplit; k0 < (w + 1) * kSplit; k0 += kRW) {
        const f32x4 A0 = ta ? *reinterpret_cast<const f32x4*>(xa + k0) : zero;
        const f32x4 A1 = tb ? *reinterpret_cast<const f32x4*>(xb + k0) : zero;
        const int64_t wo = (int64_t)(k0 / kRW) * E * kRW;
        const f32x4 B0 = ea ? *reinterpret_cast<const f32x4*>(wa + wo) : zero;
        const f32x4 B1 = eb ? *reinterpret_cast<const f32x4*>(wb + wo) : zero;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(A0[j], B0[j], acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(A0[j], B1[j], acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(A1[j], B0[j], acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(A1[j], B1[j], acc[1][1], 0, 0, 0);
        }
    }
    __shared__ __align__(16) f32x4 part[4][4][64];  // [wave][tile m*2+n][lane]
#pragma unroll
    for (int q = 0; q < 4; ++q) part[w][q][lane] = acc[q >> 1][q & 1];
    __syncthreads();
    // wave w finishes tile q = w: lane (i, g) holds rows 4g..4g+3 of column i
    const int m = w >> 1, n = w & 1;
    const f32x4 sum = ((part[0][w][lane] + part[1][w][lane]) + part[2][w][lane]) + part[3][w][lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int tok = t0 + 16 * m + 4 * g + r;
        const int e = e0 + 16 * n + i;
        if (tok >= a.T || e >= E) continue;
        const float inv = a.inv[tok];
        float bias = 0.0f;
        if (a.bias) {
            int row = a.bias_row ? a.bias_row[tok] : 0;
            row = row < 0 ? 0 : (row >= a.n_bias_rows ? a.n_bias_rows - 1 : row);
            bias = a.bias[(int64_t)row * E + e];
        }
        a.logits[(int64_t)tok * E + e] = sum[r] * inv + bias;
    }
}

// ---------------------------------------------------------------- top-k

// Grid T, 256 threads: top-K and gates of one token; routing counts and the
// assignment histogram (integer atomics: the totals are exact).
__global__ __launch_bounds__(kPfThreads) void pf_topk_kernel(PfArgs a) {
    const int t = blockIdx.x, tid = threadIdx.x;
    const int E = a.E, K = a.K;
    __shared__ __align__(16) float lg[kMaxE];
    __shared__ __align__(16) uint64_t kpad[kPfThreads];
    __shared__ __align__(16) uint64_t cand[kMaxE / 64 * kQ4MaxK + 16];
    __shared__ int s_e[kMaxK];
    __shared__ float s_l[kMaxK];
    for (int e = tid; e < E; e += kPfThreads) lg[e] = a.logits[(int64_t)t * E + e];
    __syncthreads();
    block_topk(lg, E, K, kpad, cand, s_e, s_l);
    if (tid < K) {
        const int e = s_e[tid];
        float z = 0.0f;
        for (int kk = 0; kk < K; ++kk) z += expf(s_l[kk] - s_l[0]);
        const float g = expf(s_l[tid] - s_l[0]) / z;
        a.topk[(int64_t)t * K + tid] = e;
        a.gates[(int64_t)t * K + tid] = g;
        atomicAdd(reinterpret_cast<unsigned long long*>(a.pt.counts + (int64_t)a.layer * E + e), 1ull);
        atomicAdd(a.hist + e, 1);
        const int64_t tt = (int64_t)*a.tr_base + t;
        if (a.tr_topk && tt < a.tr_cap) {
            const int64_t o = (tt * a.L + a.layer) * K + tid;
            a.tr_topk[o] = e;
            a.tr_gates[o] = g;
        }
    }
}

// ---------------------------------------------------------------- scatter

// Grid E, 256 threads: work-group e lists the tokens that chose expert e, in
// ascending token order, at positions goff[e] .. goff[e+1]-1.
__global__ __launch_bounds__(kPfThreads) void pf_scatter_kernel(PfArgs a) {
    const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int K = a.K;
    if (a.goff[e + 1] == a.goff[e]) return;
    __shared__ int wtot[4];
    int base = a.goff[e];
    for (int t0 = 0; t0 < a.T; t0 += kPfThreads) {
        const int t = t0 + tid;
        int kk = -1;
        if (t < a.T)
            for (int q = 0; q < K; ++q)
                if (a.topk[(int64_t)t * K + q] == e) kk = q;
        const uint64_t m = __ballot(kk >= 0);
        const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (lane == 0) wtot[w] = __builtin_popcountll(m);
        __syncthreads();
        int off = base;
        for (int q = 0; q < w; ++q) off += wtot[q];
        if (kk >= 0) {
            const int pos = off + before;
            a.perm[pos] = t;
            a.apos[(int64_t)t * K + kk] = pos;
        }
        base += (wtot[0] + wtot[1]) + (wtot[2] + wtot[3]);
        __syncthreads();
    }
}

// ---------------------------------------------------------------- policy

// Lane 0 keeps an access's slot; a fill that the fill kernel pulls goes on
// the fill list and needs no wait (the fill kernel runs before the GEMMs on
// the same stream); a fill copied by the host agent is waited for.
__device__ __forceinline__ void pf_record(const PfArgs& a, int e, int slot, uint64_t wseq, int& nf) {
    if (threadIdx.x == 0) {
        a.pslot[e] = slot;
        a.pwait[e] = a.arena ? 0ull : wseq;
        if (a.arena && wseq && nf < a.pt.R) {
            a.pfill[1 + 2 * nf] = a.layer * a.E + e;
            a.pfill[2 + 2 * nf] = slot;
        }
    }
    if (a.arena && wseq) ++nf;
}

// One wave: the chunk's experts (ascending id) through the placement policy.
__global__ __launch_bounds__(64) void pf_policy_kernel(PfArgs a) {
    __shared__ int32_t r_owner[kMaxR];
    __shared__ uint64_t r_stamp[kMaxR];
    __shared__ uint64_t r_seq[kMaxR];
    const PolicyTables& pt = a.pt;
    RingState rs{};
    ring_load(pt, r_owner, r_stamp, r_seq, rs);
    int nf = 0;
    for (int i = 0; i < a.n_pf_experts; ++i) {
        const int e = a.pf_experts[i];
        int slot;
        uint64_t wseq;
        ring_access(pt, a.layer, e, pt.slot_of[(int64_t)a.layer * a.E + e], r_owner, r_stamp, r_seq, rs, slot,
                    wseq);
        pf_record(a, e, slot, wseq, nf);
    }
    if (threadIdx.x == 0) a.pfill[0] = nf;
    ring_store(pt, r_owner, r_stamp, r_seq, rs);
    stats_flush(pt, a.n_pf_experts, rs);
}

// One wave, right after the routing: the first chunk's experts through the
// placement policy, so that its fills start before the host has planned the
// layer.  The chunk is cut by the host's rule: the layer's experts with
// assignments (hist > 0), ascending, up to and excluding the one that would
// be the (R+1)-th unpinned expert.
__global__ __launch_bounds__(64) void pf_policy_first_kernel(PfArgs a) {
    __shared__ int32_t r_owner[kMaxR];
    __shared__ uint64_t r_stamp[kMaxR];
    __shared__ uint64_t r_seq[kMaxR];
    const PolicyTables& pt = a.pt;
    const int lane = threadIdx.x, E = a.E;
    const int64_t lbase = (int64_t)a.layer * E;
    RingState rs{};
    ring_load(pt, r_owner, r_stamp, r_seq, rs);
    int cold = 0, n = 0, nf = 0;
    bool full = false;
    for (int base = 0; base < E && !full; base += 64) {
        const int e = base + lane;
        const bool used = e < E && a.hist[e] > 0;
        uint64_t mu = __ballot(used);
        const uint64_t mc = __ballot(used && pt.slot_of[lbase + e] < 0);
        while (mu) {
            const int b = __builtin_ctzll(mu);
            mu &= mu - 1;
            const bool is_cold = (mc >> b) & 1ull;
            if (is_cold && cold == pt.R) {
                full = true;
                break;
            }
            cold += is_cold;
            const int ex = base + b;
            int slot;
            uint64_t wseq;
            ring_access(pt, a.layer, ex, pt.slot_of[lbase + ex], r_owner, r_stamp, r_seq, rs, slot, wseq);
            pf_record(a, ex, slot, wseq, nf);
            ++n;
        }
    }
    if (lane == 0) a.pfill[0] = nf;
    ring_store(pt, r_owner, r_stamp, r_seq, rs);
    stats_flush(pt, n, rs);
}

// ---------------------------------------------------------------- pulled fills

constexpr int kFillPiece = 16384;  // bytes of a slot per copy step
constexpr int kFillGUShare = 192;  // of 256: the part of the fill pieces the gate/up launch copies, down the rest

// Work-group wid of nwg: copies pieces lo + wid, lo + wid + nwg, ... below
// hi of the last policy run's fills, where the pieces are numbered over all
// fills (fill j, piece p = bytes [p*kFillPiece, (p+1)*kFillPiece) of the
// slot) and [lo, hi) is the share [s0/256, s1/256) of them; from the host
// arena, across PCIe, into the fills' ring slots.
__device__ void pf_fill_pieces(const PfArgs& a, int wid, int nwg, int s0, int s1) {
    const int t = threadIdx.x;
    const int nf = min(a.pfill[0], a.pt.R);
    const int pieces = (int)((a.slot_bytes + kFillPiece - 1) / kFillPiece);
    const int lo = nf * pieces * s0 / 256, hi = nf * pieces * s1 / 256;
    constexpr int kPer = kFillPiece / 16 / kPfThreads;
    for (int u = lo + wid; u < hi; u += nwg) {
        const int j = u / pieces, p = u - j * pieces;
        const int key = a.pfill[1 + 2 * j], slot = a.pfill[2 + 2 * j];
        if (key < 0 || key >= a.L * a.E || slot < a.P || slot >= a.n_slots) {
            if (t == 0 && p == 0) atomicOr(a.pt.error, (int)ERR_BAD_SLOT);
            continue;
        }
        const int64_t off = (int64_t)p * kFillPiece;
        const int nw = (int)(min((int64_t)kFillPiece, a.slot_bytes - off) / 16);
        const u32x4* src = reinterpret_cast<const u32x4*>(a.arena + (int64_t)key * a.slot_bytes + off);
        u32x4* dst = reinterpret_cast<u32x4*>(a.slots + (int64_t)slot * a.slot_bytes + off);
        u32x4 v[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if (t + i * kPfThreads < nw) v[i] = __builtin_nontemporal_load(src + t + i * kPfThreads);
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if (t + i * kPfThreads < nw) __builtin_nontemporal_store(v[i], dst + t + i * kPfThreads);
    }
}

// ---------------------------------------------------------------- grouped GEMMs

// Resolve a GEMM work item: expert, first row of its group, rows in the tile,
// slot.  Waits (bounded) for a fill that is still in flight.  Returns false
// if the work-group has nothing valid to do.
__device__ bool pf_item(const PfArgs& a, int item, int& e, int& pos0, int& rows, const uint8_t*& S) {
    e = a.items[2 * item];
    const int m0 = a.items[2 * item + 1];
    const int n_e = a.goff[e + 1] - a.goff[e];
    pos0 = a.goff[e] + m0;
    rows = min(kBM, n_e - m0);
    const int slot = a.pslot[e];
    const uint64_t wseq = a.pwait[e];
    if (rows <= 0 || slot < 0 || slot >= a.n_slots) {
        if (threadIdx.x == 0 && rows > 0) atomicOr(a.pt.error, (int)ERR_BAD_SLOT);
        return false;
    }
    if (wseq && slot >= a.P) {
        if (threadIdx.x == 0) {
            const uint64_t* flag = a.ready + (slot - a.P);
            const uint64_t t0 = wall_clock64();
            int polls = 0;
            while (__hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM) < wseq) {
                fill_poll_pause(polls);
                if (wall_clock64() - t0 > a.spin_limit_ticks ||
                    (__hip_atomic_load(a.pt.error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & ERR_FILL_TIMEOUT)) {
                    atomicOr(a.pt.error, (int)ERR_FILL_TIMEOUT);
                    break;
                }
            }
        }
        __syncthreads();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
    }
    S = a.slots + (int64_t)slot * a.slot_bytes;
    return true;
}

// MFMA tile compute of one kBK step: wave (wm, wn) owns rows wm*64..+63 and
// the 4 16-column groups listed in cols[]; acc[mi][nj] is 16x16.
__device__ __forceinline__ void mfma_step(const uint16_t* As, const uint16_t* Bs, int wm, const int* cols,
                                          f32x4 (&acc)[4][4]) {
    const int lane = threadIdx.x & 63;
    const int lr = lane & 15, lk = (lane >> 4) * 8;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
        bf16x8 af[4], bfr[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
            af[mi] = *reinterpret_cast<const bf16x8*>(As + (wm * 64 + mi * 16 + lr) * kLdsRow + kh * 32 + lk);
#pragma unroll
        for (int nj = 0; nj < 4; ++nj)
            bfr[nj] = *reinterpret_cast<const bf16x8*>(Bs + (cols[nj] + lr) * kLdsRow + kh * 32 + lk);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int nj = 0; nj < 4; ++nj)
                acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bfr[nj], acc[mi][nj], 0, 0, 0);
    }
}

// Grid (n_items, f/64), 256 threads.  Work-group tile: kBM tokens of one
// expert group x (64 gate rows + the same 64 up rows); wave w: rows
// (w&1)*64.., gate and up columns (w>>1)*32..; SwiGLU in the epilogue.
// B rows come from the slot's gate/up region (chunk g = row/16: codes at
// ((ww*8 + i)*64 + b)*16, scales at 32768 + (ww*64 + b)*16 + 2i).
__global__ __launch_bounds__(kPfThreads) void pf_gateup_kernel(PfArgs a) {
    if ((int)blockIdx.x < a.n_fill_x) {  // the leading columns pull the fills
        pf_fill_pieces(a, (int)(blockIdx.y * a.n_fill_x + blockIdx.x), a.n_fill_x * (int)gridDim.y, 0, kFillGUShare);
        return;
    }
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n0 = blockIdx.y * 64;
    int e, pos0, rows;
    const uint8_t* S;
    if (!pf_item(a, (int)blockIdx.x - a.n_fill_x, e, pos0, rows, S)) return;
    __shared__ __align__(16) uint16_t As[kBM * kLdsRow];
    __shared__ __align__(16) uint16_t Bs[128 * kLdsRow];
    __shared__ int tok[kBM];
    if (tid < kBM) tok[tid] = tid < rows ? a.perm[pos0 + tid] : -1;
    __syncthreads();
    // A loads: row tid>>1, 32 bf16 (64 B) at column half (tid&1)*32
    const int ar = tid >> 1, ah = (tid & 1) * 32;
    const int atok = tok[ar];
    const u32x4* arow = atok >= 0 ? reinterpret_cast<const u32x4*>(a.u + (int64_t)atok * kQD + ah) : nullptr;
    // B loads: row br = tid>>1 (gate rows 0..63, up rows 64..127), block (tid&1) of the step
    const int br = tid >> 1, bb = tid & 1;
    const int mrow = n0 + (br & 63);
    const int ww = (br >= 64 ? 2 : 0) + ((mrow >> 3) & 1);
    const uint8_t* bchunk = S + (int64_t)(mrow >> 4) * kGUChunk;
    const int bi = mrow & 7;

    f32x4 acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) acc[mi][nj] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int wm = w & 1, wn = w >> 1;
    const int cols[4] = {wn * 32, wn * 32 + 16, 64 + wn * 32, 64 + wn * 32 + 16};

    u32x4 ra[4], rc;
    uint32_t rsc;
    auto load = [&](int k0) {
        const int b = k0 / 32 + bb;
        if (arow) {
#pragma unroll
            for (int j = 0; j < 4; ++j) ra[j] = arow[k0 / 8 + j];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) ra[j] = u32x4{0u, 0u, 0u, 0u};
        }
        rc = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(bchunk + ((ww * 8 + bi) * 64 + b) * 16));
        rsc = *reinterpret_cast<const uint16_t*>(bchunk + 32768 + (ww * 64 + b) * 16 + bi * 2);
    };
    load(0);
    for (int k0 = 0; k0 < kQD; k0 += kBK) {
        __syncthreads();
        {
            u32x4* ad = reinterpret_cast<u32x4*>(As + ar * kLdsRow + ah);
#pragma unroll
            for (int j = 0; j < 4; ++j) ad[j] = ra[j];
            dequant_block_bf16(rc, half_bits_to_float(rsc), Bs + br * kLdsRow + bb * 32);
        }
        __syncthreads();
        if (k0 + kBK < kQD) load(k0 + kBK);
        mfma_step(As, Bs, wm, cols, acc);
    }
    // epilogue: h = silu(gate) * up, bf16
    const int lr = lane & 15, lq = (lane >> 4) * 4;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int nj = 0; nj < 2; ++nj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wm * 64 + mi * 16 + lq + r;
                if (row < rows) {
                    const float g = acc[mi][nj][r], u = acc[mi][nj + 2][r];
                    a.h[(int64_t)(pos0 + row) * kQF + n0 + wn * 32 + nj * 16 + lr] = bf16_bits(silu(g) * u);
                }
            }
}

// Grid (n_items, d/128), 256 threads.  Work-group tile: kBM tokens x 128
// down rows; wave w: rows (w&1)*64.., columns (w>>1)*64...  B rows from the
// slot's down region: codes [r][b][16 B], scales [r/4][b][4] fp16.
__global__ __launch_bounds__(kPfThreads) void pf_down_kernel(PfArgs a) {
    if ((int)blockIdx.x < a.n_fill_x) {  // the leading columns pull the rest of the fills
        pf_fill_pieces(a, (int)(blockIdx.y * a.n_fill_x + blockIdx.x), a.n_fill_x * (int)gridDim.y, kFillGUShare,
                       256);
        return;
    }
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n0 = blockIdx.y * 128;
    int e, pos0, rows;
    const uint8_t* S;
    if (!pf_item(a, (int)blockIdx.x - a.n_fill_x, e, pos0, rows, S)) return;
    __shared__ __align__(16) uint16_t As[kBM * kLdsRow];
    __shared__ __align__(16) uint16_t Bs[128 * kLdsRow];
    const int ar = tid >> 1, ah = (tid & 1) * 32;
    const u32x4* arow = ar < rows ? reinterpret_cast<const u32x4*>(a.h + (int64_t)(pos0 + ar) * kQF + ah) : nullptr;
    const int br = tid >> 1, bb = tid & 1;
    const int drow = n0 + br;
    const uint8_t* dcodes = S + kGURegion + (int64_t)drow * 256;
    const uint8_t* dscales = S + kGURegion + kDownCodes + (int64_t)(drow >> 2) * 128 + (drow & 3) * 2;

    f32x4 acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) acc[mi][nj] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int wm = w & 1, wn = w >> 1;
    const int cols[4] = {wn * 64, wn * 64 + 16, wn * 64 + 32, wn * 64 + 48};

    u32x4 ra[4], rc;
    uint32_t rsc;
    auto load = [&](int k0) {
        const int b = k0 / 32 + bb;
        if (arow) {
#pragma unroll
            for (int j = 0; j < 4; ++j) ra[j] = arow[k0 / 8 + j];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) ra[j] = u32x4{0u, 0u, 0u, 0u};
        }
        rc = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dcodes + b * 16));
        rsc = *reinterpret_cast<const uint16_t*>(dscales + b * 8);
    };
    load(0);
    for (int k0 = 0; k0 < kQF; k0 += kBK) {
        __syncthreads();
        {
            u32x4* ad = reinterpret_cast<u32x4*>(As + ar * kLdsRow + ah);
#pragma unroll
            for (int j = 0; j < 4; ++j) ad[j] = ra[j];
            dequant_block_bf16(rc, half_bits_to_float(rsc), Bs + br * kLdsRow + bb * 32);
        }
        __syncthreads();
        if (k0 + kBK < kQF) load(k0 + kBK);
        mfma_step(As, Bs, wm, cols, acc);
    }
    const int lr = lane & 15, lq = (lane >> 4) * 4;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int nj = 0; nj < 4; ++nj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wm * 64 + mi * 16 + lq + r;
                if (row < rows) a.y[(int64_t)(pos0 + row) * kQD + n0 + cols[nj] + lr] = acc[mi][nj][r];
            }
}

// ---------------------------------------------------------------- combine

// Grid (T, d/256): x[t][i] += sum_k g[t][k] Y[pos(t,k)][i], rank order.
__global__ __launch_bounds__(kPfThreads) void pf_combine_kernel(PfArgs a) {
    const int t = blockIdx.x, i = blockIdx.y * kPfThreads + threadIdx.x;
    const int K = a.K;
    // every load first, without branches (ranks past K read rank K-1 again
    // and are not summed): positions and gates, then the expert outputs and
    // x; then the sum in rank order
    int pos[kQ4MaxK];
    float g[kQ4MaxK], v[kQ4MaxK];
#pragma unroll
    for (int k = 0; k < kQ4MaxK; ++k) {
        const int64_t o = (int64_t)t * K + min(k, K - 1);
        pos[k] = a.apos[o];
        g[k] = a.gates[o];
    }
#pragma unroll
    for (int k = 0; k < kQ4MaxK; ++k) v[k] = a.y[(int64_t)pos[k] * kQD + i];
    float* xp = a.x + (int64_t)t * kQD + i;
    const float x0 = *xp;
    float y = 0.0f;
#pragma unroll
    for (int k = 0; k < kQ4MaxK; ++k)
        if (k < K) y += g[k] * v[k];
    *xp = x0 + y;
}

__global__ void cursor_add_kernel(int32_t* cursor, int32_t n) {
    if (threadIdx.x == 0) *cursor += n;
}

}  // namespace

hipError_t launch_cursor_add(int32_t* cursor, int32_t n, hipStream_t s) {
    hipLaunchKernelGGL(cursor_add_kernel, dim3(1), dim3(64), 0, s, cursor, n);
    return hipGetLastError();
}

hipError_t launch_pf_front(const PfArgs& a, hipStream_t s) {
    if (a.T <= 0 || a.K < 1 || a.K > kQ4MaxK || a.E > kMaxE) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pf_norm_kernel, dim3(a.T), dim3(kPfThreads), 0, s, a);
    hipLaunchKernelGGL(pf_router_kernel, dim3((a.T + 31) / 32, (a.E + 31) / 32), dim3(256), 0, s, a);
    hipLaunchKernelGGL(pf_topk_kernel, dim3(a.T), dim3(kPfThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pf_policy_first(const PfArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(pf_policy_first_kernel, dim3(1), dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pf_scatter(const PfArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(pf_scatter_kernel, dim3(a.E), dim3(kPfThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pf_policy(const PfArgs& a, hipStream_t s) {
    if (a.n_pf_experts > 0) hipLaunchKernelGGL(pf_policy_kernel, dim3(1), dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pf_gemms(const PfArgs& a, hipStream_t s) {
    if (a.n_fill_x < 0 || (a.n_fill_x > 0 && (!a.arena || a.slot_bytes % 16 || a.pt.R > kMaxR)))
        return hipErrorInvalidValue;
    if (a.n_items + a.n_fill_x > 0)
        hipLaunchKernelGGL(pf_gateup_kernel, dim3(a.n_items + a.n_fill_x, kQF / 64), dim3(kPfThreads), 0, s, a);
    if (a.n_items + a.n_fill_x > 0)
        hipLaunchKernelGGL(pf_down_kernel, dim3(a.n_items + a.n_fill_x, kQD / 128), dim3(kPfThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pf_combine(const PfArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(pf_combine_kernel, dim3(a.T, kQD / kPfThreads), dim3(kPfThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
