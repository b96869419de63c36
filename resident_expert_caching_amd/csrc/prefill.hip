// gfx950 batched prefill of the Q4_0 MoE stack: T tokens through one layer
// at a time.
//
//   norm     RMSNorm per token; the normalised input for the expert GEMMs
//            rounded once to fp16, 1/rms kept in fp32 for the router.
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
//            per expert group.  Each Q4_0 code enters the matrix cores as the
//            exact fp16 value q - 8; v_mfma_f32_16x16x32_f16 covers one Q4_0
//            block per instruction with fp32 accumulation, and the block's
//            fp16 scale multiplies the block's sum in fp32.  So no weight is
//            rounded; each activation is rounded once to fp16, as the batch-1
//            and batched decode kernels round theirs.
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

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kPfThreads = 256;
constexpr int kBM = 128;       // tokens per GEMM tile
constexpr int kNB = 128;       // weight rows per GEMM tile

// Matrix-core operand order of one Q4_0 block.  v_mfma_f32_16x16x32_f16
// gives lane (i, g) = (lane % 16, lane / 16) eight consecutive k positions
// 8g..8g+7 of row i of A and of column i of B.  Position 8g + j holds block
// element 4g + {0, 1, 2, 3, 16, 17, 18, 19}[j]: exactly the
// eight codes of the block's 32-bit code word g (bytes 4g..4g+3; a byte's low
// nibble is element 4g + byte, its high nibble element 16 + 4g + byte) in the
// order q4_operand unpacks them.  Activations are stored in the same order,
// so a lane's A and B values always meet at the same element.  op_pos gives
// the operand position of block element e.
__device__ __forceinline__ int op_pos(int e) { return 8 * ((e & 15) >> 2) + 4 * (e >> 4) + (e & 3); }

// Code word g of a Q4_0 block -> its eight operand values q - 8 as fp16,
// exact: a byte permute sets each code under the byte 0x64, so each fp16 is
// 1024 + q (0x6400 is fp16 1024.0, whose last mantissa bits count units), and
// subtracting 1032 is exact.
__device__ __forceinline__ u32x4 q4_operand(uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    constexpr uint32_t kHi = 0x64646464u, k01 = 0x04010400u, k23 = 0x04030402u;
    const f16x2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
    const uint32_t d[4] = {__builtin_amdgcn_perm(kHi, lo, k01), __builtin_amdgcn_perm(kHi, lo, k23),
                           __builtin_amdgcn_perm(kHi, hi, k01), __builtin_amdgcn_perm(kHi, hi, k23)};
    u32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, d[j]) - off);
    return v;
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, f16x2{(_Float16)lo, (_Float16)hi});
}

// ---------------------------------------------------------------- norm

// Grid T, 256 threads: one token per work-group.  Thread (b, g) = (tid / 4,
// tid % 4) writes operand positions 8g..8g+7 of Q4_0 block b of the normalised
// input, rounded to fp16.
__global__ __launch_bounds__(kPfThreads) void pf_norm_kernel(PfArgs a) {
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int b = tid >> 2, g = tid & 3;
    const float* xt = a.x + (int64_t)t * kQD;
    // elements 32b + 4g .. +3 and 32b + 16 + 4g .. +3 of x
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(xt + 32 * b + 4 * g);
    const f32x4 v1 = *reinterpret_cast<const f32x4*>(xt + 32 * b + 16 + 4 * g);
    float ss = (v0.x * v0.x + v0.y * v0.y) + (v0.z * v0.z + v0.w * v0.w);
    ss += (v1.x * v1.x + v1.y * v1.y) + (v1.z * v1.z + v1.w * v1.w);
    ss = wave_sum(ss);
    __shared__ float part[4];
    if (lane == 0) part[w] = ss;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    const float inv = a.norm ? 1.0f / sqrtf(tot / (float)kQD + a.eps) : 1.0f;
    if (tid == 0) a.inv[t] = inv;
    // operand order: j = 0..7 -> elements 4g + {0, 1, 2, 3, 16, 17, 18, 19}
    const u32x4 v = {pack_f16x2(v0.x * inv, v0.y * inv), pack_f16x2(v0.z * inv, v0.w * inv),
                     pack_f16x2(v1.x * inv, v1.y * inv), pack_f16x2(v1.z * inv, v1.w * inv)};
    *reinterpret_cast<u32x4*>(a.u + ((int64_t)t * (kQD / 32) + b) * 32 + 8 * g) = v;
    const int64_t tt = (int64_t)*a.tr_base + t;
    if (a.tr_x && tt < a.tr_cap) {
        f32x4* tr = reinterpret_cast<f32x4*>(a.tr_x + (tt * a.L + a.layer) * kQD + 32 * b + 4 * g);
        tr[0] = v0;
        tr[4] = v1;
    }
}

// ---------------------------------------------------------------- router

// One work-group of 8 waves per 32 tokens x 32 experts, on the fp32 matrix
// cores (v_mfma_f32_16x16x4_f32: fp32 products, fp32 accumulation).  Wave w
// covers d in [256w, 256w + 256), so that many loads are in flight per tile.
// For a 16-wide slice k0..k0+15 of d, lane (i, g) = (lane % 16, lane / 16)
// loads the four consecutive values 4g..4g+3 of token row i and of expert
// row i (the router is packed [d/16][E][16], so both are 16-byte loads);
// MFMA j then takes k = k0 + 4g + j from lane group g on both operands,
// which covers the slice.  The eight waves' partial sums meet in LDS and are
// added in wave order.
// Output: logits[t][e] = inv_rms[t] * (x[t] . Wr[e]) + bias.  With a
// prediction (a.wr2), the grid has twice the rows of expert tiles and the
// second half applies the next layer's router (a.wr2, a.bias2 -> a.logits2)
// to the same input.
constexpr int kRouterWaves = 8;
__global__ __launch_bounds__(64 * kRouterWaves) void pf_router_kernel(PfArgs a) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, i = lane & 15, g = lane >> 4;
    const int E = a.E, ny = (E + 31) / 32;
    const bool second = (int)blockIdx.y >= ny;
    const float* __restrict__ wr = second ? a.wr2 : a.wr;
    const float* __restrict__ bias_tab = second ? a.bias2 : a.bias;
    float* __restrict__ logits = second ? a.logits2 : a.logits;
    const int t0 = blockIdx.x * 32, e0 = (blockIdx.y - (second ? ny : 0)) * 32;
    const bool ta = t0 + i < a.T, tb = t0 + 16 + i < a.T;
    const bool ea = e0 + i < E, eb = e0 + 16 + i < E;
    const float* xa = a.x + (int64_t)(ta ? t0 + i : 0) * kQD + 4 * g;
    const float* xb = a.x + (int64_t)(tb ? t0 + 16 + i : 0) * kQD + 4 * g;
    const float* wa = wr + (int64_t)(ea ? e0 + i : 0) * kRW + 4 * g;
    const float* wb = wr + (int64_t)(eb ? e0 + 16 + i : 0) * kRW + 4 * g;
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 acc[2][2] = {{zero, zero}, {zero, zero}};
    constexpr int kSplit = kQD / kRouterWaves;
#pragma unroll
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
    __shared__ __align__(16) f32x4 part[kRouterWaves][4][64];  // [wave][tile m*2+n][lane]
#pragma unroll
    for (int q = 0; q < 4; ++q) part[w][q][lane] = acc[q >> 1][q & 1];
    __syncthreads();
    if (w >= 4) return;
    // wave w < 4 finishes tile q = w: lane (i, g) holds rows 4g..4g+3 of column i
    const int m = w >> 1, n = w & 1;
    f32x4 sum = part[0][w][lane];
#pragma unroll
    for (int v = 1; v < kRouterWaves; ++v) sum += part[v][w][lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int tok = t0 + 16 * m + 4 * g + r;
        const int e = e0 + 16 * n + i;
        if (tok >= a.T || e >= E) continue;
        const float inv = a.inv[tok];
        float bias = 0.0f;
        if (bias_tab) {
            int row = a.bias_row ? a.bias_row[tok] : 0;
            row = row < 0 ? 0 : (row >= a.n_bias_rows ? a.n_bias_rows - 1 : row);
            bias = bias_tab[(int64_t)row * E + e];
        }
        logits[(int64_t)tok * E + e] = sum[r] * inv + bias;
    }
}

// ---------------------------------------------------------------- top-k

// Grid T, 256 threads: top-K and gates of one token (pf_count_kernel then
// counts the choices per expert).
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
        const int64_t tt = (int64_t)*a.tr_base + t;
        if (a.tr_topk && tt < a.tr_cap) {
            const int64_t o = (tt * a.L + a.layer) * K + tid;
            a.tr_topk[o] = e;
            a.tr_gates[o] = g;
        }
    }
    if (!a.hist2) return;
    // the next layer's top-K from its router on this input: a prediction
    // that only steers the prefetch
    __syncthreads();
    for (int e = tid; e < E; e += kPfThreads) lg[e] = a.logits2[(int64_t)t * E + e];
    __syncthreads();
    block_topk(lg, E, K, kpad, cand, s_e, s_l);
    if (tid < K) a.topk2[(int64_t)t * K + tid] = s_e[tid];
}

// Grid ceil(T*K / kCountSlice), 256 threads: each work-group counts its
// slice of the top-K table per expert in LDS, then adds the non-zero counts
// to hist (zeroed before the launch) and to the layer's routing counts; with
// a prediction, the predicted table the same way into hist2.  A popular
// expert thus gets one global atomic per work-group instead of one per
// assignment (thousands on one address).
constexpr int kCountSlice = 2048;
__global__ __launch_bounds__(kPfThreads) void pf_count_kernel(PfArgs a) {
    const int tid = threadIdx.x, E = a.E;
    const int n = a.T * a.K;
    const int i0 = blockIdx.x * kCountSlice, i1 = min(n, i0 + kCountSlice);
    __shared__ int h[kMaxE], h2[kMaxE];
    for (int e = tid; e < E; e += kPfThreads) {
        h[e] = 0;
        h2[e] = 0;
    }
    __syncthreads();
    for (int i = i0 + tid; i < i1; i += kPfThreads) {
        atomicAdd(&h[a.topk[i]], 1);
        if (a.topk2) atomicAdd(&h2[a.topk2[i]], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += kPfThreads) {
        if (h[e]) {
            atomicAdd(a.hist + e, h[e]);
            atomicAdd(reinterpret_cast<unsigned long long*>(a.pt.counts + (int64_t)a.layer * E + e),
                      (unsigned long long)h[e]);
        }
        if (a.topk2 && h2[e]) atomicAdd(a.hist2 + e, h2[e]);
    }
}

// The host mirror's parts (see PfArgs::host_state).
__device__ __forceinline__ int32_t* pf_host_hist(const PfArgs& a) { return a.host_state + 2; }
__device__ __forceinline__ int32_t* pf_host_fills(const PfArgs& a) { return a.host_state + 2 + a.E; }
__device__ __forceinline__ int32_t* pf_host_prefetch(const PfArgs& a) { return a.host_state + 2 + a.E + 1 + 2 * kMaxR; }

// Publish `seq` in flag f of the host mirror after this wave's earlier
// stores to it (whole wave calls).
__device__ __forceinline__ void pf_host_flag(const PfArgs& a, int f) {
    __threadfence_system();
    if ((threadIdx.x & 63) == 0) __hip_atomic_store(a.host_state + f, a.seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ---------------------------------------------------------------- prefetch

// The prefetch rule, run by one wave after the layer's last policy run, on
// the ring tables already in LDS: the experts of layer a.layer + 1 that the
// prediction histogram a.hist2 names (count > 0), in ascending id, each
// copied into a ring slot unless pinned or already in the ring, at most
// `budget` copies.  The copies are listed in a.pfill2 (count, then
// (layer*E + expert, slot) pairs; always written, possibly empty) for the
// host to hand to the DMA engine.  Not an access: no counts, and the slots
// of the experts that the layer still computes are never chosen (the
// caller's budget leaves the least-recently-used victims among older ring
// entries).
__device__ void pf_prefetch_run(const PfArgs& a, int budget, int32_t* r_owner, uint64_t* r_stamp, uint64_t* r_seq,
                                RingState& rs, bool host) {
    const PolicyTables& pt = a.pt;
    const int lane = threadIdx.x & 63, layer = a.layer + 1;
    const int64_t lbase = (int64_t)layer * a.E;
    int nf = 0;
    for (int base = 0; base < a.E && nf < budget; base += 64) {
        const int e = base + lane;
        uint64_t m = __ballot(e < a.E && a.hist2[e] > 0 && pt.slot_of[lbase + e] < 0);  // pinned: nothing to do
        while (m && nf < budget) {
            const int ex = base + __builtin_ctzll(m);
            m &= m - 1;
            int slot;
            uint64_t wseq;
            if (ring_prefetch(pt, layer, ex, pt.slot_of[lbase + ex], r_owner, r_stamp, r_seq, rs, slot, wseq)) {
                if (lane == 0) {
                    a.pfill2[1 + 2 * nf] = (int32_t)(lbase + ex);
                    a.pfill2[2 + 2 * nf] = slot;
                    if (a.host_state && host) {
                        pf_host_prefetch(a)[1 + 2 * nf] = (int32_t)(lbase + ex);
                        pf_host_prefetch(a)[2 + 2 * nf] = slot;
                    }
                }
                ++nf;
            }
        }
    }
    if (lane == 0) {
        a.pfill2[0] = nf;
        if (a.host_state && host) pf_host_prefetch(a)[0] = nf;
    }
}

// One wave: the prefetch rule after a layer's last chunk when the layer took
// several chunks (a single-chunk layer runs it in its first policy kernel).
__global__ __launch_bounds__(64) void pf_prefetch_kernel(PfArgs a) {
    __shared__ int32_t r_owner[kMaxR];
    __shared__ uint64_t r_stamp[kMaxR];
    __shared__ uint64_t r_seq[kMaxR];
    const PolicyTables& pt = a.pt;
    RingState rs{};
    ring_load(pt, r_owner, r_stamp, r_seq, rs);
    pf_prefetch_run(a, a.pf_budget, r_owner, r_stamp, r_seq, rs, false);
    ring_store(pt, r_owner, r_stamp, r_seq, rs);
    stats_flush(pt, 0, rs);
}

// ---------------------------------------------------------------- scatter

// Grid E, 256 threads: work-group e lists the tokens that chose expert e, in
// ascending token order, at positions goff[e] .. goff[e+1]-1.
__global__ __launch_bounds__(kPfThreads) void pf_scatter_kernel(PfArgs a) {
    const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int K = a.K;
    const int32_t* goff = a.goff;
    if (a.meta_host) {
        // the plan comes from mapped host memory: each work-group copies its
        // share to the device for the GEMM launches, and reads goff there
        int32_t* dst = const_cast<int32_t*>(a.goff);
        for (int i = e * kPfThreads + tid; i < a.n_meta; i += gridDim.x * kPfThreads) dst[i] = a.meta_host[i];
        goff = a.meta_host;
    }
    const int g0 = goff[e], g1 = goff[e + 1];
    if (g1 == g0) return;
    __shared__ int wtot[4];
    int base = g0;
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
            if (a.host_state) {
                pf_host_fills(a)[1 + 2 * nf] = a.layer * a.E + e;
                pf_host_fills(a)[2 + 2 * nf] = slot;
            }
        }
    }
    if (a.arena && wseq) ++nf;
}

// A pinned expert's access leaves the ring, its clock and the fill log
// alone (ring_access only counts it), so the pinned experts of a policy run
// are recorded lane-parallel; the unpinned ones go through ring_access one
// by one in ascending id.  Lane `lane` records pinned expert e (is_pinned).
__device__ __forceinline__ void pf_record_pinned(const PfArgs& a, int e, bool is_pinned, RingState& rs) {
    if (is_pinned) {
        a.pslot[e] = a.pt.slot_of[(int64_t)a.layer * a.E + e];
        a.pwait[e] = 0ull;
    }
    rs.n_pin += __popcll(__ballot(is_pinned));
}

// One wave: the chunk's experts (ascending id) through the placement policy.
__global__ __launch_bounds__(64) void pf_policy_kernel(PfArgs a) {
    __shared__ int32_t r_owner[kMaxR];
    __shared__ uint64_t r_stamp[kMaxR];
    __shared__ uint64_t r_seq[kMaxR];
    const PolicyTables& pt = a.pt;
    const int lane = threadIdx.x & 63;
    const int64_t lbase = (int64_t)a.layer * a.E;
    RingState rs{};
    ring_load(pt, r_owner, r_stamp, r_seq, rs);
    int nf = 0;
    for (int base = 0; base < a.n_pf_experts; base += 64) {
        const int i = base + lane;
        const int e = i < a.n_pf_experts ? a.pf_experts[i] : 0;
        const bool valid = i < a.n_pf_experts;
        const bool pinned = valid && pt.slot_of[lbase + e] >= 0;
        pf_record_pinned(a, e, pinned, rs);
        uint64_t mc = __ballot(valid && !pinned);
        while (mc) {
            const int b = __builtin_ctzll(mc);
            mc &= mc - 1;
            const int ex = __shfl(e, b, 64);
            int slot;
            uint64_t wseq;
            ring_access(pt, a.layer, ex, -1, r_owner, r_stamp, r_seq, rs, slot, wseq);
            pf_record(a, ex, slot, wseq, nf);
        }
    }
    if (lane == 0) a.pfill[0] = nf;
    ring_store(pt, r_owner, r_stamp, r_seq, rs);
    stats_flush(pt, a.n_pf_experts, rs);
}

// One wave, right after the routing: the first chunk's experts through the
// placement policy, so that its fills start before the host has planned the
// layer.  The chunk is cut by the host's rule: the layer's experts with
// assignments (hist > 0), ascending, up to and excluding the one that would
// be the (R+1)-th unpinned expert.  With prediction (a.hist2), the prefetch
// rule for the next layer follows when the chunk is the whole layer.
__global__ __launch_bounds__(64) void pf_policy_first_kernel(PfArgs a) {
    __shared__ int32_t r_owner[kMaxR];
    __shared__ uint64_t r_stamp[kMaxR];
    __shared__ uint64_t r_seq[kMaxR];
    const PolicyTables& pt = a.pt;
    const int lane = threadIdx.x, E = a.E;
    const int64_t lbase = (int64_t)a.layer * E;
    if (a.host_state) {  // the histogram first: the host plans the layer while the policy runs
        for (int e = lane; e < E; e += 64) pf_host_hist(a)[e] = a.hist[e];
        pf_host_flag(a, 0);
    }
    RingState rs{};
    ring_load(pt, r_owner, r_stamp, r_seq, rs);
    int cold = 0, n = 0, nf = 0;
    bool full = false;
    for (int base = 0; base < E && !full; base += 64) {
        const int e = base + lane;
        const bool used = e < E && a.hist[e] > 0;
        const bool is_cold = used && pt.slot_of[lbase + e] < 0;
        const uint64_t mc = __ballot(is_cold);
        // the cut: this group's cold experts up to the one that would be the
        // (R+1)-th of the chunk; experts from that one on belong to the next chunk
        int cut = 64;
        if (cold + __popcll(mc) > pt.R) {
            uint64_t m = mc;
            for (int k = 0; k < pt.R - cold; ++k) m &= m - 1;
            cut = __builtin_ctzll(m);
            full = true;
        }
        const bool in = used && lane < cut;
        pf_record_pinned(a, e, in && !is_cold, rs);
        n += __popcll(__ballot(in));
        uint64_t m = __ballot(in && is_cold);
        while (m) {
            const int ex = base + __builtin_ctzll(m);
            m &= m - 1;
            int slot;
            uint64_t wseq;
            ring_access(pt, a.layer, ex, -1, r_owner, r_stamp, r_seq, rs, slot, wseq);
            pf_record(a, ex, slot, wseq, nf);
            ++cold;
        }
    }
    if (lane == 0) {
        a.pfill[0] = nf;
        if (a.host_state) pf_host_fills(a)[0] = nf;
    }
    // with prediction: when the whole layer fitted this chunk, the prefetch
    // rule follows at once, with R minus the chunk's unpinned experts as its
    // budget; otherwise it runs after the last chunk (empty list here)
    if (a.hist2) {
        if (full) {
            if (lane == 0) {
                a.pfill2[0] = 0;
                if (a.host_state) pf_host_prefetch(a)[0] = 0;
            }
        } else {
            pf_prefetch_run(a, pt.R - cold, r_owner, r_stamp, r_seq, rs, true);
        }
    }
    ring_store(pt, r_owner, r_stamp, r_seq, rs);
    stats_flush(pt, n, rs);
    if (a.host_state) pf_host_flag(a, 1);
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

// One Q4_0 block of a grouped-GEMM tile (kBM tokens x kNB weight rows),
// staged in LDS as matrix-core operands.  The tile is double-buffered over
// two of these: while the matrix cores work on block b, the next block's
// loads wait in registers, and their LDS stores go to the other stage, so
// one barrier per block suffices.  The weight codes are converted to fp16
// once, at the LDS store, so the waves that share them read operands.
//
// Operands are kept in fragment order: the 16-byte granule of row r and lane
// group g (operand positions 8g..8g+7) is granule ((r/16)*4 + g)*16 + slot,
// slot = (r%16) XOR 12(g/2), so a wave's operand read for 16 rows is one
// contiguous 1 KiB (in permuted lane order).  Two adjacent threads load the
// two halves of one row (coalesced global loads); the XOR sends the halves
// stored by one instruction to other LDS banks than the rows beside them,
// both when 8 lanes share 32 banks per cycle and when 16 lanes share 64, so
// no bank is hit twice in a store or a read.
struct PfStage {
    u32x4 a[kBM * 4];  // activation rows, fp16, operand order
    u32x4 b[kNB * 4];  // weight rows, fp16 q - 8, operand order
    float s[kNB];      // the weight rows' block scales
};

__device__ __forceinline__ int pf_granule(int r, int g) {
    return ((r >> 4) * 4 + g) * 16 + ((r & 15) ^ (12 * (g >> 1)));
}

// Thread tid's row of the tile and half of that row's operands (positions
// 16h..16h+15, lane groups 2h and 2h + 1) for the loads and the LDS stores.
__device__ __forceinline__ int pf_row(int tid) { return tid >> 1; }
__device__ __forceinline__ int pf_half(int tid) { return tid & 1; }

// Wave (wm, wn) of a 2 x 2 arrangement over the tile: rows wm*64..wm*64+63,
// the four 16-column groups cols[0..3].  Per 16 x 16 output tile and block:
// c = A B on the matrix cores (B = q - 8 exact, so c is the block's
// exact-code dot product up to fp32 rounding), then acc += s * c in fp32:
// the block scale is applied to the block's sum, never rounded into a weight.
__device__ __forceinline__ f16x8 pf_frag(const u32x4* base, int row) {
    const int lane = threadIdx.x & 63;
    return __builtin_bit_cast(f16x8, base[pf_granule(row + (lane & 15), lane >> 4)]);
}

// Software-pipelined over the four 16-row groups: group mi's MFMAs are
// issued together with group mi-1's scale FMAs and group mi+1's LDS operand
// reads, so the matrix cores need not wait for the VALU or for LDS.
__device__ __forceinline__ void pf_mfma_block(const PfStage& st, int wm, const int* cols, f32x4 (&acc)[4][4]) {
    const int lane = threadIdx.x & 63, li = lane & 15;
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    f16x8 bq[4];
    float sc[4];
#pragma unroll
    for (int nj = 0; nj < 4; ++nj) {
        bq[nj] = pf_frag(st.b, cols[nj]);
        sc[nj] = st.s[cols[nj] + li];
    }
    f16x8 f = pf_frag(st.a, wm * 64);
    f32x4 cp[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        f16x8 fn;
        if (mi + 1 < 4) fn = pf_frag(st.a, wm * 64 + (mi + 1) * 16);
        f32x4 c[4];
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) c[nj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f, bq[nj], zero, 0, 0, 0);
        if (mi > 0) {
#pragma unroll
            for (int nj = 0; nj < 4; ++nj)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[mi - 1][nj][r] = fmaf(sc[nj], cp[nj][r], acc[mi - 1][nj][r]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) cp[nj] = c[nj];
        if (mi + 1 < 4) f = fn;
    }
#pragma unroll
    for (int nj = 0; nj < 4; ++nj)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[3][nj][r] = fmaf(sc[nj], cp[nj][r], acc[3][nj][r]);
}

// Registers a thread carries from the global loads of a block to its LDS stores.
struct PfLoad {
    u32x4 a[2];
    u32x2 q;
    uint32_t sc;  // bits of a weight row's fp16 scale: converted only at the LDS store, so that
                  // nothing waits for the loads before the block's matrix-core work has been issued
};

// A thread's global sources for the blocks of a tile, as block-0 pointers
// and per-block strides.  Thread tid: activation row pf_row(tid) and weight
// row pf_row(tid) of the tile, half pf_half(tid) of each (32 B of fp16
// activations, two code words); threads 0..127 also the fp16 scale of weight
// row tid (threads 128..255 read row tid - 128's again and store nothing).
// Rows past the group read the group's first row instead: a GEMM output row
// depends only on its own activation row, and those output rows are never
// stored.
struct PfSrc {
    const u32x4* a;      // 4 u32x4 per block
    const u32x2* q;      // q_stride u32x2 per block
    const uint16_t* s;   // s_stride halves per block
    int q_stride, s_stride;
};

__device__ __forceinline__ void pf_load(PfLoad& ld, int b, const PfSrc& src) {
    const u32x4* p = src.a + 4 * b;
    ld.a[0] = p[0];
    ld.a[1] = p[1];
    ld.q = src.q[src.q_stride * b];  // cached: a 128-byte line serves the row's next blocks too
    ld.sc = src.s[src.s_stride * b];  // threads 128..255 load row tid - 128's again: no branch
}

__device__ __forceinline__ void pf_store(PfStage& st, const PfLoad& ld) {
    const int tid = threadIdx.x, r = pf_row(tid), h = pf_half(tid);
    const int o0 = pf_granule(r, 2 * h), o1 = pf_granule(r, 2 * h + 1);
    st.a[o0] = ld.a[0];
    st.a[o1] = ld.a[1];
    st.b[o0] = q4_operand(ld.q.x);
    st.b[o1] = q4_operand(ld.q.y);
    if (tid < kNB) st.s[tid] = half_bits_to_float(ld.sc);
}

// The k loop of a tile over NB Q4_0 blocks, two blocks of loads ahead: while
// the matrix cores work on block b (in one LDS stage), block b + 1's loads
// wait in registers for the other stage and block b + 2's are in flight.
// One barrier per block.  Every load is unconditional (the last blocks'
// look-ahead re-reads block NB - 1), so the compiler's wait for a block's
// loads never has to cover the loads issued after them.  A wave whose 64
// token rows all lie past the group's end (`active` false: the tile's last
// rows are padding) takes part in the loads and barriers but skips the
// matrix cores and the scale FMAs; its rows are never stored.
template <int NB>
__device__ __forceinline__ void pf_tile(PfStage (&st)[2], const PfSrc& src, int wm, bool active, const int* cols,
                                        f32x4 (&acc)[4][4]) {
    static_assert(NB >= 2 && NB % 2 == 0, "the k loop takes the blocks in pairs");
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) acc[mi][nj] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    PfLoad l0, l1;
    pf_load(l0, 0, src);
    pf_load(l1, 1, src);
    pf_store(st[0], l0);
    __syncthreads();
    for (int b = 0; b < NB; b += 2) {
        // st[0] holds block b; l1 holds block b + 1's loads
        pf_load(l0, min(b + 2, NB - 1), src);
        if (active) pf_mfma_block(st[0], wm, cols, acc);
        pf_store(st[1], l1);
        __syncthreads();
        pf_load(l1, min(b + 3, NB - 1), src);
        if (active) pf_mfma_block(st[1], wm, cols, acc);
        pf_store(st[0], l0);
        __syncthreads();
    }
}

// Work-group -> role in a grouped-GEMM launch (1-D grid).  The first
// n_fill_x * ncols work-groups pull fills (returns -1, wid = their index).
// The rest compute tiles, XCD-aware: work-groups are dealt to the 8 XCDs
// round-robin in launch order, so the (L'/8)-th tile work-group of XCD L'%8
// gets item X = (L'%8) * per + (L'/8) / ncols, weight-row tile
// Y = (L'/8) % ncols, with per = ceil(n_items / 8).  Each XCD thus takes a
// contiguous range of items, all ncols tiles of an item in a row: the tiles
// that share an item's activation rows, and the items that share an
// expert's weights (a group's items are adjacent), run under one L2.
// Returns 1 for a tile, 0 for padding.
__device__ __forceinline__ int pf_role(const PfArgs& a, int ncols, int& X, int& Y) {
    const int L = (int)blockIdx.x, nfill = a.n_fill_x * ncols;
    if (L < nfill) {
        X = L;
        return -1;
    }
    const int Lp = L - nfill, j = Lp >> 3, per = (a.n_items + 7) >> 3;
    X = (Lp & 7) * per + j / ncols;
    Y = j % ncols;
    return X < a.n_items ? 1 : 0;
}

// silu(g) * u with the hardware base-2 exponential and reciprocal (each
// within about 1 ulp; the result is rounded to fp16 right after): the IEEE
// exp and division took about a tenth of the gate/up launch's vector
// instructions.  Large |g| still gives 0 (g -> -inf) and g u (g -> +inf).
__device__ __forceinline__ float pf_swiglu(float g, float u) {
    const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
    return g * u * __builtin_amdgcn_rcpf(1.0f + e);
}

// 1-D grid (pf_role), 256 threads.  Work-group tile: kBM tokens of one
// expert group x (64 gate rows + the same 64 up rows); wave w: token rows
// (w&1)*64.., gate and up columns (w>>1)*32..; SwiGLU in the epilogue, h
// written per Q4_0 block of f as fp16 in operand order.  Weight rows come
// from the slot's gate/up region (chunk g = row/16: codes at
// ((ww*8 + i)*64 + b)*16, scales at 32768 + (ww*64 + b)*16 + 2i).
__global__ __launch_bounds__(kPfThreads, 2) void pf_gateup_kernel(PfArgs a) {
    constexpr int ncols = kQF / 64;
    int X, Y;
    const int role = pf_role(a, ncols, X, Y);
    if (role < 0) {  // the leading work-groups pull the fills
        pf_fill_pieces(a, X, a.n_fill_x * ncols, 0, kFillGUShare);
        return;
    }
    if (role == 0) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n0 = Y * 64;
    int e, pos0, rows;
    const uint8_t* S;
    if (!pf_item(a, X, e, pos0, rows, S)) return;
    __shared__ __align__(16) PfStage st[2];
    __shared__ int tok[kBM];
    if (tid < kBM) tok[tid] = tid < rows ? a.perm[pos0 + tid] : -1;
    __syncthreads();
    constexpr int nbd = kQD / 32;
    const int r2 = pf_row(tid), half = pf_half(tid);
    PfSrc src;
    src.a = reinterpret_cast<const u32x4*>(a.u + (int64_t)tok[r2 < rows ? r2 : 0] * nbd * 32) + 2 * half;
    // weight row r of the tile: gate rows n0..n0+63, then the same up rows;
    // chunk mrow/16 holds it as wave-row (ww, bi)
    {
        const int mrow = n0 + (r2 & 63);
        const int ww = (r2 >= 64 ? 2 : 0) + ((mrow >> 3) & 1), bi = mrow & 7;
        const uint8_t* ch = S + (int64_t)(mrow >> 4) * kGUChunk;
        src.q = reinterpret_cast<const u32x2*>(ch + (ww * 8 + bi) * 64 * 16) + half;
        src.q_stride = 2;
    }
    {
        const int r = tid & (kNB - 1);  // the scale's row (threads 0..127)
        const int mrow = n0 + (r & 63);
        const int ww = (r >= 64 ? 2 : 0) + ((mrow >> 3) & 1), bi = mrow & 7;
        const uint8_t* ch = S + (int64_t)(mrow >> 4) * kGUChunk;
        src.s = reinterpret_cast<const uint16_t*>(ch + 32768 + ww * 64 * 16 + bi * 2);
        src.s_stride = 8;
    }
    const int wm = w & 1, wn = w >> 1;
    const int cols[4] = {wn * 32, wn * 32 + 16, 64 + wn * 32, 64 + wn * 32 + 16};
    f32x4 acc[4][4];
    pf_tile<nbd>(st, src, wm, wm * 64 < rows, cols, acc);

    // Epilogue.  The wave's 32 h columns are one Q4_0 block fb of f: element
    // nj*16 + li of it for nj = 0, 1.  Rows are staged in LDS (the stages are
    // free after the loop's last barrier) in operand order, then written out
    // 16 bytes per lane.  A staged row takes 40 halves (80 B), so the rows
    // 4 apart that one store instruction writes fall on distinct LDS banks.
    const int li = lane & 15, lg = lane >> 4;
    constexpr int kHRow = 40;
    static_assert(2 * kBM * kHRow * sizeof(uint16_t) <= 2 * sizeof(PfStage), "h staging fits the stages");
    uint16_t* stage = reinterpret_cast<uint16_t*>(&st[0]);  // [wn][128 rows][kHRow]
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = wm * 64 + mi * 16 + 4 * lg + r;
#pragma unroll
            for (int nj = 0; nj < 2; ++nj) {
                const float g = acc[mi][nj][r], u = acc[mi][nj + 2][r];
                stage[(wn * kBM + row) * kHRow + op_pos(nj * 16 + li)] =
                    __builtin_bit_cast(uint16_t, (_Float16)pf_swiglu(g, u));
            }
        }
    __syncthreads();
    // 128 rows x 2 blocks x 64 B: thread tid copies 16 B pieces tid, tid + 256, ...
    for (int i = tid; i < kBM * 2 * 4; i += kPfThreads) {
        const int row = i >> 3, wb = (i >> 2) & 1, piece = i & 3;
        if (row < rows) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(stage + (wb * kBM + row) * kHRow + piece * 8);
            *reinterpret_cast<u32x4*>(a.h + ((int64_t)(pos0 + row) * (kQF / 32) + Y * 2 + wb) * 32 + piece * 8) = v;
        }
    }
}

// 1-D grid (pf_role), 256 threads.  Work-group tile: kBM tokens x 128
// down rows; wave w: token rows (w&1)*64.., columns (w>>1)*64...  Weight
// rows from the slot's down region: codes [r][b][16 B], scales
// [r/4][b][4] fp16.
__global__ __launch_bounds__(kPfThreads, 2) void pf_down_kernel(PfArgs a) {
    constexpr int ncols = kQD / kNB;
    int X, Y;
    const int role = pf_role(a, ncols, X, Y);
    if (role < 0) {  // the leading work-groups pull the rest of the fills
        pf_fill_pieces(a, X, a.n_fill_x * ncols, kFillGUShare, 256);
        return;
    }
    if (role == 0) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n0 = Y * kNB;
    int e, pos0, rows;
    const uint8_t* S;
    if (!pf_item(a, X, e, pos0, rows, S)) return;
    __shared__ __align__(16) PfStage st[2];
    constexpr int nbf = kQF / 32;
    const int r2 = pf_row(tid), half = pf_half(tid);
    PfSrc src;
    src.a = reinterpret_cast<const u32x4*>(a.h + (int64_t)(pos0 + (r2 < rows ? r2 : 0)) * nbf * 32) + 2 * half;
    src.q = reinterpret_cast<const u32x2*>(S + kGURegion + (int64_t)(n0 + r2) * 256) + half;
    src.q_stride = 2;
    {
        const int n = n0 + (tid & (kNB - 1));  // the scale's row (threads 0..127)
        src.s = reinterpret_cast<const uint16_t*>(S + kGURegion + kDownCodes + (int64_t)(n >> 2) * 128 + (n & 3) * 2);
        src.s_stride = 4;
    }
    const int wm = w & 1, wn = w >> 1;
    const int cols[4] = {wn * 64, wn * 64 + 16, wn * 64 + 32, wn * 64 + 48};
    f32x4 acc[4][4];
    pf_tile<nbf>(st, src, wm, wm * 64 < rows, cols, acc);
    const int li = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int nj = 0; nj < 4; ++nj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wm * 64 + mi * 16 + 4 * lg + r;
                if (row < rows) a.y[(int64_t)(pos0 + row) * kQD + n0 + cols[nj] + li] = acc[mi][nj][r];
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
    const bool predict = a.hist2 != nullptr;
    if (predict && (!a.wr2 || !a.logits2 || !a.topk2 || !a.pfill2 || a.layer + 1 >= a.L))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(pf_norm_kernel, dim3(a.T), dim3(kPfThreads), 0, s, a);
    hipLaunchKernelGGL(pf_router_kernel, dim3((a.T + 31) / 32, (predict ? 2 : 1) * ((a.E + 31) / 32)),
                       dim3(64 * kRouterWaves), 0, s, a);
    hipLaunchKernelGGL(pf_topk_kernel, dim3(a.T), dim3(kPfThreads), 0, s, a);
    hipLaunchKernelGGL(pf_count_kernel, dim3((a.T * a.K + kCountSlice - 1) / kCountSlice), dim3(kPfThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pf_prefetch(const PfArgs& a, hipStream_t s) {
    if (a.pf_budget < 1 || a.pf_budget > a.pt.R || a.pt.R > kMaxR || !a.hist2 || !a.pfill2 || a.layer + 1 >= a.L)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(pf_prefetch_kernel, dim3(1), dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pf_policy_first(const PfArgs& a, hipStream_t s) {
    if (a.hist2 && (!a.pfill2 || a.layer + 1 >= a.L)) return hipErrorInvalidValue;
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
    // 1-D grids: the fill work-groups, then the tiles with the item count
    // padded to a multiple of 8 (the XCD-aware mapping, pf_role)
    const int nx = a.n_fill_x + ((a.n_items + 7) & ~7);
    if (nx > 0) hipLaunchKernelGGL(pf_gateup_kernel, dim3(nx * (kQF / 64)), dim3(kPfThreads), 0, s, a);
    if (nx > 0) hipLaunchKernelGGL(pf_down_kernel, dim3(nx * (kQD / kNB)), dim3(kPfThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pf_combine(const PfArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(pf_combine_kernel, dim3(a.T, kQD / kPfThreads), dim3(kPfThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t prepare_pf_kernels() {
    // Querying each kernel's attributes makes the runtime resolve it now, at
    // context creation, rather than on its first launch inside a prefill.
    const void* fns[] = {reinterpret_cast<const void*>(pf_norm_kernel),
                         reinterpret_cast<const void*>(pf_router_kernel),
                         reinterpret_cast<const void*>(pf_topk_kernel),
                         reinterpret_cast<const void*>(pf_count_kernel),
                         reinterpret_cast<const void*>(pf_prefetch_kernel),
                         reinterpret_cast<const void*>(pf_scatter_kernel),
                         reinterpret_cast<const void*>(pf_policy_kernel),
                         reinterpret_cast<const void*>(pf_policy_first_kernel),
                         reinterpret_cast<const void*>(pf_gateup_kernel),
                         reinterpret_cast<const void*>(pf_down_kernel),
                         reinterpret_cast<const void*>(pf_combine_kernel),
                         reinterpret_cast<const void*>(cursor_add_kernel)};
    for (const void* f : fns) {
        hipFuncAttributes at;
        const hipError_t e = hipFuncGetAttributes(&at, f);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace moe
