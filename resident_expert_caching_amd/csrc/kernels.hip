// gfx950 kernels of the resident-expert-caching MoE decode path, fp32-weight
// variant (the small configuration); Q4_0 decode runs in q4_decode.hip.
//
// Per layer and token (decode, batch 1):
//   route   RMSNorm, router GEMV (+ Zipf bias), top-k, renormalised softmax,
//           per-expert counts, slot lookup and the LRU spare-ring policy
//           ("Luce Spark runs 35B MoE models on 16GB GPU without speed loss",
//           opening paragraph for top-k routing; paragraph "The key
//           components" for counts, pinned set and the LRU ring).
//   gateup  h_k = silu(Wg_k u) * (Wu_k u) for the K chosen experts.
//   down    x += sum_k g_k Wd_k h_k, summed in rank order.
// The expert kernels read weights from whichever slot the route kernel chose;
// the arithmetic never depends on the slot, so results are bit-identical at
// every residency (same paragraph: full residency is bit-identical to
// all-GPU execution).
//
// The GEMVs here read fp32 weights only; the Q4_0 expert GEMVs live in
// q4_decode.hip.  Every reduction has a fixed tree; there are no
// floating-point atomics.
#include <hip/hip_runtime.h>
#include <math.h>

#include "device_common.h"
#include "internal.h"
#include "policy.h"

namespace moe {

namespace {

// Wait until ring slot `ring` holds fill number `seq` (written by the host
// fill agent after its copy completed).  Bounded: after `limit` wall-clock
// ticks the error flag is raised and the work-group proceeds, so a lost fill
// can never hang the GPU.  Every wave then acquires at system scope so that no
// stale line of the slot's previous content is read.
__device__ void wait_fill(const ExpertArgs& a, int ring, uint64_t seq) {
    if (threadIdx.x == 0) {
        const uint64_t* flag = a.ready + ring;
        const uint64_t t0 = wall_clock64();
        int polls = 0;
        while (__hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM) < seq) {
            fill_poll_pause(polls);
            // once one fill has timed out, nobody waits again (no cascade of waits)
            if (wall_clock64() - t0 > a.spin_limit_ticks ||
                (__hip_atomic_load(a.error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & ERR_FILL_TIMEOUT)) {
                atomicOr(a.error, (int)ERR_FILL_TIMEOUT);
                break;
            }
        }
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
}

// ---------------------------------------------------------------- route

// Grid: E/4 work-groups of 4 waves; wave w of group g computes logit 4g+w.
// The last group to finish (device-scope counter) runs top-k, the gates and
// the placement policy in its first wave.
template <int NV>  // f32x4 per lane: d / 256
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int tok = tok_value(a.tok);
    const int d = a.d, E = a.E, K = a.K;
    const f32x4* x4 = reinterpret_cast<const f32x4*>(a.x_base + (int64_t)tok * d);

    f32x4 xv[NV];
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        xv[j] = x4[j * 64 + lane];
        ss += (xv[j].x * xv[j].x + xv[j].y * xv[j].y) + (xv[j].z * xv[j].z + xv[j].w * xv[j].w);
    }
    ss = wave_sum(ss);
    const float inv = a.norm ? 1.0f / sqrtf(ss / (float)d + a.eps) : 1.0f;
    f32x4 uv[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j)
        uv[j] = xv[j] * inv;

    const int e = blockIdx.x * 4 + w;
    if (e < E) {
        const f32x4* wr4 = reinterpret_cast<const f32x4*>(a.wr + (int64_t)e * d);
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const f32x4 wv = wr4[j * 64 + lane];
            acc += (wv.x * uv[j].x + wv.y * uv[j].y) + (wv.z * uv[j].z + wv.w * uv[j].w);
        }
        acc = wave_sum(acc);
        if (lane == 0) {
            float b = 0.0f;
            if (a.bias) {
                int row = a.bias_row ? a.bias_row[tok] : 0;
                row = row < 0 ? 0 : (row >= a.n_bias_rows ? a.n_bias_rows - 1 : row);
                b = a.bias[(int64_t)row * E + e];
            }
            a.logits[e] = acc + b;
        }
    }
    if (blockIdx.x == 0 && w == 0) {
        f32x4* u4 = reinterpret_cast<f32x4*>(a.u);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int c = j * 64 + lane;  // f32x4 index: floats 4c .. 4c+3, block c/8
            u4[c] = uv[j];
            if (a.q4) reinterpret_cast<f32x4*>(a.ut)[(c & 7) * (d / 32) + (c >> 3)] = uv[j];
        }
        const int ttok = tok_value(a.trace_tok);
        if (a.tr_x && ttok < a.tr_cap) {
            f32x4* t4 = reinterpret_cast<f32x4*>(a.tr_x + ((int64_t)ttok * a.L + a.layer) * d);
#pragma unroll
            for (int j = 0; j < NV; ++j) t4[j * 64 + lane] = xv[j];
        }
    }

    __shared__ int s_last;
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        const unsigned prev = atomicAdd(a.done, 1u);
        s_last = (prev == gridDim.x - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (w != 0) return;
    if (lane == 0) atomicExch(a.done, 0u);

    // ---- top-k over (logit desc, index asc), K rounds of wave argmax
    float lv[kMaxE / 64];
    const int per = (E + 63) / 64;
#pragma unroll
    for (int i = 0; i < kMaxE / 64; ++i) {
        const int ee = i * 64 + lane;
        lv[i] = (i < per && ee < E) ? __builtin_nontemporal_load(a.logits + ee) : -INFINITY;
    }
    uint32_t taken = 0;
    int sel_e[kMaxK];
    float sel_l[kMaxK];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
        if (k >= K) continue;
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < kMaxE / 64; ++i) {
            const int ee = i * 64 + lane;
            if (i < per && ee < E && !(taken >> i & 1u)) {
                if (lv[i] > bv || (lv[i] == bv && ee < be)) { bv = lv[i]; be = ee; }
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            const float ov = __shfl_xor(bv, m, 64);
            const int oe = __shfl_xor(be, m, 64);
            if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
        }
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        sel_e[k] = be;
        sel_l[k] = bv;
    }
    // ---- gates: softmax over the chosen logits, shifted by the first
    float gk[kMaxK];
    float z = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
        if (k >= K) continue;
        gk[k] = expf(sel_l[k] - sel_l[0]);
        z += gk[k];
    }
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
        if (k >= K) continue;
        gk[k] = gk[k] / z;
    }

    // ---- placement policy, in rank order (single wave): the shared policy
    // of policy.h, as in the Q4_0 decode and the prefill
    const PolicyTables& pt = a.pt;
    const int32_t kbase = a.layer * E;
    int my_slot = -1;
    uint64_t my_wait = 0;
    int any_cold = 0;
    int pin_slot[kMaxK];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
        if (k >= K) continue;
        pin_slot[k] = pt.slot_of[kbase + sel_e[k]];
        any_cold |= pin_slot[k] < 0;
    }
    if (lane < K) {
        int myk = 0;
#pragma unroll
        for (int k = 0; k < kMaxK; ++k)
            if (k == lane) myk = sel_e[k];
        atomicAdd(reinterpret_cast<unsigned long long*>(pt.counts + kbase + myk), 1ull);
    }
    __shared__ int32_t r_owner[kMaxR];
    __shared__ uint64_t r_stamp[kMaxR];
    __shared__ uint64_t r_seq[kMaxR];
    RingState rs{};
    if (!any_cold) {
#pragma unroll
        for (int k = 0; k < kMaxK; ++k) {
            if (k >= K) continue;
            if (lane == k) my_slot = pin_slot[k];
        }
        rs.n_pin = K;
    } else {
        ring_load(pt, r_owner, r_stamp, r_seq, rs);
#pragma unroll
        for (int k = 0; k < kMaxK; ++k) {
            if (k >= K) continue;
            int slot;
            uint64_t wseq;
            ring_access(pt, a.layer, sel_e[k], pin_slot[k], r_owner, r_stamp, r_seq, rs, slot, wseq);
            if (lane == k) {
                my_slot = slot;
                my_wait = wseq;
            }
        }
        ring_store(pt, r_owner, r_stamp, r_seq, rs);
    }
    stats_flush(pt, K, rs);
    if (lane == 0) a.sel->inv_rms = inv;
    if (lane < K) {
        int myk = 0;
        float myg = 0.0f;
#pragma unroll
        for (int k = 0; k < kMaxK; ++k)
            if (k == lane) { myk = sel_e[k]; myg = gk[k]; }
        a.sel->idx[lane] = myk;
        a.sel->slot[lane] = my_slot;
        a.sel->gate[lane] = myg;
        a.sel->wait[lane] = my_wait;
        const int ttok = tok_value(a.trace_tok);
        if (a.tr_topk && ttok < a.tr_cap) {
            const int64_t o = ((int64_t)ttok * a.L + a.layer) * K + lane;
            a.tr_topk[o] = myk;
            a.tr_gates[o] = myg;
        }
        if (a.topk_out) {
            a.topk_out[(int64_t)tok * K + lane] = myk;
            a.gates_out[(int64_t)tok * K + lane] = myg;
        }
    }
}

// ---------------------------------------------------------------- fp32 experts

// Grid (ceil(f/4), K); wave w computes row 4*bx + w of gate and up.
__global__ __launch_bounds__(256) void gateup_f32_kernel(ExpertArgs a) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int k = blockIdx.y;
    const int slot = a.sel->slot[k];
    const uint64_t wseq = a.sel->wait[k];
    if (slot < 0 || slot >= a.n_slots) {
        if (threadIdx.x == 0) atomicOr(a.error, (int)ERR_BAD_SLOT);
        return;
    }
    if (wseq && slot >= a.P) wait_fill(a, (int)(slot - a.P), wseq);
    const int n = blockIdx.x * 4 + w;
    if (n >= a.f) return;
    const int d4 = a.d / 4;
    const float* base = reinterpret_cast<const float*>(a.slots + (int64_t)slot * a.slot_bytes);
    const f32x4* gr = reinterpret_cast<const f32x4*>(base + (int64_t)n * a.d);
    const f32x4* ur = reinterpret_cast<const f32x4*>(base + (int64_t)a.f * a.d + (int64_t)n * a.d);
    const f32x4* u4 = reinterpret_cast<const f32x4*>(a.u);
    float ag = 0.0f, au = 0.0f;
    for (int c = lane; c < d4; c += 64) {
        const f32x4 uv = u4[c], gv = gr[c], vv = ur[c];
        ag += (gv.x * uv.x + gv.y * uv.y) + (gv.z * uv.z + gv.w * uv.w);
        au += (vv.x * uv.x + vv.y * uv.y) + (vv.z * uv.z + vv.w * uv.w);
    }
    ag = wave_sum(ag);
    au = wave_sum(au);
    if (lane == 0) a.h[(int64_t)k * a.f + n] = silu(ag) * au;
}

// Grid ceil(d/4); wave w computes output row 4*bx + w over all K experts.
__global__ __launch_bounds__(256) void down_f32_kernel(ExpertArgs a) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = blockIdx.x * 4 + w;
    const int tok = tok_value(a.tok);
    if (r < a.d) {
        const int f4 = a.f / 4;
        float y = 0.0f;
        for (int kk = 0; kk < a.K; ++kk) {
            int slot = a.sel->slot[kk];
            if (slot < 0 || slot >= a.n_slots) {
                if (lane == 0) atomicOr(a.error, (int)ERR_BAD_SLOT);
                slot = 0;
            }
            const float* base = reinterpret_cast<const float*>(a.slots + (int64_t)slot * a.slot_bytes);
            const f32x4* dr = reinterpret_cast<const f32x4*>(base + 2 * (int64_t)a.f * a.d + (int64_t)r * a.f);
            const f32x4* h4 = reinterpret_cast<const f32x4*>(a.h + (int64_t)kk * a.f);
            float zz = 0.0f;
            for (int c = lane; c < f4; c += 64) {
                const f32x4 dv = dr[c], hv = h4[c];
                zz += (dv.x * hv.x + dv.y * hv.y) + (dv.z * hv.z + dv.w * hv.w);
            }
            zz = wave_sum(zz);
            y += a.sel->gate[kk] * zz;
        }
        if (lane == 0) {
            const int64_t o = (int64_t)tok * a.d + r;
            a.y_base[o] = a.residual ? a.x_base[o] + y : y;
        }
    }
    if (a.advance) {
        __syncthreads();
        if (threadIdx.x == 0) {
            __threadfence();
            const unsigned prev = atomicAdd(a.done, 1u);
            if (prev == gridDim.x - 1) {
                atomicExch(a.done, 0u);
                a.cursors[0] += 1;
                a.cursors[1] += 1;
                a.stats[DS_TOKENS] += 1;
                __threadfence();
            }
        }
    }
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
    const dim3 grid((a.E + 3) / 4), block(256);
    switch (a.d / 256) {
        case 1: hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, s, a); break;
        case 16: hipLaunchKernelGGL(route_kernel<16>, grid, block, 0, s, a); break;
        case 32: hipLaunchKernelGGL(route_kernel<32>, grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gateup(const ExpertArgs& a, int wfmt, hipStream_t s) {
    if (wfmt != MOE_SPARK_W_F32) return hipErrorInvalidValue;  // Q4_0 runs in q4_decode.hip
    hipLaunchKernelGGL(gateup_f32_kernel, dim3((a.f + 3) / 4, a.K), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_down(const ExpertArgs& a, int wfmt, hipStream_t s) {
    if (wfmt != MOE_SPARK_W_F32) return hipErrorInvalidValue;  // Q4_0 runs in q4_decode.hip
    hipLaunchKernelGGL(down_f32_kernel, dim3((a.d + 3) / 4), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
