// Device helpers shared by the decode kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>

#include "internal.h"

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Sum over the 64 lanes of a wave with a fixed butterfly tree.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(bits & 0xffffu));
}

__device__ __forceinline__ float silu(float a) { return a / (1.0f + expf(-a)); }

__device__ __forceinline__ int tok_value(const TokRef& t) { return t.base + (t.ptr ? *t.ptr : 0); }

// Dot product of one Q4_0 block's 32 codes (16 bytes, GGUF nibble order:
// weight j in the low nibble of byte j, weight j+16 in the high nibble) with
// the block's activations u[0..31] held as 8 f32x4 (uu[j] = u[4j..4j+3]).
__device__ __forceinline__ float q4_dot(const u32x4 c, const f32x4* uu) {
    const uint32_t wd[4] = {c.x, c.y, c.z, c.w};
    float acc = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t lo = wd[m] & 0x0F0F0F0Fu;
        const uint32_t hi = (wd[m] >> 4) & 0x0F0F0F0Fu;
        const f32x4 ul = uu[m], uh = uu[4 + m];
        acc += (float)(lo & 0xffu) * ul.x;
        acc += (float)((lo >> 8) & 0xffu) * ul.y;
        acc += (float)((lo >> 16) & 0xffu) * ul.z;
        acc += (float)(lo >> 24) * ul.w;
        acc += (float)(hi & 0xffu) * uh.x;
        acc += (float)((hi >> 8) & 0xffu) * uh.y;
        acc += (float)((hi >> 16) & 0xffu) * uh.z;
        acc += (float)(hi >> 24) * uh.w;
    }
    return acc;
}

// Exact top-K of lg[0..E) under (value desc, index asc), for a 256-thread
// work-group (K <= kQ4MaxK).  Two ranking passes, all comparisons branch-free:
//  1. wave w ranks each 64-expert chunk c = w, w+4, ... within the chunk and
//     keeps the chunk's first K as candidates (padding lanes past E hold -inf
//     with an index >= E, so they rank below every real expert);
//  2. every candidate is ranked among the candidates.
// The global top K are all candidates, and a candidate's rank among the
// candidates equals its global rank whenever that is below K.  Result:
// s_e[r], s_l[r] for r < K.  LDS scratch: lg_pad[256],
// cand_v/cand_e[kMaxE/64*kQ4MaxK + 4] (16-byte aligned).  Contains barriers:
// every thread of the work-group must call it.
__device__ inline void block_topk(const float* lg, int E, int K, float* lg_pad, float* cand_v, int32_t* cand_e,
                                  int* s_e, float* s_l) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    if (t < K) {  // defined even if NaN logits leave a rank unfilled
        s_e[t] = 0;
        s_l[t] = -INFINITY;
    }
    const int n_chunks = (E + 63) >> 6;
    for (int c = w; c < n_chunks; c += 4) {
        const int e = c * 64 + lane;
        const float v = e < E ? lg[e] : -INFINITY;
        lg_pad[lane + 64 * w] = v;
        __builtin_amdgcn_wave_barrier();
        int r = 0;
#pragma unroll 4
        for (int j = 0; j < 64; j += 4) {
            const f32x4 q = *reinterpret_cast<const f32x4*>(&lg_pad[64 * w + j]);
            r += (int)(q.x > v) + (int)((q.x == v) & (j < lane));
            r += (int)(q.y > v) + (int)((q.y == v) & (j + 1 < lane));
            r += (int)(q.z > v) + (int)((q.z == v) & (j + 2 < lane));
            r += (int)(q.w > v) + (int)((q.w == v) & (j + 3 < lane));
        }
        if (r < K) {
            cand_v[c * K + r] = v;
            cand_e[c * K + r] = e;
        }
        __builtin_amdgcn_wave_barrier();
    }
    if (t < 4) {  // padding past the candidates: -inf with an index no expert has
        cand_v[n_chunks * K + t] = -INFINITY;
        cand_e[n_chunks * K + t] = 0x7fffffff;
    }
    __syncthreads();
    const int nc = n_chunks * K;
    for (int i = t; i < nc; i += 256) {
        const float v = cand_v[i];
        const int e = cand_e[i];
        int r = 0;
#pragma unroll 2
        for (int j = 0; j < nc; j += 4) {  // entries past nc are padding that ranks last
            const f32x4 q = *reinterpret_cast<const f32x4*>(&cand_v[j]);
            const int4 qe = *reinterpret_cast<const int4*>(&cand_e[j]);
            r += (int)(q.x > v) + (int)((q.x == v) & (qe.x < e));
            r += (int)(q.y > v) + (int)((q.y == v) & (qe.y < e));
            r += (int)(q.z > v) + (int)((q.z == v) & (qe.z < e));
            r += (int)(q.w > v) + (int)((q.w == v) & (qe.w < e));
        }
        if (r < K && e >= 0 && e < E) {
            s_e[r] = e;
            s_l[r] = v;
        }
    }
    __syncthreads();
}

__device__ __forceinline__ float block_sum(const f32x4* uu) {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += (uu[j].x + uu[j].y) + (uu[j].z + uu[j].w);
    return s;
}

}  // namespace moe
