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

// (value, index) argmax across a wave64: the larger value wins, the lower
// index on equal values.  That is a total order, so the result does not depend
// on the reduction tree.  Within each 16-lane row the partner values move by
// DPP (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror); the four row results are then combined from scalar reads.
// The result is wave-uniform.
template <int CTRL>
__device__ __forceinline__ void argmax_dpp_step(float& v, int& i) {
    const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
    const int oi = __builtin_amdgcn_update_dpp(0, i, CTRL, 0xF, 0xF, false);
    if (ov > v || (ov == v && oi < i)) {
        v = ov;
        i = oi;
    }
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
    argmax_dpp_step<0xB1>(v, i);
    argmax_dpp_step<0x4E>(v, i);
    argmax_dpp_step<0x141>(v, i);
    argmax_dpp_step<0x140>(v, i);
    float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        const float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r));
        const int ri = __builtin_amdgcn_readlane(i, 16 * r);
        if (rv > bv || (rv == bv && ri < bi)) {
            bv = rv;
            bi = ri;
        }
    }
    v = bv;
    i = bi;
}

__device__ __forceinline__ float block_sum(const f32x4* uu) {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += (uu[j].x + uu[j].y) + (uu[j].z + uu[j].w);
    return s;
}

}  // namespace moe
