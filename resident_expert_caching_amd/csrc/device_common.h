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

// Pause between polls of a fill's ready flag, which lives in host memory:
// every poll is a read across PCIe, the link the fill itself is using, so
// after the first 16 quick polls (~0.1 us apart) a waiter polls about once
// a microsecond.
__device__ __forceinline__ void fill_poll_pause(int& polls) {
    if (polls < 16) {
        ++polls;
        __builtin_amdgcn_s_sleep(4);
    } else {
        __builtin_amdgcn_s_sleep(32);
    }
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// One Q4_0 block's 32 activations u[0..31] (uu[j] = u[4j..4j+3]) rounded to
// fp16 and paired in the order q4_dot forms its nibble pairs: for word m of
// the codes, a[4m] = (u[4m], u[4m+2]), a[4m+1] = (u[4m+1], u[4m+3]),
// a[4m+2] = (u[16+4m], u[18+4m]), a[4m+3] = (u[17+4m], u[19+4m]).
// Returns the fp32 sum of the rounded values, taken from the packed pairs
// themselves: a second, unpacked rounding of u could be contracted with the
// product that formed u and round some element differently.
__device__ __forceinline__ float q4_pairs(const f32x4* uu, f16x2* a) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const f32x4 lo = uu[m], hi = uu[4 + m];
        a[4 * m + 0] = f16x2{(_Float16)lo.x, (_Float16)lo.z};
        a[4 * m + 1] = f16x2{(_Float16)lo.y, (_Float16)lo.w};
        a[4 * m + 2] = f16x2{(_Float16)hi.x, (_Float16)hi.z};
        a[4 * m + 3] = f16x2{(_Float16)hi.y, (_Float16)hi.w};
    }
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    float U = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) U = __builtin_amdgcn_fdot2(a[i], one, U, false);
    return U;
}

// Sum over one Q4_0 block of (1024 + q_i) * a_i, for 32 codes (16 bytes,
// GGUF nibble order: weight j in the low nibble of byte j, weight j+16 in
// the high nibble) against the fp16 pairs of q4_pairs.  The nibbles of a
// code word are masked into bytes, and a byte permute sets each code byte
// under the byte 0x64: (0x64 << 8) | q is the fp16 1024 + q exactly, so two
// codes two bytes apart form one fp16 pair, consumed by one fp16 dot product
// with fp32 accumulation.  The caller subtracts (1024 + 8) * U to obtain
// sum_i (q_i - 8) a_i.
__device__ __forceinline__ float q4_dot(const u32x4 c, const f16x2* a) {
    const uint32_t wd[4] = {c.x, c.y, c.z, c.w};
    constexpr uint32_t kHi = 0x64646464u;
    // v_perm_b32 selectors over {kHi : nibble bytes}: 0-3 pick a nibble byte, 4 a 0x64
    constexpr uint32_t kEven = 0x04020400u, kOdd = 0x04030401u;
    float acc = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t lo = wd[m] & 0x0F0F0F0Fu, hi = (wd[m] >> 4) & 0x0F0F0F0Fu;
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, __builtin_amdgcn_perm(kHi, lo, kEven)),
                                     a[4 * m + 0], acc, false);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, __builtin_amdgcn_perm(kHi, lo, kOdd)),
                                     a[4 * m + 1], acc, false);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, __builtin_amdgcn_perm(kHi, hi, kEven)),
                                     a[4 * m + 2], acc, false);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, __builtin_amdgcn_perm(kHi, hi, kOdd)),
                                     a[4 * m + 3], acc, false);
    }
    return acc;
}

constexpr float kQ4Offset = 1032.0f;  // 1024 from the fp16 encoding + the Q4_0 zero point 8

// Total-order key of (logit v, expert e) for the top-K: larger key = larger
// value, or equal value and smaller index.  High word: the float's bits made
// monotone as an unsigned integer (-0 is first folded into +0, so the two
// compare equal); low word: ~e.  Every real expert's key is above 0, the key
// of padding entries.
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
    const uint32_t b = __float_as_uint(v + 0.0f);
    const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)o << 32) | (uint32_t)~(uint32_t)e;
}

__device__ __forceinline__ float topk_key_value(uint64_t key) {
    const uint32_t o = (uint32_t)(key >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// Exact top-K under (value desc, index asc), in two ranking passes over
// unique keys (an entry's rank is the number of keys above it):
//  1. topk_rank_chunk: a wave ranks one chunk of 64 keys among themselves and
//     keeps the chunk's first K as candidates cand[c*K .. c*K+K);
//  2. topk_merge: every candidate is ranked among the candidates.
// The global top K are all candidates, and a candidate's rank among the
// candidates equals its global rank whenever that is below K.  A NaN logit
// ranks above every number.  Keys of entries past E are 0 and never chosen.
// LDS scratch: kpad[256] (64 per wave), cand[kMaxE/64*kQ4MaxK + 16]
// (16-byte aligned).

// Wave-wide: this lane's key (0 for no entry) in chunk c of wave w.
__device__ __forceinline__ void topk_rank_chunk(uint64_t key, int c, int K, uint64_t* kpad, uint64_t* cand) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    kpad[lane + 64 * w] = key;
    if (lane < K) cand[c * K + lane] = 0ull;  // a chunk may hold fewer than K entries
    __builtin_amdgcn_wave_barrier();
    int r0 = 0, r1 = 0, r2 = 0, r3 = 0;  // four counts, so compares do not wait on one another
#pragma unroll
    for (int j = 0; j < 64; j += 8) {
        const ulonglong2* q = reinterpret_cast<const ulonglong2*>(&kpad[64 * w + j]);
        const ulonglong2 q0 = q[0], q1 = q[1], q2 = q[2], q3 = q[3];
        r0 += (int)(q0.x > key) + (int)(q0.y > key);
        r1 += (int)(q1.x > key) + (int)(q1.y > key);
        r2 += (int)(q2.x > key) + (int)(q2.y > key);
        r3 += (int)(q3.x > key) + (int)(q3.y > key);
    }
    const int r = (r0 + r1) + (r2 + r3);
    if (r < K && key != 0ull) cand[c * K + r] = key;
    __builtin_amdgcn_wave_barrier();
}

// Work-group-wide (256 threads, barriers inside): rank the n_chunks*K
// candidates; result s_e[r], s_l[r] for r < K.
__device__ inline void topk_merge(int n_chunks, int K, uint64_t* cand, int* s_e, float* s_l) {
    const int t = threadIdx.x;
    if (t < K) {  // defined even when fewer than K entries exist
        s_e[t] = 0;
        s_l[t] = -INFINITY;
    }
    const int nc = n_chunks * K;
    const int part = ((nc + 15) & ~15) >> 3;  // candidates each of 8 threads compares against (even)
    if (t < 8 * part - nc) cand[nc + t] = 0ull;  // padding past the candidates ranks last
    __syncthreads();
    // 8 threads per candidate, each counting the keys above it in one eighth
    // of the candidates; the counts meet in lanes 8c..8c+7 of one wave
    const int sub = t & 7;
    for (int base = 0; base < nc; base += 32) {
        const int i = base + (t >> 3);
        const uint64_t key = i < nc ? cand[i] : 0ull;
        int r = 0;
        for (int j = sub * part; j < (sub + 1) * part; j += 2) {
            const ulonglong2 q = *reinterpret_cast<const ulonglong2*>(&cand[j]);
            r += (int)(q.x > key) + (int)(q.y > key);
        }
        r += __shfl_xor(r, 1, 64);
        r += __shfl_xor(r, 2, 64);
        r += __shfl_xor(r, 4, 64);
        if (sub == 0 && r < K && key != 0ull) {
            s_e[r] = (int)~(uint32_t)key;
            s_l[r] = topk_key_value(key);
        }
    }
    __syncthreads();
}

// Top-K of lg[0..E) held in LDS, for a 256-thread work-group: wave w ranks
// the 64-expert chunks w, w+4, ...  Every thread must call it.
__device__ inline void block_topk(const float* lg, int E, int K, uint64_t* kpad, uint64_t* cand, int* s_e,
                                  float* s_l) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n_chunks = (E + 63) >> 6;
    for (int c = w; c < n_chunks; c += 4) {
        const int e = c * 64 + lane;
        topk_rank_chunk(e < E ? topk_key(lg[e], e) : 0ull, c, K, kpad, cand);
    }
    topk_merge(n_chunks, K, cand, s_e, s_l);
}

}  // namespace moe
