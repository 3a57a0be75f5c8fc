// common.h -- device helpers shared by the gfx950 kernels of libqsmoe.
//
// Affine codes ([LILY] "Dequantize weights during matrix multiplication": an integer
// code per weight, one scale and bias per group of 64) are turned into fp16 without
// any int->float conversion instruction: OR-ing a code q < 1024 into the mantissa of
// the fp16 constant 1024.0 (bit pattern 0x6400) gives exactly the fp16 value 1024+q.
// One 32-bit AND-OR therefore produces two fp16 operands.  The order in which the
// codes land in the packed registers is a fixed permutation of each group of 8
// consecutive columns; activations are stored with the same permutation, so every
// dot product / MFMA pairs the right activation with the right weight.
//
//   4-bit codes, one dword = columns 0..7 (column n in bits 4n..4n+3):
//       packed fp16 order [0, 4, 1, 5, 2, 6, 3, 7]
//   8-bit codes, two dwords = columns 0..7 (column n in byte n):
//       packed fp16 order [0, 2, 1, 3, 4, 6, 5, 7]
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define QS_MAGIC 0x64006400u       // two fp16 1024.0
#define QS_WAVE 64

namespace qs {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// round-to-nearest-even to bfloat16 (NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// fp32 -> fp16 with |v| < 2^-14 flushed to zero, so that every consumer of the fp16
// value (dot2, MFMA, sums) sees the same number whatever its denormal mode.
__device__ __forceinline__ _Float16 f32_to_f16_ftz(float v) {
    return (__builtin_fabsf(v) < 6.103515625e-05f) ? (_Float16)0.0f : (_Float16)v;
}

// reinterpret a dword as two fp16 (by value: never bit_cast a vector-element lvalue)
__device__ __forceinline__ f16x2 as_h2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }

__device__ __forceinline__ uint32_t pack_f16x2(_Float16 lo, _Float16 hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

// ---------------------------------------------------------------- code unpacking
// 8 four-bit codes -> 4 dwords of fp16 pairs (1024+q), order [0,4],[1,5],[2,6],[3,7]
__device__ __forceinline__ void magic_u4(uint32_t w, uint32_t o[4]) {
    o[0] = (w & 0x000F000Fu) | QS_MAGIC;
    o[1] = ((w >> 4) & 0x000F000Fu) | QS_MAGIC;
    o[2] = ((w >> 8) & 0x000F000Fu) | QS_MAGIC;
    o[3] = ((w >> 12) & 0x000F000Fu) | QS_MAGIC;
}
// 4 eight-bit codes -> 2 dwords of fp16 pairs (1024+q), order [0,2],[1,3]
__device__ __forceinline__ void magic_u8(uint32_t w, uint32_t o[2]) {
    o[0] = (w & 0x00FF00FFu) | QS_MAGIC;
    o[1] = ((w >> 8) & 0x00FF00FFu) | QS_MAGIC;
}

// permute 8 consecutive fp16 activations (as 4 dwords of natural-order pairs) into
// the packed-code order of BITS
template <int BITS>
__device__ __forceinline__ u32x4 perm8(u32x4 v) {
    u32x4 o;
    if constexpr (BITS == 4) {            // [0,4,1,5,2,6,3,7]
        o[0] = __builtin_amdgcn_perm(v[2], v[0], 0x05040100u);   // lo(v0), lo(v2)
        o[1] = __builtin_amdgcn_perm(v[2], v[0], 0x07060302u);   // hi(v0), hi(v2)
        o[2] = __builtin_amdgcn_perm(v[3], v[1], 0x05040100u);   // lo(v1), lo(v3)
        o[3] = __builtin_amdgcn_perm(v[3], v[1], 0x07060302u);   // hi(v1), hi(v3)
    } else {                              // [0,2,1,3,4,6,5,7]
        o[0] = __builtin_amdgcn_perm(v[1], v[0], 0x05040100u);   // lo(v0), lo(v1)
        o[1] = __builtin_amdgcn_perm(v[1], v[0], 0x07060302u);   // hi(v0), hi(v1)
        o[2] = __builtin_amdgcn_perm(v[3], v[2], 0x05040100u);   // lo(v2), lo(v3)
        o[3] = __builtin_amdgcn_perm(v[3], v[2], 0x07060302u);   // hi(v2), hi(v3)
    }
    return o;
}

// position, inside its 8-column group, where column (c % 8) is stored under perm8
template <int BITS>
__device__ __forceinline__ int perm_pos(int c) {
    if constexpr (BITS == 4) return (c & 4) ? (((c & 3) << 1) | 1) : ((c & 3) << 1);
    else return (c & 4) | ((c & 1) << 1) | ((c >> 1) & 1);
}

// ------------------------------------------------------------------ wave helpers
__device__ __forceinline__ float wave_sum(float v) {
    // butterfly in a fixed order: every lane ends with the same, deterministic sum
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, QS_WAVE);
    return v;
}

template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int off = WIDTH / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, QS_WAVE);
    return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// ------------------------------------------------------------------------ top-k
// One wave selects the top_k largest of n_experts (<= 256) fp32 logits read from
// `logits` (any address space), exact ties to the lower expert id, and renormalises
// w_j = exp(l_j - l_max) / sum_selected exp(l_i - l_max).  On return lanes j < top_k
// hold (idx, w) of the j-th selected expert in ASCENDING expert-id order.
struct TopkOut {
    int idx;
    float w;
};

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

template <typename LoadFn>
__device__ __forceinline__ TopkOut wave_topk(LoadFn load, int n_experts, int top_k) {
    const int lane = threadIdx.x & 63;
    float v[4];
    bool live[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        live[i] = e < n_experts;
        v[i] = live[i] ? load(e) : 0.0f;
    }
    int my_idx = 0x7fffffff;
    float my_val = 0.0f;
    for (int r = 0; r < top_k; ++r) {
        float bv = 0.0f;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            if (live[i] && (bi == 0x7fffffff || better(v[i], e, bv, bi))) { bv = v[i]; bi = e; }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off, QS_WAVE);
            const int oi = __shfl_xor(bi, off, QS_WAVE);
            if (oi != 0x7fffffff && (bi == 0x7fffffff || better(ov, oi, bv, bi))) { bv = ov; bi = oi; }
        }
        // bi is now wave-uniform: retire it from its owner lane
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (bi == lane + 64 * i) live[i] = false;
        if (lane == r) { my_idx = bi; my_val = bv; }
    }
    // renormalised weights over the selection: the first pick holds the maximum
    const float vmax = __shfl(my_val, 0, QS_WAVE);
    const float ex = (lane < top_k) ? expf(my_val - vmax) : 0.0f;
    const float z = wave_sum(ex);
    const float w = ex / z;
    // rank by expert id (ids are distinct)
    int rank = 0;
    for (int j = 0; j < top_k; ++j) {
        const int oj = __shfl(my_idx, j, QS_WAVE);
        rank += (oj < my_idx) ? 1 : 0;
    }
    // move (idx, w) of rank j to lane j
    TopkOut out;
    out.idx = 0;
    out.w = 0.0f;
    for (int j = 0; j < top_k; ++j) {
        const int rj = __shfl(rank, j, QS_WAVE);
        const int ij = __shfl(my_idx, j, QS_WAVE);
        const float wj = __shfl(w, j, QS_WAVE);
        if (lane == rj) { out.idx = ij; out.w = wj; }
    }
    return out;
}

// XCD-aware remap: consecutive hardware workgroup ids go round-robin to the 8 XCDs;
// give each XCD a contiguous range of logical ids so that neighbouring tiles (which
// share weights or activations) meet in the same L2.  Requires gridDim.x % 8 == 0.
__device__ __forceinline__ int xcd_remap(int b, int grid) {
    const int per = grid >> 3;
    return (b & 7) * per + (b >> 3);
}

}  // namespace qs
