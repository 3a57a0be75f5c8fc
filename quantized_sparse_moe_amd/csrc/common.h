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

// global-memory views of addresses held as integers (e.g. read from another lane), so
// that loads through them are global loads rather than flat ones
typedef __attribute__((address_space(1))) const u32x4 g_u32x4;
typedef __attribute__((address_space(1))) const uint16_t g_u16;

// a wave-uniform lane's 64-bit value, as a scalar
__device__ __forceinline__ uint64_t readlane64(uint64_t x, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

#define QS_MAGIC 0x64006400u       // two fp16 1024.0
#define QS_WAVE 64

namespace qs {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
// a quantization scale or bias: fp16 bits, or bf16 bits (the upper half of an fp32)
__device__ __forceinline__ float sb_to_f32(uint32_t bits, int bf16) {
    return bf16 ? __uint_as_float(bits << 16) : f16_to_f32((uint16_t)bits);
}
__device__ __forceinline__ float sigmoid(float z) { return 1.0f / (1.0f + __expf(-z)); }

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

// ------------------------------------------------------------------ range scaling
// fp16 operands carry power-of-two range scales wherever a row of values could leave
// fp16's range (65504 at the top; the flush above at 2^-14 at the bottom).  A scale 2^e
// and its later removal by 2^-e are exact, so a row that is scaled gives the same
// products as an unscaled row in a wider format.
//
// floor(log2 m) for m > 0 (subnormal fp32 counts as -127)
__device__ __forceinline__ int ilog2f(float m) { return (int)((__float_as_uint(m) >> 23) & 0xffu) - 127; }
__device__ __forceinline__ int clamp_exp(int e) { return e < -120 ? -120 : (e > 120 ? 120 : e); }
// 2^e for |e| <= 126
__device__ __forceinline__ float exp2i(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }

// Scale of a row whose largest magnitude is m: 0 when m is 0 or in [2^-2, 2^15), where
// fp16 holds the row with at most 2^-12 of its largest value lost to the flush; else
// the e with m 2^e in [2^14, 2^15) (clamped to +-120).  Rows of ordinary magnitude are
// left exactly as they are.
__device__ __forceinline__ int range_exp(float m) {
    if (!(m > 0.0f) || (m >= 0.25f && m < 32768.0f)) return 0;
    return clamp_exp(14 - ilog2f(m));
}
// The same for row pieces that are later joined under one scale (the column blocks of an
// h row): multiples of 8 only, so that pieces of similar magnitude share their scale and
// the join rarely has to rescale.  0 on [2^-2, 2^15); above, m 2^e lands in [2^7, 2^15);
// below, in [2^-2, 2^6).
__device__ __forceinline__ int block_exp(float m) {
    if (!(m > 0.0f) || (m >= 0.25f && m < 32768.0f)) return 0;
    const int l = ilog2f(m);
    return clamp_exp(l > 14 ? -8 * ((l - 14 + 7) >> 3) : 8 * ((-2 - l + 7) >> 3));
}

// reinterpret a dword as two fp16 (by value: never bit_cast a vector-element lvalue)
__device__ __forceinline__ f16x2 as_h2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }

__device__ __forceinline__ uint32_t pack_f16x2(_Float16 lo, _Float16 hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

// ---------------------------------------------------------------- code unpacking
// (x & m) | c in one VALU op (the masks and the magic live in registers)
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "v"(c));
    return r;
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
// Sums over aligned groups of `width` lanes (a power of two, 1..64), the same value in
// every lane of a group.  Inside a 16-lane row the butterfly runs on DPP lane
// permutations (a few cycles each, where a generic shuffle goes through the LDS unit);
// rows are combined through scalar reads of one lane per row, in row order.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_value(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float group_sum(float v, int width) {
    if (width >= 2) v += dpp<0xB1>(v);        // quad_perm [1,0,3,2]: lane ^ 1
    if (width >= 4) v += dpp<0x4E>(v);        // quad_perm [2,3,0,1]: lane ^ 2
    if (width >= 8) v += dpp<0x141>(v);       // row_half_mirror: the other quad of the 8
    if (width >= 16) v += dpp<0x140>(v);      // row_mirror: the other 8 of the row
    if (width >= 32) {
        const float r0 = lane_value(v, 0), r1 = lane_value(v, 16), r2 = lane_value(v, 32), r3 = lane_value(v, 48);
        if (width == 32) v = ((threadIdx.x & 63) < 32) ? r0 + r1 : r2 + r3;
        else v = (r0 + r1) + (r2 + r3);
    }
    return v;
}
__device__ __forceinline__ float wave_sum(float v) { return group_sum(v, 64); }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
// maximum over the wave in every lane, without leaving the vector unit: DPP within each
// 16-lane row, then the gfx950 half- and row-swaps across rows
__device__ __forceinline__ uint32_t wave_max_bcast(uint32_t v) {
    v = max(v, dpp_u32<0xB1>(v));
    v = max(v, dpp_u32<0x4E>(v));
    v = max(v, dpp_u32<0x141>(v));
    v = max(v, dpp_u32<0x140>(v));
    const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = max(h[0], h[1]);
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return max(r[0], r[1]);
}
// maximum over the wave, returned uniform (in a scalar register)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<0xB1>(v));
    v = max(v, dpp_u32<0x4E>(v));
    v = max(v, dpp_u32<0x141>(v));
    v = max(v, dpp_u32<0x140>(v));                     // every lane: its row's maximum
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// (the reciprocal instruction: within 1 ulp, where an IEEE divide costs a dozen instructions)
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// ------------------------------------------------------------------------ top-k
// One wave selects the top_k largest of n_experts (<= 256) fp32 logits read through
// `load(e)` (NaN ranks as -inf), exact ties going to the lower expert id, and
// renormalises w_j = exp(l_j - l_max) / sum_selected exp(l_i - l_max).  On return lanes
// j < top_k hold (idx, w) of the j-th selected expert in ASCENDING expert-id order.
//
// The k-th largest value is found on order-preserving integer keys by at most top_k
// rounds over per-lane sorted lists (a DPP wave maximum of the lanes' heads, then one
// ballot); ties at that threshold are taken in expert-id order; the normaliser is a
// wave sum; only the compaction into id order goes through a small LDS slot.  Every
// step is a dependent chain of one wave, so the instruction count is the latency.
struct TopkOut {
    int idx;
    float w;
};

__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (v != v) u = 0xff800000u;                       // NaN ranks as -inf
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u); // monotone in v; live keys > 0
}

// v[i] = value of expert lane + 64 i (ignored for ids >= n_experts).  WEIGHTS = false:
// the selection only (out.w is 0), for callers that need the experts and not their weights.
template <bool WEIGHTS = true>
__device__ __forceinline__ TopkOut wave_topk_regs(const float (&v)[4], int n_experts, int top_k) {
    __shared__ int tk_idx[16][16];
    __shared__ float tk_w[16][16];
    const int lane = threadIdx.x & 63, wv = (threadIdx.x >> 6) & 15;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t key[4];
    float val[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool live = lane + 64 * i < n_experts;
        val[i] = live ? v[i] : 0.0f;
        key[i] = live ? order_key(val[i]) : 0u;
    }
    // T = the top_k-th largest key, counting repeats.  Each lane sorts its four keys.
    // Fast path: top_k rounds, each popping the wave maximum of the lanes' heads; if
    // exactly top_k keys are >= the last maximum, it is T (no repeats were involved).
    uint32_t q0 = max(key[0], key[1]), q1 = min(key[0], key[1]);
    uint32_t q2 = max(key[2], key[3]), q3 = min(key[2], key[3]);
    {
        const uint32_t h0 = max(q0, q2), l0 = min(q0, q2), h1 = max(q1, q3), l1 = min(q1, q3);
        q0 = h0;
        q1 = max(l0, h1);
        q2 = min(l0, h1);
        q3 = l1;
    }
    const uint32_t s0 = q0, s1 = q1, s2 = q2, s3 = q3;
    const uint32_t top = wave_max_bcast(q0);
    uint32_t T = top;
    for (int r = 0;;) {
        const bool pop = q0 == T;
        q0 = pop ? q1 : q0;
        q1 = pop ? q2 : q1;
        q2 = pop ? q3 : q2;
        q3 = pop ? 0u : q3;
        if (++r == top_k) break;
        T = wave_max_bcast(q0);
    }
    int ge = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) ge += __popcll(__ballot(key[i] >= T));
    bool sel[4];
    int pos[4];
    if (ge == top_k) {
        int base = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sel[i] = key[i] >= T;
            const uint64_t sm = __ballot(sel[i]);
            pos[i] = base + __popcll(sm & lt);         // rank by expert id = lane + 64 i
            base += __popcll(sm);
        }
    } else {
        // repeated keys: rounds that pop every copy of the maximum and count them
        q0 = s0;
        q1 = s1;
        q2 = s2;
        q3 = s3;
        int left = top_k;
        for (int r = 0; r < top_k; ++r) {
            const uint32_t m = wave_max_u32(q0);
            const bool pop = q0 == m;
            left -= __popcll(__ballot(pop));
            if (left <= 0 || m == 0u) {
                T = m;
                break;
            }
            if (pop) {
                q0 = q1;
                q1 = q2;
                q2 = q3;
                q3 = 0u;
            }
        }
        // keys above T, then ties at T in expert-id order
        int gt = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) gt += __popcll(__ballot(key[i] > T));
        const int need = top_k - gt;
        int ties_before = 0, base = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint64_t tie = __ballot(key[i] == T);
            sel[i] = key[i] > T || (key[i] == T && ties_before + __popcll(tie & lt) < need);
            ties_before += __popcll(tie);
            const uint64_t sm = __ballot(sel[i]);
            pos[i] = base + __popcll(sm & lt);
            base += __popcll(sm);
        }
    }
    if constexpr (WEIGHTS) {
        // renormalised weights: exp(l - l_max) over the selection, l_max = the key `top`
        const float vmax = __uint_as_float((top & 0x80000000u) ? (top & 0x7fffffffu) : ~top);
        float e[4], part = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            e[i] = sel[i] ? __expf(val[i] - vmax) : 0.0f;
            part += e[i];
        }
        const float rz = 1.0f / wave_sum(part);           // (one division, not one per slot)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (sel[i]) {
                tk_idx[wv][pos[i]] = lane + 64 * i;
                tk_w[wv][pos[i]] = e[i] * rz;
            }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (sel[i]) tk_idx[wv][pos[i]] = lane + 64 * i;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    TopkOut out;
    out.idx = lane < top_k ? tk_idx[wv][lane] : 0;
    out.w = (WEIGHTS && lane < top_k) ? tk_w[wv][lane] : 0.0f;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    return out;
}

template <typename LoadFn>
__device__ __forceinline__ TopkOut wave_topk(LoadFn load, int n_experts, int top_k) {
    const int lane = threadIdx.x & 63;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (lane + 64 * i < n_experts) ? load(lane + 64 * i) : 0.0f;
    return wave_topk_regs(v, n_experts, top_k);
}

// XCD-aware remap: consecutive hardware workgroup ids go round-robin to the 8 XCDs;
// give each XCD a contiguous range of logical ids so that neighbouring tiles (which
// share weights or activations) meet in the same L2.  Requires gridDim.x % 8 == 0.
__device__ __forceinline__ int xcd_remap(int b, int grid) {
    const int per = grid >> 3;
    return (b & 7) * per + (b >> 3);
}

}  // namespace qs
