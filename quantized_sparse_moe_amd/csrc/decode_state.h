// decode_state.h -- what the one-launch decode kernels (T = 1: decode.hip; T = 2..4:
// decode_small.hip) share: the workgroup shape, the layout of the decode state at the
// start of the workspace (generation, completion counters, tagged hand-off words), the
// device-scope hand-off primitives, the in-register dequantising dot product and the
// selector.
//
// Hand-offs between workgroups use device-scope (sc1) stores/loads and device-scope
// atomics, which are coherent across the XCDs without L2 write-back/invalidate.  Every
// hand-off word carries the call's tag in its upper half, so a reader knows a word is
// current without any ordering between words.
#pragma once
#include "common.h"
#include "internal.h"

namespace qs {

namespace {

constexpr int DT = 512;                     // threads per workgroup (8 waves)
constexpr int NW = DT / 64;
constexpr uint32_t SPIN_LIMIT = 1u << 22;
constexpr int NGRP = 16;                    // group counters of the completion count

// Decode state at the start of the workspace, in uint32 units.  It must be zero before
// the first call and is kept by the library between calls.
constexpr int CTL_ERR = 0;                  // MOE_WS_ERR_* bits: a bounded wait gave up
constexpr int CTL_SPIN = 32;                // 0: every wait polls at most SPIN_LIMIT times;
                                            // else at most this many (set only by a test of
                                            // the give-up path, which must not hang)
                                            // (word 33: CTL_HBLOCK_EXACT, read by the grouped GEMM)
constexpr int CTL_GEN = 64;                 // calls completed; this call's tag is gen + 1
constexpr int CNT_BASE = 128;               // + g * 64: completion group counters
constexpr int CNT_TOP = CNT_BASE + NGRP * 64;
// Hand-off words are written in several copies, 256 bytes off a multiple of the copy
// size apart, so that the many workgroups polling them spread over memory channels
// instead of queueing on a few lines.
constexpr int LOGIT_COPIES = 32;
constexpr int LOGIT_STRIDE = 2 * 256 + 64;  // per copy: E words of 64 bits, logit bits | tag << 32
constexpr int LOGIT_BASE = CNT_TOP + 64;
constexpr int H_COPIES = 8;
constexpr int H_WORDS_MAX = 24576 / 2;      // (top_k + 1) * inter <= 24576
// per copy (T = 1): (K+1)*I/2 words (fp16 h[j], h[j+1] scaled by 2^e | tag << 32), then
// one word (e | tag << 32) per slice of h that one gate/up workgroup computes
constexpr int HEXP_MAX = 2304;              // slices per copy: (K+1) * I / 16 <= 1536
constexpr int H_EXP = 2 * H_WORDS_MAX;      // u32 offset of the slice words in a copy
constexpr int H_STRIDE = 2 * (H_WORDS_MAX + HEXP_MAX) + 64;
constexpr int H_BASE = LOGIT_BASE + LOGIT_COPIES * LOGIT_STRIDE;
constexpr int TOPK_COPIES = 32;
constexpr int TOPK_STRIDE = 1088;           // per copy: 2 words of 64 bits per selected expert,
                                            // (id | tag << 32) and (weight bits | tag << 32)
constexpr int TOPK_BASE = H_BASE + H_COPIES * H_STRIDE;
constexpr int N_SELECT = 8;                 // selector workgroups of a layer call
static_assert((TOPK_BASE + TOPK_COPIES * TOPK_STRIDE) * 4 <= (int)WS_CTL_BYTES, "decode state region");


__device__ __forceinline__ void st_dev(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev64(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes (two tagged words) written through to device scope in one store: hand-off
// lines are written whole by one instruction, not merged from many small writes.  A
// store wider than 8 bytes reads its data registers after it issues, and a vector-ALU
// write to them within two wait states replaces data not yet read; the compiler pads its
// own stores for that but cannot see inside this one, so the padding is part of it.
__device__ __forceinline__ void st_dev128(void *p, u32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 4" ::"v"(p), "v"(v) : "memory");
}
// 32 bytes (four tagged words) read at device scope with two 16-byte loads, waited for
// here (the compiler does not track loads issued from inline assembly)
__device__ __forceinline__ void ld_dev256(const void *p, u32x4 &a, u32x4 &b) {
    asm volatile(
        "global_load_dwordx4 %0, %2, off sc1\n\t"
        "global_load_dwordx4 %1, %2, off offset:16 sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(a), "=&v"(b)
        : "v"(p)
        : "memory");
}
// one h group (the 64-bit word of its slice and its four tagged words), read at device
// scope, and waited for here
__device__ __forceinline__ void ld_dev_group(const uint64_t *pe, const void *pd, uint64_t &e, u32x4 &a, u32x4 &b) {
    asm volatile(
        "global_load_dwordx2 %0, %3, off sc1\n\t"
        "global_load_dwordx4 %1, %4, off sc1\n\t"
        "global_load_dwordx4 %2, %4, off offset:16 sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(e), "=&v"(a), "=&v"(b)
        : "v"(pe), "v"(pd)
        : "memory");
}
// the same for one group or two through the caches (every load in flight at once):
// workgroups of one XCD reading one copy then fetch each line from beyond the L2 once.
// A cached line may predate the producer's write; its tags show it, and such a word is
// then read again at device scope.
__device__ __forceinline__ void ld_cached_group(const uint64_t *pe, const void *pd, uint64_t &e, u32x4 &a, u32x4 &b) {
    asm volatile(
        "global_load_dwordx2 %0, %3, off\n\t"
        "global_load_dwordx4 %1, %4, off\n\t"
        "global_load_dwordx4 %2, %4, off offset:16\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(e), "=&v"(a), "=&v"(b)
        : "v"(pe), "v"(pd)
        : "memory");
}
__device__ __forceinline__ void ld_cached_group2(const uint64_t *pe0, const void *pd0, const uint64_t *pe1,
                                                 const void *pd1, uint64_t &e0, u32x4 &a0, u32x4 &b0, uint64_t &e1,
                                                 u32x4 &a1, u32x4 &b1) {
    asm volatile(
        "global_load_dwordx2 %0, %6, off\n\t"
        "global_load_dwordx4 %1, %7, off\n\t"
        "global_load_dwordx4 %2, %7, off offset:16\n\t"
        "global_load_dwordx2 %3, %8, off\n\t"
        "global_load_dwordx4 %4, %9, off\n\t"
        "global_load_dwordx4 %5, %9, off offset:16\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(e0), "=&v"(a0), "=&v"(b0), "=&v"(e1), "=&v"(a1), "=&v"(b1)
        : "v"(pe0), "v"(pd0), "v"(pe1), "v"(pd1)
        : "memory");
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev64(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// +1 at device scope, returning the old value.  Written as a wrapping increment with
// bound 2^32 - 1 (the same result as an add of 1): the compiler's wave-level rewrite of
// atomic adds reads the returned value at once, which would stall the wave for the
// atomic's full round trip where the value is only needed much later.
__device__ __forceinline__ uint32_t add_dev(uint32_t *p) {
    return __builtin_amdgcn_atomic_inc32(p, 0xffffffffu, __ATOMIC_RELAXED, "agent");
}
__device__ __forceinline__ uint32_t tag_of(uint64_t w) { return (uint32_t)(w >> 32); }

__device__ void raise_error(uint32_t *ctl) {
    __hip_atomic_fetch_or(ctl + CTL_ERR, MOE_WS_ERR_DECODE_WAIT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// the bound on the polls of one wait
__device__ __forceinline__ uint32_t wait_bound(const uint32_t *ctl) {
    const uint32_t v = ld_dev(ctl + CTL_SPIN);
    return v ? v : SPIN_LIMIT;
}

// this call's tag: the generation of the last completed call plus one, skipping 0 (the
// tag of words never written since the workspace was zeroed) when the counter wraps
__device__ __forceinline__ uint32_t call_tag(const uint32_t *ctl) {
    const uint32_t t = ld_dev(ctl + CTL_GEN) + 1u;
    return t ? t : 1u;
}

// back-off between polls of a word another workgroup has not yet written
__device__ __forceinline__ void poll_pause(uint32_t n) {
    if (n < 8) __builtin_amdgcn_s_sleep(1);
    else __builtin_amdgcn_s_sleep(4);
}

// the last workgroup of a call: counters back to zero, generation advanced
__device__ void finish_call(uint32_t *ctl, uint32_t tag) {
    const int t = threadIdx.x;
    if (t < NGRP) st_dev(ctl + CNT_BASE + t * 64, 0u);
    if (t == NGRP) st_dev(ctl + CNT_TOP, 0u);
    if (t == NGRP + 1) st_dev(ctl + CTL_GEN, tag);
}

__device__ __forceinline__ float no_nan(float v) { return (v != v) ? -__builtin_inff() : v; }


// sum_c (s q_c + b) x_c over one 16-byte chunk of codes.  4-bit: the low nibble of each
// byte (even columns) becomes 1024 + q, the high nibble (odd columns) is taken in place as
// 1024 + 16 q, both exact in fp16, so one shift serves 8 codes; with A_e, A_o the dot
// products of those magic values with x over the even and odd columns,
//   A = A_e + A_o / 16 = sum q x + 1024 X_e + 64 X_o,
// and  sum (s q + b) x = s (A - Y) + b X  with X = X_e + X_o, Y = 1024 X_e + 64 X_o, the
// pair chunk_sums forms once per chunk when x or h is staged.  8-bit: 1024 + q for all
// columns, Y = 1024 X.
template <int BITS>
__device__ __forceinline__ float2 chunk_sums(float se, float so) {
    if constexpr (BITS == 4) return make_float2(se + so, __builtin_fmaf(1024.0f, se, 64.0f * so));
    else return make_float2(se + so, 1024.0f * (se + so));
}
template <int BITS>
__device__ __forceinline__ float chunk_dot(const u32x4 &q, const uint32_t *xs, uint32_t s16, uint32_t b16, float2 XY,
                                           int sb_bf16) {
    const u32x4 *xv = (const u32x4 *)xs;
    const uint32_t magic = QS_MAGIC;
    const float s = sb_to_f32(s16, sb_bf16), b = sb_to_f32(b16, sb_bf16);
    float A;
    if constexpr (BITS == 4) {
        const uint32_t lo = 0x000F000Fu, hi = 0x00F000F0u;
        float ae = 0.0f, ao = 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t w8 = q[d] >> 8;
            const u32x4 xx = xv[d];
            ae = __builtin_amdgcn_fdot2(as_h2(and_or(q[d], lo, magic)), as_h2(xx[0]), ae, false);
            ao = __builtin_amdgcn_fdot2(as_h2(and_or(q[d], hi, magic)), as_h2(xx[1]), ao, false);
            ae = __builtin_amdgcn_fdot2(as_h2(and_or(w8, lo, magic)), as_h2(xx[2]), ae, false);
            ao = __builtin_amdgcn_fdot2(as_h2(and_or(w8, hi, magic)), as_h2(xx[3]), ao, false);
        }
        A = __builtin_fmaf(ao, 0.0625f, ae);
    } else {
        const uint32_t lo = 0x00FF00FFu;
        float acc[2] = {0.0f, 0.0f};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const u32x4 xx = xv[d >> 1];
            const int o = 2 * (d & 1);
            acc[d & 1] = __builtin_amdgcn_fdot2(as_h2(and_or(q[d], lo, magic)), as_h2(xx[o]), acc[d & 1], false);
            acc[d & 1] = __builtin_amdgcn_fdot2(as_h2(and_or(q[d] >> 8, lo, magic)), as_h2(xx[o + 1]), acc[d & 1], false);
        }
        A = acc[0] + acc[1];
    }
    return __builtin_fmaf(s, A - XY.y, b * XY.x);
}

// Selector (one wave): waits (bounded) until every logit of this call is in and takes
// the top-k: lanes j < K return (id, weight) of the j-th selected expert in ascending
// id.  One poll is in flight at a time: a read still in flight when the data is found
// would have to be waited for before its registers are reused, a full extra round trip.
// gated: logit E is the shared-expert gate's, polled with the others; *gate gets
// sigmoid of it (every lane).  WEIGHTS = false: the experts only (w = 0).
template <bool WEIGHTS = true>
__device__ TopkOut select_topk_from(uint32_t *ctl, const uint64_t *lg, uint32_t tag, int E, int K, int gated,
                                    float *gate) {
    const int lane = threadIdx.x & 63;
    const uint64_t none = (uint64_t)tag << 32;
    uint64_t w[4], wg;
    const uint32_t lim = wait_bound(ctl);
    for (uint32_t n = 0;; ++n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = lane + 64 * i < E ? ld_dev64(lg + lane + 64 * i) : none;
        wg = (gated && lane == 0) ? ld_dev64(lg + E) : none;
        bool miss = tag_of(wg) != tag;
#pragma unroll
        for (int i = 0; i < 4; ++i) miss |= tag_of(w[i]) != tag;
        if (__ballot(miss) == 0ull) break;
        if (n > lim) {
            if (lane == 0) raise_error(ctl);
            break;
        }
        poll_pause(n);
    }
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = no_nan(__uint_as_float((uint32_t)w[i]));
    TopkOut tk = wave_topk_regs<WEIGHTS>(v, E, K);
    tk.idx = min(max(tk.idx, 0), E - 1);
    *gate = sigmoid(__builtin_bit_cast(float, __builtin_amdgcn_readfirstlane((int)(uint32_t)wg)));
    return tk;
}
// lanes sharing one row: the largest power of two <= min(64, 16-byte chunks per row)
int lanes_per_row(int ncols, int bits) {
    const int chunks = ncols * bits / 128;
    int l = 64;
    while (l > chunks) l >>= 1;
    return l;
}

}  // namespace

}  // namespace qs
