// decode.hip -- batch-1 (T = 1) MoE layer: one kernel on the vector ALUs of gfx950.
//
// [LILY] "Optimize the single-row weight path": with one activation row there is no
// weight reuse; the layer is bound by how fast the active experts' quantized weights
// stream from HBM.  Rows are read with 16-byte coalesced loads, several lanes share a
// row (split-K) and reduce with cross-lane shuffles.
// [LILY] "Reduce intermediate and state traffic": the two expert input projections are
// fused with the gated activation, and the output projection with the routing weight
// and the shared-expert result.
// [LILY] "Overlap independent GPU work": phases without a data dependency run at the
// same time, and a phase waits only for the results it consumes.
//
// One launch (a dependent launch costs ~1.5 us on this part, as much as streaming
// 12 MB), five roles chosen by workgroup index:
//   R  router logits (fp32), one wave per expert
//   P  selectors: one wave each waits for all logits, takes the top-k and publishes it
//      (several selectors write disjoint sets of copies)
//   S  shared expert gate/up + SwiGLU (needs nothing)
//   G  routed expert gate/up + SwiGLU, one [gate; up] row pair per row group (waits
//      for the top-k)
//   D  down projections of the k routed + shared experts for a block of output rows,
//      weighted and combined in a fixed order; issues its weight loads as soon as the
//      top-k is known, then waits for all of h.
// Roles only wait for workgroups of lower index (dispatched first), and the grid is
// sized to be resident all at once; every wait is bounded (an error flag is raised if
// a bound is ever exceeded) so the kernel always ends.
//
// Hand-offs between workgroups use device-scope (sc1) stores/loads and device-scope
// atomics, which are coherent across the XCDs without L2 write-back/invalidate.  Every
// hand-off word carries the call's tag in its upper half, so a reader knows a word is
// current without any ordering between words; a producer gathers its words in LDS and
// writes each run with whole 16-byte stores (a line assembled from many small writes
// of different waves becomes visible far later).
// The D workgroups count themselves in, in two levels (NGRP group counters, then one top
// counter, so that no single line absorbs one atomic per workgroup), as soon as they
// hold all of h: by then every workgroup of the call has read the generation.  The last
// to arrive puts the counters back to zero and advances the generation.  Hand-off words
// are replicated so that no single line absorbs all the polling.
//
// Dequantization in registers: codes become fp16 (1024+q) by bit operations and meet
// fp16 activations in v_dot2_f32_f16 with fp32 accumulation; per 16-byte chunk of codes
// the affine map is applied once:  sum_c (s q_c + b) x_c = s A + (b - 1024 s) X  with
// A = sum_c (1024+q_c) x_c and X = sum_c x_c.
//
// Code is kept compact on purpose: a cold kernel fetches its instructions from L2, so
// long unrolled straight-line code costs microseconds here.
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
constexpr int CTL_ERR = 0;                  // set if a bounded wait ever gave up
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
constexpr int H_STRIDE = 2 * H_WORDS_MAX + 64;  // per copy: (K+1)*I/2 words, fp16 h[j], h[j+1] | tag << 32
constexpr int H_BASE = LOGIT_BASE + LOGIT_COPIES * LOGIT_STRIDE;
constexpr int TOPK_COPIES = 32;
constexpr int TOPK_STRIDE = 1088;           // per copy: 2 words of 64 bits per selected expert,
                                            // (id | tag << 32) and (weight bits | tag << 32)
constexpr int TOPK_BASE = H_BASE + H_COPIES * H_STRIDE;
constexpr int N_SELECT = 8;                 // selector workgroups of a layer call
static_assert((TOPK_BASE + TOPK_COPIES * TOPK_STRIDE) * 4 <= (int)WS_CTL_BYTES, "decode state region");

struct DecArgs {
    Layer L;
    const uint16_t *x;
    uint32_t *ctl;
    int32_t *out_idx;
    float *out_w;
    void *y;
    int y_dtype;
    int shared;
    int nR, nP, nS, nG, nD;     // workgroups per role (route only: nP = 1, nS = nG = nD = 0)
    int route_only;
    int lprg;                   // gate/up: lanes per row (row groups per wave = 64 / lprg)
    int lprd;                   // down: lanes per row (rows per wave = 64 / lprd)
    int vs;                     // down: wave groups splitting the vectors of a row block
};

__device__ __forceinline__ void st_dev(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev64(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes (two tagged words) written through to device scope in one store: hand-off
// lines are written whole by one instruction, not merged from many small writes
__device__ __forceinline__ void st_dev128(void *p, u32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
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
__device__ __forceinline__ uint32_t ld_dev(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev64(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev(uint32_t *p) {
    return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t tag_of(uint64_t w) { return (uint32_t)(w >> 32); }

__device__ void raise_error(uint32_t *ctl) {
    __hip_atomic_fetch_or(ctl + CTL_ERR, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// x (bf16) -> LDS fp16 in code order (|v| < 2^-14 flushed) + per-chunk fp32 sums of
// the even and of the odd columns
template <int BITS>
__device__ void stage_x(const uint16_t *x, int H, uint32_t *xs, float2 *xsum) {
    constexpr int CPC = 128 / BITS;
    for (int c = threadIdx.x; c < H / CPC; c += DT) {
        float se = 0.0f, so = 0.0f;
        for (int g = 0; g < CPC / 8; ++g) {
            const u32x4 v = *(const u32x4 *)(x + c * CPC + 8 * g);
            u32x4 nat;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const _Float16 lo = f32_to_f16_ftz(__uint_as_float(v[i] << 16));
                const _Float16 hi = f32_to_f16_ftz(__uint_as_float(v[i] & 0xffff0000u));
                se += (float)lo;
                so += (float)hi;
                nat[i] = pack_f16x2(lo, hi);
            }
            *(u32x4 *)(xs + (c * CPC + 8 * g) / 2) = perm8<BITS>(nat);
        }
        xsum[c] = make_float2(se, so);
    }
}

// sum_c (s q_c + b) x_c over one 16-byte chunk of codes; X = (sum of x over the even
// columns, over the odd columns).  4-bit: the low nibble of each byte (even columns)
// becomes 1024 + q, the high nibble (odd columns) is taken in place as 1024 + 16 q, both
// exact in fp16, so one shift serves 8 codes:
//   sum (s q + b) x = s A_e + (s / 16) A_o + (b - 1024 s) X_e + (b - 64 s) X_o
// with A_e, A_o the dot products of the magic values with x.  8-bit: 1024 + q for all.
template <int BITS>
__device__ __forceinline__ float chunk_dot(const u32x4 &q, const uint32_t *xs, uint32_t s16, uint32_t b16, float2 X) {
    const u32x4 *xv = (const u32x4 *)xs;
    const uint32_t magic = QS_MAGIC;
    const float s = f16_to_f32((uint16_t)s16), b = f16_to_f32((uint16_t)b16);
    if constexpr (BITS == 4) {
        const uint32_t lo = 0x000F000Fu, hi = 0x00F000F0u;
        float ae[2] = {0.0f, 0.0f}, ao[2] = {0.0f, 0.0f};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t w8 = q[d] >> 8;
            const u32x4 xx = xv[d];
            ae[d & 1] = __builtin_amdgcn_fdot2(as_h2(and_or(q[d], lo, magic)), as_h2(xx[0]), ae[d & 1], false);
            ao[d & 1] = __builtin_amdgcn_fdot2(as_h2(and_or(q[d], hi, magic)), as_h2(xx[1]), ao[d & 1], false);
            ae[d & 1] = __builtin_amdgcn_fdot2(as_h2(and_or(w8, lo, magic)), as_h2(xx[2]), ae[d & 1], false);
            ao[d & 1] = __builtin_amdgcn_fdot2(as_h2(and_or(w8, hi, magic)), as_h2(xx[3]), ao[d & 1], false);
        }
        const float Ae = ae[0] + ae[1], Ao = ao[0] + ao[1];
        return s * Ae + (s * 0.0625f) * Ao + (b - 1024.0f * s) * X.x + (b - 64.0f * s) * X.y;
    } else {
        const uint32_t lo = 0x00FF00FFu;
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const u32x4 xx = xv[d >> 1];
            const int o = 2 * (d & 1);
            acc[d] = __builtin_amdgcn_fdot2(as_h2(and_or(q[d], lo, magic)), as_h2(xx[o]), acc[d], false);
            acc[d] = __builtin_amdgcn_fdot2(as_h2(and_or(q[d] >> 8, lo, magic)), as_h2(xx[o + 1]), acc[d], false);
        }
        const float A = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        return s * A + (b - 1024.0f * s) * (X.x + X.y);
    }
}

// [gate; up] row pairs j0 and j0 + 1 of expert e in matrix stacks (mg, mu): SwiGLU
// values (in every lane of the row group; lpr lanes share a pair).  Each step loads one
// chunk of each of the 4 rows; loads are unconditional (a lane past the row end re-reads
// the last chunk and discards it) so that all of a step's loads are issued before any
// wait.  Addresses are a uniform matrix base plus a 32-bit per-lane offset.
template <int BITS>
__device__ void pairs_swiglu(const QMat &mg, const QMat &mu, int e, int j0, int H, int lpr,
                             const uint32_t *xs, const float2 *xsum, float hv[2]) {
    constexpr int CPC = 128 / BITS;
    const int lr = (threadIdx.x & 63) % lpr;
    const int nch = H / CPC, ng = H / 64;
    const uint32_t rb = (uint32_t)H * BITS / 8;
    const int64_t eg = (int64_t)e * mg.stride, eu = (int64_t)e * mu.stride;
    const uint64_t cg = (uint64_t)(mg.codes + eg * rb), cu = (uint64_t)(mu.codes + eu * rb);
    const uint64_t sg = (uint64_t)(mg.scales + eg * ng), bg = (uint64_t)(mg.biases + eg * ng);
    const uint64_t su = (uint64_t)(mu.scales + eu * ng), bu = (uint64_t)(mu.biases + eu * ng);
    const uint32_t oc0 = (uint32_t)j0 * rb, os0 = (uint32_t)j0 * ng;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = 0; k0 < nch; k0 += lpr) {
        const int c = k0 + lr;
        const bool ok = c < nch;
        const int cc = ok ? c : nch - 1;
        const uint32_t oc = oc0 + 16u * cc, os = os0 + ((cc * CPC) >> 6);
        u32x4 q[4];
        uint32_t sc[4], bi[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {               // r = 2 * (row j0 + r/2) + (0 gate | 1 up)
            const uint32_t dc = (r >> 1) ? rb : 0u, ds = (r >> 1) ? (uint32_t)ng : 0u;
            q[r] = __builtin_nontemporal_load((g_u32x4 *)(((r & 1) ? cu : cg) + oc + dc));
            sc[r] = *(g_u16 *)(((r & 1) ? su : sg) + 2u * (os + ds));
            bi[r] = *(g_u16 *)(((r & 1) ? bu : bg) + 2u * (os + ds));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = chunk_dot<BITS>(q[r], xs + cc * (CPC / 2), sc[r], bi[r], xsum[cc]);
            acc[r] += ok ? p : 0.0f;
        }
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const float g = group_sum(acc[2 * p], lpr);
        const float u = group_sum(acc[2 * p + 1], lpr);
        hv[p] = silu(g) * u;
    }
}

// Selector (one wave): waits (bounded) until every logit of this call is in and takes
// the top-k: lanes j < K return (id, weight) of the j-th selected expert in ascending
// id.  One poll is in flight at a time: a read still in flight when the data is found
// would have to be waited for before its registers are reused, a full extra round trip.
__device__ TopkOut select_topk_from(uint32_t *ctl, const uint64_t *lg, uint32_t tag, int E, int K) {
    const int lane = threadIdx.x & 63;
    const uint64_t none = (uint64_t)tag << 32;
    uint64_t w[4];
    for (uint32_t n = 0;; ++n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = lane + 64 * i < E ? ld_dev64(lg + lane + 64 * i) : none;
        bool miss = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) miss |= tag_of(w[i]) != tag;
        if (__ballot(miss) == 0ull) break;
        if (n > SPIN_LIMIT) {
            if (lane == 0) raise_error(ctl);
            break;
        }
        poll_pause(n);
    }
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = no_nan(__uint_as_float((uint32_t)w[i]));
    TopkOut tk = wave_topk_regs(v, E, K);
    tk.idx = min(max(tk.idx, 0), E - 1);
    return tk;
}
__device__ TopkOut select_topk(uint32_t *ctl, uint32_t tag, int E, int K) {
    return select_topk_from(ctl, (const uint64_t *)(ctl + LOGIT_BASE + (blockIdx.x % LOGIT_COPIES) * LOGIT_STRIDE),
                            tag, E, K);
}

// Consumer: wave 0 waits (bounded) for the published selection, one poll in flight;
// the workgroup gets (s_idx, s_w): experts in ascending id, renormalised weights.
__device__ void get_topk(uint32_t *ctl, uint32_t tag, int E, int K, int *s_idx, float *s_w) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const uint64_t *tp = (const uint64_t *)(ctl + TOPK_BASE + (blockIdx.x % TOPK_COPIES) * TOPK_STRIDE);
        const bool act = lane < 2 * K;
        const uint64_t none = (uint64_t)tag << 32;
        uint64_t w;
        for (uint32_t n = 0;; ++n) {
            w = act ? ld_dev64(tp + lane) : none;
            if (__ballot(tag_of(w) != tag) == 0ull) break;
            if (n > SPIN_LIMIT) {
                if (lane == 0) raise_error(ctl);
                break;
            }
            poll_pause(n);
        }
        if (act) {
            if (lane & 1) s_w[lane >> 1] = __uint_as_float((uint32_t)w);
            else s_idx[lane >> 1] = min(max((int)(uint32_t)w, 0), E - 1);
        }
    }
    __syncthreads();
}

template <int BITS>
__global__ __launch_bounds__(DT) __attribute__((amdgpu_waves_per_eu(4))) void k_decode(DecArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint32_t dsm[];
    __shared__ uint32_t s_flag;
    __shared__ int s_idx[16];
    __shared__ float s_w[16];
    __shared__ float s_part[NW][DT / 64 * 16];
    constexpr int CPC = 128 / BITS;
    const Layer &L = a.L;
    uint32_t *ctl = a.ctl;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = L.H, I = L.I, E = L.E, K = L.K;
    int nR = a.nR;
    const int nS = a.nS, nG = a.nG, nD = a.nD;
    const int b = blockIdx.x;

    if (b < nR) {
        // ------------------------------------------------- R: one router logit per wave
        // the workgroup's NW logits are gathered in LDS, then written to every copy in
        // 16-byte pieces (one 64-byte run per copy)
        __shared__ float s_lg[NW];
        const int e = b * NW + wave;
        const uint32_t tag = ld_dev(ctl + CTL_GEN) + 1;
        float acc = 0.0f;
        if (e < E) {
            const uint16_t *wr = L.router_w + (int64_t)e * H;
            for (int c0 = lane; c0 < H / 8; c0 += 4 * 64) {
                u32x4 xv[4], wv[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int c = c0 + 64 * k;
                    xv[k] = wv[k] = (u32x4){0u, 0u, 0u, 0u};
                    if (c < H / 8) {
                        xv[k] = *(const u32x4 *)(a.x + 8 * c);
                        wv[k] = __builtin_nontemporal_load((const u32x4 *)(wr + 8 * c));
                    }
                }
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc = __builtin_fmaf(__uint_as_float(xv[k][i] << 16), __uint_as_float(wv[k][i] << 16), acc);
                        acc = __builtin_fmaf(__uint_as_float(xv[k][i] & 0xffff0000u),
                                             __uint_as_float(wv[k][i] & 0xffff0000u), acc);
                    }
            }
            acc = wave_sum(acc) + (L.router_bias ? L.router_bias[e] : 0.0f);
        }
        if (lane == 0) s_lg[wave] = acc;
        __syncthreads();
        if (wave == 0) {
            constexpr int PIECES = NW / 2;                   // 16-byte pieces per copy
            for (int t = lane; t < LOGIT_COPIES * PIECES; t += 64) {
                const int c = t / PIECES, q = t % PIECES, e0 = b * NW + 2 * q;
                uint32_t *dst = ctl + LOGIT_BASE + c * LOGIT_STRIDE + 2 * e0;
                if (e0 + 1 < E)
                    st_dev128(dst, (u32x4){__float_as_uint(s_lg[2 * q]), tag, __float_as_uint(s_lg[2 * q + 1]), tag});
                else if (e0 < E)
                    st_dev64((uint64_t *)dst, __float_as_uint(s_lg[2 * q]) | ((uint64_t)tag << 32));
            }
        }
        return;
    }
    const uint32_t tag = ld_dev(ctl + CTL_GEN) + 1;
    if (b < nR + a.nP) {
        // ------------------------------------------- P: selectors (wave 0 works)
        if (wave != 0) return;
        const int sel = b - nR;
        const TopkOut tk = select_topk(ctl, tag, E, K);
        if (a.route_only) {
            if (lane < K) {
                if (a.out_idx) a.out_idx[lane] = tk.idx;
                if (a.out_w) a.out_w[lane] = tk.w;
            }
            if (lane == 0) st_dev(ctl + CTL_GEN, tag);       // the only reader of this call's logits
            return;
        }
        if (lane < K)
            for (int c = sel; c < TOPK_COPIES; c += a.nP)
                st_dev128(ctl + TOPK_BASE + c * TOPK_STRIDE + 4 * lane,
                          (u32x4){(uint32_t)tk.idx, tag, __float_as_uint(tk.w), tag});
        return;
    }
    nR += a.nP;                                              // the roles below follow the selectors
    if (b < nR + nS + nG) {
        // ------------------------------------------- S / G: gate/up + SwiGLU -> h
        uint32_t *xs = dsm;
        float2 *xsum = (float2 *)(dsm + H / 2);
        const int rpw = 64 / a.lprg;                         // row groups per wave
        const int pb = 2 * NW * rpw;                         // pairs per workgroup (2 per row group)
        const bool sh = b < nR + nS;
        const int g = sh ? b - nR : b - nR - nS;
        const int bpe = (I + pb - 1) / pb;                   // workgroups per expert
        const int slot = sh ? K : g / bpe;                   // h row (K = shared)
        const int j0 = (sh ? g : g % bpe) * pb + 2 * (wave * rpw + lane / a.lprg);
        stage_x<BITS>(a.x, H, xs, xsum);
        int e = 0;
        if (sh) {
            __syncthreads();
        } else {
            get_topk(ctl, tag, E, K, s_idx, s_w);            // ends with a barrier
            e = __builtin_amdgcn_readfirstlane(s_idx[slot]);
        }
        const int jj = j0 < I ? j0 : I - 2;
        float hv[2];
        pairs_swiglu<BITS>(sh ? L.s_gate : L.gate, sh ? L.s_up : L.up, e, jj, H, a.lprg, xs, xsum, hv);
        // the workgroup's pb / 2 words (one per row group, consecutive in j) are gathered
        // in LDS and written to every copy in 16-byte pieces
        __shared__ uint32_t s_hw[NW * 64];
        const int wi = wave * rpw + lane / a.lprg;           // word within the workgroup
        if (lane % a.lprg == 0) s_hw[wi] = pack_f16x2(f32_to_f16_ftz(hv[0]), f32_to_f16_ftz(hv[1]));
        __syncthreads();
        const int jb = j0 - 2 * wi;                          // first j of the workgroup
        const int nw = min(pb, I - jb) / 2;                  // valid words
        const int pieces = (nw + 1) / 2;
        for (int t = tid; t < H_COPIES * pieces; t += DT) {
            const int cp = t / pieces, q = t % pieces;
            uint32_t *dst = ctl + H_BASE + cp * H_STRIDE + 2 * (slot * (I / 2) + jb / 2 + 2 * q);
            if (2 * q + 1 < nw)
                st_dev128(dst, (u32x4){s_hw[2 * q], tag, s_hw[2 * q + 1], tag});
            else
                st_dev64((uint64_t *)dst, s_hw[2 * q] | ((uint64_t)tag << 32));
        }
        return;
    }
    {
        // ------------------------------------------ D: down + weighted combine
        const int d = b - nR - nS - nG;
        get_topk(ctl, tag, E, K, s_idx, s_w);
        if (d == 0 && tid < K) {
            if (a.out_idx) a.out_idx[tid] = s_idx[tid];
            if (a.out_w) a.out_w[tid] = s_w[tid];
        }
        const int nvec = K + (a.shared ? 1 : 0);
        const int lpr = a.lprd, rpw = 64 / lpr;
        const int nch = I / CPC, ng = I / 64;
        const int64_t rb = (int64_t)I * BITS / 8;
        const int lr = lane % lpr;
        // the waves form a.vs groups; group gv takes vectors [v_lo, v_hi) of the same rows
        const int wpg = NW / a.vs, gv = wave / wpg, wg = wave % wpg;
        const int vpg = (nvec + a.vs - 1) / a.vs;
        const int v_lo = min(gv * vpg, nvec), v_hi = min(v_lo + vpg, nvec);
        const int rloc = wg * rpw + lane / lpr;               // row within the workgroup
        const int n = d * wpg * rpw + rloc;
        const int nc = n < H ? n : H - 1;
        // h in LDS: fp16 in code order, each chunk padded to CPITCH so that the 16 lanes
        // of a row, reading 16 different chunks, meet distinct banks
        constexpr int CPITCH = CPC + 8;
        uint16_t *hs16 = (uint16_t *)dsm;                     // nvec * nch chunks
        float2 *hsum = (float2 *)(dsm + nvec * nch * CPITCH / 2);   // chunk sums (even, odd columns)
        // lane j < nvec holds row 0 of vector j's down matrix (the k routed experts in
        // ascending id, then the shared one) and its combine weight
        uint64_t pc = 0, ps = 0, pbi = 0;
        float wl = 1.0f;
        if (lane < nvec) {
            const bool routed = lane < K;
            const QMat &mm = routed ? L.down : L.s_down;
            const int64_t R0 = routed ? (int64_t)s_idx[lane] * mm.stride : 0;
            pc = (uint64_t)(mm.codes + R0 * rb);
            ps = (uint64_t)(mm.scales + R0 * ng);
            pbi = (uint64_t)(mm.biases + R0 * ng);
            if (routed) wl = s_w[lane];
        }
        float yv = 0.0f;
        uint32_t arrived = 0;
        // items (vector v, chunk lr + k*lpr), NB per step, loaded unconditionally (clamped
        // to a valid chunk and discarded) so that all of a step's loads are in flight
        constexpr int NB = 5;
        const int cpl = (nch + lpr - 1) / lpr;                 // chunks per lane per vector
        const int nit = (v_hi - v_lo) * cpl;
        const int vlast = v_hi > v_lo ? v_hi - 1 : v_lo;       // a valid vector to clamp to
        const uint32_t rowc = (uint32_t)nc * (uint32_t)rb, rows = (uint32_t)nc * ng;
        int v = v_lo, k = 0;
        for (int base = 0; base == 0 || base < nit; base += NB) {
            u32x4 q[NB];
            uint32_t sv[NB], bv[NB];
            int v2 = v, k2 = k;
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int vi = base + i < nit ? v : min(vlast, nvec - 1);
                const int c = lr + k * lpr, cc = c < nch ? c : nch - 1;
                const uint32_t gi = rows + ((cc * CPC) >> 6);
                q[i] = __builtin_nontemporal_load((g_u32x4 *)(readlane64(pc, vi) + (rowc + 16u * cc)));
                sv[i] = *(g_u16 *)(readlane64(ps, vi) + 2u * gi);
                bv[i] = *(g_u16 *)(readlane64(pbi, vi) + 2u * gi);
                if (++k == cpl) { k = 0; ++v; }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (base == 0) {
                // all of h (S and G) as it arrives.  Thread t takes groups of 8
                // consecutive values (4 words): fp16 into LDS in code order with one
                // 16-byte write, and the chunk sums by a DPP sum over the chunk's groups
                const uint64_t *hw = (const uint64_t *)(ctl + H_BASE + (d % H_COPIES) * H_STRIDE);
                const int ngrp = nvec * I / 8;
                for (int g0 = 0; g0 < ngrp; g0 += DT) {
                    const int g = g0 + tid;
                    const bool live = g < ngrp;
                    const int gg = live ? g : ngrp - 1;
                    u32x4 w0, w1;                                // words (value pair, tag) x 4
                    for (uint32_t t = 0;; ++t) {
                        ld_dev256(hw + 4 * gg, w0, w1);
                        if (w0[1] == tag && w0[3] == tag && w1[1] == tag && w1[3] == tag) break;
                        if (t > SPIN_LIMIT) {
                            raise_error(ctl);
                            break;
                        }
                        poll_pause(t);
                    }
                    const u32x4 nat = {w0[0], w0[2], w1[0], w1[2]};
                    float se = 0.0f, so = 0.0f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const f16x2 hh = as_h2(nat[j]);
                        se += (float)hh[0];
                        so += (float)hh[1];
                    }
                    if (live) *(u32x4 *)(hs16 + (g / (CPC / 8)) * CPITCH + 8 * (g % (CPC / 8))) = perm8<BITS>(nat);
                    se = group_sum(se, CPC / 8);                 // groups of a chunk are adjacent lanes
                    so = group_sum(so, CPC / 8);
                    if (live && (g % (CPC / 8)) == 0) hsum[g / (CPC / 8)] = make_float2(se, so);
                }
                __syncthreads();
                // this workgroup has all it reads of the call's state: count it in now
                // (the reply is needed only at the end)
                if (tid == 0) arrived = add_dev(ctl + CNT_BASE + (d % NGRP) * 64);
            }
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const bool live = base + i < nit;
                const int vi = live ? v2 : min(vlast, nvec - 1);
                const int c = lr + k2 * lpr, cc = c < nch ? c : nch - 1;
                const float p = chunk_dot<BITS>(q[i], (const uint32_t *)(hs16 + (vi * nch + cc) * CPITCH), sv[i], bv[i],
                                                hsum[vi * nch + cc]);
                const float wv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), vi));
                yv += (live && c < nch) ? wv * p : 0.0f;       // experts in ascending id, shared last
                if (++k2 == cpl) { k2 = 0; ++v2; }
                __builtin_amdgcn_sched_barrier(0);             // one item at a time: bounded registers
            }
        }
        yv = group_sum(yv, lpr);
        // groups' partial sums combined in group order
        if (lr == 0) s_part[gv][rloc] = yv;
        __syncthreads();
        if (gv == 0 && lr == 0 && n < H) {
            float y = s_part[0][rloc];
            for (int j = 1; j < a.vs; ++j) y += s_part[j][rloc];
            if (a.y_dtype == QSMOE_F32) ((float *)a.y)[n] = y;
            else ((uint16_t *)a.y)[n] = f32_to_bf16(y);
        }
        // the last of the D workgroups to have arrived (every other workgroup of the call
        // has read the generation before any D workgroup could arrive) resets the state
        if (tid == 0) {
            const int g = d % NGRP;
            const int gsize = nD / NGRP + (g < nD % NGRP ? 1 : 0);
            const int ngroups = nD < NGRP ? nD : NGRP;
            uint32_t last = 0;
            if (arrived == (uint32_t)(gsize - 1)) last = add_dev(ctl + CNT_TOP) == (uint32_t)(ngroups - 1);
            s_flag = last;
        }
        __syncthreads();
        if (s_flag) finish_call(ctl, tag);
    }
}

int n_compute_units() {
    static int n = 0;
    if (n == 0) {
        int dev = 0, cu = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cu > 0)
            n = cu;
        else
            n = 256;
    }
    return n;
}

// ------------------------------------------------------------------ small batches
// [LILY] "Optimize the single-row weight path" at T = 2 .. SM_TMAX tokens (batched or
// verification decode): the T = 1 structure with every role covering all T tokens.  The
// routed experts are the union U of the tokens' selections: each touched expert's
// weights are read once (G: gate/up rows for the tokens that chose it; D: down rows for
// all of them).  The hand-off regions of the T = 1 path are reused with other strides
// (every word carries the call's tag, so the two paths cannot mistake each other's words).
constexpr int SM_TMAX = 4;
constexpr int SM_LCOPIES = 8;
constexpr int SM_TE = 256;                                  // logit words per token and copy
constexpr int SM_LSTRIDE = 2 * SM_TMAX * SM_TE + 64;        // u32 per logits copy
static_assert(SM_LCOPIES * SM_LSTRIDE <= LOGIT_COPIES * LOGIT_STRIDE, "small-T logits region");
constexpr int SM_HCOPIES = 2;
constexpr int SM_HSTRIDE = H_COPIES * H_STRIDE / SM_HCOPIES;   // u32 per h copy
constexpr int SM_HWORDS = SM_HSTRIDE / 2 - 32;                 // h words per copy
constexpr size_t SMALL_LDS_MAX = 76 * 1024;                    // dynamic LDS of a small-batch call
static_assert(2 * SM_TMAX * 16 <= TOPK_STRIDE / 2, "small-T selection region");

struct SmallArgs {
    Layer L;
    const uint16_t *x;          // [T][H]
    uint32_t *ctl;
    int32_t *out_idx;           // [T][K] or null
    float *out_w;
    void *y;                    // [T][H]
    int y_dtype;
    int T, shared;
    int nR, nP, nS, nG, nD;     // route only: nP = 1, nS = nG = nD = 0
    int route_only;
    int lprg, lprd;
};

// wave 0 waits for the published selection of all tokens (entry l = t K + j: id word,
// weight word); the workgroup then has s_si / s_sw, the union U in ascending id (s_ul,
// s_nu) and, per union slot and token, the token's position of that expert (s_jt, -1 if
// the token did not choose it)
struct SmallSel {
    int si[SM_TMAX * 16];
    float sw[SM_TMAX * 16];
    uint32_t ub[8];
    int ul[SM_TMAX * 16];
    int jt[SM_TMAX * 16][SM_TMAX];
    int nu;
};
__device__ void small_get_sel(uint32_t *ctl, uint32_t tag, int E, int K, int T, SmallSel &S) {
    const int tid = threadIdx.x, n = T * K;
    if (tid < 8) S.ub[tid] = 0u;
    if (tid < SM_TMAX * 16 * SM_TMAX) (&S.jt[0][0])[tid] = -1;
    if (tid < 64) {
        const int lane = tid;
        const uint64_t *tp = (const uint64_t *)(ctl + TOPK_BASE + (blockIdx.x % TOPK_COPIES) * TOPK_STRIDE);
        const bool act = lane < n;
        const uint64_t none = (uint64_t)tag << 32;
        uint64_t w0, w1;
        for (uint32_t it = 0;; ++it) {
            w0 = act ? ld_dev64(tp + 2 * lane) : none;
            w1 = act ? ld_dev64(tp + 2 * lane + 1) : none;
            if (__ballot(tag_of(w0) != tag || tag_of(w1) != tag) == 0ull) break;
            if (it > SPIN_LIMIT) {
                if (lane == 0) raise_error(ctl);
                break;
            }
            poll_pause(it);
        }
        if (act) {
            S.si[lane] = min(max((int)(uint32_t)w0, 0), E - 1);
            S.sw[lane] = __uint_as_float((uint32_t)w1);
        }
    }
    __syncthreads();
    if (tid < n) atomicOr(&S.ub[S.si[tid] >> 5], 1u << (S.si[tid] & 31));
    __syncthreads();
    auto rank = [&](int e) {                                 // union slot of expert e
        int r = __popc(S.ub[e >> 5] & ((1u << (e & 31)) - 1u));
        for (int w = 0; w < (e >> 5); ++w) r += __popc(S.ub[w]);
        return r;
    };
    if (tid < 256 && ((S.ub[tid >> 5] >> (tid & 31)) & 1u)) S.ul[rank(tid)] = tid;
    if (tid < n) S.jt[rank(S.si[tid])][tid / K] = tid % K;
    if (tid == 0) {
        int c = 0;
        for (int w = 0; w < 8; ++w) c += __popc(S.ub[w]);
        S.nu = c;
    }
    __syncthreads();
}

// u32 per staged x chunk of the small-batch path: the chunk, then its even / odd column
// sums in a 16-byte pad, so that the 16-byte LDS reads of consecutive lanes (consecutive
// chunks) fall in distinct banks
template <int BITS>
constexpr int small_xpitch() { return 64 / BITS + 4; }

// x of T tokens (bf16, [T][H]) -> LDS fp16 in code order (chunk c of token t at
// xs + (t nch + c) * pitch, its column sums right after it), one (token, chunk) per thread
template <int BITS>
__device__ void stage_x_tokens(const uint16_t *x, int T, int H, uint32_t *xs) {
    constexpr int CPC = 128 / BITS, XP = small_xpitch<BITS>();
    const int nch = H / CPC;
    for (int i = threadIdx.x; i < T * nch; i += DT) {
        const int t = i / nch, c = i % nch;
        const uint16_t *xc = x + (int64_t)t * H + c * CPC;
        uint32_t *xd = xs + i * XP;
        float se = 0.0f, so = 0.0f;
        for (int g = 0; g < CPC / 8; ++g) {
            const u32x4 v = *(const u32x4 *)(xc + 8 * g);
            u32x4 nat;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const _Float16 lo = f32_to_f16_ftz(__uint_as_float(v[k] << 16));
                const _Float16 hi = f32_to_f16_ftz(__uint_as_float(v[k] & 0xffff0000u));
                se += (float)lo;
                so += (float)hi;
                nat[k] = pack_f16x2(lo, hi);
            }
            *(u32x4 *)(xd + 4 * g) = perm8<BITS>(nat);
        }
        *(float2 *)(xd + CPC / 2) = make_float2(se, so);
    }
}

// one chunk step of gate/up row pairs j0, j0 + 1 of expert e: per lane, the 16-byte
// code chunk and the scale and bias of each of the 4 rows (gate j0, up j0, gate j0+1,
// up j0+1); loaded ahead of their use so that several items' loads overlap
struct PairW {
    u32x4 q[4];
    uint32_t sc[4], bi[4];
};
template <int BITS>
__device__ __forceinline__ void load_pairs(const QMat &mg, const QMat &mu, int e, int j0, int H, int lpr, int k0,
                                           PairW &w) {
    constexpr int CPC = 128 / BITS;
    const int lr = (threadIdx.x & 63) % lpr;
    const int nch = H / CPC, ng = H / 64;
    const uint32_t rb = (uint32_t)H * BITS / 8;
    const int64_t eg = (int64_t)e * mg.stride, eu = (int64_t)e * mu.stride;
    const uint64_t cg = (uint64_t)(mg.codes + eg * rb), cu = (uint64_t)(mu.codes + eu * rb);
    const uint64_t sg = (uint64_t)(mg.scales + eg * ng), bg = (uint64_t)(mg.biases + eg * ng);
    const uint64_t su = (uint64_t)(mu.scales + eu * ng), bu = (uint64_t)(mu.biases + eu * ng);
    const int c = k0 + lr, cc = c < nch ? c : nch - 1;
    const uint32_t oc = (uint32_t)j0 * rb + 16u * cc, os = (uint32_t)j0 * ng + ((cc * CPC) >> 6);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t dc = (r >> 1) ? rb : 0u, ds = (r >> 1) ? (uint32_t)ng : 0u;
        w.q[r] = __builtin_nontemporal_load((g_u32x4 *)(((r & 1) ? cu : cg) + oc + dc));
        w.sc[r] = *(g_u16 *)(((r & 1) ? su : sg) + 2u * (os + ds));
        w.bi[r] = *(g_u16 *)(((r & 1) ? bu : bg) + 2u * (os + ds));
    }
}

// the same loads as load_pairs, direct to LDS (no registers held while they are in
// flight): row r's chunk of lane l lands at wb + 1024 r + 16 l, its scale and bias
// (zero-extended to a dword) at wb + 4096 + 256 r + 4 l and wb + 5120 + 256 r + 4 l
constexpr int PAIR_DMA_BYTES = 6144;                        // per wave
typedef __attribute__((address_space(3))) void lds_void;
template <int BITS>
__device__ __forceinline__ void load_pairs_dma(const QMat &mg, const QMat &mu, int e, int j0, int H, int lpr,
                                               uint8_t *wb) {
    constexpr int CPC = 128 / BITS;
    const int lr = (threadIdx.x & 63) % lpr;
    const int nch = H / CPC, ng = H / 64;
    const uint32_t rb = (uint32_t)H * BITS / 8;
    const int64_t eg = (int64_t)e * mg.stride, eu = (int64_t)e * mu.stride;
    const uint64_t cg = (uint64_t)(mg.codes + eg * rb), cu = (uint64_t)(mu.codes + eu * rb);
    const uint64_t sg = (uint64_t)(mg.scales + eg * ng), bg = (uint64_t)(mg.biases + eg * ng);
    const uint64_t su = (uint64_t)(mu.scales + eu * ng), bu = (uint64_t)(mu.biases + eu * ng);
    const int cc = lr < nch ? lr : nch - 1;
    const uint32_t oc = (uint32_t)j0 * rb + 16u * cc, os = (uint32_t)j0 * ng + ((cc * CPC) >> 6);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t dc = (r >> 1) ? rb : 0u, ds = (r >> 1) ? (uint32_t)ng : 0u;
        __builtin_amdgcn_global_load_lds((const void *)(((r & 1) ? cu : cg) + oc + dc), (lds_void *)(wb + 1024 * r),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void *)(((r & 1) ? su : sg) + 2u * (os + ds)),
                                         (lds_void *)(wb + 4096 + 256 * r), 2, 0, 0);
        __builtin_amdgcn_global_load_lds((const void *)(((r & 1) ? bu : bg) + 2u * (os + ds)),
                                         (lds_void *)(wb + 5120 + 256 * r), 2, 0, 0);
    }
}
__device__ __forceinline__ void read_pairs(const uint8_t *wb, PairW &w) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        w.q[r] = *(const u32x4 *)(wb + 1024 * r + 16 * lane);
        w.sc[r] = *(const uint32_t *)(wb + 4096 + 256 * r + 4 * lane);
        w.bi[r] = *(const uint32_t *)(wb + 5120 + 256 * r + 4 * lane);
    }
}

// Sums of 16 values over the 64 lanes of a wave in one transposing butterfly: each step
// halves the values a lane holds, a lane keeping one half and taking its partner's copy
// of that half (gfx950 half- and row-swaps across rows, DPP mirrors inside a row), so the
// wave spends 35 instructions where 16 separate reductions would spend ~180.  On return
// every lane holds the sum of value (lane >> 2).
__device__ __forceinline__ float wave_sum16(float (&v)[SM_TMAX * 4]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 8; ++i) {                            // lanes ^ 32: value i or i + 8
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 8]), false, false);
        v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {                            // lanes ^ 16: value i or i + 4
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 4]), false, false);
        v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    const bool b3 = lane & 8, b2 = lane & 4;
#pragma unroll
    for (int i = 0; i < 2; ++i) {                            // row mirror (bit 3 differs)
        const float keep = b3 ? v[i + 2] : v[i], send = b3 ? v[i] : v[i + 2];
        v[i] = keep + dpp<0x140>(send);
    }
    {                                                        // half-row mirror (bit 2 differs)
        const float keep = b2 ? v[1] : v[0], send = b2 ? v[0] : v[1];
        v[0] = keep + dpp<0x141>(send);
    }
    v[0] += dpp<0xB1>(v[0]);                                 // lanes ^ 1, lanes ^ 2
    v[0] += dpp<0x4E>(v[0]);
    return v[0];
}

// gate/up row pairs j0, j0 + 1 of expert e for the tokens in `tmask` (x chunks and chunk
// sums as stage_x_tokens leaves them): the SwiGLU words (fp16 h[j0], h[j0 + 1]) of token t
// go to hq[t * wpi + wi].  The codes of a gate/up row pair are unpacked once and meet every
// token's activations; when one row spans the wave (lpr = 64) the 16 partial sums of the
// lane are reduced together.
template <int BITS>
__device__ void pairs_swiglu_tokens(const QMat &mg, const QMat &mu, int e, int j0, int H, int lpr, const PairW &w0,
                                    const uint32_t *xs, int T, int tmask, uint32_t *hq, int wpi,
                                    int wi) {
    constexpr int CPC = 128 / BITS, XP = small_xpitch<BITS>();
    const int lane = threadIdx.x & 63;
    const int lr = lane % lpr;
    const int nch = H / CPC;
    float acc[SM_TMAX * 4];                                 // value 4 t + r: token t, row r
#pragma unroll
    for (int i = 0; i < SM_TMAX * 4; ++i) acc[i] = 0.0f;
    // one K step: the lane's chunk of each of the 4 rows, against every token
    auto kstep = [&](const PairW &w, int k0) __attribute__((always_inline)) {
        const int c = k0 + lr;
        const bool ok = c < nch;
        const int cc = ok ? c : nch - 1;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            // gate row 2p and up row 2p + 1 against every token: the codes are unpacked
            // once (all of the chunk), each token's x chunk is read in one go (one wait
            // per token), and each token keeps even / odd column sums (4-bit, as
            // chunk_dot) or two partial sums (8-bit) per row
            const u32x4 &qg = w.q[2 * p], &qu = w.q[2 * p + 1];
            constexpr int NJ = BITS == 4 ? 4 : 2;          // 16-byte x reads per chunk
            uint32_t dg[NJ][4], du[NJ][4];                   // fp16 words meeting x word i of read j
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                if constexpr (BITS == 4) {
                    const uint32_t lo = 0x000F000Fu, hi = 0x00F000F0u;
                    const uint32_t g8 = qg[j] >> 8, u8 = qu[j] >> 8;
                    dg[j][0] = and_or(qg[j], lo, QS_MAGIC);
                    dg[j][1] = and_or(qg[j], hi, QS_MAGIC);
                    dg[j][2] = and_or(g8, lo, QS_MAGIC);
                    dg[j][3] = and_or(g8, hi, QS_MAGIC);
                    du[j][0] = and_or(qu[j], lo, QS_MAGIC);
                    du[j][1] = and_or(qu[j], hi, QS_MAGIC);
                    du[j][2] = and_or(u8, lo, QS_MAGIC);
                    du[j][3] = and_or(u8, hi, QS_MAGIC);
                } else {
                    const uint32_t lo = 0x00FF00FFu;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        dg[j][2 * h] = and_or(qg[2 * j + h], lo, QS_MAGIC);
                        dg[j][2 * h + 1] = and_or(qg[2 * j + h] >> 8, lo, QS_MAGIC);
                        du[j][2 * h] = and_or(qu[2 * j + h], lo, QS_MAGIC);
                        du[j][2 * h + 1] = and_or(qu[2 * j + h] >> 8, lo, QS_MAGIC);
                    }
                }
            }
            float ag[SM_TMAX][2], au[SM_TMAX][2];
#pragma unroll
            for (int t = 0; t < SM_TMAX; ++t) {
                ag[t][0] = ag[t][1] = au[t][0] = au[t][1] = 0.0f;
                if (t >= T || !((tmask >> t) & 1)) continue;
                u32x4 xx[NJ];
#pragma unroll
                for (int j = 0; j < NJ; ++j) xx[j] = *(const u32x4 *)(xs + (t * nch + cc) * XP + 4 * j);
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        // 4-bit: words 0, 2 are even columns, 1, 3 odd (high nibbles as 16 q)
                        const int o = BITS == 4 ? (i & 1) : (i >> 1);
                        ag[t][o] = __builtin_amdgcn_fdot2(as_h2(dg[j][i]), as_h2(xx[j][i]), ag[t][o], false);
                        au[t][o] = __builtin_amdgcn_fdot2(as_h2(du[j][i]), as_h2(xx[j][i]), au[t][o], false);
                    }
            }
            const float sg = f16_to_f32((uint16_t)w.sc[2 * p]), bg = f16_to_f32((uint16_t)w.bi[2 * p]);
            const float su = f16_to_f32((uint16_t)w.sc[2 * p + 1]), bu = f16_to_f32((uint16_t)w.bi[2 * p + 1]);
#pragma unroll
            for (int t = 0; t < SM_TMAX; ++t) {
                if (t >= T || !((tmask >> t) & 1)) continue;
                const u32x4 xp = *(const u32x4 *)(xs + (t * nch + cc) * XP + CPC / 2);   // the sums' pad
                const float2 X = make_float2(__uint_as_float(xp[0]), __uint_as_float(xp[1]));
                float pg, pu;
                if constexpr (BITS == 4) {
                    pg = sg * ag[t][0] + (sg * 0.0625f) * ag[t][1] + (bg - 1024.0f * sg) * X.x + (bg - 64.0f * sg) * X.y;
                    pu = su * au[t][0] + (su * 0.0625f) * au[t][1] + (bu - 1024.0f * su) * X.x + (bu - 64.0f * su) * X.y;
                } else {
                    pg = sg * (ag[t][0] + ag[t][1]) + (bg - 1024.0f * sg) * (X.x + X.y);
                    pu = su * (au[t][0] + au[t][1]) + (bu - 1024.0f * su) * (X.x + X.y);
                }
                acc[4 * t + 2 * p] += ok ? pg : 0.0f;
                acc[4 * t + 2 * p + 1] += ok ? pu : 0.0f;
            }
        }
    };
    // the first step's weights are in registers already; only later steps (rows longer
    // than lpr chunks) load here, so that the compiler's wait for them is the only wait
    kstep(w0, 0);
    for (int k0 = lpr; k0 < nch; k0 += lpr) {
        PairW w;
        load_pairs<BITS>(mg, mu, e, j0, H, lpr, k0, w);
        kstep(w, k0);
    }
    if (lpr == 64) {
        // value 4 t + r ends in lanes 16 t + 4 r .. + 3: gate (r = 0, 2) meets up (r + 1)
        // four lanes up, and the pair's second h value sits eight lanes up
        const float v = wave_sum16(acc);
        const float h = silu(v) * dpp<0x104>(v);
        const float h1 = dpp<0x108>(h);
        const int t = lane >> 4;
        if ((lane & 15) == 0 && t < T)
            hq[t * wpi + wi] = pack_f16x2(f32_to_f16_ftz(h), f32_to_f16_ftz(h1));
    } else {
#pragma unroll
        for (int t = 0; t < SM_TMAX; ++t) {
            if (t >= T) continue;
            float hv[2];
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const float g = group_sum(acc[4 * t + 2 * p], lpr);
                const float u = group_sum(acc[4 * t + 2 * p + 1], lpr);
                hv[p] = silu(g) * u;
            }
            if (lr == 0) hq[t * wpi + wi] = pack_f16x2(f32_to_f16_ftz(hv[0]), f32_to_f16_ftz(hv[1]));
        }
    }
}

template <int BITS>
__global__ __launch_bounds__(DT) __attribute__((amdgpu_waves_per_eu(4))) void k_decode_small(SmallArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint32_t dsm[];
    __shared__ SmallSel S;
    __shared__ uint32_t s_flag;
    __shared__ float s_lg[SM_TMAX][NW];
    constexpr int CPC = 128 / BITS;
    const Layer &L = a.L;
    uint32_t *ctl = a.ctl;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = L.H, I = L.I, E = L.E, K = L.K, T = a.T;
    const int nR = a.nR, nP = a.nP, nS = a.nS, nG = a.nG, nD = a.nD;
    const int b = blockIdx.x;
    const uint32_t tag = ld_dev(ctl + CTL_GEN) + 1;

    if (b < nR) {
        // -------------------------------------------- R: one expert per wave, all tokens
        // (x of all tokens staged raw in LDS; the router row is read once per wave)
        uint16_t *xr = (uint16_t *)dsm;
        for (int i = tid; i < T * H / 8; i += DT) *(u32x4 *)(xr + 8 * i) = *(const u32x4 *)(a.x + 8 * (int64_t)i);
        __syncthreads();
        const int e = b * NW + wave;
        float acc[SM_TMAX] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (e < E) {
            const uint16_t *wr = L.router_w + (int64_t)e * H;
            for (int c0 = lane; c0 < H / 8; c0 += 4 * 64) {
                u32x4 wv[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int c = c0 + 64 * k;
                    wv[k] = c < H / 8 ? __builtin_nontemporal_load((const u32x4 *)(wr + 8 * c)) : (u32x4){0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int t = 0; t < SM_TMAX; ++t) {
                    if (t >= T) break;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int c = c0 + 64 * k;
                        if (c >= H / 8) break;
                        const u32x4 xv = *(const u32x4 *)(xr + t * H + 8 * c);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            acc[t] = __builtin_fmaf(__uint_as_float(xv[i] << 16), __uint_as_float(wv[k][i] << 16), acc[t]);
                            acc[t] = __builtin_fmaf(__uint_as_float(xv[i] & 0xffff0000u),
                                                    __uint_as_float(wv[k][i] & 0xffff0000u), acc[t]);
                        }
                    }
                }
            }
        }
        const float bias = (e < E && L.router_bias) ? L.router_bias[e] : 0.0f;
#pragma unroll
        for (int t = 0; t < SM_TMAX; ++t) {
            const float v = wave_sum(acc[t]) + bias;
            if (lane == 0) s_lg[t][wave] = v;
        }
        __syncthreads();
        if (wave == 0) {
            constexpr int PIECES = NW / 2;
            for (int i = lane; i < SM_LCOPIES * SM_TMAX * PIECES; i += 64) {
                const int c = i / (SM_TMAX * PIECES), t = (i / PIECES) % SM_TMAX, q = i % PIECES;
                const int e0 = b * NW + 2 * q;
                if (t >= T) continue;
                uint32_t *dst = ctl + LOGIT_BASE + c * SM_LSTRIDE + 2 * (t * SM_TE + e0);
                if (e0 + 1 < E)
                    st_dev128(dst, (u32x4){__float_as_uint(s_lg[t][2 * q]), tag, __float_as_uint(s_lg[t][2 * q + 1]), tag});
                else if (e0 < E)
                    st_dev64((uint64_t *)dst, __float_as_uint(s_lg[t][2 * q]) | ((uint64_t)tag << 32));
            }
        }
        return;
    }
    if (b < nR + nP) {
        // ----------------------------- P: selectors, wave t takes token t's top-k
        const int sel = b - nR;
        if (wave < T) {
            const uint64_t *lg = (const uint64_t *)(ctl + LOGIT_BASE + (sel % SM_LCOPIES) * SM_LSTRIDE) + wave * SM_TE;
            const TopkOut tk = select_topk_from(ctl, lg, tag, E, K);
            if (lane < K) {
                S.si[wave * K + lane] = tk.idx;
                S.sw[wave * K + lane] = tk.w;
            }
        }
        __syncthreads();
        if (a.route_only) {
            if (tid < T * K) {
                if (a.out_idx) a.out_idx[tid] = S.si[tid];
                if (a.out_w) a.out_w[tid] = S.sw[tid];
            }
            if (tid == 0) st_dev(ctl + CTL_GEN, tag);          // the only reader of the logits
            return;
        }
        if (tid < T * K)
            for (int c = sel; c < TOPK_COPIES; c += nP)
                st_dev128(ctl + TOPK_BASE + c * TOPK_STRIDE + 4 * tid,
                          (u32x4){(uint32_t)S.si[tid], tag, __float_as_uint(S.sw[tid]), tag});
        return;
    }
    const int nRP = nR + nP;
    if (b < nRP + nS + nG) {
        // ------------------------------ S / G: gate/up + SwiGLU for all tokens -> h
        constexpr int XP = small_xpitch<BITS>();
        uint8_t *wb = (uint8_t *)dsm + wave * PAIR_DMA_BYTES;   // this wave's next-item weights
        uint32_t *xs = dsm + NW * PAIR_DMA_BYTES / 4;        // [T][H / CPC] chunks + sums, code order
        const int rpw = 64 / a.lprg;
        const int pb = 2 * NW * rpw;                         // h values per item
        const int bpe = (I + pb - 1) / pb;
        const bool sh = b < nRP + nS;
        const int g = sh ? b - nRP : b - nRP - nS;
        stage_x_tokens<BITS>(a.x, T, H, xs);
        int nitems = 1;
        if (!sh) {
            small_get_sel(ctl, tag, E, K, T, S);             // ends with a barrier
            nitems = (S.nu * bpe - g + nG - 1) / nG;         // items g, g + nG, ... < |U| bpe
        } else {
            __syncthreads();
        }
        const int wi = wave * rpw + lane / a.lprg;           // word (row pair) within the item
        const QMat &mg = sh ? L.s_gate : L.gate, &mu = sh ? L.s_up : L.up;
        auto item_at = [&](int m, int &u, int &rbk, int &e, int &jj) {
            const int item = sh ? g : g + m * nG;
            u = sh ? 0 : item / bpe;
            rbk = item % bpe;
            e = sh ? 0 : __builtin_amdgcn_readfirstlane(S.ul[u]);   // uniform: scalar bases
            const int j0 = rbk * pb + 2 * wi;
            jj = j0 < I ? j0 : I - 2;
        };
        {
            int u, rbk, e, jj;
            item_at(0, u, rbk, e, jj);
            load_pairs_dma<BITS>(mg, mu, e, jj, H, a.lprg, wb);
        }
        // the waves run through the items on their own (no barrier between items); each
        // wave's next item streams into its LDS slot while the current one is computed
        // from registers; the h words of all items collect in LDS and are stored once at
        // the end
        const int wpi = pb / 2;                              // h words per item and token
        uint32_t *hq = xs + SM_TMAX * (H / CPC) * XP;        // [item][T][wpi]
        for (int m = 0; m < nitems; ++m) {
            int u, rbk, e, jj;
            item_at(m, u, rbk, e, jj);
            PairW wcur;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's slot has landed
            read_pairs(wb, wcur);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // and is read before it is refilled
            if (m + 1 < nitems) {
                int u2, rbk2, e2, jj2;
                item_at(m + 1, u2, rbk2, e2, jj2);
                load_pairs_dma<BITS>(mg, mu, e2, jj2, H, a.lprg, wb);
            }
            int tmask = 0;
            for (int t = 0; t < T; ++t) tmask |= (sh || S.jt[u][t] >= 0) ? (1 << t) : 0;
            pairs_swiglu_tokens<BITS>(mg, mu, e, jj, H, a.lprg, wcur, xs, T, tmask, hq + m * T * wpi, wpi, wi);
        }
        __syncthreads();
        const int pieces = (wpi + 1) / 2;
        const int per_copy = nitems * T * pieces;
        for (int i = tid; i < SM_HCOPIES * per_copy; i += DT) {
            const int cp = i / per_copy, r = i % per_copy;
            const int m = r / (T * pieces), t = (r / pieces) % T, q = r % pieces;
            int u, rbk, e, jj;
            item_at(m, u, rbk, e, jj);
            if (!sh && S.jt[u][t] < 0) continue;             // the token did not choose the expert
            const int jb = rbk * pb;
            const int nw = min(pb, I - jb) / 2;
            if (2 * q >= nw) continue;
            const int slot = t * (K + 1) + (sh ? K : S.jt[u][t]);
            const uint32_t *src = hq + (m * T + t) * wpi + 2 * q;
            uint32_t *dst = ctl + H_BASE + cp * SM_HSTRIDE + 2 * (slot * (I / 2) + jb / 2 + 2 * q);
            if (2 * q + 1 < nw)
                st_dev128(dst, (u32x4){src[0], tag, src[1], tag});
            else
                st_dev64((uint64_t *)dst, src[0] | ((uint64_t)tag << 32));
        }
        return;
    }
    {
        // --------------------- D: down + weighted combine for all tokens, rows of a block
        // four row groups of 64 / lprd rows; wave w takes row group w % 4 and the union
        // slots of parity w / 4 (the shared expert is slot |U|)
        const int d = b - nRP - nS - nG;
        small_get_sel(ctl, tag, E, K, T, S);
        if (d == 0 && tid < T * K) {
            if (a.out_idx) a.out_idx[tid] = S.si[tid];
            if (a.out_w) a.out_w[tid] = S.sw[tid];
        }
        const int nu = __builtin_amdgcn_readfirstlane(S.nu), nslot = T * (K + 1);
        const int nv = nu + (a.shared ? 1 : 0);              // union slots incl. the shared one
        const int lpr = a.lprd, rpw = 64 / lpr;
        const int nch = I / CPC, ng = I / 64;
        const uint32_t rb = (uint32_t)I * BITS / 8;
        const int lr = lane % lpr, rr = lane / lpr;
        const int rg = wave & 3, par = wave >> 2;
        const int rloc = rg * rpw + rr;
        const int n = d * 4 * rpw + rloc;
        const int nc = n < H ? n : H - 1;
        const int cpl = (nch + lpr - 1) / lpr;
        const int nvp = (nv - par + 1) / 2;                  // union slots of this parity
        const int nit = nvp * cpl;
        constexpr int CPITCH = CPC + 8;
        uint16_t *hs16 = (uint16_t *)dsm;                     // [nslot][nch] chunks, padded
        float2 *hsum = (float2 *)(dsm + nslot * nch * CPITCH / 2);
        float *s_part = (float *)(hsum + nslot * nch);        // [2][T][4 rpw]: the two parities' sums
        uint32_t arrived = 0;
        // item it: union slot v = par + 2 (it / cpl), chunk lr + lpr (it % cpl).  Lane j < |U|
        // holds row 0 of routed slot j's down matrix; a slot's bases are read from its lane
        // as scalars (the shared slot's are the layer's)
        uint64_t pc = 0, ps = 0, pbi = 0;
        if (lane < nu) {
            const int64_t r0 = (int64_t)S.ul[lane] * L.down.stride;
            pc = (uint64_t)(L.down.codes + r0 * rb);
            ps = (uint64_t)(L.down.scales + r0 * ng);
            pbi = (uint64_t)(L.down.biases + r0 * ng);
        }
        auto slot_base = [&](int v, uint64_t &bc, uint64_t &bs, uint64_t &bb) __attribute__((always_inline)) {
            const bool routed = v < nu;
            bc = routed ? readlane64(pc, v) : (uint64_t)L.s_down.codes;
            bs = routed ? readlane64(ps, v) : (uint64_t)L.s_down.scales;
            bb = routed ? readlane64(pbi, v) : (uint64_t)L.s_down.biases;
        };
        // NB items per batch, two batches in flight: the next batch's loads are issued
        // before the current one is multiplied; loads are unconditional (clamped to a
        // valid item and discarded)
        constexpr int NB = 4;
        struct DW {
            u32x4 q[NB];
            uint32_t sv[NB], bv[NB];
        };
        auto dload = [&](int base, DW &w) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int it = min(base + i, max(nit - 1, 0));
                const int v = min(par + 2 * (it / cpl), nv - 1);
                const int c = lr + lpr * (it % cpl), cc = c < nch ? c : nch - 1;
                uint64_t bc, bs, bb;
                slot_base(v, bc, bs, bb);
                w.q[i] = __builtin_nontemporal_load((g_u32x4 *)(bc + (uint32_t)nc * rb + 16u * cc));
                const uint32_t gi = (uint32_t)nc * ng + ((cc * CPC) >> 6);
                w.sv[i] = *(g_u16 *)(bs + 2u * gi);
                w.bv[i] = *(g_u16 *)(bb + 2u * gi);
            }
        };
        float yv[SM_TMAX] = {0.0f, 0.0f, 0.0f, 0.0f};
        auto dcompute = [&](int base, const DW &w) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int it = base + i;
                const bool live = it < nit;
                const int v = min(par + 2 * (min(it, max(nit - 1, 0)) / cpl), nv - 1);
                const int c = lr + lpr * (it % cpl), cc = c < nch ? c : nch - 1;
#pragma unroll
                for (int t = 0; t < SM_TMAX; ++t) {
                    if (t >= T) break;
                    const int j = v < nu ? S.jt[v][t] : K;
                    if (!live || j < 0) continue;                // uniform: the token did not choose it
                    const float wt = v < nu ? S.sw[t * K + j] : 1.0f;
                    const int ch = (t * (K + 1) + j) * nch + cc;
                    const float p = chunk_dot<BITS>(w.q[i], (const uint32_t *)(hs16 + ch * CPITCH), w.sv[i], w.bv[i],
                                                    hsum[ch]);
                    yv[t] += c < nch ? wt * p : 0.0f;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        DW wa, wb;
        dload(0, wa);
        if (NB < nit) dload(NB, wb);
        __builtin_amdgcn_sched_barrier(0);
        {
            // all of h: groups of 8 values, 16-byte device loads, fp16 into LDS in code
            // order, chunk sums by a DPP sum over the chunk's groups
            const uint32_t *hw = ctl + H_BASE + (d % SM_HCOPIES) * SM_HSTRIDE;
            const int ngrp = nslot * I / 8;
            for (int g0 = 0; g0 < ngrp; g0 += DT) {
                const int g = g0 + tid;
                const bool live = g < ngrp;
                const int gg = live ? g : ngrp - 1;
                const int j = (gg / (I / 8)) % (K + 1);
                // slots nobody writes (a token's shared slot without a shared expert)
                const bool used = j < K || a.shared;
                u32x4 w0 = {0u, tag, 0u, tag}, w1 = {0u, tag, 0u, tag};
                for (uint32_t it = 0; used; ++it) {
                    ld_dev256(hw + 8 * gg, w0, w1);
                    if (w0[1] == tag && w0[3] == tag && w1[1] == tag && w1[3] == tag) break;
                    if (it > SPIN_LIMIT) {
                        raise_error(ctl);
                        break;
                    }
                    poll_pause(it);
                }
                const u32x4 nat = {w0[0], w0[2], w1[0], w1[2]};
                float se = 0.0f, so = 0.0f;
#pragma unroll
                for (int jx = 0; jx < 4; ++jx) {
                    const f16x2 hh = as_h2(nat[jx]);
                    se += (float)hh[0];
                    so += (float)hh[1];
                }
                if (live) *(u32x4 *)(hs16 + (g / (CPC / 8)) * CPITCH + 8 * (g % (CPC / 8))) = perm8<BITS>(nat);
                se = group_sum(se, CPC / 8);
                so = group_sum(so, CPC / 8);
                if (live && (g % (CPC / 8)) == 0) hsum[g / (CPC / 8)] = make_float2(se, so);
            }
            __syncthreads();
            if (tid == 0) arrived = add_dev(ctl + CNT_BASE + (d % NGRP) * 64);
        }
        for (int base = 0; base < nit; base += 2 * NB) {
            dcompute(base, wa);
            if (base + 2 * NB < nit) dload(base + 2 * NB, wa);
            if (base + NB < nit) {
                dcompute(base + NB, wb);
                if (base + 3 * NB < nit) dload(base + 3 * NB, wb);
            }
        }
#pragma unroll
        for (int t = 0; t < SM_TMAX; ++t) {
            if (t >= T) break;
            const float s = group_sum(yv[t], lpr);
            if (lr == 0) s_part[(par * SM_TMAX + t) * 4 * rpw + rloc] = s;
        }
        __syncthreads();
        for (int i = tid; i < T * 4 * rpw; i += DT) {
            const int t = i / (4 * rpw), r = i % (4 * rpw);
            const int nn = d * 4 * rpw + r;
            if (nn < H) {
                const float yy = s_part[t * 4 * rpw + r] + s_part[(SM_TMAX + t) * 4 * rpw + r];
                if (a.y_dtype == QSMOE_F32) ((float *)a.y)[(int64_t)t * H + nn] = yy;
                else ((uint16_t *)a.y)[(int64_t)t * H + nn] = f32_to_bf16(yy);
            }
        }
        if (tid == 0) {
            const int g = d % NGRP;
            const int gsize = nD / NGRP + (g < nD % NGRP ? 1 : 0);
            const int ngroups = nD < NGRP ? nD : NGRP;
            uint32_t last = 0;
            if (arrived == (uint32_t)(gsize - 1)) last = add_dev(ctl + CNT_TOP) == (uint32_t)(ngroups - 1);
            s_flag = last;
        }
        __syncthreads();
        if (s_flag) finish_call(ctl, tag);
    }
}

// lanes sharing one row: the largest power of two <= min(64, 16-byte chunks per row)
int lanes_per_row(int ncols, int bits) {
    const int chunks = ncols * bits / 128;
    int l = 64;
    while (l > chunks) l >>= 1;
    return l;
}

hipError_t launch(DecArgs a, hipStream_t s) {
    const Layer &L = a.L;
    const int cpc = 128 / L.bits;
    a.lprg = lanes_per_row(L.H, L.bits);
    a.lprd = lanes_per_row(L.I, L.bits);
    const int pb = 2 * NW * (64 / a.lprg);
    const int bpe = (L.I + pb - 1) / pb;
    a.nR = (L.E + NW - 1) / NW;
    size_t lds = 16;
    a.vs = 1;
    if (a.route_only) {
        a.nP = 1;
        a.nS = a.nG = a.nD = 0;
    } else {
        a.nP = N_SELECT;                               // reduced below to what the consumers need
        a.nS = a.shared ? bpe : 0;
        a.nG = L.K * bpe;
        const int nvec = L.K + (a.shared ? 1 : 0);
        // split the vectors of a row block over more waves while the grid stays within
        // what the device holds at once (two workgroups per CU)
        const int resident = 2 * n_compute_units();
        a.vs = 1;
        while (a.vs < 4 && 2 * a.vs <= nvec) {
            const int rows = NW / (2 * a.vs) * (64 / a.lprd);
            if (a.nR + a.nP + a.nS + a.nG + (L.H + rows - 1) / rows > resident) break;
            a.vs *= 2;
        }
        const int rows = NW / a.vs * (64 / a.lprd);
        a.nD = (L.H + rows - 1) / rows;
        // consumer b reads copy b % TOPK_COPIES, written by selector b % nP: with nP a power
        // of two no larger than the (contiguous) G and D range, every selector is read, so
        // every selector has started before the call can complete
        while (a.nP > 1 && a.nP > a.nG + a.nD) a.nP >>= 1;
        const size_t lds_g = (size_t)L.H * 2 + (size_t)(L.H / cpc) * 8;
        const size_t lds_d = (size_t)nvec * (L.I / cpc) * (cpc + 8) * 2 + (size_t)nvec * (L.I / cpc) * 8;
        lds = lds_g > lds_d ? lds_g : lds_d;
    }
    const int grid = a.nR + a.nP + a.nS + a.nG + a.nD;
    if (L.bits == 4)
        hipLaunchKernelGGL((k_decode<4>), dim3(grid), dim3(DT), lds, s, a);
    else
        hipLaunchKernelGGL((k_decode<8>), dim3(grid), dim3(DT), lds, s, a);
    return hipGetLastError();
}

// dynamic LDS of a small-batch call: the largest of the roles' needs
//   S / G: per wave a slot for the next item's weights (direct-to-LDS), the tokens' x
//          chunks with their column sums, the h words of up to SM_TMAX items (a G
//          workgroup has at most T: |U| <= T K items of blocks over nG = K bpe workgroups)
//   D:     h of every slot as padded fp16 chunks with chunk sums, the two parities' sums
//   R:     x of all tokens, raw
size_t small_lds_bytes(const Layer &L, int T) {
    const int cpc = 128 / L.bits;
    const int pb = 2 * NW * (64 / lanes_per_row(L.H, L.bits));
    const int rows = 4 * (64 / lanes_per_row(L.I, L.bits));
    const size_t nslot = (size_t)T * (L.K + 1);
    const size_t g = (size_t)NW * PAIR_DMA_BYTES + (size_t)SM_TMAX * (L.H / cpc) * (cpc / 2 + 4) * 4 +
                     (size_t)SM_TMAX * SM_TMAX * (pb / 2) * 4;
    const size_t d = nslot * (L.I / cpc) * (cpc + 8) * 2 + nslot * (L.I / cpc) * 8 + (size_t)2 * SM_TMAX * rows * 4;
    const size_t r = (size_t)T * L.H * 2;
    return std::max(std::max(g, d), r);
}

hipError_t launch_small(SmallArgs a, hipStream_t s) {
    const Layer &L = a.L;
    a.lprg = lanes_per_row(L.H, L.bits);
    a.lprd = lanes_per_row(L.I, L.bits);
    const int pb = 2 * NW * (64 / a.lprg);
    const int bpe = (L.I + pb - 1) / pb;
    a.nR = (L.E + NW - 1) / NW;
    size_t lds = (size_t)a.T * L.H * 2;                // R: x of all tokens, raw
    if (a.route_only) {
        a.nP = 1;
        a.nS = a.nG = a.nD = 0;
    } else {
        a.nS = a.shared ? bpe : 0;
        a.nG = L.K * bpe;                              // every G workgroup gets at least one item
        const int rows = 4 * (64 / a.lprd);
        a.nD = (L.H + rows - 1) / rows;
        a.nP = N_SELECT;
        while (a.nP > 1 && a.nP > a.nG + a.nD) a.nP >>= 1;
        lds = small_lds_bytes(L, a.T);
    }
    const int grid = a.nR + a.nP + a.nS + a.nG + a.nD;
    if (L.bits == 4)
        hipLaunchKernelGGL((k_decode_small<4>), dim3(grid), dim3(DT), lds, s, a);
    else
        hipLaunchKernelGGL((k_decode_small<8>), dim3(grid), dim3(DT), lds, s, a);
    return hipGetLastError();
}

SmallArgs make_small_args(const Layer &L, const uint16_t *x, int64_t T, const DecodeBufs &b) {
    SmallArgs a{};
    a.L = L;
    a.x = x;
    a.ctl = b.ctl;
    a.T = (int)T;
    a.y_dtype = QSMOE_F32;
    a.shared = L.has_shared;
    return a;
}

DecArgs make_args(const Layer &L, const uint16_t *x, const DecodeBufs &b) {
    DecArgs a{};
    a.L = L;
    a.x = x;
    a.ctl = b.ctl;
    a.y_dtype = QSMOE_F32;
    a.shared = L.has_shared;
    return a;
}

}  // namespace

hipError_t launch_decode_layer(const Layer &L, const uint16_t *x, const DecodeBufs &b, void *y,
                               int y_dtype, int32_t *out_idx, float *out_w, hipStream_t s) {
    DecArgs a = make_args(L, x, b);
    a.y = y;
    a.y_dtype = y_dtype;
    a.out_idx = out_idx;
    a.out_w = out_w;
    return launch(a, s);
}

// (LDS bound: two workgroups per CU keep the whole grid resident on these shapes; larger
// ones take the grouped path)
bool decode_small_eligible(const Layer &L, int64_t T) {
    return T >= 2 && T <= SM_TMAX && T * (L.K + 1) * L.I / 2 <= SM_HWORDS && L.E <= SM_TE &&
           small_lds_bytes(L, (int)T) <= SMALL_LDS_MAX;
}

hipError_t launch_decode_small_layer(const Layer &L, const uint16_t *x, int64_t T, const DecodeBufs &b, void *y,
                                     int y_dtype, int32_t *out_idx, float *out_w, hipStream_t s) {
    SmallArgs a = make_small_args(L, x, T, b);
    a.y = y;
    a.y_dtype = y_dtype;
    a.out_idx = out_idx;
    a.out_w = out_w;
    return launch_small(a, s);
}

hipError_t launch_decode_small_route(const Layer &L, const uint16_t *x, int64_t T, const DecodeBufs &b,
                                     int32_t *out_idx, float *out_w, hipStream_t s) {
    SmallArgs a = make_small_args(L, x, T, b);
    a.shared = 0;
    a.route_only = 1;
    a.out_idx = out_idx;
    a.out_w = out_w;
    return launch_small(a, s);
}

hipError_t launch_decode_route(const Layer &L, const uint16_t *x, const DecodeBufs &b, int32_t *out_idx,
                               float *out_w, hipStream_t s) {
    DecArgs a = make_args(L, x, b);
    a.shared = 0;
    a.route_only = 1;
    a.out_idx = out_idx;
    a.out_w = out_w;
    return launch(a, s);
}

}  // namespace qs
