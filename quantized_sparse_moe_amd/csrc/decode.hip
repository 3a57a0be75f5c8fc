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
// 12 MB), four roles chosen by workgroup index:
//   R  router logits (fp32), one wave per expert; the last R workgroup to finish takes
//      the top-k and publishes it
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
// atomics, which are coherent across the XCDs without L2 write-back/invalidate.
// Completion is counted in two levels (NGRP group counters, then one top counter) so
// that no single line absorbs one atomic per workgroup; "ready" flags are replicated
// NCOPY times so that no single line absorbs all the polling.  The last D workgroup
// puts every control word back to zero for the next call.
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
constexpr int NGRP = 16;                    // group counters per completion count
constexpr int NCOPY = 16;                   // copies of the ready flags / routing

// control region layout, in uint32 units (each counter on a line of its own)
enum { K_ROUTER = 0, K_H = 1, K_DONE = 2 };
constexpr int CTL_ERR = 0;
constexpr int CNT_BASE = 64;                               // + (kind * NGRP + g) * 64
constexpr int TOP_BASE = CNT_BASE + 3 * NGRP * 64;         // + kind * 64
constexpr int COPY_BASE = TOP_BASE + 3 * 64;               // + copy * COPY_STRIDE
constexpr int COPY_STRIDE = 1088;                          // 4352 bytes between copies
constexpr int CP_TOPK = 0, CP_H = 1, CP_IDX = 16, CP_W = 32;
static_assert(COPY_BASE + NCOPY * COPY_STRIDE <= (int)(WS_CTL_BYTES / 4), "control region");

struct DecArgs {
    Layer L;
    const uint16_t *x;
    DecodeBufs b;
    int32_t *out_idx;
    float *out_w;
    void *y;
    int y_dtype;
    int shared;
    int nR, nS, nG, nD;         // workgroups per role
    int lprg;                   // gate/up: lanes per row (pairs per wave = 64 / lprg)
    int lprd;                   // down: lanes per row (rows per wave = 64 / lprd)
};

__device__ __forceinline__ void st_dev(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// member `m` of `total` signals completion of its device-scope stores; true (in every
// thread) for exactly one workgroup: the last of all members
__device__ bool signal_all(uint32_t *ctl, int kind, int m, int total, uint32_t *s_flag) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const int g = m % NGRP;
        const int gsize = total / NGRP + (g < total % NGRP ? 1 : 0);
        const int ngroups = total < NGRP ? total : NGRP;
        uint32_t last = 0;
        if (add_dev(ctl + CNT_BASE + (kind * NGRP + g) * 64) == (uint32_t)(gsize - 1))
            last = add_dev(ctl + TOP_BASE + kind * 64) == (uint32_t)(ngroups - 1);
        *s_flag = last;
    }
    __syncthreads();
    return *s_flag != 0;
}

// raise a ready flag in every copy, after this workgroup's stores are acknowledged
__device__ void raise_flag(uint32_t *ctl, int which) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x < NCOPY) st_dev(ctl + COPY_BASE + threadIdx.x * COPY_STRIDE + which, 1u);
}

// thread 0 waits (bounded, with back-off) for a non-zero flag; then the workgroup goes on
__device__ void wait_flag(uint32_t *ctl, const uint32_t *p) {
    if (threadIdx.x == 0) {
        uint32_t n = 0;
        while (ld_dev(p) == 0u) {
            if (n < 8) __builtin_amdgcn_s_sleep(1);
            else __builtin_amdgcn_s_sleep(6);
            if (++n > SPIN_LIMIT) {
                __hip_atomic_fetch_or(ctl + CTL_ERR, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
}

__device__ void reset_controls(uint32_t *ctl) {
    const int t = threadIdx.x;
    if (t < 3 * NGRP) st_dev(ctl + CNT_BASE + t * 64, 0u);
    if (t < 3) st_dev(ctl + TOP_BASE + t * 64, 0u);
    if (t < NCOPY) {
        st_dev(ctl + COPY_BASE + t * COPY_STRIDE + CP_TOPK, 0u);
        st_dev(ctl + COPY_BASE + t * COPY_STRIDE + CP_H, 0u);
    }
}

__device__ __forceinline__ float no_nan(float v) { return (v != v) ? -__builtin_inff() : v; }

// x (bf16) -> LDS fp16 in code order (|v| < 2^-14 flushed) + per-chunk fp32 sums
template <int BITS>
__device__ void stage_x(const uint16_t *x, int H, uint32_t *xs, float *xsum) {
    constexpr int CPC = 128 / BITS;
    for (int c = threadIdx.x; c < H / CPC; c += DT) {
        float sum = 0.0f;
        for (int g = 0; g < CPC / 8; ++g) {
            const u32x4 v = *(const u32x4 *)(x + c * CPC + 8 * g);
            u32x4 nat;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const _Float16 lo = f32_to_f16_ftz(__uint_as_float(v[i] << 16));
                const _Float16 hi = f32_to_f16_ftz(__uint_as_float(v[i] & 0xffff0000u));
                sum += (float)lo + (float)hi;
                nat[i] = pack_f16x2(lo, hi);
            }
            *(u32x4 *)(xs + (c * CPC + 8 * g) / 2) = perm8<BITS>(nat);
        }
        xsum[c] = sum;
    }
}

// sum_c (s q_c + b) x_c over one 16-byte chunk of codes
template <int BITS>
__device__ __forceinline__ float chunk_dot(const u32x4 &q, const uint32_t *xs, uint32_t s16, uint32_t b16, float X) {
    const u32x4 *xv = (const u32x4 *)xs;
    float acc = 0.0f;
    if constexpr (BITS == 4) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t m[4];
            magic_u4(q[d], m);
            const u32x4 xx = xv[d];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2(as_h2(m[i]), as_h2(xx[i]), acc, false);
        }
    } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t m[2];
            magic_u8(q[d], m);
            const u32x4 xx = xv[d >> 1];
            const int o = 2 * (d & 1);
            acc = __builtin_amdgcn_fdot2(as_h2(m[0]), as_h2(xx[o]), acc, false);
            acc = __builtin_amdgcn_fdot2(as_h2(m[1]), as_h2(xx[o + 1]), acc, false);
        }
    }
    const float s = f16_to_f32((uint16_t)s16), b = f16_to_f32((uint16_t)b16);
    return s * acc + (b - 1024.0f * s) * X;
}

__device__ __forceinline__ float group_reduce(float v, int width) {
    for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// [gate; up] row pairs j0 and j1 of matrix stacks (mg, mu), expert e: SwiGLU values
// (in every lane of the row group; lpr lanes share a pair).  All loads of a step --
// 2 pairs x 2 rows x 2 chunks -- are issued before any is used.
template <int BITS>
__device__ void pairs_swiglu(const QMat &mg, const QMat &mu, int64_t e, int j0, int j1, int H, int lpr,
                             const uint32_t *xs, const float *xsum, float hv[2]) {
    constexpr int CPC = 128 / BITS;
    const int lr = (threadIdx.x & 63) % lpr;
    const int nch = H / CPC, ng = H / 64;
    const int64_t rb = (int64_t)H * BITS / 8;
    const uint8_t *cp[4];
    const uint16_t *sp[4], *bp[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {               // r = 2 * pair + (0 gate | 1 up)
        const QMat &m = (r & 1) ? mu : mg;
        const int64_t R = e * m.stride + ((r >> 1) ? j1 : j0);
        cp[r] = m.codes + R * rb;
        sp[r] = m.scales + R * ng;
        bp[r] = m.biases + R * ng;
    }
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c0 = lr; c0 < nch; c0 += 2 * lpr) {
        u32x4 q[8];
        uint32_t s[8], b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = i >> 1, c = c0 + (i & 1) * lpr;
            q[i] = (u32x4){0u, 0u, 0u, 0u};
            s[i] = b[i] = 0;
            if (c < nch) {
                const int gi = (c * CPC) >> 6;
                q[i] = __builtin_nontemporal_load((const u32x4 *)(cp[r] + 16 * c));
                s[i] = sp[r][gi];
                b[i] = bp[r][gi];
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = c0 + (i & 1) * lpr;
            if (c < nch) acc[i >> 1] += chunk_dot<BITS>(q[i], xs + c * (CPC / 2), s[i], b[i], xsum[c]);
        }
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const float g = group_reduce(acc[2 * p], lpr);
        const float u = group_reduce(acc[2 * p + 1], lpr);
        hv[p] = silu(g) * u;
    }
}

template <int BITS>
__global__ __launch_bounds__(DT) void k_decode(DecArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint32_t dsm[];
    __shared__ uint32_t s_flag;
    __shared__ __attribute__((aligned(16))) float s_logit[256];
    __shared__ int s_idx[16];
    __shared__ float s_w[16];
    constexpr int CPC = 128 / BITS;
    const Layer &L = a.L;
    uint32_t *ctl = a.b.ctl;
    uint32_t *copy = ctl + COPY_BASE + (blockIdx.x % NCOPY) * COPY_STRIDE;    // the copy this WG reads
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = L.H, I = L.I, E = L.E, K = L.K;
    const int nR = a.nR, nS = a.nS, nG = a.nG, nD = a.nD;
    const int b = blockIdx.x;

    auto get_topk = [&]() {
        wait_flag(ctl, copy + CP_TOPK);
        if (tid < K) {
            s_idx[tid] = min(max((int)ld_dev(copy + CP_IDX + tid), 0), E - 1);
            s_w[tid] = __uint_as_float(ld_dev(copy + CP_W + tid));
        }
        __syncthreads();
    };

    if (b < nR) {
        // ---------------------------------------------------------------- R: logits
        const int e = b * NW + wave;
        if (e < E) {
            const uint16_t *wr = L.router_w + (int64_t)e * H;
            float acc = 0.0f;
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
            acc = wave_sum(acc);
            if (lane == 0)
                st_dev((uint32_t *)a.b.logits + e, __float_as_uint(acc + (L.router_bias ? L.router_bias[e] : 0.0f)));
        }
        if (signal_all(ctl, K_ROUTER, b, nR, &s_flag)) {
            // the last router workgroup: every logit is in; select and publish
            if (tid < 256)
                s_logit[tid] = (tid < E) ? __uint_as_float(ld_dev((const uint32_t *)a.b.logits + tid)) : -__builtin_inff();
            __syncthreads();
            if (wave == 0) {
                // one wave: K rounds of butterfly arg-max over 4 logits per lane
                const TopkOut tk = wave_topk([&](int e2) { return no_nan(s_logit[e2]); }, E, K);
                if (lane < K) { s_idx[lane] = min(max(tk.idx, 0), E - 1); s_w[lane] = tk.w; }
            }
            __syncthreads();
            for (int i = tid; i < NCOPY * K; i += DT) {
                uint32_t *cp = ctl + COPY_BASE + (i / K) * COPY_STRIDE;
                st_dev(cp + CP_IDX + i % K, (uint32_t)s_idx[i % K]);
                st_dev(cp + CP_W + i % K, __float_as_uint(s_w[i % K]));
            }
            if (tid < K) {
                if (a.out_idx) a.out_idx[tid] = s_idx[tid];
                if (a.out_w) a.out_w[tid] = s_w[tid];
            }
            if (nS + nG + nD == 0) reset_controls(ctl);      // routing only: nobody waits
            else raise_flag(ctl, CP_TOPK);
        }
        return;
    }
    if (b < nR + nS + nG) {
        // ------------------------------------------- S / G: gate/up + SwiGLU -> h
        uint32_t *xs = dsm;
        float *xsum = (float *)(dsm + H / 2);
        const int rpw = 64 / a.lprg;                         // row groups per wave
        const int pb = 2 * NW * rpw;                         // pairs per workgroup (2 per row group)
        const bool sh = b < nR + nS;
        const int m = b - nR;                                // member index among S and G
        const int g = sh ? m : m - nS;
        const int bpe = (I + pb - 1) / pb;                   // workgroups per expert
        const int slot = sh ? K : g / bpe;                   // h row (K = shared)
        const int j0 = (sh ? g : g % bpe) * pb + wave * rpw + lane / a.lprg;
        const int j1 = j0 + NW * rpw;
        stage_x<BITS>(a.x, H, xs, xsum);
        int64_t e = 0;
        if (sh) {
            __syncthreads();
        } else {
            get_topk();                                      // ends with a barrier
            e = s_idx[slot];
        }
        float hv[2];
        pairs_swiglu<BITS>(sh ? L.s_gate : L.gate, sh ? L.s_up : L.up, e, j0 < I ? j0 : I - 1,
                           j1 < I ? j1 : I - 1, H, a.lprg, xs, xsum, hv);
        if (lane % a.lprg == 0) {
            float *hrow = a.b.h + (int64_t)slot * I;
            if (j0 < I) st_dev((uint32_t *)hrow + j0, __float_as_uint(hv[0]));
            if (j1 < I) st_dev((uint32_t *)hrow + j1, __float_as_uint(hv[1]));
        }
        if (signal_all(ctl, K_H, m, nS + nG, &s_flag)) raise_flag(ctl, CP_H);
        return;
    }
    if (b < nR + nS + nG + nD) {
        // ------------------------------------------ D: down + weighted combine
        const int d = b - nR - nS - nG;
        get_topk();
        const int nvec = K + (a.shared ? 1 : 0);
        const int lpr = a.lprd, rpw = 64 / lpr;
        const int nch = I / CPC, ng = I / 64;
        const int64_t rb = (int64_t)I * BITS / 8;
        const int lr = lane % lpr;
        const int n = d * NW * rpw + wave * rpw + lane / lpr;
        const int nc = n < H ? n : H - 1;
        uint16_t *hs16 = (uint16_t *)dsm;                     // nvec * I fp16, code order
        float *hsum = (float *)(dsm + nvec * I / 2);          // nvec * nch chunk sums
        float yv = 0.0f;
        // items (vector v, chunk c = lr + ci*lpr), NB in flight per lane
        constexpr int NB = 9;
        int v = 0, ci = 0;
        for (int base = 0; v < nvec; base += NB) {
            u32x4 q[NB];
            uint32_t sv[NB], bv[NB];
            int vv[NB], cc[NB];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int c = lr + ci * lpr;
                vv[i] = v;
                cc[i] = c;
                q[i] = (u32x4){0u, 0u, 0u, 0u};
                sv[i] = bv[i] = 0;
                if (v < nvec && c < nch) {
                    const QMat &mm = v < K ? L.down : L.s_down;
                    const int64_t R = (int64_t)(v < K ? s_idx[v] : 0) * mm.stride + nc;
                    q[i] = __builtin_nontemporal_load((const u32x4 *)(mm.codes + R * rb + 16 * c));
                    const int64_t gi = R * ng + ((c * CPC) >> 6);
                    sv[i] = mm.scales[gi];
                    bv[i] = mm.biases[gi];
                }
                if (v < nvec && (++ci) * lpr >= nch) { ci = 0; ++v; }
            }
            if (base == 0) {
                // all of h (S and G), read coalesced: fp16 in code order, then chunk sums
                wait_flag(ctl, copy + CP_H);
                const uint64_t *h2 = (const uint64_t *)a.b.h;
                const int npairs = nvec * I / 2;
                for (int p0 = 0; p0 < npairs; p0 += 4 * DT) {
                    uint64_t hv[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int p = p0 + k * DT + tid;
                        hv[k] = p < npairs ? ld_dev64(h2 + p) : 0ull;
                    }
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int p = p0 + k * DT + tid;
                        if (p < npairs) {
                            const int i0 = 2 * p, gb = i0 & ~7;
                            hs16[gb + perm_pos<BITS>(i0 & 7)] =
                                __builtin_bit_cast(uint16_t, f32_to_f16_ftz(__uint_as_float((uint32_t)hv[k])));
                            hs16[gb + perm_pos<BITS>((i0 + 1) & 7)] =
                                __builtin_bit_cast(uint16_t, f32_to_f16_ftz(__uint_as_float((uint32_t)(hv[k] >> 32))));
                        }
                    }
                }
                __syncthreads();
                for (int c2 = tid; c2 < nvec * nch; c2 += DT) {
                    const u32x4 *src = (const u32x4 *)(hs16 + c2 * CPC);
                    float sum = 0.0f;
                    for (int g8 = 0; g8 < CPC / 8; ++g8) {
                        const u32x4 w4 = src[g8];
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const f16x2 hh = as_h2(w4[k]);
                            sum += (float)hh[0] + (float)hh[1];
                        }
                    }
                    hsum[c2] = sum;
                }
                __syncthreads();
            }
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                if (vv[i] < nvec && cc[i] < nch) {
                    const float p = chunk_dot<BITS>(q[i], (const uint32_t *)(hs16 + vv[i] * I + cc[i] * CPC), sv[i],
                                                    bv[i], hsum[vv[i] * nch + cc[i]]);
                    yv += (vv[i] < K ? s_w[vv[i]] : 1.0f) * p;   // experts in ascending id, shared last
                }
            }
        }
        yv = group_reduce(yv, lpr);
        if (n < H && lr == 0) {
            if (a.y_dtype == QSMOE_F32) ((float *)a.y)[n] = yv;
            else ((uint16_t *)a.y)[n] = f32_to_bf16(yv);
        }
        if (signal_all(ctl, K_DONE, d, nD, &s_flag)) reset_controls(ctl);
    }
}

// lanes sharing one row: the largest power of two <= min(64, 16-byte chunks per row)
int lanes_per_row(int ncols, int bits) {
    const int chunks = ncols * bits / 128;
    int l = 64;
    while (l > chunks) l >>= 1;
    return l;
}

hipError_t launch(DecArgs a, bool route_only, hipStream_t s) {
    const Layer &L = a.L;
    const int cpc = 128 / L.bits;
    a.lprg = lanes_per_row(L.H, L.bits);
    a.lprd = lanes_per_row(L.I, L.bits);
    const int pb = 2 * NW * (64 / a.lprg);
    const int bpe = (L.I + pb - 1) / pb;
    a.nR = (L.E + NW - 1) / NW;
    a.nS = (!route_only && a.shared) ? bpe : 0;
    a.nG = route_only ? 0 : L.K * bpe;
    a.nD = route_only ? 0 : (L.H + NW * (64 / a.lprd) - 1) / (NW * (64 / a.lprd));
    const int nvec = L.K + (a.shared ? 1 : 0);
    const size_t lds_g = (size_t)L.H * 2 + (size_t)(L.H / cpc) * 4;
    const size_t lds_d = (size_t)nvec * L.I * 2 + (size_t)nvec * (L.I / cpc) * 4;
    const size_t lds = route_only ? 16 : (lds_g > lds_d ? lds_g : lds_d);
    const int grid = a.nR + a.nS + a.nG + a.nD;
    if (L.bits == 4)
        hipLaunchKernelGGL((k_decode<4>), dim3(grid), dim3(DT), lds, s, a);
    else
        hipLaunchKernelGGL((k_decode<8>), dim3(grid), dim3(DT), lds, s, a);
    return hipGetLastError();
}

DecArgs make_args(const Layer &L, const uint16_t *x, const DecodeBufs &b) {
    DecArgs a{};
    a.L = L;
    a.x = x;
    a.b = b;
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
    return launch(a, false, s);
}

hipError_t launch_decode_route(const Layer &L, const uint16_t *x, const DecodeBufs &b, int32_t *out_idx,
                               float *out_w, hipStream_t s) {
    DecArgs a = make_args(L, x, b);
    a.shared = 0;
    a.out_idx = out_idx;
    a.out_w = out_w;
    return launch(a, true, s);
}

}  // namespace qs
