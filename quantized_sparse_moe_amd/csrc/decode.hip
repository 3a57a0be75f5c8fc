// decode.hip -- batch-1 (T = 1) MoE layer: one kernel on the vector ALUs of gfx950.
//
// [LILY] "Optimize the single-row weight path": with one activation row there is no
// weight reuse; the layer is bound by how fast the active experts' quantized weights
// stream from HBM.  Rows are read with 16-byte coalesced loads, several lanes share a
// row (split-K) and reduce with cross-lane shuffles.
// [LILY] "Reduce intermediate and state traffic": the two expert input projections are
// fused with the gated activation, and the output projection with the routing weight
// and the shared-expert result; temporaries stay in registers / LDS.
// [LILY] "Overlap independent GPU work": phases without a data dependency run at the
// same time, and a phase waits only for the results it consumes.
//
// One launch, four phases.  A workgroup takes a ticket when it starts; the ticket, not
// blockIdx, picks its phase, so a workgroup only ever waits for workgroups that took
// earlier tickets and are therefore already running: no deadlock whatever the
// occupancy.
//   R  router logits (fp32), one wave per expert                      -> router_done
//   S  shared expert gate/up + SwiGLU (needs nothing)                 -> h_done
//   G  routed expert gate/up + SwiGLU: waits for R, takes the top-k   -> h_done
//   D  down projections of the k routed + shared experts for a block of output rows,
//      weighted and summed in a fixed order (ascending expert id, shared last): waits
//      for R, takes the top-k, issues its weight loads, then waits for all of h.
// Counters live in the first bytes of the caller's workspace: zero before the first
// call, and the last workgroup to exit puts them back to zero.  Waits are bounded: a
// wait that exceeds SPIN_LIMIT polls raises an error flag and the kernel still ends.
//
// Dequantization happens in registers: codes become fp16 (1024+q) by bit operations
// and meet fp16 activations in v_dot2_f32_f16 with fp32 accumulation; per 16-byte chunk
// the affine map is applied once:  sum_c (s q_c + b) x_c = s A + (b - 1024 s) X  with
// A = sum_c (1024+q_c) x_c and X = sum_c x_c.
#include "common.h"
#include "internal.h"

namespace qs {

namespace {

constexpr int DT = 256;                 // threads per workgroup
constexpr int NBUF_G = 8;               // (row, chunk) loads a G/S lane keeps in flight
constexpr int NBUF_D = 18;              // (expert, chunk) loads a D lane keeps in flight
constexpr uint32_t SPIN_LIMIT = 1u << 22;

// Control words (uint32 offsets into the workspace's control region).  Counters that
// many workgroups increment sit on lines of their own; the "ready" flags that many
// workgroups poll are replicated NCOPY times, far apart, each waiting workgroup polling
// one copy, so no single line carries all the polling traffic.
constexpr int CTL_TICKET = 0, CTL_EXIT = 1, CTL_ERR = 2;
constexpr int CTL_ROUTER = 64, CTL_H = 128;
constexpr int NCOPY = 16;
constexpr int COPY_BASE = 256, COPY_STRIDE = 1088;          // 4352 bytes between copies
constexpr int CP_TOPK = 0, CP_H = 1, CP_IDX = 16, CP_W = 32;  // inside one copy
static_assert(COPY_BASE + NCOPY * COPY_STRIDE <= (int)(WS_CTL_BYTES / 4), "control region");

struct DecArgs {
    Layer L;
    const uint16_t *x;
    DecodeBufs b;
    int32_t *out_idx;
    float *out_w;
    void *y;
    int y_dtype;
    int shared;                 // shared expert present
    int route_only;             // moe_route: router + publish the top-k only
    int nR, nS, nG, nD;         // workgroups per phase
    int lprg, prw, pbg;         // gate/up: lanes per row, pair rounds per wave, pairs per workgroup
    int lprd, prd, rbd;         // down: lanes per row, row rounds per wave, output rows per workgroup
};

// Cross-workgroup data (logits, h) is written and read with device-scope (sc1)
// stores and loads, which go to the coherence point shared by all XCDs; counters are
// device-scope atomics.  That avoids whole-L2 write-back / invalidate operations that a
// release / acquire fence at device scope would issue in every workgroup.
__device__ __forceinline__ void st_dev(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev_u(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev_u64(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// thread 0 waits (bounded, with back-off) until the flag at p is non-zero, then the
// whole workgroup proceeds
__device__ void wait_flag(uint32_t *ctl, const uint32_t *p) {
    if (threadIdx.x == 0) {
        uint32_t n = 0;
        while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
            if (n < 8) __builtin_amdgcn_s_sleep(1);
            else __builtin_amdgcn_s_sleep(8);
            if (++n > SPIN_LIMIT) {
                __hip_atomic_fetch_or(ctl + CTL_ERR, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
}

// every wave's device-scope stores are acknowledged, then one increment; returns (to
// every thread) the counter value before the increment
__device__ uint32_t signal(uint32_t *p, uint32_t *s_old) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) *s_old = __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    return *s_old;
}

__device__ __forceinline__ float no_nan(float v) { return (v != v) ? -__builtin_inff() : v; }

// Top-k of the E <= 256 logits in LDS by rank counting (one thread per expert, exact
// ties to the lower id), renormalised over the selection; result ascending by id in
// s_idx / s_w.
__device__ void block_topk(const float *lg, int E, int K, int *sel_idx, float *sel_val, int *s_idx,
                           float *s_w) {
    const int e = threadIdx.x;
    if (e < K) { sel_idx[e] = 0; sel_val[e] = -__builtin_inff(); }
    __syncthreads();
    if (e < E) {
        const float v = no_nan(lg[e]);
        int rank = 0;
        for (int i = 0; i < E; ++i) {
            const float u = no_nan(lg[i]);
            rank += (u > v || (u == v && i < e)) ? 1 : 0;
        }
        if (rank < K) { sel_idx[rank] = e; sel_val[rank] = v; }
    }
    __syncthreads();
    if (e < K) {
        const float m = sel_val[0];
        float z = 0.0f;
        for (int j = 0; j < K; ++j) z += expf(sel_val[j] - m);
        const float wv = expf(sel_val[e] - m) / z;
        const int my = sel_idx[e];
        int r2 = 0;
        for (int j = 0; j < K; ++j) r2 += (sel_idx[j] < my) ? 1 : 0;
        s_idx[r2] = my;
        s_w[r2] = wv;
    }
    __syncthreads();
}

// Stage activations into LDS as fp16 (|v| < 2^-14 flushed), each group of 8 permuted
// into the code order of BITS, plus the fp32 sum of every 16-byte code chunk (CPC
// columns).  One thread per chunk.  `load8(col, v)` fetches 8 consecutive values.
template <int BITS, typename Load8>
__device__ void stage_chunks(Load8 load8, int nchunks, uint32_t *xs, float *xsum) {
    constexpr int CPC = 128 / BITS;
    for (int c = threadIdx.x; c < nchunks; c += DT) {
        float sum = 0.0f;
#pragma unroll
        for (int g = 0; g < CPC / 8; ++g) {
            float v[8];
            load8(c * CPC + 8 * g, v);
            _Float16 hv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                hv[i] = f32_to_f16_ftz(v[i]);
                sum += (float)hv[i];
            }
            u32x4 nat;
#pragma unroll
            for (int i = 0; i < 4; ++i) nat[i] = pack_f16x2(hv[2 * i], hv[2 * i + 1]);
            *(u32x4 *)(xs + (c * CPC + 8 * g) / 2) = perm8<BITS>(nat);
        }
        xsum[c] = sum;
    }
}

// sum_c (s q_c + b) x_c over one 16-byte chunk of codes
template <int BITS>
__device__ __forceinline__ float chunk_dot(const u32x4 &q, const uint32_t *xs, float s, float b, float X) {
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
    return s * acc + (b - 1024.0f * s) * X;
}

__device__ __forceinline__ float group_reduce(float v, int width) {
    for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

struct Row {
    const uint8_t *codes;
    const uint16_t *sc, *bi;
};

__device__ __forceinline__ Row row_of(const QMat &m, int64_t e, int64_t r, int ncols, int bits) {
    const int64_t R = e * m.stride + r;
    Row p;
    p.codes = m.codes + R * (int64_t)(ncols * bits / 8);
    p.sc = m.scales + R * (ncols / 64);
    p.bi = m.biases + R * (ncols / 64);
    return p;
}

// gate/up + SwiGLU for the pairs of one workgroup.  `pre` runs after the first batch of
// weight loads is issued and before any of them is consumed (x staging, waits).
template <int BITS, typename Pre>
__device__ void gate_up_block(const DecArgs &a, const QMat &mg, const QMat &mu, int64_t e, int p0,
                              float *h, uint32_t *xs, float *xsum, Pre pre) {
    constexpr int CPC = 128 / BITS;
    const Layer &L = a.L;
    const int H = L.H, I = L.I;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lpr = a.lprg, rpw = 64 / lpr, prw = a.prw;
    const int nch = H / CPC;
    const int cpl = (nch + lpr - 1) / lpr;
    const int nitems = 2 * prw * cpl;
    const int lr = lane % lpr;
    float part[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) part[i] = 0.0f;
    bool first = true;
    for (int base = 0; base < nitems; base += NBUF_G) {
        u32x4 q[NBUF_G];
        uint16_t sv[NBUF_G], bv[NBUF_G];
#pragma unroll
        for (int i = 0; i < NBUF_G; ++i) {
            const int it = base + i;
            const int r = it / (2 * cpl), row = (it / cpl) & 1, ci = it % cpl;
            const int j = p0 + (r * 4 + wave) * rpw + lane / lpr;
            const int c = lr + ci * lpr;
            q[i] = (u32x4){0u, 0u, 0u, 0u};
            sv[i] = bv[i] = 0;
            if (it < nitems && j < I && c < nch) {
                const Row rp = row_of(row ? mu : mg, e, j, H, BITS);
                q[i] = __builtin_nontemporal_load((const u32x4 *)(rp.codes + 16 * c));
                const int g = (c * CPC) >> 6;
                sv[i] = rp.sc[g];
                bv[i] = rp.bi[g];
            }
        }
        if (first) { pre(); first = false; }
#pragma unroll
        for (int i = 0; i < NBUF_G; ++i) {
            const int it = base + i;
            const int r = it / (2 * cpl), row = (it / cpl) & 1, ci = it % cpl;
            const int c = lr + ci * lpr;
            if (it < nitems && c < nch) {
                const float d = chunk_dot<BITS>(q[i], xs + c * (CPC / 2), f16_to_f32(sv[i]), f16_to_f32(bv[i]), xsum[c]);
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (k == r * 2 + row) part[k] += d;
            }
        }
    }
    if (first) pre();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if (r < prw) {
            const float g = group_reduce(part[2 * r], lpr);
            const float u = group_reduce(part[2 * r + 1], lpr);
            const int j = p0 + (r * 4 + wave) * rpw + lane / lpr;
            if (lr == 0 && j < I) st_dev(&h[j], silu(g) * u);
        }
    }
}

template <int BITS>
__global__ __launch_bounds__(DT) void k_decode(DecArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint32_t dsm[];
    __shared__ uint32_t s_ticket, s_old;
    __shared__ float s_logit[256];
    __shared__ int s_sel_idx[16], s_idx[16];
    __shared__ float s_sel_val[16], s_w[16];
    constexpr int CPC = 128 / BITS;
    const Layer &L = a.L;
    uint32_t *ctl = a.b.ctl;
    uint32_t *copy = ctl + COPY_BASE + (blockIdx.x % NCOPY) * COPY_STRIDE;   // the copy this WG polls
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = L.H, I = L.I, E = L.E, K = L.K;
    if (tid == 0) s_ticket = __hip_atomic_fetch_add(ctl + CTL_TICKET, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int t = (int)s_ticket;
    const int nR = a.nR, nS = a.nS, nG = a.nG, nD = a.nD;

    auto load_x8 = [&](int col, float v[8]) {
        const u32x4 xv = *(const u32x4 *)(a.x + col);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(xv[i] << 16);
            v[2 * i + 1] = __uint_as_float(xv[i] & 0xffff0000u);
        }
    };
    // the routing, published once (in every copy) by the last router workgroup
    auto get_topk = [&]() {
        wait_flag(ctl, copy + CP_TOPK);
        if (tid < K) {
            s_idx[tid] = min(max((int)ld_dev_u(copy + CP_IDX + tid), 0), E - 1);
            s_w[tid] = ld_dev((const float *)(copy + CP_W + tid));
        }
        __syncthreads();
    };
    // raise a ready flag in every copy (after this WG's own stores are acknowledged)
    auto raise = [&](int which) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid < NCOPY) st_dev_u(ctl + COPY_BASE + tid * COPY_STRIDE + which, 1u);
    };

    if (t < nR) {
        // ---------------------------------------------------------------- R: logits
        const int e = t * 4 + wave;
        if (e < E) {
            const uint16_t *wr = L.router_w + (int64_t)e * H;
            float acc = 0.0f;
            for (int c = lane; c < H / 8; c += 64) {
                const u32x4 xv = *(const u32x4 *)(a.x + 8 * c);
                const u32x4 wv = __builtin_nontemporal_load((const u32x4 *)(wr + 8 * c));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc = __builtin_fmaf(__uint_as_float(xv[i] << 16), __uint_as_float(wv[i] << 16), acc);
                    acc = __builtin_fmaf(__uint_as_float(xv[i] & 0xffff0000u),
                                         __uint_as_float(wv[i] & 0xffff0000u), acc);
                }
            }
            acc = wave_sum(acc);
            if (lane == 0) st_dev(&a.b.logits[e], acc + (L.router_bias ? L.router_bias[e] : 0.0f));
        }
        if (signal(ctl + CTL_ROUTER, &s_old) == (uint32_t)(nR - 1)) {
            // last router workgroup: every logit is in; select and publish the top-k
            if (tid < E) s_logit[tid] = ld_dev(&a.b.logits[tid]);
            __syncthreads();
            block_topk(s_logit, E, K, s_sel_idx, s_sel_val, s_idx, s_w);
            for (int i = tid; i < NCOPY * K; i += DT) {
                uint32_t *cp = ctl + COPY_BASE + (i / K) * COPY_STRIDE;
                const int j = i % K;
                st_dev_u(cp + CP_IDX + j, (uint32_t)s_idx[j]);
                st_dev((float *)(cp + CP_W + j), s_w[j]);
            }
            if (tid < K) {
                if (a.out_idx) a.out_idx[tid] = s_idx[tid];
                if (a.out_w) a.out_w[tid] = s_w[tid];
            }
            raise(CP_TOPK);
        }
    } else if (t < nR + nS) {
        // ---------------------------------------------- S: shared expert gate/up
        uint32_t *xs = dsm;
        float *xsum = (float *)(dsm + H / 2);
        gate_up_block<BITS>(a, L.s_gate, L.s_up, 0, (t - nR) * a.pbg, a.b.h + (int64_t)K * I, xs, xsum, [&]() {
            stage_chunks<BITS>(load_x8, H / CPC, xs, xsum);
            __syncthreads();
        });
        if (signal(ctl + CTL_H, &s_old) == (uint32_t)(nS + nG - 1)) raise(CP_H);
    } else if (t < nR + nS + nG) {
        // ---------------------------------------------- G: routed expert gate/up
        uint32_t *xs = dsm;
        float *xsum = (float *)(dsm + H / 2);
        const int g = t - nR - nS;
        const int bpe = (I + a.pbg - 1) / a.pbg;
        const int slot = g / bpe;
        stage_chunks<BITS>(load_x8, H / CPC, xs, xsum);      // independent of routing
        get_topk();                                          // ends with a barrier
        gate_up_block<BITS>(a, L.gate, L.up, s_idx[slot], (g % bpe) * a.pbg, a.b.h + (int64_t)slot * I, xs,
                            xsum, []() {});
        if (signal(ctl + CTL_H, &s_old) == (uint32_t)(nS + nG - 1)) raise(CP_H);
    } else if (t < nR + nS + nG + nD) {
        // ------------------------------------------ D: down + weighted combine
        const int d = t - nR - nS - nG;
        get_topk();
        const int nvec = K + (a.shared ? 1 : 0);
        const int lpr = a.lprd, rpw = 64 / lpr, prd = a.prd;
        const int nch = I / CPC;
        const int cpl = (nch + lpr - 1) / lpr;
        const int per_row = nvec * cpl;                       // items per (lane, output row)
        const int nitems = prd * per_row;
        const int lr = lane % lpr;
        uint16_t *hs16 = (uint16_t *)dsm;                     // nvec * I fp16, code order
        float *hsum = (float *)(dsm + nvec * I / 2);          // nvec * nch chunk sums
        float yv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int base = 0; base < nitems; base += NBUF_D) {
            u32x4 q[NBUF_D];
            uint16_t sv[NBUF_D], bv[NBUF_D];
#pragma unroll
            for (int i = 0; i < NBUF_D; ++i) {
                const int it = base + i;
                const int r = it / per_row, v = (it % per_row) / cpl, c = lr + (it % cpl) * lpr;
                const int n = d * a.rbd + (wave * prd + r) * rpw + lane / lpr;
                q[i] = (u32x4){0u, 0u, 0u, 0u};
                sv[i] = bv[i] = 0;
                if (it < nitems && c < nch && n < H) {
                    const Row rp = row_of(v < K ? L.down : L.s_down, v < K ? s_idx[v] : 0, n, I, BITS);
                    q[i] = __builtin_nontemporal_load((const u32x4 *)(rp.codes + 16 * c));
                    const int g = (c * CPC) >> 6;
                    sv[i] = rp.sc[g];
                    bv[i] = rp.bi[g];
                }
            }
            if (base == 0) {
                // all of h (S and G workgroups), read coalesced: fp16 in code order + sums
                wait_flag(ctl, copy + CP_H);
                const uint64_t *h2 = (const uint64_t *)a.b.h;
                for (int p0 = 0; p0 < nvec * I / 2; p0 += 8 * DT) {
                    uint64_t hv[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const int p = p0 + k * DT + tid;
                        hv[k] = p < nvec * I / 2 ? ld_dev_u64(h2 + p) : 0ull;
                    }
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const int p = p0 + k * DT + tid;
                        if (p < nvec * I / 2) {
                            const int i0 = 2 * p;                     // element index (even)
                            const int gb = i0 & ~7;
                            hs16[gb + perm_pos<BITS>(i0 & 7)] =
                                __builtin_bit_cast(uint16_t, f32_to_f16_ftz(__uint_as_float((uint32_t)hv[k])));
                            hs16[gb + perm_pos<BITS>((i0 + 1) & 7)] =
                                __builtin_bit_cast(uint16_t, f32_to_f16_ftz(__uint_as_float((uint32_t)(hv[k] >> 32))));
                        }
                    }
                }
                __syncthreads();
                for (int cc = tid; cc < nvec * nch; cc += DT) {
                    const u32x4 *src = (const u32x4 *)(hs16 + cc * CPC);
                    float sum = 0.0f;
#pragma unroll
                    for (int g8 = 0; g8 < CPC / 8; ++g8) {
                        const u32x4 w4 = src[g8];
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const f16x2 hh = as_h2(w4[k]);
                            sum += (float)hh[0] + (float)hh[1];
                        }
                    }
                    hsum[cc] = sum;
                }
                __syncthreads();
            }
#pragma unroll
            for (int i = 0; i < NBUF_D; ++i) {
                const int it = base + i;
                const int r = it / per_row, v = (it % per_row) / cpl, c = lr + (it % cpl) * lpr;
                if (it < nitems && c < nch) {
                    const float p = chunk_dot<BITS>(q[i], (const uint32_t *)(hs16 + v * I + c * CPC),
                                                    f16_to_f32(sv[i]), f16_to_f32(bv[i]), hsum[v * nch + c]);
                    const float contrib = (v < K ? s_w[v] : 1.0f) * p;   // ascending expert id, shared last
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        if (k == r) yv[k] += contrib;
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (r < prd) {
                const float y = group_reduce(yv[r], lpr);
                const int n = d * a.rbd + (wave * prd + r) * rpw + lane / lpr;
                if (n < H && lr == 0) {
                    if (a.y_dtype == QSMOE_F32) ((float *)a.y)[n] = y;
                    else ((uint16_t *)a.y)[n] = f32_to_bf16(y);
                }
            }
        }
    }
    // the last workgroup out resets counters and flags for the next call
    __syncthreads();
    if (tid == 0)
        s_old = __hip_atomic_fetch_add(ctl + CTL_EXIT, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_old == gridDim.x - 1) {
        if (tid < NCOPY) {
            st_dev_u(ctl + COPY_BASE + tid * COPY_STRIDE + CP_TOPK, 0u);
            st_dev_u(ctl + COPY_BASE + tid * COPY_STRIDE + CP_H, 0u);
        }
        if (tid == 0) {
            st_dev_u(ctl + CTL_TICKET, 0u);
            st_dev_u(ctl + CTL_ROUTER, 0u);
            st_dev_u(ctl + CTL_H, 0u);
            st_dev_u(ctl + CTL_EXIT, 0u);
        }
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
    a.route_only = route_only ? 1 : 0;
    a.lprg = lanes_per_row(L.H, L.bits);
    const int cplg = (L.H / cpc + a.lprg - 1) / a.lprg;
    a.prw = NBUF_G / (2 * cplg);
    if (a.prw < 1) a.prw = 1;
    if (a.prw > 4) a.prw = 4;
    a.pbg = 4 * (64 / a.lprg) * a.prw;
    a.lprd = lanes_per_row(L.I, L.bits);
    const int nvec = L.K + (a.shared ? 1 : 0);
    const int per_row = nvec * ((L.I / cpc + a.lprd - 1) / a.lprd);
    a.prd = NBUF_D / per_row;
    if (a.prd < 1) a.prd = 1;
    if (a.prd > 4) a.prd = 4;
    a.rbd = 4 * (64 / a.lprd) * a.prd;
    const int bpe = (L.I + a.pbg - 1) / a.pbg;
    a.nR = (L.E + 3) / 4;
    a.nS = (!route_only && a.shared) ? bpe : 0;
    a.nG = route_only ? 0 : L.K * bpe;
    a.nD = route_only ? 0 : (L.H + a.rbd - 1) / a.rbd;
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
