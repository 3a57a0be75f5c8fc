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
// 12 MB), roles chosen by workgroup index:
//   R  router logits (fp32), one wave per expert
//   S  shared expert gate/up + SwiGLU (needs nothing)
//   G  routed expert gate/up + SwiGLU, one [gate; up] row pair per row group; one wave
//      waits for all logits and takes the top-k itself
//   D  down projections of the k routed + shared experts for a block of output rows,
//      weighted and combined in a fixed order; takes the top-k like G, issues its weight
//      loads at once, then waits for all of h
//   P  (routing-only calls) one selector that writes the routing out.
// Each hand-off between workgroups costs ~0.6 us (a device-scope store seen by a poll on
// another XCD), so the consumers repeat the selection rather than wait for a published
// one.
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
// have the selection, behind their first weight loads; the last of a group counts the
// group in at the top while it waits for h, so both replies are back long before the
// end.  The workgroup that completes the top count, at its end, puts the counters back
// to zero and advances the generation: by then every D workgroup has counted in, and it
// has seen all of h and all logits, so every workgroup of the call has read the
// generation.  Hand-off words are replicated so that no single line absorbs all the
// polling.
//
// Dequantization in registers: codes become fp16 (1024+q) by bit operations and meet
// fp16 activations in v_dot2_f32_f16 with fp32 accumulation; per 16-byte chunk of codes
// the affine map is applied once:  sum_c (s q_c + b) x_c = s (A - Y) + b X  with
// A = sum_c (1024+q_c) x_c, X = sum_c x_c and Y its magic-value part, X and Y formed once
// per chunk when x or h is staged (chunk_dot, chunk_sums).
//
// Code is kept compact on purpose: a cold kernel fetches its instructions from L2, so
// long unrolled straight-line code costs microseconds here.
#include "decode_state.h"

namespace qs {

namespace {

struct DecArgs {
    Layer L;
    const uint16_t *x;
    uint32_t *ctl;
    int32_t *out_idx;
    float *out_w;
    void *y;
    int y_dtype;
    int shared;
    int nR, nP, nS, nG, nD;     // workgroups per role (nP = 1 and nS = nG = nD = 0 for routing
                                // only, else nP = 0)
    int route_only;
    int lprg;                   // gate/up: lanes per row (row groups per wave = 64 / lprg)
    int lprd;                   // down: lanes per row (rows per wave = 64 / lprd)
    int vs;                     // down: wave groups splitting the vectors of a row block
};

// x (bf16) -> LDS fp16 in code order (|v| < 2^-14 flushed) + per-chunk sums (chunk_sums
// of the even and of the odd columns' fp32 sums), under the row's range scale 2^e (returned; 0 for rows
// of ordinary magnitude, which are staged in one pass); s_wm holds one word per wave.
// Ends with a barrier.
template <int BITS>
__device__ void stage_x_pass(const uint16_t *x, int nch, float f, uint32_t *xs, float2 *xsum, uint32_t &mb) {
    constexpr int CPC = 128 / BITS;
    for (int c = threadIdx.x; c < nch; c += DT) {
        float se = 0.0f, so = 0.0f;
        for (int g = 0; g < CPC / 8; ++g) {
            const u32x4 v = *(const u32x4 *)(x + c * CPC + 8 * g);
            u32x4 nat;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                mb = max(mb, max((v[i] << 16) & 0x7fffffffu, v[i] & 0x7fff0000u));
                const _Float16 lo = f32_to_f16_ftz(__uint_as_float(v[i] << 16) * f);
                const _Float16 hi = f32_to_f16_ftz(__uint_as_float(v[i] & 0xffff0000u) * f);
                se += (float)lo;
                so += (float)hi;
                nat[i] = pack_f16x2(lo, hi);
            }
            *(u32x4 *)(xs + (c * CPC + 8 * g) / 2) = perm8<BITS>(nat);
        }
        xsum[c] = chunk_sums<BITS>(se, so);
    }
}
template <int BITS>
__device__ int stage_x(const uint16_t *x, int H, uint32_t *xs, float2 *xsum, uint32_t *s_wm) {
    const int nch = H * BITS / 128;
    uint32_t mb = 0u;                                        // largest |x| as ordered bits
    stage_x_pass<BITS>(x, nch, 1.0f, xs, xsum, mb);
    mb = wave_max_u32(mb);
    if ((threadIdx.x & 63) == 0) s_wm[threadIdx.x >> 6] = mb;
    __syncthreads();
    uint32_t all = s_wm[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) all = max(all, s_wm[w]);
    const int e = range_exp(__uint_as_float(all));
    if (e != 0) {                                            // rows of extreme magnitude only
        stage_x_pass<BITS>(x, nch, exp2i(e), xs, xsum, mb);
        __syncthreads();
    }
    return e;
}

// [gate; up] row pairs j0 and j0 + 1 of expert e in matrix stacks (mg, mu): SwiGLU
// values (in every lane of the row group; lpr lanes share a pair), g and u taken out of
// x's range scale by xinv.  Each step loads one
// chunk of each of the 4 rows; loads are unconditional (a lane past the row end re-reads
// the last chunk and discards it) so that all of a step's loads are issued before any
// wait.  Addresses are a uniform matrix base plus a 32-bit per-lane offset.
template <int BITS>
__device__ void pairs_swiglu(const QMat &mg, const QMat &mu, int e, int j0, int H, int lpr,
                             const uint32_t *xs, const float2 *xsum, int sb_bf16, float xinv, float hv[2]) {
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
            const float p = chunk_dot<BITS>(q[r], xs + cc * (CPC / 2), sc[r], bi[r], xsum[cc], sb_bf16);
            acc[r] += ok ? p : 0.0f;
        }
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const float g = group_sum(acc[2 * p], lpr) * xinv;
        const float u = group_sum(acc[2 * p + 1], lpr) * xinv;
        hv[p] = silu(g) * u;
    }
}

template <bool WEIGHTS = true>
__device__ TopkOut select_topk(uint32_t *ctl, uint32_t tag, int E, int K, int gated, float *gate) {
    return select_topk_from<WEIGHTS>(ctl, (const uint64_t *)(ctl + LOGIT_BASE + (blockIdx.x % LOGIT_COPIES) * LOGIT_STRIDE),
                            tag, E, K, gated, gate);
}

// Consumer: wave 0 waits (bounded) for every logit of the call and takes the top-k
// itself (a selection published by other workgroups would cost one more hand-off); the
// workgroup gets (s_idx, s_w): experts in ascending id, renormalised weights (and, gated,
// entry K: the shared expert's gate in s_w[K]); WEIGHTS = false leaves the weights 0 (G
// needs only the experts).  Ends with a barrier.
template <bool WEIGHTS = true>
__device__ void get_topk(uint32_t *ctl, uint32_t tag, int E, int K, int gated, int *s_idx, float *s_w) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        float gate;
        const TopkOut tk = select_topk<WEIGHTS>(ctl, tag, E, K, gated, &gate);
        if (lane < K) {
            s_idx[lane] = tk.idx;
            s_w[lane] = tk.w;
        }
        if (gated && lane == K) s_w[K] = gate;
    }
    __syncthreads();
}

// SBF: the layer's scales and biases are bf16 (else fp16), fixed per instantiation so that
// their widening is one instruction
template <int BITS, int SBF>
__global__ __launch_bounds__(DT) __attribute__((amdgpu_waves_per_eu(4))) void k_decode(DecArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint32_t dsm[];
    __shared__ uint32_t s_flag;
    __shared__ int s_idx[17];
    __shared__ float s_w[17];
    __shared__ float s_part[NW][DT / 64 * 16];
    __shared__ uint32_t s_wm[NW];
    constexpr int CPC = 128 / BITS;
    const Layer &L = a.L;
    uint32_t *ctl = a.ctl;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = L.H, I = L.I, E = L.E, K = L.K;
    const int sb_bf16 = SBF, gated = L.shared_gate_w != nullptr && a.shared;
    int nR = a.nR;
    const int nS = a.nS, nG = a.nG, nD = a.nD;
    const int b = blockIdx.x;

    if (b < nR) {
        // ------------------------------------------------- R: one router logit per wave
        // the workgroup's NW logits are gathered in LDS, then written to every copy in
        // 16-byte pieces (one 64-byte run per copy)
        __shared__ float s_lg[NW];
        const int e = b * NW + wave;
        const uint32_t tag = call_tag(ctl);
        float acc = 0.0f;
        if (e < E + gated) {                                  // e = E: the shared expert's gate
            const uint16_t *wr = e < E ? L.router_w + (int64_t)e * H : L.shared_gate_w;
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
            acc = wave_sum(acc) + ((L.router_bias && e < E) ? L.router_bias[e] : 0.0f);
        }
        if (lane == 0) s_lg[wave] = acc;
        __syncthreads();
        if (wave == 0) {
            constexpr int PIECES = NW / 2;                   // 16-byte pieces per copy
            for (int t = lane; t < LOGIT_COPIES * PIECES; t += 64) {
                const int c = t / PIECES, q = t % PIECES, e0 = b * NW + 2 * q;
                uint32_t *dst = ctl + LOGIT_BASE + c * LOGIT_STRIDE + 2 * e0;
                if (e0 + 1 < E + gated)
                    st_dev128(dst, (u32x4){__float_as_uint(s_lg[2 * q]), tag, __float_as_uint(s_lg[2 * q + 1]), tag});
                else if (e0 < E + gated)
                    st_dev64((uint64_t *)dst, __float_as_uint(s_lg[2 * q]) | ((uint64_t)tag << 32));
            }
        }
        return;
    }
    const uint32_t tag = call_tag(ctl);
    if (b < nR + a.nP) {
        // ------------------------------------------- P (routing only): the selector
        if (wave != 0) return;
        float gate;
        const TopkOut tk = select_topk(ctl, tag, E, K, 0, &gate);
        if (lane < K) {
            if (a.out_idx) a.out_idx[lane] = tk.idx;
            if (a.out_w) a.out_w[lane] = tk.w;
        }
        if (lane == 0) st_dev(ctl + CTL_GEN, tag);           // the only reader of this call's logits
        return;
    }
    nR += a.nP;                                              // the roles below follow it
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
        const int xe = stage_x<BITS>(a.x, H, xs, xsum, s_wm);     // ends with a barrier
        int e = 0;
        if (!sh) {
            get_topk<false>(ctl, tag, E, K, gated, s_idx, s_w);   // (experts only); ends with a barrier
            e = __builtin_amdgcn_readfirstlane(s_idx[slot]);
        }
        const int jj = j0 < I ? j0 : I - 2;
        float hv[2];
        pairs_swiglu<BITS>(sh ? L.s_gate : L.gate, sh ? L.s_up : L.up, e, jj, H, a.lprg, xs, xsum, sb_bf16,
                           exp2i(-xe), hv);
        // the workgroup's pb values (two per row group, consecutive in j: one slice of h)
        // are gathered in LDS; fp16 pairs under the slice's range scale 2^es go to every
        // copy in 16-byte pieces, and es itself to the slice's word
        // (each wave's largest magnitude goes with them; a storing thread takes the
        // slice's from those NW words.  Row groups past the end repeat the last pair.)
        __shared__ float s_hv[2 * NW * 64];
        __shared__ uint32_t s_hm[NW];
        const int wi = wave * rpw + lane / a.lprg;           // word within the workgroup
        if (lane % a.lprg == 0) {
            s_hv[2 * wi] = hv[0];
            s_hv[2 * wi + 1] = hv[1];
        }
        const uint32_t wm = wave_max_u32(max(__float_as_uint(hv[0]) & 0x7fffffffu, __float_as_uint(hv[1]) & 0x7fffffffu));
        if (lane == 0) s_hm[wave] = wm;
        __syncthreads();
        const int jb = j0 - 2 * wi;                          // first j of the workgroup
        const int nw = min(pb, I - jb) / 2;                  // valid words
        if (tid >= H_COPIES * ((nw + 1) / 2) && tid >= H_COPIES) return;   // no store to make
        uint32_t mb = s_hm[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) mb = max(mb, s_hm[w]);
        const int es = range_exp(__uint_as_float(mb));
        const float f = exp2i(es);
        auto word = [&](int i) { return pack_f16x2(f32_to_f16_ftz(s_hv[2 * i] * f), f32_to_f16_ftz(s_hv[2 * i + 1] * f)); };
        const int pieces = (nw + 1) / 2;
        for (int t = tid; t < H_COPIES * pieces; t += DT) {
            const int cp = t / pieces, q = t % pieces;
            uint32_t *dst = ctl + H_BASE + cp * H_STRIDE + 2 * (slot * (I / 2) + jb / 2 + 2 * q);
            if (2 * q + 1 < nw)
                st_dev128(dst, (u32x4){word(2 * q), tag, word(2 * q + 1), tag});
            else
                st_dev64((uint64_t *)dst, word(2 * q) | ((uint64_t)tag << 32));
        }
        if (tid < H_COPIES)
            st_dev64((uint64_t *)(ctl + H_BASE + tid * H_STRIDE + H_EXP + 2 * (slot * bpe + jb / pb)),
                     (uint32_t)es | ((uint64_t)tag << 32));
        return;
    }
    {
        // ------------------------------------------ D: down + weighted combine
        const int d = b - nR - nS - nG;
        get_topk(ctl, tag, E, K, gated, s_idx, s_w);
        uint32_t arrived = 0, top = 0;                      // replies of the two counters
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
        float2 *hsum = (float2 *)(dsm + nvec * nch * CPITCH / 2);   // chunk sums (chunk_sums)
        float *hinv = (float *)(hsum + nvec * nch);                 // chunk range scales, inverted
        // lane j < nvec holds row 0 of vector j's down matrix (the k routed experts in
        // ascending id, then the shared one) and its combine weight
        uint64_t pc = 0, ps = 0, pbi = 0;
        float wl = 1.0f;
        // (the matrix fields are read as uniform values and selected per lane: a per-lane
        // choice between the two descriptors would read them with vector loads and wait)
        if (lane < nvec) {
            const bool routed = lane < K;
            const int64_t R0 = routed ? (int64_t)s_idx[lane] * L.down.stride : 0;
            pc = routed ? (uint64_t)(L.down.codes + R0 * rb) : (uint64_t)L.s_down.codes;
            ps = routed ? (uint64_t)(L.down.scales + R0 * ng) : (uint64_t)L.s_down.scales;
            pbi = routed ? (uint64_t)(L.down.biases + R0 * ng) : (uint64_t)L.s_down.biases;
            if (routed || gated) wl = s_w[lane];             // lane K, gated: the shared gate
        }
        float yv = 0.0f;
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
                // this workgroup has read the generation: count it in now, behind the
                // first weight loads (the polls below wait for the reply with them; its
                // value is needed only at the end)
                if (tid == 0) arrived = add_dev(ctl + CNT_BASE + (d % NGRP) * 64);
                // all of h (S and G).  Wave 0 first waits for the slice words of the copy
                // (one small word per slice: light polling while the producers work); the
                // data words, stored along with them, are then read once.  Thread t takes
                // groups of 8 consecutive values (4 words) and the word of their slice, two
                // groups at a time with every load in flight: the chunk's slices are brought
                // to their smallest range scale (exact: a power of two), fp16 into LDS in
                // code order with one 16-byte write, and the chunk sums by a DPP sum over
                // the chunk's groups.  A word not yet visible is polled for on its own.
                const uint64_t *hw = (const uint64_t *)(ctl + H_BASE + (d % H_COPIES) * H_STRIDE);
                const uint64_t *he = (const uint64_t *)(ctl + H_BASE + (d % H_COPIES) * H_STRIDE + H_EXP);
                const int ngrp = nvec * I / 8;
                const int pbg = 2 * NW * (64 / a.lprg);               // values per slice
                const int nsl = (I + pbg - 1) / pbg;                  // slices per vector
                const uint32_t lim = wait_bound(ctl);
                // the last of a group to count in counts the group in at the top (this
                // waits for the first reply; both are back long before the end)
                if (tid == 0) {
                    const int grp = d % NGRP;
                    const int gsize = nD / NGRP + (grp < nD % NGRP ? 1 : 0);
                    if (arrived == (uint32_t)(gsize - 1)) top = add_dev(ctl + CNT_TOP) + 1u;
                }
                if (wave == 0) {
                    const int nslt = nvec * nsl;
                    for (uint32_t t = 0;; ++t) {
                        bool miss = false;
                        for (int i0 = 0; i0 < nslt; i0 += 8 * 64) {
                            uint64_t ew[8];
#pragma unroll
                            for (int u = 0; u < 8; ++u) {
                                const int i = i0 + 64 * u + lane;
                                ew[u] = i < nslt ? ld_dev64(he + i) : (uint64_t)tag << 32;
                            }
#pragma unroll
                            for (int u = 0; u < 8; ++u) miss |= tag_of(ew[u]) != tag;
                        }
                        if (__ballot(miss) == 0ull) break;
                        if (t > lim) {
                            if (lane == 0) raise_error(ctl);
                            break;
                        }
                        poll_pause(t);
                    }
                }
                __syncthreads();
                auto fresh = [&](uint64_t e, const u32x4 &w0, const u32x4 &w1) {
                    return w0[1] == tag && w0[3] == tag && w1[1] == tag && w1[3] == tag && tag_of(e) == tag;
                };
                // (a stale word: this XCD's L2 lines are dropped, as for an acquire, and the
                // group is polled for at device scope)
                auto poll_group = [&](const uint64_t *ep, int gg, uint64_t &e, u32x4 &w0, u32x4 &w1) {
                    for (uint32_t t = 0; !fresh(e, w0, w1); ++t) {
                        if (t > lim) {
                            raise_error(ctl);
                            break;
                        }
                        if (t == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                        else poll_pause(t);
                        ld_dev_group(ep, hw + 4 * gg, e, w0, w1);
                    }
                };
                auto put_group = [&](int g, bool live, uint64_t we, const u32x4 &w0, const u32x4 &w1) {
                    const int es = (int)(uint32_t)we;
                    int ec = es;                                 // the chunk's smallest slice scale
                    if (CPC / 8 >= 2) ec = min(ec, (int)dpp_u32<0xB1>((uint32_t)ec + 128u) - 128);
                    if (CPC / 8 >= 4) ec = min(ec, (int)dpp_u32<0x4E>((uint32_t)ec + 128u) - 128);
                    u32x4 nat = {w0[0], w0[2], w1[0], w1[2]};
                    if (ec != es) {                              // (slices of extreme magnitude only)
                        const float fr = exp2i(ec - es);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const f16x2 hh = as_h2(nat[j]);
                            nat[j] = pack_f16x2(f32_to_f16_ftz((float)hh[0] * fr), f32_to_f16_ftz((float)hh[1] * fr));
                        }
                    }
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
                    if (live && (g % (CPC / 8)) == 0) {
                        hsum[g / (CPC / 8)] = chunk_sums<BITS>(se, so);
                        hinv[g / (CPC / 8)] = exp2i(-ec);
                    }
                };
                for (int g0 = 0; g0 < ngrp; g0 += 2 * DT) {
                    const int ga = g0 + tid, gb = ga + DT;
                    const int gga = min(ga, ngrp - 1), ggb = min(gb, ngrp - 1);
                    const uint64_t *epa = he + (8 * gga) / I * nsl + (8 * gga) % I / pbg;
                    const uint64_t *epb = he + (8 * ggb) / I * nsl + (8 * ggb) % I / pbg;
                    uint64_t ea, eb = 0;
                    u32x4 a0, a1, b0, b1;
                    const bool two = g0 + DT + 64 * wave < ngrp;     // (uniform) a live second group
                    if (two)
                        ld_cached_group2(epa, hw + 4 * gga, epb, hw + 4 * ggb, ea, a0, a1, eb, b0, b1);
                    else
                        ld_cached_group(epa, hw + 4 * gga, ea, a0, a1);
                    poll_group(epa, gga, ea, a0, a1);
                    put_group(ga, ga < ngrp, ea, a0, a1);
                    if (g0 + DT < ngrp) {                          // (uniform over the workgroup)
                        if (two) poll_group(epb, ggb, eb, b0, b1);
                        else b0 = b1 = (u32x4){0u, tag, 0u, tag};
                        put_group(gb, gb < ngrp && two, eb, b0, b1);
                    }
                }
                __syncthreads();
            }
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const bool live = base + i < nit;
                const int vi = live ? v2 : min(vlast, nvec - 1);
                const int c = lr + k2 * lpr, cc = c < nch ? c : nch - 1;
                const float p = chunk_dot<BITS>(q[i], (const uint32_t *)(hs16 + (vi * nch + cc) * CPITCH), sv[i], bv[i],
                                                hsum[vi * nch + cc], sb_bf16) * hinv[vi * nch + cc];
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
            if (a.y_dtype == MOE_F32) ((float *)a.y)[n] = y;
            else ((uint16_t *)a.y)[n] = f32_to_bf16(y);
        }
        // the workgroup that completed the top count resets the state, here at its end:
        // every D workgroup read the generation before counting in, and this one has
        // seen all of h and all logits, which every S, G and R workgroup produced after
        // reading it
        if (tid == 0) s_flag = top == (uint32_t)(nD < NGRP ? nD : NGRP);
        __syncthreads();
        if (s_flag) finish_call(ctl, tag);
    }
}


hipError_t launch(DecArgs a, hipStream_t s) {
    const Layer &L = a.L;
    const int cpc = 128 / L.bits;
    a.lprg = lanes_per_row(L.H, L.bits);
    a.lprd = lanes_per_row(L.I, L.bits);
    const int pb = 2 * NW * (64 / a.lprg);
    const int bpe = (L.I + pb - 1) / pb;
    a.nR = (L.E + (L.shared_gate_w && a.shared ? 1 : 0) + NW - 1) / NW;   // + the shared gate's logit
    size_t lds = 16;
    a.vs = 1;
    if (a.route_only) {
        a.nP = 1;
        a.nS = a.nG = a.nD = 0;
    } else {
        a.nP = 0;                                      // the consumers select for themselves
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
        const size_t lds_g = (size_t)L.H * 2 + (size_t)(L.H / cpc) * 8;
        const size_t lds_d = (size_t)nvec * (L.I / cpc) * (cpc + 8) * 2 + (size_t)nvec * (L.I / cpc) * 12;
        lds = lds_g > lds_d ? lds_g : lds_d;
    }
    const int grid = a.nR + a.nP + a.nS + a.nG + a.nD;
    void (*kern)(DecArgs) = L.bits == 4 ? (L.sb_bf16 ? k_decode<4, 1> : k_decode<4, 0>)
                                       : (L.sb_bf16 ? k_decode<8, 1> : k_decode<8, 0>);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(DT), lds, s, a);
    return hipGetLastError();
}

DecArgs make_args(const Layer &L, const uint16_t *x, const DecodeBufs &b) {
    DecArgs a{};
    a.L = L;
    a.x = x;
    a.ctl = b.ctl;
    a.y_dtype = MOE_F32;
    a.shared = L.has_shared;
    return a;
}

}  // namespace

// compute units of the current device (queried once)
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

namespace {
__global__ void k_ws_status(uint32_t *ctl, uint32_t *out, int clear) {
    out[0] = clear ? __hip_atomic_exchange(ctl + CTL_ERR, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                   : ld_dev(ctl + CTL_ERR);
}
}  // namespace

hipError_t launch_ws_status(uint32_t *ctl, uint32_t *out, bool clear, hipStream_t s) {
    hipLaunchKernelGGL(k_ws_status, dim3(1), dim3(1), 0, s, ctl, out, clear ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_decode_layer(const Layer &L, const uint16_t *x, const DecodeBufs &b, void *y,
                               int y_dtype, int32_t *out_idx, float *out_w, hipStream_t s) {
    DecArgs a = make_args(L, x, b);
    a.y = y;
    a.y_dtype = y_dtype;
    a.out_idx = out_idx;
    a.out_w = out_w;
    return launch(a, s);
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
