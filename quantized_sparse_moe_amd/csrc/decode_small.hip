// decode_small.hip -- small-batch decode (T = 2 .. 4 tokens: batched or verification
// decode) in one launch.
//
// [LILY] "Optimize the single-row weight path" at a few rows: the T = 1 structure
// (decode.hip) with every role covering all T tokens.  The routed experts are the union U
// of the tokens' selections, and each touched expert's weights are read once: G reads the
// gate/up rows of an expert for the tokens that chose it, D the down rows for all of them.
// The hand-off regions of the T = 1 path are reused with other strides (every word
// carries the call's tag, so the two paths cannot mistake each other's words).
//
//   R  router logits of all tokens, one expert per wave (x of all tokens in LDS, each
//      router row read once)
//   P  selectors: wave t takes token t's top-k and publishes it
//   S  shared expert gate/up + SwiGLU for all tokens
//   G  items (union slot, block of row pairs), several per workgroup; each wave runs
//      through its items on its own: the next item's codes and scales stream into the
//      wave's LDS slot by direct-to-LDS loads while the current one is computed; a row
//      pair's codes are unpacked once and meet every token that chose the expert; the
//      16 partial sums of a lane (4 tokens x 4 rows) are reduced in one transposing
//      butterfly
//   D  down + weighted combine of all tokens for a block of output rows: weight loads
//      as soon as the selection is known, then all of h, then a fixed-order sum
#include "decode_state.h"

namespace qs {

namespace {

constexpr int SM_TMAX = SMALL_TMAX;
constexpr int SM_LCOPIES = 8;
constexpr int SM_TE = 264;                                  // logit words per token and copy (E + gate)
constexpr int SM_LSTRIDE = 2 * SM_TMAX * SM_TE + 64;        // u32 per logits copy
static_assert(SM_LCOPIES * SM_LSTRIDE <= LOGIT_COPIES * LOGIT_STRIDE, "small-T logits region");
constexpr int SM_HCOPIES = 2;
constexpr int SM_HSTRIDE = H_COPIES * H_STRIDE / SM_HCOPIES;   // u32 per h copy
constexpr int SM_HEXPW = 2304;                                 // block-scale words per copy
constexpr int SM_HWORDS = SM_HSTRIDE / 2 - 64 - SM_HEXPW;      // h words per copy
constexpr int SM_HEXP = 2 * (SM_HWORDS + 32);                  // u32 offset of the scale words
constexpr size_t SMALL_LDS_MAX = 76 * 1024;                    // dynamic LDS of a small-batch call
static_assert(2 * SM_TMAX * 16 <= TOPK_STRIDE / 2, "small-T selection region");
static_assert(4 * (64 + SM_TMAX) <= TOPK_STRIDE, "small-T gate entries");

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
    float sg[SM_TMAX];                                      // the shared expert's gate per token
};
// (gated: entry 64 + t holds token t's shared-expert gate)
__device__ void small_get_sel(uint32_t *ctl, uint32_t tag, int E, int K, int T, int gated, SmallSel &S) {
    const int tid = threadIdx.x, n = T * K;
    if (tid < 8) S.ub[tid] = 0u;
    if (tid < SM_TMAX * 16 * SM_TMAX) (&S.jt[0][0])[tid] = -1;
    if (tid < 64) {
        const int lane = tid;
        const uint64_t *tp = (const uint64_t *)(ctl + TOPK_BASE + (blockIdx.x % TOPK_COPIES) * TOPK_STRIDE);
        const bool act = lane < n, actg = gated && lane < T;
        const uint64_t none = (uint64_t)tag << 32;
        uint64_t w0, w1, wg;
        const uint32_t lim = wait_bound(ctl);
        for (uint32_t it = 0;; ++it) {
            w0 = act ? ld_dev64(tp + 2 * lane) : none;
            w1 = act ? ld_dev64(tp + 2 * lane + 1) : none;
            wg = actg ? ld_dev64(tp + 2 * (64 + lane) + 1) : none;
            if (__ballot(tag_of(w0) != tag || tag_of(w1) != tag || tag_of(wg) != tag) == 0ull) break;
            if (it > lim) {
                if (lane == 0) raise_error(ctl);
                break;
            }
            poll_pause(it);
        }
        if (act) {
            S.si[lane] = min(max((int)(uint32_t)w0, 0), E - 1);
            S.sw[lane] = __uint_as_float((uint32_t)w1);
        }
        if (lane < SM_TMAX) S.sg[lane] = actg ? __uint_as_float((uint32_t)wg) : 1.0f;
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
// xs + (t nch + c) * pitch, its column sums right after it), one (token, chunk) per thread,
// each token under its range scale 2^e_t (0 for rows of ordinary magnitude, which are
// staged in one pass); the returned LDS array holds 2^-e_t.  Ends with a barrier.
template <int BITS>
__device__ __forceinline__ uint32_t stage_x_row(const uint16_t *x, int t, int H, uint32_t *xs, float f) {
    constexpr int CPC = 128 / BITS, XP = small_xpitch<BITS>();
    const int nch = H / CPC;
    uint32_t m = 0u;                                         // largest |x| as ordered bits
    for (int c = threadIdx.x & 63; c < nch; c += 64) {
        const uint16_t *xc = x + (int64_t)t * H + c * CPC;
        uint32_t *xd = xs + (t * nch + c) * XP;
        float se = 0.0f, so = 0.0f;
        for (int g = 0; g < CPC / 8; ++g) {
            const u32x4 v = *(const u32x4 *)(xc + 8 * g);
            u32x4 nat;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                m = max(m, max((v[k] << 16) & 0x7fffffffu, v[k] & 0x7fff0000u));
                const _Float16 lo = f32_to_f16_ftz(__uint_as_float(v[k] << 16) * f);
                const _Float16 hi = f32_to_f16_ftz(__uint_as_float(v[k] & 0xffff0000u) * f);
                se += (float)lo;
                so += (float)hi;
                nat[k] = pack_f16x2(lo, hi);
            }
            *(u32x4 *)(xd + 4 * g) = perm8<BITS>(nat);
        }
        *(float2 *)(xd + CPC / 2) = chunk_sums<BITS>(se, so);
    }
    return m;
}
// wave t stages token t: the wave finds the row's largest |x| itself and, for a row of
// extreme magnitude only, stages it again under 2^e; the returned LDS array holds 2^-e_t,
// visible after the caller's next barrier
template <int BITS>
__device__ const float *stage_x_tokens(const uint16_t *x, int T, int H, uint32_t *xs) {
    __shared__ float s_xinv[SM_TMAX];
    const int t = threadIdx.x >> 6;
    if (t < T) {
        const uint32_t m = wave_max_u32(stage_x_row<BITS>(x, t, H, xs, 1.0f));
        const int e = range_exp(__uint_as_float(m));
        if (e != 0) stage_x_row<BITS>(x, t, H, xs, exp2i(e));
        if ((threadIdx.x & 63) == 0) s_xinv[t] = exp2i(-e);
    }
    return s_xinv;
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
                                    const uint32_t *xs, int T, int tmask, float *hq, int pb,
                                    int wi, int sb_bf16, const float *xinv) {
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
            const float sg = sb_to_f32(w.sc[2 * p], sb_bf16), bg = sb_to_f32(w.bi[2 * p], sb_bf16);
            const float su = sb_to_f32(w.sc[2 * p + 1], sb_bf16), bu = sb_to_f32(w.bi[2 * p + 1], sb_bf16);
#pragma unroll
            for (int t = 0; t < SM_TMAX; ++t) {
                if (t >= T || !((tmask >> t) & 1)) continue;
                const u32x4 xp = *(const u32x4 *)(xs + (t * nch + cc) * XP + CPC / 2);   // the sums' pad
                const float2 XY = make_float2(__uint_as_float(xp[0]), __uint_as_float(xp[1]));   // chunk_sums
                // (the affine map of chunk_dot: s (A - Y) + b X)
                const float Ag = BITS == 4 ? __builtin_fmaf(ag[t][1], 0.0625f, ag[t][0]) : ag[t][0] + ag[t][1];
                const float Au = BITS == 4 ? __builtin_fmaf(au[t][1], 0.0625f, au[t][0]) : au[t][0] + au[t][1];
                const float pg = __builtin_fmaf(sg, Ag - XY.y, bg * XY.x);
                const float pu = __builtin_fmaf(su, Au - XY.y, bu * XY.x);
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
        // four lanes up, and the pair's second h value sits eight lanes up (x's scale of
        // token t taken out first)
        const int t = lane >> 4;
        const float v = wave_sum16(acc) * xinv[t];
        const float h = silu(v) * dpp<0x104>(v);
        const float h1 = dpp<0x108>(h);
        if ((lane & 15) == 0 && t < T) {
            hq[t * pb + 2 * wi] = h;
            hq[t * pb + 2 * wi + 1] = h1;
        }
    } else {
#pragma unroll
        for (int t = 0; t < SM_TMAX; ++t) {
            if (t >= T) continue;
            float hv[2];
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const float g = group_sum(acc[4 * t + 2 * p], lpr) * xinv[t];
                const float u = group_sum(acc[4 * t + 2 * p + 1], lpr) * xinv[t];
                hv[p] = silu(g) * u;
            }
            if (lr == 0) {
                hq[t * pb + 2 * wi] = hv[0];
                hq[t * pb + 2 * wi + 1] = hv[1];
            }
        }
    }
}

// SBF: the layer's scales and biases are bf16 (else fp16), fixed per instantiation so that
// their widening is one instruction
template <int BITS, int SBF>
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
    const int sb_bf16 = SBF, gated = L.shared_gate_w != nullptr && a.shared;
    const int nR = a.nR, nP = a.nP, nS = a.nS, nG = a.nG, nD = a.nD;
    const int b = blockIdx.x;
    const uint32_t tag = call_tag(ctl);

    if (b < nR) {
        // -------------------------------------------- R: one expert per wave, all tokens
        // (x of all tokens staged raw in LDS; the router row is read once per wave)
        uint16_t *xr = (uint16_t *)dsm;
        for (int i = tid; i < T * H / 8; i += DT) *(u32x4 *)(xr + 8 * i) = *(const u32x4 *)(a.x + 8 * (int64_t)i);
        __syncthreads();
        const int e = b * NW + wave;
        float acc[SM_TMAX] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (e < E + gated) {                                  // e = E: the shared expert's gate
            const uint16_t *wr = e < E ? L.router_w + (int64_t)e * H : L.shared_gate_w;
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
                if (e0 + 1 < E + gated)
                    st_dev128(dst, (u32x4){__float_as_uint(s_lg[t][2 * q]), tag, __float_as_uint(s_lg[t][2 * q + 1]), tag});
                else if (e0 < E + gated)
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
            float gate;
            const TopkOut tk = select_topk_from(ctl, lg, tag, E, K, gated, &gate);
            if (lane < K) {
                S.si[wave * K + lane] = tk.idx;
                S.sw[wave * K + lane] = tk.w;
            }
            if (lane == 0) S.sg[wave] = gate;
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
        if (gated && tid < T)                                // entry 64 + t: token t's shared gate
            for (int c = sel; c < TOPK_COPIES; c += nP)
                st_dev128(ctl + TOPK_BASE + c * TOPK_STRIDE + 4 * (64 + tid),
                          (u32x4){(uint32_t)E, tag, __float_as_uint(S.sg[tid]), tag});
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
        const float *xinv = stage_x_tokens<BITS>(a.x, T, H, xs);
        int nitems = 1;
        if (!sh) {
            small_get_sel(ctl, tag, E, K, T, gated, S);             // ends with a barrier
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
        // from registers; the h values of all items collect in LDS and are stored once at
        // the end, as fp16 pairs under one range scale per (item, token)
        const int wpi = pb / 2;                              // h words per item and token
        float *hq = (float *)(xs + SM_TMAX * (H / CPC) * XP);   // [item][T][pb]
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
            pairs_swiglu_tokens<BITS>(mg, mu, e, jj, H, a.lprg, wcur, xs, T, tmask, hq + m * T * pb, pb, wi,
                                      sb_bf16, xinv);
        }
        __syncthreads();
        // the scale of each (item, token): from the largest |h| of its valid values
        __shared__ int s_es[SM_TMAX * SM_TMAX];
        if (tid < nitems * T) {
            const int m = tid / T;
            int u, rbk, e, jj;
            item_at(m, u, rbk, e, jj);
            const int nv = min(pb, I - rbk * pb);
            const float *hv = hq + tid * pb;
            uint32_t mb = 0u;
            for (int i = 0; i < nv; ++i) mb = max(mb, __float_as_uint(hv[i]) & 0x7fffffffu);
            s_es[tid] = range_exp(__uint_as_float(mb));
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
            const int es = s_es[m * T + t];
            const float f = exp2i(es);
            const float *src = hq + (m * T + t) * pb + 4 * q;
            auto word = [&](int i) { return pack_f16x2(f32_to_f16_ftz(src[2 * i] * f), f32_to_f16_ftz(src[2 * i + 1] * f)); };
            uint32_t *dst = ctl + H_BASE + cp * SM_HSTRIDE + 2 * (slot * (I / 2) + jb / 2 + 2 * q);
            if (2 * q + 1 < nw)
                st_dev128(dst, (u32x4){word(0), tag, word(1), tag});
            else
                st_dev64((uint64_t *)dst, word(0) | ((uint64_t)tag << 32));
            if (q == 0)
                st_dev64((uint64_t *)(ctl + H_BASE + cp * SM_HSTRIDE + SM_HEXP + 2 * (slot * bpe + rbk)),
                         (uint32_t)es | ((uint64_t)tag << 32));
        }
        return;
    }
    {
        // --------------------- D: down + weighted combine for all tokens, rows of a block
        // four row groups of 64 / lprd rows; wave w takes row group w % 4 and the union
        // slots of parity w / 4 (the shared expert is slot |U|)
        const int d = b - nRP - nS - nG;
        small_get_sel(ctl, tag, E, K, T, gated, S);
        // counted in as soon as the generation has been read, ahead of the weight loads
        // (their waits cover the reply, which is needed only at the end)
        uint32_t arrived = 0;
        if (tid == 0) arrived = add_dev(ctl + CNT_BASE + (d % NGRP) * 64);
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
        float *hinv = (float *)(hsum + nslot * nch);          // 2^-e of each chunk's h scale
        float *s_part = hinv + nslot * nch;                   // [2][T][4 rpw]: the two parities' sums
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
                    const float wt = v < nu ? S.sw[t * K + j] : S.sg[t];   // shared: its gate (or 1)
                    const int ch = (t * (K + 1) + j) * nch + cc;
                    const float p = chunk_dot<BITS>(w.q[i], (const uint32_t *)(hs16 + ch * CPITCH), w.sv[i], w.bv[i],
                                                    hsum[ch], sb_bf16) * hinv[ch];
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
            // all of h: groups of 8 values, 16-byte device loads with their block's scale
            // word, brought to the chunk's smallest block scale (a power of two), fp16
            // into LDS in code order, chunk sums by a DPP sum over the chunk's groups
            const uint32_t *hw = ctl + H_BASE + (d % SM_HCOPIES) * SM_HSTRIDE;
            const uint64_t *he = (const uint64_t *)(hw + SM_HEXP);
            const int pbg = 2 * NW * (64 / a.lprg);           // values per item block (a power of two)
            const int pbsh = 31 - __builtin_clz(pbg);
            const int bpe = (I + pbg - 1) / pbg;
            const int ngrp = nslot * I / 8;
            const uint32_t lim = wait_bound(ctl);
            for (int g0 = 0; g0 < ngrp; g0 += DT) {
                const int g = g0 + tid;
                const bool live = g < ngrp;
                const int gg = live ? g : ngrp - 1;
                const int sv = gg / (I / 8), sj = 8 * (gg - sv * (I / 8));
                const int j = sv % (K + 1);
                // slots nobody writes (a token's shared slot without a shared expert)
                const bool used = j < K || a.shared;
                u32x4 w0 = {0u, tag, 0u, tag}, w1 = {0u, tag, 0u, tag};
                uint64_t we = (uint64_t)tag << 32;
                for (uint32_t it = 0; used; ++it) {
                    we = ld_dev64(he + sv * bpe + (sj >> pbsh));
                    ld_dev256(hw + 8 * gg, w0, w1);
                    if (w0[1] == tag && w0[3] == tag && w1[1] == tag && w1[3] == tag && tag_of(we) == tag) break;
                    if (it > lim) {
                        raise_error(ctl);
                        break;
                    }
                    poll_pause(it);
                }
                const int es = (int)(uint32_t)we;
                int ec = es;                                 // the chunk's smallest block scale
                if (CPC / 8 >= 2) ec = min(ec, (int)dpp_u32<0xB1>((uint32_t)ec + 128u) - 128);
                if (CPC / 8 >= 4) ec = min(ec, (int)dpp_u32<0x4E>((uint32_t)ec + 128u) - 128);
                u32x4 nat = {w0[0], w0[2], w1[0], w1[2]};
                if (ec != es) {                              // (blocks of extreme magnitude only)
                    const float fr = exp2i(ec - es);
#pragma unroll
                    for (int jx = 0; jx < 4; ++jx) {
                        const f16x2 hh = as_h2(nat[jx]);
                        nat[jx] = pack_f16x2(f32_to_f16_ftz((float)hh[0] * fr), f32_to_f16_ftz((float)hh[1] * fr));
                    }
                }
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
                if (live && (g % (CPC / 8)) == 0) {
                    hsum[g / (CPC / 8)] = chunk_sums<BITS>(se, so);
                    hinv[g / (CPC / 8)] = exp2i(-ec);
                }
            }
            __syncthreads();
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
                if (a.y_dtype == MOE_F32) ((float *)a.y)[(int64_t)t * H + nn] = yy;
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
                     (size_t)SM_TMAX * SM_TMAX * pb * 4;
    const size_t d = nslot * (L.I / cpc) * (cpc + 8) * 2 + nslot * (L.I / cpc) * 12 + (size_t)2 * SM_TMAX * rows * 4;
    const size_t r = (size_t)T * L.H * 2;
    return std::max(std::max(g, d), r);
}

hipError_t launch_small(SmallArgs a, hipStream_t s) {
    const Layer &L = a.L;
    a.lprg = lanes_per_row(L.H, L.bits);
    a.lprd = lanes_per_row(L.I, L.bits);
    const int pb = 2 * NW * (64 / a.lprg);
    const int bpe = (L.I + pb - 1) / pb;
    a.nR = (L.E + (L.shared_gate_w && a.shared ? 1 : 0) + NW - 1) / NW;   // + the shared gate's logit
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
    void (*kern)(SmallArgs) = L.bits == 4 ? (L.sb_bf16 ? k_decode_small<4, 1> : k_decode_small<4, 0>)
                                       : (L.sb_bf16 ? k_decode_small<8, 1> : k_decode_small<8, 0>);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(DT), lds, s, a);
    return hipGetLastError();
}

SmallArgs make_small_args(const Layer &L, const uint16_t *x, int64_t T, const DecodeBufs &b) {
    SmallArgs a{};
    a.L = L;
    a.x = x;
    a.ctl = b.ctl;
    a.T = (int)T;
    a.y_dtype = MOE_F32;
    a.shared = L.has_shared;
    return a;
}

}  // namespace

// (LDS bound: two workgroups per CU keep the whole grid resident on these shapes; larger
// ones take the grouped path)
bool decode_small_eligible(const Layer &L, int64_t T) {
    const int pb = 2 * NW * (64 / lanes_per_row(L.H, L.bits));
    return T >= 2 && T <= SM_TMAX && T * (L.K + 1) * L.I / 2 <= SM_HWORDS && L.E <= SM_TE &&
           T * (L.K + 1) * ((L.I + pb - 1) / pb) <= SM_HEXPW && small_lds_bytes(L, (int)T) <= SMALL_LDS_MAX;
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

}  // namespace qs
