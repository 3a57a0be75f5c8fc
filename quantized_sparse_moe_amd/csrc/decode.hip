// decode.hip -- batch-1 (T = 1) MoE layer on the vector ALUs of gfx950.
//
// [LILY] "Optimize the single-row weight path": with one activation row there is no
// weight reuse, so the layer is bound by how fast the active experts' quantized
// weights stream from HBM.  Each row is read with 16-byte coalesced loads, several
// lanes cooperate on one row (split-K) and reduce with cross-lane shuffles.
// [LILY] "Reduce intermediate and state traffic": the two expert input projections
// are fused with the gated activation (one kernel, [gate; up] pairs), and the output
// projection is fused with the routing weight and the shared-expert result.
//
// Three launches, in stream order:
//   1. router logits (fp32) for every expert, and -- independent of routing -- the
//      shared expert's gate/up + SwiGLU;
//   2. every workgroup re-derives the top-k from the logits (L2-resident), then the
//      routed experts' gate/up + SwiGLU;
//   3. down projections of the k routed experts and the shared expert for each output
//      row, weighted and summed in a fixed order (ascending expert id, shared last).
//
// Dequantization happens in registers: codes become fp16 (1024+q) by bit operations
// and meet fp16 activations in v_dot2_f32_f16 with fp32 accumulation; per group the
// affine map is applied exactly once:  sum_c (s*q_c + b) x_c = s*A + (b - 1024 s)*X
// with A = sum_c (1024+q_c) x_c and X = sum_c x_c over the 16-byte chunk.
#include "common.h"
#include "internal.h"

namespace qs {

namespace {

constexpr int DEC_THREADS = 256;

// Stage an activation vector into LDS: fp16 (|v| < 2^-14 flushed), each group of 8
// permuted into the code order of BITS, plus the fp32 sum of every 16-byte chunk of
// codes it will meet (CPC = 128/BITS columns).
template <int BITS, typename Src>
__device__ void stage_vec(Src src, int n, uint32_t *xs, float *xsum, float *gsum) {
    constexpr int CPC = 128 / BITS;
    constexpr int GPC = CPC / 8;
    for (int g = threadIdx.x; g < n / 8; g += blockDim.x) {
        float v[8];
        src(g, v);
        _Float16 hv[8];
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            hv[i] = f32_to_f16_ftz(v[i]);
            sum += (float)hv[i];
        }
        u32x4 nat;
#pragma unroll
        for (int i = 0; i < 4; ++i) nat[i] = pack_f16x2(hv[2 * i], hv[2 * i + 1]);
        *(u32x4 *)(xs + 4 * g) = perm8<BITS>(nat);
        gsum[g] = sum;
    }
    __syncthreads();
    for (int c = threadIdx.x; c < n / CPC; c += blockDim.x) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < GPC; ++i) s += gsum[c * GPC + i];
        xsum[c] = s;
    }
    __syncthreads();
}

// Dot product of one quantized row (ncols columns) with a staged vector; LPR lanes
// share the row (lane_in_row = lane % LPR), every lane returns the full sum.
template <int BITS, int LPR>
__device__ __forceinline__ float row_dot(const uint8_t *__restrict__ codes,
                                         const uint16_t *__restrict__ sc,
                                         const uint16_t *__restrict__ bi, int ncols,
                                         int lane_in_row, const uint32_t *xs, const float *xsum) {
    constexpr int CPC = 128 / BITS;
    const int nch = ncols / CPC;
    float part = 0.0f;
    for (int c = lane_in_row; c < nch; c += LPR) {
        const u32x4 q = __builtin_nontemporal_load((const u32x4 *)(codes + 16 * c));
        const u32x4 *xv = (const u32x4 *)(xs + c * (CPC / 2));
        float acc = 0.0f;
        if constexpr (BITS == 4) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t m[4];
                magic_u4(q[d], m);
                const u32x4 xx = xv[d];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc = __builtin_amdgcn_fdot2(as_h2(m[i]), as_h2(xx[i]), acc, false);
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
        const int g = (c * CPC) >> 6;
        const float s = f16_to_f32(sc[g]);
        const float b = f16_to_f32(bi[g]);
        part += s * acc + (b - 1024.0f * s) * xsum[c];
    }
    return group_sum<LPR>(part);
}

struct RowPtr {
    const uint8_t *codes;
    const uint16_t *sc, *bi;
};

__device__ __forceinline__ RowPtr row_of(const QMat &m, int64_t e, int64_t r, int ncols, int bits) {
    const int64_t R = e * m.stride + r;
    RowPtr p;
    p.codes = m.codes + R * (int64_t)(ncols * bits / 8);
    p.sc = m.scales + R * (ncols / 64);
    p.bi = m.biases + R * (ncols / 64);
    return p;
}

// gate/up + SwiGLU for `npairs` rows of expert (mg, mu, e), output h[j] for j in
// [j0, j0 + pairs handled by this block)
template <int BITS, int LPR>
__device__ void gate_up_rows(const QMat &mg, const QMat &mu, int64_t e, int H, int I, int j0,
                             const uint32_t *xs, const float *xsum, float *h) {
    constexpr int RPW = 64 / LPR;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = j0 + wave * RPW + lane / LPR;
    const int jc = j < I ? j : I - 1;               // keep every lane in the shuffles
    const RowPtr g = row_of(mg, e, jc, H, BITS);
    const RowPtr u = row_of(mu, e, jc, H, BITS);
    const float gv = row_dot<BITS, LPR>(g.codes, g.sc, g.bi, H, lane % LPR, xs, xsum);
    const float uv = row_dot<BITS, LPR>(u.codes, u.sc, u.bi, H, lane % LPR, xs, xsum);
    if (j < I && lane % LPR == 0) h[j] = silu(gv) * uv;
}

struct DecArgs {
    Layer L;
    const uint16_t *x;
    DecodeBufs b;
    int32_t *out_idx;
    float *out_w;
    void *y;
    int y_dtype;
    int n_router_blocks;
    int shared;
};

template <int BITS, int LPR>
__global__ __launch_bounds__(DEC_THREADS) void k_router_shared(DecArgs a) {
    __shared__ uint32_t xs[8192 / 2];
    __shared__ float xsum[8192 / 16];
    __shared__ float gsum[8192 / 8];
    const Layer &L = a.L;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if ((int)blockIdx.x < a.n_router_blocks) {
        // one wave per expert: fp32 logit over bf16 x and bf16 router weights
        const int e = blockIdx.x * (DEC_THREADS / 64) + wave;
        if (e >= L.E) return;
        const uint16_t *wr = L.router_w + (int64_t)e * L.H;
        float acc = 0.0f;
        for (int c = lane; c < L.H / 8; c += 64) {
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
        if (lane == 0) a.b.logits[e] = acc + (L.router_bias ? L.router_bias[e] : 0.0f);
        return;
    }
    // shared expert gate/up (no dependence on routing)
    stage_vec<BITS>([&](int g, float v[8]) {
        const u32x4 xv = *(const u32x4 *)(a.x + 8 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[2 * i] = __uint_as_float(xv[i] << 16); v[2 * i + 1] = __uint_as_float(xv[i] & 0xffff0000u); }
    }, L.H, xs, xsum, gsum);
    constexpr int PAIRS = (DEC_THREADS / 64) * (64 / LPR);
    const int j0 = (blockIdx.x - a.n_router_blocks) * PAIRS;
    gate_up_rows<BITS, LPR>(L.s_gate, L.s_up, 0, L.H, L.I, j0, xs, xsum, a.b.h + (int64_t)L.K * L.I);
}

template <int BITS, int LPR>
__global__ __launch_bounds__(DEC_THREADS) void k_gate_up(DecArgs a) {
    __shared__ uint32_t xs[8192 / 2];
    __shared__ float xsum[8192 / 16];
    __shared__ float gsum[8192 / 8];
    const Layer &L = a.L;
    constexpr int PAIRS = (DEC_THREADS / 64) * (64 / LPR);
    const int bpe = (L.I + PAIRS - 1) / PAIRS;
    const int slot = blockIdx.x / bpe;
    const int lane = threadIdx.x & 63;
    // every wave derives the routing from the L2-resident logits
    const float *lg = a.b.logits;
    const TopkOut tk = wave_topk([&](int e) { return lg[e]; }, L.E, L.K);
    const int e = __shfl(tk.idx, slot, 64);
    if (blockIdx.x == 0 && threadIdx.x < 64 && lane < L.K) {
        a.b.idx[lane] = tk.idx;
        a.b.w[lane] = tk.w;
        if (a.out_idx) a.out_idx[lane] = tk.idx;
        if (a.out_w) a.out_w[lane] = tk.w;
    }
    stage_vec<BITS>([&](int g, float v[8]) {
        const u32x4 xv = *(const u32x4 *)(a.x + 8 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[2 * i] = __uint_as_float(xv[i] << 16); v[2 * i + 1] = __uint_as_float(xv[i] & 0xffff0000u); }
    }, L.H, xs, xsum, gsum);
    const int j0 = (blockIdx.x - slot * bpe) * PAIRS;
    gate_up_rows<BITS, LPR>(L.gate, L.up, e, L.H, L.I, j0, xs, xsum, a.b.h + (int64_t)slot * L.I);
}

template <int BITS>
__global__ __launch_bounds__(64) void k_topk_only(DecArgs a) {
    const Layer &L = a.L;
    const float *lg = a.b.logits;
    const TopkOut tk = wave_topk([&](int e) { return lg[e]; }, L.E, L.K);
    const int lane = threadIdx.x & 63;
    if (lane < L.K) {
        if (a.out_idx) a.out_idx[lane] = tk.idx;
        if (a.out_w) a.out_w[lane] = tk.w;
    }
}

constexpr int DOWN_THREADS = 128;

template <int BITS, int LPR>
__global__ __launch_bounds__(DOWN_THREADS) void k_down(DecArgs a, int nvec) {
    extern __shared__ uint32_t smem[];
    const Layer &L = a.L;
    constexpr int CPC = 128 / BITS;
    const int I = L.I;
    uint32_t *hs = smem;                                    // nvec * I/2 dwords
    float *hsum = (float *)(hs + (int64_t)nvec * I / 2);    // nvec * I/CPC
    float *gsum = hsum + nvec * (I / CPC);                  // I/8 scratch
    for (int v = 0; v < nvec; ++v) {
        const float *hv = a.b.h + (int64_t)v * I;
        stage_vec<BITS>([&](int g, float o[8]) {
            const f32x4 p0 = *(const f32x4 *)(hv + 8 * g);
            const f32x4 p1 = *(const f32x4 *)(hv + 8 * g + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) { o[i] = p0[i]; o[4 + i] = p1[i]; }
        }, I, hs + (int64_t)v * I / 2, hsum + v * (I / CPC), gsum);
    }
    constexpr int RPW = 64 / LPR;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = (blockIdx.x * (DOWN_THREADS / 64) + wave) * RPW + lane / LPR;
    const int nc = n < L.H ? n : L.H - 1;
    float y = 0.0f;
    for (int j = 0; j < L.K; ++j) {                         // ascending expert id
        const int e = a.b.idx[j];
        const RowPtr r = row_of(L.down, e, nc, I, BITS);
        const float p = row_dot<BITS, LPR>(r.codes, r.sc, r.bi, I, lane % LPR,
                                           hs + (int64_t)j * I / 2, hsum + j * (I / CPC));
        y += a.b.w[j] * p;
    }
    if (a.shared) {
        const RowPtr r = row_of(L.s_down, 0, nc, I, BITS);
        y += row_dot<BITS, LPR>(r.codes, r.sc, r.bi, I, lane % LPR,
                                hs + (int64_t)L.K * I / 2, hsum + L.K * (I / CPC));
    }
    if (n < L.H && lane % LPR == 0) {
        if (a.y_dtype == QSMOE_F32) ((float *)a.y)[n] = y;
        else ((uint16_t *)a.y)[n] = f32_to_bf16(y);
    }
}

// lanes sharing one row: the largest power of two <= min(64, 16-byte chunks per row)
template <int BITS>
int lpr_for(int ncols) {
    const int chunks = ncols * BITS / 128;
    int l = 64;
    while (l > chunks) l >>= 1;
    return l;
}

#define QS_DISPATCH_LPR(lpr, ...)                                                           \
    switch (lpr) {                                                                          \
        case 64: { constexpr int LPR = 64; __VA_ARGS__; } break;                            \
        case 32: { constexpr int LPR = 32; __VA_ARGS__; } break;                            \
        case 16: { constexpr int LPR = 16; __VA_ARGS__; } break;                            \
        case 8: { constexpr int LPR = 8; __VA_ARGS__; } break;                              \
        case 4: { constexpr int LPR = 4; __VA_ARGS__; } break;                              \
        default: { constexpr int LPR = 2; __VA_ARGS__; } break;                             \
    }

template <int BITS>
hipError_t router_shared(const DecArgs &a, hipStream_t s) {
    const int lpr = lpr_for<BITS>(a.L.H);
    const int nR = (a.L.E + 3) / 4;
    QS_DISPATCH_LPR(lpr, {
        constexpr int PAIRS = (DEC_THREADS / 64) * (64 / LPR);
        const int nS = a.shared ? (a.L.I + PAIRS - 1) / PAIRS : 0;
        DecArgs b = a;
        b.n_router_blocks = nR;
        hipLaunchKernelGGL((k_router_shared<BITS, LPR>), dim3(nR + nS), dim3(DEC_THREADS), 0, s, b);
    })
    return hipGetLastError();
}

template <int BITS>
hipError_t gate_up(const DecArgs &a, hipStream_t s) {
    const int lpr = lpr_for<BITS>(a.L.H);
    QS_DISPATCH_LPR(lpr, {
        constexpr int PAIRS = (DEC_THREADS / 64) * (64 / LPR);
        const int bpe = (a.L.I + PAIRS - 1) / PAIRS;
        hipLaunchKernelGGL((k_gate_up<BITS, LPR>), dim3(bpe * a.L.K), dim3(DEC_THREADS), 0, s, a);
    })
    return hipGetLastError();
}

template <int BITS>
hipError_t down(const DecArgs &a, hipStream_t s) {
    const int lpr = lpr_for<BITS>(a.L.I);
    const int nvec = a.L.K + (a.shared ? 1 : 0);
    constexpr int CPC = 128 / BITS;
    const size_t lds = (size_t)nvec * a.L.I * 2 + (size_t)nvec * (a.L.I / CPC) * 4 + (a.L.I / 8) * 4;
    QS_DISPATCH_LPR(lpr, {
        constexpr int ROWS = (DOWN_THREADS / 64) * (64 / LPR);
        const int nb = (a.L.H + ROWS - 1) / ROWS;
        hipLaunchKernelGGL((k_down<BITS, LPR>), dim3(nb), dim3(DOWN_THREADS), lds, s, a, nvec);
    })
    return hipGetLastError();
}

DecArgs make_args(const Layer &L, const uint16_t *x, const DecodeBufs &b) {
    DecArgs a;
    a.L = L;
    a.x = x;
    a.b = b;
    a.out_idx = nullptr;
    a.out_w = nullptr;
    a.y = nullptr;
    a.y_dtype = QSMOE_F32;
    a.n_router_blocks = 0;
    a.shared = L.has_shared;
    return a;
}

}  // namespace

hipError_t launch_decode_router_shared(const Layer &L, const uint16_t *x, const DecodeBufs &b,
                                       bool shared, hipStream_t s) {
    DecArgs a = make_args(L, x, b);
    a.shared = shared && L.has_shared;
    return L.bits == 4 ? router_shared<4>(a, s) : router_shared<8>(a, s);
}

hipError_t launch_decode_gate_up(const Layer &L, const uint16_t *x, const DecodeBufs &b,
                                 int32_t *out_idx, float *out_w, hipStream_t s) {
    DecArgs a = make_args(L, x, b);
    a.out_idx = out_idx;
    a.out_w = out_w;
    return L.bits == 4 ? gate_up<4>(a, s) : gate_up<8>(a, s);
}

hipError_t launch_decode_down(const Layer &L, const DecodeBufs &b, void *y, int y_dtype,
                              hipStream_t s) {
    DecArgs a = make_args(L, nullptr, b);
    a.y = y;
    a.y_dtype = y_dtype;
    return L.bits == 4 ? down<4>(a, s) : down<8>(a, s);
}

hipError_t launch_decode_topk(const Layer &L, const DecodeBufs &b, int32_t *out_idx,
                              float *out_w, hipStream_t s) {
    DecArgs a = make_args(L, nullptr, b);
    a.out_idx = out_idx;
    a.out_w = out_w;
    hipLaunchKernelGGL((k_topk_only<4>), dim3(1), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace qs
