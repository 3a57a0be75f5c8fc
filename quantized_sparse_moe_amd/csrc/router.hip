// router.hip -- prefill router (T >= 2): logits, then top-k and per-block expert counts.
//
// [LILY] "Qwen creates three distinct workload shapes": a router scores 256 experts and
// picks eight per token.  [LILY] "Keep expert routing on the GPU": after the choice a
// histogram counts the assignments of every expert; here each 16-token block's counts
// are written by the top-k pass, and the binning pass turns them into offsets.
//
// Logits are a dense [T x H] x [H x E] contraction: bf16 activations against bf16
// router weights on MFMA (v_mfma_f32_16x16x32_bf16, exact products, fp32 accumulation),
// tiled LT tokens x 64 experts per workgroup with both operands staged in LDS, so each
// router row is read once per LT tokens (from L2: the 1 MiB router matrix stays there).
// LT = 32 when 64-token tiles would leave fewer than two workgroups per CU (T = 4096:
// four waves per CU did not hide the latency), else 64.  The workgroups of a token block also write
// the fp16 copy of x (taking K chunks in turn), each group of 8 columns permuted into
// the code order used by the expert GEMMs, and the largest |x| of each token over the
// chunks they wrote.  The top-k pass then gives one wave to each token; it also picks
// the token's range scale 2^a from those maxima (0 for ordinary rows) and, for a row
// outside fp16's range, writes the copy again as x 2^a.
#include "common.h"
#include "internal.h"

namespace qs {

namespace {

constexpr int LE = 64;              // experts per logits tile
constexpr int LK = 128;             // K chunk
constexpr int LPITCH = LK + 8;      // bf16 per LDS row (breaks bank alignment)
constexpr int TK_TOKENS = ROUTER_TOKENS;   // tokens per top-k workgroup (= one binning block)

struct LogitArgs {
    const uint16_t *x;              // [T][H] bf16
    const uint16_t *wr;             // [E][H] bf16
    const float *bias;              // [E] or null
    const uint16_t *gate_w;         // [H] bf16 shared-expert gate, logit column E; or null
    float *logits;                  // [T][LS]
    int LS;                         // logit row stride: E (+ 1 with a gate)
    uint16_t *x16;                  // [T][H] fp16 in code order, or null
    uint32_t *xmax;                 // [T][8] largest |x| (fp32 bits) per token and expert block
    int64_t T;
    int H, E;
};

template <int BITS, int LT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_logits(LogitArgs a) {
    constexpr int TW = LT / 16;                     // 16-token blocks of the tile (2 or 4)
    constexpr int NPW = TW;                         // 16-expert blocks per wave
    __shared__ __attribute__((aligned(16))) uint16_t xa[LT * LPITCH];
    __shared__ __attribute__((aligned(16))) uint16_t wa[LE * LPITCH];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n16 = lane & 15, cg = lane >> 4;
    const int64_t t0 = (int64_t)blockIdx.x * LT;
    const int e0 = blockIdx.y * LE;
    const int H = a.H, E = a.E;
    // staging: thread tid moves chunk (tid % 16) of rows tid / 16 + 16 i of the x tile
    // (i < TW, LT rows) and of the router tile (i < 4, LE rows)
    const int sr = tid >> 4, sc = (tid & 15) * 8;
    int64_t xrow[TW];
    int wrow[4];
#pragma unroll
    for (int i = 0; i < TW; ++i) {
        const int64_t t = t0 + sr + 16 * i;
        xrow[i] = t < a.T ? t : -1;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = e0 + sr + 16 * i;
        wrow[i] = e < a.LS ? e : -1;                        // e = E: the shared gate's row
    }
    // (a chunk past the end of a row, when H % 128 == 64, loads zeros)
    auto load = [&](int kc, u32x4 (&xv)[TW], u32x4 (&wv)[4]) {
        const bool in = kc + sc < H;
#pragma unroll
        for (int i = 0; i < TW; ++i)
            xv[i] = in && xrow[i] >= 0 ? *(const u32x4 *)(a.x + xrow[i] * H + kc + sc) : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            wv[i] = in && wrow[i] >= 0
                        ? *(const u32x4 *)((wrow[i] < E ? a.wr + (int64_t)wrow[i] * H : a.gate_w) + kc + sc)
                        : (u32x4){0u, 0u, 0u, 0u};
    };
    // wave w: tokens 16 (w % TW) .. + 16 against the NPW 16-expert blocks from NPW (w / TW)
    const int tw = wave % TW, eh = wave / TW;
    f32x4 acc[NPW];
#pragma unroll
    for (int n = 0; n < NPW; ++n) acc[n] = (f32x4){0.f, 0.f, 0.f, 0.f};
    uint32_t xm[TW];                                // largest |x| written, per staged row
#pragma unroll
    for (int i = 0; i < TW; ++i) xm[i] = 0u;
    // chunk kc: registers -> LDS (and the fp16 copy of x), then 4 x NPW MFMAs; two chunks
    // are in flight in registers while one is multiplied
    auto step = [&](int kc, const u32x4 (&xv)[TW], const u32x4 (&wv)[4]) __attribute__((always_inline)) {
        // the expert blocks of a token block take turns writing the fp16 copy of x
        const bool write_x16 = a.x16 && (int)((kc / LK) % gridDim.y) == (int)blockIdx.y;
        __syncthreads();                                 // the previous chunk is consumed
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4 *)(wa + (sr + 16 * i) * LPITCH + sc) = wv[i];
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            *(u32x4 *)(xa + (sr + 16 * i) * LPITCH + sc) = xv[i];
            if (write_x16 && xrow[i] >= 0 && kc + sc < H) {   // this chunk's share of the fp16 copy
                u32x4 h;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    xm[i] = max(xm[i], max((xv[i][c] << 16) & 0x7fffffffu, xv[i][c] & 0x7fff0000u));
                    h[c] = pack_f16x2(f32_to_f16_ftz(__uint_as_float(xv[i][c] << 16)),
                                      f32_to_f16_ftz(__uint_as_float(xv[i][c] & 0xffff0000u)));
                }
                *(u32x4 *)(a.x16 + xrow[i] * H + kc + sc) = perm8<BITS>(h);
            }
        }
        __syncthreads();
    };
    auto mult = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < LK / 32; ++s) {
            const bf16x8 A = *(const bf16x8 *)(xa + (tw * 16 + n16) * LPITCH + s * 32 + 8 * cg);
#pragma unroll
            for (int n = 0; n < NPW; ++n) {
                const bf16x8 B = *(const bf16x8 *)(wa + ((NPW * eh + n) * 16 + n16) * LPITCH + s * 32 + 8 * cg);
                acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[n], 0, 0, 0);
            }
        }
    };
    u32x4 xv0[TW], wv0[4], xv1[TW], wv1[4];
    load(0, xv0, wv0);
    if (LK < H) load(LK, xv1, wv1);
    for (int kc = 0; kc < H; kc += 2 * LK) {
        step(kc, xv0, wv0);
        if (kc + 2 * LK < H) load(kc + 2 * LK, xv0, wv0);
        mult();
        if (kc + LK < H) {
            step(kc + LK, xv1, wv1);
            if (kc + 3 * LK < H) load(kc + 3 * LK, xv1, wv1);
            mult();
        }
    }
    // the 16 lanes staging a row hold its maxima: one word per (token, expert block)
    if (a.x16) {
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            uint32_t m = xm[i];
            m = max(m, dpp_u32<0xB1>(m));
            m = max(m, dpp_u32<0x4E>(m));
            m = max(m, dpp_u32<0x141>(m));
            m = max(m, dpp_u32<0x140>(m));
            if ((tid & 15) == 0 && xrow[i] >= 0) a.xmax[xrow[i] * 8 + blockIdx.y] = m;
        }
    }
    // acc[n][r]: token 16 tw + 4 cg + r, expert e0 + 16 (NPW eh + n) + n16
#pragma unroll
    for (int n = 0; n < NPW; ++n) {
        const int e = e0 + 16 * (NPW * eh + n) + n16;
        if (e >= a.LS) continue;
        const float b = (a.bias && e < E) ? a.bias[e] : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t t = t0 + tw * 16 + 4 * cg + r;
            if (t < a.T) a.logits[t * a.LS + e] = acc[n][r] + b;
        }
    }
}

struct TopkArgs {
    const float *logits;            // [T][LS]
    int64_t T;
    int E, K, LS;
    float *sgate;                   // [T] sigmoid of logit column E (gated layers), or null
    int32_t *idx;                   // [T][K]
    float *w;
    int32_t *out_idx;               // optional copies for the caller
    float *out_w;
    int32_t *blkcnt;                // [T / 16][E] or null
    // range scale of the fp16 copy of x (prefill only; x16 null otherwise)
    const uint16_t *x;              // [T][H] bf16
    uint16_t *x16;                  // [T][H] fp16 in code order
    const uint32_t *xmax;           // [T][8]
    int nxmax;                      // expert blocks of the logits grid (words of xmax used)
    int32_t *xexp;                  // [T] the exponent a of each token's copy (x 2^a)
    int H;
};

// One wave per token (4 tokens per wave), 16 tokens per workgroup: the block's expert
// histogram is counted in LDS with integer atomics and written once.
template <int BITS>
__global__ __launch_bounds__(64 * TK_TOKENS) void k_topk(TopkArgs a) {
    __shared__ int hist[256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = a.E, K = a.K;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    // one wave per token: the selection is a chain of dependent single-wave steps, and the
    // SIMD interleaves the chains of the workgroup's waves
    const int64_t t = (int64_t)blockIdx.x * TK_TOKENS + wave;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (t < a.T && lane + 64 * i < E) ? a.logits[t * a.LS + lane + 64 * i] : 0.0f;
    if (t < a.T) {
        if (a.x16) {
            // the token's range scale; a row outside fp16's range is copied again, scaled
            uint32_t m = 0u;
            for (int y = 0; y < a.nxmax; ++y) m = max(m, a.xmax[t * 8 + y]);
            const int xe = range_exp(__uint_as_float(m));
            if (lane == 0) a.xexp[t] = xe;
            if (xe != 0) {
                const float f = exp2i(xe);
                for (int c = lane * 8; c < a.H; c += 512) {
                    const u32x4 xv = *(const u32x4 *)(a.x + t * a.H + c);
                    u32x4 h;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        h[i] = pack_f16x2(f32_to_f16_ftz(__uint_as_float(xv[i] << 16) * f),
                                          f32_to_f16_ftz(__uint_as_float(xv[i] & 0xffff0000u) * f));
                    *(u32x4 *)(a.x16 + t * a.H + c) = perm8<BITS>(h);
                }
            }
        }
        const TopkOut tk = wave_topk_regs(v, E, K);
        if (a.sgate && lane == 0) a.sgate[t] = sigmoid(a.logits[t * a.LS + E]);
        if (lane < K) {
            a.idx[t * K + lane] = tk.idx;
            a.w[t * K + lane] = tk.w;
            if (a.out_idx) a.out_idx[t * K + lane] = tk.idx;
            if (a.out_w) a.out_w[t * K + lane] = tk.w;
            if (a.blkcnt) atomicAdd(&hist[tk.idx], 1);
        }
    }
    __syncthreads();
    if (a.blkcnt && tid < E) a.blkcnt[(int64_t)blockIdx.x * E + tid] = hist[tid];
}

}  // namespace

hipError_t launch_prefill_router(const Layer &L, const uint16_t *x, int64_t T,
                                 const PrefillBufs &b, bool write_x16, int32_t *out_idx,
                                 float *out_w, hipStream_t s) {
    LogitArgs la;
    la.x = x;
    la.wr = L.router_w;
    la.bias = L.router_bias;
    const bool gated = L.shared_gate_w && L.has_shared && write_x16;   // moe_route needs no gate
    la.gate_w = gated ? L.shared_gate_w : nullptr;
    la.LS = L.E + (gated ? 1 : 0);
    la.logits = b.logits;
    la.x16 = write_x16 ? b.x16 : nullptr;
    la.xmax = b.xmax;
    la.T = T;
    la.H = L.H;
    la.E = L.E;
    // 32-token tiles when 64-token ones would not give every CU two workgroups
    const int eblk = (la.LS + LE - 1) / LE;
    const bool small = (T + 63) / 64 * eblk < 2 * n_compute_units();
    const dim3 lgrid((unsigned)(small ? (T + 31) / 32 : (T + 63) / 64), (unsigned)eblk);
    void (*kern)(LogitArgs) = L.bits == 4 ? (small ? k_logits<4, 32> : k_logits<4, 64>)
                                          : (small ? k_logits<8, 32> : k_logits<8, 64>);
    hipLaunchKernelGGL(kern, lgrid, dim3(256), 0, s, la);
    TopkArgs ta;
    ta.logits = b.logits;
    ta.T = T;
    ta.E = L.E;
    ta.K = L.K;
    ta.LS = la.LS;
    ta.sgate = gated ? b.sgate : nullptr;
    ta.idx = b.idx;
    ta.w = b.w;
    ta.out_idx = out_idx;
    ta.out_w = out_w;
    ta.blkcnt = write_x16 ? b.blkcnt : nullptr;
    ta.x = x;
    ta.x16 = write_x16 ? b.x16 : nullptr;
    ta.xmax = b.xmax;
    ta.nxmax = (int)lgrid.y;
    ta.xexp = b.xexp;
    ta.H = L.H;
    const dim3 tgrid((unsigned)((T + TK_TOKENS - 1) / TK_TOKENS));
    if (L.bits == 4)
        hipLaunchKernelGGL((k_topk<4>), tgrid, dim3(64 * TK_TOKENS), 0, s, ta);
    else
        hipLaunchKernelGGL((k_topk<8>), tgrid, dim3(64 * TK_TOKENS), 0, s, ta);
    return hipGetLastError();
}

}  // namespace qs
