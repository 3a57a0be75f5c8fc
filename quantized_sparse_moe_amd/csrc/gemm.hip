// gemm.hip -- grouped expert GEMMs of the prefill path on MFMA (gfx950).
//
// [LILY] "Dequantize weights during matrix multiplication": the quantized weights are
// never expanded in memory; each workgroup dequantizes the small weight tile it is
// about to multiply, straight into MFMA operand registers, with fp32 accumulation.
// [LILY] "Keep expert routing on the GPU" / "Match tile size to expert load": work is
// enumerated as (expert row block, column block) items from the device-side block map.
// [OMLX] "Fusion principle": gate and up rows of one expert are handled by the same
// wave, so SwiGLU is formed in registers and only h leaves the kernel.
//
// Operands: activations fp16 (x copy from the router, h from the gate/up kernel), with
// each group of 8 columns permuted into the code order (see common.h); weights fp16
// w = fma(s, q, b) with q recovered exactly from the codes by the 1024-magic; MFMA
// v_mfma_f32_16x16x32_f16 with fp32 accumulation.  (fp16 rather than bf16 operands:
// at these sizes weights rounded to bf16 leave ~2e-2 x RMS of error in the layer
// output, fp16 ~2e-3; the matrix rate is the same.)
//
// Workgroup = 4 waves, tile = GEMM_BM rows x (4 waves x 64 weight rows).  Lane l of a
// wave owns weight row (l % 16) of each 16-row subtile and columns [32c, 32c+32) of each
// 128-column K step (c = l / 16); the MFMA K slots of lane group c are those columns in
// code order, which the LDS activation tile mirrors.
//
// Modes: 0 = [gate; up] + SwiGLU -> h (routed rows gathered through perm, shared rows
// direct); 1 = routed down projection -> slot[t, j] = w_tj * o (fp16); 2 = shared down
// projection whose epilogue adds the k slots of the token in ascending expert order and
// writes y: a deterministic, atomic-free combine.
#include "common.h"
#include "internal.h"

namespace qs {

namespace {

constexpr int MT = GEMM_MT;
constexpr int BM = GEMM_BM;
constexpr int KT = 128;              // K step
constexpr int APITCH = KT + 8;       // fp16 per LDS row (272 bytes)

struct GemmArgs {
    Layer L;
    int64_t T;
    const uint16_t *x16;             // [T][H] fp16 (permuted)
    uint16_t *h;                     // [(T*K + T)][I] fp16 (permuted)
    const int32_t *perm;
    const Tile *tiles;
    const int32_t *ntiles;
    const float *w;                  // [T*K]
    uint16_t *slot;                  // [T*K][H]
    void *y;
    int y_dtype;
    int nb;                          // column blocks per tile
};

template <int BITS>
__device__ __forceinline__ f16x8 dequant_step(const u32x4 &c0, const u32x4 &c1, int s, f16x2 sc, f16x2 bi) {
    uint32_t m[4];
    if constexpr (BITS == 4) {
        magic_u4(c0[s], m);
    } else {
        const u32x4 &c = (s < 2) ? c0 : c1;
        magic_u8(c[(2 * s) & 3], m);
        magic_u8(c[(2 * s + 1) & 3], m + 2);
    }
    f16x8 out;
    const f16x2 k1024 = (f16x2){(_Float16)1024.0f, (_Float16)1024.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f16x2 q = as_h2(m[i]) - k1024;   // exact
        const f16x2 v = __builtin_elementwise_fma(q, sc, bi);       // one rounding
        out[2 * i] = v[0];
        out[2 * i + 1] = v[1];
    }
    return out;
}

template <int BITS, int MODE>
__global__ __launch_bounds__(256, 2) void k_gemm(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * APITCH];
    const Layer &L = a.L;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int ti = lid / a.nb, nbi = lid % a.nb;
    int tcount, tbase;
    if (MODE == 0) { tbase = 0; tcount = a.ntiles[1]; }
    else if (MODE == 1) { tbase = 0; tcount = a.ntiles[0]; }
    else { tbase = a.ntiles[0]; tcount = a.ntiles[1] - a.ntiles[0]; }
    if (ti >= tcount) return;
    const Tile tile = a.tiles[tbase + ti];
    const int E = L.E, K = L.K, H = L.H, I = L.I;
    const bool shared = tile.expert == E;
    const int64_t e = shared ? 0 : tile.expert;
    const int Kdim = (MODE == 0) ? H : I;
    const int64_t TK = a.T * K;

    // ---- weight rows of this lane (4 subtiles)
    const int n16 = lane & 15, cgrp = lane >> 4;
    const int row_bytes = Kdim * BITS / 8;
    int wrow[4];
    bool wvalid[4];
    const uint8_t *wcodes[4];
    const uint16_t *wsc[4], *wbi[4];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
        QMat m;
        if (MODE == 0) {
            wrow[sub] = nbi * 128 + wave * 32 + (sub & 1) * 16 + n16;
            wvalid[sub] = true;                               // I % 128 == 0
            m = (sub < 2) ? (shared ? L.s_gate : L.gate) : (shared ? L.s_up : L.up);
        } else {
            const int col = nbi * 256 + wave * 64 + sub * 16 + n16;
            wvalid[sub] = col < H;
            wrow[sub] = wvalid[sub] ? col : H - 1;
            m = shared ? L.s_down : L.down;
        }
        const int64_t R = e * m.stride + wrow[sub];
        wcodes[sub] = m.codes + R * row_bytes;
        wsc[sub] = m.scales + R * (Kdim / 64);
        wbi[sub] = m.biases + R * (Kdim / 64);
    }

    // ---- activation rows staged by this thread: rows tid/16 + 16 i, chunk tid % 16
    const int arow0 = tid >> 4, achunk = tid & 15;
    int64_t asrc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int r = arow0 + 16 * i;
        int64_t src = -1;
        if (r < tile.nrows) {
            if (MODE == 0) {
                const int64_t t = shared ? (tile.row0 - TK + r) : (a.perm[tile.row0 + r] / K);
                src = t * H;
            } else {
                src = (int64_t)(tile.row0 + r) * I;
            }
        }
        asrc[i] = src;
    }
    const uint16_t *abase = (MODE == 0) ? a.x16 : a.h;

    f32x4 acc[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[i][n] = (f32x4){0.f, 0.f, 0.f, 0.f};

    for (int kt = 0; kt < Kdim; kt += KT) {
        // weight codes, scales and biases of this K step (issued first: longest latency)
        u32x4 c0[4], c1[4];
        f16x2 sc[4], bi[4];
        const int kc = kt + 32 * cgrp;
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
            const uint8_t *p = wcodes[sub] + kc * BITS / 8;
            c0[sub] = __builtin_nontemporal_load((const u32x4 *)p);
            if (BITS == 8) c1[sub] = __builtin_nontemporal_load((const u32x4 *)(p + 16));
            else c1[sub] = c0[sub];
            const uint16_t s16 = wsc[sub][kc >> 6], b16 = wbi[sub][kc >> 6];
            const _Float16 sv = __builtin_bit_cast(_Float16, s16), bv = __builtin_bit_cast(_Float16, b16);
            sc[sub] = (f16x2){sv, sv};
            bi[sub] = (f16x2){bv, bv};
        }
        // activation tile -> LDS
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            u32x4 v = (u32x4){0u, 0u, 0u, 0u};
            if (asrc[i] >= 0) v = *(const u32x4 *)(abase + asrc[i] + kt + achunk * 8);
            *(u32x4 *)(As + (arow0 + 16 * i) * APITCH + achunk * 8) = v;
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            f16x8 B[4];
#pragma unroll
            for (int sub = 0; sub < 4; ++sub) B[sub] = dequant_step<BITS>(c0[sub], c1[sub], s, sc[sub], bi[sub]);
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const f16x8 A = *(const f16x8 *)(As + (i * 16 + n16) * APITCH + 32 * cgrp + 8 * s);
#pragma unroll
                for (int sub = 0; sub < 4; ++sub)
                    acc[i][sub] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B[sub], acc[i][sub], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // ---- epilogues.  acc[i][sub][r]: row i*16 + 4*cgrp + r, weight row wrow[sub]
    if (MODE == 0) {
        uint16_t *hout = a.h;
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                const int hcol = wrow[sub];
                const int pcol = (hcol & ~7) | perm_pos<BITS>(hcol & 7);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = i * 16 + 4 * cgrp + r;
                    if (row < tile.nrows) {
                        const float hv = silu(acc[i][sub][r]) * acc[i][sub + 2][r];
                        hout[(int64_t)(tile.row0 + row) * I + pcol] =
                            __builtin_bit_cast(uint16_t, f32_to_f16_ftz(hv));
                    }
                }
            }
    } else if (MODE == 1) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = i * 16 + 4 * cgrp + r;
                if (row < tile.nrows) {
                    const int64_t p = a.perm[tile.row0 + row];
                    const float wv = a.w[p];
#pragma unroll
                    for (int sub = 0; sub < 4; ++sub)
                        if (wvalid[sub])
                            a.slot[p * H + wrow[sub]] =
                                __builtin_bit_cast(uint16_t, (_Float16)(acc[i][sub][r] * wv));
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = i * 16 + 4 * cgrp + r;
                if (row < tile.nrows) {
                    const int64_t t = tile.row0 - TK + row;
#pragma unroll
                    for (int sub = 0; sub < 4; ++sub)
                        if (wvalid[sub]) {
                            const int col = wrow[sub];
                            float sum = 0.0f;
                            for (int j = 0; j < K; ++j)             // ascending expert id
                                sum += f16_to_f32(a.slot[(t * K + j) * H + col]);
                            sum += acc[i][sub][r];                    // shared expert last
                            if (a.y_dtype == QSMOE_F32) ((float *)a.y)[t * H + col] = sum;
                            else ((uint16_t *)a.y)[t * H + col] = f32_to_bf16(sum);
                        }
                }
            }
    }
}

// routed-only layers (no shared expert): y = sum of the k slots, fixed order
__global__ __launch_bounds__(256) void k_combine_routed(const uint16_t *__restrict__ slot, void *y,
                                                        int y_dtype, int64_t T, int K, int H) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= T * H) return;
    const int64_t t = i / H, col = i % H;
    float sum = 0.0f;
    for (int j = 0; j < K; ++j) sum += f16_to_f32(slot[(t * K + j) * H + col]);
    if (y_dtype == QSMOE_F32) ((float *)y)[i] = sum;
    else ((uint16_t *)y)[i] = f32_to_bf16(sum);
}

inline int round8(int64_t n) { return (int)(((n + 7) / 8) * 8); }

template <int BITS>
hipError_t gemms(GemmArgs a, hipStream_t s) {
    const Layer &L = a.L;
    const int64_t maxr = prefill_max_routed_tiles(a.T, L.K, L.E);
    const int64_t maxs = L.has_shared ? (a.T + GEMM_BM - 1) / GEMM_BM : 0;
    // [gate; up] + SwiGLU over routed and shared tiles
    a.nb = L.I / 128;
    hipLaunchKernelGGL((k_gemm<BITS, 0>), dim3(round8((maxr + maxs) * a.nb)), dim3(256), 0, s, a);
    // routed down -> slots
    a.nb = (L.H + 255) / 256;
    hipLaunchKernelGGL((k_gemm<BITS, 1>), dim3(round8(maxr * a.nb)), dim3(256), 0, s, a);
    if (L.has_shared) {
        hipLaunchKernelGGL((k_gemm<BITS, 2>), dim3(round8(maxs * a.nb)), dim3(256), 0, s, a);
    } else {
        const int64_t n = a.T * L.H;
        hipLaunchKernelGGL(k_combine_routed, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           a.slot, a.y, a.y_dtype, a.T, L.K, L.H);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_gemms(const Layer &L, int64_t T, const PrefillBufs &b, void *y,
                                int y_dtype, hipStream_t s) {
    GemmArgs a;
    a.L = L;
    a.T = T;
    a.x16 = b.x16;
    a.h = b.h;
    a.perm = b.perm;
    a.tiles = b.tiles;
    a.ntiles = b.ntiles;
    a.w = b.w;
    a.slot = b.slot;
    a.y = y;
    a.y_dtype = y_dtype;
    a.nb = 1;
    return L.bits == 4 ? gemms<4>(a, s) : gemms<8>(a, s);
}

}  // namespace qs
