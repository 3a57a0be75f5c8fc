// router.hip -- prefill router (T >= 2): logits, top-k, per-block expert counts.
//
// [LILY] "Qwen creates three distinct workload shapes": a router scores 256 experts and
// picks eight per token.  [LILY] "Keep expert routing on the GPU": after the choice a
// histogram counts the assignments of every expert; here each 32-token workgroup writes
// the counts of its block, which the binning pass turns into offsets.
//
// Logits are a dense [T x H] x [H x E] contraction: bf16 activations against bf16
// router weights on MFMA (v_mfma_f32_16x16x32_bf16, exact products, fp32 accumulation).
// A workgroup owns 32 tokens and all experts (each wave 64 of them), so the top-k of a
// token is taken straight from LDS.  The same pass writes an fp16 copy of x with each
// group of 8 columns permuted into the code order used by the expert GEMMs.
#include "common.h"
#include "internal.h"

namespace qs {

namespace {

constexpr int RT = ROUTER_TOKENS;   // tokens per workgroup
constexpr int RKT = 256;            // K tile (columns of x staged per step)
constexpr int RPITCH = RKT + 8;     // bf16 elements per LDS row (breaks bank alignment)

struct RouterArgs {
    Layer L;
    const uint16_t *x;
    int64_t T;
    uint16_t *x16;
    int32_t *idx;
    float *w;
    int32_t *blkcnt;
    int32_t *out_idx;
    float *out_w;
};

template <int BITS>
__global__ __launch_bounds__(256) void k_router(RouterArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t xa[RT * RPITCH];
    __shared__ float lg[RT * 257];
    __shared__ int hist[256];
    const Layer &L = a.L;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * RT;
    const int H = L.H, E = L.E;

    f32x4 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[i][n] = (f32x4){0.f, 0.f, 0.f, 0.f};

    for (int kt = 0; kt < H; kt += RKT) {
        const int kw = (H - kt) < RKT ? (H - kt) : RKT;     // H % 128 == 0
        for (int q = tid; q < RT * (RKT / 8); q += 256) {
            const int r = q / (RKT / 8), cc = q % (RKT / 8);
            const int64_t t = t0 + r;
            u32x4 v = (u32x4){0u, 0u, 0u, 0u};
            if (t < a.T && cc * 8 < kw) {
                v = *(const u32x4 *)(a.x + t * H + kt + cc * 8);
                if (a.x16) {
                    u32x4 h;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        h[i] = pack_f16x2(f32_to_f16_ftz(__uint_as_float(v[i] << 16)),
                                          f32_to_f16_ftz(__uint_as_float(v[i] & 0xffff0000u)));
                    *(u32x4 *)(a.x16 + t * H + kt + cc * 8) = perm8<BITS>(h);
                }
            }
            *(u32x4 *)(xa + r * RPITCH + cc * 8) = v;
        }
        __syncthreads();
        for (int s = 0; s < kw / 32; ++s) {
            bf16x8 A[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                A[i] = *(const bf16x8 *)(xa + (i * 16 + (lane & 15)) * RPITCH + s * 32 + 8 * (lane >> 4));
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const int e = wave * 64 + n * 16 + (lane & 15);
                bf16x8 B;
                if (e < E)
                    B = *(const bf16x8 *)(L.router_w + (int64_t)e * H + kt + s * 32 + 8 * (lane >> 4));
                else
                    B = (bf16x8){};
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    acc[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i], B, acc[i][n], 0, 0, 0);
            }
        }
        __syncthreads();
    }
    // logits -> LDS (+ bias)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int e = wave * 64 + n * 16 + (lane & 15);
            const float bias = (e < E && L.router_bias) ? L.router_bias[e] : 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = i * 16 + 4 * (lane >> 4) + r;
                if (e < E) lg[row * 257 + e] = acc[i][n][r] + bias;
            }
        }
    for (int e = tid; e < 256; e += 256) hist[e] = 0;
    __syncthreads();
    for (int r = wave; r < RT; r += 4) {
        const int64_t t = t0 + r;
        if (t >= a.T) break;
        const float *row = lg + r * 257;
        const TopkOut tk = wave_topk([&](int e) { return row[e]; }, E, L.K);
        if (lane < L.K) {
            a.idx[t * L.K + lane] = tk.idx;
            a.w[t * L.K + lane] = tk.w;
            if (a.out_idx) a.out_idx[t * L.K + lane] = tk.idx;
            if (a.out_w) a.out_w[t * L.K + lane] = tk.w;
            if (a.blkcnt) atomicAdd(&hist[tk.idx], 1);     // integer LDS histogram
        }
    }
    __syncthreads();
    if (a.blkcnt)
        for (int e = tid; e < E; e += 256) a.blkcnt[(int64_t)blockIdx.x * E + e] = hist[e];
}

}  // namespace

hipError_t launch_prefill_router(const Layer &L, const uint16_t *x, int64_t T,
                                 const PrefillBufs &b, bool write_x16, int32_t *out_idx,
                                 float *out_w, hipStream_t s) {
    RouterArgs a;
    a.L = L;
    a.x = x;
    a.T = T;
    a.x16 = write_x16 ? b.x16 : nullptr;
    a.idx = b.idx;
    a.w = b.w;
    a.blkcnt = write_x16 ? b.blkcnt : nullptr;
    a.out_idx = out_idx;
    a.out_w = out_w;
    const int nblk = (int)((T + RT - 1) / RT);
    if (L.bits == 4)
        hipLaunchKernelGGL((k_router<4>), dim3(nblk), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((k_router<8>), dim3(nblk), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace qs
