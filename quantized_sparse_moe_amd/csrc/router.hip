// router.hip -- prefill router (T >= 2): logits, top-k, per-block expert counts.
//
// [LILY] "Qwen creates three distinct workload shapes": a router scores 256 experts and
// picks eight per token.  [LILY] "Keep expert routing on the GPU": after the choice a
// histogram counts the assignments of every expert; here each 16-token workgroup writes
// the counts of its block, which the binning pass turns into offsets.
//
// Logits are a dense [T x H] x [H x E] contraction: bf16 activations against bf16
// router weights on MFMA (v_mfma_f32_16x16x32_bf16, exact products, fp32 accumulation).
// A workgroup owns 16 tokens and all experts (each wave 64 of them), so the top-k of a
// token is taken straight from LDS.  The same pass writes an fp16 copy of x with each
// group of 8 columns permuted into the code order used by the expert GEMMs.
#include "common.h"
#include "internal.h"

namespace qs {

namespace {

constexpr int RT = ROUTER_TOKENS;   // tokens per workgroup (one 16-row MFMA subtile)
constexpr int RKC = 1024;           // columns of x staged per chunk
constexpr int RPITCH = RKC + 8;     // bf16 elements per LDS row (breaks bank alignment)
constexpr int RU = 2;               // 32-column K slices per batch of router-weight loads

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

// One workgroup = RT tokens x all experts; wave w owns experts 64w .. 64w+63.  x is
// staged a chunk of RKC columns at a time with every load of the chunk in flight at
// once (the fp16 copy for the expert GEMMs is written from the same registers); router
// weights stream from L2 straight into MFMA operands, RU K slices per batch of loads.
template <int BITS>
__global__ __launch_bounds__(256) void k_router(RouterArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t xa[RT * RPITCH];
    __shared__ float lg[RT * 257];
    __shared__ int hist[256];
    const Layer &L = a.L;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * RT;
    const int H = L.H, E = L.E;
    const int n16 = lane & 15, cg = lane >> 4;

    f32x4 acc[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[n] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const uint16_t *wrow[4];
    bool wlive[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const int e = wave * 64 + n * 16 + n16;
        wlive[n] = e < E;
        wrow[n] = L.router_w + (int64_t)(wlive[n] ? e : 0) * H + 8 * cg;
    }

    for (int kc = 0; kc < H; kc += RKC) {
        const int kw = (H - kc) < RKC ? (H - kc) : RKC;          // multiple of 128
        // stage: RT rows x kw columns, 16 bytes per item, all loads first
        constexpr int PER = RT * RKC / 8 / 256;                    // items per thread (8)
        u32x4 v[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = tid + 256 * i, r = q / (RKC / 8), cc = q % (RKC / 8);
            const int64_t t = t0 + r;
            v[i] = (u32x4){0u, 0u, 0u, 0u};
            if (t < a.T && cc * 8 < kw) v[i] = *(const u32x4 *)(a.x + t * H + kc + cc * 8);
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = tid + 256 * i, r = q / (RKC / 8), cc = q % (RKC / 8);
            const int64_t t = t0 + r;
            *(u32x4 *)(xa + r * RPITCH + cc * 8) = v[i];
            if (a.x16 && t < a.T && cc * 8 < kw) {
                u32x4 h;
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    h[c] = pack_f16x2(f32_to_f16_ftz(__uint_as_float(v[i][c] << 16)),
                                      f32_to_f16_ftz(__uint_as_float(v[i][c] & 0xffff0000u)));
                *(u32x4 *)(a.x16 + t * H + kc + cc * 8) = perm8<BITS>(h);
            }
        }
        __syncthreads();
        // router-weight fragments of RU K slices per batch; the next batch's loads are in
        // flight while the current one is multiplied (kw / 32 is a multiple of RU)
        auto load_b = [&](int s0, bf16x8 (&B)[RU][4]) {
#pragma unroll
            for (int u = 0; u < RU; ++u)
#pragma unroll
                for (int n = 0; n < 4; ++n) B[u][n] = *(const bf16x8 *)(wrow[n] + kc + (s0 + u) * 32);
        };
        auto mma = [&](int s0, const bf16x8 (&B)[RU][4]) {
#pragma unroll
            for (int u = 0; u < RU; ++u) {
                const bf16x8 A = *(const bf16x8 *)(xa + n16 * RPITCH + (s0 + u) * 32 + 8 * cg);
#pragma unroll
                for (int n = 0; n < 4; ++n)
                    acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, wlive[n] ? B[u][n] : (bf16x8){}, acc[n], 0, 0, 0);
            }
        };
        bf16x8 B0[RU][4], B1[RU][4];
        const int nsub = kw / 32;
        load_b(0, B0);
        for (int s0 = 0; s0 < nsub; s0 += 2 * RU) {
            if (s0 + RU < nsub) load_b(s0 + RU, B1);
            mma(s0, B0);
            if (s0 + RU < nsub) {
                if (s0 + 2 * RU < nsub) load_b(s0 + 2 * RU, B0);
                mma(s0 + RU, B1);
            }
        }
        __syncthreads();
    }
    // logits -> LDS (+ bias).  acc[n][r]: token 4*cg + r, expert 64*wave + 16*n + n16
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const int e = wave * 64 + n * 16 + n16;
        const float bias = (e < E && L.router_bias) ? L.router_bias[e] : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (e < E) lg[(4 * cg + r) * 257 + e] = acc[n][r] + bias;
    }
    hist[tid] = 0;
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
