// q8.hip -- dense Q8_0 decode GEMV over 16-row packed tiles, and the load-time packer.
//
// [EMBER] packed 16-row tile: rows are packed 16 at a time; for each block of 32 input
// columns, the bytes of the same 4 columns of the 16 rows sit next to each other
// (eight 64-byte groups), followed by the 16 fp16 scales -- 544 bytes, the size of 16
// ordinary Q8_0 blocks.  On x86 this lets one VNNI step broadcast 4 activation bytes
// against a 64-byte weight group.  On gfx950 the same layout makes a wave's 16-byte loads
// contiguous runs of whole groups: k_q8_gemv_wide (many panels) and k_q8_gemv_part (few
// panels, two workgroups per panel) read tiles 16 bytes per lane -- 4 columns of 4 rows --
// and, beside each chunk, the 4 activations it multiplies; k_q8_gemv (any K) reads 4 bytes
// per lane against a copy of x staged in LDS.
//
// Codes are widened exactly: (q ^ 0x80) is q + 128 as an unsigned byte, which the
// byte-to-float conversion turns into fp32 in one instruction; the +128 is removed per
// lane with the sum of the activations the lane multiplies.
//
// [EMBER] also quantizes the activation once (Q8_0 blocks) for all the projections that
// read it; k_q8_quantize_x and k_q8_gemv_q8x are that variant, with exact int8 dot
// products.
#include "common.h"
#include "internal.h"

namespace qs {

namespace {

constexpr int Q8_THREADS = 512;           // 8 waves share one 16-row panel (split-K)
constexpr int Q8_WAVES = Q8_THREADS / 64;
constexpr int TILE = 544;

// byte N of p as fp32 (selected as a single v_cvt_f32_ubyteN)
template <int N>
__device__ __forceinline__ float ubyte(uint32_t p) { return (float)((p >> (8 * N)) & 0xffu); }

template <int UNROLL>
__global__ __launch_bounds__(Q8_THREADS) void k_q8_gemv(const uint8_t *__restrict__ tiles, int64_t K,
                                                        const uint16_t *__restrict__ x, void *y,
                                                        int y_dtype) {
    extern __shared__ float q8s[];
    const int nb = (int)(K / 32);
    float *xl = q8s;                      // [nb*4][8]
    float *x8 = q8s + (int64_t)nb * 32;   // [nb*4]
    __shared__ float red[Q8_WAVES][16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // stage x: slot (b, j) holds x[32b+4j .. +4] and x[32b+16+4j .. +4]
    for (int sl = tid; sl < nb * 4; sl += Q8_THREADS) {
        const int b = sl >> 2, j = sl & 3;
        const uint2 lo = *(const uint2 *)(x + 32 * b + 4 * j);
        const uint2 hi = *(const uint2 *)(x + 32 * b + 16 + 4 * j);
        float v[8];
        v[0] = __uint_as_float(lo.x << 16); v[1] = __uint_as_float(lo.x & 0xffff0000u);
        v[2] = __uint_as_float(lo.y << 16); v[3] = __uint_as_float(lo.y & 0xffff0000u);
        v[4] = __uint_as_float(hi.x << 16); v[5] = __uint_as_float(hi.x & 0xffff0000u);
        v[6] = __uint_as_float(hi.y << 16); v[7] = __uint_as_float(hi.y & 0xffff0000u);
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s += v[i];
        *(f32x4 *)(xl + 8 * sl) = (f32x4){v[0], v[1], v[2], v[3]};
        *(f32x4 *)(xl + 8 * sl + 4) = (f32x4){v[4], v[5], v[6], v[7]};
        x8[sl] = s;
    }
    __syncthreads();

    const int r = lane & 15, j = lane >> 4;
    const uint8_t *panel = tiles + (int64_t)blockIdx.x * nb * TILE;
    float acc = 0.0f;
    int b = wave;
    for (; b + (UNROLL - 1) * Q8_WAVES < nb; b += UNROLL * Q8_WAVES) {
        uint32_t w0[UNROLL], w1[UNROLL];
        uint16_t dd[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const uint8_t *t = panel + (int64_t)(b + u * Q8_WAVES) * TILE;
            w0[u] = __builtin_nontemporal_load((const uint32_t *)(t + 64 * j + 4 * r));
            w1[u] = __builtin_nontemporal_load((const uint32_t *)(t + 64 * (j + 4) + 4 * r));
            dd[u] = __builtin_nontemporal_load((const uint16_t *)(t + 512 + 2 * r));
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int sl = (b + u * Q8_WAVES) * 4 + j;
            const f32x4 xa = *(const f32x4 *)(xl + 8 * sl);
            const f32x4 xb = *(const f32x4 *)(xl + 8 * sl + 4);
            const uint32_t p0 = w0[u] ^ 0x80808080u, p1 = w1[u] ^ 0x80808080u;
            float s = 0.0f;
            s = __builtin_fmaf(ubyte<0>(p0), xa[0], s);
            s = __builtin_fmaf(ubyte<1>(p0), xa[1], s);
            s = __builtin_fmaf(ubyte<2>(p0), xa[2], s);
            s = __builtin_fmaf(ubyte<3>(p0), xa[3], s);
            s = __builtin_fmaf(ubyte<0>(p1), xb[0], s);
            s = __builtin_fmaf(ubyte<1>(p1), xb[1], s);
            s = __builtin_fmaf(ubyte<2>(p1), xb[2], s);
            s = __builtin_fmaf(ubyte<3>(p1), xb[3], s);
            acc = __builtin_fmaf(f16_to_f32(dd[u]), s - 128.0f * x8[sl], acc);
        }
    }
    for (; b < nb; b += Q8_WAVES) {
        const uint8_t *t = panel + (int64_t)b * TILE;
        const uint32_t p0 = *(const uint32_t *)(t + 64 * j + 4 * r) ^ 0x80808080u;
        const uint32_t p1 = *(const uint32_t *)(t + 64 * (j + 4) + 4 * r) ^ 0x80808080u;
        const uint16_t d = *(const uint16_t *)(t + 512 + 2 * r);
        const int sl = b * 4 + j;
        const f32x4 xa = *(const f32x4 *)(xl + 8 * sl);
        const f32x4 xb = *(const f32x4 *)(xl + 8 * sl + 4);
        float s = 0.0f;
        s = __builtin_fmaf(ubyte<0>(p0), xa[0], s);
        s = __builtin_fmaf(ubyte<1>(p0), xa[1], s);
        s = __builtin_fmaf(ubyte<2>(p0), xa[2], s);
        s = __builtin_fmaf(ubyte<3>(p0), xa[3], s);
        s = __builtin_fmaf(ubyte<0>(p1), xb[0], s);
        s = __builtin_fmaf(ubyte<1>(p1), xb[1], s);
        s = __builtin_fmaf(ubyte<2>(p1), xb[2], s);
        s = __builtin_fmaf(ubyte<3>(p1), xb[3], s);
        acc = __builtin_fmaf(f16_to_f32(d), s - 128.0f * x8[sl], acc);
    }
    // lanes r, r+16, r+32, r+48 hold row r of this wave's blocks
    acc += __shfl_xor(acc, 16, 64);
    acc += __shfl_xor(acc, 32, 64);
    if (lane < 16) red[wave][lane] = acc;
    __syncthreads();
    if (tid < 16) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < Q8_WAVES; ++w) s += red[w][tid];
        const int64_t n = (int64_t)blockIdx.x * 16 + tid;
        if (y_dtype == MOE_F32) ((float *)y)[n] = s;
        else ((uint16_t *)y)[n] = f32_to_bf16(s);
    }
}

// Many panels: one workgroup per 16-row panel, 16-byte loads and every tile of the wave in
// flight at once.  A wave reads two consecutive tiles per instruction: lane (t, g, q) =
// (lane >> 5, (lane >> 2) & 7, lane & 3) takes bytes 64 g + 16 q of tile t -- the 4 columns
// of group g for rows 4q .. 4q+3 -- the fp16 scales of those rows, and the 4 activations
// the chunk multiplies (8 bytes through the caches: every wave reads the same x, so no
// staged copy is waited for).  A wave owns PPW tile pairs (nb = 2 PPW WAVES).  Each lane
// keeps four row sums; the 16 lanes of a row quad are reduced across the wave, then the
// waves across LDS.
template <int PPW, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_q8_gemv_wide(const uint8_t *__restrict__ tiles, int64_t K,
                                                                const uint16_t *__restrict__ x, void *y, int y_dtype) {
    constexpr int NB = 2 * PPW * WAVES;                 // blocks of 32 columns (K / 32)
    __shared__ float red[WAVES][16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = lane & 3, g = (lane >> 2) & 7, tt = lane >> 5;
    const uint8_t *panel = tiles + (int64_t)blockIdx.x * NB * TILE;
    u32x4 c[PPW];
    uint64_t sc[PPW], xv[PPW];
#pragma unroll
    for (int u = 0; u < PPW; ++u) {
        const int b = 2 * (wave + u * WAVES) + tt;
        const uint8_t *t = panel + (int64_t)b * TILE;
        c[u] = __builtin_nontemporal_load((const u32x4 *)(t + 64 * g + 16 * q));
        sc[u] = __builtin_nontemporal_load((const uint64_t *)(t + 512 + 8 * q));
        xv[u] = *(const uint64_t *)(x + 32 * b + 4 * g);
    }
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < PPW; ++u) {
        const uint32_t lo = (uint32_t)xv[u], hi = (uint32_t)(xv[u] >> 32);
        const float x0 = __uint_as_float(lo << 16), x1 = __uint_as_float(lo & 0xffff0000u);
        const float x2 = __uint_as_float(hi << 16), x3 = __uint_as_float(hi & 0xffff0000u);
        const float x4 = 128.0f * ((x0 + x1) + (x2 + x3));
        const uint32_t d2[2] = {(uint32_t)sc[u], (uint32_t)(sc[u] >> 32)};
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const uint32_t p = c[u][rr] ^ 0x80808080u;
            float s = ubyte<0>(p) * x0;
            s = __builtin_fmaf(ubyte<1>(p), x1, s);
            s = __builtin_fmaf(ubyte<2>(p), x2, s);
            s = __builtin_fmaf(ubyte<3>(p), x3, s);
            const float d = f16_to_f32((uint16_t)(d2[rr >> 1] >> (16 * (rr & 1))));
            acc[rr] = __builtin_fmaf(d, s - x4, acc[rr]);
        }
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        float a = acc[rr];
        a += __shfl_xor(a, 4, 64);
        a += __shfl_xor(a, 8, 64);
        a += __shfl_xor(a, 16, 64);
        a += __shfl_xor(a, 32, 64);
        acc[rr] = a;
    }
    if (lane < 4) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) red[wave][4 * lane + rr] = acc[rr];
    }
    __syncthreads();
    if (tid < 16) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) s += red[w][tid];
        const int64_t n = (int64_t)blockIdx.x * 16 + tid;
        if (y_dtype == MOE_F32) ((float *)y)[n] = s;
        else ((uint16_t *)y)[n] = f32_to_bf16(s);
    }
}

// Few panels: PARTS workgroups per panel (two; four measured slower), each taking
// 16 / PARTS of its 16 rows over the whole row length, so that PARTS times the compute
// units read and no partial sums need combining.  Row quad rq's 16 bytes of group g are chunk 4 g + rq of a tile;
// lane (t, g, q) = (lane / LT, (lane / QL) % 8, lane % QL), with QL = 4 / PARTS quads per
// workgroup and LT = 8 QL lanes per tile, takes chunk 4 g + QL part + q of tile t (TPI =
// 64 / LT consecutive tiles per 16-byte load), that quad's fp16 scales, and the 4
// activations the chunk multiplies (8 bytes through the caches: every wave and every part
// reads the same x, and nothing waits for a staged copy).  The parts of a panel run on one
// XCD (workgroups b, b + 8, ... share b % 8), so each line is fetched into its L2 once.
// A wave owns QPW groups of TPI tiles (nb = TPI QPW Q8_WAVES), all loads in flight at once.
template <int QPW, int PARTS>
__global__ __launch_bounds__(Q8_THREADS) void k_q8_gemv_part(const uint8_t *__restrict__ tiles, int64_t K,
                                                             const uint16_t *__restrict__ x, void *y, int y_dtype) {
    constexpr int QL = 4 / PARTS, LT = 8 * QL, TPI = 64 / LT, PLOG = PARTS == 4 ? 2 : 1;
    constexpr int NB = TPI * QPW * Q8_WAVES;                          // blocks of 32 columns (K / 32)
    __shared__ float red[Q8_WAVES][16 / PARTS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = lane % QL, g = (lane / QL) & 7, tt = lane / LT;
    const int bid = blockIdx.x, part = (bid >> 3) & (PARTS - 1), panel = (bid >> (3 + PLOG)) * 8 + (bid & 7);
    const int rq = QL * part + q;                                     // rows 4 rq .. 4 rq + 3
    const uint8_t *pnl = tiles + (int64_t)panel * NB * TILE;
    u32x4 c[QPW];
    uint64_t sc[QPW], xv[QPW];
#pragma unroll
    for (int u = 0; u < QPW; ++u) {
        const int b = TPI * (wave + u * Q8_WAVES) + tt;                // this lane's block of 32 columns
        const uint8_t *t = pnl + (int64_t)b * TILE;
        c[u] = __builtin_nontemporal_load((const u32x4 *)(t + 64 * g + 16 * rq));
        sc[u] = __builtin_nontemporal_load((const uint64_t *)(t + 512 + 8 * rq));
        xv[u] = *(const uint64_t *)(x + 32 * b + 4 * g);
    }
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < QPW; ++u) {
        const uint32_t lo = (uint32_t)xv[u], hi = (uint32_t)(xv[u] >> 32);
        const float x0 = __uint_as_float(lo << 16), x1 = __uint_as_float(lo & 0xffff0000u);
        const float x2 = __uint_as_float(hi << 16), x3 = __uint_as_float(hi & 0xffff0000u);
        const float x4 = 128.0f * ((x0 + x1) + (x2 + x3));
        const uint32_t d2[2] = {(uint32_t)sc[u], (uint32_t)(sc[u] >> 32)};
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const uint32_t p = c[u][rr] ^ 0x80808080u;
            float s = ubyte<0>(p) * x0;
            s = __builtin_fmaf(ubyte<1>(p), x1, s);
            s = __builtin_fmaf(ubyte<2>(p), x2, s);
            s = __builtin_fmaf(ubyte<3>(p), x3, s);
            const float d = f16_to_f32((uint16_t)(d2[rr >> 1] >> (16 * (rr & 1))));
            acc[rr] = __builtin_fmaf(d, s - x4, acc[rr]);
        }
    }
    // the lanes of one quad (all lane bits but q's) in a fixed butterfly, then the waves
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        float a = acc[rr];
#pragma unroll
        for (int m = QL; m < 64; m <<= 1) a += __shfl_xor(a, m, 64);
        acc[rr] = a;
    }
    if (lane < QL) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) red[wave][4 * lane + rr] = acc[rr];
    }
    __syncthreads();
    if (tid < 16 / PARTS) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < Q8_WAVES; ++w) s += red[w][tid];
        const int64_t n = (int64_t)panel * 16 + (16 / PARTS) * part + tid;
        if (y_dtype == MOE_F32) ((float *)y)[n] = s;
        else ((uint16_t *)y)[n] = f32_to_bf16(s);
    }
}

// the activation quantizer's scale and code (one definition for both kernels below)
__device__ __forceinline__ float q8x_scale(float amax) { return amax / 127.0f; }
__device__ __forceinline__ int8_t q8x_code(float v, float d) {
    const float r = d != 0.0f ? roundf(v / d) : 0.0f;
    return (int8_t)fminf(fmaxf(r, -127.0f), 127.0f);
}

// [EMBER] one activation quantization shared by the projections that read a vector:
// x (bf16) -> Q8_0 blocks of 32, split into int8 codes [K] and fp16 scales [K/32].
// d = max|x| / 127 in binary32 (IEEE division), stored as fp16 (round to nearest even);
// q = x / d (binary32, the unrounded d) rounded half away from zero, clamped to
// [-127, 127]; an all-zero block gets d = 0 and zero codes.  One thread per value, 32
// lanes per block.
__global__ __launch_bounds__(256) void k_q8_quantize_x(const uint16_t *__restrict__ x, int64_t K,
                                                       int8_t *__restrict__ xq, uint16_t *__restrict__ xd) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool live = i < K;
    const float v = live ? __uint_as_float((uint32_t)x[i] << 16) : 0.0f;
    float amax = fabsf(v);
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 32));
    const float d = q8x_scale(amax);
    if (live) {
        xq[i] = q8x_code(v, d);
        if ((i & 31) == 0) xd[i >> 5] = __builtin_bit_cast(uint16_t, (_Float16)d);
    }
}

// Q8_0 GEMV with a Q8_0 activation: the tile walk of k_q8_gemv, the products as exact
// 4-way int8 dot products (v_dot4_i32_i8) of a lane's 8 codes, scaled once per lane and
// block by dw * dx (both fp16, so their product is exact in fp32).
// QUANT: the workgroup quantizes x (bf16) itself while staging it, with the arithmetic
// of k_q8_quantize_x (the same codes and scales, bit for bit),
// instead of reading codes a separate launch wrote
template <int UNROLL, bool QUANT>
__global__ __launch_bounds__(Q8_THREADS) void k_q8_gemv_q8x(const uint8_t *__restrict__ tiles, int64_t K,
                                                            const int8_t *__restrict__ xq,
                                                            const uint16_t *__restrict__ xd,
                                                            const uint16_t *__restrict__ x, void *y,
                                                            int y_dtype) {
    extern __shared__ uint32_t q8x[];
    const int nb = (int)(K / 32);
    uint32_t *xl = q8x;                              // [nb*4][2]: codes 32b+4j.. and 32b+16+4j..
    float *dl = (float *)(q8x + (int64_t)nb * 8);    // [nb]
    __shared__ float red[Q8_WAVES][16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if constexpr (QUANT) {
        // one slot (8 values) per thread, the 4 slots of a block in 4 adjacent lanes
        for (int sl0 = 0; sl0 < nb * 4; sl0 += Q8_THREADS) {
            const int sl = sl0 + tid;
            const bool live = sl < nb * 4;
            const int b = sl >> 2, j = sl & 3;
            uint2 lo = {0u, 0u}, hi = {0u, 0u};
            if (live) {
                lo = *(const uint2 *)(x + 32 * b + 4 * j);
                hi = *(const uint2 *)(x + 32 * b + 16 + 4 * j);
            }
            const float v[8] = {__uint_as_float(lo.x << 16), __uint_as_float(lo.x & 0xffff0000u),
                                __uint_as_float(lo.y << 16), __uint_as_float(lo.y & 0xffff0000u),
                                __uint_as_float(hi.x << 16), __uint_as_float(hi.x & 0xffff0000u),
                                __uint_as_float(hi.y << 16), __uint_as_float(hi.y & 0xffff0000u)};
            float amax = 0.0f;
#pragma unroll
            for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(v[c]));
            amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
            amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
            const float d = q8x_scale(amax);
            if (live) {
                uint32_t p0 = 0, p1 = 0;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    p0 |= (uint32_t)(uint8_t)q8x_code(v[c], d) << (8 * c);
                    p1 |= (uint32_t)(uint8_t)q8x_code(v[4 + c], d) << (8 * c);
                }
                xl[2 * sl] = p0;
                xl[2 * sl + 1] = p1;
                if (j == 0) dl[b] = f16_to_f32(__builtin_bit_cast(uint16_t, (_Float16)d));
            }
        }
    } else {
        for (int sl = tid; sl < nb * 4; sl += Q8_THREADS) {
            const int b = sl >> 2, j = sl & 3;
            xl[2 * sl] = *(const uint32_t *)(xq + 32 * b + 4 * j);
            xl[2 * sl + 1] = *(const uint32_t *)(xq + 32 * b + 16 + 4 * j);
        }
        for (int b = tid; b < nb; b += Q8_THREADS) dl[b] = f16_to_f32(xd[b]);
    }
    __syncthreads();

    const int r = lane & 15, j = lane >> 4;
    const uint8_t *panel = tiles + (int64_t)blockIdx.x * nb * TILE;
    float acc = 0.0f;
    auto tile = [&](int b, uint32_t w0, uint32_t w1, uint16_t dw) __attribute__((always_inline)) {
        const int sl = b * 4 + j;
        const int s = __builtin_amdgcn_sdot4((int)w1, (int)xl[2 * sl + 1],
                                             __builtin_amdgcn_sdot4((int)w0, (int)xl[2 * sl], 0, false), false);
        acc = __builtin_fmaf(f16_to_f32(dw) * dl[b], (float)s, acc);
    };
    int b = wave;
    for (; b + (UNROLL - 1) * Q8_WAVES < nb; b += UNROLL * Q8_WAVES) {
        uint32_t w0[UNROLL], w1[UNROLL];
        uint16_t dd[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const uint8_t *t = panel + (int64_t)(b + u * Q8_WAVES) * TILE;
            w0[u] = __builtin_nontemporal_load((const uint32_t *)(t + 64 * j + 4 * r));
            w1[u] = __builtin_nontemporal_load((const uint32_t *)(t + 64 * (j + 4) + 4 * r));
            dd[u] = __builtin_nontemporal_load((const uint16_t *)(t + 512 + 2 * r));
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) tile(b + u * Q8_WAVES, w0[u], w1[u], dd[u]);
    }
    for (; b < nb; b += Q8_WAVES) {
        const uint8_t *t = panel + (int64_t)b * TILE;
        tile(b, *(const uint32_t *)(t + 64 * j + 4 * r), *(const uint32_t *)(t + 64 * (j + 4) + 4 * r),
             *(const uint16_t *)(t + 512 + 2 * r));
    }
    acc += __shfl_xor(acc, 16, 64);
    acc += __shfl_xor(acc, 32, 64);
    if (lane < 16) red[wave][lane] = acc;
    __syncthreads();
    if (tid < 16) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < Q8_WAVES; ++w) sum += red[w][tid];
        const int64_t n = (int64_t)blockIdx.x * 16 + tid;
        if (y_dtype == MOE_F32) ((float *)y)[n] = sum;
        else ((uint16_t *)y)[n] = f32_to_bf16(sum);
    }
}

// one thread per 16-byte chunk of the packed output
__global__ __launch_bounds__(256) void k_q8_pack(const uint8_t *__restrict__ rows, int64_t N, int64_t K,
                                                 uint8_t *__restrict__ tiles) {
    const int64_t nb = K / 32;
    const int64_t chunks = (N / 16) * nb * 34;
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= chunks) return;
    const int64_t tt = c / 34;
    const int i = (int)(c % 34);
    const int64_t p = tt / nb, b = tt % nb;
    uint8_t out[16];
    if (i < 32) {
        const int j = i >> 2, r0 = 4 * (i & 3);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const uint8_t *blk = rows + ((p * 16 + r0 + rr) * nb + b) * 34;
#pragma unroll
            for (int q = 0; q < 4; ++q) out[4 * rr + q] = blk[2 + 4 * j + q];
        }
    } else {
        const int r0 = 8 * (i - 32);
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const uint8_t *blk = rows + ((p * 16 + r0 + rr) * nb + b) * 34;
            out[2 * rr] = blk[0];
            out[2 * rr + 1] = blk[1];
        }
    }
    u32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        v[q] = (uint32_t)out[4 * q] | ((uint32_t)out[4 * q + 1] << 8) | ((uint32_t)out[4 * q + 2] << 16) |
               ((uint32_t)out[4 * q + 3] << 24);
    *(u32x4 *)(tiles + tt * TILE + 16 * i) = v;
}

}  // namespace

hipError_t launch_q8_gemv(const uint8_t *tiles, int64_t N, int64_t K, const uint16_t *x, void *y,
                          int y_dtype, hipStream_t s) {
    const dim3 grid((unsigned)(N / 16)), block(Q8_THREADS), block16(1024);
    // few panels (at most one per two compute units): two workgroups per panel, eight panels
    // at a time, both halves on one XCD
    if (2 * (N / 16) <= n_compute_units() && (N / 16) % 8 == 0 && K % (128 * Q8_WAVES) == 0) {
        const dim3 grid2((unsigned)(N / 8));
        switch (K / (128 * Q8_WAVES)) {                       // groups of 4 tiles per wave
        case 2: hipLaunchKernelGGL((k_q8_gemv_part<2, 2>), grid2, block, 0, s, tiles, K, x, y, y_dtype); return hipGetLastError();
        case 4: hipLaunchKernelGGL((k_q8_gemv_part<4, 2>), grid2, block, 0, s, tiles, K, x, y, y_dtype); return hipGetLastError();
        case 8: hipLaunchKernelGGL((k_q8_gemv_part<8, 2>), grid2, block, 0, s, tiles, K, x, y, y_dtype); return hipGetLastError();
        default: break;
        }
    }
    // (16 waves pay off for long rows only: 8 tile pairs or more per wave)
    const bool few = N / 16 < n_compute_units() && K % (64 * 16) == 0 && K >= 8 * 64 * 16;
    switch (few ? 100 + K / (64 * 16) : K % (64 * Q8_WAVES) == 0 ? K / (64 * Q8_WAVES) : 0) {   // tile pairs per wave
    case 2: hipLaunchKernelGGL((k_q8_gemv_wide<2, Q8_WAVES>), grid, block, 0, s, tiles, K, x, y, y_dtype); break;
    case 4: hipLaunchKernelGGL((k_q8_gemv_wide<4, Q8_WAVES>), grid, block, 0, s, tiles, K, x, y, y_dtype); break;
    case 8: hipLaunchKernelGGL((k_q8_gemv_wide<8, Q8_WAVES>), grid, block, 0, s, tiles, K, x, y, y_dtype); break;
    case 16: hipLaunchKernelGGL((k_q8_gemv_wide<16, Q8_WAVES>), grid, block, 0, s, tiles, K, x, y, y_dtype); break;
    case 108: hipLaunchKernelGGL((k_q8_gemv_wide<8, 16>), grid, block16, 0, s, tiles, K, x, y, y_dtype); break;
    default: {
        const size_t lds = (size_t)(K / 32) * 32 * 4 + (size_t)(K / 32) * 4 * 4;
        hipLaunchKernelGGL((k_q8_gemv<4>), grid, block, lds, s, tiles, K, x, y, y_dtype);
        break;
    }
    }
    return hipGetLastError();
}

hipError_t launch_q8_quantize_x(const uint16_t *x, int64_t K, int8_t *xq, uint16_t *xd, hipStream_t s) {
    hipLaunchKernelGGL(k_q8_quantize_x, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, s, x, K, xq, xd);
    return hipGetLastError();
}

hipError_t launch_q8_gemv_q8x(const uint8_t *tiles, int64_t N, int64_t K, const int8_t *xq, const uint16_t *xd,
                              const uint16_t *x, void *y, int y_dtype, hipStream_t s) {
    const size_t lds = (size_t)(K / 32) * 8 * 4 + (size_t)(K / 32) * 4;
    if (x)
        hipLaunchKernelGGL((k_q8_gemv_q8x<4, true>), dim3((unsigned)(N / 16)), dim3(Q8_THREADS), lds, s, tiles, K,
                           nullptr, nullptr, x, y, y_dtype);
    else
        hipLaunchKernelGGL((k_q8_gemv_q8x<4, false>), dim3((unsigned)(N / 16)), dim3(Q8_THREADS), lds, s, tiles, K,
                           xq, xd, nullptr, y, y_dtype);
    return hipGetLastError();
}

hipError_t launch_q8_pack(const uint8_t *rows, int64_t N, int64_t K, uint8_t *tiles, hipStream_t s) {
    const int64_t chunks = (N / 16) * (K / 32) * 34;
    hipLaunchKernelGGL(k_q8_pack, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s, rows, N, K, tiles);
    return hipGetLastError();
}

}  // namespace qs
