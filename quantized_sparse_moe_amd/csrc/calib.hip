// calib.hip -- measured ceilings of the two resources the layer's kernels are bound by,
// for reporting each kernel's rate as a fraction of what the chip sustains, next to its
// fraction of the published peak ([LILY] "Limits of further optimization": the matrix
// multiply and the weight reads are judged against the fastest sustained rates for their
// access patterns, not only against the data sheet).
//
//   k_calib_read  a read-only stream over a buffer (16-byte nontemporal loads, four in
//                 flight per lane, grid-stride): the sustained HBM read rate.
//   k_calib_mfma  back-to-back v_mfma_f32_16x16x32_f16 on register operands, eight
//                 independent accumulators per wave, two waves per SIMD: the sustained
//                 dense fp16 matrix rate.
// Neither kernel stores anything unless its result equals a value it cannot take, so
// neither moves bytes beyond its reads.
#include "common.h"
#include "internal.h"

namespace qs {

namespace {

__global__ __launch_bounds__(256) void k_calib_read(const u32x4 *__restrict__ p, int64_t n16, uint32_t *out) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    uint32_t acc = 0u;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(p + i), b = __builtin_nontemporal_load(p + i + stride);
        const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride), d = __builtin_nontemporal_load(p + i + 3 * stride);
        acc ^= (a[0] ^ a[1] ^ a[2] ^ a[3]) + (b[0] ^ b[1] ^ b[2] ^ b[3]) + (c[0] ^ c[1] ^ c[2] ^ c[3]) +
               (d[0] ^ d[1] ^ d[2] ^ d[3]);
    }
    for (; i < n16; i += stride) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    if (acc == 0x9e3779b9u && out) out[0] = acc;             // keeps the loads; never taken on real data
}

__global__ __launch_bounds__(256, 2) void k_calib_mfma(int iters, float *out) {
    const int lane = threadIdx.x & 63;
    f16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(0.001f * (float)((lane + i) & 7));
        b[i] = (_Float16)(0.002f * (float)((lane * 3 + i) & 7));
    }
    f32x4 c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
    if (s == -1.0f && out) out[0] = s;                       // all operands are non-negative
}

}  // namespace

hipError_t launch_calib_read(const void *buf, int64_t bytes, uint32_t *out, hipStream_t s) {
    const int64_t n16 = bytes / 16;
    hipLaunchKernelGGL(k_calib_read, dim3(256 * 8), dim3(256), 0, s, (const u32x4 *)buf, n16, out);
    return hipGetLastError();
}

hipError_t launch_calib_mfma(int iters, int blocks, float *out, hipStream_t s) {
    hipLaunchKernelGGL(k_calib_mfma, dim3(blocks), dim3(256), 0, s, iters, out);
    return hipGetLastError();
}

}  // namespace qs
