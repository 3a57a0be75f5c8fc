/*
 * qsmoe.h -- C ABI of the MI355X (gfx950) quantized sparse mixture-of-experts FFN
 * layer and the dense Q8_0 decode GEMV.
 *
 * Sources, cited by page title and section:
 *   [LILY]  "Optimizing on-device inference for Apple Silicon" (Perplexity blog):
 *           "Qwen creates three distinct workload shapes" (router scores 256 experts,
 *           picks eight; a shared expert processes every token), "Dequantize weights
 *           during matrix multiplication" (4-bit integer codes, one scale and bias per
 *           group of 64 weights; fp32 accumulation), "Keep expert routing on the GPU"
 *           (histogram -> prefix scan -> scatter -> block map, no CPU round trip),
 *           "Match tile size to expert load", "Optimize the single-row weight path",
 *           "Reduce intermediate and state traffic" (fused expert input projections
 *           with the gated activation; fused output projection with the routing score
 *           and the shared-expert result).
 *   [OMLX]  "oMLX MoE gate/up fusion: qwen35_moe_gate_up implementation analysis"
 *           (pwwt.cn): "Fusion principle" ([gate; up] concatenated along the output
 *           axis is bit-identical to separate gate and up), "_can_fuse" (eligibility:
 *           equal group size, bits, shapes and dtypes).
 *   [EMBER] "Ember packed Q8 decode" (voidwest.dev): Q8_0 blocks ([fp16 scale][32 x
 *           int8]) and the packed 16-row tile (eight 64-byte groups + 16 fp16 scales,
 *           544 bytes); a reusable decode workspace instead of per-layer temporaries.
 *
 * General conventions
 *   - Every tensor pointer is a DEVICE pointer (HBM) unless stated otherwise; every
 *     call only enqueues work on `stream` (a hipStream_t; NULL = the null stream) and
 *     never synchronizes with the host.
 *   - The caller owns and frees every buffer.  The library allocates no device memory
 *     and keeps no state between calls.  Descriptors are read during the call only.
 *   - All validation runs on the host before the first enqueue; on any error nothing
 *     is enqueued and the outputs are untouched.  No exception or abort crosses the ABI.
 *   - Results are bit-deterministic for equal inputs, device and build: there are no
 *     floating-point atomics and every reduction has a fixed order.
 *   - Calls on different streams with distinct workspaces and outputs may run
 *     concurrently.
 */
#ifndef QSMOE_H
#define QSMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3

typedef int32_t moe_status;
#define MOE_OK               0
#define MOE_ERR_INVALID     -1   /* NULL / misaligned pointer, negative size, bad enum   */
#define MOE_ERR_UNSUPPORTED -2   /* shape or format outside the supported limits         */
#define MOE_ERR_WORKSPACE   -3   /* workspace NULL, misaligned or too small              */
#define MOE_ERR_DEVICE      -4   /* a HIP launch failed (hipGetLastError)                */

/* Bits of the workspace error word (read with moe_workspace_status).  Every wait of one
 * workgroup for another inside a launch is bounded; a wait that gives up sets its bit and
 * lets the kernel finish, so the grid always drains, and that call's outputs are not to be
 * trusted.  A correct call on a device that runs the whole grid sets no bit. */
#define MOE_WS_ERR_DECODE_WAIT 1u   /* a one-launch decode kernel (T <= 8) gave up a wait  */
#define MOE_WS_ERR_GEMM_WAIT   2u   /* a grouped-GEMM down tile gave up waiting for its h  */

/* element types */
#define MOE_BF16 0
#define MOE_F16  1
#define MOE_F32  2

/*
 * A stack of affine-quantized matrices, each [rows][cols], quantized in groups of
 * 64 consecutive columns of one row ([LILY] "Dequantize weights during matrix
 * multiplication"):  W[r][c] = scale[r][c/64] * q[r][c] + bias[r][c/64]
 * with an unsigned integer code q in [0, 2^bits).
 *   codes   uint8; matrix e, row r starts at byte (e*mat_stride + r) * cols*bits/8.
 *           4-bit codes: column 2i in the low nibble of byte i, 2i+1 in the high.
 *   scales  fp16, [..][cols/64]; matrix e, row r at element (e*mat_stride + r)*cols/64
 *   biases  fp16, same shape and indexing as scales
 *   mat_stride  rows between consecutive matrices: `rows` for a plain stack, or
 *           2*inter when gate and up are the two halves of one fused [gate; up]
 *           stack ([OMLX] "Fusion principle"; then up.codes = gate.codes +
 *           inter*cols*bits/8 and up.scales/biases = gate.* + inter*cols/64).
 * codes must be 16-byte aligned (every row then starts 16-byte aligned, given the
 * shape limits below); scales and biases 2-byte aligned.
 */
typedef struct {
    const void *codes;
    const void *scales;
    const void *biases;
    int64_t     mat_stride;
} moe_qmat;

/*
 * One MoE FFN layer ([LILY] "Qwen creates three distinct workload shapes").
 *   router_w     [n_experts][hidden] bf16
 *   router_bias  [n_experts] fp32 added to the logits before selection, or NULL
 *   gate, up     [n_experts][inter][hidden] stacks;  down [n_experts][hidden][inter]
 *   has_shared   1: the shared expert (s_gate, s_up [inter][hidden], s_down
 *                [hidden][inter], one matrix each) processes every token with weight 1
 *                (or, with shared_gate_w, with weight sigmoid(shared_gate_w . x))
 *   scale_dtype  MOE_F16 or MOE_BF16: the format of every qmat's scales and biases
 *                (bf16 is the checkpoint format the pages print)
 *   shared_gate_w  [hidden] bf16 (16-byte aligned) or NULL; needs has_shared
 * Limits (else MOE_ERR_UNSUPPORTED): group == 64; bits in {4, 8};
 *   1 <= n_experts <= 256; 1 <= top_k <= min(n_experts, 16);
 *   hidden % 64 == 0, 64 <= hidden <= 8192; inter % 64 == 0, 64 <= inter <= 2048;
 *   (top_k + 1) * inter <= 24576 (the batch-1 kernel hands every h value of a call
 *   between workgroups through a fixed region of the workspace).
 * Every qmat needs mat_stride >= its rows (MOE_ERR_INVALID otherwise).
 */
typedef struct {
    int32_t hidden, inter, n_experts, top_k, bits, group;
    int32_t scale_dtype;
    const void  *router_w;
    const float *router_bias;
    moe_qmat gate, up, down;
    int32_t    has_shared;
    moe_qmat s_gate, s_up, s_down;
    const void *shared_gate_w;
} moe_layer_desc;

int          moe_abi_version(void);                 /* MOE_ABI_VERSION of the library */
const char  *moe_status_string(moe_status s);   /* static string, never NULL */

/*
 * Bytes of device workspace moe_route / moe_layer_forward need for T tokens
 * (0 when T <= 0; SIZE_MAX when the descriptor is invalid).  The workspace must be
 * 256-byte aligned.  Its first 2 MiB are the state of the one-launch decode kernels
 * (T <= 8): a call counter, completion counters, tagged words the workgroups of one call
 * hand to each other, and the error word.  It must be zero before the first call that
 * uses the workspace (allocate it zero-filled) and then belongs to the library: every
 * call leaves it ready for the next one, so no clearing launch is needed per call
 * ([EMBER] "packed Q8 decode": one reusable decode workspace instead of per-layer
 * temporaries).  A caller that writes it must zero it again before the next call.  The
 * rest is scratch whose contents are undefined between calls.  Calls that share one
 * workspace must not overlap in time (issue them on one stream).  T >= 2 is processed in
 * chunks inside one call ([LILY] "Reduce intermediate and state traffic": bounded
 * intermediate buffers): this size is for chunks of MOE_PREFILL_CHUNK tokens, so it stops
 * growing there (~200 MiB for any T >= 4096 at hidden 2048, inter 512, top-8).
 */
size_t moe_workspace_size(const moe_layer_desc *d, int64_t T);

/* Default tokens per prefill chunk (T >= 2). */
#define MOE_PREFILL_CHUNK 4096

/*
 * Bytes of workspace for T tokens run in chunks of `chunk` tokens (0: the default
 * MOE_PREFILL_CHUNK; chunk >= T: unchunked; 1 counts as 2).  moe_route /
 * moe_layer_forward accept any workspace at least as large as the chunk-2 size and take
 * the largest chunk whose buffers fit in the ws_bytes they are given, so a caller that can
 * spare the memory avoids re-reading the expert weights once per chunk, and one short of
 * memory can bound it.  Chunking changes no result: every token is computed by the same
 * kernels whatever chunk it falls in, bit for bit.  SIZE_MAX for an invalid descriptor,
 * T > 2^20 or chunk < 0.
 */
size_t moe_workspace_size_chunked(const moe_layer_desc *d, int64_t T, int64_t chunk);

/*
 * Enqueues on `stream` a copy of the workspace's error word (MOE_WS_ERR_* bits, 0 when
 * every call so far completed every wait) into *status_out, a device uint32, and, when
 * `clear` is nonzero, resets the word to 0 afterwards.  ws must be a workspace of
 * ws_bytes >= 2 MiB used by moe_route / moe_layer_forward (or freshly zeroed); the call
 * is ordered with the layer calls on the same stream.
 */
moe_status moe_workspace_status(void *ws, size_t ws_bytes, uint32_t *status_out, int32_t clear,
                                void *stream);

/*
 * Router only ([LILY] "Qwen creates three distinct workload shapes"): fp32 logits
 * l[t][e] = sum_c x[t][c] * router_w[e][c] (+ router_bias[e]), the top_k largest per
 * token (exact ties to the lower expert id), and weights renormalised over the
 * selection, w_j = exp(l_j - l_max) / sum_{i in selection} exp(l_i - l_max).
 *   x        [T][hidden] bf16
 *   topk_idx [T][top_k] int32, ascending expert id within a token (written)
 *   topk_w   [T][top_k] fp32, aligned with topk_idx (written)
 *   ws       device workspace of ws_bytes >= moe_workspace_size(d, T)
 * T == 0 returns MOE_OK and enqueues nothing; T > 2^20 is MOE_ERR_UNSUPPORTED.
 */
moe_status moe_route(const moe_layer_desc *d, const void *x, int64_t T,
                       int32_t *topk_idx, float *topk_w,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * The whole layer: router, top-k, (T >= 2) expert binning, fused [gate; up]
 * projection + SwiGLU h = silu(g) * u with silu(z) = z / (1 + e^-z), down
 * projection, and the combine
 *     y[t] = sum over the selected experts in ascending id of w_j * o_j  +  o_shared,
 * accumulated in fp32 in that fixed order ([LILY] "Reduce intermediate and state
 * traffic"; [OMLX] "Fusion principle").
 *   x        [T][hidden] bf16, any finite values: every fp16 operand of the kernels
 *            (x, the dequantized weights, h, the routed outputs) carries an exact
 *            power-of-two range scale, so results stay within the parity bound of
 *            an fp64 evaluation for activations, scales and biases anywhere in
 *            bf16's range, as long as the intermediate values fit in fp32
 *   y        [T][hidden], y_dtype MOE_BF16 (round-to-nearest-even) or MOE_F32
 *   topk_idx, topk_w  optional outputs as in moe_route (NULL to skip)
 * Path: T == 1 runs the batch-1 decode kernel (register dequantization on the vector
 * ALUs, fp32 intermediates); T = 2 .. 4 the same kernel design over all tokens at once,
 * each expert any token selected read once (when T * (top_k + 1) * inter <= 98496);
 * T = 5 .. 8 two such launches of ceil(T/2) and floor(T/2) tokens (when both fit);
 * larger T runs the grouped-GEMM path (MFMA on fp16 operands dequantized in registers,
 * fp32 accumulation, fp16 intermediates, each under its range scale).
 * For a given T the result does not depend on whether gate/up are fused or separate,
 * nor on the other tokens of the call (tokens are independent), bit for bit.
 */
moe_status moe_layer_forward(const moe_layer_desc *d, const void *x, int64_t T,
                               void *y, int32_t y_dtype,
                               int32_t *topk_idx, float *topk_w,
                               void *ws, size_t ws_bytes, void *stream);

/*
 * moe_layer_forward for callers that cannot allocate device memory or pass a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and the same results, bit for bit, with the workspace replaced by a
 * 64 MiB array the library holds on each GPU from load until the process ends.  This
 * call allocates nothing.  The caller still passes x, y and the optional topk outputs
 * (as for moe_layer_forward).  The array is shared by every call of this entry point on
 * one GPU and keeps the last call's contents: calls that overlap in time on one GPU race
 * (issue them on one stream).  Prompts longer than the array holds run in chunks that
 * fit it (no result changes, only more passes over the expert weights); a layer whose
 * 2-token chunk does not fit returns MOE_ERR_WORKSPACE (none within the limits above
 * does).  Errors and limits otherwise as for moe_layer_forward; MOE_ERR_DEVICE when the
 * array's address cannot be obtained on the current device.
 */
moe_status moe_layer_forward_static(const moe_layer_desc *d, const void *x, int64_t T,
                                    void *y, int32_t y_dtype,
                                    int32_t *topk_idx, float *topk_w, void *stream);

/*
 * Dense Q8_0 decode GEMV over 16-row packed tiles ([EMBER] packed 16-row tile):
 *     y[n] = sum_b d[n][b] * sum_{c<32} q[n][32b + c] * x[32b + c]
 * with fp32 accumulation.
 *   w_tiles  (N/16)*(K/32) tiles of 544 bytes, panel-major (tile p*(K/32) + b holds
 *            rows 16p..16p+15, columns 32b..32b+31): eight 64-byte groups, group j =
 *            rows 0..15 x codes 4j..4j+3 (4 bytes per row, rows in order), then the
 *            16 fp16 scales in row order.  16-byte aligned.
 *   x        [K] bf16;  y  [N], y_dtype MOE_BF16 or MOE_F32
 * Limits: N % 16 == 0, K % 32 == 0, N >= 16, 32 <= K <= 8192 (else MOE_ERR_UNSUPPORTED).
 */
moe_status q8_gemv(const void *w_tiles, int64_t N, int64_t K, const void *x,
                     void *y, int32_t y_dtype, void *stream);

/*
 * Activation quantization for the Q8_0 GEMV ([EMBER]: the activation is quantized once
 * and the quantized copy is shared by the projections that read it, Q/K/V and gate/up).
 * Each block of 32 values of x becomes a Q8_0 block, stored split:
 *     d[b]  = max_c |x[32b + c]| / 127, computed in binary32, stored as fp16 (nearest even)
 *     q[i]  = x[i] / d[b] in binary32 (the unrounded d), rounded half away from zero,
 *             clamped to [-127, 127]; an all-zero block has d = 0 and q = 0
 *   x   [K] bf16 (2-byte aligned);  xq [K] int8 (4-byte aligned);  xd [K/32] fp16
 *       (2-byte aligned); all device memory, xq / xd written, owned by the caller.
 * Limits: K % 32 == 0, K <= 8192 (else MOE_ERR_UNSUPPORTED); K = 0 enqueues nothing.
 */
moe_status q8_quantize_x(const void *x, int64_t K, void *xq, void *xd, void *stream);

/*
 * Dense Q8_0 GEMV with a quantized activation (from q8_quantize_x):
 *     y[n] = sum_b d[n][b] * xd[b] * sum_{c<32} q[n][32b + c] * xq[32b + c]
 * the inner sums exact in int32 (v_dot4_i32_i8), the scaling and the sum over b in fp32.
 *   w_tiles  as for q8_gemv;  xq [K] int8 (4-byte aligned), xd [K/32] fp16;
 *   y [N], y_dtype MOE_BF16 or MOE_F32.  Limits as for q8_gemv.
 */
moe_status q8_gemv_q8x(const void *w_tiles, int64_t N, int64_t K, const void *xq, const void *xd,
                         void *y, int32_t y_dtype, void *stream);

/*
 * The same GEMV taking x [K] bf16 (8-byte aligned) and quantizing it inside the kernel
 * with q8_quantize_x's rule (identical codes and scales, so identical y) while staging
 * it: no separate launch and no codes in memory.  Limits as for q8_gemv.
 */
moe_status q8_gemv_qx(const void *w_tiles, int64_t N, int64_t K, const void *x, void *y,
                        int32_t y_dtype, void *stream);

/*
 * Load-time repacking ([EMBER] packed 16-row tile): row-contiguous Q8_0 blocks
 * w_rows [N][K/32] x 34 bytes ([fp16 d][32 x int8]) -> w_tiles (layout of q8_gemv).
 * Pure byte moves, idempotent; w_rows and w_tiles must not overlap.
 * Limits: N % 16 == 0, K % 32 == 0.
 */
moe_status q8_pack_rows16(const void *w_rows, int64_t N, int64_t K, void *w_tiles,
                            void *stream);

/*
 * Measured ceilings ([LILY] "Limits of further optimization": kernels are judged
 * against the fastest sustained rate of their resource, next to the data-sheet peak).
 * Measurement helpers only; they compute nothing the layer uses.
 *   moe_calib_read  one read-only pass over buf (bytes % 16 == 0, 16-byte aligned) with
 *                   16-byte nontemporal loads: time it to get the sustained HBM read
 *                   rate (use a buffer far larger than the 256 MB on-die cache).
 *   moe_calib_mfma  `blocks` workgroups of 4 waves, each wave issuing iters x 8
 *                   v_mfma_f32_16x16x32_f16 (16384 flops each) on register operands:
 *                   the sustained dense fp16 matrix rate.
 * Both enqueue one kernel on `stream` and store nothing.
 */
moe_status moe_calib_read(const void *buf, size_t bytes, void *stream);
moe_status moe_calib_mfma(int32_t iters, int32_t blocks, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* QSMOE_H */
