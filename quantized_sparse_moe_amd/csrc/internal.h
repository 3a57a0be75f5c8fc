// internal.h -- argument blocks passed from the host entry points (api.cpp) to the
// kernel launchers of libqsmoe.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qsmoe.h"

namespace qs {

struct QMat {                      // one stack of affine-quantized matrices
    const uint8_t *codes;
    const uint16_t *scales;        // fp16 bits
    const uint16_t *biases;        // fp16 bits
    int64_t stride;                // rows between matrices
};

struct Layer {
    int H, I, E, K, bits;          // hidden, inter, experts, top_k, code bits
    const uint16_t *router_w;      // bf16 [E][H]
    const float *router_bias;      // [E] or null
    QMat gate, up, down;
    int has_shared;
    QMat s_gate, s_up, s_down;
    int sb_bf16;                   // scales and biases are bf16 (else fp16)
    const uint16_t *shared_gate_w; // bf16 [H]: shared output scaled by sigmoid(g . x); or null
};

// -------------------------------------------------------------------- decode T = 1
// Decode state at the start of every workspace: zero before the first call, then kept
// by the library between calls (call generation, completion counters, and the tagged
// logit and h words the workgroups of one call hand to each other).
constexpr size_t WS_CTL_BYTES = 2 * 1024 * 1024;

struct DecodeBufs {
    uint32_t *ctl;                 // WS_CTL_BYTES of decode state
};

// the workspace's error word (word 0 of the state) copied to *out, then optionally cleared
hipError_t launch_ws_status(uint32_t *ctl, uint32_t *out, bool clear, hipStream_t s);

hipError_t launch_decode_layer(const Layer &L, const uint16_t *x, const DecodeBufs &b, void *y,
                               int y_dtype, int32_t *out_idx, float *out_w, hipStream_t s);
// T = 2 .. 4 tokens in one launch, the routed experts read once for all of them
constexpr int SMALL_TMAX = 4;   // tokens of one small-batch decode launch
bool decode_small_eligible(const Layer &L, int64_t T);
hipError_t launch_decode_small_layer(const Layer &L, const uint16_t *x, int64_t T, const DecodeBufs &b, void *y,
                                     int y_dtype, int32_t *out_idx, float *out_w, hipStream_t s);
hipError_t launch_decode_small_route(const Layer &L, const uint16_t *x, int64_t T, const DecodeBufs &b,
                                     int32_t *out_idx, float *out_w, hipStream_t s);
hipError_t launch_decode_route(const Layer &L, const uint16_t *x, const DecodeBufs &b,
                               int32_t *out_idx, float *out_w, hipStream_t s);

// ------------------------------------------------------------------- prefill T >= 2
constexpr int ROUTER_TOKENS = 16;  // tokens per router workgroup (= one binning block)
constexpr int GEMM_MT = 10;        // 16-row MFMA subtiles per GEMM tile (even)
constexpr int GEMM_BM = 16 * GEMM_MT;

struct Tile {                      // one row block of one expert bin
    int32_t expert;                // 0..E-1, or E for the shared expert
    int32_t row0;                  // first row in the h / perm position space
    int32_t nrows;                 // 1..GEMM_BM
    int32_t pad;
};

// fp16 operands of the grouped path carry power-of-two range scales: x 2^a per token
// (a in xexp), h 2^e per (row, 128-column block) (e in hexp, block-major: the exponents
// of one block for all T*K + T rows together), slot rows 2^e per (row, 64-column block)
// (sexp, block-major as well, rows padded to a multiple of 16)
constexpr int HEXP_STRIDE = 16;    // inter <= 2048: at most 16 blocks of 128 columns
// a state word read by the grouped GEMM: nonzero gives every h block the scale that puts
// its largest value in [2^14, 2^15) instead of the shared one (0 for ordinary blocks), so
// that nearly every down tile must rescale (set only by tests of that rescale)
constexpr int CTL_HBLOCK_EXACT = 33;

struct PrefillBufs {
    uint16_t *x16;                 // [T][H] fp16 x 2^a, columns permuted per 8-group (code order)
    uint32_t *xmax;                // [T][8] largest |x| per token and logits expert block
    int32_t *xexp;                 // [T] the a of each token's x16 row
    float *logits;                 // [T][E] router logits
    int32_t *idx;                  // [T][K]
    float *w;                      // [T][K]
    int32_t *blkcnt;               // [nblk][E]  assignments per (16-token block, expert)
    int32_t *blkoff;               // [nblk][E]  first position of that block's rows in the expert bin
    int32_t *expert_off;           // [E+1]
    int32_t *perm;                 // [T*K]      position -> t*K + j
    Tile *tiles;                   // [max_tiles] routed full, routed partial, then shared tiles
    int32_t *ntiles;               // [3] routed tiles, routed + shared tiles, and a flag the
                                   // down pass sets when some slot block has a nonzero scale
    int32_t *tile_done;            // [max_tiles] gate/up column blocks finished per tile
    uint32_t *ctl;                 // the workspace's state region (word 0: bounded-wait error flag)
    uint16_t *h;                   // [(T*K + T)][I] fp16, columns permuted per 8-group
    int8_t *hexp;                  // [HEXP_STRIDE][T*K + T]
    uint16_t *slot;                // [T*K + T][H] fp16: w_j * o_j per (token, slot), then shared o
    int8_t *sexp;                  // [H / 64][sexp_rows(T, K)]
    float *sgate;                  // [T] shared-expert gate sigmoid(g . x_t) (gated layers)
};

__host__ __device__ inline int64_t sexp_rows(int64_t T, int K) { return (T * K + T + 15) / 16 * 16; }
int64_t prefill_max_routed_tiles(int64_t T, int K, int E);
int64_t prefill_max_tiles(int64_t T, int K, int E);

hipError_t launch_prefill_router(const Layer &L, const uint16_t *x, int64_t T,
                                 const PrefillBufs &b, bool write_x16, int32_t *out_idx,
                                 float *out_w, hipStream_t s);
hipError_t launch_prefill_binning(const Layer &L, int64_t T, const PrefillBufs &b, hipStream_t s);
hipError_t launch_prefill_gemms(const Layer &L, int64_t T, const PrefillBufs &b, void *y,
                                int y_dtype, hipStream_t s);

// --------------------------------------------------------------------------- Q8_0
int n_compute_units();   // of the current device, queried once
hipError_t launch_q8_gemv(const uint8_t *tiles, int64_t N, int64_t K, const uint16_t *x,
                          void *y, int y_dtype, hipStream_t s);
hipError_t launch_q8_quantize_x(const uint16_t *x, int64_t K, int8_t *xq, uint16_t *xd, hipStream_t s);
hipError_t launch_q8_gemv_q8x(const uint8_t *tiles, int64_t N, int64_t K, const int8_t *xq, const uint16_t *xd,
                              const uint16_t *x, void *y, int y_dtype, hipStream_t s);
hipError_t launch_q8_pack(const uint8_t *rows, int64_t N, int64_t K, uint8_t *tiles,
                          hipStream_t s);

// ---------------------------------------------------------------- measured ceilings
hipError_t launch_calib_read(const void *buf, int64_t bytes, uint32_t *out, hipStream_t s);
hipError_t launch_calib_mfma(int iters, int blocks, float *out, hipStream_t s);

}  // namespace qs
