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

struct PrefillBufs {
    uint16_t *x16;                 // [T][H] fp16, columns permuted per 8-group (code order)
    float *logits;                 // [T][E] router logits
    int32_t *idx;                  // [T][K]
    float *w;                      // [T][K]
    int32_t *blkcnt;               // [nblk][E]  assignments per (32-token block, expert)
    int32_t *blkoff;               // [nblk][E]  first position of that block's rows in the expert bin
    int32_t *expert_off;           // [E+1]
    int32_t *perm;                 // [T*K]      position -> t*K + j
    Tile *tiles;                   // [max_tiles] routed full, routed partial, then shared tiles
    int32_t *ntiles;               // [2] routed tiles, routed + shared tiles
    int32_t *tile_done;            // [max_tiles] gate/up column blocks finished per tile
    uint32_t *ctl;                 // the workspace's state region (word 0: bounded-wait error flag)
    uint16_t *h;                   // [(T*K + T)][I] fp16, columns permuted per 8-group
    uint16_t *slot;                // [T*K + T][H] fp16: w_j * o_j per (token, slot), then shared o
    float *sgate;                  // [T] shared-expert gate sigmoid(g . x_t) (gated layers)
};

int64_t prefill_max_routed_tiles(int64_t T, int K, int E);
int64_t prefill_max_tiles(int64_t T, int K, int E);

hipError_t launch_prefill_router(const Layer &L, const uint16_t *x, int64_t T,
                                 const PrefillBufs &b, bool write_x16, int32_t *out_idx,
                                 float *out_w, hipStream_t s);
hipError_t launch_prefill_binning(const Layer &L, int64_t T, const PrefillBufs &b, hipStream_t s);
hipError_t launch_prefill_gemms(const Layer &L, int64_t T, const PrefillBufs &b, void *y,
                                int y_dtype, hipStream_t s);

// --------------------------------------------------------------------------- Q8_0
hipError_t launch_q8_gemv(const uint8_t *tiles, int64_t N, int64_t K, const uint16_t *x,
                          void *y, int y_dtype, hipStream_t s);
hipError_t launch_q8_quantize_x(const uint16_t *x, int64_t K, int8_t *xq, uint16_t *xd, hipStream_t s);
hipError_t launch_q8_gemv_q8x(const uint8_t *tiles, int64_t N, int64_t K, const int8_t *xq, const uint16_t *xd,
                              const uint16_t *x, void *y, int y_dtype, hipStream_t s);
hipError_t launch_q8_pack(const uint8_t *rows, int64_t N, int64_t K, uint8_t *tiles,
                          hipStream_t s);

}  // namespace qs
