/*
 * oracle.h -- plain fp64 CPU oracle for the quantized sparse MoE FFN layer and the
 * dense Q8_0 decode GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or call
 * this.  Only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no source, header, table or helper with the HIP
 * library: it decodes every byte format with its own code.
 *
 * Sources (cited by page title and section):
 *   [LILY]  "Optimizing on-device inference for Apple Silicon" (Perplexity blog),
 *           sections "Qwen creates three distinct workload shapes",
 *           "Dequantize weights during matrix multiplication",
 *           "Keep expert routing on the GPU", "Reduce intermediate and state traffic".
 *   [OMLX]  "oMLX MoE gate/up fusion: qwen35_moe_gate_up implementation analysis"
 *           (pwwt.cn), section "Fusion principle".
 *   [EMBER] "Ember packed Q8 decode" (voidwest.dev), the row-contiguous source /
 *           packed 16-row tile figure and the paragraph after it.
 *
 * All floating-point work is double precision.  fp16 and bf16 values are passed as
 * their raw 16-bit patterns (uint16_t) and decoded here.
 */
#ifndef QSMOE_ORACLE_H
#define QSMOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One stack of affine-quantized matrices (group 64 along the column axis).
 * Matrix e, row r starts at code byte (e*mat_stride + r) * cols*bits/8 and at
 * scale/bias index (e*mat_stride + r) * cols/64. */
typedef struct {
    const uint8_t  *codes;
    const uint16_t *scales;   /* fp16 bit patterns (bf16 when sb_bf16) */
    const uint16_t *biases;   /* fp16 bit patterns (bf16 when sb_bf16) */
    int64_t         mat_stride;
    int32_t         sb_bf16;  /* 1: scales and biases are bfloat16 */
} orc_qmat;

typedef struct {
    int32_t hidden, inter, n_experts, top_k, bits, group;
    const uint16_t *router_w;     /* [E][hidden] bf16 bit patterns          */
    const float    *router_bias;  /* [E] or NULL                            */
    orc_qmat gate, up, down;      /* gate/up [E][inter][hidden], down [E][hidden][inter] */
    int32_t  has_shared;
    orc_qmat s_gate, s_up, s_down;/* shared expert, one matrix each         */
    const uint16_t *shared_gate_w;/* [hidden] bf16: shared output scaled by
                                     sigmoid(shared_gate_w . x); NULL: weight 1 */
} orc_layer;

/* decoders of the 16-bit formats */
double orc_f16_to_double(uint16_t h);
double orc_bf16_to_double(uint16_t b);
/* binary64 -> binary16 bit patterns, round to nearest, ties to even; overflow to inf */
void orc_f64_to_f16(const double *v, int64_t n, uint16_t *out);

/* W[r, c] of matrix `e` of `m` (rows x cols), fp64.  out is [rows][cols]. */
void orc_dequant_matrix(const orc_qmat *m, int32_t bits, int64_t e, int64_t rows,
                        int64_t cols, double *out);

/* router logits l[t, e] (fp64), [T][E] */
void orc_router_logits(const orc_layer *L, const uint16_t *x, int64_t T, double *logits);

/* top-k + renormalised weights.  idx [T][k] ascending expert id, w [T][k];
 * gap[t] = (k-th largest logit) - ((k+1)-th largest logit), or +inf when k == E.
 * gap may be NULL. */
void orc_route(const orc_layer *L, const uint16_t *x, int64_t T, int32_t *idx,
               double *w, double *gap);

/* whole layer: y [T][hidden] fp64; idx/w may be NULL */
void orc_layer_forward(const orc_layer *L, const uint16_t *x, int64_t T, double *y,
                       int32_t *idx, double *w);

/* layer with a given routing (idx [T][k] any order, w [T][k]) */
void orc_layer_forward_with_routing(const orc_layer *L, const uint16_t *x, int64_t T,
                                    const int32_t *idx, const double *w, double *y);

/* one expert's SwiGLU MLP for one token: o [hidden] */
void orc_expert_mlp(const orc_layer *L, const orc_qmat *g, const orc_qmat *u,
                    const orc_qmat *d, int64_t e, const double *x, double *o);

/* Q8_0: rows [N][K/32] blocks of 34 bytes ([fp16 d][32 x int8]); x bf16 [K] */
void orc_q8_gemv(const uint8_t *rows, int64_t N, int64_t K, const uint16_t *x, double *y);

/* 16-row packed tiles <-> row-contiguous Q8_0 blocks (N % 16 == 0, K % 32 == 0) */
void orc_q8_pack_rows16(const uint8_t *rows, int64_t N, int64_t K, uint8_t *tiles);
void orc_q8_unpack_rows16(const uint8_t *tiles, int64_t N, int64_t K, uint8_t *rows);

/* Q8_0 block quantizer / dequantizer for one row of K floats (K % 32 == 0) */
void orc_q8_quantize_row(const float *v, int64_t K, uint8_t *blocks);
void orc_q8_dequantize_row(const uint8_t *blocks, int64_t K, double *v);
/* Q8_0 quantization of an activation vector (bf16 [K] -> int8 [K] + fp16 [K/32]) and the
 * GEMV over Q8_0 rows with it (integer dots, fp64 scaling). */
void orc_q8_quantize_x(const uint16_t *x, int64_t K, int8_t *q, uint16_t *d);
void orc_q8_gemv_q8x(const uint8_t *rows, int64_t N, int64_t K, const int8_t *xq, const uint16_t *xd,
                     double *y);

int orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
