/*
 * oracle.c -- plain, slow, obviously correct fp64 CPU oracle (TEST INFRASTRUCTURE).
 *
 * Only tests, the smoke check and the benchmark's cpu_baseline leg may load this
 * library.  It shares no code with the HIP path.  Every function follows the
 * definition on the pages (see oracle.h for the page list) written out with plain
 * loops; OpenMP spreads independent tokens / rows over cores and changes nothing
 * in the arithmetic of any single output.
 *
 * Readings of points the pages leave open (the same list is kept in the design
 * notes of the repository):
 *   - affine code: W = s*q + b with unsigned q in [0, 2^bits), s and b shared by
 *     64 consecutive columns of one row ([LILY] "Dequantize weights during matrix
 *     multiplication": integer code plus a per-group-of-64 scale and bias);
 *     scale/bias stored as fp16 (or bf16, see below);
 *   - 4-bit packing: column 2i in the low nibble of byte i, column 2i+1 in the high;
 *   - router: logits l = Wr x (+ optional per-expert bias), softmax over all
 *     experts, the k most probable kept (ties to the lower expert id) and their
 *     probabilities renormalised to sum to one ([LILY] "Qwen creates three
 *     distinct workload shapes": the router scores 256 experts and picks eight);
 *   - SwiGLU: h = silu(gate) * up with silu(z) = z / (1 + e^-z); gate rows come
 *     first in the fused [gate; up] stack ([OMLX] "Fusion principle");
 *   - shared expert: weight 1, same shapes as a routed expert ([LILY]: a shared
 *     expert processes every token); the checkpoint variant with a shared-expert
 *     gate scales its output by sigmoid(g . x), g a bf16 vector over the hidden size;
 *   - scales and biases fp16, or bf16 in the checkpoint variant the pages print;
 *   - Q8_0 block: [fp16 d][32 x int8 q], value d*q ([EMBER] row-contiguous source);
 *     16-row tile: eight 64-byte groups, group j holding codes 4j..4j+3 of rows
 *     0..15 in row order, then the 16 fp16 scales in row order ([EMBER] packed
 *     16-row tile figure); tiles ordered panel-major, block-minor.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- 16-bit formats */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_f16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);                  /* subnormal: frac * 2^-24 */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp(1.0 + (double)frac / 1024.0, expo - 15);
    return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double orc_bf16_to_double(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int expo = (b >> 7) & 0xff;
    int frac = b & 0x7f;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -133);                 /* subnormal: frac * 2^-126 / 128 */
    else if (expo == 255)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp(1.0 + (double)frac / 128.0, expo - 127);
    return sign ? -v : v;
}

/* round-to-nearest-even of a finite double into binary16 (used by the Q8_0
 * quantizer only; values here are far inside the binary16 range) */
static uint16_t double_to_f16(double v)
{
    uint16_t sign = 0;
    if (signbit(v)) { sign = 0x8000; v = -v; }   /* -0.0 keeps its sign, as IEEE 754 conversion does */
    if (v == 0) return sign;
    if (v >= 65520.0) return sign | 0x7c00;
    int e;
    frexp(v, &e);                       /* v = m * 2^e, m in [0.5, 1) */
    int expo = e - 1;                   /* v in [2^expo, 2^(expo+1)) */
    if (expo < -14) expo = -14;         /* subnormal range shares the 2^-24 step */
    double step = ldexp(1.0, expo - 10);
    double n = v / step;                /* exact: power-of-two scaling */
    double r = floor(n);
    double rem = n - r;
    if (rem > 0.5 || (rem == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    /* r * step is the rounded value; rebuild the bit pattern */
    double rv = r * step;
    if (rv >= 65520.0) return sign | 0x7c00;
    if (rv < ldexp(1.0, -14))
        return sign | (uint16_t)(rv / ldexp(1.0, -24));
    frexp(rv, &e);
    expo = e - 1;
    uint16_t frac = (uint16_t)((rv / ldexp(1.0, expo) - 1.0) * 1024.0);
    return sign | (uint16_t)((expo + 15) << 10) | frac;
}

/* the encoder above over an array: the fp16 bit patterns of v[0..n) */
void orc_f64_to_f16(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = double_to_f16(v[i]);
}

/* ------------------------------------------------------------ affine dequantize */

static int64_t row_code_bytes(int32_t bits, int64_t cols) { return cols * bits / 8; }

/* W[r, c] of matrix e: s * q + b with the group of 64 columns containing c */
static double weight(const orc_qmat *m, int32_t bits, int64_t e, int64_t r, int64_t c,
                     int64_t cols)
{
    int64_t R = e * m->mat_stride + r;
    const uint8_t *row = m->codes + R * row_code_bytes(bits, cols);
    unsigned q;
    if (bits == 8)
        q = row[c];
    else                                   /* 4-bit: even column in the low nibble */
        q = (c & 1) ? (row[c / 2] >> 4) : (row[c / 2] & 0x0f);
    int64_t gi = R * (cols / 64) + c / 64;
    double s = m->sb_bf16 ? orc_bf16_to_double(m->scales[gi]) : orc_f16_to_double(m->scales[gi]);
    double b = m->sb_bf16 ? orc_bf16_to_double(m->biases[gi]) : orc_f16_to_double(m->biases[gi]);
    return s * (double)q + b;
}

void orc_dequant_matrix(const orc_qmat *m, int32_t bits, int64_t e, int64_t rows,
                        int64_t cols, double *out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = weight(m, bits, e, r, c, cols);
}

/* ----------------------------------------------------------------------- router */

static void logits_one(const orc_layer *L, const uint16_t *xt, double *l)
{
    const int64_t H = L->hidden;
    for (int e = 0; e < L->n_experts; ++e) {
        double acc = 0.0;
        for (int64_t c = 0; c < H; ++c)
            acc += orc_bf16_to_double(xt[c]) *
                   orc_bf16_to_double(L->router_w[(int64_t)e * H + c]);
        if (L->router_bias) acc += (double)L->router_bias[e];
        l[e] = acc;
    }
}

void orc_router_logits(const orc_layer *L, const uint16_t *x, int64_t T, double *logits)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t)
        logits_one(L, x + t * L->hidden, logits + t * L->n_experts);
}

/* a ranks above b: larger logit, ties to the lower expert id */
static int ranks_above(const double *l, int a, int b)
{
    return l[a] > l[b] || (l[a] == l[b] && a < b);
}

static void route_one(const orc_layer *L, const double *l, int32_t *idx, double *w,
                      double *gap)
{
    const int E = L->n_experts, k = L->top_k;
    if (E < 1 || k < 1 || k > E) return;
    int *order = (int *)malloc(sizeof(int) * E);
    double *p = (double *)malloc(sizeof(double) * E);
    for (int e = 0; e < E; ++e) order[e] = e;
    /* selection sort by rank: plain and obviously correct */
    for (int i = 0; i < E; ++i) {
        int best = i;
        for (int j = i + 1; j < E; ++j)
            if (ranks_above(l, order[j], order[best])) best = j;
        int tmp = order[i]; order[i] = order[best]; order[best] = tmp;
    }
    if (gap) *gap = (k < E) ? l[order[k - 1]] - l[order[k]] : INFINITY;
    /* softmax over all experts */
    double mx = l[order[0]], z = 0.0;
    for (int e = 0; e < E; ++e) { p[e] = exp(l[e] - mx); z += p[e]; }
    for (int e = 0; e < E; ++e) p[e] /= z;
    /* the k selected experts in ascending id order */
    int32_t sel[256];
    for (int j = 0; j < k; ++j) sel[j] = order[j];
    for (int i = 0; i < k; ++i)
        for (int j = i + 1; j < k; ++j)
            if (sel[j] < sel[i]) { int32_t t = sel[i]; sel[i] = sel[j]; sel[j] = t; }
    double zs = 0.0;
    for (int j = 0; j < k; ++j) zs += p[sel[j]];
    for (int j = 0; j < k; ++j) {
        idx[j] = sel[j];
        w[j] = p[sel[j]] / zs;                      /* renormalise over the selection */
    }
    free(order);
    free(p);
}

void orc_route(const orc_layer *L, const uint16_t *x, int64_t T, int32_t *idx, double *w,
               double *gap)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        double *l = (double *)malloc(sizeof(double) * L->n_experts);
        logits_one(L, x + t * L->hidden, l);
        route_one(L, l, idx + t * L->top_k, w + t * L->top_k, gap ? gap + t : NULL);
        free(l);
    }
}

/* --------------------------------------------------------------------- expert MLP */

static double silu(double z) { return z / (1.0 + exp(-z)); }

void orc_expert_mlp(const orc_layer *L, const orc_qmat *g, const orc_qmat *u,
                    const orc_qmat *d, int64_t e, const double *x, double *o)
{
    const int64_t H = L->hidden, I = L->inter;
    double *h = (double *)malloc(sizeof(double) * I);
    for (int64_t i = 0; i < I; ++i) {
        double gi = 0.0, ui = 0.0;
        for (int64_t c = 0; c < H; ++c) {
            gi += weight(g, L->bits, e, i, c, H) * x[c];
            ui += weight(u, L->bits, e, i, c, H) * x[c];
        }
        h[i] = silu(gi) * ui;
    }
    for (int64_t n = 0; n < H; ++n) {
        double acc = 0.0;
        for (int64_t i = 0; i < I; ++i)
            acc += weight(d, L->bits, e, n, i, I) * h[i];
        o[n] = acc;
    }
    free(h);
}

/* --------------------------------------------------------------------- the layer */

void orc_layer_forward_with_routing(const orc_layer *L, const uint16_t *x, int64_t T,
                                    const int32_t *idx, const double *w, double *y)
{
    const int64_t H = L->hidden;
    const int k = L->top_k;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        double *xt = (double *)malloc(sizeof(double) * H);
        double *o = (double *)malloc(sizeof(double) * H);
        double *yt = y + t * H;
        for (int64_t c = 0; c < H; ++c) { xt[c] = orc_bf16_to_double(x[t * H + c]); yt[c] = 0.0; }
        for (int j = 0; j < k; ++j) {
            int64_t e = idx[t * k + j];
            orc_expert_mlp(L, &L->gate, &L->up, &L->down, e, xt, o);
            for (int64_t c = 0; c < H; ++c) yt[c] += w[t * k + j] * o[c];
        }
        if (L->has_shared) {
            orc_expert_mlp(L, &L->s_gate, &L->s_up, &L->s_down, 0, xt, o);
            double gs = 1.0;
            if (L->shared_gate_w) {
                double z = 0.0;
                for (int64_t c = 0; c < H; ++c) z += orc_bf16_to_double(L->shared_gate_w[c]) * xt[c];
                gs = 1.0 / (1.0 + exp(-z));
            }
            for (int64_t c = 0; c < H; ++c) yt[c] += gs * o[c];
        }
        free(xt);
        free(o);
    }
}

void orc_layer_forward(const orc_layer *L, const uint16_t *x, int64_t T, double *y,
                       int32_t *idx, double *w)
{
    const int k = L->top_k;
    int32_t *ii = idx ? idx : (int32_t *)malloc(sizeof(int32_t) * (size_t)(T * k + 1));
    double *ww = w ? w : (double *)malloc(sizeof(double) * (size_t)(T * k + 1));
    orc_route(L, x, T, ii, ww, NULL);
    orc_layer_forward_with_routing(L, x, T, ii, ww, y);
    if (!idx) free(ii);
    if (!w) free(ww);
}

/* -------------------------------------------------------------------------- Q8_0 */

#define Q8_BLOCK_BYTES 34   /* [fp16 d][32 x int8] */
#define Q8_TILE_BYTES 544   /* 16 blocks, re-ordered */

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

void orc_q8_gemv(const uint8_t *rows, int64_t N, int64_t K, const uint16_t *x, double *y)
{
    const int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = rows + (n * nb + b) * Q8_BLOCK_BYTES;
            double d = orc_f16_to_double(rd16(blk));
            double dot = 0.0;
            for (int c = 0; c < 32; ++c)
                dot += (double)(int8_t)blk[2 + c] * orc_bf16_to_double(x[b * 32 + c]);
            acc += d * dot;
        }
        y[n] = acc;
    }
}

/* byte offset, inside a tile, of code c (0..31) of tile row r (0..15) */
static int64_t tile_code_offset(int r, int c) { return (int64_t)(c / 4) * 64 + r * 4 + (c % 4); }

void orc_q8_pack_rows16(const uint8_t *rows, int64_t N, int64_t K, uint8_t *tiles)
{
    const int64_t nb = K / 32;
    for (int64_t p = 0; p < N / 16; ++p)
        for (int64_t b = 0; b < nb; ++b) {
            uint8_t *tile = tiles + (p * nb + b) * Q8_TILE_BYTES;
            for (int r = 0; r < 16; ++r) {
                const uint8_t *blk = rows + ((p * 16 + r) * nb + b) * Q8_BLOCK_BYTES;
                for (int c = 0; c < 32; ++c) tile[tile_code_offset(r, c)] = blk[2 + c];
                tile[512 + 2 * r] = blk[0];
                tile[512 + 2 * r + 1] = blk[1];
            }
        }
}

void orc_q8_unpack_rows16(const uint8_t *tiles, int64_t N, int64_t K, uint8_t *rows)
{
    const int64_t nb = K / 32;
    for (int64_t p = 0; p < N / 16; ++p)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *tile = tiles + (p * nb + b) * Q8_TILE_BYTES;
            for (int r = 0; r < 16; ++r) {
                uint8_t *blk = rows + ((p * 16 + r) * nb + b) * Q8_BLOCK_BYTES;
                for (int c = 0; c < 32; ++c) blk[2 + c] = tile[tile_code_offset(r, c)];
                blk[0] = tile[512 + 2 * r];
                blk[1] = tile[512 + 2 * r + 1];
            }
        }
}

/* d = max|v| / 127 computed in binary32 and stored as binary16;
 * q = v / d (binary32, the unrounded d) rounded half away from zero, clamped. */
void orc_q8_quantize_row(const float *v, int64_t K, uint8_t *blocks)
{
    for (int64_t b = 0; b < K / 32; ++b) {
        const float *vb = v + b * 32;
        uint8_t *blk = blocks + b * Q8_BLOCK_BYTES;
        float amax = 0.0f;
        for (int c = 0; c < 32; ++c) {
            float a = fabsf(vb[c]);
            if (a > amax) amax = a;
        }
        float d = amax / 127.0f;
        uint16_t dh = double_to_f16((double)d);
        blk[0] = (uint8_t)(dh & 0xff);
        blk[1] = (uint8_t)(dh >> 8);
        for (int c = 0; c < 32; ++c) {
            float qf = (d != 0.0f) ? vb[c] / d : 0.0f;
            float r = (qf >= 0.0f) ? floorf(qf + 0.5f) : -floorf(-qf + 0.5f);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            blk[2 + c] = (uint8_t)(int8_t)r;
        }
    }
}

void orc_q8_dequantize_row(const uint8_t *blocks, int64_t K, double *v)
{
    for (int64_t b = 0; b < K / 32; ++b) {
        const uint8_t *blk = blocks + b * Q8_BLOCK_BYTES;
        double d = orc_f16_to_double(rd16(blk));
        for (int c = 0; c < 32; ++c) v[b * 32 + c] = d * (double)(int8_t)blk[2 + c];
    }
}

/* Activation quantization shared by the projections that read one vector ([EMBER]:
 * Q/K/V, and gate/up, read one quantized copy of their input).  Each block of 32 values
 * becomes a Q8_0 block: d = max|x| / 127 in binary32, stored as binary16; q = x / d in
 * binary32 (the unrounded d), rounded half away from zero (roundf), clamped to
 * [-127, 127]; an all-zero block has d = 0 and q = 0.  The codes are an integer
 * decision, taken in binary32 on both sides. */
void orc_q8_quantize_x(const uint16_t *x, int64_t K, int8_t *q, uint16_t *d)
{
    for (int64_t b = 0; b < K / 32; ++b) {
        float v[32], amax = 0.0f;
        for (int c = 0; c < 32; ++c) {
            v[c] = (float)orc_bf16_to_double(x[b * 32 + c]);      /* exact */
            if (fabsf(v[c]) > amax) amax = fabsf(v[c]);
        }
        const float db = amax / 127.0f;
        d[b] = double_to_f16((double)db);
        for (int c = 0; c < 32; ++c) {
            float r = (db != 0.0f) ? roundf(v[c] / db) : 0.0f;
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q[b * 32 + c] = (int8_t)r;
        }
    }
}

/* Q8_0 GEMV with a Q8_0 activation: y[n] = sum_b dw[n,b] dx[b] sum_c qw[n,32b+c] qx[32b+c],
 * the integer dot exact, the rest in fp64 (rows row-contiguous, as orc_q8_gemv). */
void orc_q8_gemv_q8x(const uint8_t *rows, int64_t N, int64_t K, const int8_t *xq, const uint16_t *xd,
                     double *y)
{
    const int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = rows + (n * nb + b) * Q8_BLOCK_BYTES;
            int64_t dot = 0;
            for (int c = 0; c < 32; ++c) dot += (int64_t)(int8_t)blk[2 + c] * (int64_t)xq[b * 32 + c];
            acc += orc_f16_to_double(rd16(blk)) * orc_f16_to_double(xd[b]) * (double)dot;
        }
        y[n] = acc;
    }
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
