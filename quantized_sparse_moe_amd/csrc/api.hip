// api.hip -- the C ABI of libqsmoe (declared in include/qsmoe.h): host-side validation,
// workspace carving and the launch sequence on the caller's stream.
//
// [LILY] "Keep expert routing on the GPU": a layer call enqueues its whole sequence
// (router, binning, expert GEMMs, combine) and never waits for the device.
// [OMLX] "_can_fuse": eligibility is checked up front (equal group size and bits,
// matching shapes); unlike that patch, an ineligible layer is an error here, never a
// silent fallback to a second code path.
// [EMBER]: decode reuses one caller-provided workspace instead of per-layer temporaries.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "internal.h"

using namespace qs;

namespace {

constexpr size_t ALIGN = 256;

inline size_t up(size_t n) { return (n + ALIGN - 1) / ALIGN * ALIGN; }

inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status check_qmat(const moe_qmat &m, int64_t rows) {
    if (!m.codes || !m.scales || !m.biases) return MOE_ERR_INVALID;
    if (!aligned(m.codes, 16) || !aligned(m.scales, 2) || !aligned(m.biases, 2)) return MOE_ERR_INVALID;
    if (m.mat_stride < rows) return MOE_ERR_INVALID;
    return MOE_OK;
}

moe_status check_desc(const moe_layer_desc *d) {
    if (!d) return MOE_ERR_INVALID;
    if (d->group != 64 || (d->bits != 4 && d->bits != 8) ||
        (d->scale_dtype != MOE_F16 && d->scale_dtype != MOE_BF16))
        return MOE_ERR_UNSUPPORTED;
    if (d->n_experts < 1 || d->n_experts > 256) return MOE_ERR_UNSUPPORTED;
    if (d->top_k < 1 || d->top_k > 16 || d->top_k > d->n_experts) return MOE_ERR_UNSUPPORTED;
    if (d->hidden < 64 || d->hidden > 8192 || d->hidden % 64) return MOE_ERR_UNSUPPORTED;
    if (d->inter < 64 || d->inter > 2048 || d->inter % 64) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)(d->top_k + 1) * d->inter > 24576) return MOE_ERR_UNSUPPORTED;
    if (!d->router_w || !aligned(d->router_w, 16)) return MOE_ERR_INVALID;
    if (d->router_bias && !aligned(d->router_bias, 4)) return MOE_ERR_INVALID;
    if (d->has_shared != 0 && d->has_shared != 1) return MOE_ERR_INVALID;
    if (d->shared_gate_w && (!d->has_shared || !aligned(d->shared_gate_w, 16))) return MOE_ERR_INVALID;
    moe_status s;
    if ((s = check_qmat(d->gate, d->inter)) || (s = check_qmat(d->up, d->inter)) ||
        (s = check_qmat(d->down, d->hidden)))
        return s;
    if (d->has_shared &&
        ((s = check_qmat(d->s_gate, d->inter)) || (s = check_qmat(d->s_up, d->inter)) ||
         (s = check_qmat(d->s_down, d->hidden))))
        return s;
    return MOE_OK;
}

QMat to_qmat(const moe_qmat &m) {
    QMat q;
    q.codes = (const uint8_t *)m.codes;
    q.scales = (const uint16_t *)m.scales;
    q.biases = (const uint16_t *)m.biases;
    q.stride = m.mat_stride;
    return q;
}

Layer to_layer(const moe_layer_desc *d) {
    Layer L;
    L.H = d->hidden;
    L.I = d->inter;
    L.E = d->n_experts;
    L.K = d->top_k;
    L.bits = d->bits;
    L.router_w = (const uint16_t *)d->router_w;
    L.router_bias = d->router_bias;
    L.gate = to_qmat(d->gate);
    L.up = to_qmat(d->up);
    L.down = to_qmat(d->down);
    L.has_shared = d->has_shared;
    if (d->has_shared) {
        L.s_gate = to_qmat(d->s_gate);
        L.s_up = to_qmat(d->s_up);
        L.s_down = to_qmat(d->s_down);
    } else {
        L.s_gate = L.s_up = L.s_down = QMat{nullptr, nullptr, nullptr, 0};
    }
    L.sb_bf16 = d->scale_dtype == MOE_BF16;
    L.shared_gate_w = (const uint16_t *)d->shared_gate_w;
    return L;
}

// ---------------------------------------------------------------- workspace layouts
struct Carver {
    char *base;
    size_t off = 0;
    template <typename T>
    T *take(size_t count) {
        T *p = base ? (T *)(base + off) : nullptr;
        off += up(count * sizeof(T));
        return p;
    }
};

DecodeBufs carve_decode(const moe_layer_desc *d, void *ws, size_t *bytes) {
    Carver c{(char *)ws};
    DecodeBufs b;
    b.ctl = c.take<uint32_t>(WS_CTL_BYTES / 4);
    *bytes = c.off;
    return b;
}

PrefillBufs carve_prefill(const moe_layer_desc *d, int64_t T, void *ws, size_t *bytes) {
    Carver c{(char *)ws};
    const int64_t H = d->hidden, I = d->inter, K = d->top_k, E = d->n_experts;
    const int64_t nblk = (T + ROUTER_TOKENS - 1) / ROUTER_TOKENS;
    PrefillBufs b;
    b.ctl = c.take<uint32_t>(WS_CTL_BYTES / 4);      // decode state stays untouched (but word 0)
    b.x16 = c.take<uint16_t>((size_t)(T * H));
    b.xmax = c.take<uint32_t>((size_t)(T * 8));
    b.xexp = c.take<int32_t>((size_t)T);
    b.logits = c.take<float>((size_t)(T * (E + 1)));     // + the shared-expert gate's logit
    b.idx = c.take<int32_t>((size_t)(T * K));
    b.w = c.take<float>((size_t)(T * K));
    b.blkcnt = c.take<int32_t>((size_t)(nblk * E));
    b.blkoff = c.take<int32_t>((size_t)(nblk * E));
    b.expert_off = c.take<int32_t>((size_t)(2 * E + 1));
    b.perm = c.take<int32_t>((size_t)(T * K));
    b.tiles = c.take<Tile>((size_t)prefill_max_tiles(T, (int)K, (int)E));
    b.ntiles = c.take<int32_t>(3);
    b.tile_done = c.take<int32_t>((size_t)prefill_max_tiles(T, (int)K, (int)E));
    b.h = c.take<uint16_t>((size_t)((T * K + T) * I));
    b.hexp = c.take<int8_t>((size_t)((T * K + T) * HEXP_STRIDE));
    b.slot = c.take<uint16_t>((size_t)((T * K + T) * H));
    b.sexp = c.take<int8_t>((size_t)(sexp_rows(T, (int)K) * (H / 64)));
    b.sgate = c.take<float>((size_t)T);
    *bytes = c.off;
    return b;
}

// T >= 2 runs in chunks, one after another on the stream, each through the whole
// prefill sequence in the same workspace: chunks of `chunk` tokens need this much
size_t ws_size_chunked(const moe_layer_desc *d, int64_t T, int64_t chunk) {
    size_t n = 0;
    if (T <= 0) return 0;
    if (T == 1) carve_decode(d, nullptr, &n);
    else carve_prefill(d, T < chunk ? T : chunk, nullptr, &n);
    return n;
}
size_t ws_size(const moe_layer_desc *d, int64_t T) { return ws_size_chunked(d, T, MOE_PREFILL_CHUNK); }

// the smallest chunk a workspace may be sized for
constexpr int64_t MIN_CHUNK = 2;

// the largest chunk whose buffers fit in ws_bytes (check_ws has made sure MIN_CHUNK fits)
int64_t pick_chunk(const moe_layer_desc *d, int64_t T, size_t ws_bytes) {
    if (ws_size_chunked(d, T, T) <= ws_bytes) return T;
    int64_t lo = MIN_CHUNK, hi = T;                   // lo fits, hi does not
    while (hi - lo > 1) {
        const int64_t mid = lo + (hi - lo) / 2;
        if (ws_size_chunked(d, T, mid) <= ws_bytes) lo = mid;
        else hi = mid;
    }
    return lo;
}

moe_status check_ws(const moe_layer_desc *d, int64_t T, void *ws, size_t ws_bytes) {
    if (!ws || !aligned(ws, ALIGN)) return MOE_ERR_WORKSPACE;
    if (ws_bytes < ws_size_chunked(d, T, MIN_CHUNK)) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

inline moe_status dev(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

// Batches of SMALL_TMAX + 1 .. 2 SMALL_TMAX tokens (verification batches of a few rows) run
// as two small-batch launches of ceil(T/2) and floor(T/2) tokens: a token's result depends
// only on its own row, so the split changes the time, not the values. Returns the first
// part's size, or 0 when the grouped path is taken.
static int64_t small_split(const Layer &L, int64_t T) {
    const int64_t T0 = (T + 1) / 2;
    if (T <= SMALL_TMAX || T > 2 * SMALL_TMAX) return 0;
    return decode_small_eligible(L, T0) && decode_small_eligible(L, T - T0) ? T0 : 0;
}

// tokens * hidden must stay addressable with the kernels' 32-bit row offsets
constexpr int64_t MAX_TOKENS = 1 << 20;

// the argument checks of a layer call (workspace aside), all on the host; T == 0 passes
moe_status check_layer_call(const moe_layer_desc *d, const void *x, int64_t T, const void *y, int32_t y_dtype,
                            const int32_t *topk_idx, const float *topk_w) {
    moe_status s = check_desc(d);
    if (s) return s;
    if (T < 0) return MOE_ERR_INVALID;
    if (T > MAX_TOKENS) return MOE_ERR_UNSUPPORTED;
    if (y_dtype != MOE_BF16 && y_dtype != MOE_F32) return MOE_ERR_INVALID;
    if (T == 0) return MOE_OK;
    if (!x || !aligned(x, 16) || !y || !aligned(y, y_dtype == MOE_F32 ? 4 : 2)) return MOE_ERR_INVALID;
    if ((topk_idx && !aligned(topk_idx, 4)) || (topk_w && !aligned(topk_w, 4))) return MOE_ERR_INVALID;
    return MOE_OK;
}

moe_status forward_impl(const moe_layer_desc *d, const void *x, int64_t T, void *y, int32_t y_dtype,
                        int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes, void *stream) {
    moe_status s = check_layer_call(d, x, T, y, y_dtype, topk_idx, topk_w);
    if (s || T == 0) return s;
    if ((s = check_ws(d, T, ws, ws_bytes))) return s;
    const Layer L = to_layer(d);
    hipStream_t st = (hipStream_t)stream;
    const uint16_t *xx = (const uint16_t *)x;
    hipError_t e;
    if (T == 1) {
        size_t n;
        const DecodeBufs b = carve_decode(d, ws, &n);
        return dev(launch_decode_layer(L, xx, b, y, y_dtype, topk_idx, topk_w, st));
    }
    if (decode_small_eligible(L, T)) {
        size_t n;
        const DecodeBufs b = carve_decode(d, ws, &n);
        return dev(launch_decode_small_layer(L, xx, T, b, y, y_dtype, topk_idx, topk_w, st));
    }
    if (const int64_t T0 = small_split(L, T)) {
        size_t n;
        const DecodeBufs b = carve_decode(d, ws, &n);
        const int64_t K = d->top_k, H = d->hidden;
        void *y1 = (char *)y + (size_t)(T0 * H) * (y_dtype == MOE_F32 ? 4 : 2);
        e = launch_decode_small_layer(L, xx, T0, b, y, y_dtype, topk_idx, topk_w, st);
        if (e == hipSuccess)
            e = launch_decode_small_layer(L, xx + T0 * H, T - T0, b, y1, y_dtype, topk_idx ? topk_idx + T0 * K : nullptr,
                                          topk_w ? topk_w + T0 * K : nullptr, st);
        return dev(e);
    }
    // chunks of the prefill sequence: every token goes through the same kernels whatever
    // the chunk it falls in, so the result is bit-identical to one unchunked pass
    size_t n;
    const int64_t C = pick_chunk(d, T, ws_bytes), K = d->top_k, H = d->hidden;
    const PrefillBufs b = carve_prefill(d, C, ws, &n);
    const size_t ysz = y_dtype == MOE_F32 ? 4 : 2;
    for (int64_t t0 = 0; t0 < T; t0 += C) {
        const int64_t Tc = T - t0 < C ? T - t0 : C;
        void *yc = (char *)y + (size_t)(t0 * H) * ysz;
        e = launch_prefill_router(L, xx + t0 * H, Tc, b, true, topk_idx ? topk_idx + t0 * K : nullptr,
                                  topk_w ? topk_w + t0 * K : nullptr, st);
        if (e == hipSuccess) e = launch_prefill_binning(L, Tc, b, st);
        if (e == hipSuccess) e = launch_prefill_gemms(L, Tc, b, yc, y_dtype, st);
        if (e != hipSuccess) return MOE_ERR_DEVICE;
    }
    return MOE_OK;
}

// The static scratch of moe_layer_forward_static: device memory beyond the inputs and
// outputs for callers that cannot allocate (code under HIP graph capture, tight serving
// loops).  Each GPU holds its own copy from module load until the process ends; it is
// zero at load (static storage), so the decode state at its start begins valid, and every
// call leaves that state ready for the next one.  In host code `scratch` is only a
// stand-in for the symbol: its device address comes from hipGetSymbolAddress, once per
// device with that device current, and only that address is handed to kernels.
constexpr size_t SCRATCH_BYTES = 64u << 20;
static __device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::atomic<void *> scratch_ptr[MAX_DEVICES];
std::mutex scratch_mu;

moe_status scratch_for_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return MOE_ERR_DEVICE;
    void *p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> g(scratch_mu);
        p = scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_DEVICE;
            scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID: return "invalid argument (null or misaligned pointer, bad size or enum)";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or format";
        case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case MOE_ERR_DEVICE: return "HIP launch failed";
        default: return "unknown status";
    }
}

size_t moe_workspace_size(const moe_layer_desc *d, int64_t T) {
    if (check_desc(d) != MOE_OK) return SIZE_MAX;
    if (T > MAX_TOKENS) return SIZE_MAX;
    return ws_size(d, T);
}

size_t moe_workspace_size_chunked(const moe_layer_desc *d, int64_t T, int64_t chunk) {
    if (check_desc(d) != MOE_OK) return SIZE_MAX;
    if (T > MAX_TOKENS || chunk < 0) return SIZE_MAX;
    if (chunk == 0) chunk = MOE_PREFILL_CHUNK;
    return ws_size_chunked(d, T, chunk < MIN_CHUNK ? MIN_CHUNK : chunk);
}

moe_status moe_workspace_status(void *ws, size_t ws_bytes, uint32_t *status_out, int32_t clear, void *stream) {
    if (!ws || !aligned(ws, ALIGN) || !status_out || !aligned(status_out, 4)) return MOE_ERR_INVALID;
    if (ws_bytes < WS_CTL_BYTES) return MOE_ERR_WORKSPACE;
    return dev(launch_ws_status((uint32_t *)ws, status_out, clear != 0, (hipStream_t)stream));
}

moe_status moe_route(const moe_layer_desc *d, const void *x, int64_t T, int32_t *topk_idx,
                       float *topk_w, void *ws, size_t ws_bytes, void *stream) {
    moe_status s = check_desc(d);
    if (s) return s;
    if (T < 0) return MOE_ERR_INVALID;
    if (T > MAX_TOKENS) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !aligned(x, 16) || !topk_idx || !topk_w || !aligned(topk_idx, 4) || !aligned(topk_w, 4))
        return MOE_ERR_INVALID;
    if ((s = check_ws(d, T, ws, ws_bytes))) return s;
    const Layer L = to_layer(d);
    hipStream_t st = (hipStream_t)stream;
    if (T == 1) {
        size_t n;
        const DecodeBufs b = carve_decode(d, ws, &n);
        return dev(launch_decode_route(L, (const uint16_t *)x, b, topk_idx, topk_w, st));
    }
    if (decode_small_eligible(L, T)) {
        size_t n;
        const DecodeBufs b = carve_decode(d, ws, &n);
        return dev(launch_decode_small_route(L, (const uint16_t *)x, T, b, topk_idx, topk_w, st));
    }
    if (const int64_t T0 = small_split(L, T)) {
        size_t n;
        const DecodeBufs b = carve_decode(d, ws, &n);
        const int64_t K = d->top_k;
        const uint16_t *xx = (const uint16_t *)x;
        hipError_t e = launch_decode_small_route(L, xx, T0, b, topk_idx, topk_w, st);
        if (e == hipSuccess)
            e = launch_decode_small_route(L, xx + T0 * d->hidden, T - T0, b, topk_idx + T0 * K, topk_w + T0 * K, st);
        return dev(e);
    }
    size_t n;
    const int64_t C = pick_chunk(d, T, ws_bytes), K = d->top_k, H = d->hidden;
    PrefillBufs b = carve_prefill(d, C, ws, &n);
    for (int64_t t0 = 0; t0 < T; t0 += C) {
        const int64_t Tc = T - t0 < C ? T - t0 : C;
        b.idx = topk_idx + t0 * K;
        b.w = topk_w + t0 * K;
        const hipError_t e = launch_prefill_router(L, (const uint16_t *)x + t0 * H, Tc, b, false, nullptr, nullptr, st);
        if (e != hipSuccess) return MOE_ERR_DEVICE;
    }
    return MOE_OK;
}

moe_status moe_layer_forward(const moe_layer_desc *d, const void *x, int64_t T, void *y, int32_t y_dtype,
                             int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes, void *stream) {
    return forward_impl(d, x, T, y, y_dtype, topk_idx, topk_w, ws, ws_bytes, stream);
}

moe_status moe_layer_forward_static(const moe_layer_desc *d, const void *x, int64_t T, void *y, int32_t y_dtype,
                                    int32_t *topk_idx, float *topk_w, void *stream) {
    // the argument checks of moe_layer_forward come first, so a call that is refused
    // touches no device
    moe_status s = check_layer_call(d, x, T, y, y_dtype, topk_idx, topk_w);
    if (s || T == 0) return s;
    if (ws_size_chunked(d, T, MIN_CHUNK) > SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    void *ws = nullptr;
    if ((s = scratch_for_current_device(&ws))) return s;
    return forward_impl(d, x, T, y, y_dtype, topk_idx, topk_w, ws, SCRATCH_BYTES, stream);
}

moe_status q8_gemv(const void *w_tiles, int64_t N, int64_t K, const void *x, void *y,
                     int32_t y_dtype, void *stream) {
    if (N < 0 || K < 0) return MOE_ERR_INVALID;
    if (y_dtype != MOE_BF16 && y_dtype != MOE_F32) return MOE_ERR_INVALID;
    if (N % 16 || K % 32 || N < 16 || K < 32 || K > 8192 || N / 16 > INT32_MAX)
        return MOE_ERR_UNSUPPORTED;
    if (!w_tiles || !aligned(w_tiles, 16) || !x || !aligned(x, 16) || !y ||
        !aligned(y, y_dtype == MOE_F32 ? 4 : 2))
        return MOE_ERR_INVALID;
    return dev(launch_q8_gemv((const uint8_t *)w_tiles, N, K, (const uint16_t *)x, y, y_dtype,
                              (hipStream_t)stream));
}

moe_status q8_quantize_x(const void *x, int64_t K, void *xq, void *xd, void *stream) {
    if (K < 0) return MOE_ERR_INVALID;
    if (K % 32 || K > 8192) return MOE_ERR_UNSUPPORTED;
    if (K == 0) return MOE_OK;
    if (!x || !aligned(x, 2) || !xq || !aligned(xq, 4) || !xd || !aligned(xd, 2)) return MOE_ERR_INVALID;
    return dev(launch_q8_quantize_x((const uint16_t *)x, K, (int8_t *)xq, (uint16_t *)xd, (hipStream_t)stream));
}

moe_status q8_gemv_q8x(const void *w_tiles, int64_t N, int64_t K, const void *xq, const void *xd, void *y,
                         int32_t y_dtype, void *stream) {
    if (N < 0 || K < 0) return MOE_ERR_INVALID;
    if (y_dtype != MOE_BF16 && y_dtype != MOE_F32) return MOE_ERR_INVALID;
    if (N % 16 || K % 32 || N < 16 || K < 32 || K > 8192 || N / 16 > INT32_MAX)
        return MOE_ERR_UNSUPPORTED;
    if (!w_tiles || !aligned(w_tiles, 16) || !xq || !aligned(xq, 4) || !xd || !aligned(xd, 2) || !y ||
        !aligned(y, y_dtype == MOE_F32 ? 4 : 2))
        return MOE_ERR_INVALID;
    return dev(launch_q8_gemv_q8x((const uint8_t *)w_tiles, N, K, (const int8_t *)xq, (const uint16_t *)xd,
                                  nullptr, y, y_dtype, (hipStream_t)stream));
}

moe_status q8_gemv_qx(const void *w_tiles, int64_t N, int64_t K, const void *x, void *y, int32_t y_dtype,
                        void *stream) {
    if (N < 0 || K < 0) return MOE_ERR_INVALID;
    if (y_dtype != MOE_BF16 && y_dtype != MOE_F32) return MOE_ERR_INVALID;
    if (N % 16 || K % 32 || N < 16 || K < 32 || K > 8192 || N / 16 > INT32_MAX)
        return MOE_ERR_UNSUPPORTED;
    if (!w_tiles || !aligned(w_tiles, 16) || !x || !aligned(x, 8) || !y || !aligned(y, y_dtype == MOE_F32 ? 4 : 2))
        return MOE_ERR_INVALID;
    return dev(launch_q8_gemv_q8x((const uint8_t *)w_tiles, N, K, nullptr, nullptr, (const uint16_t *)x, y,
                                  y_dtype, (hipStream_t)stream));
}

moe_status q8_pack_rows16(const void *w_rows, int64_t N, int64_t K, void *w_tiles, void *stream) {
    if (N < 0 || K < 0) return MOE_ERR_INVALID;
    if (N % 16 || K % 32) return MOE_ERR_UNSUPPORTED;
    if (N == 0 || K == 0) return MOE_OK;
    if (!w_rows || !w_tiles || !aligned(w_tiles, 16)) return MOE_ERR_INVALID;
    const size_t bytes = (size_t)N * (size_t)(K / 32) * 34;
    const uintptr_t a = (uintptr_t)w_rows, b = (uintptr_t)w_tiles;
    if (a < b + bytes && b < a + bytes) return MOE_ERR_INVALID;   // overlap
    return dev(launch_q8_pack((const uint8_t *)w_rows, N, K, (uint8_t *)w_tiles, (hipStream_t)stream));
}

moe_status moe_calib_read(const void *buf, size_t bytes, void *stream) {
    if (!buf || !aligned(buf, 16) || bytes % 16) return MOE_ERR_INVALID;
    if (bytes == 0) return MOE_OK;
    return dev(launch_calib_read(buf, (int64_t)bytes, nullptr, (hipStream_t)stream));
}

moe_status moe_calib_mfma(int32_t iters, int32_t blocks, void *stream) {
    if (iters < 0 || blocks < 0) return MOE_ERR_INVALID;
    if (iters == 0 || blocks == 0) return MOE_OK;
    return dev(launch_calib_mfma(iters, blocks, nullptr, (hipStream_t)stream));
}

}  // extern "C"
