// gemm.hip -- grouped expert GEMMs of the prefill path on MFMA (gfx950).
//
// [LILY] "Dequantize weights during matrix multiplication": the quantized weights are
// never expanded in memory; each workgroup dequantizes the weight tile it is about to
// multiply, straight into MFMA operand registers, with fp32 accumulation.
// [LILY] "Keep expert routing on the GPU" / "Match tile size to expert load": work is
// enumerated as (expert row block, column block) items from the device-side block map.
// [OMLX] "Fusion principle": gate row j and up row j of one expert are handled by the
// same wave, so SwiGLU is formed in registers and only h leaves the kernel.
//
// Tile: 160 activation rows x 256 weight rows, K step 64 (one quantization group), four
// waves, each owning 64 weight rows (four 16-row MFMA subtiles) against all 160 rows
// (ten subtiles): 40 v_mfma_f32_16x16x32_f16 per 32-wide K slice.  160 rows take an
// expert's whole bin in one tile at the mean load of the prefill workload (128 rows per
// expert, uneven), where 128-row tiles left a sliver tile behind half of the experts that
// costs a full pass of dequantization for a few rows.  Every tile runs all ten subtiles
// (rows past the tile repeat a valid row and are discarded): per-subtile branches cost
// more than the idle MFMAs.
//
// Data movement: every operand of a K step -- the activation rows (fp16), the weight
// codes, scales and biases -- goes global -> LDS by direct-to-LDS loads
// (global_load_lds), which take no registers and no ALU.  Scales and biases come 8 groups
// (16 bytes) per row at a time every 8 K steps (4-bit; 2 groups for 8-bit, whose larger
// code stages leave less LDS): a per-step 2-byte load per row costs the address unit as
// much as a 16-byte one.  A ring of two stages holds the K step being multiplied and the
// next one in flight; each wave waits only for its own loads (vmcnt) and one barrier per
// step publishes the stage to the whole workgroup.  The position of each 16-byte chunk of
// an activation row in LDS is XOR-swizzled by row (a_swizzle), so that the fragment reads
// are free of bank conflicts (direct-to-LDS loads place lane l at byte 16 l, so the
// swizzle is chosen by which global chunk each lane fetches).
//
// Operands: activations fp16 (x copy from the router, h from the gate/up pass) with
// each group of 8 columns permuted into the order the packed codes unpack in (see
// common.h); weights fp16 w = fma(s, q, b) with q recovered exactly from the codes by
// the 1024-magic.  (fp16 rather than bf16 operands: at these sizes weights rounded to
// bf16 leave ~2e-2 x RMS of error in the layer output, fp16 ~2e-3; the matrix rate is
// the same.)
//
// Range: fp16 holds neither bf16's range nor every product of the layer, so every fp16
// operand carries an exact power-of-two scale, removed in fp32 after the MFMAs.
//   - x: per token (x16 row t is x 2^a_t, chosen by the router).
//   - weights: per wave (its 64 weight rows), 2^p with p set before the K loop from a
//     bound on their |w| (max over rows and groups of |s| (2^bits - 1) + |b|), so the
//     largest weight lies in [2^14, 2^15); p = 0 (scales used as loaded) when fp16
//     scales already keep every weight and every s / 16 in fp16's normal range.  Scales
//     and biases are converted to fp16 s 2^p, b 2^p when their window lands in LDS, by
//     the thread that loaded them (bf16 or fp16 in; exact), and s 2^p / 16 stays normal
//     for every group within 2^24 of the largest.
//     The factor is taken out with the row factors, at no cost per element.
//   - h: per (row, 128-column block), 2^e with e from the block's largest |h|: 0 for
//     blocks in [2^-2, 2^15), else a multiple of 8 (blocks of similar magnitude share
//     it).  The down pass multiplies h row r under the smallest e_r of its blocks: a tile
//     whose rows all have one e per row reads h as it is; otherwise each wave rescales
//     the chunks it loaded by 2^(e_r - e) in LDS before the stage is published.
//   - slot rows: per (row, 64-column block), 2^e from the block's largest value, taken
//     out by the combine.
// With every scale 0 (ordinary data) the arithmetic is exactly that of unscaled fp16.
//
// Modes: 0 = [gate; up] + SwiGLU -> h (routed rows gathered through perm, shared rows
// direct); 1 = down projection: routed tiles -> slot row t*k + j = w_tj * o (fp16),
// shared tiles -> slot row T*k + t, in one launch (the shared tiles, full ones, first, so
// the ragged routed tiles fill the last round).  k_combine then adds each token's k slot rows in
// ascending expert order and its shared row, in fp32, and writes y: a deterministic,
// atomic-free combine.
#include "common.h"
#include "internal.h"

namespace qs {

namespace {

constexpr int BM = GEMM_BM;          // activation rows per tile
constexpr int MT = BM / 16;          // 16-row subtiles
constexpr int BN = 256;              // weight rows per workgroup
constexpr int BK = 64;               // K step
constexpr int NT = 256;              // threads (4 waves)

template <int BITS>
struct Cfg {
    static constexpr int A_BYTES = BM * BK * 2;               // fp16 rows, 128 B each
    static constexpr int B_BYTES = BN * BK * BITS / 8;        // codes, 32 or 64 B per row
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int NSTAGE = 2;                          // two workgroups per CU fit
    // scales and biases: a ring of two windows of up to WMAX groups per row (16 or 4 bytes)
    static constexpr int WMAX = BITS == 4 ? 8 : 2;
    static constexpr int S_BYTES = BN * (WMAX == 8 ? 16 : 4); // one window of scales (or biases)
    static constexpr int B_DMA = B_BYTES / 1024 / 4;          // per wave and stage
    static constexpr int A_DMA = MT / 2;                      // 8-row pieces per wave and stage
    static constexpr int DMA = A_DMA + B_DMA + 2;             // A, codes, scales, biases
    static constexpr int LDS = NSTAGE * STAGE + 4 * S_BYTES;
};
static_assert(Cfg<4>::NSTAGE == 2 && Cfg<8>::NSTAGE == 2, "every stage wait is a full drain (vmcnt 0)");
// the gate/up epilogue's staging (four waves' h rows, row maxima, block scales and their
// factors) and the down epilogue's fit in the ring
static_assert(4 * GEMM_BM * 40 * 2 + 4 * GEMM_BM * 4 + (GEMM_BM + 15) / 16 * 16 + GEMM_BM * 4 <= Cfg<4>::LDS &&
                  4 * (32 * 68 * 4) <= Cfg<4>::LDS, "epilogue staging");

struct GemmArgs {
    Layer L;
    int64_t T;
    const uint16_t *x16;             // [T][H] fp16 (permuted); row t is x_t 2^xexp[t]
    const int32_t *xexp;             // [T]
    uint16_t *h;                     // [(T*K + T)][I] fp16 (permuted), per-block scaled
    int8_t *hexp;                    // [HEXP_STRIDE][T*K + T] the scale of each 128-column block
    const int32_t *perm;
    const Tile *tiles;
    int32_t *ntiles;                 // tile counts; [2] = 1 once a down workgroup stored a scaled slot block
    const float *w;                  // [T*K]
    uint16_t *slot;                  // [T*K + T][H]
    int8_t *sexp;                    // [H / 64][sexp_rows(T, K)]
    void *y;
    int y_dtype;
    int nb;                          // column blocks per tile
    int wlog;                        // log2 of the scale / bias window (groups per row per load)
    int sb16;                        // scale / bias rows are runs of 8 groups, 16-byte aligned
    int32_t *tile_done;              // [tiles] gate/up column blocks finished (zeroed by binning)
    const float *sgate;              // [T] shared-expert gate per token (gated layers), or null
    int nb_gateup;                   // down pass: the gate/up column blocks a tile waits for
    uint32_t *err;                   // the workspace's state words (0: bounded-wait error flag)
};

// per-row values of a tile beside the ring: the gate/up pass needs each row's 2^-a of x,
// the down pass each row's (token, slot) position, weight, and h block scales
struct DownRows {
    int pos[BM];
    float w[BM];                     // routing weight (or shared gate) x 2^-e_r
    int8_t e[BM];                    // e_r: the smallest block scale of h row r
    int8_t hx[BM * HEXP_STRIDE];     // the block scales of each row
    int mixed[4];                    // per wave: some row's block scales differ
};
union TileRows {
    float xs[BM];
    DownRows dn;
};

// The LDS position of 16-byte chunk c of activation row r is c ^ a_swizzle(r).  A 128-bit
// read is served 16 lanes per cycle from 64 four-byte banks, the lanes of one cycle being
// those of one wave half with equal parity of lane bits 2..4 (measured on gfx950 with the
// LDS bank-conflict counter); under this key the ten fragment reads of a K slice (lane
// n16 + 16 cg: row n16, chunk 2 cg + s) hit 64 distinct banks in every cycle.
__device__ __forceinline__ int a_swizzle(int r) { return ((r >> 1) & 1) | (r & 4); }

typedef __attribute__((address_space(3))) void lds_t;

__device__ __forceinline__ void dma16(const void *g, void *l) {
    __builtin_amdgcn_global_load_lds(g, (lds_t *)l, 16, 0, 0);
}
// the same at device scope (sc1): data another XCD wrote in this launch, not a stale
// line of this XCD's L2
__device__ __forceinline__ void dma16_dev(const void *g, void *l) {
    __builtin_amdgcn_global_load_lds(g, (lds_t *)l, 16, 0, 16);
}
__device__ __forceinline__ void dma4(const void *g, void *l) {
    __builtin_amdgcn_global_load_lds(g, (lds_t *)l, 4, 0, 0);
}
__device__ __forceinline__ void dma2(const void *g, void *l) {
    __builtin_amdgcn_global_load_lds(g, (lds_t *)l, 2, 0, 0);   // lands zero-extended in a dword
}
// this wave's direct-to-LDS loads: all but the most recent N have landed
template <int N>
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
// the workgroup's LDS reads issued so far are complete and every wave has arrived
__device__ __forceinline__ void block_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// order this wave's own LDS writes before its later LDS reads (no cross-wave effect)
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// 8 codes of one lane and K slice as MFMA operand: w = fma(q, s, b), q exact, in the
// order [0,4,1,5,2,6,3,7] (4-bit) or [0,2,1,3,4,6,5,7] (8-bit) of the 8 columns.
// 4-bit: the high nibble of each byte is taken in place (value 16 q, exact in fp16
// next to the 1024 magic) and paired with s/16, which is exact, so that only one
// shift is needed per 8 codes; the product (16 q)(s / 16) equals q s exactly, so the
// result is the same single rounding of q s + b.
struct DqConst {
    uint32_t lo, hi, magic;
};
template <int BITS>
__device__ __forceinline__ f16x8 dequant8(uint32_t w0, uint32_t w1, f16x2 sc, f16x2 sc16, f16x2 bi,
                                          const DqConst &k) {
    uint32_t m[4];
    if constexpr (BITS == 4) {
        const uint32_t w8 = w0 >> 8;
        m[0] = and_or(w0, k.lo, k.magic);
        m[1] = and_or(w0, k.hi, k.magic);
        m[2] = and_or(w8, k.lo, k.magic);
        m[3] = and_or(w8, k.hi, k.magic);
    } else {
        m[0] = and_or(w0, k.lo, k.magic);
        m[1] = and_or(w0 >> 8, k.lo, k.magic);
        m[2] = and_or(w1, k.lo, k.magic);
        m[3] = and_or(w1 >> 8, k.lo, k.magic);
    }
    const f16x2 k1024 = (f16x2){(_Float16)1024.0f, (_Float16)1024.0f};
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f16x2 q = as_h2(m[i]) - k1024;
        const f16x2 sv = (BITS == 4 && (i & 1)) ? sc16 : sc;
        out[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, sv, bi));
    }
    return __builtin_bit_cast(f16x8, out);
}

template <int BITS, int MODE>
__device__ __forceinline__ void gemm_body(const GemmArgs &a, const int bid, uint8_t *smem, TileRows &sx) {
    using C = Cfg<BITS>;
    const Layer &L = a.L;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the test word that forces exact h block scales (read now: its latency is hidden)
    const bool exact = MODE == 0 && __hip_atomic_load(a.err + CTL_HBLOCK_EXACT, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT) != 0;

    // ---- which tile and column block: the nb column blocks of a tile (which share its
    // activation rows) run on one XCD; consecutive tiles go round the XCDs in list order
    const int xcd = bid & 7, bslot = bid >> 3;
    const int ti = (bslot / a.nb) * 8 + xcd, nbi = bslot % a.nb;
    const int nrt = a.ntiles[0], nsh = a.ntiles[1] - nrt;
    int tix;
    if (ti >= nrt + nsh) return;
    tix = ti < nsh ? nrt + ti : ti - nsh;              // shared (full) tiles first
    const Tile tile = a.tiles[tix];
    const int E = L.E, K = L.K, H = L.H, I = L.I;
    const bool shared = tile.expert == E;
    const int64_t e = shared ? 0 : tile.expert;
    const int Kdim = (MODE == 0) ? H : I;
    const int nk = Kdim / BK;
    const int64_t TK = a.T * K;
    const int nrows = tile.nrows;
    const int msub = (nrows + 15) >> 4;

    // ---- weight row of workgroup row slot rs (0..255)
    auto wrow = [&](int rs, QMat &m) __attribute__((always_inline)) -> int {
        if (MODE == 0) {
            const int j = (rs >> 4) & 3;
            m = (j < 2) ? (shared ? L.s_gate : L.gate) : (shared ? L.s_up : L.up);
            // h column; past I (the last block when I % 128 == 64) a valid row is re-read
            // and its results discarded
            const int col = nbi * 128 + (rs >> 6) * 32 + (j & 1) * 16 + (rs & 15);
            return col < I ? col : I - 1;
        }
        m = shared ? L.s_down : L.down;
        const int col = nbi * BN + rs;
        return col < H ? col : H - 1;
    };
    const int row_bytes = Kdim * BITS / 8;
    const int ngrp = Kdim / 64;

    // ---- per-lane sources of the direct-to-LDS loads.  Activation piece i of this wave
    // is rows 8 p .. 8 p + 7 of the tile (p = A_DMA wave + i); the lane fetches, for row
    // 8 p + lane / 8, the chunk that the swizzle stores at position lane % 8.  Sources are
    // kept as 16-byte chunk indices from a uniform base (x16, or the tile's first h row).
    auto apiece = [&](int i, int &r, int &ach) __attribute__((always_inline)) {
        const int rpos = 8 * (C::A_DMA * wave + i) + (lane >> 3);
        ach = (lane & 7) ^ a_swizzle(rpos);
        r = rpos < nrows ? rpos : nrows - 1;             // rows past the tile repeat a valid one
    };
    const uint16_t *abase = MODE == 0 ? a.x16 : a.h + (int64_t)tile.row0 * I;
    uint32_t achunk[C::A_DMA];
#pragma unroll
    for (int i = 0; i < C::A_DMA; ++i) {
        int r, ach;
        apiece(i, r, ach);
        if (MODE == 0) {
            const int64_t t = shared ? (tile.row0 - TK + r) : (a.perm[tile.row0 + r] / K);
            achunk[i] = (uint32_t)(t * (H / 8) + ach);
        } else {
            achunk[i] = (uint32_t)(r * (I / 8) + ach);
        }
    }
    // code sources: the matrix of DMA d is the same for the whole wave (MODE 0: the first
    // half of the DMAs fetch gate rows, the second half up rows), so each is a uniform
    // matrix base plus a 32-bit lane offset
    const uint8_t *bbase[C::B_DMA];
    uint32_t boff[C::B_DMA];
#pragma unroll
    for (int d = 0; d < C::B_DMA; ++d) {
        QMat m;
        int rs, sel;
        if constexpr (BITS == 4) {
            rs = 64 * wave + 32 * d + (lane >> 1);
            sel = (lane & 1) ^ ((rs >> 2) & 1);
        } else {
            rs = 64 * wave + 16 * d + (lane >> 2);
            sel = (lane & 3) ^ ((rs >> 1) & 3);
        }
        const int r = wrow(rs, m);
        const QMat mu = MODE == 0 ? (2 * d < C::B_DMA ? (shared ? L.s_gate : L.gate) : (shared ? L.s_up : L.up))
                                  : (shared ? L.s_down : L.down);
        bbase[d] = mu.codes + e * mu.stride * row_bytes;
        boff[d] = (uint32_t)(r * row_bytes + 16 * sel);
    }
    // this thread's weight row (slot 64 wave + lane): its scale / bias windows, and its range
    const uint16_t *ssrc, *bisrc;
    {
        QMat m;
        const int r = wrow(64 * wave + lane, m);
        ssrc = m.scales + (e * m.stride + r) * ngrp;
        bisrc = m.biases + (e * m.stride + r) * ngrp;
    }

    auto issue = [&](int k) __attribute__((always_inline)) {
        uint8_t *st = smem + (k % C::NSTAGE) * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::A_DMA; ++i) {
            const uint16_t *src = abase + (uint64_t)achunk[i] * 8 + k * BK;
            if (MODE == 1) dma16_dev(src, st + (8 * C::A_DMA * wave + 8 * i) * 128);
            else dma16(src, st + (8 * C::A_DMA * wave + 8 * i) * 128);
        }
        uint8_t *bst = st + C::A_BYTES;
#pragma unroll
        for (int d = 0; d < C::B_DMA; ++d) {
            if constexpr (BITS == 4) dma16(bbase[d] + boff[d] + k * 32, bst + (64 * wave + 32 * d) * 32);
            else dma16(bbase[d] + boff[d] + k * 64, bst + (64 * wave + 16 * d) * 64);
        }
        // scales and biases: W = 2^wlog groups of each row every W K steps, into a ring of
        // two windows (one 2-byte read per lane costs the address unit as much as a 16-byte
        // one, so the wider and rarer the better)
        if ((k & ((1 << a.wlog) - 1)) == 0) {
            uint8_t *sw = smem + C::NSTAGE * C::STAGE + ((k >> a.wlog) & 1) * 2 * C::S_BYTES;
            if (C::WMAX == 8 && a.wlog == 3) {                    // 16 bytes per row
                dma16(ssrc + k, sw + 64 * wave * 16);
                dma16(bisrc + k, sw + C::S_BYTES + 64 * wave * 16);
            } else if (a.wlog == 1) {                             // 4 bytes per row
                dma4(ssrc + k, sw + 64 * wave * 4);
                dma4(bisrc + k, sw + C::S_BYTES + 64 * wave * 4);
            } else {                                              // 2 bytes in a 4-byte slot
                dma2(ssrc + k, sw + 64 * wave * 4);
                dma2(bisrc + k, sw + C::S_BYTES + 64 * wave * 4);
            }
        }
    };

    // ---- the down pass waits for its tile's h rows and reads their block scales
    bool slow = false;                   // some row's h blocks differ in scale: rescale in LDS
    const bool routed_down = MODE == 1 && !shared;
    const int my_row = tid < nrows ? tid : nrows - 1;
    // the (token, slot) position and routing weight (or shared gate) of tile row `tid`,
    // fetched first, so that they have landed when the rows' factors are set below
    int my_pos = 0;
    float my_w = 0.0f;
    if (MODE == 1 && tid < BM) {
        if (routed_down) {
            my_pos = a.perm[tile.row0 + my_row];
            my_w = a.w[my_pos];
        } else {
            my_w = a.sgate ? a.sgate[tile.row0 + my_row - TK] : 1.0f;
        }
    }
    if (MODE == 1) {
        // this tile's h rows are complete once all gate/up column blocks of the tile have
        // counted themselves in; they run earlier in the grid (lower workgroup index,
        // dispatched first), so the wait ends; it is bounded regardless
        if (tid == 0) {
            // the bound: 2^24 polls, or the workspace's test bound (state word 32) when set
            const uint32_t tb = __hip_atomic_load(a.err + 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t lim = tb ? tb : (1u << 24);
            for (uint32_t it = 0;
                 __hip_atomic_load(a.tile_done + tix, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < a.nb_gateup;
                 ++it) {
                if (it > lim) {
                    __hip_atomic_fetch_or(a.err, MOE_WS_ERR_GEMM_WAIT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(8);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int p = 0; p < C::NSTAGE - 1; ++p)
        if (p < nk) issue(p);
    u32x4 hw = {0u, 0u, 0u, 0u};         // down pass: the block scales of h row `tid`
    if (MODE == 1 && tid < BM) {
        // (device scope: written by other workgroups of this launch; block-major, so the
        // rows of a tile are consecutive bytes)
        const int8_t *hp = a.hexp + tile.row0 + my_row;
        const int64_t rtot = TK + a.T;
#pragma unroll
        for (int bk = 0; bk < HEXP_STRIDE; ++bk)
            if (bk < a.nb_gateup) {
                const uint32_t v = (uint8_t)__hip_atomic_load(hp + bk * rtot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                hw[bk >> 2] |= v << (8 * (bk & 3));
            }
    }
    int my_xe = 0;                       // gate/up pass: the scale exponent of x in row `tid`
    if (MODE == 0 && tid < BM) {
        const int64_t t = shared ? (tile.row0 - TK + my_row) : (a.perm[tile.row0 + my_row] / K);
        my_xe = a.xexp[t];
    }
    // ---- the bound max_g |s_g| (2^bits - 1) + |b_g| on the |w| of this thread's weight
    // row; the largest over the wave's 64 rows sets the wave's prescale 2^p (largest weight
    // in [2^14, 2^15)).  Per wave, no barrier: the loads' latency passes under the first
    // stage's, and the factor is taken out by the wave itself (its own output columns).
    float wsc, winv;
    bool convert;                        // scales / biases need converting (bf16 in, or p != 0)
    {
        constexpr float QMAX = (float)((1 << BITS) - 1);
        const int bf = L.sb_bf16;
        float M = 0.0f, smin = __builtin_inff();
        auto bound = [&](uint32_t sbits, uint32_t bbits) __attribute__((always_inline)) {
            const float sv = fabsf(sb_to_f32(sbits & 0xffffu, bf));
            M = fmaxf(M, fmaf(sv, QMAX, fabsf(sb_to_f32(bbits & 0xffffu, bf))));
            smin = fminf(smin, sv > 0.0f ? sv : __builtin_inff());
        };
        if (a.sb16) {                                             // rows of 8-group runs, 16-byte aligned
#pragma unroll 4
            for (int g = 0; g < ngrp; g += 8) {
                const u32x4 sv = *(const u32x4 *)(ssrc + g), bv = *(const u32x4 *)(bisrc + g);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    bound(sv[q], bv[q]);
                    bound(sv[q] >> 16, bv[q] >> 16);
                }
            }
        } else if (a.wlog == 1) {                                 // 2-group runs, 4-byte aligned
#pragma unroll 4
            for (int g = 0; g < ngrp; g += 2) {
                const uint32_t sv = *(const uint32_t *)(ssrc + g), bv = *(const uint32_t *)(bisrc + g);
                bound(sv, bv);
                bound(sv >> 16, bv >> 16);
            }
        } else {
#pragma unroll 4
            for (int g = 0; g < ngrp; ++g) bound(ssrc[g], bisrc[g]);
        }
        // (non-negative floats order as their bit patterns; the minimum as the maximum of
        // the complements)
        M = __uint_as_float(wave_max_u32(__float_as_uint(M)));
        smin = __uint_as_float(~wave_max_u32(~__float_as_uint(smin)));
        // no prescale where the weights already sit in fp16's range: largest bound in
        // [2^-2, 2^15) and (4-bit) every nonzero s / 16 a normal number
        const bool in_range = M >= 0.25f && M < 32768.0f && (BITS == 8 || smin >= 0.0009765625f);
        const int p = in_range || !(M > 0.0f) ? 0 : clamp_exp(14 - ilog2f(M));
        wsc = exp2i(p);
        winv = exp2i(-p);
        convert = L.sb_bf16 || p != 0;
    }
    // ---- per-row factors, parked in LDS until the epilogue (published by the K loop's
    // first barrier): gate/up, 2^-a (x's scale); down, the routing weight times 2^-e_r,
    // with the row's block scales for the rescale
    if (MODE == 0 && tid < BM) sx.xs[tid] = exp2i(-my_xe);
    if (MODE == 1) {
        bool mixed = false;
        if (tid < BM) {
            int lo = 127, hi = -128;
#pragma unroll
            for (int bk = 0; bk < HEXP_STRIDE; ++bk)
                if (bk < a.nb_gateup) {
                    const int v = (int)(int8_t)(hw[bk >> 2] >> (8 * (bk & 3)));
                    lo = v < lo ? v : lo;
                    hi = v > hi ? v : hi;
                }
            mixed = lo != hi;
            sx.dn.e[tid] = (int8_t)lo;
            *(u32x4 *)(sx.dn.hx + tid * HEXP_STRIDE) = hw;
            sx.dn.pos[tid] = my_pos;
            sx.dn.w[tid] = my_w * exp2i(-lo);
        }
        // (each wave's flag is read after the K loop's first barrier; the ballot is taken
        // by the whole wave)
        const bool wm = __builtin_amdgcn_ballot_w64(mixed) != 0;
        if (lane == 0) sx.dn.mixed[wave] = wm;
    }

    f32x4 acc[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[i][n] = (f32x4){0.f, 0.f, 0.f, 0.f};

    const int n16 = lane & 15, cg = lane >> 4;
    constexpr int CW = BITS == 4 ? 2 : 4;           // code dwords per lane and subtile per K step

    // wait until stage `k` has landed: `newer` stages were issued after it
    auto wait_stage = [&](int newer) __attribute__((always_inline)) {
        if (newer >= 2) wait_dma<2 * C::DMA>();
        else if (newer == 1) wait_dma<C::DMA>();
        else wait_dma<0>();
    };
    // the scale / bias window of K step k (its first step), as this thread loaded it for
    // its own row: converted in place to fp16 s 2^p, b 2^p (exact) with the wave's p
    auto convert_window = [&](int k) __attribute__((always_inline)) {
        uint8_t *sw = smem + C::NSTAGE * C::STAGE + ((k >> a.wlog) & 1) * 2 * C::S_BYTES;
        const int rs = 64 * wave + lane, bf = L.sb_bf16;
        auto cv = [&](uint32_t bits) __attribute__((always_inline)) -> uint32_t {
            return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(sb_to_f32(bits & 0xffffu, bf) * wsc));
        };
        auto cv2 = [&](uint32_t v) __attribute__((always_inline)) -> uint32_t { return cv(v) | (cv(v >> 16) << 16); };
        if (C::WMAX == 8 && a.wlog == 3) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                u32x4 *p = (u32x4 *)(sw + h * C::S_BYTES + rs * 16);
                u32x4 v = *p;
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = cv2(v[q]);
                *p = v;
            }
        } else if (a.wlog == 1) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t *p = (uint32_t *)(sw + h * C::S_BYTES + rs * 4);
                *p = cv2(*p);
            }
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t *p = (uint32_t *)(sw + h * C::S_BYTES + rs * 4);
                *p = cv(*p);
            }
        }
    };
    // down pass, tiles whose rows mix h block scales: the chunks this thread loaded for K
    // step k, brought from their block's scale 2^e to the row's 2^e_r (e_r <= e)
    auto rescale_a = [&](int k) __attribute__((always_inline)) {
        uint8_t *st = smem + (k % C::NSTAGE) * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::A_DMA; ++i) {
            int r, ach;
            apiece(i, r, ach);
            const int blk = (k * BK + 8 * ach) >> 7;
            const int d = (int)sx.dn.e[r] - (int)sx.dn.hx[r * HEXP_STRIDE + blk];
            if (d != 0) {
                const float f = d < -100 ? 0.0f : exp2i(d);
                u32x4 *p = (u32x4 *)(st + (8 * C::A_DMA * wave + 8 * i) * 128 + lane * 16);
                u32x4 v = *p;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f16x2 h2 = as_h2(v[q]);
                    v[q] = pack_f16x2(f32_to_f16_ftz((float)h2[0] * f), f32_to_f16_ftz((float)h2[1] * f));
                }
                *p = v;
            }
        }
    };
    // operands of K step k from the LDS ring: per weight subtile j, the code dwords of
    // K slice s of this lane, and the scale and bias
    auto load_codes = [&](int k, int s, uint32_t (&cw)[4][CW / 2]) __attribute__((always_inline)) {
        const uint8_t *bst = smem + (k % C::NSTAGE) * C::STAGE + C::A_BYTES;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rs = 64 * wave + 16 * j + n16;
            if constexpr (BITS == 4) {
                const int hsel = (cg >> 1) ^ ((rs >> 2) & 1);
                cw[j][0] = *(const uint32_t *)(bst + rs * 32 + hsel * 16 + (cg & 1) * 8 + 4 * s);
            } else {
                const int q = cg ^ ((rs >> 1) & 3);
                const uint32_t *p = (const uint32_t *)(bst + rs * 64 + q * 16 + 8 * s);
                cw[j][0] = p[0];
                cw[j][1] = p[1];
            }
        }
    };
    auto load_sb = [&](int k, f16x2 (&sc)[4], f16x2 (&sc16)[4], f16x2 (&bi)[4]) __attribute__((always_inline)) {
        // row rs, group k % W of the window: 16 (W = 8) or 4 bytes per row, 2 bytes per
        // group (W = 1: the low half of the dword a 2-byte load fills); fp16, prescaled
        const int pitch = a.wlog == 3 ? 16 : 4;
        const uint8_t *sw = smem + C::NSTAGE * C::STAGE + ((k >> a.wlog) & 1) * 2 * C::S_BYTES +
                            2 * (k & ((1 << a.wlog) - 1));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rs = 64 * wave + 16 * j + n16;
            const _Float16 sv = __builtin_bit_cast(_Float16, *(const uint16_t *)(sw + rs * pitch));
            const _Float16 bv = __builtin_bit_cast(_Float16, *(const uint16_t *)(sw + C::S_BYTES + rs * pitch));
            sc[j] = (f16x2){sv, sv};
            const _Float16 sv16 = sv * (_Float16)0.0625f;        // exact: prescaled scales are normal
            sc16[j] = (f16x2){sv16, sv16};
            bi[j] = (f16x2){bv, bv};
        }
    };
    uint32_t cw[4][CW / 2];
    f16x2 sc[4], sc16[4], bi[4];
    DqConst dk;
    dk.lo = BITS == 4 ? 0x000F000Fu : 0x00FF00FFu;
    dk.hi = 0x00F000F0u;
    dk.magic = QS_MAGIC;
    auto deq = [&](const uint32_t (&cw)[4][CW / 2], f16x8 (&B)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (BITS == 4) B[j] = dequant8<4>(cw[j][0], 0u, sc[j], sc16[j], bi[j], dk);
            else B[j] = dequant8<8>(cw[j][0], cw[j][1], sc[j], sc16[j], bi[j], dk);
        }
    };

    // The K loop: per 64-wide step, one barrier (stage k visible, stage k-1 consumed),
    // the refill of stage k-1's buffer with stage k+NSTAGE-1, then two MFMA blocks
    // (32-wide slices), each on a weight slice dequantized just before it.  All ten row
    // subtiles run, so every fragment read of a block is issued ahead of its MFMAs.
    // Before the barrier each thread finishes what it loaded itself: a new scale window
    // is converted, and (down pass, mixed tiles) its activation chunks are rescaled.
    auto kloop = [&]() __attribute__((always_inline)) {
        for (int k = 0; k < nk; ++k) {
            // stage k has landed once at most the later stages' loads are outstanding
            const int issued = k + C::NSTAGE - 1 < nk ? C::NSTAGE - 2 : nk - 1 - k;
            wait_stage(issued < 0 ? 0 : issued);
            if (convert && (k & ((1 << a.wlog) - 1)) == 0) convert_window(k);
            if (MODE == 1 && slow) rescale_a(k);
            block_sync();
            if (MODE == 1 && k == 0) {
                // the down pass learns here whether the tile mixes h block scales; if so,
                // step 0's chunks are rescaled now, behind one more barrier
                slow = (sx.dn.mixed[0] | sx.dn.mixed[1] | sx.dn.mixed[2] | sx.dn.mixed[3]) != 0;
                if (slow) {
                    rescale_a(0);
                    block_sync();
                }
            }
            if (k + C::NSTAGE - 1 < nk) issue(k + C::NSTAGE - 1);
            const uint8_t *st = smem + (k % C::NSTAGE) * C::STAGE;
            load_sb(k, sc, sc16, bi);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int pos = (2 * cg + s) ^ a_swizzle(n16);
                f16x8 A[MT];
#pragma unroll
                for (int i = 0; i < MT; ++i) A[i] = *(const f16x8 *)(st + (i * 16 + n16) * 128 + pos * 16);
                load_codes(k, s, cw);
                f16x8 B[4];
                deq(cw, B);
#pragma unroll
                for (int i = 0; i < MT; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[i], B[j], acc[i][j], 0, 0, 0);
            }
        }
    };
    kloop();
    block_sync();                     // the ring is free: epilogues stage through it

    // ---- epilogues.  acc[i][j][r]: tile row i*16 + 4*cg + r, weight row slot 64*wave + 16*j + n16
    if (MODE == 0) {
        constexpr int HP = 40;                                   // fp16 per staged row
        uint16_t *hs = (uint16_t *)(smem + wave * (BM * HP * 2));
        uint32_t *s_hm = (uint32_t *)(smem + 4 * (BM * HP * 2)); // [4][BM] row maxima per wave
        int8_t *s_eh = (int8_t *)(s_hm + 4 * BM);                // [BM] the block scale of each row
        float *s_rf = (float *)(s_eh + (BM + 15) / 16 * 16);     // [BM] 2^e of each row
        const bool cols_live = nbi * 128 + wave * 32 < I;      // this wave's 32 h columns exist
        // h = silu(g) u in fp32 (scales of x and of the weight rows taken out), in place of
        // the gate accumulators; then the largest |h| of each row over this wave's columns
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            if (i < msub) {
                const f32x4 rf = *(const f32x4 *)(sx.xs + i * 16 + 4 * cg) * winv;
                uint32_t m[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const float g = acc[i][j][r] * rf[r];
                        const float u = acc[i][j + 2][r] * rf[r];
                        acc[i][j][r] = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
                    }
                    uint32_t v = cols_live ? __float_as_uint(__builtin_fmaxf(__builtin_fabsf(acc[i][0][r]),
                                                                            __builtin_fabsf(acc[i][1][r])))
                                           : 0u;
                    v = max(v, dpp_u32<0xB1>(v));
                    v = max(v, dpp_u32<0x4E>(v));
                    v = max(v, dpp_u32<0x141>(v));
                    v = max(v, dpp_u32<0x140>(v));
                    m[r] = v;
                }
                if (n16 == 0) *(u32x4 *)(s_hm + wave * BM + i * 16 + 4 * cg) = (u32x4){m[0], m[1], m[2], m[3]};
            }
        }
        __syncthreads();
        // the block's scale per row, once per row (thread `row`, from the four waves'
        // maxima), then h 2^e staged as fp16
        if (tid < BM) {
            uint32_t mb = s_hm[tid];
#pragma unroll
            for (int w = 1; w < 4; ++w) mb = max(mb, s_hm[w * BM + tid]);
            const float m = __uint_as_float(mb);
            const int eh = exact ? (m > 0.0f ? clamp_exp(14 - ilog2f(m)) : 0) : block_exp(m);
            s_eh[tid] = (int8_t)eh;
            s_rf[tid] = exp2i(eh);
        }
        __syncthreads();
        int pcol[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = j * 16 + n16;
            pcol[j] = (col & ~7) | perm_pos<BITS>(col & 7);
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            if (i < msub) {
                const f32x4 f = *(const f32x4 *)(s_rf + i * 16 + 4 * cg);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = i * 16 + 4 * cg + r;
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        hs[row * HP + pcol[j]] = __builtin_bit_cast(uint16_t, f32_to_f16_ftz(acc[i][j][r] * f[r]));
                }
            }
        }
        wave_lds_sync();
        // the block scales of the tile's rows: consecutive bytes of block nbi, stored by
        // wave 0 at device scope (as h) in runs of 64
        if (wave == 0) {
            int8_t *he = a.hexp + (int64_t)nbi * (TK + a.T) + tile.row0;
#pragma unroll
            for (int q = 0; q < (BM + 63) / 64; ++q) {
                const int row = 64 * q + lane;
                if (row < nrows) __hip_atomic_store(he + row, s_eh[row], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        const int chunk = lane & 3;
        uint16_t *hout = a.h + (int64_t)tile.row0 * I + nbi * 128 + wave * 32 + chunk * 8;
        // h goes out at device scope (sc1, written through), and once every wave's stores
        // have completed the workgroup counts itself in for the tile's down pass
#pragma unroll
        for (int q = 0; q < BM / 16; ++q) {
            const int row = (lane >> 2) + 16 * q;
            if (row < nrows && cols_live) {
                const u32x4 v = *(const u32x4 *)(hs + row * HP + chunk * 8);
                // (padded: a vector-ALU write to the data registers of a store wider than 8
                // bytes within two wait states replaces data the store has not yet read)
                asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 4" ::"v"(hout + (int64_t)row * I), "v"(v)
                             : "memory");
            }
        }
        // every store the down pass reads (h rows, their block scales) is a device-scope
        // (sc1) store, coherent across the XCDs once complete: the count follows once all
        // of them have completed, with no L2 write-back (which, once per workgroup, cost a
        // tenth of the launch)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) __hip_atomic_fetch_add(a.tile_done + tix, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    // MODE 1: 32 rows at a time through a per-wave fp32 staging area; lane l then
    // owns row 32*hp + (l % 32) and 32 of the wave's 64 columns, and the lane pair of a
    // row sets the scale of the row's 64 columns from their largest value
    const int colbase = nbi * BN + wave * 64;
    if (colbase >= H) return;                                    // columns past H (H % 256 != 0)
    constexpr int FP = 68;                                       // floats per staged row
    float *fs = (float *)(smem + wave * (32 * FP * 4));
    const int er = lane & 31, ecol = colbase + 32 * (lane >> 5);
    int8_t *sexp_blk = a.sexp + (int64_t)(colbase >> 6) * sexp_rows(a.T, K);
#pragma unroll
    for (int hp = 0; hp < MT / 2; ++hp) {
        if (32 * hp >= nrows) break;
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    fs[(ii * 16 + 4 * cg + r) * FP + j * 16 + n16] = acc[2 * hp + ii][j][r];
        wave_lds_sync();
        const int row = 32 * hp + er;
        const bool live = row < nrows;
        // routed rows: the (token, slot) row with its routing weight; shared rows:
        // row T*K + t with the shared gate (or 1); both with h's row scale and the
        // weights' prescale taken out
        const float wv = sx.dn.w[live ? row : 0] * winv;
        const float *src = fs + er * FP + 32 * (lane >> 5);
        f32x4 v[8];
        float mx = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            v[c] = *(const f32x4 *)(src + 4 * c);
            mx = __builtin_fmaxf(mx, __builtin_fmaxf(__builtin_fabsf(v[c][0]), __builtin_fabsf(v[c][1])));
            mx = __builtin_fmaxf(mx, __builtin_fmaxf(__builtin_fabsf(v[c][2]), __builtin_fabsf(v[c][3])));
        }
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * __builtin_fabsf(wv);
        const int es = range_exp(mx);
        const float f = wv * exp2i(es);
        if (live) {
            const int64_t p = routed_down ? (int64_t)sx.dn.pos[row] : (int64_t)tile.row0 + row;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const f32x4 v0 = v[2 * c] * f, v1 = v[2 * c + 1] * f;
                u32x4 o;
                o[0] = pack_f16x2(f32_to_f16_ftz(v0[0]), f32_to_f16_ftz(v0[1]));
                o[1] = pack_f16x2(f32_to_f16_ftz(v0[2]), f32_to_f16_ftz(v0[3]));
                o[2] = pack_f16x2(f32_to_f16_ftz(v1[0]), f32_to_f16_ftz(v1[1]));
                o[3] = pack_f16x2(f32_to_f16_ftz(v1[2]), f32_to_f16_ftz(v1[3]));
                *(u32x4 *)(a.slot + p * H + ecol + 8 * c) = o;
            }
            if (lane < 32) sexp_blk[p] = (int8_t)es;
        }
        // a nonzero scale anywhere sends the combine through its scaled path
        if (__builtin_amdgcn_ballot_w64(live && es != 0) != 0 && lane == 0) a.ntiles[2] = 1;
        wave_lds_sync();
    }
}

// gate/up (workgroups [0, g0)) and down (the rest) in one launch: a down workgroup waits
// only for the gate/up column blocks of its own tile, so down tiles fill the slots the
// last, partial round of gate/up tiles leaves free
template <int BITS>
__global__ __launch_bounds__(NT, 2) void k_gemm(GemmArgs a0, GemmArgs a1, int g0) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[Cfg<BITS>::LDS];
    __shared__ TileRows sx;
    if ((int)blockIdx.x < g0) gemm_body<BITS, 0>(a0, (int)blockIdx.x, smem, sx);
    else gemm_body<BITS, 1>(a1, (int)blockIdx.x - g0, smem, sx);
}

// The combine: y[t] = sum of the token's k slot rows in ascending expert id, then its
// shared-expert row, in fp32, each slot value taken out of its block scale (read only when
// the down pass flagged a nonzero one); one thread per 8 columns of a token (16-byte loads).
__global__ __launch_bounds__(256) void k_combine(const uint16_t *__restrict__ slot, const int8_t *__restrict__ sexp,
                                                 const int32_t *__restrict__ scaled, void *y, int y_dtype,
                                                 int64_t T, int K, int H, int shared) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;     // (token, 8-column chunk)
    const int cpr = H / 8;
    if (i >= T * cpr) return;
    const int64_t t = i / cpr;
    const int col = (int)(i % cpr) * 8;
    u32x4 v[17];
    float f[17];
#pragma unroll
    for (int j = 0; j < 17; ++j)
        if (j < K || (j == K && shared)) {
            const int64_t row = j < K ? t * K + j : T * K + t;
            v[j] = *(const u32x4 *)(slot + row * H + col);
            f[j] = 1.0f;
        }
    if (*scaled) {                       // some slot block carries a scale (extreme data only)
        const int8_t *se = sexp + (int64_t)(col >> 6) * sexp_rows(T, K);
#pragma unroll
        for (int j = 0; j < 17; ++j)
            if (j < K || (j == K && shared)) f[j] = exp2i(-(int)se[j < K ? t * K + j : T * K + t]);
    }
    float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 17; ++j)
        if (j < K || (j == K && shared))
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f16x2 h2 = as_h2(v[j][q]);
                sum[2 * q] = fmaf((float)h2[0], f[j], sum[2 * q]);
                sum[2 * q + 1] = fmaf((float)h2[1], f[j], sum[2 * q + 1]);
            }
    if (y_dtype == MOE_F32) {
        float *yp = (float *)y + t * H + col;
        *(f32x4 *)yp = (f32x4){sum[0], sum[1], sum[2], sum[3]};
        *(f32x4 *)(yp + 4) = (f32x4){sum[4], sum[5], sum[6], sum[7]};
    } else {
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[q] = (uint32_t)f32_to_bf16(sum[2 * q]) | ((uint32_t)f32_to_bf16(sum[2 * q + 1]) << 16);
        *(u32x4 *)((uint16_t *)y + t * H + col) = o;
    }
}

// workgroups for `tiles` tiles of nb column blocks: a multiple of 8 * nb (see k_gemm)
inline unsigned grid_for(int64_t tiles, int nb) {
    const int64_t per = 8 * (int64_t)nb;
    return (unsigned)(((tiles + 7) / 8) * per);
}

// log2 of the widest scale / bias window (at most wmax groups) for matrices with `cols`
// columns: every row's run of W groups must be a multiple of W and 2W-byte aligned
int window_log(const QMat *const *ms, int n, int cols, int wmax) {
    const int ngrp = cols / 64;
    for (int w = wmax; w > 1; w >>= 1) {
        bool ok = ngrp % w == 0;
        for (int i = 0; i < n; ++i)
            ok = ok && (uintptr_t)ms[i]->scales % (2 * w) == 0 && (uintptr_t)ms[i]->biases % (2 * w) == 0;
        if (ok) return w == 8 ? 3 : w == 4 ? 2 : 1;
    }
    return 0;
}

template <int BITS>
hipError_t gemms(GemmArgs a, hipStream_t s) {
    using C = Cfg<BITS>;
    const Layer &L = a.L;
    const int64_t maxr = prefill_max_routed_tiles(a.T, L.K, L.E);
    const int64_t maxs = L.has_shared ? (a.T + GEMM_BM - 1) / GEMM_BM : 0;
    // [gate; up] + SwiGLU over routed and shared tiles
    GemmArgs a0 = a;
    a0.nb = (L.I + 127) / 128;
    {
        const QMat *ms[4] = {&L.gate, &L.up, &L.s_gate, &L.s_up};
        a0.wlog = window_log(ms, L.has_shared ? 4 : 2, L.H, C::WMAX);
        if (a0.wlog == 2) a0.wlog = 1;                     // windows of 8, 2 or 1 groups
        a0.sb16 = window_log(ms, L.has_shared ? 4 : 2, L.H, 8) == 3;
    }
    // down: routed tiles -> weighted slot rows, shared tiles -> their own slot rows
    GemmArgs a1 = a;
    a1.nb = (L.H + BN - 1) / BN;
    a1.nb_gateup = a0.nb;
    {
        const QMat *ms[2] = {&L.down, &L.s_down};
        a1.wlog = window_log(ms, L.has_shared ? 2 : 1, L.I, C::WMAX);
        if (a1.wlog == 2) a1.wlog = 1;
        a1.sb16 = window_log(ms, L.has_shared ? 2 : 1, L.I, 8) == 3;
    }
    const unsigned g0 = grid_for(maxr + maxs, a0.nb), g1 = grid_for(maxr + maxs, a1.nb);
    hipLaunchKernelGGL((k_gemm<BITS>), dim3(g0 + g1), dim3(NT), 0, s, a0, a1, (int)g0);
    const int64_t n = a.T * (L.H / 8);
    hipLaunchKernelGGL(k_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.slot, a.sexp,
                       a.ntiles + 2, a.y, a.y_dtype, a.T, L.K, L.H, L.has_shared);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_gemms(const Layer &L, int64_t T, const PrefillBufs &b, void *y,
                                int y_dtype, hipStream_t s) {
    GemmArgs a;
    a.L = L;
    a.T = T;
    a.x16 = b.x16;
    a.xexp = b.xexp;
    a.h = b.h;
    a.hexp = b.hexp;
    a.sexp = b.sexp;
    a.perm = b.perm;
    a.tiles = b.tiles;
    a.ntiles = b.ntiles;
    a.w = b.w;
    a.slot = b.slot;
    a.tile_done = b.tile_done;
    a.sgate = (L.shared_gate_w && L.has_shared) ? b.sgate : nullptr;
    a.err = b.ctl;
    a.nb_gateup = 0;
    a.y = y;
    a.y_dtype = y_dtype;
    a.nb = 1;
    return L.bits == 4 ? gemms<4>(a, s) : gemms<8>(a, s);
}

}  // namespace qs
