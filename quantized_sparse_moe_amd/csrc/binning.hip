// binning.hip -- expert binning on the GPU (T >= 2).
//
// [LILY] "Keep expert routing on the GPU": the grouped GEMM needs the activation rows
// of each expert stored together.  A histogram counts the assignments per expert (done
// per ROUTER_TOKENS-token block by the router), a prefix scan turns counts into start offsets, a
// scatter places every (token, slot) assignment into its expert's group, and a block
// map lists the fixed-size row blocks the grouped GEMM processes.  Everything stays on
// the device: no count is read back by the host.  [LILY] "Match tile size to expert
// load": bins are uneven, so work is enumerated per (expert, row block) from the bins'
// real sizes; the GEMM grid is sized for the worst case and surplus workgroups exit.
//
// The scatter is deterministic: within a bin, assignments appear in increasing
// (token, slot) order, computed with wave ballots (no atomics).
#include "common.h"
#include "internal.h"

namespace qs {

namespace {

// Per expert: exclusive scan of the block counts over the blocks.  64 threads per
// expert, each owning a contiguous run of blocks.
__global__ __launch_bounds__(256) void k_colscan(const int32_t *__restrict__ blkcnt,
                                                 int32_t *__restrict__ blkoff,
                                                 int32_t *__restrict__ counts, int nblk, int E) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.x * 4 + wave;
    if (e >= E) return;
    const int per = (nblk + 63) / 64;
    const int b0 = lane * per, b1 = min(nblk, b0 + per);
    int local = 0;
    for (int b = b0; b < b1; ++b) local += blkcnt[(int64_t)b * E + e];
    // exclusive scan of `local` across the wave
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    int run = incl - local;
    for (int b = b0; b < b1; ++b) {
        const int c = blkcnt[(int64_t)b * E + e];
        blkoff[(int64_t)b * E + e] = run;
        run += c;
    }
    if (lane == 63) counts[e] = incl;
}

// Expert offsets (exclusive scan over experts) and the block map.  Tiles are listed
// full ones first (in expert order), then every expert's partial last tile, then the
// shared expert's tiles, so that the grouped GEMM meets the heavy tiles first.
__global__ __launch_bounds__(256) void k_tiles(const int32_t *__restrict__ counts,
                                               int32_t *__restrict__ expert_off,
                                               Tile *__restrict__ tiles, int32_t *__restrict__ ntiles,
                                               int32_t *__restrict__ tile_done, int max_tiles,
                                               int E, int64_t T, int K, int shared) {
    for (int i = threadIdx.x; i < max_tiles; i += 256) tile_done[i] = 0;   // the GEMMs' tile counters
    __shared__ int wsum[3][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = tid < E ? counts[tid] : 0;
    const int nf = n / GEMM_BM, np = (n % GEMM_BM) ? 1 : 0;
    int in = n, itf = nf, itp = np;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o1 = __shfl_up(in, off, 64), o2 = __shfl_up(itf, off, 64), o3 = __shfl_up(itp, off, 64);
        if (lane >= off) { in += o1; itf += o2; itp += o3; }
    }
    if (lane == 63) { wsum[0][wave] = in; wsum[1][wave] = itf; wsum[2][wave] = itp; }
    __syncthreads();
    int bn = 0, bf = 0, bp = 0;
    for (int w = 0; w < wave; ++w) { bn += wsum[0][w]; bf += wsum[1][w]; bp += wsum[2][w]; }
    const int nfull = wsum[1][0] + wsum[1][1] + wsum[1][2] + wsum[1][3];
    const int npart = wsum[2][0] + wsum[2][1] + wsum[2][2] + wsum[2][3];
    const int off = bn + in - n, foff = bf + itf - nf, poff = nfull + bp + itp - np;
    if (tid < E) expert_off[tid] = off;
    if (tid == E - 1) expert_off[E] = off + n;
    for (int m = 0; m < nf; ++m) {
        Tile t;
        t.expert = tid;
        t.row0 = off + m * GEMM_BM;
        t.nrows = GEMM_BM;
        t.pad = 0;
        tiles[foff + m] = t;
    }
    if (np) {
        Tile t;
        t.expert = tid;
        t.row0 = off + nf * GEMM_BM;
        t.nrows = n - nf * GEMM_BM;
        t.pad = 0;
        tiles[poff] = t;
    }
    const int routed = nfull + npart;
    const int nsh = shared ? (int)((T + GEMM_BM - 1) / GEMM_BM) : 0;
    for (int m = tid; m < nsh; m += 256) {
        Tile t;
        t.expert = E;
        t.row0 = (int)(T * K) + m * GEMM_BM;
        t.nrows = (int)min((int64_t)GEMM_BM, T - (int64_t)m * GEMM_BM);
        t.pad = 0;
        tiles[routed + m] = t;
    }
    if (tid == 0) { ntiles[0] = routed; ntiles[1] = routed + nsh; ntiles[2] = 0; }
}

// Stable scatter of the assignments of one ROUTER_TOKENS-token block into the expert bins.
__global__ __launch_bounds__(256) void k_scatter(const int32_t *__restrict__ idx,
                                                 const int32_t *__restrict__ blkoff,
                                                 const int32_t *__restrict__ expert_off,
                                                 int32_t *__restrict__ perm, int64_t T, int K, int E) {
    __shared__ int wcnt[4][256];
    __shared__ int base[256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int blk = blockIdx.x;
    for (int i = tid; i < 4 * 256; i += 256) (&wcnt[0][0])[i] = 0;
    base[tid] = 0;
    __syncthreads();
    const int items = ROUTER_TOKENS * K;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int r0 = 0; r0 < items; r0 += 256) {
        const int item = r0 + tid;
        const int64_t t = (int64_t)blk * ROUTER_TOKENS + item / K;
        const int j = item % K;
        const bool valid = item < items && t < T;
        const int e = valid ? idx[t * K + j] : 0;
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t bal = __ballot(valid && bit);
            peers &= bit ? bal : ~bal;
        }
        const int rank = __popcll(peers & lt);
        const bool leader = valid && rank == 0;
        if (leader) wcnt[wave][e] = __popcll(peers);
        __syncthreads();
        if (valid) {
            int before = base[e];
            for (int w = 0; w < wave; ++w) before += wcnt[w][e];
            const int pos = expert_off[e] + blkoff[(int64_t)blk * E + e] + before + rank;
            perm[pos] = (int32_t)(t * K + j);
        }
        __syncthreads();
        base[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
        wcnt[0][tid] = wcnt[1][tid] = wcnt[2][tid] = wcnt[3][tid] = 0;
        __syncthreads();
    }
}

}  // namespace

int64_t prefill_max_routed_tiles(int64_t T, int K, int E) {
    const int64_t a = T * K;
    return a / GEMM_BM + (a < E ? a : E);
}

int64_t prefill_max_tiles(int64_t T, int K, int E) {
    return prefill_max_routed_tiles(T, K, E) + (T + GEMM_BM - 1) / GEMM_BM;
}

hipError_t launch_prefill_binning(const Layer &L, int64_t T, const PrefillBufs &b, hipStream_t s) {
    const int nblk = (int)((T + ROUTER_TOKENS - 1) / ROUTER_TOKENS);
    int32_t *counts = b.expert_off + (L.E + 1);        // E ints after expert_off
    hipLaunchKernelGGL(k_colscan, dim3((L.E + 3) / 4), dim3(256), 0, s, b.blkcnt, b.blkoff, counts,
                       nblk, L.E);
    hipLaunchKernelGGL(k_tiles, dim3(1), dim3(256), 0, s, counts, b.expert_off, b.tiles, b.ntiles, b.tile_done,
                       (int)prefill_max_tiles(T, L.K, L.E), L.E, T, L.K, L.has_shared);
    hipLaunchKernelGGL(k_scatter, dim3(nblk), dim3(256), 0, s, b.idx, b.blkoff, b.expert_off, b.perm,
                       T, L.K, L.E);
    return hipGetLastError();
}

}  // namespace qs
