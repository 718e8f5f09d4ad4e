// Token-to-expert permutation: expert histogram, exclusive prefix sum in LDS
// and a stable scatter of the (t, j) pairs into expert-grouped order, plus
// the tile lists of the grouped GEMMs.  Everything stays on the device: the
// GEMM grids are sized by the upper bound of the tile count and surplus
// workgroups exit.
//
// Pages: "Jetson Orin Nano MoE ... expert cache", nondeterminism section (an
// expert that became ready between two readiness checks was never computed;
// here every pair is placed exactly once by a single counting pass), and
// "MoE prefill quantum" (cause section: tokens per expert set the cost).
//
// Determinism: counts use LDS atomics (order-free); positions come from
// ballot-based ranks inside one wave that walks its block's pairs in order,
// so the grouped order is t ascending, then j, within every expert, the same
// as a stable counting sort.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int PAIRS_PER_BLOCK = 1024;

int permute_blocks(int n_pairs)
{
    return (n_pairs + PAIRS_PER_BLOCK - 1) / PAIRS_PER_BLOCK;
}

// Per-block expert histogram: blk[b * E + e] = pairs of block b with expert e.
__global__ __launch_bounds__(256) void permute_hist(const int32_t *__restrict__ idx,
                                                    int32_t *__restrict__ blk, int n_pairs, int E)
{
    extern __shared__ int32_t cnt[];
    for (int e = threadIdx.x; e < E; e += 256)
        cnt[e] = 0;
    __syncthreads();
    const int base = blockIdx.x * PAIRS_PER_BLOCK;
    for (int i = threadIdx.x; i < PAIRS_PER_BLOCK; i += 256) {
        int p = base + i;
        if (p < n_pairs) {
            int e = idx[p];
            atomicAdd(&cnt[e], 1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256)
        blk[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// One workgroup: counts, offsets (exclusive prefix in LDS), per-block start
// positions (written over blk), the shared-expert group and both tile lists.
__global__ __launch_bounds__(1024) void permute_scan(
    int32_t *__restrict__ blk, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    Tile *__restrict__ tiles_a, int32_t *__restrict__ ntiles_a, Tile *__restrict__ tiles_b,
    int32_t *__restrict__ ntiles_b, int bm_a, int bm_b, int nblk, int E, int n_pairs, int T,
    int shared)
{
    __shared__ int32_t s_cnt[1025];
    __shared__ int32_t s_ta[1025];
    __shared__ int32_t s_tb[1025];
    __shared__ int32_t s_off[1025];
    __shared__ int32_t s_warp[3][16];
    const int tid = threadIdx.x;
    const int G = E + (shared ? 1 : 0);  // groups
    // Column sums over blocks; blk[b][e] becomes the running prefix.
    for (int e = tid; e < E; e += 1024) {
        int run = 0;
        for (int b = 0; b < nblk; ++b) {
            int c = blk[(int64_t)b * E + e];
            blk[(int64_t)b * E + e] = run;
            run += c;
        }
        s_cnt[e] = run;
    }
    if (tid == 0 && shared)
        s_cnt[E] = T;
    __syncthreads();
    // Exclusive scan over the groups of: row counts, tiles of bm_a, tiles of bm_b.
    int c = tid < G ? s_cnt[tid] : 0;
    int va = tid < G ? (c + bm_a - 1) / bm_a : 0;
    int vb = tid < G ? (c + bm_b - 1) / bm_b : 0;
    int ic = c, ia = va, ib = vb;  // inclusive scans within the wave
    const int lane = tid & 63, wv = tid >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int tc = __shfl_up(ic, off), ta = __shfl_up(ia, off), tb = __shfl_up(ib, off);
        if (lane >= off) {
            ic += tc;
            ia += ta;
            ib += tb;
        }
    }
    if (lane == 63) {
        s_warp[0][wv] = ic;
        s_warp[1][wv] = ia;
        s_warp[2][wv] = ib;
    }
    __syncthreads();
    int pc = 0, pa = 0, pb = 0;
    for (int w = 0; w < wv; ++w) {
        pc += s_warp[0][w];
        pa += s_warp[1][w];
        pb += s_warp[2][w];
    }
    const int exc = pc + ic - c, exa = pa + ia - va, exb = pb + ib - vb;
    if (tid < G) {
        counts[tid] = c;
        offsets[tid] = exc;
        s_off[tid] = exc;
        s_ta[tid] = exa;
        s_tb[tid] = exb;
    }
    if (tid == G - 1) {
        offsets[G] = exc + c;
        *ntiles_a = exa + va;
        *ntiles_b = exb + vb;
    }
    if (!shared && tid == 0)
        offsets[E + 1] = n_pairs;  // empty shared group
    __syncthreads();
    // Per-block start positions inside each expert's range.
    for (int e = tid; e < E; e += 1024) {
        int o = s_off[e];
        for (int b = 0; b < nblk; ++b)
            blk[(int64_t)b * E + e] += o;
    }
    // Tile lists.
    for (int g = tid; g < G; g += 1024) {
        int cg = g < E ? s_cnt[g] : T;
        int og = s_off[g];
        for (int r = 0, t = s_ta[g]; r < cg; r += bm_a, ++t)
            tiles_a[t] = Tile{g, og + r};
        for (int r = 0, t = s_tb[g]; r < cg; r += bm_b, ++t)
            tiles_b[t] = Tile{g, og + r};
    }
}

// Stable scatter.  One wave per block walks the block's pairs 64 at a time in
// pair order; lanes with equal experts are ranked by lane index from a
// ballot-built match mask, and the lowest such lane advances the expert's
// running position in LDS.
__global__ __launch_bounds__(64) void permute_scatter(const int32_t *__restrict__ idx,
                                                     const int32_t *__restrict__ blk,
                                                     int32_t *__restrict__ row_src,
                                                     int32_t *__restrict__ row_tok,
                                                     int32_t *__restrict__ row_of, int n_pairs,
                                                     int E, int T, int k, int shared)
{
    extern __shared__ int32_t run[];
    const int lane = threadIdx.x;
    for (int e = lane; e < E; e += 64)
        run[e] = blk[(int64_t)blockIdx.x * E + e];
    __syncthreads();
    const int base = blockIdx.x * PAIRS_PER_BLOCK;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int s = 0; s < PAIRS_PER_BLOCK; s += 64) {
        const int p = base + s + lane;
        const bool valid = p < n_pairs;
        const int e = valid ? idx[p] : 0;
        uint64_t match = __ballot(valid);
        for (int bit = 0; bit < 10; ++bit) {
            uint64_t ones = __ballot(valid && ((e >> bit) & 1));
            match &= ((e >> bit) & 1) ? ones : ~ones;
        }
        const int rank = __popcll(match & lt);
        int pos = 0;
        if (valid)
            pos = run[e] + rank;
        __syncthreads();
        if (valid) {
            row_src[pos] = p;
            row_tok[pos] = p / k;
            row_of[p] = pos;
            if (rank == 0)
                run[e] += __popcll(match);
        }
        __syncthreads();
    }
    // Shared-expert rows follow the routed ones, in token order.
    if (shared && blockIdx.x == 0) {
        for (int t = lane; t < T; t += 64) {
            row_src[n_pairs + t] = n_pairs + t;
            row_tok[n_pairs + t] = t;
        }
    }
}

// Work items of the streaming GEMMs, one thread per (tile, column tile):
// expert-major, then column tile, then row tile, so that item lists dealt out
// in contiguous runs keep an expert on one XCD.  The tiles of expert g start
// at s_g = tile index - its rank inside the expert; its items at ntn * s_g.
__global__ __launch_bounds__(256) void permute_items(const Tile *__restrict__ tiles,
                                                     const int32_t *__restrict__ ntiles,
                                                     const int32_t *__restrict__ offsets, int bm,
                                                     int ntn, int wrows, int4 *__restrict__ items)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int n_t = *ntiles;
    const int tau = i / ntn, nt = i - tau * ntn;
    if (tau >= n_t)
        return;
    const Tile tl = tiles[tau];
    const int og = offsets[tl.g], cg = offsets[tl.g + 1] - og;
    const int rank = (tl.row0 - og) / bm;
    const int sg = tau - rank;
    const int na = (cg + bm - 1) / bm;
    items[ntn * sg + nt * na + rank] = int4{tl.g, tl.row0, min(bm, cg - (tl.row0 - og)), nt * wrows};
}

void launch_permute(const PermuteArgs &a, hipStream_t st)
{
    const int n_pairs = a.T * a.k;
    const int nblk = permute_blocks(n_pairs);
    if (nblk > 0)
        permute_hist<<<nblk, 256, a.E * sizeof(int32_t), st>>>(a.idx, a.blk, n_pairs, a.E);
    permute_scan<<<1, 1024, 0, st>>>(a.blk, a.counts, a.offsets, a.tiles_a, a.ntiles_a, a.tiles_b,
                                     a.ntiles_b, a.bm_a, a.bm_b, nblk, a.E, n_pairs, a.T, a.shared);
    if (nblk > 0)
        permute_scatter<<<nblk, 64, a.E * sizeof(int32_t), st>>>(
            a.idx, a.blk, a.row_src, a.row_tok, a.row_of, n_pairs, a.E, a.T, a.k, a.shared);
    if (a.items_a && a.max_tiles_a > 0)
        permute_items<<<(a.max_tiles_a * a.ntn_a + 255) / 256, 256, 0, st>>>(
            a.tiles_a, a.ntiles_a, a.offsets, a.bm_a, a.ntn_a, a.wrows_a, a.items_a);
    if (a.items_b && a.max_tiles_b > 0)
        permute_items<<<(a.max_tiles_b * a.ntn_b + 255) / 256, 256, 0, st>>>(
            a.tiles_b, a.ntiles_b, a.offsets, a.bm_b, a.ntn_b, a.wrows_b, a.items_b);
}

}  // namespace moe
