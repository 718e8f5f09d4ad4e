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
// Determinism: counts use integer atomics (order-free), in LDS here or in
// global memory where the segmented router's top-k kernel counts the block
// histogram; positions come from ballot-based ranks inside waves that walk
// their pairs in order, so the grouped order is t ascending, then j, within
// every expert, the same as a stable counting sort.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int PAIRS_PER_BLOCK = PERMUTE_PAIRS_PER_BLOCK;
// Passes whose per-block histograms fit in this many LDS counters build them
// inside the scan kernel (one launch less).
constexpr int FUSED_HIST = 8192;
// Most permutation blocks placed by permute_place (see launch_permute).
constexpr int PLACE_MAX_BLOCKS = 256;

// Orders one wave's LDS accesses across its lanes (no other wave shares
// the data).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

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

// One workgroup of 1024 threads: counts, offsets (exclusive prefix in LDS),
// the shared-expert group and both tile lists; with POS also the per-block
// start positions (written over blk), and with idx given (nblk * E <=
// FUSED_HIST) it counts the blocks' pairs itself.  Without POS blk is only
// read (the scatter workgroups of permute_place read it at the same time).
template <bool POS>
__device__ __forceinline__ void scan_groups(
    const int32_t *__restrict__ idx,
    int32_t *__restrict__ blk, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    Tile *__restrict__ tiles_a, int32_t *__restrict__ ntiles_a, Tile *__restrict__ tiles_b,
    int32_t *__restrict__ ntiles_b, int bm_a, int bm_b, int nblk, int E, int n_pairs, int T,
    int shared, int4 *__restrict__ items_a, int ntn_a, int wrows_a, int4 *__restrict__ items_b,
    int ntn_b, int wrows_b)
{
    __shared__ int32_t s_cnt[1025];
    __shared__ int32_t s_ta[1025];
    __shared__ int32_t s_tb[1025];
    __shared__ int32_t s_off[1025];
    __shared__ int32_t s_warp[3][16];
    __shared__ int32_t s_nt[2];
    __shared__ int32_t s_blk[POS ? FUSED_HIST : 1];
    const int tid = threadIdx.x;
    const int G = E + (shared ? 1 : 0);  // groups
    constexpr int SCH = 16;
    if constexpr (!POS) {
        // column sums over blocks only
        for (int e = tid; e < E; e += 1024) {
            int run = 0;
            for (int b0 = 0; b0 < nblk; b0 += SCH) {
                int c[SCH];
#pragma unroll
                for (int i = 0; i < SCH; ++i)
                    c[i] = b0 + i < nblk ? blk[(int64_t)(b0 + i) * E + e] : 0;
#pragma unroll
                for (int i = 0; i < SCH; ++i)
                    run += c[i];
            }
            s_cnt[e] = run;
        }
    } else if (idx) {
        // Per-block histograms in LDS, then their running prefixes in place.
        for (int i = tid; i < nblk * E; i += 1024)
            s_blk[i] = 0;
        __syncthreads();
        // the pairs' experts are loaded PB at a time, all in flight together
        constexpr int PB = 16;
        for (int p0 = tid; p0 < n_pairs; p0 += 1024 * PB) {
            int ev[PB];
#pragma unroll
            for (int i = 0; i < PB; ++i) {
                const int p = p0 + 1024 * i;
                ev[i] = p < n_pairs ? idx[p] : -1;
            }
#pragma unroll
            for (int i = 0; i < PB; ++i)
                if (ev[i] >= 0)
                    atomicAdd(&s_blk[((p0 + 1024 * i) / PAIRS_PER_BLOCK) * E + ev[i]], 1);
        }
        __syncthreads();
        for (int e = tid; e < E; e += 1024) {
            int run = 0;
            for (int b0 = 0; b0 < nblk; b0 += SCH) {
                int c[SCH];
#pragma unroll
                for (int i = 0; i < SCH; ++i)  // all reads in flight together
                    c[i] = b0 + i < nblk ? s_blk[(b0 + i) * E + e] : 0;
#pragma unroll
                for (int i = 0; i < SCH; ++i)
                    if (b0 + i < nblk) {
                        s_blk[(b0 + i) * E + e] = run;
                        run += c[i];
                    }
            }
            s_cnt[e] = run;
        }
    } else
    // Column sums over blocks (the block counts are read SCH at a time, all
    // in flight together); blk[b][e] becomes the running prefix.
    for (int e = tid; e < E; e += 1024) {
        int run = 0;
        for (int b0 = 0; b0 < nblk; b0 += SCH) {
            int c[SCH];
#pragma unroll
            for (int i = 0; i < SCH; ++i)
                c[i] = b0 + i < nblk ? blk[(int64_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < SCH; ++i)
                if (b0 + i < nblk) {
                    blk[(int64_t)(b0 + i) * E + e] = run;
                    run += c[i];
                }
        }
        s_cnt[e] = run;
    }
    if (tid == 0 && shared)
        s_cnt[E] = T;
    __syncthreads();
    // Exclusive scan over the groups of: row counts, tiles of bm_a, tiles of
    // bm_b (only the waves holding groups take part).
    const int lane = tid & 63, wv = tid >> 6, ngw = (G + 63) / 64;
    int c = 0, va = 0, vb = 0, ic = 0, ia = 0, ib = 0;
    if (wv < ngw) {  // uniform
        if (tid < G) {
            c = s_cnt[tid];
            va = (c + bm_a - 1) / bm_a;
            vb = (c + bm_b - 1) / bm_b;
        }
        ic = wave_scan_add(c);
        ia = wave_scan_add(va);
        ib = wave_scan_add(vb);
        if (lane == 63) {
            s_warp[0][wv] = ic;
            s_warp[1][wv] = ia;
            s_warp[2][wv] = ib;
        }
    }
    __syncthreads();
    if (wv < ngw) {
        int pc = 0, pa = 0, pb = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) {  // all reads in flight together
            const bool in = w < wv;
            pc += in ? s_warp[0][w] : 0;
            pa += in ? s_warp[1][w] : 0;
            pb += in ? s_warp[2][w] : 0;
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
            s_nt[0] = exa + va;
            s_nt[1] = exb + vb;
        }
        if (!shared && tid == 0)
            offsets[E + 1] = n_pairs;  // empty shared group
    }
    __syncthreads();
    // Per-block start positions inside each expert's range.
    if constexpr (POS)
    for (int e = tid; e < E; e += 1024) {
        const int o = s_off[e];
        if (idx) {
            for (int b = 0; b < nblk; ++b)
                blk[(int64_t)b * E + e] = s_blk[b * E + e] + o;
            continue;
        }
        for (int b0 = 0; b0 < nblk; b0 += SCH) {
            int c[SCH];
#pragma unroll
            for (int i = 0; i < SCH; ++i)
                c[i] = b0 + i < nblk ? blk[(int64_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < SCH; ++i)
                if (b0 + i < nblk)
                    blk[(int64_t)(b0 + i) * E + e] = c[i] + o;
        }
    }
    // Tile lists, and the work items of the streaming GEMMs: expert-major,
    // then column tile, then row tile, so that item lists dealt out in
    // contiguous runs keep an expert on one XCD.  One thread per tile; a
    // tile's group is the last one whose first tile is not after it (groups
    // without rows take no tiles).
    const int nta = s_nt[0], ntb = s_nt[1];
    for (int i = tid; i < nta + ntb; i += 1024) {
        const bool a = i < nta;
        const int j = a ? i : i - nta;
        const int *st = a ? s_ta : s_tb;
        int lo = 0, hi = G - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (st[mid] <= j)
                lo = mid;
            else
                hi = mid - 1;
        }
        const int g = lo, m = j - st[g];
        const int cg = g < E ? s_cnt[g] : T, og = s_off[g];
        const int bm = a ? bm_a : bm_b;
        const int r0 = og + m * bm, nr = min(bm, cg - m * bm);
        (a ? tiles_a : tiles_b)[j] = Tile{g, r0};
        int4 *items = a ? items_a : items_b;
        if (items) {
            const int ntn = a ? ntn_a : ntn_b, wrows = a ? wrows_a : wrows_b;
            const int nt_g = (cg + bm - 1) / bm;  // the group's row tiles
            for (int nt = 0; nt < ntn; ++nt)
                items[ntn * st[g] + nt * nt_g + m] = int4{g, r0, nr, nt * wrows};
        }
    }
}

__global__ __launch_bounds__(1024) void permute_scan(
    const int32_t *__restrict__ idx,
    int32_t *__restrict__ blk, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    Tile *__restrict__ tiles_a, int32_t *__restrict__ ntiles_a, Tile *__restrict__ tiles_b,
    int32_t *__restrict__ ntiles_b, int bm_a, int bm_b, int nblk, int E, int n_pairs, int T,
    int shared, int4 *__restrict__ items_a, int ntn_a, int wrows_a, int4 *__restrict__ items_b,
    int ntn_b, int wrows_b)
{
    scan_groups<true>(idx, blk, counts, offsets, tiles_a, ntiles_a, tiles_b, ntiles_b, bm_a, bm_b,
                      nblk, E, n_pairs, T, shared, items_a, ntn_a, wrows_a, items_b, ntn_b, wrows_b);
}

// One block of PAIRS_PER_BLOCK pairs placed by 1024 threads, one pair each,
// without a separate scan pass: the block's first position in each expert's
// range is the expert's offset (exclusive prefix over the experts of the
// column sums of the block histograms) plus that expert's pairs in the
// earlier blocks, both formed here from the histograms; inside the block the
// waves follow in order and a wave's lanes with equal experts are ranked by
// a ballot-built match mask.  The same grouped order as permute_scatter (t,
// then j, within every expert).
__device__ __forceinline__ void place_block(const int32_t *__restrict__ idx,
                                            const int32_t *__restrict__ blk, int nblk, int b,
                                            int32_t *__restrict__ row_src,
                                            int32_t *__restrict__ row_tok,
                                            int32_t *__restrict__ row_of, int n_pairs, int E,
                                            int T, int k, int shared)
{
    static_assert(PAIRS_PER_BLOCK == 1024, "one pair per thread");
    __shared__ int32_t s_start[1024];
    __shared__ uint16_t s_wc[16][1024];  // per wave and expert: pairs, then pairs in earlier waves
    __shared__ int32_t s_wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int p = b * PAIRS_PER_BLOCK + tid;
    const int e = p < n_pairs ? idx[p] : -1;
    constexpr int SCH = 16;
    // column sums over all blocks (the expert's rows) and over those before b
    int tot = 0, pre = 0;
    if (tid < E) {
        for (int b0 = 0; b0 < nblk; b0 += SCH) {
            int c[SCH];
#pragma unroll
            for (int i = 0; i < SCH; ++i)  // all reads in flight together
                c[i] = b0 + i < nblk ? blk[(int64_t)(b0 + i) * E + tid] : 0;
#pragma unroll
            for (int i = 0; i < SCH; ++i) {
                tot += c[i];
                pre += b0 + i < b ? c[i] : 0;
            }
        }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q)
        s_wc[q][tid] = 0;
    // exclusive prefix of the experts' rows
    const int inc = wave_scan_add(tot);
    if (lane == 63)
        s_wsum[wv] = inc;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w)
        before += w < wv ? s_wsum[w] : 0;
    if (tid < E)
        s_start[tid] = before + inc - tot + pre;
    // rank among this wave's earlier pairs of the same expert
    const bool valid = e >= 0;
    uint64_t same = __ballot(valid);
    for (int bit = 0; bit < 10; ++bit) {
        const bool on = (e >> bit) & 1;
        const uint64_t ones = __ballot(valid && on);
        same &= on ? ones : ~ones;
    }
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(same & below);
    if (valid && rank == 0)  // one writer per wave and expert
        s_wc[wv][e] = (uint16_t)__popcll(same);
    __syncthreads();
    if (tid < E) {
        int run = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            const int c = s_wc[w][tid];
            s_wc[w][tid] = (uint16_t)run;
            run += c;
        }
    }
    __syncthreads();
    if (valid) {
        const int pos = s_start[e] + s_wc[wv][e] + rank;
        row_src[pos] = p;
        row_tok[pos] = p / k;
        row_of[p] = pos;
    }
    // shared-expert rows follow the routed ones, in token order
    if (shared && b == 0) {
        for (int t = tid; t < T; t += 1024) {
            row_src[n_pairs + t] = n_pairs + t;
            row_tok[n_pairs + t] = t;
        }
    }
}

// The permutation of a pass whose block histograms are counted already (by
// the segmented router's top-k kernel), in one launch: workgroups 0 ..
// nblk-1 place their blocks' pairs (place_block) while workgroup nblk forms
// the counts, offsets, tile lists and work items (scan_groups without the
// per-block positions, reading the histograms the others read too).
__global__ __launch_bounds__(1024) void permute_place(
    const int32_t *__restrict__ idx, int32_t *__restrict__ blk, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, Tile *__restrict__ tiles_a, int32_t *__restrict__ ntiles_a,
    Tile *__restrict__ tiles_b, int32_t *__restrict__ ntiles_b, int bm_a, int bm_b, int nblk,
    int E, int n_pairs, int T, int shared, int4 *__restrict__ items_a, int ntn_a, int wrows_a,
    int4 *__restrict__ items_b, int ntn_b, int wrows_b, int32_t *__restrict__ row_src,
    int32_t *__restrict__ row_tok, int32_t *__restrict__ row_of, int k)
{
    if ((int)blockIdx.x == nblk) {  // uniform
        scan_groups<false>(nullptr, blk, counts, offsets, tiles_a, ntiles_a, tiles_b, ntiles_b,
                           bm_a, bm_b, nblk, E, n_pairs, T, shared, items_a, ntn_a, wrows_a,
                           items_b, ntn_b, wrows_b);
        return;
    }
    place_block(idx, blk, nblk, blockIdx.x, row_src, row_tok, row_of, n_pairs, E, T, k, shared);
}

// Stable scatter.  Each of a block's 4 waves walks a quarter of its pairs 64
// at a time in pair order, starting every expert after the earlier quarters'
// pairs of that expert (integer LDS counts); lanes with equal experts are
// ranked by lane index from a ballot-built match mask, and the lowest such
// lane advances the expert's running position.
__global__ __launch_bounds__(256) void permute_scatter(const int32_t *__restrict__ idx,
                                                      const int32_t *__restrict__ blk,
                                                      int32_t *__restrict__ row_src,
                                                      int32_t *__restrict__ row_tok,
                                                      int32_t *__restrict__ row_of, int n_pairs,
                                                      int E, int T, int k, int shared)
{
    // run[w * E + e]: next position of expert e for wave w, which owns the
    // block's pairs w*256 .. +255 (a quarter, in pair order).
    extern __shared__ int32_t run[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int base = blockIdx.x * PAIRS_PER_BLOCK + wave * (PAIRS_PER_BLOCK / 4);
    constexpr int NS = PAIRS_PER_BLOCK / 4 / 64;
    int ev[NS];  // this wave's experts, all loads in flight at once
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int p = base + 64 * i + lane;
        ev[i] = p < n_pairs ? idx[p] : -1;
    }
    for (int i = threadIdx.x; i < 4 * E; i += 256)
        run[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NS; ++i)
        if (ev[i] >= 0)
            atomicAdd(&run[wave * E + ev[i]], 1);  // integer counts: order-free
    __syncthreads();
    // Each wave starts after the earlier quarters' pairs of the same expert.
    for (int e = threadIdx.x; e < E; e += 256) {
        int pos = blk[(int64_t)blockIdx.x * E + e];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int c = run[w * E + e];
            run[w * E + e] = pos;
            pos += c;
        }
    }
    __syncthreads();
    int32_t *wrun = run + wave * E;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int p = base + 64 * i + lane;
        const int e = ev[i];
        const bool valid = e >= 0;
        uint64_t match = __ballot(valid);
        for (int bit = 0; bit < 10; ++bit) {
            const uint64_t ones = __ballot(valid && ((e >> bit) & 1));
            match &= ((e >> bit) & 1) ? ones : ~ones;
        }
        const int rank = __popcll(match & lt);
        int pos = 0;
        if (valid)
            pos = wrun[e] + rank;
        wave_lds_sync();
        if (valid) {
            row_src[pos] = p;
            row_tok[pos] = p / k;
            row_of[p] = pos;
            if (rank == 0)
                wrun[e] += __popcll(match);
        }
        wave_lds_sync();
    }
    // Shared-expert rows follow the routed ones, in token order.
    if (shared && blockIdx.x == 0) {
        for (int t = threadIdx.x; t < T; t += 256) {
            row_src[n_pairs + t] = n_pairs + t;
            row_tok[n_pairs + t] = t;
        }
    }
}

void launch_permute(const PermuteArgs &a, hipStream_t st)
{
    const int n_pairs = a.T * a.k;
    const int nblk = permute_blocks(n_pairs);
    // Each placing workgroup sums the histograms of all blocks, so the work
    // and L2 reads of the one-launch form grow as nblk^2: beyond 256 blocks
    // (T*k > 262,144 pairs; the sweep's T=65,536 was 3% slower with it) the
    // separate scan, whose one workgroup forms the prefixes once, is used.
    if (a.hist_done && nblk > 0 && nblk <= PLACE_MAX_BLOCKS && a.E <= 1024) {
        permute_place<<<nblk + 1, 1024, 0, st>>>(
            a.idx, a.blk, a.counts, a.offsets, a.tiles_a, a.ntiles_a, a.tiles_b, a.ntiles_b,
            a.bm_a, a.bm_b, nblk, a.E, n_pairs, a.T, a.shared, a.items_a, a.ntn_a, a.wrows_a,
            a.items_b, a.ntn_b, a.wrows_b, a.row_src, a.row_tok, a.row_of, a.k);
        return;
    }
    const bool fused = !a.hist_done && nblk * a.E <= FUSED_HIST;
    if (nblk > 0 && !fused && !a.hist_done)
        permute_hist<<<nblk, 256, a.E * sizeof(int32_t), st>>>(a.idx, a.blk, n_pairs, a.E);
    permute_scan<<<1, 1024, 0, st>>>(fused ? a.idx : nullptr, a.blk, a.counts, a.offsets, a.tiles_a, a.ntiles_a, a.tiles_b,
                                     a.ntiles_b, a.bm_a, a.bm_b, nblk, a.E, n_pairs, a.T, a.shared,
                                     a.items_a, a.ntn_a, a.wrows_a, a.items_b, a.ntn_b, a.wrows_b);
    if (nblk > 0)
        permute_scatter<<<nblk, 256, 4 * a.E * sizeof(int32_t), st>>>(
            a.idx, a.blk, a.row_src, a.row_tok, a.row_of, n_pairs, a.E, a.T, a.k, a.shared);
}

}  // namespace moe
