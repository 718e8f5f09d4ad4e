// Weight-streaming grouped expert GEMM on bf16 MFMA (gfx950).
//
// Same contract as the tiled kernel in expert_gemm.hip (gate+up with the
// SwiGLU epilogue, or down with the routing-weight scale into per-pair
// staging rows); built for the shapes of this layer, where every workload sits
// below the bf16 ridge point and the expert weights are the traffic that
// matters ("MoE prefill quantum", Table 9 and the text after it: small chunks
// read nearly every expert's weights for a few rows each).
//
//  * Each wave owns 32 weight rows per matrix (two 16-row MFMA blocks) and
//    streams them from HBM straight into registers through a prefetch ring of
//    4 or 8 steps of 32 K: no LDS and no barrier on the weight path, every
//    weight element read once per tile.
//  * The tile's token rows (gathered through row_src) are staged in LDS in
//    double-buffered 128-wide K chunks shared by the 4 waves.
//  * The MFMA takes the weights as its A operand and the tokens as B; with
//    the weight rows of the two column blocks interleaved by fours, a lane
//    ends up with 8 adjacent output columns of one token row and stores them
//    as one 16-byte word (64 contiguous bytes per row and wave).
//  * Work items are ordered expert-major (then weight tile, then row tile)
//    and dealt out XCD by XCD in contiguous runs, so an expert's weight tiles
//    and token rows are fetched into one XCD's L2 and reused there.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int SKC = 128;      // K elements of one staged token chunk
constexpr int SLD = SKC + 8;  // padded LDS row (bf16), 272 bytes
constexpr int WROWS = 128;    // weight rows per workgroup and matrix (4 waves x 32)

struct StreamP {
    const uint16_t *x;        // GU: activations [T, H]; DC: h [rows, ldh]
    const uint16_t *w0, *w1;  // routed matrices [E, N, K]
    const uint16_t *s0, *s1;  // shared expert matrices [N, K]
    const int32_t *row_src, *offsets;
    const float *topk_w;
    uint16_t *out;            // GU: h; DC: stage
    const Tile *tiles;
    const int32_t *ntiles;
    const uint32_t *items;
    int T, H, E, k, I, Is, ldh, ntn;
};

// Token chunk registers as one vector value (an array here would be placed
// in scratch memory by the compiler).
template <int N>
using u32v = uint32_t __attribute__((ext_vector_type(4 * N)));

template <int N>
__device__ __forceinline__ void chunk_load(u32v<N> &r, const uint16_t *const (&src)[N], int off)
{
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const uint4 t = *(const uint4 *)(src[i] + off);
        r[4 * i] = t.x;
        r[4 * i + 1] = t.y;
        r[4 * i + 2] = t.z;
        r[4 * i + 3] = t.w;
    }
}

template <int N>
__device__ __forceinline__ void chunk_store(const u32v<N> &r, uint16_t *dst, const int (&off)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i)
        *(uint4 *)(dst + off[i]) = uint4{r[4 * i], r[4 * i + 1], r[4 * i + 2], r[4 * i + 3]};
}

template <int BM, bool GU>
__global__ __launch_bounds__(256) void expert_stream(StreamP p)
{
    constexpr int NB = GU ? 2 : 1;             // weight matrices
    constexpr int CB = 2;                      // 16-row weight blocks per wave
    constexpr int MB = BM / 16;                // 16-row token blocks
    constexpr int ACH = BM * (SKC / 8) / 256;  // 16-byte token chunks per thread
    constexpr int SD = 8;                      // prefetch ring depth in 32-wide K steps
    static_assert(ACH >= 1 && ACH * 256 == BM * SKC / 8, "token staging");
    static_assert(CB == 2, "the epilogue packs two column blocks per lane");

    __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * SLD];

    // Work item: the item list (expert-major, column tile, row tile) is
    // dealt out in 8 contiguous runs, one per XCD (workgroups go round-robin
    // over the XCDs), so one expert's tiles share an L2.
    const int ntiles = *p.ntiles;
    const int total = ntiles * p.ntn;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per = (total + 7) >> 3;
    const int wi = xcd * per + slot;
    if (slot >= per || wi >= total)
        return;
    const uint32_t item = p.items[wi];
    const int nt = (int)(item >> 20);
    const Tile tile = p.tiles[item & 0xFFFFF];
    const int g = tile.g, row0 = tile.row0;
    const bool routed = g < p.E;
    const int nrows = min(BM, p.offsets[g + 1] - row0);
    const int n_pairs = p.T * p.k;
    const int N = GU ? (routed ? p.I : p.Is) : p.H;
    const int K = GU ? p.H : (routed ? p.I : p.Is);
    const int n0 = nt * WROWS;
    if (n0 >= N)
        return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int mbn = (nrows + 15) >> 4;  // row blocks holding tokens (uniform)

    // Weight rows of this lane: MFMA row l16 of block cb is weight row
    // n0 + wave*32 + 8*(l16/4) + 4*cb + l16%4, so that after the MFMA the lane
    // with lg = l16/4 holds 8 consecutive output columns (4 per block) and
    // stores them as one 16-byte word.
    const int64_t wstride = (int64_t)N * K;
    const uint16_t *wbase0 = routed ? p.w0 + (int64_t)g * wstride : p.s0;
    const uint16_t *wbase1 = GU ? (routed ? p.w1 + (int64_t)g * wstride : p.s1) : nullptr;
    const uint16_t *wp[NB][CB];
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
            wp[m][cb] = (m == 0 ? wbase0 : wbase1) +
                        (int64_t)(n0 + wave * 32 + 8 * (l16 >> 2) + 4 * cb + (l16 & 3)) * K +
                        lg * 8;

    // Token rows staged by this thread: all row_src loads first, then the
    // row pointers (selects, no branches).
    const uint16_t *asrc[ACH];
    int aoff[ACH];
    int prow[ACH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        const int r = (tid + 256 * i) >> 4;
        prow[i] = GU ? p.row_src[row0 + min(r, nrows - 1)] : row0 + min(r, nrows - 1);
    }
    const int nsteps = K / 32;
    const int nchunks = K / SKC;  // even: K % 256 == 0

    // Weight prefetch goes out before the row pointers are needed.
    uint4 bq[SD][NB][CB];
    // Loads are never predicated (a branch around a load makes the compiler
    // wait for every outstanding load): steps past the end re-read the last.
#pragma unroll
    for (int d = 0; d < SD; ++d)
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
                bq[d][m][cb] = *(const uint4 *)(wp[m][cb] + min(d, nsteps - 1) * 32);

#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        const int q = tid + 256 * i;
        const int r = q >> 4, c8 = q & 15;
        int64_t roff;
        if (GU) {
            const int pr = prow[i];
            const int t = pr < n_pairs ? pr / p.k : pr - n_pairs;
            roff = (int64_t)t * p.H;
        } else {
            roff = (int64_t)prow[i] * p.ldh;
        }
        asrc[i] = p.x + roff + c8 * 8;
        aoff[i] = r * SLD + c8 * 8;
    }
    u32v<ACH> ra;

    floatx4 acc[NB][CB][MB];
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[m][cb][mb] = floatx4{0, 0, 0, 0};

    chunk_load<ACH>(ra, asrc, 0);
    chunk_store<ACH>(ra, sA[0], aoff);
    __syncthreads();
    chunk_load<ACH>(ra, asrc, min(1, nchunks - 1) * SKC);

    for (int c = 0; c < nchunks; c += 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int cc = c + h;
            const uint16_t *As = sA[cc & 1];
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const int d = (h * 4 + s4) % SD;
                const int step = cc * 4 + s4;
                bf16x8 tf[MB];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    tf[mb] = as_bf16x8(*(const uint4 *)(As + (mb * 16 + l16) * SLD + s4 * 32 + lg * 8));
#pragma unroll
                for (int m = 0; m < NB; ++m)
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        const bf16x8 wf = as_bf16x8(bq[d][m][cb]);
                        bq[d][m][cb] = *(const uint4 *)(wp[m][cb] + min(step + SD, nsteps - 1) * 32);
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
                            if (mb < mbn)  // row blocks past the tile's rows are skipped
                                acc[m][cb][mb] = mfma16(wf, tf[mb], acc[m][cb][mb]);
                    }
            }
            chunk_store<ACH>(ra, sA[(cc + 1) & 1], aoff);
            __syncthreads();
            chunk_load<ACH>(ra, asrc, min(cc + 2, nchunks - 1) * SKC);
        }
    }

    // Epilogue: lane holds columns n .. n+7 of token row mb*16 + l16
    // (block cb covers n + 4*cb .. n + 4*cb + 3).
    const int n = n0 + wave * 32 + lg * 8;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int mr = mb * 16 + l16;
        if (mr >= nrows)
            continue;
        const int pos = row0 + mr;
        uint4 o;
        if (GU) {
            const floatx4 g0 = acc[0][0][mb], u0 = acc[NB - 1][0][mb];
            const floatx4 g1 = acc[0][1][mb], u1 = acc[NB - 1][1][mb];
            o.x = pack_bf2(silu(g0[0]) * u0[0], silu(g0[1]) * u0[1]);
            o.y = pack_bf2(silu(g0[2]) * u0[2], silu(g0[3]) * u0[3]);
            o.z = pack_bf2(silu(g1[0]) * u1[0], silu(g1[1]) * u1[1]);
            o.w = pack_bf2(silu(g1[2]) * u1[2], silu(g1[3]) * u1[3]);
            *(uint4 *)(p.out + (int64_t)pos * p.ldh + n) = o;
        } else {
            const int pr = p.row_src[pos];
            const float wt = pr < n_pairs ? p.topk_w[pr] : 1.0f;
            const floatx4 v0 = acc[0][0][mb], v1 = acc[0][1][mb];
            o.x = pack_bf2(v0[0] * wt, v0[1] * wt);
            o.y = pack_bf2(v0[2] * wt, v0[3] * wt);
            o.z = pack_bf2(v1[0] * wt, v1[1] * wt);
            o.w = pack_bf2(v1[2] * wt, v1[3] * wt);
            *(uint4 *)(p.out + (int64_t)pr * p.H + n) = o;
        }
    }
}

template <int BM, bool GU>
void run(const ExpertArgs &a, hipStream_t st)
{
    StreamP p;
    p.x = (const uint16_t *)(GU ? a.x : a.h);
    p.w0 = (const uint16_t *)(GU ? a.w_gate : a.w_down);
    p.w1 = (const uint16_t *)(GU ? a.w_up : nullptr);
    p.s0 = (const uint16_t *)(GU ? a.sh_gate : a.sh_down);
    p.s1 = (const uint16_t *)(GU ? a.sh_up : nullptr);
    p.row_src = a.row_src;
    p.offsets = a.offsets;
    p.topk_w = a.topk_w;
    p.out = (uint16_t *)(GU ? a.h : a.stage);
    p.tiles = GU ? a.tiles_gu : a.tiles_dc;
    p.ntiles = GU ? a.ntiles_gu : a.ntiles_dc;
    p.items = GU ? a.items_gu : a.items_dc;
    p.T = a.T;
    p.H = a.H;
    p.E = a.E;
    p.k = a.k;
    p.I = a.I;
    p.Is = a.I_shared;
    p.ldh = a.I > a.I_shared ? a.I : a.I_shared;
    const int N = GU ? p.ldh : a.H;
    p.ntn = (N + WROWS - 1) / WROWS;
    const int64_t items = (int64_t)p.ntn * (GU ? a.max_tiles_gu : a.max_tiles_dc);
    if (items == 0)
        return;
    const unsigned grid = (unsigned)((items + 7) / 8 * 8);
    expert_stream<BM, GU><<<grid, 256, 0, st>>>(p);
}

}  // namespace

bool stream_ok(const ExpertArgs &a, bool gu)
{
    if (a.act != ACT_BF16 || a.wdt != W_BF16)
        return false;
    if (gu)
        return a.H % 256 == 0 && a.I % WROWS == 0 && a.I_shared % WROWS == 0;
    return a.I % 256 == 0 && a.I_shared % 256 == 0 && a.H % WROWS == 0;
}

int stream_ntn(const ExpertArgs &a, bool gu)
{
    if (!stream_ok(a, gu))
        return 0;
    const int N = gu ? (a.I > a.I_shared ? a.I : a.I_shared) : a.H;
    return (N + WROWS - 1) / WROWS;
}

int stream_bm(const ExpertArgs &a)
{
    const int64_t avg = (int64_t)a.shape_T * a.k / a.E;
    if (avg <= 16)
        return 16;
    if (avg <= 32)
        return 32;
    return 128;
}

void launch_stream(const ExpertArgs &a, bool gu, hipStream_t st)
{
    const int bm = stream_bm(a);
    if (gu) {
        if (bm == 16)
            run<16, true>(a, st);
        else if (bm == 32)
            run<32, true>(a, st);
        else if (bm == 64)
            run<64, true>(a, st);
        else
            run<128, true>(a, st);
    } else {
        if (bm == 16)
            run<16, false>(a, st);
        else if (bm == 32)
            run<32, false>(a, st);
        else if (bm == 64)
            run<64, false>(a, st);
        else
            run<128, false>(a, st);
    }
}

}  // namespace moe
