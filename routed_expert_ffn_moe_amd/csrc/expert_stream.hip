// Weight-streaming grouped expert GEMM on bf16 MFMA (gfx950).
//
// Same contract as the tiled kernel in expert_gemm.hip (gate+up with the
// SwiGLU epilogue, or down into per-pair staging rows, unscaled: the combine
// applies the routing weights); built for the shapes of this layer, where every workload sits
// below the bf16 ridge point and the expert weights are the traffic that
// matters ("MoE prefill quantum", Table 9 and the text after it: small chunks
// read nearly every expert's weights for a few rows each).
//
//  * Each wave owns 32 weight rows per matrix (gate+up: two matrices) or 64
//    (down) and streams them from HBM straight into registers through a
//    prefetch ring of 4 or 8 steps of 32 K: no LDS and no barrier on the
//    weight path, every weight element read once per tile.  Wide tiles
//    (128 token rows, for passes with 128 or more rows per expert on
//    average) give each wave twice the weight rows, their accumulators all
//    256 AGPRs, and a ring of 2 steps (as many MFMA cycles as 4 narrow ones).  The weights are
//    in the packed layout (moe_pack_bf16): one K step of a 16-row block is a
//    contiguous kilobyte, so each load instruction of a wave fetches whole
//    cache lines (row-major rows would give 64 bytes of each of 16 lines).
//  * The tile's token rows (gathered through row_tok) are staged in LDS in
//    double-buffered 128- or 256-wide K chunks shared by the 4 waves.  The
//    128-row bf16 down tiles and both 128-row MXFP4 tiles run 8 waves
//    instead, two per SIMD, each with half
//    the weight rows (16 of the 32 of a 4-wave wave's pair of blocks, or 32
//    of 64): the same tile and the same MFMAs per output.
//  * The MFMA takes the weights as its A operand and the tokens as B; with
//    the weight rows of the two blocks of a 32-row group interleaved by fours,
//    a lane ends up with 8 adjacent output columns of one token row and
//    stores them as one 16-byte word (64 contiguous bytes per row and wave).
//  * Work items are ordered expert-major (then weight tile, then row tile)
//    and dealt out XCD by XCD in contiguous runs, so an expert's weight tiles
//    and token rows are fetched into one XCD's L2 and reused there.
//  * MXFP4 expert weights (W4, prefill chunks with more than 16 rows per
//    expert on average): the same items and tiles, the weights streamed in
//    the packed MXFP4 layout - one 16-byte load per lane and 16-row block
//    covers 128 K (a lane holds 32 consecutive K of its row), plus the
//    block's E8M0 scale byte - and turned into bf16 in registers with the
//    scaled fp4 -> bf16 conversion (exact: an E2M1 value times a power of
//    two has at most two significant bits).  The MFMA is the bf16 one with
//    the K order permuted alike in both operands: in sub-step s of a 128-K
//    chunk, lane group b holds K = 32b + 8s .. +7 of the weights and of the
//    tokens.  Weight bytes are 17/32 of a byte per weight, so a slice streams
//    in 0.27 of the bf16 time; the hi/lo MXFP8 split of the decode kernels
//    would run the same number of MFMA passes with no gain in precision.
//    Pages: "MoE prefill quantum", the section ruling out the hardware
//    (dequantising MXFP4 and applying the scale streams at read speed).
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <cstdlib>

namespace moe {

namespace {

// A staged token chunk is SKC (128 or 256) K elements wide; its LDS rows are
// padded by 8 elements, so the 16 rows a fragment read touches fall on
// distinct banks.
constexpr int sld_of(int skc) { return skc + 8; }
// Weight rows per work item and matrix: 4 waves x 32 (gate+up, two
// matrices) or 4 waves x 64 (down, one matrix); twice that in the wide
// tiles, whose 128-row accumulators take all 256 accumulation registers.
constexpr int wrows_of(bool gu, bool wide) { return (gu ? 128 : 256) * (wide ? 2 : 1); }

struct StreamP {
    const uint16_t *x;        // GU: activations [T, H]; DC: h [rows, ldh]
    const uint16_t *w0, *w1;  // routed matrices [E, N, K] (MXFP4: packed codes)
    const uint16_t *s0, *s1;  // shared expert matrices [N, K]
    const uint8_t *q0, *q1;   // MXFP4 only: packed E8M0 scales of w0, w1
    const int32_t *row_src, *offsets;
    const float *topk_w;
    uint16_t *out;            // GU: h; DC: stage
    const Tile *tiles;
    const int32_t *ntiles;
    const int4 *items;
    const int32_t *row_tok;
    int T, H, E, k, I, Is, ldh, ntn;
};

// A weight fragment.  With NT the load is non-temporal: small row tiles
// read each weight once, and keeping those lines out of the caches leaves
// room for the token rows (measured faster there, slower for large tiles
// whose weights are re-read by several row tiles).
template <bool NT>
__device__ __forceinline__ uint4 wload(const uint16_t *p)
{
    if (NT) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
        return uint4{v[0], v[1], v[2], v[3]};
    }
    return *(const uint4 *)p;
}

template <int N>
__device__ __forceinline__ void chunk_store(const u32v<N> &r, uint16_t *dst, const int (&off)[N],
                                            int part = 0, int nparts = 1)
{
#pragma unroll
    for (int i = 0; i < N; ++i)
        if (i % nparts == part)
            *(uint4 *)(dst + off[i]) = uint4{r[4 * i], r[4 * i + 1], r[4 * i + 2], r[4 * i + 3]};
}

// The next token chunk goes to LDS (the other buffer, free since the last
// barrier) during a chunk's MFMAs: the even pieces after the first K step,
// the odd ones after the third (the last, for shorter chunks), instead of
// all after the chunk, where the matrix cores waited for the LDS writes
// (T=2048 MXFP4 gate+up 185.6 -> 181.3 us, the bf16 layers -0.5%, the same
// results bit for bit).  Returns the part written after step st, or -1.
template <int SPC>
__device__ __forceinline__ int store_part(int st)
{
    static_assert(SPC >= 2, "both parts of the chunk are written");
    if (st == 0)
        return 0;
    return st == (SPC > 2 ? 2 : SPC - 1) ? 1 : -1;
}

// One work item: up to BM rows of one expert (group g) and a 128-row slice
// of its weight matrices starting at weight row n0.  Uniform across the
// workgroup; read as one 16-byte record.
struct Item {
    int g, row0, nrows, n0;
};

__device__ __forceinline__ Item item_at(const int4 *__restrict__ items, int wi)
{
    // A uniform index into read-only memory: a scalar load, waited for on
    // its own counter, so fetching records never drains the weight stream;
    // and every branch and select on the record stays uniform.
    const int4 r = items[__builtin_amdgcn_readfirstlane(wi)];
    return Item{__builtin_amdgcn_readfirstlane(r.x), __builtin_amdgcn_readfirstlane(r.y),
                __builtin_amdgcn_readfirstlane(r.z), __builtin_amdgcn_readfirstlane(r.w)};
}

// Element offsets (into x or h) of the token rows this thread stages.
template <int ACH, bool GU, int SKC, int NT>
__device__ __forceinline__ void item_rows(const StreamP &p, const Item &it, int tid, int (&aro)[ACH])
{
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        const int pos = it.row0 + min((tid + NT * i) / (SKC / 8), it.nrows - 1);
        aro[i] = GU ? p.row_tok[pos] * p.H : pos * p.ldh;
    }
}

template <int ACH>
__device__ __forceinline__ void rows_load(u32v<ACH> &r, const uint16_t *x, const int (&aro)[ACH],
                                          int off)
{
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        const uint4 t = *(const uint4 *)(x + aro[i] + off);
        r[4 * i] = t.x;
        r[4 * i + 1] = t.y;
        r[4 * i + 2] = t.z;
        r[4 * i + 3] = t.w;
    }
}

// Token fragments of K step s4 of the staged chunk: lane (l16, lg) holds
// token row mb*16 + l16, K = 32*s4 + 8*lg .. +7.
template <int NMB, int SLD>
__device__ __forceinline__ void frag_load(bf16x8 (&tf)[NMB], const uint16_t *As, int s4, int l16,
                                          int lg, bool full)
{
#pragma unroll
    for (int mb = 0; mb < NMB / 2; ++mb)
        tf[mb] = as_bf16x8(*(const uint4 *)(As + (mb * 16 + l16) * SLD + s4 * 32 + lg * 8));
    if (full || NMB < 2) {
#pragma unroll
        for (int mb = NMB / 2; mb < NMB; ++mb)
            tf[mb] = as_bf16x8(*(const uint4 *)(As + (mb * 16 + l16) * SLD + s4 * 32 + lg * 8));
    }
}

// The SKC/32 K steps of a staged token chunk.  Step s consumes the weight
// fragments of ring slot (slot0 + s) % SD and refills it from the step SD
// ahead (chunk wl[(s + SD) / SPC], step (s + SD) % SPC); the token fragments
// of step s + 1 are read from LDS while the MFMAs of step s run, so LDS
// latency hides behind them.
// With `full` false (uniform) only the first half of the MB token blocks is
// read and multiplied: the rest of the item's row tile is empty.
// One MFMA step into an accumulator: in place in the accumulation
// registers (AGPR) for the large row tiles, whose accumulators live there,
// else the compiler's own form.
template <bool AGPR>
__device__ __forceinline__ void mac(floatx4 &c, bf16x8 a, bf16x8 b)
{
    if (AGPR)
        mfma16_acc(c, a, b);
    else
        c = mfma16(a, b, c);
}

template <int MB, int NB, int CB, int SD, int SKC, bool AGPR, class Store>
__device__ __forceinline__ void kchunk(bool full, const uint16_t *As, int slot0, int l16, int lg,
                                       uint4 (&bq)[SD][NB][CB],
                                       const uint16_t *const (&wl)[3][NB],
                                       const int (&woff)[CB], floatx4 (&acc)[NB][CB][MB],
                                       const Store &store)
{
    constexpr int SPC = SKC / 32, SLD = sld_of(SKC);
    static_assert((SPC - 1 + SD) / SPC <= 2, "refills reach at most two chunks ahead");
    bf16x8 tf[2][MB];
    frag_load<MB, SLD>(tf[0], As, 0, l16, lg, full);
#pragma unroll
    for (int st = 0; st < SPC; ++st) {
        const int slot = (slot0 + st) % SD;
        bf16x8 wf[NB][CB];
        const uint16_t *const *w = wl[(st + SD) / SPC];
        const int wk = ((st + SD) % SPC) * 32;
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                wf[m][cb] = as_bf16x8(bq[slot][m][cb]);
                bq[slot][m][cb] = wload<(MB <= 2)>(w[m] + woff[cb] + wk * 32);
            }
        // The next step's token fragments are read after the MFMAs of this
        // step's second token block (before the MFMAs when the first half
        // holds fewer than two blocks).  Read before all of them, they were
        // waited for together with this step's own: the LDS wait counter
        // holds 15 operations and a step reads 8, so the compiler drained
        // both steps' reads before the first MFMA (T=2048 gate+up 172 ->
        // 170 us, the same results bit for bit).
        constexpr int AT = MB / 2 >= 2 ? 1 : MB / 2 - 1;
        if (AT < 0 && st + 1 < SPC)
            frag_load<MB, SLD>(tf[(st + 1) & 1], As, st + 1, l16, lg, full);
        // issue the refills here, not later: the waits for this step's
        // operands must not have to wait for them
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mb = 0; mb < MB / 2; ++mb) {
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
                    mac<AGPR>(acc[m][cb][mb], wf[m][cb], tf[st & 1][mb]);
            if (mb == AT && st + 1 < SPC)
                frag_load<MB, SLD>(tf[(st + 1) & 1], As, st + 1, l16, lg, full);
        }
        if (full || MB < 2) {
#pragma unroll
            for (int mb = MB / 2; mb < MB; ++mb)
#pragma unroll
                for (int m = 0; m < NB; ++m)
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
                        mac<AGPR>(acc[m][cb][mb], wf[m][cb], tf[st & 1][mb]);
        }
        if (store_part<SPC>(st) >= 0)
            store(store_part<SPC>(st));
    }
}

// The wide tiles' K steps (accumulators in AGPRs, NMB token blocks).  The
// MFMAs of a step go weight fragment by weight fragment, all token blocks of
// one fragment back to back, and a fragment's ring slot is refilled right
// after its last MFMA: the ring then needs no second copy of the fragments
// in use, for which the 256 accumulators of a wide tile leave no registers.
// A refill still lands SD steps ahead of its use.
template <int NMB, int MB, int NB, int CB, int SD, int SKC, class Store>
__device__ __forceinline__ void kchunk_wide(const uint16_t *As, int slot0, int l16, int lg,
                                            uint4 (&bq)[SD][NB][CB],
                                            const uint16_t *const (&wl)[3][NB],
                                            const int (&woff)[CB], floatx4 (&acc)[NB][CB][MB],
                                            const Store &store)
{
    constexpr int SPC = SKC / 32, SLD = sld_of(SKC);
    static_assert((SPC - 1 + SD) / SPC <= 2, "refills reach at most two chunks ahead");
    bf16x8 tf[2][NMB];
    frag_load<NMB, SLD>(tf[0], As, 0, l16, lg, true);
#pragma unroll
    for (int st = 0; st < SPC; ++st) {
        const int slot = (slot0 + st) % SD;
        const uint16_t *const *w = wl[(st + SD) / SPC];
        const int wk = ((st + SD) % SPC) * 32;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const bf16x8 wf = as_bf16x8(bq[slot][m][cb]);
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb)
                    mfma16_acc(acc[m][cb][mb], wf, tf[st & 1][mb]);
                bq[slot][m][cb] = wload<false>(w[m] + woff[cb] + wk * 32);
                // the next step's fragments once the first fragment's MFMAs
                // have taken all of this step's (see kchunk)
                if (m == 0 && cb == 0 && st + 1 < SPC)
                    frag_load<NMB, SLD>(tf[(st + 1) & 1], As, st + 1, l16, lg, true);
                __builtin_amdgcn_sched_barrier(0);
            }
        if (store_part<SPC>(st) >= 0)
            store(store_part<SPC>(st));
    }
}

// MXFP4 weights: 8 E2M1 codes (K = 8 consecutive elements, low nibble
// first) times 2^(scale - 127) as a bf16 MFMA operand; the conversion takes
// the E8M0 scale as the exponent field of an fp32.
__device__ __forceinline__ bf16x8 fp4x8_bf16(uint32_t codes, uint32_t scale)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const float sc = __uint_as_float(scale << 23);
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Token fragments of sub-step s of a 128-wide staged chunk in the MXFP4
// order: lane (l16, lg) holds token row mb*16 + l16, K = 32*lg + 8*s .. +7.
template <int NMB, int SLD>
__device__ __forceinline__ void frag_load_w4(bf16x8 (&tf)[NMB], const uint16_t *As, int s, int l16,
                                             int lg, bool full)
{
#pragma unroll
    for (int mb = 0; mb < NMB / 2; ++mb)
        tf[mb] = as_bf16x8(*(const uint4 *)(As + (mb * 16 + l16) * SLD + lg * 32 + s * 8));
    if (full || NMB < 2) {
#pragma unroll
        for (int mb = NMB / 2; mb < NMB; ++mb)
            tf[mb] = as_bf16x8(*(const uint4 *)(As + (mb * 16 + l16) * SLD + lg * 32 + s * 8));
    }
}

// One 128-wide K chunk with MXFP4 weights: ring slot `slot` holds this
// chunk's codes and scales of every block and is refilled from chunk d = SD
// ahead (codes at wl[m] + cb's block offset, scale bytes at sl[m]); the
// token fragments of sub-step s + 1 are read from LDS before the MFMAs of
// sub-step s.
template <int MB, int NB, int CB, int SD, bool AGPR, class Store>
__device__ __forceinline__ void kchunk_w4(bool full, const uint16_t *As, int slot, int l16, int lg,
                                          uint4 (&bq)[SD][NB][CB], uint32_t (&sq)[SD][NB][CB],
                                          const uint8_t *const (&wl)[NB],
                                          const uint8_t *const (&sl)[NB], const int (&woff)[CB],
                                          const int (&soff)[CB], floatx4 (&acc)[NB][CB][MB],
                                          const Store &store)
{
    constexpr int SLD = sld_of(128);
    uint4 wq[NB][CB];
    uint32_t ws[NB][CB];
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            wq[m][cb] = bq[slot][m][cb];
            ws[m][cb] = sq[slot][m][cb];
            bq[slot][m][cb] = wload<(MB <= 2)>((const uint16_t *)(wl[m] + woff[cb]));
            sq[slot][m][cb] = sl[m][soff[cb]];
        }
    bf16x8 tf[2][MB];
    frag_load_w4<MB, SLD>(tf[0], As, 0, l16, lg, full);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        // the next sub-step's fragments after the second token block's
        // MFMAs, as in kchunk
        constexpr int AT = MB / 2 >= 2 ? 1 : MB / 2 - 1;
        if (AT < 0 && st + 1 < 4)
            frag_load_w4<MB, SLD>(tf[(st + 1) & 1], As, st + 1, l16, lg, full);
        bf16x8 wf[NB][CB];
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const uint32_t c4[4] = {wq[m][cb].x, wq[m][cb].y, wq[m][cb].z, wq[m][cb].w};
                wf[m][cb] = fp4x8_bf16(c4[st], ws[m][cb]);
            }
#pragma unroll
        for (int mb = 0; mb < MB / 2; ++mb) {
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
                    mac<AGPR>(acc[m][cb][mb], wf[m][cb], tf[st & 1][mb]);
            if (mb == AT && st + 1 < 4)
                frag_load_w4<MB, SLD>(tf[(st + 1) & 1], As, st + 1, l16, lg, full);
        }
        if (full || MB < 2) {
#pragma unroll
            for (int mb = MB / 2; mb < MB; ++mb)
#pragma unroll
                for (int m = 0; m < NB; ++m)
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
                        mac<AGPR>(acc[m][cb][mb], wf[m][cb], tf[st & 1][mb]);
        }
        if (store_part<4>(st) >= 0)
            store(store_part<4>(st));
    }
}

// Persistent: the workgroup walks its run of work items; the weight prefetch
// ring and the token-chunk pipeline run on across item boundaries, so the
// next item's first weights and rows are in flight while the current one
// finishes.  Item records are fetched two items ahead and row tokens one item
// ahead, so no wait on them ever drains the weight stream.  All items of a
// launch share N and K (the shared expert, if any, has the routed width).
// Workgroups per CU the register budget is held to: more resident waves hide
// the LDS and L2 latency that one wave's own schedule cannot.
constexpr int wg_per_cu(int bm) { return bm <= 16 ? 3 : bm <= 64 ? 2 : 1; }

// NWV waves per workgroup: 4 (one per SIMD), or 8 for the 128-row narrow
// tiles (bf16 or MXFP4 weights) - two per SIMD, each with half the weight
// rows of the tile, so that one wave's matrix instructions issue beside the
// other's memory instructions; the tile, and every output's sum over K,
// stay the same.
template <int BM, bool GU, int SD, int SKC, bool W4, int TL, bool WIDE, int NWV>
__global__ __launch_bounds__(64 * NWV, NWV == 8 ? 1 : wg_per_cu(BM)) void expert_stream(
    StreamP p, const int4 *__restrict__ items)
{
    constexpr int NT = 64 * NWV;               // threads
    constexpr int SLD = sld_of(SKC), SPC = SKC / 32, RW = SKC / 8;  // 16-byte pieces per row
    constexpr int NB = GU ? 2 : 1;             // weight matrices
    // 16-row weight blocks per wave and matrix
    constexpr int CB = (GU ? 2 : 4) * (WIDE ? 2 : 1) * 4 / NWV;
    constexpr int MB = BM / 16;                // 16-row token blocks
    constexpr int ACH = BM * (SKC / 8) / NT;   // 16-byte token chunks per thread
    static_assert(W4 || SD == 4 || SD == 8 || (WIDE && SD == 2), "prefetch ring depth in K steps");
    static_assert(!WIDE || (BM == 128 && !W4), "wide tiles: 128 bf16 rows");
    static_assert(W4 || (2 * SPC) % SD == 0, "ring slots line up with chunk pairs");
    static_assert(!W4 || (SD == 2 && SKC == 128), "MXFP4: a ring of two 128-K chunks");
    static_assert(ACH >= 1 && ACH * NT == BM * SKC / 8, "token staging");
    static_assert(NWV == 4 || (NWV == 8 && BM == 128 && !WIDE), "eight waves: 128-row narrow tiles");
    static_assert((CB % 2 == 0 || NWV == 8) && NWV * CB * 16 == wrows_of(GU, WIDE),
                  "column blocks go in pairs (one block per wave with eight waves)");
    // the 128-row tiles' accumulators fill the accumulation registers
    constexpr bool AGPR = BM >= 128;

    __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * SLD];

    const int ntiles = *p.ntiles;
    const int total = ntiles * p.ntn;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, nslot = gridDim.x >> 3;
    const int per = (total + 7) >> 3;
    // The items of this workgroup: run position slot + j * nslot, j = 0, 1, ...
    const int base = xcd * per;
    const int lim = min(per, total - base);  // items in this XCD's run
    if (slot >= lim)
        return;
    const int nitems = (lim - slot + nslot - 1) / nslot;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int n_pairs = p.T * p.k;
    const int N = GU ? p.I : p.H;
    const int K = GU ? p.H : p.I;
    const int nchunks = K / SKC;  // even, >= 4
    const int64_t wstride = (int64_t)N * K;

    // Weight fragments of this lane in the packed layout: block cb of the
    // wave is block (cb & 1) of 32-row group wave * CB / 2 + cb / 2 of the
    // item's slice, whose MFMA row l16 is weight row 32 * group + 8 * (l16 / 4)
    // + 4 * (cb % 2) + l16 % 4; so after the MFMA the lane with lg = l16 / 4
    // holds 8 consecutive output columns per pair of blocks and stores them
    // as one 16-byte word.  One K step of a block is a contiguous kilobyte
    // (1024 elements per 32 K: offsets below scale K positions by 32).
    // MXFP4: block cb of the wave is 16-row block n0/16 + wave*CB + cb of
    // the expert (row 16 * block + l16), codes [blocks][Q][64 lanes][16 B]
    // and scales [blocks][64 lanes][Q], Q = K / 128 chunks.
    const int Q4 = K / 128;
    int woff[CB], soff[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        if (W4) {
            woff[cb] = (wave * CB + cb) * Q4 * 1024 + lane * 16;  // bytes
            soff[cb] = ((wave * CB + cb) * 64 + lane) * Q4;
        } else {
            const int gb = wave * CB + cb;  // 16-row block of the item's slice
            woff[cb] = ((gb >> 1) * (K / 32) * 2 + (gb & 1)) * 512 + lane * 8;
            soff[cb] = 0;
        }
    }
    auto wbase = [&](const Item &it, int m) -> const uint16_t * {
        if (W4)  // packed codes of the item's first block (bytes)
            return (const uint16_t *)((const uint8_t *)(m == 0 ? p.w0 : p.w1) +
                                      ((int64_t)it.g * (N / 16) + it.n0 / 16) * Q4 * 1024);
        const bool routed = it.g < p.E;
        const uint16_t *W = m == 0 ? (routed ? p.w0 + (int64_t)it.g * wstride : p.s0)
                                   : (routed ? p.w1 + (int64_t)it.g * wstride : p.s1);
        return W + (int64_t)it.n0 * K;
    };
    auto qbase = [&](const Item &it, int m) -> const uint8_t * {  // MXFP4 scales
        return (m == 0 ? p.q0 : p.q1) + ((int64_t)it.g * (N / 16) + it.n0 / 16) * 64 * Q4;
    };
    int aoff[ACH];
#pragma unroll
    for (int i = 0; i < ACH; ++i)
        aoff[i] = ((tid + NT * i) / RW) * SLD + (tid % RW) * 8;

    // Prologue: first item's weights for chunk 0, its token rows, chunk 0 in LDS.
    Item cur = item_at(items, base + slot);
    Item nxt = item_at(items, base + slot + min(1, nitems - 1) * nslot);
    const uint16_t *wc[NB];
#pragma unroll
    for (int m = 0; m < NB; ++m)
        wc[m] = wbase(cur, m);
    const uint8_t *qc[NB];
#pragma unroll
    for (int m = 0; m < NB; ++m)
        qc[m] = W4 ? qbase(cur, m) : nullptr;
    uint4 bq[SD][NB][CB];
    uint32_t sq[SD][NB][CB];
#pragma unroll
    for (int d = 0; d < SD; ++d)
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                if (W4) {  // chunk d (SD = 2 <= K / 128)
                    bq[d][m][cb] = wload<(MB <= 2)>(
                        (const uint16_t *)((const uint8_t *)wc[m] + woff[cb] + d * 1024));
                    sq[d][m][cb] = qc[m][soff[cb] + d];
                } else {
                    bq[d][m][cb] = wload<(MB <= 2)>(wc[m] + woff[cb] + d * 1024);  // SD <= 8 <= K/32
                    sq[d][m][cb] = 0;
                }
            }
    int aro[ACH], aro_n[ACH];
    item_rows<ACH, GU, SKC, NT>(p, cur, tid, aro);
    item_rows<ACH, GU, SKC, NT>(p, nxt, tid, aro_n);
    // Token chunks in flight: TL (1 or 2) ahead of the one in LDS.
    static_assert(TL == 1 || TL == 2, "token chunks in flight");
    u32v<ACH> rt[TL];
    rows_load<ACH>(rt[0], p.x, aro, (tid % RW) * 8);
    chunk_store<ACH>(rt[0], sA[0], aoff);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TL; ++t)
        rows_load<ACH>(rt[t], p.x, aro, (1 + t) * SKC + (tid % RW) * 8);  // 1 + TL <= nchunks
    int buf = 0;

    for (int j = 0; j < nitems; ++j) {
        // record of the item after next (clamped: re-read of the last one)
        const Item nn = item_at(items, base + slot + min(j + 2, nitems - 1) * nslot);
        // Next item's weights; the last item points them at itself, so the
        // prefetches that run past it stay in bounds and no branch is needed.
        const uint16_t *wn[NB];
        const uint8_t *qn[NB];
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            wn[m] = j + 1 < nitems ? wbase(nxt, m) : wc[m];
            qn[m] = W4 ? (j + 1 < nitems ? qbase(nxt, m) : qc[m]) : nullptr;
        }

        floatx4 acc[NB][CB][MB];
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[m][cb][mb] = floatx4{0, 0, 0, 0};

        const bool full = cur.nrows > BM / 2;  // uniform
        for (int c = 0; c < nchunks; c += 2) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int cc = c + h;
                const uint16_t *As = sA[buf];
                // Token chunk pipeline: rt[h % TL] holds the chunk after this
                // one; it goes to the other LDS buffer during this chunk's
                // MFMAs and is reloaded with the chunk TL + 1 ahead.
                u32v<ACH> &ra = rt[h % TL];
                uint16_t *const Bn = sA[buf ^ 1];
                const auto store = [&](int part) { chunk_store<ACH>(ra, Bn, aoff, part, 2); };
                if (W4) {
                    // the chunk SD = 2 ahead refills this one's ring slot
                    const int t = cc + 2;
                    const int over = t >= nchunks;
                    const int tq = t - over * nchunks;
                    const uint8_t *wl4[NB], *sl4[NB];
#pragma unroll
                    for (int m = 0; m < NB; ++m) {
                        wl4[m] = (const uint8_t *)(over ? wn[m] : wc[m]) + tq * 1024;
                        sl4[m] = (over ? qn[m] : qc[m]) + tq;
                    }
                    kchunk_w4<MB, NB, CB, SD, AGPR>(full, As, h, l16, lg, bq, sq, wl4, sl4, woff,
                                                    soff, acc, store);
                } else {
                    // Weight chunks d = 0, 1, 2 after this one, from this item
                    // or (past its end) from the next one; branch-free on purpose.
                    const uint16_t *wl[3][NB];
#pragma unroll
                    for (int d = 0; d < 3; ++d) {
                        const int t = cc + d;
                        const int over = t >= nchunks;
                        const int tk = (t - over * nchunks) * SKC * 32;  // packed: 32 per K
#pragma unroll
                        for (int m = 0; m < NB; ++m)
                            wl[d][m] = (over ? wn[m] : wc[m]) + tk;
                    }
                    // Items whose rows fit the first half of the row tile skip
                    // the MFMAs of the second half (the tile's other empty row
                    // blocks are computed: finer splits cost more than they save).
                    // (the wide tiles always run every MFMA: a second
                    // instantiation for half-filled tiles costs their
                    // accumulators a round of copies at each branch)
                    if (WIDE)
                        kchunk_wide<MB, MB, NB, CB, SD, SKC>(As, h * SPC, l16, lg, bq, wl, woff, acc,
                                                             store);
                    else
                        kchunk<MB, NB, CB, SD, SKC, AGPR>(full, As, h * SPC, l16, lg, bq, wl, woff,
                                                          acc, store);
                }
                __syncthreads();
                buf ^= 1;
                const int c2 = cc + 1 + TL;
                const int over = c2 >= nchunks;
                int rsel[ACH];
#pragma unroll
                for (int i = 0; i < ACH; ++i)
                    rsel[i] = over ? aro_n[i] : aro[i];
                rows_load<ACH>(ra, p.x, rsel, (c2 - over * nchunks) * SKC + (tid % RW) * 8);
                // keep these loads ahead of the next steps' weight loads, so
                // that waiting for them never waits for the weight stream
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        if (AGPR)
            mfma_acc_drain();
        // Epilogue: for block pair q the lane holds columns n + 32q .. +7 of
        // token row mb*16 + l16 (block 2q covers the first four); with MXFP4
        // weights block cb gives columns n4 + 16 cb .. +3.
        const int n = cur.n0 + wave * 16 * CB + lg * 8;
        const int n4 = cur.n0 + wave * 16 * CB + lg * 4;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int mr = mb * 16 + l16;
            if (mr >= cur.nrows)
                continue;
            const int pos = cur.row0 + mr;
            if (W4) {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const floatx4 g = acc[0][cb][mb], u = acc[NB - 1][cb][mb];
                    uint2 o;
                    if (GU) {
                        o.x = pack_bf2(silu(g[0]) * u[0], silu(g[1]) * u[1]);
                        o.y = pack_bf2(silu(g[2]) * u[2], silu(g[3]) * u[3]);
                    } else {
                        o.x = pack_bf2(g[0], g[1]);
                        o.y = pack_bf2(g[2], g[3]);
                    }
                    *(uint2 *)(p.out + (int64_t)pos * (GU ? p.ldh : p.H) + n4 + 16 * cb) = o;
                }
            } else if (GU && CB == 1) {
                // block wave & 1 of 32-row group wave / 2: 4 adjacent columns
                const int n1 = cur.n0 + 32 * (wave >> 1) + 8 * lg + 4 * (wave & 1);
                const floatx4 g = acc[0][0][mb], u = acc[NB - 1][0][mb];
                uint2 o;
                o.x = pack_bf2(silu(g[0]) * u[0], silu(g[1]) * u[1]);
                o.y = pack_bf2(silu(g[2]) * u[2], silu(g[3]) * u[3]);
                *(uint2 *)(p.out + (int64_t)pos * p.ldh + n1) = o;
            } else if (GU) {
#pragma unroll
                for (int q = 0; q < CB / 2; ++q) {
                    const floatx4 g0 = acc[0][2 * q][mb], u0 = acc[NB - 1][2 * q][mb];
                    const floatx4 g1 = acc[0][2 * q + 1][mb], u1 = acc[NB - 1][2 * q + 1][mb];
                    uint4 o;
                    o.x = pack_bf2(silu(g0[0]) * u0[0], silu(g0[1]) * u0[1]);
                    o.y = pack_bf2(silu(g0[2]) * u0[2], silu(g0[3]) * u0[3]);
                    o.z = pack_bf2(silu(g1[0]) * u1[0], silu(g1[1]) * u1[1]);
                    o.w = pack_bf2(silu(g1[2]) * u1[2], silu(g1[3]) * u1[3]);
                    *(uint4 *)(p.out + (int64_t)pos * p.ldh + n + 32 * q) = o;
                }
            } else {
#pragma unroll
                for (int q = 0; q < CB / 2; ++q) {
                    const floatx4 v0 = acc[0][2 * q][mb], v1 = acc[0][2 * q + 1][mb];
                    uint4 o;
                    o.x = pack_bf2(v0[0], v0[1]);
                    o.y = pack_bf2(v0[2], v0[3]);
                    o.z = pack_bf2(v1[0], v1[1]);
                    o.w = pack_bf2(v1[2], v1[3]);
                    *(uint4 *)(p.out + (int64_t)pos * p.H + n + 32 * q) = o;
                }
            }
        }
        cur = nxt;
        nxt = nn;
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            wc[m] = wn[m];
            qc[m] = qn[m];
        }
#pragma unroll
        for (int i = 0; i < ACH; ++i)
            aro[i] = aro_n[i];
        item_rows<ACH, GU, SKC, NT>(p, nxt, tid, aro_n);
    }
}

// CUs of the current device (read once per process).
int device_cus()
{
    static const int cus = [] {
        int dev = 0, n = 0;
        (void)hipGetDevice(&dev);
        (void)hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        return n > 0 ? n : 256;
    }();
    return cus;
}

template <int BM, bool GU, int SD, int SKC, bool W4, int TL, bool WIDE = false, int NWV = 4>
void run(const ExpertArgs &a, hipStream_t st)
{
    StreamP p;
    p.x = (const uint16_t *)(GU ? a.x : a.h);
    p.w0 = (const uint16_t *)(GU ? a.w_gate : a.w_down);
    p.w1 = (const uint16_t *)(GU ? a.w_up : nullptr);
    p.q0 = W4 ? (GU ? a.s_gate : a.s_down) : nullptr;
    p.q1 = W4 && GU ? a.s_up : nullptr;
    p.s0 = (const uint16_t *)(GU ? a.sh_gate : a.sh_down);
    p.s1 = (const uint16_t *)(GU ? a.sh_up : nullptr);
    p.row_src = a.row_src;
    p.offsets = a.offsets;
    p.topk_w = a.topk_w;
    p.out = (uint16_t *)(GU ? a.h : a.stage);
    p.tiles = GU ? a.tiles_gu : a.tiles_dc;
    p.ntiles = GU ? a.ntiles_gu : a.ntiles_dc;
    p.items = GU ? a.items_gu : a.items_dc;
    p.row_tok = a.row_tok;
    p.T = a.T;
    p.H = a.H;
    p.E = a.E;
    p.k = a.k;
    p.I = a.I;
    p.Is = a.I_shared;
    p.ldh = a.I > a.I_shared ? a.I : a.I_shared;
    const int N = GU ? p.ldh : a.H;
    p.ntn = (N + wrows_of(GU, WIDE) - 1) / wrows_of(GU, WIDE);
    const int64_t items = (int64_t)p.ntn * (GU ? a.max_tiles_gu : a.max_tiles_dc);
    if (items == 0)
        return;
    // Persistent grid: as many workgroups per XCD as fit at once, never more
    // than the items an XCD can receive.
    static int per_cu[2] = {0, 0};
    const int cus = device_cus();
    int &occ = per_cu[GU ? 1 : 0];
    if (!occ) {
        int b = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, expert_stream<BM, GU, SD, SKC, W4, TL, WIDE, NWV>, 64 * NWV,
                                                         0) != hipSuccess ||
            b < 1)
            b = 1;
        occ = b;
    }
    const int64_t per_xcd = (items + 7) / 8;
    const int64_t slots = std::min<int64_t>(per_xcd, (int64_t)(cus / 8) * occ);
    expert_stream<BM, GU, SD, SKC, W4, TL, WIDE, NWV><<<(unsigned)(slots * 8), 64 * NWV, 0, st>>>(p, p.items);
}

}  // namespace

// MXFP4 experts take the streaming kernels in prefill passes (more than 16
// rows per expert on average); decode and verify passes take the fp4-MFMA
// kernels of mxfp4.hip.
static bool stream_w4(const ExpertArgs &a)
{
    return a.wdt == W_MXFP4 && a.I_shared == 0 && (int64_t)a.shape_T * a.k > 16 * (int64_t)a.E;
}

bool stream_ok(const ExpertArgs &a, bool gu)
{
    if (a.act != ACT_BF16 || !(a.wdt == W_BF16 || stream_w4(a)))
        return false;
    // one width for every item of a launch: no shared expert, or one as wide
    // as the routed experts
    if (a.I_shared != 0 && a.I_shared != a.I)
        return false;
    // K in an even number of at least four 128-wide chunks
    if (gu)
        return a.H % 256 == 0 && a.H >= 512 && a.I % wrows_of(true, false) == 0;
    return a.I % 256 == 0 && a.I >= 512 && a.H % wrows_of(false, false) == 0;
}

// Wide tiles for the 128-row bf16 tiles when the experts hold 128 rows or
// more on average, the weight slices divide N and the pass still deals out
// at least 12 wide items per CU: per MFMA they read half the LDS bytes and
// stage half the token bytes of the narrow tiles, but they always run the
// whole tile's MFMAs and come in half as many items.  Measured (ms per
// layer, narrow -> wide): the 384-expert top-6 layer at T=8192 (128 rows per
// expert, ~26 items per CU) 4.96 -> 4.56; the 256-expert top-8 layer
// (I=768) at T=16384 1.65 -> 1.55 and T=32768 3.07 -> 2.83, at T=8192
// (~9 items per CU) 0.93 -> 0.95, at T=4096 (~6) 0.65 -> 0.68, at T=2048
// with Zipf bias (64 rows per expert) 0.36 -> 0.38.  The down projection
// (K = I) takes them only with at least 16 K chunks per item: against the
// eight-wave narrow down tiles, with I=768 (six chunks, where the wide
// item's store burst of 128 rows x 512 columns weighs more than its halved
// token bytes) narrow is faster - down us, narrow vs wide, T=8192 277 vs
// 325, T=16384 488 vs 526, T=32768 951 vs 994 - and with I=2048 wide still
// is (the 384-expert layer at T=8192: 1581 vs 1642).  MOE_STREAM_WIDE (0 or
// 1) overrides the rule for tuning runs and tests; it is read at each call,
// so a workspace sized under one setting may be refused under the other.
static bool stream_wide(const ExpertArgs &a, bool gu)
{
    const char *e = getenv("MOE_STREAM_WIDE");
    const int forced = e && (e[0] == '0' || e[0] == '1') ? e[0] - '0' : -1;
    if (forced == 0 || a.wdt != W_BF16 || stream_bm(a) != 128)
        return false;
    const int N = gu ? (a.I > a.I_shared ? a.I : a.I_shared) : a.H;
    if (N % wrows_of(gu, true) != 0)
        return false;
    if (forced == 1)
        return true;
    if (!gu && a.I < 16 * 128)
        return false;
    const int64_t pairs = (int64_t)a.shape_T * a.k;
    const int64_t tiles = pairs / 128 + a.E + (a.I_shared > 0 ? a.shape_T / 128 : 0);
    return pairs >= 128 * (int64_t)a.E &&
           tiles * (N / wrows_of(gu, true)) >= 12 * (int64_t)device_cus();
}

int stream_wrows(const ExpertArgs &a, bool gu) { return wrows_of(gu, stream_wide(a, gu)); }

int stream_ntn(const ExpertArgs &a, bool gu)
{
    if (!stream_ok(a, gu))
        return 0;
    const int N = gu ? (a.I > a.I_shared ? a.I : a.I_shared) : a.H;
    const int wr = wrows_of(gu, stream_wide(a, gu));
    return (N + wr - 1) / wr;
}

// Row-tile size by the mean rows per expert; MOE_STREAM_BM (16, 32, 64 or
// 128) overrides it (read at each call, so that one process can compare
// tile sizes; a workspace sized under one setting may be refused under
// another).
int stream_bm(const ExpertArgs &a)
{
    const char *e = getenv("MOE_STREAM_BM");
    const int forced = e ? atoi(e) : 0;
    if (forced == 16 || forced == 32 || forced == 64 || forced == 128)
        return forced;
    // Measured on the 256-expert top-8 layer (uniform routing, one chunk):
    // 16-row tiles up to 4 rows per expert on average, 32 up to 16 (T=512:
    // 436 vs 519 us with 16), 128 beyond (T=1024: 482 vs 615 us with 32 -
    // with 32-row tiles the experts a little above the mean read their
    // weights twice; 64-row tiles are slower at every T from 1024 to 8192,
    // 487-895 us against 493-1129).
    const int64_t avg = (int64_t)a.shape_T * a.k / a.E;
    if (avg <= 4)
        return 16;
    if (avg <= 16)
        return 32;
    // MXFP4 weights take a quarter of the bytes, so the two workgroups per
    // CU of the 64-row tiles (each wave reads 64 token rows from LDS instead
    // of the eight-wave 128-row tile's 128) win from 32 rows per expert on;
    // 32-row tiles below that.  Measured, us per layer with 32 / 64 / 128-row
    // tiles: T=600 159 / 171 / 216, T=1024 221 / 185 / 227, T=2048 332 / 264
    // / 296 (Zipf-routed 289 / 234 / 296), T=4096 - / 438 / 497, T=8192 - /
    // 756 / 795; the same results bit for bit.
    if (a.wdt == W_MXFP4)
        return avg <= 24 ? 32 : 64;
    return 128;
}

// Prefetch ring depth in K steps; MOE_STREAM_SD (4 or 8) overrides the
// default for tuning runs (read once per process).
static int stream_sd(int bm)
{
    static const int forced = [] {
        const char *e = getenv("MOE_STREAM_SD");
        const int v = e ? atoi(e) : 0;
        return (v == 4 || v == 8) ? v : 0;
    }();
    if (forced)
        return forced;
    (void)bm;
    return 4;  // deeper rings spill under the occupancy bounds (see wg_per_cu) or gain nothing
}

// Token chunk width: 256 K for the small row tiles where the chunks still
// come in pairs, else 128;
// MOE_STREAM_SKC (128 or 256) overrides it for tuning runs.
static int stream_skc(int K, int bm)
{
    static const int forced = [] {
        const char *e = getenv("MOE_STREAM_SKC");
        const int v = e ? atoi(e) : 0;
        return (v == 128 || v == 256) ? v : 0;
    }();
    if (forced == 128 || (forced == 256 && K % 512 == 0))
        return forced;
    // the wide chunk's staging registers only fit beside the small row tiles
    return K % 512 == 0 && bm <= 32 ? 256 : 128;
}

// Token chunks in flight for the MXFP4 kernels (their fp4 weight ring frees
// the registers of a second one); MOE_STREAM_TL (1 or 2) overrides it for
// tuning runs.
static int stream_tl_w4()
{
    static const int forced = [] {
        const char *e = getenv("MOE_STREAM_TL");
        const int v = e ? atoi(e) : 0;
        return (v == 1 || v == 2) ? v : 0;
    }();
    return forced ? forced : 2;
}

// Waves per workgroup of the 128-row narrow tiles.  bf16 weights: eight for
// the down projection (T=2048 layer: down 106.1 -> 103.5 us, the same results
// bit for bit), four for gate+up (unchanged at eight: 170.0 vs 169.4 us); a
// ring of eight K steps with eight waves spills.  MXFP4 weights: eight for
// both (T=2048 MXFP4 layer: gate+up 182 -> 166 us, down 109 -> 100 us, the
// same results bit for bit), where four waves hold all 256 registers at one
// wave per SIMD and eight hold 128 each at two.  MOE_STREAM_NWV (4 or 8)
// overrides all of them (read at each call, so that one process can compare
// the two).
static int stream_nwv(bool gu, bool w4)
{
    const char *e = getenv("MOE_STREAM_NWV");
    const int v = e ? atoi(e) : 0;
    if (v == 4 || v == 8)
        return v;
    return w4 || !gu ? 8 : 4;
}

template <int BM, bool GU, int SKC>
static void run_skc(const ExpertArgs &a, hipStream_t st)
{
    if constexpr (BM == 128 && SKC == 128) {
        if (stream_nwv(GU, false) == 8) {
            if (stream_sd(BM) == 4)
                run<BM, GU, 4, SKC, false, 1, false, 8>(a, st);
            else
                run<BM, GU, 8, SKC, false, 1, false, 8>(a, st);
            return;
        }
    }
    if (stream_sd(BM) == 8)
        run<BM, GU, 8, SKC, false, 1>(a, st);
    else
        run<BM, GU, 4, SKC, false, 1>(a, st);
}

template <int BM, bool GU>
static void run_sd(const ExpertArgs &a, hipStream_t st)
{
    if (BM == 128 && stream_wide(a, GU)) {  // a ring of two K steps: as many cycles as four narrow ones
        run<128, GU, 2, 128, false, 1, true>(a, st);
        return;
    }
    if (a.wdt == W_MXFP4) {  // a ring of two 128-K chunks of fp4 codes
        if (BM == 128 && stream_tl_w4() == 2 && stream_nwv(GU, true) == 8)
            run<128, GU, 2, 128, true, 2, false, 8>(a, st);
        else if (stream_tl_w4() == 1)
            run<BM, GU, 2, 128, true, 1>(a, st);
        else
            run<BM, GU, 2, 128, true, 2>(a, st);
    } else if (stream_skc(GU ? a.H : a.I, BM) == 256)
        run_skc<BM, GU, 256>(a, st);
    else
        run_skc<BM, GU, 128>(a, st);
}

template <bool GU>
static void run_bm(const ExpertArgs &a, hipStream_t st)
{
    const int bm = stream_bm(a);
    if (bm == 16)
        run_sd<16, GU>(a, st);
    else if (bm == 32)
        run_sd<32, GU>(a, st);
    else if (bm == 64)
        run_sd<64, GU>(a, st);
    else
        run_sd<128, GU>(a, st);
}

void launch_stream(const ExpertArgs &a, bool gu, hipStream_t st)
{
    if (gu)
        run_bm<true>(a, st);
    else
        run_bm<false>(a, st);
}

}  // namespace moe
