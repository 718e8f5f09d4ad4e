// Router and permutation for short passes (decode, verify and small chunks:
// at most 128 tokens and 1024 (token, slot) pairs): two launches instead of
// seven.
//
//  router_small: logits; a workgroup owns 16 experts x 16 tokens and its 8
//                waves split K in eight equal parts, then add their partial
//                sums in wave order (deterministic).  The long-pass router
//                GEMM keeps the same eight partial sums and adds them in the
//                same order, so both give the same bits.
//  route_small:  one workgroup per 4 tokens (16 if they are all) does their
//                top-k and weights;
//                the last workgroup to finish (a ticket counter that
//                router_small clears) then builds the expert histogram, the
//                prefix sums, the stable grouping of the pairs, the tile
//                lists and the work items, all in LDS.  With one workgroup
//                there is no ticket.
//
// Pages: "DeepSeek V4.1F Q4 with native DSpark MTP" (decode paragraph: the
// time went to hundreds of small dispatches per token, and the router was
// cut from nine dispatches to one; verify rows are 6 at a time).
#include "common.h"
#include "kernels.h"
#include "mxfp8.h"
#include "topk.h"

namespace moe {

constexpr int RS_RING = 8;  // K steps in flight per wave

// RW waves split K in RW equal parts (RW * 32 dividing H); for H = 2048 and
// RW = 8 every wave's whole share is in flight at once.  Grid: (E / 16,
// ceil(T / 16)).
// With xrec set (MXFP4 experts), the workgroups also quantise the token rows
// of their token block once for every expert kernel that reads them: row t
// as a record of mx_row_bytes(H) bytes at xrec + t * mx_row_bytes(H) (hi, lo,
// hi scales, lo scales: the LDS staging layout of one row), the 32-element
// blocks dealt over the workgroups of the token block; the loads go out with
// the router's own and the conversion follows its logits.
template <int RW>
__global__ __launch_bounds__(64 * RW) void router_small(const uint16_t *__restrict__ x,
                                                        const uint16_t *__restrict__ wr,
                                                        const float *__restrict__ bias,
                                                        float *__restrict__ logits,
                                                        int32_t *__restrict__ ticket,
                                                        uint8_t *__restrict__ xrec, int T, int H,
                                                        int E)
{
    __shared__ float red[RW][16][17];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 16;
    if (ticket && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0)
        *ticket = 0;  // the route kernel after this one counts on it
    // this thread's block of the token block's rows: (row qr, block qb)
    const int nblk = H / 32;
    const int qi = tid * gridDim.x + blockIdx.x;
    const int qr = qi / nblk, qb = qi - qr * nblk;
    const bool quant = xrec && qr < 16 && t0 + qr < T;
    uint4 raw[4];
    if (quant)
        block_load(raw, x + (int64_t)(t0 + qr) * H + qb * 32);
    const int kq = H / RW;  // K share of this wave (multiple of 32)
    const uint16_t *wp = wr + (int64_t)min(e0 + l16, E - 1) * H + wave * kq + lg * 8;
    const uint16_t *xp = x + (int64_t)min(t0 + l16, T - 1) * H + wave * kq + lg * 8;
    const int nst = kq / 32;
    uint4 wq[RS_RING], xq[RS_RING];
#pragma unroll
    for (int d = 0; d < RS_RING; ++d)
        if (d < nst) {
            wq[d] = *(const uint4 *)(wp + d * 32);
            xq[d] = *(const uint4 *)(xp + d * 32);
        }
    floatx4 acc = {0, 0, 0, 0};
    for (int s0 = 0; s0 < nst; s0 += RS_RING) {
#pragma unroll
        for (int d = 0; d < RS_RING; ++d) {
            const int s = s0 + d;
            if (s < nst) {
                const bf16x8 wf = as_bf16x8(wq[d]), xf = as_bf16x8(xq[d]);
                if (s + RS_RING < nst) {
                    wq[d] = *(const uint4 *)(wp + (s + RS_RING) * 32);
                    xq[d] = *(const uint4 *)(xp + (s + RS_RING) * 32);
                }
                acc = mfma16(wf, xf, acc);
            }
        }
    }
    // C[expert 4*lg + i][token l16]
#pragma unroll
    for (int i = 0; i < 4; ++i)
        red[wave][4 * lg + i][l16] = acc[i];
    __syncthreads();
    if (tid < 256) {
        const int er = tid >> 4, t = t0 + (tid & 15);  // 16 experts x 16 tokens
        const int e = e0 + er;
        if (t < T && e < E) {
            float v = red[0][er][tid & 15];
#pragma unroll
            for (int w = 1; w < RW; ++w)  // in wave order: a fixed sum
                v += red[w][er][tid & 15];
            logits[(int64_t)t * E + e] = v + (bias ? bias[e] : 0.0f);
        }
    }
    if (quant) {
        uint8_t *rec = xrec + (int64_t)(t0 + qr) * mx_row_bytes(H);
        const int ld = H + MX_PAD;
        block_quantise(raw, 0, qb, H, rec, rec + ld, rec + 2 * ld, rec + 2 * ld + nblk);
    }
}

// Short passes (T <= 64): router_small's eight K-segment waves as eight
// workgroups of one wave each, so that the router matrix is read by eight
// times as many CUs.  Segment `seg` (blockIdx.y) of expert block blockIdx.x
// and token block blockIdx.z writes its partial sums to part[t][e][seg] (a
// logit's eight
// parts in 32 contiguous bytes); the decode gate+up kernel adds the eight in
// segment order and then the bias, which is the sum router_small forms in
// LDS (so the logits have the same bits).
__global__ __launch_bounds__(64) void router_split(const uint16_t *__restrict__ x,
                                                   const uint16_t *__restrict__ wr,
                                                   float *__restrict__ part,
                                                   int32_t *__restrict__ ticket, int T, int H,
                                                   int E)
{
    const int lane = threadIdx.x, l16 = lane & 15, lg = lane >> 4;
    const int e0 = blockIdx.x * 16, seg = blockIdx.y, t = blockIdx.z * 16 + l16;
    if (ticket && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && lane == 0)
        *ticket = 0;  // the route kernel after this one counts on it
    const int kq = H / 8;  // K share of this segment (multiple of 32)
    const uint16_t *wp = wr + (int64_t)min(e0 + l16, E - 1) * H + seg * kq + lg * 8;
    const uint16_t *xp = x + (int64_t)min(t, T - 1) * H + seg * kq + lg * 8;
    const int nst = kq / 32;
    uint4 wq[RS_RING], xq[RS_RING];
#pragma unroll
    for (int d = 0; d < RS_RING; ++d)
        if (d < nst) {
            wq[d] = *(const uint4 *)(wp + d * 32);
            xq[d] = *(const uint4 *)(xp + d * 32);
        }
    floatx4 acc = {0, 0, 0, 0};
    for (int s0 = 0; s0 < nst; s0 += RS_RING) {
#pragma unroll
        for (int d = 0; d < RS_RING; ++d) {
            const int s = s0 + d;
            if (s < nst) {
                const bf16x8 wf = as_bf16x8(wq[d]), xf = as_bf16x8(xq[d]);
                if (s + RS_RING < nst) {
                    wq[d] = *(const uint4 *)(wp + (s + RS_RING) * 32);
                    xq[d] = *(const uint4 *)(xp + (s + RS_RING) * 32);
                }
                acc = mfma16(wf, xf, acc);
            }
        }
    }
    // C[expert 4*lg + i][token l16 of the block]
    if (t < T) {
        float *dst = part + ((int64_t)t * E + e0 + 4 * lg) * 8 + seg;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (e0 + 4 * lg + i < E)
                dst[8 * i] = acc[i];
    }
}

// Tokens whose top-k one route workgroup takes: 16 when it is the only one,
// else 4 (one wave per SIMD: the selection is a chain of wave reductions).
constexpr int route_tpw(int T) { return T <= 16 ? 16 : 4; }

template <int PER>
__global__ __launch_bounds__(1024) void route_small(
    const float *__restrict__ logits, const float *__restrict__ bias, int nparts,
    int32_t *__restrict__ idx, float *__restrict__ w, int T,
    int E, int k, int shared, int32_t *__restrict__ ticket, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ row_src, int32_t *__restrict__ row_tok,
    int32_t *__restrict__ row_of, Tile *__restrict__ tiles_a, int32_t *__restrict__ ntiles_a,
    Tile *__restrict__ tiles_b, int32_t *__restrict__ ntiles_b, int bm_a, int bm_b,
    int4 *__restrict__ items_a, int ntn_a, int wrows_a, int4 *__restrict__ items_b, int ntn_b,
    int wrows_b)
{
    __shared__ int s_idx[1024];
    __shared__ int s_cnt[1025], s_off[1025], s_ta[1025], s_tb[1025];
    // per wave and group: the wave's pairs of the group, then the pairs of
    // the group in the waves before it
    __shared__ uint16_t s_wc[16][1024];
    __shared__ int s_warp[2][16];
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int P = T * k;
    const int G = E + (shared ? 1 : 0);
    const bool one = gridDim.x == 1;

    // 1. top-k and weights of this workgroup's tokens, one wave per token
    const int tpw = route_tpw(T);
    const int t = blockIdx.x * tpw + wv;
    if (wv < tpw && t < T) {
        if (nparts == 8) {  // the split router's partial sums
            float v[PER];
            wave_logits_from_parts<PER>(logits, bias, t, E, v);
            wave_topk_vals<PER>(v, E, k, idx + (int64_t)t * k, w + (int64_t)t * k,
                                one ? s_idx + t * k : nullptr);
        } else {
            wave_topk<PER>(logits + (int64_t)t * E, E, k, idx + (int64_t)t * k,
                           w + (int64_t)t * k, one ? s_idx + t * k : nullptr);
        }
    }
    if (!one) {
        // The last workgroup through here does the rest.  The barrier orders
        // the workgroup's stores before thread 0's device-scope release, which
        // publishes them all before the ticket is taken.
        __syncthreads();
        if (tid == 0) {
            __threadfence();
            s_last = atomicAdd(ticket, 1) == (int)gridDim.x - 1;
            __threadfence();
        }
        __syncthreads();
        if (!s_last)
            return;
        if (tid < P)
            s_idx[tid] = __hip_atomic_load(idx + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int nwv = (P + 63) / 64;  // waves holding pairs
    if (tid < G)
        for (int q = 0; q < nwv; ++q)
            s_wc[q][tid] = 0;
    __syncthreads();

    // 2. rank of each pair among the earlier pairs of its wave with the same
    // expert: the lanes holding the same expert are found bit by bit of the
    // expert index (a ballot per bit); the last such lane records the wave's
    // count (one writer)
    const int e = tid < P ? s_idx[tid] : -1;
    int rank = 0;
    if (wv < nwv) {  // uniform
        uint64_t same = __ballot(e >= 0);
        for (int b = 0; (E - 1) >> b; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t ones = __ballot(bit);
            same &= bit ? ones : ~ones;
        }
        const uint64_t below = (1ull << lane) - 1;
        rank = __popcll(same & below);
        if (e >= 0 && (same >> lane) == 1ull)  // no later lane of the expert
            s_wc[wv][e] = (uint16_t)(rank + 1);
    }
    __syncthreads();

    // 3. pairs per group and, per wave, the group's pairs in earlier waves;
    // 4. exclusive prefix sums of the rows and of the tiles of both lists
    // (two packed scans: rows and tiles a in 16-bit fields, tiles b).  Only
    // the waves holding groups take part.
    const int ngw = (G + 63) / 64;
    int c = 0, va = 0, vb = 0, i1 = 0, i2 = 0;
    if (wv < ngw) {  // uniform
        if (tid < E) {
            int n[16];
#pragma unroll
            for (int q = 0; q < 16; ++q)  // all reads in flight together
                n[q] = q < nwv ? s_wc[q][tid] : 0;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                if (q < nwv)
                    s_wc[q][tid] = (uint16_t)c;
                c += n[q];
            }
        } else if (tid < G) {
            c = T;  // the shared expert: every token
        }
        if (tid < G) {
            s_cnt[tid] = c;
            va = (c + bm_a - 1) / bm_a;
            vb = (c + bm_b - 1) / bm_b;
        }
        i1 = wave_scan_add(c | (va << 16));
        i2 = wave_scan_add(vb);
        if (lane == 63) {
            s_warp[0][wv] = i1;
            s_warp[1][wv] = i2;
        }
    }
    __syncthreads();
    if (wv < ngw) {
        int p1 = 0, p2 = 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) {  // all reads in flight together
            const bool in = q < wv;
            p1 += in ? s_warp[0][q] : 0;
            p2 += in ? s_warp[1][q] : 0;
        }
        const int ex1 = p1 + i1 - (c | (va << 16)), exb = p2 + i2 - vb;
        const int exc = ex1 & 0xFFFF, exa = ex1 >> 16;
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
            offsets[E + 1] = P;
    }
    __syncthreads();

    // 5. grouped position of each pair: stable (t, j) order within its expert
    if (e >= 0) {
        const int pos = s_off[e] + s_wc[wv][e] + rank;
        row_src[pos] = tid;
        row_tok[pos] = tid / k;
        row_of[tid] = pos;
    }
    if (shared && tid < T) {
        row_src[P + tid] = P + tid;
        row_tok[P + tid] = tid;
    }

    // 6. tile lists and work items, one thread per group
    for (int g = tid; g < G; g += 1024) {
        const int cg = s_cnt[g], og = s_off[g];
        if (cg == 0)
            continue;
        const int na = (cg + bm_a - 1) / bm_a, nb = (cg + bm_b - 1) / bm_b;
        for (int m = 0; m < na; ++m) {
            tiles_a[s_ta[g] + m] = Tile{g, og + m * bm_a};
            if (items_a)
                for (int nt = 0; nt < ntn_a; ++nt)
                    items_a[ntn_a * s_ta[g] + nt * na + m] =
                        int4{g, og + m * bm_a, min(bm_a, cg - m * bm_a), nt * wrows_a};
        }
        for (int m = 0; m < nb; ++m) {
            tiles_b[s_tb[g] + m] = Tile{g, og + m * bm_b};
            if (items_b)
                for (int nt = 0; nt < ntn_b; ++nt)
                    items_b[ntn_b * s_tb[g] + nt * nb + m] =
                        int4{g, og + m * bm_b, min(bm_b, cg - m * bm_b), nt * wrows_b};
        }
    }
}

bool route_small_ok(int T, int k, int E, int H, int act)
{
    if (T > 128 || T * k > 1024 || k > 16 || E > 1023)
        return false;
    // more than one route workgroup needs the ticket that router_small clears
    return T <= 16 || router_small_rw(E, H, act) > 0;
}

bool router_xq_ok(int E, int H, int act)
{
    return router_small_rw(E, H, act) > 0 && H % 512 == 0;
}

size_t router_xq_bytes(int T, int H) { return (size_t)T * mx_row_bytes(H); }

int router_small_rw(int E, int H, int act)
{
    if (act != ACT_BF16 || E % 16 != 0)
        return 0;
    return H % 256 == 0 ? 8 : H % 128 == 0 ? 4 : 0;
}

bool router_split_ok(int T, int E, int H, int act)
{
    return T >= 1 && T <= 64 && router_small_rw(E, H, act) == 8;
}

void launch_router_split(const RouterArgs &r, hipStream_t st)
{
    router_split<<<dim3(r.E / 16, 8, (r.T + 15) / 16), 64, 0, st>>>(
        (const uint16_t *)r.x, (const uint16_t *)r.wr, r.logits, r.ticket, r.T, r.H, r.E);
}

void launch_router_small(const RouterArgs &r, hipStream_t st)
{
    const dim3 grid(r.E / 16, (r.T + 15) / 16);
    switch (router_small_rw(r.E, r.H, r.act)) {
    case 8:
        router_small<8><<<grid, 512, 0, st>>>((const uint16_t *)r.x, (const uint16_t *)r.wr, r.bias,
                                              r.logits, r.ticket, r.xq, r.T, r.H, r.E);
        break;
    case 4:
        router_small<4><<<grid, 256, 0, st>>>((const uint16_t *)r.x, (const uint16_t *)r.wr, r.bias,
                                              r.logits, r.ticket, r.xq, r.T, r.H, r.E);
        break;
    default:
        launch_router_logits(r, st);  // one route workgroup only: no ticket
        break;
    }
}

template <int PER>
static void route_small_per(const RouterArgs &r, const PermuteArgs &a, hipStream_t st)
{
    const int tpw = route_tpw(r.T);
    route_small<PER><<<(r.T + tpw - 1) / tpw, 1024, 0, st>>>(
        r.logits, r.bias, r.nparts, r.idx, r.w, r.T, r.E, r.k, a.shared, r.ticket, a.counts,
        a.offsets, a.row_src,
        a.row_tok, a.row_of, a.tiles_a, a.ntiles_a, a.tiles_b, a.ntiles_b, a.bm_a, a.bm_b,
        a.items_a, a.ntn_a, a.wrows_a, a.items_b, a.ntn_b, a.wrows_b);
}

void launch_route_small(const RouterArgs &r, const PermuteArgs &a, hipStream_t st)
{
    switch (topk_per(r.E)) {
    case 1: route_small_per<1>(r, a, st); break;
    case 2: route_small_per<2>(r, a, st); break;
    case 4: route_small_per<4>(r, a, st); break;
    case 8: route_small_per<8>(r, a, st); break;
    default: route_small_per<16>(r, a, st); break;
    }
}

}  // namespace moe
