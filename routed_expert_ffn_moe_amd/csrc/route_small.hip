// Router and permutation for short passes (decode and verify shapes, at most
// 16 tokens and 256 (token, slot) pairs): two launches instead of seven.
//
//  router_small: logits of <= 16 tokens; each workgroup owns 16 experts and
//                its 8 (or 4) waves split K, then add their partial sums in
//                a fixed order (deterministic).
//  route_small:  one workgroup: top-k and weights of every token, then the
//                expert histogram, the prefix sums, the stable grouping of the
//                pairs, the tile lists and the work items, all in LDS.
//
// Pages: "DeepSeek V4.1F Q4 with native DSpark MTP" (decode paragraph: the
// time went to hundreds of small dispatches per token, and the router was
// cut from nine dispatches to one; verify rows are 6 at a time).
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

constexpr int RS_RING = 8;  // K steps in flight per wave

// RW waves split K in RW equal parts (RW * 32 dividing H); for H = 2048 and
// RW = 8 every wave's whole share is in flight at once.
template <int RW>
__global__ __launch_bounds__(64 * RW) void router_small(const uint16_t *__restrict__ x,
                                                        const uint16_t *__restrict__ wr,
                                                        const float *__restrict__ bias,
                                                        float *__restrict__ logits, int T, int H,
                                                        int E)
{
    __shared__ float red[RW][16][17];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int e0 = blockIdx.x * 16;
    const int kq = H / RW;  // K share of this wave (multiple of 32)
    const uint16_t *wp = wr + (int64_t)min(e0 + l16, E - 1) * H + wave * kq + lg * 8;
    const uint16_t *xp = x + (int64_t)min(l16, T - 1) * H + wave * kq + lg * 8;
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
        const int er = tid >> 4, t = tid & 15;  // 16 experts x 16 tokens
        const int e = e0 + er;
        if (t < T && e < E) {
            float v = red[0][er][t];
#pragma unroll
            for (int w = 1; w < RW; ++w)  // in wave order: a fixed sum
                v += red[w][er][t];
            logits[(int64_t)t * E + e] = v + (bias ? bias[e] : 0.0f);
        }
    }
}

template <int PER>
__global__ __launch_bounds__(1024) void route_small(
    const float *__restrict__ logits, int32_t *__restrict__ idx, float *__restrict__ w, int T,
    int E, int k, int shared, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ row_src, int32_t *__restrict__ row_tok, int32_t *__restrict__ row_of,
    Tile *__restrict__ tiles_a, int32_t *__restrict__ ntiles_a, Tile *__restrict__ tiles_b,
    int32_t *__restrict__ ntiles_b, int bm_a, int bm_b, int4 *__restrict__ items_a, int ntn_a,
    int wrows_a, int4 *__restrict__ items_b, int ntn_b, int wrows_b)
{
    __shared__ int s_idx[256];
    __shared__ int s_cnt[1025], s_off[1025], s_ta[1025], s_tb[1025];
    __shared__ int s_warp[16];
    __shared__ TopkLds s_topk[16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int P = T * k;
    const int G = E + (shared ? 1 : 0);

    // 1. top-k and weights, one wave per token
    for (int g = tid; g < G; g += 1024)
        s_cnt[g] = g < E ? 0 : T;
    for (int t = wv; t < T; t += 16)
        wave_topk<PER>(logits + (int64_t)t * E, E, k, idx + (int64_t)t * k, w + (int64_t)t * k,
                       s_idx + t * k, s_topk + wv);
    __syncthreads();

    // 2. pairs per group (integer counts: the order of the additions is immaterial)
    if (tid < P)
        atomicAdd(&s_cnt[s_idx[tid]], 1);
    __syncthreads();

    // 3. exclusive prefix sums of the rows and of the tiles of both lists, in
    // one scan of packed fields (rows < 2^11, tiles < 2^10: at most 272 rows)
    const int c = tid < G ? s_cnt[tid] : 0;
    const int va = tid < G ? (c + bm_a - 1) / bm_a : 0;
    const int vb = tid < G ? (c + bm_b - 1) / bm_b : 0;
    const int v = c | (va << 11) | (vb << 21);
    int iv = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(iv, off);
        if (lane >= off)
            iv += t;
    }
    if (lane == 63)
        s_warp[wv] = iv;
    __syncthreads();
    int pv = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q)  // all 16 reads in flight together
        pv += q < wv ? s_warp[q] : 0;
    const int ex = pv + iv - v;
    const int exc = ex & 0x7FF, exa = (ex >> 11) & 0x3FF, exb = (ex >> 21) & 0x3FF;
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
    __syncthreads();

    // 4. stable grouping: rank of pair p among earlier pairs of its expert
    if (tid < P) {
        const int e = s_idx[tid];
        int rank = 0;
        for (int q = 0; q < tid; ++q)
            rank += s_idx[q] == e;
        const int pos = s_off[e] + rank;
        row_src[pos] = tid;
        row_tok[pos] = tid / k;
        row_of[tid] = pos;
    }
    if (shared && tid < T) {
        row_src[P + tid] = P + tid;
        row_tok[P + tid] = tid;
    }

    // 5. tile lists and work items, one thread per group
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

bool route_small_ok(int T, int k, int E) { return T <= 16 && T * k <= 256 && E <= 1023; }

void launch_router_small(const RouterArgs &r, hipStream_t st)
{
    if (r.act == ACT_BF16 && r.E % 16 == 0 && r.H % 256 == 0)
        router_small<8><<<r.E / 16, 512, 0, st>>>((const uint16_t *)r.x, (const uint16_t *)r.wr,
                                                  r.bias, r.logits, r.T, r.H, r.E);
    else if (r.act == ACT_BF16 && r.E % 16 == 0 && r.H % 128 == 0)
        router_small<4><<<r.E / 16, 256, 0, st>>>((const uint16_t *)r.x, (const uint16_t *)r.wr,
                                                  r.bias, r.logits, r.T, r.H, r.E);
    else
        launch_router_logits(r, st);
}

template <int PER>
static void route_small_per(const RouterArgs &r, const PermuteArgs &a, hipStream_t st)
{
    route_small<PER><<<1, 1024, 0, st>>>(r.logits, r.idx, r.w, r.T, r.E, r.k, a.shared, a.counts,
                                         a.offsets, a.row_src, a.row_tok, a.row_of, a.tiles_a,
                                         a.ntiles_a, a.tiles_b, a.ntiles_b, a.bm_a, a.bm_b,
                                         a.items_a, a.ntn_a, a.wrows_a, a.items_b, a.ntn_b,
                                         a.wrows_b);
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
