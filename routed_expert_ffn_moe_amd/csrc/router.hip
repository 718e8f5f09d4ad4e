// Router: logits = x . router_w^T (+ bias) in fp32, then top-k and the
// renormalised softmax weights of the selected experts.
//
// Pages: "MoE prefill quantum" (cause section: k of E experts per token) and
// "DeepSeek V4.1F Q4 with native DSpark MTP" (decode paragraph: the router
// is one fused dispatch instead of nine).  Logits are accumulated in fp32 and
// never rounded to bf16; selection is on the logits, ties to the lower index.
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

// bf16 logits on MFMA 16x16x32.  One wave owns 16 experts x 32 tokens (two
// 16-row MFMA blocks sharing the expert operand); WN waves per workgroup
// cover 16*WN experts.  Each lane loads 16 consecutive bf16 (32 bytes) of its
// row per 64-wide K step and feeds them to two MFMAs; A and B use the same
// lane -> k assignment, so the product is the plain dot product.
template <int WN>
__global__ __launch_bounds__(64 * WN) void router_logits_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
    const float *__restrict__ bias, float *__restrict__ logits, int T, int H, int E)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int e0 = (blockIdx.x * WN + wave) * 16;
    const int t0 = blockIdx.y * 32;
    if (e0 >= E)
        return;
    const int r = lane & 15;
    const int kq = (lane >> 4) * 16;
    const int te0 = min(t0 + r, T - 1);
    const int te1 = min(t0 + 16 + r, T - 1);
    const int ee = min(e0 + r, E - 1);
    const uint16_t *pa0 = x + (int64_t)te0 * H + kq;
    const uint16_t *pa1 = x + (int64_t)te1 * H + kq;
    const uint16_t *pb = wr + (int64_t)ee * H + kq;
    floatx4 c0 = {0, 0, 0, 0}, c1 = {0, 0, 0, 0};
    for (int k0 = 0; k0 < H; k0 += 64) {
        uint4 a0a = *(const uint4 *)(pa0 + k0), a0b = *(const uint4 *)(pa0 + k0 + 8);
        uint4 a1a = *(const uint4 *)(pa1 + k0), a1b = *(const uint4 *)(pa1 + k0 + 8);
        uint4 ba = *(const uint4 *)(pb + k0), bb = *(const uint4 *)(pb + k0 + 8);
        c0 = mfma16(as_bf16x8(a0a), as_bf16x8(ba), c0);
        c0 = mfma16(as_bf16x8(a0b), as_bf16x8(bb), c0);
        c1 = mfma16(as_bf16x8(a1a), as_bf16x8(ba), c1);
        c1 = mfma16(as_bf16x8(a1b), as_bf16x8(bb), c1);
    }
    const int e = e0 + r;
    if (e >= E)
        return;
    const float b = bias ? bias[e] : 0.0f;
    for (int i = 0; i < 4; ++i) {
        int t = t0 + (lane >> 4) * 4 + i;
        if (t < T)
            logits[(int64_t)t * E + e] = c0[i] + b;
        t += 16;
        if (t < T)
            logits[(int64_t)t * E + e] = c1[i] + b;
    }
}

// bf16 logits for T > 16: a workgroup owns RT tokens x 64 experts.  The
// token rows are staged in LDS in double-buffered 128-wide K chunks, with
// RTL more chunks in flight in registers; each wave streams its 16 expert
// rows from global memory through a 16-step register ring (no barrier on
// that path).  The GEMM does two MFMAs per 1 KB of weights a wave loads, so
// it runs at the pace its loads arrive: the chunk queue and the ring keep
// about 100 KB per workgroup in flight.  The MFMA takes the expert rows as
// its A operand, so a lane ends up with 4 consecutive experts of one token
// and stores them as one 16-byte word.  Every logit is the same sum whatever
// RT and the grid are: eight sequential chains over consecutive eighths of
// K in 32-wide MFMA steps, added in K order.
constexpr int RKC = 128;        // K chunk staged in LDS
constexpr int RLD = RKC + 8;    // padded LDS row (bf16)
constexpr int RTL = 4;          // token chunks in flight in registers
constexpr int RSD = 4 * RTL;    // weight prefetch ring (K steps): RTL chunks

template <int RT>
__global__ __launch_bounds__(256, 1) void router_gemm(const uint16_t *__restrict__ x,
                                                      const uint16_t *__restrict__ wr,
                                                      const float *__restrict__ bias,
                                                      float *__restrict__ logits, int T, int H, int E)
{
    constexpr int MB = RT / 16;              // token blocks
    constexpr int XCH = RT * (RKC / 8) / 256; // 16-byte token chunks per thread
    static_assert(XCH >= 1, "token staging");
    __shared__ __attribute__((aligned(16))) uint16_t sX[2][RT * RLD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    // Workgroups are dealt to the 8 XCDs in turn; the grid's tiles are
    // renumbered so that each XCD takes a contiguous run of them, token block
    // by token block: the expert blocks that share a token block read its
    // rows from one L2.
    const int nbx = E / 64, n = gridDim.x;
    const int b = blockIdx.x;
    const int L = (n & 7) ? b : (b & 7) * (n >> 3) + (b >> 3);
    const int t0 = (L / nbx) * RT, e0 = (L % nbx) * 64 + wave * 16;
    // expert row of this lane: MFMA row l16 -> expert e0 + l16
    const uint16_t *wp = wr + (int64_t)min(e0 + l16, E - 1) * H + lg * 8;
    int xo[XCH], so[XCH];
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
        const int q = tid + 256 * i, r = q >> 4, c8 = q & 15;
        xo[i] = min(t0 + r, T - 1) * H + c8 * 8;
        so[i] = r * RLD + c8 * 8;
    }
    const int nsteps = H / 32, nchunks = H / RKC;  // nchunks a multiple of RTL
    uint4 bq[RSD];
#pragma unroll
    for (int d = 0; d < RSD; ++d)
        bq[d] = *(const uint4 *)(wp + min(d, nsteps - 1) * 32);
    // chunk q waits in slot q % RTL (one vector value: no scratch)
    u32v<RTL * XCH> ra;
#pragma unroll
    for (int i = 0; i < XCH; ++i)
        *(uint4 *)(&sX[0][so[i]]) = *(const uint4 *)(x + xo[i]);
#pragma unroll
    for (int q = 1; q <= RTL; ++q)
#pragma unroll
        for (int i = 0; i < XCH; ++i)
            vset<RTL * XCH>(ra, (q % RTL) * XCH + i,
                            *(const uint4 *)(x + xo[i] + min(q, nchunks - 1) * RKC));
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    floatx4 acc[MB], tot[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        acc[mb] = tot[mb] = floatx4{0, 0, 0, 0};
    // K in eight equal segments (H % 256 == 0): each segment's chain of
    // MFMAs starts from zero and the segment sums are added in K order, the
    // same arithmetic as the short-pass router's eight waves.
    const int sps = nsteps / 8;
    int left = sps;
    bool first = true;
    int buf = 0;
    for (int c = 0; c < nchunks; c += RTL) {
#pragma unroll
        for (int h = 0; h < RTL; ++h) {
            const int cc = c + h;
            const uint16_t *Xs = sX[buf];
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const int step = cc * 4 + s4;
                const bf16x8 wf = as_bf16x8(bq[h * 4 + s4]);
                bq[h * 4 + s4] = *(const uint4 *)(wp + min(step + RSD, nsteps - 1) * 32);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const bf16x8 tf =
                        as_bf16x8(*(const uint4 *)(Xs + (mb * 16 + l16) * RLD + s4 * 32 + lg * 8));
                    acc[mb] = mfma16(wf, tf, acc[mb]);
                }
                if (--left == 0) {  // end of a K segment (uniform)
                    left = sps;
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        tot[mb] = first ? acc[mb] : tot[mb] + acc[mb];
                        acc[mb] = floatx4{0, 0, 0, 0};
                    }
                    first = false;
                }
            }
            // chunk cc + 1 into the other buffer, then its slot takes chunk
            // cc + 1 + RTL
            const int sl = (h + 1) % RTL;  // a constant once h is unrolled
#pragma unroll
            for (int i = 0; i < XCH; ++i)
                *(uint4 *)(&sX[buf ^ 1][so[i]]) = vget<RTL * XCH>(ra, sl * XCH + i);
            __syncthreads();
            buf ^= 1;
#pragma unroll
            for (int i = 0; i < XCH; ++i)
                vset<RTL * XCH>(ra, sl * XCH + i,
                                *(const uint4 *)(x + xo[i] + min(cc + 1 + RTL, nchunks - 1) * RKC));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // lane: experts e0 + 4*lg .. +3 of token mb*16 + l16
    const int e = e0 + 4 * lg;
    if (e >= E)
        return;
    const float4 bv = bias ? float4{bias[e], bias[e + 1], bias[e + 2], bias[e + 3]}
                           : float4{0, 0, 0, 0};
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int t = t0 + mb * 16 + l16;
        if (t < T)
            *(float4 *)(logits + (int64_t)t * E + e) =
                float4{tot[mb][0] + bv.x, tot[mb][1] + bv.y, tot[mb][2] + bv.z, tot[mb][3] + bv.w};
    }
}

// bf16 logits of long passes with K in eight segments across workgroups
// (H % 2048 == 0, E % 128 == 0): a workgroup owns RT tokens x 128 experts x
// one eighth of K and writes that segment's partial sums to part[seg][t][e];
// the top-k kernel adds the eight in K order and then the bias, the same
// arithmetic as router_gemm and the short-pass router.  Splitting K gives
// the grid enough workgroups with tiles four times the area of router_gemm's,
// so far fewer bytes cross from L2 into the CUs.  Per 256-wide pass of the
// segment, the token rows go to LDS and each wave's 32 expert rows straight
// into registers, all loads issued before the first MFMA.
constexpr int SEG_PK = 256;           // K per pass
constexpr int SEG_LD = SEG_PK + 8;    // padded LDS token row (bf16)

template <int RT>
__global__ __launch_bounds__(256, 2) void router_seg(const uint16_t *__restrict__ x,
                                                     const uint16_t *__restrict__ wr,
                                                     float *__restrict__ part, int T, int H, int E,
                                                     int32_t *__restrict__ hist, int nhist)
{
    constexpr int MB = RT / 16;                       // token blocks
    constexpr int XCH = RT * (SEG_PK / 8) / 256;      // 16-byte token pieces per thread
    constexpr int NS = SEG_PK / 32;                   // MFMA steps per pass
    __shared__ __attribute__((aligned(16))) uint16_t sX[RT * SEG_LD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    // the block histogram the top-k kernel after this one counts into
    for (int i = blockIdx.x * 256 + tid; i < nhist; i += gridDim.x * 256)
        hist[i] = 0;
    // Tiles numbered token block, then segment, then expert block, and dealt
    // to the XCDs in contiguous runs: the expert blocks of one token block and
    // segment read its rows from one L2.
    const int nbe = E / 128, n = gridDim.x, b = blockIdx.x;
    const int L = (n & 7) ? b : (b & 7) * (n >> 3) + (b >> 3);
    const int eb = L % nbe, seg = (L / nbe) & 7, tb = L / (nbe * 8);
    const int t0 = tb * RT, e0 = eb * 128 + wave * 32;
    const int ks = H / 8;
    const uint16_t *wp0 = wr + (int64_t)(e0 + l16) * H + seg * ks + lg * 8;
    const uint16_t *wp1 = wp0 + (int64_t)16 * H;
    int xo[XCH], so[XCH];
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
        const int q = tid + 256 * i, r = q / (SEG_PK / 8), c8 = q % (SEG_PK / 8);
        xo[i] = min(t0 + r, T - 1) * H + seg * ks + c8 * 8;
        so[i] = r * SEG_LD + c8 * 8;
    }
    floatx4 acc[2][MB];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            acc[m][mb] = floatx4{0, 0, 0, 0};
    for (int k0 = 0; k0 < ks; k0 += SEG_PK) {
        // held as vector values (registers, never scratch)
        u32v<NS> wq0, wq1;
        u32v<XCH> xq;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            vset<NS>(wq0, s, *(const uint4 *)(wp0 + k0 + s * 32));
            vset<NS>(wq1, s, *(const uint4 *)(wp1 + k0 + s * 32));
        }
#pragma unroll
        for (int i = 0; i < XCH; ++i)
            vset<XCH>(xq, i, *(const uint4 *)(x + xo[i] + k0));
        if (k0 > 0)
            __syncthreads();  // the previous pass's fragments are read
#pragma unroll
        for (int i = 0; i < XCH; ++i)
            *(uint4 *)(&sX[so[i]]) = vget<XCH>(xq, i);
        __syncthreads();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const bf16x8 w0 = as_bf16x8(vget<NS>(wq0, s)), w1 = as_bf16x8(vget<NS>(wq1, s));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const bf16x8 tf =
                    as_bf16x8(*(const uint4 *)(sX + (mb * 16 + l16) * SEG_LD + s * 32 + lg * 8));
                acc[0][mb] = mfma16(w0, tf, acc[0][mb]);
                acc[1][mb] = mfma16(w1, tf, acc[1][mb]);
            }
        }
    }
    // lane: experts e0 + 16m + 4*lg .. +3 of token mb*16 + l16
    float *dst = part + (int64_t)seg * T * E;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int t = t0 + mb * 16 + l16;
        if (t < T)
#pragma unroll
            for (int m = 0; m < 2; ++m)
                *(float4 *)(dst + (int64_t)t * E + e0 + 16 * m + 4 * lg) =
                    float4{acc[m][mb][0], acc[m][mb][1], acc[m][mb][2], acc[m][mb][3]};
    }
}

// fp32 logits: one thread per (token, expert), plain dot product.
__global__ __launch_bounds__(256) void router_logits_f32(
    const float *__restrict__ x, const float *__restrict__ wr,
    const float *__restrict__ bias, float *__restrict__ logits, int T, int H, int E)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * E)
        return;
    const int t = (int)(i / E), e = (int)(i % E);
    const float *a = x + (int64_t)t * H;
    const float *b = wr + (int64_t)e * H;
    float acc = 0.0f;
    for (int h = 0; h < H; ++h)
        acc = fmaf(a[h], b[h], acc);
    logits[i] = acc + (bias ? bias[e] : 0.0f);
}

// Top-k and weights: one wave per token (see wave_topk).
template <int PER>
__global__ __launch_bounds__(256) void router_topk(
    const float *__restrict__ logits, int32_t *__restrict__ idx, float *__restrict__ w,
    int T, int E, int k)
{
    const int wv = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wv;
    if (t >= T)
        return;
    wave_topk<PER>(logits + (int64_t)t * E, E, k, idx + (int64_t)t * k, w + (int64_t)t * k,
                   nullptr);
}

// The same from router_seg's eight partial sums: the logit is the sum of the
// eight in K order, then the bias.  With hist given, each selected pair also
// counts into its permutation block's row of the histogram (integer counts:
// the order of the atomic additions is immaterial).
template <int PER>
__global__ __launch_bounds__(256) void router_topk_seg(
    const float *__restrict__ part, const float *__restrict__ bias, int32_t *__restrict__ idx,
    float *__restrict__ w, int T, int E, int k, int32_t *__restrict__ hist)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wv;
    if (t >= T)
        return;
    const int64_t plane = (int64_t)T * E;
    float p[8][PER];  // all loads in flight together
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = lane + 64 * i;
            p[s][i] = e < E ? part[s * plane + (int64_t)t * E + e] : 0.0f;
        }
    float v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        float a = p[0][i];
#pragma unroll
        for (int s = 1; s < 8; ++s)
            a += p[s][i];
        v[i] = a + (bias && e < E ? bias[e] : 0.0f);
    }
    wave_topk_vals<PER>(v, E, k, idx + (int64_t)t * k, w + (int64_t)t * k, nullptr);
    if (hist && lane < k) {
        const int p = t * k + lane;  // this lane's pair, just written by this lane
        atomicAdd(&hist[(p / PERMUTE_PAIRS_PER_BLOCK) * E + idx[p]], 1);
    }
}

void launch_router_logits(const RouterArgs &a, hipStream_t st)
{
    if (a.T == 0)
        return;
    if (a.act == ACT_BF16 && a.T > 16 && a.E % 64 == 0 && a.H % (RKC * RTL) == 0) {
        // 64 tokens per workgroup for long chunks, 32 otherwise (more workgroups)
        if (a.T >= 4096) {
            const unsigned grid = (unsigned)(a.E / 64 * ((a.T + 63) / 64));
            router_gemm<64><<<grid, 256, 0, st>>>((const uint16_t *)a.x, (const uint16_t *)a.wr,
                                                 a.bias, a.logits, a.T, a.H, a.E);
        } else {
            const unsigned grid = (unsigned)(a.E / 64 * ((a.T + 31) / 32));
            router_gemm<32><<<grid, 256, 0, st>>>((const uint16_t *)a.x, (const uint16_t *)a.wr,
                                                 a.bias, a.logits, a.T, a.H, a.E);
        }
    } else if (a.act == ACT_BF16) {
        if (a.T <= 64) {
            dim3 grid((a.E + 15) / 16, (a.T + 31) / 32);
            router_logits_bf16<1><<<grid, 64, 0, st>>>((const uint16_t *)a.x, (const uint16_t *)a.wr,
                                                      a.bias, a.logits, a.T, a.H, a.E);
        } else {
            dim3 grid((a.E + 63) / 64, (a.T + 31) / 32);
            router_logits_bf16<4><<<grid, 256, 0, st>>>((const uint16_t *)a.x, (const uint16_t *)a.wr,
                                                       a.bias, a.logits, a.T, a.H, a.E);
        }
    } else {
        int64_t n = (int64_t)a.T * a.E;
        router_logits_f32<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
            (const float *)a.x, (const float *)a.wr, a.bias, a.logits, a.T, a.H, a.E);
    }
}

int router_parts(int T, int H, int E, int act)
{
    return act == ACT_BF16 && T > 16 && E % 128 == 0 && H % 2048 == 0 ? 8 : 1;
}

void launch_router(const RouterArgs &a, hipStream_t st)
{
    if (a.T == 0)
        return;
    if (router_parts(a.T, a.H, a.E, a.act) == 8) {
        const int nbe = a.E / 128;
        if (a.T > 4096)
            router_seg<128><<<(unsigned)(nbe * 8 * ((a.T + 127) / 128)), 256, 0, st>>>(
                (const uint16_t *)a.x, (const uint16_t *)a.wr, a.logits, a.T, a.H, a.E, a.hist,
                a.hist ? a.nhist : 0);
        else
            router_seg<64><<<(unsigned)(nbe * 8 * ((a.T + 63) / 64)), 256, 0, st>>>(
                (const uint16_t *)a.x, (const uint16_t *)a.wr, a.logits, a.T, a.H, a.E, a.hist,
                a.hist ? a.nhist : 0);
        const unsigned nb = (unsigned)((a.T + 3) / 4);
        switch (topk_per(a.E)) {
        case 1: router_topk_seg<1><<<nb, 256, 0, st>>>(a.logits, a.bias, a.idx, a.w, a.T, a.E, a.k, a.hist); break;
        case 2: router_topk_seg<2><<<nb, 256, 0, st>>>(a.logits, a.bias, a.idx, a.w, a.T, a.E, a.k, a.hist); break;
        case 4: router_topk_seg<4><<<nb, 256, 0, st>>>(a.logits, a.bias, a.idx, a.w, a.T, a.E, a.k, a.hist); break;
        case 8: router_topk_seg<8><<<nb, 256, 0, st>>>(a.logits, a.bias, a.idx, a.w, a.T, a.E, a.k, a.hist); break;
        default: router_topk_seg<16><<<nb, 256, 0, st>>>(a.logits, a.bias, a.idx, a.w, a.T, a.E, a.k, a.hist); break;
        }
        return;
    }
    launch_router_logits(a, st);
    const unsigned nb = (unsigned)((a.T + 3) / 4);
    switch (topk_per(a.E)) {
    case 1: router_topk<1><<<nb, 256, 0, st>>>(a.logits, a.idx, a.w, a.T, a.E, a.k); break;
    case 2: router_topk<2><<<nb, 256, 0, st>>>(a.logits, a.idx, a.w, a.T, a.E, a.k); break;
    case 4: router_topk<4><<<nb, 256, 0, st>>>(a.logits, a.idx, a.w, a.T, a.E, a.k); break;
    case 8: router_topk<8><<<nb, 256, 0, st>>>(a.logits, a.idx, a.w, a.T, a.E, a.k); break;
    default: router_topk<16><<<nb, 256, 0, st>>>(a.logits, a.idx, a.w, a.T, a.E, a.k); break;
    }
}

}  // namespace moe
