// Router: logits = x . router_w^T (+ bias) in fp32, then top-k and the
// renormalised softmax weights of the selected experts.
//
// Pages: "MoE prefill quantum" (cause section: k of E experts per token) and
// "DeepSeek V4.1F Q4 with native DSpark MTP" (decode paragraph: the router
// is one fused dispatch instead of nine).  Logits are accumulated in fp32 and
// never rounded to bf16; selection is on the logits, ties to the lower index.
#include "common.h"
#include "kernels.h"

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

// (value, index) order of the selection: larger logit first, equal logits by
// lower expert index.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib)
{
    return va > vb || (va == vb && ia < ib);
}

// Top-k and weights: one wave per token.  Lane l holds logits l, l+64, ...;
// k rounds of a wave-wide arg-max remove one expert each.
__global__ __launch_bounds__(256) void router_topk(
    const float *__restrict__ logits, int32_t *__restrict__ idx, float *__restrict__ w,
    int T, int E, int k)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T)
        return;
    const int per = (E + 63) / 64;  // <= 16
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        int e = lane + 64 * i;
        v[i] = (i < per && e < E) ? logits[(int64_t)t * E + e] : -INFINITY;
        if (v[i] != v[i])  // NaN logits rank last; indices stay valid
            v[i] = -INFINITY;
    }
    float sel_v[16];
    int sel_i[16];
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            int e = lane + 64 * i;
            if (i < per && e < E && better(v[i], e, bv, bi)) {
                bv = v[i];
                bi = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            float ov = __shfl_xor(bv, off);
            int oi = __shfl_xor(bi, off);
            if (better(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        sel_v[j] = bv;
        sel_i[j] = bi;
        if ((bi & 63) == lane) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (i == (bi >> 6))
                    v[i] = -INFINITY;
        }
    }
    // Softmax over the selected logits (the full softmax renormalised).
    const float m = sel_v[0];
    float z = 0.0f;
    float q[16];
    for (int j = 0; j < k; ++j) {
        q[j] = expf(sel_v[j] - m);
        z += q[j];
    }
    for (int j = 0; j < k; ++j) {
        if (lane == j) {
            idx[(int64_t)t * k + j] = sel_i[j];
            w[(int64_t)t * k + j] = q[j] / z;
        }
    }
}

void launch_router(const RouterArgs &a, hipStream_t st)
{
    if (a.T == 0)
        return;
    if (a.act == ACT_BF16) {
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
    router_topk<<<(a.T + 3) / 4, 256, 0, st>>>(a.logits, a.idx, a.w, a.T, a.E, a.k);
}

}  // namespace moe
