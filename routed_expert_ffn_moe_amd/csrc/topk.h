// Top-k selection and renormalised softmax of one token's router logits,
// computed by one wave.  Shared by the router kernels.
#pragma once

#include "common.h"

namespace moe {

// (value, index) order of the selection: larger logit first, equal logits by
// lower expert index.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib)
{
    return va > vb || (va == vb && ia < ib);
}

// Lane l holds logits l, l+64, ... (E <= 1024); k rounds of a wave-wide
// arg-max remove one expert each.  NaN logits rank last and the indices stay
// valid.  Writes idx[0..k) and w[0..k) (lanes j < k), and sidx[0..k) if given.
__device__ __forceinline__ void wave_topk(const float *__restrict__ lrow, int E, int k,
                                          int32_t *__restrict__ idx, float *__restrict__ w,
                                          int *sidx)
{
    const int lane = threadIdx.x & 63;
    const int per = (E + 63) / 64;  // <= 16
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int e = lane + 64 * i;
        v[i] = (i < per && e < E) ? lrow[e] : -INFINITY;
        if (v[i] != v[i])
            v[i] = -INFINITY;
    }
    float sel_v[16];
    int sel_i[16];
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int e = lane + 64 * i;
            if (i < per && e < E && better(v[i], e, bv, bi)) {
                bv = v[i];
                bi = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
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
            idx[j] = sel_i[j];
            w[j] = q[j] / z;
            if (sidx)
                sidx[j] = sel_i[j];
        }
    }
}

}  // namespace moe
