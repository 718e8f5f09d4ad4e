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

// Unsigned key with the order of the floats (NaN is taken as -inf).
__device__ __forceinline__ uint32_t order_key(float x)
{
    const uint32_t u = __float_as_uint(x != x ? -INFINITY : x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// LDS scratch of one wave: the k selected (logit, expert) pairs in selection
// order, then the logits in rank order.
struct TopkLds {
    float v[16];
    int e[16];
    float s[16];
};

// Makes one wave's LDS writes visible to its other lanes.
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Lane l holds logits l, l+64, ... (E <= 64*PER).  The k-th largest key is
// found bit by bit from the top (a radix select: 32 wave-wide counts, no
// data exchange between lanes), the keys above it and the lowest-index ties
// at it form the selection, and each selected pair's rank is its number of
// better pairs.  Weights are the softmax over the selected logits (the full
// softmax renormalised), summed in rank order.  NaN logits rank last.
// Writes idx[0..k) and w[0..k) (in rank order), and sidx[0..k) if given.
template <int PER>
__device__ __forceinline__ void wave_topk(const float *__restrict__ lrow, int E, int k,
                                          int32_t *__restrict__ idx, float *__restrict__ w,
                                          int *sidx, TopkLds *sh)
{
    const int lane = threadIdx.x & 63;
    float val[PER];
    uint32_t key[PER];  // 0 for the slots past E: below every logit's key
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        const bool ok = e < E;
        const float x = ok ? lrow[e] : -INFINITY;
        val[i] = x != x ? -INFINITY : x;
        key[i] = ok ? order_key(x) : 0u;
    }
    uint32_t thr = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = thr | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i)
            cnt += __popcll(__ballot(key[i] >= cand));
        thr = cnt >= k ? cand : thr;
    }
    int gt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i)
        gt += __popcll(__ballot(key[i] > thr));
    const int need = k - gt;  // ties at the threshold taken by lower index
    const uint64_t below = (1ull << lane) - 1;
    int base_eq = 0, base_sel = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const bool eq = key[i] == thr;
        const uint64_t meq = __ballot(eq);
        const bool sel = key[i] > thr || (eq && base_eq + __popcll(meq & below) < need);
        const uint64_t msel = __ballot(sel);
        if (sel) {
            const int slot = base_sel + __popcll(msel & below);
            sh->v[slot] = val[i];
            sh->e[slot] = lane + 64 * i;
        }
        base_eq += __popcll(meq);
        base_sel += __popcll(msel);
    }
    wave_sync();
    float vj = 0.0f;
    int ej = 0, rank = 0;
    if (lane < k) {
        vj = sh->v[lane];
        ej = sh->e[lane];
        for (int m = 0; m < k; ++m)
            rank += better(sh->v[m], sh->e[m], vj, ej);
        sh->s[rank] = vj;
    }
    wave_sync();
    if (lane < k) {
        const float mx = sh->s[0];
        float z = 0.0f;
        for (int j = 0; j < k; ++j)
            z += expf(sh->s[j] - mx);
        idx[rank] = ej;
        w[rank] = expf(vj - mx) / z;
        if (sidx)
            sidx[rank] = ej;
    }
}

// Logit slots per lane for E experts: 1, 2, 4, 8 or 16.
inline int topk_per(int E)
{
    const int per = (E + 63) / 64;
    return per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : per <= 8 ? 8 : 16;
}

}  // namespace moe
