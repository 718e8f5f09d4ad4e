// Top-k selection and renormalised softmax of one token's router logits,
// computed by one wave.  Shared by the router kernels.
#pragma once

#include "common.h"

namespace moe {

// Unsigned key with the order of the floats: larger key, larger logit.  NaN
// is taken as -inf and -0 as +0, so equal keys are equal logits.
__device__ __forceinline__ uint32_t order_key(float x)
{
    const uint32_t u = __float_as_uint(x != x ? -INFINITY : x + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The logit of a key (the canonical one: never NaN or -0).
__device__ __forceinline__ float key_value(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Largest value over the wave, in every lane: prefix maxima within each
// 16-lane row by DPP row shifts, the rows joined by the row broadcasts, and
// lane 63 read back.  Lanes a shift reaches past read 0, the smallest key,
// and rows the broadcast masks off keep their own value: each step then
// compiles to one DPP max (T=1 decode step 14.88 -> 14.57 us against a
// separate DPP move and max per step, the same results bit for bit).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    int m = (int)v;
    m = (int)max((uint32_t)m, (uint32_t)__builtin_amdgcn_update_dpp(0, m, 0x111, 0xf, 0xf, true));
    m = (int)max((uint32_t)m, (uint32_t)__builtin_amdgcn_update_dpp(0, m, 0x112, 0xf, 0xf, true));
    m = (int)max((uint32_t)m, (uint32_t)__builtin_amdgcn_update_dpp(0, m, 0x114, 0xf, 0xf, true));
    m = (int)max((uint32_t)m, (uint32_t)__builtin_amdgcn_update_dpp(0, m, 0x118, 0xf, 0xf, true));
    m = (int)max((uint32_t)m, (uint32_t)__builtin_amdgcn_update_dpp(0, m, 0x142, 0xa, 0xf, true));
    m = (int)max((uint32_t)m, (uint32_t)__builtin_amdgcn_update_dpp(0, m, 0x143, 0xc, 0xf, true));
    return (uint32_t)__builtin_amdgcn_readlane(m, 63);
}

// Smallest value over the wave (same pattern).
__device__ __forceinline__ int wave_min_i32(int v)
{
    int m = v;
    m = min(m, __builtin_amdgcn_update_dpp(m, m, 0x111, 0xf, 0xf, false));
    m = min(m, __builtin_amdgcn_update_dpp(m, m, 0x112, 0xf, 0xf, false));
    m = min(m, __builtin_amdgcn_update_dpp(m, m, 0x114, 0xf, 0xf, false));
    m = min(m, __builtin_amdgcn_update_dpp(m, m, 0x118, 0xf, 0xf, false));
    m = min(m, __builtin_amdgcn_update_dpp(m, m, 0x142, 0xa, 0xf, false));
    m = min(m, __builtin_amdgcn_update_dpp(m, m, 0x143, 0xc, 0xf, false));
    return __builtin_amdgcn_readlane(m, 63);
}

// Top-k of one token's router logits, selected by one wave.  Lane l holds
// logits l, l+64, ... (E <= 64*PER) in val, sorted once into descending
// order.  k rounds each take the best remaining (logit, expert) pair of the
// wave, the head of one lane's list: larger logit first, equal logits by
// lower expert index; NaN ranks as -inf.  So the pairs come out in rank
// order: lane r < k ends with the expert of rank r in my_e and its key in
// my_k (the other lanes with 0).
template <int PER>
__device__ __forceinline__ void wave_topk_select(const float (&val)[PER], int E, int k, int &my_e,
                                                 uint32_t &my_k)
{
    const int lane = threadIdx.x & 63;
    uint32_t key[PER];  // 0 for the slots past E: below every logit
    int slot[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        key[i] = lane + 64 * i < E ? order_key(val[i]) : 0u;
        slot[i] = i;
    }
    // this lane's list in selection order (odd-even transposition sort; a
    // later slot moves ahead only with a strictly larger key)
#pragma unroll
    for (int r = 0; r < PER; ++r)
#pragma unroll
        for (int i = r & 1; i + 1 < PER; i += 2)
            if (key[i + 1] > key[i]) {
                const uint32_t tk = key[i];
                key[i] = key[i + 1];
                key[i + 1] = tk;
                const int ts = slot[i];
                slot[i] = slot[i + 1];
                slot[i + 1] = ts;
            }
    my_e = 0;
    my_k = 0;
    for (int r = 0; r < k; ++r) {
        const uint32_t M = wave_max_u32(key[0]);
        const uint64_t tie = __ballot(key[0] == M);
        int wl;
        if (__popcll(tie) == 1) {  // uniform
            wl = __ffsll((unsigned long long)tie) - 1;
        } else {  // equal logits: the lowest expert index among the heads
            const int em = wave_min_i32(key[0] == M ? lane + 64 * slot[0] : 0x7FFFFFFF);
            wl = em & 63;
        }
        const int er = wl + 64 * __builtin_amdgcn_readlane(slot[0], wl);
        if (lane == r) {
            my_e = er;
            my_k = M;
        }
        if (lane == wl) {  // the owner's list moves up
#pragma unroll
            for (int i = 0; i + 1 < PER; ++i) {
                key[i] = key[i + 1];
                slot[i] = slot[i + 1];
            }
            key[PER - 1] = 0u;
        }
    }
}

// The weights of a selection (wave_topk_select's my_e, my_k): the softmax
// over the selected logits (the full softmax renormalised over the
// selection), summed in rank order.  Lanes r < k write idx[r], w[r] and, if
// given, sidx[r].
__device__ __forceinline__ void wave_topk_weights(int my_e, uint32_t my_k, int k,
                                                  int32_t *__restrict__ idx,
                                                  float *__restrict__ w, int *sidx)
{
    const int lane = threadIdx.x & 63;
    const float mx = key_value(__builtin_amdgcn_readlane(my_k, 0));
    const float ex = lane < k ? expf(key_value(my_k) - mx) : 0.0f;
    float z = 0.0f;
    for (int r = 0; r < k; ++r)
        z += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), r));
    if (lane < k) {
        idx[lane] = my_e;
        w[lane] = ex / z;
        if (sidx)
            sidx[lane] = my_e;
    }
}

// Top-k and weights: writes idx[0..k) and w[0..k) in rank order, and
// sidx[0..k) if given.
template <int PER>
__device__ __forceinline__ void wave_topk_vals(const float (&val)[PER], int E, int k,
                                               int32_t *__restrict__ idx, float *__restrict__ w,
                                               int *sidx)
{
    int my_e;
    uint32_t my_k;
    wave_topk_select<PER>(val, E, k, my_e, my_k);
    wave_topk_weights(my_e, my_k, k, idx, w, sidx);
}

// The same, reading the token's E logits from memory.
template <int PER>
__device__ __forceinline__ void wave_topk(const float *__restrict__ lrow, int E, int k,
                                          int32_t *__restrict__ idx, float *__restrict__ w,
                                          int *sidx)
{
    const int lane = threadIdx.x & 63;
    float v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i)
        v[i] = lane + 64 * i < E ? lrow[lane + 64 * i] : 0.0f;
    wave_topk_vals<PER>(v, E, k, idx, w, sidx);
}

// Token t's logits (lane l: experts l, l+64, ...) from the split router's
// eight partial sums per logit (32 contiguous bytes, [T][E][8]): their sum
// in segment order, then the bias - the arithmetic of router_small.  Slots
// past E hold 0.
template <int PER>
__device__ __forceinline__ void wave_logits_from_parts(const float *__restrict__ parts,
                                                       const float *__restrict__ bias, int t,
                                                       int E, float (&v)[PER])
{
    const int lane = threadIdx.x & 63;
    float4 q[PER][2];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = min(lane + 64 * i, E - 1);
        const float4 *src = (const float4 *)(parts + ((int64_t)t * E + e) * 8);
        q[i][0] = src[0];
        q[i][1] = src[1];
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        float a = q[i][0].x;
        a += q[i][0].y;
        a += q[i][0].z;
        a += q[i][0].w;
        a += q[i][1].x;
        a += q[i][1].y;
        a += q[i][1].z;
        a += q[i][1].w;
        v[i] = e < E ? a + (bias ? bias[e] : 0.0f) : 0.0f;
    }
}

// Logit slots per lane for E experts: 1, 2, 4, 8 or 16.
inline int topk_per(int E)
{
    const int per = (E + 63) / 64;
    return per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : per <= 8 ? 8 : 16;
}

}  // namespace moe
