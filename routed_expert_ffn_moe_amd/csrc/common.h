// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

#define MOE_WAVE 64

namespace moe {

// bf16 <-> fp32.  bf16 values travel as uint16_t bit patterns.
__device__ __forceinline__ float bf2f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Round-to-nearest-even fp32 -> bf16 (inputs here are finite).
__device__ __forceinline__ uint16_t f2bf(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf2(float a, float b)
{
    return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

// SiLU, z * sigmoid(z), with the hardware reciprocal (1 ulp) in place of an
// IEEE division: the result is rounded to bf16 right after, and the
// division's scaling and fix-up steps cost ten instructions per element in
// the GEMM epilogues.
__device__ __forceinline__ float silu(float z)
{
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Token row and routing weight of a grouped row.  Pairs p < n_pairs are the
// routed (t, j) pairs p = t * k + j; p >= n_pairs are shared-expert rows of
// token p - n_pairs.
__device__ __forceinline__ int pair_token(int p, int n_pairs, int k)
{
    return p < n_pairs ? p / k : p - n_pairs;
}

// MFMA wrappers (operand/result lane layouts verified on gfx950):
//  16x16x32 bf16: lane l holds A[l%16][8*(l/16) + i], B[k = 8*(l/16) + i][n = l%16],
//                 C[4*(l/16) + i][l%16].
__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The same MFMA with the accumulator held in the accumulation registers and
// updated in place.  For kernels whose accumulators fill those registers:
// there the compiler's own allocation rotates them through copies between
// MFMAs, which cost more issue slots than the MFMAs themselves.  The
// instruction is opaque to the compiler's hazard tracking, so it carries its
// own wait states for A/B operands written by a vector ALU instruction just
// before it (two are required), and ordinary instructions may read these
// accumulators only after mfma_acc_drain().
__device__ __forceinline__ void mfma16_acc(floatx4 &c, bf16x8 a, bf16x8 b)
{
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// Wait states covering the longest MFMA result latency before other
// instructions read mfma16_acc results.
__device__ __forceinline__ void mfma_acc_drain()
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v)
{
    return __builtin_bit_cast(bf16x8, v);
}

// Registers that carry a staged chunk across a loop iteration are held as
// one vector value: an array there would be placed in scratch memory.
template <int N>
using u32v = uint32_t __attribute__((ext_vector_type(4 * N)));

template <int N>
__device__ __forceinline__ void vset(u32v<N> &r, int i, uint4 t)
{
    r[4 * i] = t.x;
    r[4 * i + 1] = t.y;
    r[4 * i + 2] = t.z;
    r[4 * i + 3] = t.w;
}

template <int N>
__device__ __forceinline__ uint4 vget(const u32v<N> &r, int i)
{
    return uint4{r[4 * i], r[4 * i + 1], r[4 * i + 2], r[4 * i + 3]};
}

// Offset (elements) of the 8 K-consecutive elements (n, k .. k+7) of a bf16
// matrix [N, K] in the packed layout (k a multiple of 8): rows in groups of
// 32, K in steps of 32, each (group, step) two kilobyte blocks whose lane
// r + 16*b holds row 32*g + 8*(r/4) + 4*c + r%4 at K = 32*s + 8*b.
__device__ __forceinline__ int64_t packed_bf16_off(int n, int k, int K)
{
    const int j = n & 31, c = (j & 7) >> 2, r = 4 * (j >> 3) + (j & 3), b = (k & 31) >> 3;
    return ((((int64_t)(n >> 5) * (K >> 5) + (k >> 5)) * 2 + c) * 64 + r + 16 * b) * 8;
}

// Tile descriptor written by the permutation: group g (expert, or E for the
// shared expert) and the first grouped row of the tile.
struct Tile {
    int g;
    int row0;
};

// Inclusive prefix sum over the wave: DPP row shifts within each 16-lane
// row, then the row broadcasts carry the totals of the rows before.
__device__ __forceinline__ int wave_scan_add(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
    return v;
}

}  // namespace moe
