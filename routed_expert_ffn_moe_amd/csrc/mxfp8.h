// bf16 activations as a hi / lo pair of MXFP8 (E4M3) operands for the
// scaled fp4 MFMA: per 32-element block, e = floor(log2 amax) - 7,
// hi = fp8(x / 2^e) and lo = fp8((x / 2^e - hi) * 16) with E8M0 scales 2^e and
// 2^(e-4); the two MFMAs of a K step (hi, lo) reproduce x to about 2^-8
// relative, the precision of bf16 itself.  Shared by the MXFP4 kernels and
// the short-pass router, which quantises each token row once for all of them.
#pragma once

#include "common.h"

namespace moe {

constexpr int MX_PAD = 16;  // row padding (bytes): LDS rows fall on distinct banks

// Bytes of one quantised row of K elements: hi [K + MX_PAD], lo [K + MX_PAD],
// hi scales [K / 32], lo scales [K / 32] - the LDS staging layout of one row.
__host__ __device__ constexpr int mx_row_bytes(int K) { return 2 * (K + MX_PAD) + 2 * (K / 32); }

// E4M3 (OCP, bias 7) codes of two floats with |v| < 256, rounded to nearest
// even, into bytes 0-1 (HI false) or 2-3 (HI true) of `old`: the hardware
// conversion.  Over the quantiser's whole domain (every bf16 value times a
// power of two below 256 in magnitude, and the residuals formed from them)
// it gives the same codes as the round-to-nearest-even definition of the
// format, subnormals included (checked on gfx950 against a software encoder
// for all 2^16 bf16 patterns).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2(float a, float b, uint32_t old)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// The values of the E4M3 codes in bytes 0-1 (HI false) or 2-3 (HI true).
template <bool HI>
__device__ __forceinline__ void fp8x2_value(uint32_t codes, float &a, float &b)
{
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 v = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, HI);
    a = v[0];
    b = v[1];
}

// Activation staging: rows are quantised one 32-element block per thread and
// pass, as hi / lo E4M3 bytes [row][K + MX_PAD] and their E8M0 scales
// [row][K/32] (in LDS, or in a token's row record in memory).  A block
// travels packed (16 registers) and is converted 8 elements at a time.
__device__ __forceinline__ void block_load(uint4 (&raw)[4], const uint16_t *src)
{
#pragma unroll
    for (int c = 0; c < 4; ++c)
        raw[c] = *(const uint4 *)(src + c * 8);
}

// Source of staging block q: row q / nblk (index src[row] of the activation
// matrix), 32 elements at (q % nblk) * 32.
__device__ __forceinline__ const uint16_t *block_src(const uint16_t *a, const u32v<4> &src,
                                                    int64_t lda, int nblk, int q)
{
    const int r = q / nblk;
    uint32_t s = src[0];
#pragma unroll
    for (int i = 1; i < 16; ++i)
        s = r == i ? src[i] : s;
    return a + (int64_t)s * lda + (q - r * nblk) * 32;
}

__device__ __forceinline__ void block_quantise(const uint4 (&raw)[4], int r, int b, int K,
                                               uint8_t *ahi, uint8_t *alo, uint8_t *shi,
                                               uint8_t *slo)
{
    const int nblk = K / 32, ld = K + MX_PAD;
    // |bf16| maxima: with the sign bit cleared the bit patterns compare as
    // the magnitudes do
    uint32_t mx = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t w4[4] = {raw[c].x, raw[c].y, raw[c].z, raw[c].w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            mx = max(mx, max(w4[i] & 0x7FFFu, (w4[i] >> 16) & 0x7FFFu));
    }
    int e = (int)(mx >> 7) - 127 - 7;  // floor(log2 amax) - 7
    if (mx == 0)
        e = 0;
    e = max(e, -123);
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e
    uint8_t *dh = ahi + r * ld + b * 32;
    uint8_t *dl = alo + r * ld + b * 32;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t w4[4] = {raw[c].x, raw[c].y, raw[c].z, raw[c].w};
        uint32_t hi[2] = {0, 0}, lo[2] = {0, 0};
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // elements 2q, 2q + 1 of the eight
            const float x0 = __uint_as_float(w4[q] << 16) * inv;
            const float x1 = __uint_as_float(w4[q] & 0xFFFF0000u) * inv;
            float q0, q1;
            if (q & 1) {
                hi[q / 2] = fp8x2<true>(x0, x1, hi[q / 2]);
                fp8x2_value<true>(hi[q / 2], q0, q1);
                lo[q / 2] = fp8x2<true>((x0 - q0) * 16.0f, (x1 - q1) * 16.0f, lo[q / 2]);
            } else {
                hi[q / 2] = fp8x2<false>(x0, x1, hi[q / 2]);
                fp8x2_value<false>(hi[q / 2], q0, q1);
                lo[q / 2] = fp8x2<false>((x0 - q0) * 16.0f, (x1 - q1) * 16.0f, lo[q / 2]);
            }
        }
        *(uint2 *)(dh + 8 * c) = uint2{hi[0], hi[1]};
        *(uint2 *)(dl + 8 * c) = uint2{lo[0], lo[1]};
    }
    shi[r * nblk + b] = (uint8_t)(e + 127);
    slo[r * nblk + b] = (uint8_t)(e - 4 + 127);
}

// Pieces of 16 bytes of a row record (needs K % 512 == 0, so the scale
// areas are whole pieces): hi K/16, lo K/16, hi scales K/512, lo scales
// K/512.
__host__ __device__ constexpr int mx_rec_pieces(int K) { return K / 8 + K / 256; }

// Piece pc of row record `rec` to the LDS staging row r (bases ahi, alo,
// shi, slo as the quantiser writes them): the record's byte offset, and the
// LDS address it goes to.
__device__ __forceinline__ void mx_rec_piece(int pc, int K, int r, uint8_t *ahi, uint8_t *alo,
                                             uint8_t *shi, uint8_t *slo, int &goff,
                                             uint8_t *&dst)
{
    const int ld = K + MX_PAD, nblk = K / 32, h = K / 16, sp = nblk / 16;
    if (pc < h) {
        goff = pc * 16;
        dst = ahi + r * ld + pc * 16;
    } else if (pc < 2 * h) {
        goff = ld + (pc - h) * 16;
        dst = alo + r * ld + (pc - h) * 16;
    } else if (pc < 2 * h + sp) {
        goff = 2 * ld + (pc - 2 * h) * 16;
        dst = shi + r * nblk + (pc - 2 * h) * 16;
    } else {
        goff = 2 * ld + nblk + (pc - 2 * h - sp) * 16;
        dst = slo + r * nblk + (pc - 2 * h - sp) * 16;
    }
}

}  // namespace moe
