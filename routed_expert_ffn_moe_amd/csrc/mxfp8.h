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

// E4M3 (OCP, bias 7) encoding of |v| <= 448, round to nearest even; both the
// normal and the subnormal candidate are formed and one is selected, so the
// conversion has no branch.
__device__ __forceinline__ uint32_t e4m3(float v, float &q)
{
    const uint32_t sgn = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fabsf(v);
    // normal (2^-6 and up): round the fp32 mantissa to 3 bits
    uint32_t u = __float_as_uint(a);
    u = (u + 0x7FFFFu + ((u >> 20) & 1u)) & ~0xFFFFFu;
    uint32_t cn = ((((u >> 23) - 127u + 7u) & 0xFu) << 3) | ((u >> 20) & 7u);
    float mn = __uint_as_float(u);
    const bool sat = u > 0x43E00000u;  // above 448
    cn = sat ? 0x7Eu : cn;
    mn = sat ? 448.0f : mn;
    // subnormal: multiples of 2^-9 (8 encodes 2^-6, the smallest normal)
    const float ns = rintf(a * 512.0f);
    const bool normal = a >= 0.015625f;
    const uint32_t code = normal ? cn : (uint32_t)ns;
    const float mag = normal ? mn : ns * (1.0f / 512.0f);
    q = sgn ? -mag : mag;
    return sgn | code;
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
        for (int i = 0; i < 8; ++i) {
            const uint16_t h = (uint16_t)(i & 1 ? w4[i / 2] >> 16 : w4[i / 2] & 0xFFFF);
            float qh, ql;
            const float xs = bf2f(h) * inv;
            const uint32_t ch = e4m3(xs, qh);
            const uint32_t cl = e4m3((xs - qh) * 16.0f, ql);
            hi[i / 4] |= ch << (8 * (i % 4));
            lo[i / 4] |= cl << (8 * (i % 4));
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
