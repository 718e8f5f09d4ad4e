// MXFP4 expert weights on CDNA4's block-scaled fp4 MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4), for the bandwidth-bound small-T
// decode / verify shapes.
//
// Pages: "MoE prefill quantum" (section ruling out the hardware: unpacking
// MXFP4 and multiplying by the scale streams as fast as a plain read), the
// "DeepSeek V4.1F Q4" DSpark paragraph (the 6 verify rows share one weight
// stream) and the "Jetson Orin Nano MoE" section on other models (MXFP4
// matrix chunk size, 4.25 bits per weight).  Format: OCP MX v1.0 - E2M1
// codes, two per byte with the even element in the low nibble, one E8M0
// scale per 32 elements along K.
//
// Weight-stationary design: one wave owns one tile of the permutation (one
// expert's rows, at most 16 and at most T) and 16 output columns per weight
// matrix; every weight byte is read from HBM exactly once per tile.  The fp4
// weights are the MFMA's B operand with their own E8M0 scales.  The bf16
// activations are split into two MXFP8 (E4M3) operands, hi = fp8(x / 2^e)
// and lo = fp8((x / 2^e - hi) * 16) with scales 2^e and 2^(e-4) per 32-block,
// e = floor(log2 amax) - 7; two MFMAs (hi, lo) share the weight operand and
// reproduce x to about 2^-8 relative, the precision of bf16 itself.
//
// Lane layouts of the 16x16x128 scaled MFMA (checked on gfx950): with fp4 B,
// lane l holds column l%16 and K elements 32*(l/16) .. +31 (16 bytes); with
// fp8 A, lane l holds row l%16, bytes 0-15 at K = 16*(l/16) + i and bytes
// 16-31 at K = 64 + 16*(l/16) + i; the E8M0 scale supplied by lane 16*b + r
// applies to row (column) r and K block b.  Within a K chunk of S*128 the
// MFMA's four K blocks are mapped onto actual blocks S*b + s at step s, so
// that every lane reads S consecutive weight blocks (16*S contiguous bytes)
// and S consecutive scale bytes.
#include "common.h"
#include "kernels.h"

namespace moe {

int mxfp4_bm() { return 16; }

namespace {

struct MxP {
    const uint16_t *a;           // GU: x [T, H]; DC: h [rows, ldh]
    const uint8_t *c0, *c1;      // codes [E, N, K/2]
    const uint8_t *s0, *s1;      // scales [E, N, K/32]
    const int32_t *row_src, *offsets;
    const float *topk_w;
    uint16_t *out;
    const Tile *tiles;
    const int32_t *ntiles;
    int T, H, E, k, I, ldh, cap;
};

// E4M3 (OCP, bias 7) encoding of |v| <= 448, round to nearest even.
__device__ __forceinline__ uint32_t e4m3(float v, float &q)
{
    const uint32_t sgn = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fabsf(v);
    uint32_t code;
    float mag;
    if (a >= 0.015625f) {  // normal: 2^-6 and up
        uint32_t u = __float_as_uint(a);
        u = (u + 0x7FFFFu + ((u >> 20) & 1u)) & ~0xFFFFFu;
        const int e8 = (int)(u >> 23) - 127 + 7;
        code = ((uint32_t)e8 << 3) | ((u >> 20) & 7u);
        mag = __uint_as_float(u);
        if (code > 0x7Eu) {  // saturate at 448
            code = 0x7Eu;
            mag = 448.0f;
        }
    } else {  // subnormal: multiples of 2^-9
        const float n = rintf(a * 512.0f);
        code = (uint32_t)n;  // 8 encodes 2^-6, the smallest normal
        mag = n * (1.0f / 512.0f);
    }
    q = sgn ? -mag : mag;
    return sgn | code;
}

// Quantise the tile's activation rows into LDS: hi / lo E4M3 bytes in natural
// [row][K] order and their E8M0 scales [row][K/32].
__device__ void stage_activations(const MxP &p, bool gu, int row0, int nrows, int K,
                                  uint8_t *ahi, uint8_t *alo, uint8_t *shi, uint8_t *slo)
{
    const int lane = threadIdx.x;
    const int nblk = K / 32;
    const int n_pairs = p.T * p.k;
    for (int q = lane; q < nrows * nblk; q += 64) {
        const int r = q / nblk, b = q % nblk;
        const int pos = row0 + r;
        const uint16_t *src = gu ? p.a + (int64_t)pair_token(p.row_src[pos], n_pairs, p.k) * p.H
                                 : p.a + (int64_t)pos * p.ldh;
        src += b * 32;
        float v[32];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 w = *(const uint4 *)(src + c * 8);
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[c * 8 + 2 * i] = bf2f((uint16_t)(ww[i] & 0xFFFF));
                v[c * 8 + 2 * i + 1] = bf2f((uint16_t)(ww[i] >> 16));
            }
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i)
            amax = fmaxf(amax, fabsf(v[i]));
        int e = (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127 - 7;
        if (amax == 0.0f)
            e = 0;
        e = max(e, -123);
        const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            hi[i] = 0;
            lo[i] = 0;
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            float qh, ql;
            const float xs = v[i] * inv;
            const uint32_t ch = e4m3(xs, qh);
            const uint32_t cl = e4m3((xs - qh) * 16.0f, ql);
            hi[i / 4] |= ch << (8 * (i % 4));
            lo[i / 4] |= cl << (8 * (i % 4));
        }
        uint4 *dh = (uint4 *)(ahi + r * K + b * 32);
        uint4 *dl = (uint4 *)(alo + r * K + b * 32);
        dh[0] = uint4{hi[0], hi[1], hi[2], hi[3]};
        dh[1] = uint4{hi[4], hi[5], hi[6], hi[7]};
        dl[0] = uint4{lo[0], lo[1], lo[2], lo[3]};
        dl[1] = uint4{lo[4], lo[5], lo[6], lo[7]};
        shi[r * nblk + b] = (uint8_t)(e + 127);
        slo[r * nblk + b] = (uint8_t)(e - 4 + 127);
    }
}

// One K chunk of S*128 elements starting at kc: S scaled-MFMA steps per
// weight matrix and activation half.
template <int S, int NB>
__device__ __forceinline__ void mx_chunk(const uint8_t *const *wrow, const uint8_t *const *srow,
                                         const uint8_t *ahi, const uint8_t *alo,
                                         const uint8_t *shi, const uint8_t *slo, int K, int kc,
                                         int ar, bool arow_ok, floatx4 *acc)
{
    const int lane = threadIdx.x;
    const int g4 = lane >> 4;
    // Weights: 16*S contiguous bytes and S scale bytes per lane and matrix.
    uint4 wc[NB][S];
    uint32_t ws[NB];
#pragma unroll
    for (int m = 0; m < NB; ++m) {
        const uint8_t *cp = wrow[m] + (kc + 32 * S * g4) / 2;
#pragma unroll
        for (int s = 0; s < S; ++s)
            wc[m][s] = *(const uint4 *)(cp + 16 * s);
        const uint8_t *sp = srow[m] + kc / 32 + S * g4;
        if (S == 4)
            ws[m] = *(const uint32_t *)sp;
        else if (S == 2)
            ws[m] = *(const uint16_t *)sp;
        else
            ws[m] = *sp;
    }
    const int nblk = K / 32;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        // Activation operand for virtual K block pair (g4/2) and (2 + g4/2).
        const int off = (g4 & 1) * 16;
        const int k_lo = kc + 32 * (S * (g4 >> 1) + s) + off;
        const int k_hi = kc + 32 * (S * (2 + (g4 >> 1)) + s) + off;
        intx8 ah = {0, 0, 0, 0, 0, 0, 0, 0}, al = {0, 0, 0, 0, 0, 0, 0, 0};
        if (arow_ok) {
            const uint4 h0 = *(const uint4 *)(ahi + ar * K + k_lo);
            const uint4 h1 = *(const uint4 *)(ahi + ar * K + k_hi);
            const uint4 l0 = *(const uint4 *)(alo + ar * K + k_lo);
            const uint4 l1 = *(const uint4 *)(alo + ar * K + k_hi);
            ah = intx8{(int)h0.x, (int)h0.y, (int)h0.z, (int)h0.w,
                       (int)h1.x, (int)h1.y, (int)h1.z, (int)h1.w};
            al = intx8{(int)l0.x, (int)l0.y, (int)l0.z, (int)l0.w,
                       (int)l1.x, (int)l1.y, (int)l1.z, (int)l1.w};
        }
        const int sblk = kc / 32 + S * g4 + s;
        const int sa_h = shi[ar * nblk + sblk];
        const int sa_l = slo[ar * nblk + sblk];
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            const uint4 c = wc[m][s];
            const intx8 b = {(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
            const int sb = (int)((ws[m] >> (8 * s)) & 0xFF);
            acc[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ah, b, acc[m], 0, 4, 0, sa_h,
                                                                       0, sb);
            acc[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(al, b, acc[m], 0, 4, 0, sa_l,
                                                                       0, sb);
        }
    }
}

// Weights of one S=4 chunk (512 K) for the lane: 64 code bytes and 4 scale
// bytes per matrix.
template <int NB>
struct MxChunk {
    uint4 c[NB][4];
    uint32_t s[NB];
};

template <int NB>
__device__ __forceinline__ void mx_load4(MxChunk<NB> &w, const uint8_t *const *wrow,
                                         const uint8_t *const *srow, int kc)
{
    const int g4 = threadIdx.x >> 4;
#pragma unroll
    for (int m = 0; m < NB; ++m) {
        const uint8_t *cp = wrow[m] + (kc + 128 * g4) / 2;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            w.c[m][s] = *(const uint4 *)(cp + 16 * s);
        w.s[m] = *(const uint32_t *)(srow[m] + kc / 32 + 4 * g4);
    }
}

template <int NB>
__device__ __forceinline__ void mx_compute4(const MxChunk<NB> &w, const uint8_t *ahi,
                                            const uint8_t *alo, const uint8_t *shi,
                                            const uint8_t *slo, int K, int kc, int ar,
                                            bool arow_ok, floatx4 *acc)
{
    const int g4 = threadIdx.x >> 4;
    const int nblk = K / 32;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int off = (g4 & 1) * 16;
        const int k_lo = kc + 32 * (4 * (g4 >> 1) + s) + off;
        const int k_hi = kc + 32 * (4 * (2 + (g4 >> 1)) + s) + off;
        intx8 ah = {0, 0, 0, 0, 0, 0, 0, 0}, al = {0, 0, 0, 0, 0, 0, 0, 0};
        if (arow_ok) {
            const uint4 h0 = *(const uint4 *)(ahi + ar * K + k_lo);
            const uint4 h1 = *(const uint4 *)(ahi + ar * K + k_hi);
            const uint4 l0 = *(const uint4 *)(alo + ar * K + k_lo);
            const uint4 l1 = *(const uint4 *)(alo + ar * K + k_hi);
            ah = intx8{(int)h0.x, (int)h0.y, (int)h0.z, (int)h0.w,
                       (int)h1.x, (int)h1.y, (int)h1.z, (int)h1.w};
            al = intx8{(int)l0.x, (int)l0.y, (int)l0.z, (int)l0.w,
                       (int)l1.x, (int)l1.y, (int)l1.z, (int)l1.w};
        }
        const int sblk = kc / 32 + 4 * g4 + s;
        const int sa_h = shi[ar * nblk + sblk];
        const int sa_l = slo[ar * nblk + sblk];
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            const uint4 c = w.c[m][s];
            const intx8 b = {(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
            const int sb = (int)((w.s[m] >> (8 * s)) & 0xFF);
            acc[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ah, b, acc[m], 0, 4, 0, sa_h,
                                                                       0, sb);
            acc[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(al, b, acc[m], 0, 4, 0, sa_l,
                                                                       0, sb);
        }
    }
}

template <bool GU>
__global__ __launch_bounds__(64) void expert_mxfp4(MxP p)
{
    constexpr int NB = GU ? 2 : 1;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    if ((int)blockIdx.y >= *p.ntiles)
        return;
    const Tile tile = p.tiles[blockIdx.y];
    const int g = tile.g, row0 = tile.row0;
    const int nrows = min(16, p.offsets[g + 1] - row0);
    const int N = GU ? p.I : p.H;
    const int K = GU ? p.H : p.I;
    const int n0 = blockIdx.x * 16;
    if (n0 >= N)
        return;
    const int lane = threadIdx.x;
    const int n_pairs = p.T * p.k;

    uint8_t *ahi = smem;
    uint8_t *alo = ahi + p.cap * K;
    uint8_t *shi = alo + p.cap * K;
    uint8_t *slo = shi + p.cap * (K / 32);

    const int64_t cstride = (int64_t)N * (K / 2), sstride = (int64_t)N * (K / 32);
    const int n = n0 + (lane & 15);
    const uint8_t *wrow[NB], *srow[NB];
    wrow[0] = p.c0 + g * cstride + (int64_t)n * (K / 2);
    srow[0] = p.s0 + g * sstride + (int64_t)n * (K / 32);
    if (GU) {
        wrow[NB - 1] = p.c1 + g * cstride + (int64_t)n * (K / 2);
        srow[NB - 1] = p.s1 + g * sstride + (int64_t)n * (K / 32);
    }
    // The first two 512-wide weight chunks go out before the activations are
    // quantised, so their HBM latency overlaps that work.
    const int nfull = K / 512;
    MxChunk<NB> wa, wb;
    if (nfull > 0) {
        mx_load4<NB>(wa, wrow, srow, 0);
        mx_load4<NB>(wb, wrow, srow, min(1, nfull - 1) * 512);
    }
    stage_activations(p, GU, row0, nrows, K, ahi, alo, shi, slo);
    __syncthreads();

    const int r = lane & 15;
    const bool rok = r < nrows;
    const int ar = rok ? r : 0;

    floatx4 acc[NB];
#pragma unroll
    for (int m = 0; m < NB; ++m)
        acc[m] = floatx4{0, 0, 0, 0};
    // Two-chunk register pipeline over the 512-wide chunks (the last reloads
    // are re-reads of the final chunk, never out of bounds).
    for (int c = 0; c < nfull; c += 2) {
        mx_compute4<NB>(wa, ahi, alo, shi, slo, K, c * 512, ar, rok, acc);
        mx_load4<NB>(wa, wrow, srow, min(c + 2, nfull - 1) * 512);
        if (c + 1 < nfull) {
            mx_compute4<NB>(wb, ahi, alo, shi, slo, K, (c + 1) * 512, ar, rok, acc);
            mx_load4<NB>(wb, wrow, srow, min(c + 3, nfull - 1) * 512);
        }
    }
    int kc = nfull * 512;
    if (kc + 256 <= K) {
        mx_chunk<2, NB>(wrow, srow, ahi, alo, shi, slo, K, kc, ar, rok, acc);
        kc += 256;
    }
    if (kc + 128 <= K)
        mx_chunk<1, NB>(wrow, srow, ahi, alo, shi, slo, K, kc, ar, rok, acc);

    // Epilogue: C[4*(l/16) + i][l%16].
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = (lane >> 4) * 4 + i;
        if (m >= nrows)
            continue;
        const int pos = row0 + m;
        if (GU) {
            const float hv = silu(acc[0][i]) * acc[NB - 1][i];
            p.out[(int64_t)pos * p.ldh + n] = f2bf(hv);
        } else {
            p.out[(int64_t)pos * p.H + n] = f2bf(acc[0][i]);
        }
    }
}

template <bool GU>
void run(const ExpertArgs &a, hipStream_t st)
{
    MxP p;
    p.a = (const uint16_t *)(GU ? a.x : a.h);
    p.c0 = (const uint8_t *)(GU ? a.w_gate : a.w_down);
    p.c1 = (const uint8_t *)(GU ? a.w_up : nullptr);
    p.s0 = GU ? a.s_gate : a.s_down;
    p.s1 = GU ? a.s_up : nullptr;
    p.row_src = a.row_src;
    p.offsets = a.offsets;
    p.topk_w = a.topk_w;
    p.out = (uint16_t *)(GU ? a.h : a.stage);
    p.tiles = GU ? a.tiles_gu : a.tiles_dc;
    p.ntiles = GU ? a.ntiles_gu : a.ntiles_dc;
    p.T = a.T;
    p.H = a.H;
    p.E = a.E;
    p.k = a.k;
    p.I = a.I;
    p.ldh = a.I;
    p.cap = a.T < 16 ? a.T : 16;
    const int K = GU ? a.H : a.I;
    const int N = GU ? a.I : a.H;
    const size_t lds = (size_t)p.cap * (2 * K + 2 * (K / 32));
    dim3 grid(N / 16, GU ? a.max_tiles_gu : a.max_tiles_dc);
    if (grid.y == 0)
        return;
    if (lds > 64 * 1024 &&
        hipFuncSetAttribute((const void *)expert_mxfp4<GU>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return;  // the launch below then reports the error
    expert_mxfp4<GU><<<grid, 64, lds, st>>>(p);
}

}  // namespace

void launch_gate_up_mxfp4(const ExpertArgs &a, hipStream_t st) { run<true>(a, st); }
void launch_down_mxfp4(const ExpertArgs &a, hipStream_t st) { run<false>(a, st); }

}  // namespace moe
