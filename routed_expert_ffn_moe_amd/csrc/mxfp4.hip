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
// Weight-stationary design: a workgroup owns one tile of the permutation
// (one expert's rows, at most 16 and at most T) and NW*CPW*16 output columns
// per weight matrix; each of its waves owns CPW blocks of 16 columns.  A wave
// issues the loads of its whole weight slice (K in slabs of up to 2048) before
// anything else, so a launch has nearly all of its weight bytes in flight at
// once; meanwhile the workgroup quantises the tile's activation rows into
// LDS once for all its waves.  Every weight byte is read from HBM exactly once.
// The weights are read in the packed layout (moe_pack_mxfp4): one MFMA step
// of a 16-row block is a contiguous kilobyte, 16 bytes per lane, so every
// load instruction of a wave fetches whole cache lines.
//
// The fp4 weights are the MFMA's B operand with their own E8M0 scales.  The
// bf16 activations are split into two MXFP8 (E4M3) operands, hi = fp8(x/2^e)
// and lo = fp8((x/2^e - hi) * 16) with scales 2^e and 2^(e-4) per 32-block,
// e = floor(log2 amax) - 7; two MFMAs (hi, lo) share the weight operand and
// reproduce x to about 2^-8 relative, the precision of bf16 itself.
//
// Lane layouts of the 16x16x128 scaled MFMA (checked on gfx950): with fp4 B,
// lane l holds column l%16 and K elements 32*(l/16) .. +31 (16 bytes); with
// fp8 A, lane l holds row l%16, bytes 0-15 at K = 16*(l/16) + i and bytes
// 16-31 at K = 64 + 16*(l/16) + i; the E8M0 scale supplied by lane 16*b + r
// applies to row (column) r and K block b.
#include "common.h"
#include "kernels.h"
#include "mxfp8.h"
#include "topk.h"

#include <algorithm>
#include <cstdlib>
#include <type_traits>

namespace moe {

int mxfp4_bm() { return 16; }

namespace {

struct MxP {
    const uint16_t *a;           // GU: x [T, H]; DC: h [rows, ldh]
    const uint8_t *xq;           // GU: x quantised once per token (mxfp8.h records), or null
    const uint8_t *c0, *c1;      // codes [E, N, K/2]
    const uint8_t *s0, *s1;      // scales [E, N, K/32]
    const int32_t *row_tok, *offsets;
    uint16_t *out;
    const Tile *tiles;
    const int32_t *ntiles;
    int T, H, E, k, I, ldh, cap;
};

// A lane's weights of one K slab of NQ 128-wide steps, for one column block
// and matrix, from the packed layout: step s is 16 bytes of a contiguous
// kilobyte per wave, and the lane's scale bytes of the slab are contiguous
// (loaded AL at a time, AL the largest of 4, 2, 1 dividing NQ).
template <int NQ>
struct MxSlice {
    static constexpr int AL = NQ % 4 == 0 ? 4 : NQ % 2 == 0 ? 2 : 1;
    uint4 q[NQ];
    uint32_t sc[(NQ + 3) / 4];
};

// NT: the codes are read once per launch (no other workgroup wants them), so
// they are loaded with the streaming hint and do not displace what other
// workgroups will read again (decode and verify rows, T=6: 31.4 -> 29.6 us;
// T=64: 114 -> 104 us).  Codes that a second row tile of the same expert
// reads again take plain loads (streamed, that reuse costs T=512 5%).
template <int NQ, bool NT = true>
__device__ __forceinline__ void slice_load(MxSlice<NQ> &w, const uint8_t *cbase,
                                           const uint8_t *sbase, int q0, int s_begin, int s_end)
{
    using W = MxSlice<NQ>;
    if (s_begin == 0) {  // the scales of the whole slab go ahead of its codes
#pragma unroll
        for (int i = 0; i < (NQ + 3) / 4; ++i)
            w.sc[i] = 0;
#pragma unroll
        for (int a = 0; a < NQ / W::AL; ++a) {
            const int s = a * W::AL;
            uint32_t v;
            if (W::AL == 4)
                v = *(const uint32_t *)(sbase + q0 + s);
            else if (W::AL == 2)
                v = *(const uint16_t *)(sbase + q0 + s);
            else
                v = sbase[q0 + s];
            w.sc[s / 4] |= v << (8 * (s % 4));
        }
    }
#pragma unroll
    for (int s = 0; s < NQ; ++s)
        if (s >= s_begin && s < s_end) {
            const uint4 *src = (const uint4 *)(cbase + (size_t)(q0 + s) * 1024);
            if (NT) {
                const u32v<1> t = __builtin_nontemporal_load((const u32v<1> *)src);
                w.q[s] = uint4{t[0], t[1], t[2], t[3]};
            } else {
                w.q[s] = *src;
            }
        }
}

// One 128-wide K step (hi and lo halves) at absolute step q: the activation
// operand of row ar from LDS (lane group g4: K = 128q + 16*g4 .. +15 and
// 64 more), its scale for block 4q + g4, and the weights' operands.
template <int NB, int CPW>
__device__ __forceinline__ void mx_step(const uint4 (&b)[NB][CPW], const int (&sb)[NB][CPW],
                                        const uint8_t *ahi, const uint8_t *alo, const uint8_t *shi,
                                        const uint8_t *slo, int ld, int nblk, int q, int ar,
                                        floatx4 (&acc)[NB][CPW])
{
    const int g4 = threadIdx.x >> 4 & 3;
    const int k_lo = 128 * q + 16 * g4;
    const uint4 h0 = *(const uint4 *)(ahi + ar * ld + k_lo);
    const uint4 h1 = *(const uint4 *)(ahi + ar * ld + k_lo + 64);
    const uint4 l0 = *(const uint4 *)(alo + ar * ld + k_lo);
    const uint4 l1 = *(const uint4 *)(alo + ar * ld + k_lo + 64);
    const intx8 ah = {(int)h0.x, (int)h0.y, (int)h0.z, (int)h0.w,
                      (int)h1.x, (int)h1.y, (int)h1.z, (int)h1.w};
    const intx8 al = {(int)l0.x, (int)l0.y, (int)l0.z, (int)l0.w,
                      (int)l1.x, (int)l1.y, (int)l1.z, (int)l1.w};
    const int sa_h = shi[ar * nblk + 4 * q + g4];
    const int sa_l = slo[ar * nblk + 4 * q + g4];
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int cb = 0; cb < CPW; ++cb) {
            const intx8 bb = {(int)b[m][cb].x, (int)b[m][cb].y, (int)b[m][cb].z,
                              (int)b[m][cb].w, 0, 0, 0, 0};
            acc[m][cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                ah, bb, acc[m][cb], 0, 4, 0, sa_h, 0, sb[m][cb]);
            acc[m][cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                al, bb, acc[m][cb], 0, 4, 0, sa_l, 0, sb[m][cb]);
        }
}

// Workgroup barrier that waits for this wave's LDS operations only (the
// global loads in flight stay in flight).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The tile list, its length and the group offsets come in as read-only
// kernel arguments: uniform scalar loads, the first two issued together, so
// a workgroup starts its weight stream one memory latency after it starts.
template <bool GU, int CPW, int NW, int NQ, bool ONE, bool WF = false>
__global__ __launch_bounds__(64 * NW, WF ? 2 : 3) void expert_mxfp4(MxP p, const int32_t *__restrict__ ntiles,
                                                           const Tile *__restrict__ tiles,
                                                           const int32_t *__restrict__ offsets,
                                                           const int32_t *__restrict__ row_tok)
{
    constexpr int NB = GU ? 2 : 1;
    using W = MxSlice<NQ>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int nt = *ntiles;
    const Tile tile = tiles[blockIdx.y];  // within the list's capacity
    // both loads feed the test (no short circuit), so they are issued together
    if (((int)blockIdx.y >= nt) | (tile.g < 0))
        return;
    const int g = tile.g, row0 = tile.row0;
    const int N = GU ? p.I : p.H;
    const int K = GU ? p.H : p.I;  // a multiple of NQ * 128
    const int Q = K / 128;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ld = K + MX_PAD;

    uint8_t *ahi = smem;
    uint8_t *alo = ahi + p.cap * ld;
    uint8_t *shi = alo + p.cap * ld;
    uint8_t *slo = shi + p.cap * (K / 32);

    // This wave's CPW 16-row blocks of each matrix in the packed layout.
    const uint8_t *cbase[NB][CPW], *sbase[NB][CPW];
#pragma unroll
    for (int cb = 0; cb < CPW; ++cb) {
        const int64_t blk = (int64_t)g * (N / 16) + (blockIdx.x * NW + wave) * CPW + cb;
        cbase[0][cb] = p.c0 + blk * Q * 1024 + 16 * lane;
        sbase[0][cb] = p.s0 + (blk * 64 + lane) * Q;
        if (GU) {
            cbase[NB - 1][cb] = p.c1 + blk * Q * 1024 + 16 * lane;
            sbase[NB - 1][cb] = p.s1 + (blk * 64 + lane) * Q;
        }
    }

    floatx4 acc[NB][CPW];
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int cb = 0; cb < CPW; ++cb)
            acc[m][cb] = floatx4{0, 0, 0, 0};

    // The tile's rows (scalar loads): their count and, for gate+up, the token
    // of each, which locates its activation row.
    const int nrows = min(16, offsets[g + 1] - row0);
    // the expert's rows fit this one tile: its weights are read once
    const bool once = (offsets[g] == row0) & (offsets[g + 1] - row0 <= 16);
    const int last = p.T * p.k - 1;  // last grouped row
    u32v<4> src;  // 16 row indices, held as one vector value (registers)
#pragma unroll
    for (int r = 0; r < 16; ++r)
        src[r] = (uint32_t)(GU ? row_tok[min(row0 + r, last)] : min(row0 + r, last));
    const int nblk = K / 32;
    const int nq = nrows * nblk;  // activation blocks to stage
    const int64_t lda = GU ? p.H : p.ldh;

    // The tile's activation rows are quantised into LDS before any weight is
    // requested: the registers the conversion needs are free again before
    // the weight slice lands, so three workgroups fit on a CU and a decode
    // grid is resident at once (no second round of workgroups).  Two blocks
    // per thread are loaded together; only tiles of more than 8 rows loop.
    const int tid = threadIdx.x;
    W w[NB][CPW];
    auto issue_as = [&](auto nt) {
#pragma unroll
        for (int s = 0; s < NQ; ++s) {
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int cb = 0; cb < CPW; ++cb)
                    slice_load<NQ, decltype(nt)::value>(w[m][cb], cbase[m][cb], sbase[m][cb], 0,
                                                        s, s + 1);
            __builtin_amdgcn_sched_barrier(0);  // keep the issue order
        }
    };
    auto issue_weights = [&]() {
        if (once)
            issue_as(std::true_type{});
        else
            issue_as(std::false_type{});
    };
    if (WF) {
        // Grids far smaller than the chip (one decode row): the
        // weight slab is requested right behind the first activation blocks
        // and the quantisation waits for those blocks only (a wave's loads
        // complete in order for its wait counter), so the two memory
        // latencies overlap; it holds the slab's registers through the
        // quantisation, hence two workgroups per CU.
        uint4 raw0[4];
        block_load(raw0, block_src(p.a, src, lda, nblk, tid < nq ? tid : 0));
        __builtin_amdgcn_sched_barrier(0);
        issue_weights();
        if (tid < nq)
            block_quantise(raw0, tid / nblk, tid % nblk, K, ahi, alo, shi, slo);
        for (int q = tid + 64 * NW; q < nq; q += 64 * NW) {
            block_load(raw0, block_src(p.a, src, lda, nblk, q));
            block_quantise(raw0, q / nblk, q % nblk, K, ahi, alo, shi, slo);
        }
    } else if (GU && p.xq) {
        // The router quantised every token row once: copy the tile rows'
        // records into LDS, PB 16-byte pieces per thread at a time (decode
        // and verify tiles hold a few rows: one or two rounds; four when the
        // slice pointers stay live over K slabs).
        constexpr int PB = ONE ? 8 : 4;
        const int per = mx_rec_pieces(K), total = nrows * per;
        for (int b0 = 0; b0 < total; b0 += PB * 64 * NW) {
            uint4 pv[PB];
#pragma unroll
            for (int i = 0; i < PB; ++i) {
                const int q = b0 + tid + 64 * NW * i;
                const int r = q / per;
                int goff;
                uint8_t *dst;
                mx_rec_piece(q - r * per, K, r, ahi, alo, shi, slo, goff, dst);
                uint32_t tok = src[0];  // src[r] by selects: a vector indexed at run time
#pragma unroll                          // would be placed in scratch memory
                for (int k2 = 1; k2 < 16; ++k2)
                    tok = r == k2 ? src[k2] : tok;
                if (q < total)
                    pv[i] = *(const uint4 *)(p.xq + (int64_t)tok * mx_row_bytes(K) + goff);
            }
#pragma unroll
            for (int i = 0; i < PB; ++i) {
                const int q = b0 + tid + 64 * NW * i;
                const int r = q / per;
                int goff;
                uint8_t *dst;
                mx_rec_piece(q - r * per, K, r, ahi, alo, shi, slo, goff, dst);
                if (q < total)
                    *(uint4 *)dst = pv[i];
            }
        }
        issue_weights();
    } else {
        {
            uint4 raw0[4], raw1[4];
            const int q1 = tid + 64 * NW;
            block_load(raw0, block_src(p.a, src, lda, nblk, tid < nq ? tid : 0));
            block_load(raw1, block_src(p.a, src, lda, nblk, q1 < nq ? q1 : 0));
            if (tid < nq)
                block_quantise(raw0, tid / nblk, tid % nblk, K, ahi, alo, shi, slo);
            if (q1 < nq)
                block_quantise(raw1, q1 / nblk, q1 % nblk, K, ahi, alo, shi, slo);
            for (int q = tid + 2 * 64 * NW; q < nq; q += 64 * NW) {  // tiles of many rows
                block_load(raw0, block_src(p.a, src, lda, nblk, q));
                block_quantise(raw0, q / nblk, q % nblk, K, ahi, alo, shi, slo);
            }
        }
        // Slab 0 of the weights, all of it in flight before the barrier, step
        // by step across the slices (the scales of a slice go with its first
        // step), so the MFMAs of step s wait only for the loads up to step s.
        issue_weights();
    }
    // A barrier for the LDS stores only: __syncthreads would also wait for
    // every weight load to land before the first MFMA.
    lds_barrier();
    const int ar = (lane & 15) < nrows ? (lane & 15) : 0;  // rows past the tile repeat row 0

    // ONE: K is a single slab (the slice pointers are dead once issued)
    for (int q0 = 0; q0 < (ONE ? NQ : Q); q0 += NQ) {
        if (!ONE && q0 > 0) {
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int cb = 0; cb < CPW; ++cb) {
                    if (once)
                        slice_load<NQ, true>(w[m][cb], cbase[m][cb], sbase[m][cb], q0, 0, NQ);
                    else
                        slice_load<NQ, false>(w[m][cb], cbase[m][cb], sbase[m][cb], q0, 0, NQ);
                }
        }
#pragma unroll
        for (int s = 0; s < NQ; ++s) {
            uint4 b[NB][CPW];
            int sb[NB][CPW];
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int cb = 0; cb < CPW; ++cb) {
                    b[m][cb] = w[m][cb].q[s];
                    sb[m][cb] = (int)(w[m][cb].sc[s / 4] >> (8 * (s % 4)) & 0xFF);
                }
            mx_step<NB, CPW>(b, sb, ahi, alo, shi, slo, ld, nblk, q0 + s, ar, acc);
        }
    }

    // Epilogue: C[4*(l/16) + i][l%16].
    const int nw0 = (blockIdx.x * NW + wave) * 16 * CPW + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = (lane >> 4) * 4 + i;
        if (m >= nrows)
            continue;
        const int64_t pos = row0 + m;
#pragma unroll
        for (int cb = 0; cb < CPW; ++cb) {
            const int n = nw0 + 16 * cb;
            if (GU)
                p.out[(int64_t)pos * p.ldh + n] = f2bf(silu(acc[0][cb][i]) * acc[NB - 1][cb][i]);
            else
                p.out[(int64_t)pos * p.H + n] = f2bf(acc[0][cb][i]);
        }
    }
}

// Gate+up of decode rows (T <= 8) straight from the router's logits, with
// no permutation pass: one workgroup per (token t, slot j) pair and 16 * NW
// columns of both matrices.  Its waves read the token's logits and select
// its top k with the same wave selection as the routing kernels (so the
// same experts in the same order), take expert idx[t, j], quantise the
// token's activation row into LDS (hi / lo MXFP8, as the grouped kernel
// does) and stream their 16 columns' weights over the whole K.  The h row
// of pair t * k + j is written in pair order; the workgroup of pair (t, 0)
// and column block 0 also writes the token's indices and weights.  With
// decode rows every expert has about one row (a 6-row verify block puts its
// 48 pairs on ~47 experts), so grouping the pairs by expert first would
// save almost no weight bytes and costs a launch.  WF: the weights are
// requested right after the selection and the row is quantised while they
// are in flight (two workgroups' registers per SIMD pair), else the row is
// quantised first and three fit.
struct MxPairP {
    const uint16_t *x;            // [T, H]
    const uint8_t *xq;            // x quantised once per token (mxfp8.h records), or null
    const float *logits;          // [T, E], or with nparts 8 the router's parts [T, E, 8]
    const float *bias;            // [E] or null: added here when nparts is 8
    const uint8_t *c0, *c1;       // gate / up codes, packed
    const uint8_t *s0, *s1;       // their scales, packed
    uint16_t *h;                  // [T * k, I]: the row of pair t * k + j
    int32_t *idx;                 // [T, k]
    float *w;                     // [T, k]
    int T, H, E, k, I, nparts;
};

// PRE: the router quantised the token's row already (one record per token,
// shared by all its pairs and column blocks); the workgroup copies it into
// LDS - requested with the logits, stored once the weights are requested -
// instead of quantising the bf16 row itself.
template <int NW, int NQ, int PER, bool WF, bool PRE>
__global__ __launch_bounds__(64 * NW, (WF && !PRE) ? 2 : 3) void expert_mxfp4_pair(MxPairP p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int pr = blockIdx.y, t = pr / p.k, j = pr - t * p.k;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = p.H, nblk = K / 32, ld = K + MX_PAD;  // K = NQ * 128
    uint8_t *ahi = smem, *alo = ahi + ld, *shi = alo + ld, *slo = shi + nblk;

    // The token's logits and its activation row, requested together.  From
    // the split router's eight partial sums (32 contiguous bytes per logit)
    // the logit is their sum in segment order plus the bias, as router_small
    // forms it.
    float v[PER];
    if (p.nparts == 8) {
        wave_logits_from_parts<PER>(p.logits, p.bias, t, p.E, v);
    } else {
#pragma unroll
        for (int i = 0; i < PER; ++i)
            v[i] = lane + 64 * i < p.E ? p.logits[(int64_t)t * p.E + lane + 64 * i] : 0.0f;
    }
    const uint16_t *xrow = p.x + (int64_t)t * p.H;
    uint4 raw[4];
    constexpr int PP = (mx_rec_pieces(2048) + 64 * NW - 1) / (64 * NW);  // pieces per thread, K <= 2048
    uint4 rp[PRE ? PP : 1];
    if (PRE) {
        const uint8_t *rec = p.xq + (int64_t)t * mx_row_bytes(K);
#pragma unroll
        for (int i = 0; i < PP; ++i) {
            const int pc = tid + 64 * NW * i;
            int goff;
            uint8_t *dst;
            mx_rec_piece(pc, K, 0, ahi, alo, shi, slo, goff, dst);
            if (pc < mx_rec_pieces(K))
                rp[i] = *(const uint4 *)(rec + goff);
        }
    } else if (tid < nblk) {
        block_load(raw, xrow + tid * 32);
    }
    auto quantise = [&]() {
        if (tid < nblk)
            block_quantise(raw, 0, tid, K, ahi, alo, shi, slo);
        for (int q = tid + 64 * NW; q < nblk; q += 64 * NW) {  // rows wider than the workgroup
            uint4 r2[4];
            block_load(r2, xrow + q * 32);
            block_quantise(r2, 0, q, K, ahi, alo, shi, slo);
        }
    };
    if (!WF && !PRE)
        quantise();

    // The pair's expert: rank j of the token's selection (every wave selects).
    int my_e;
    uint32_t my_k;
    wave_topk_select<PER>(v, p.E, p.k, my_e, my_k);
    const int e = __builtin_amdgcn_readlane(my_e, j);

    // This wave's 16 columns of the gate and up matrices of expert e.
    const int64_t blk = (int64_t)e * (p.I / 16) + blockIdx.x * NW + wave;
    MxSlice<NQ> w[2];
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
        slice_load<NQ>(w[0], p.c0 + blk * NQ * 1024 + 16 * lane, p.s0 + (blk * 64 + lane) * NQ, 0,
                       s, s + 1);
        slice_load<NQ>(w[1], p.c1 + blk * NQ * 1024 + 16 * lane, p.s1 + (blk * 64 + lane) * NQ, 0,
                       s, s + 1);
        __builtin_amdgcn_sched_barrier(0);  // keep the issue order
    }
    if (PRE) {
#pragma unroll
        for (int i = 0; i < PP; ++i) {
            const int pc = tid + 64 * NW * i;
            int goff;
            uint8_t *dst;
            mx_rec_piece(pc, K, 0, ahi, alo, shi, slo, goff, dst);
            if (pc < mx_rec_pieces(K))
                *(uint4 *)dst = rp[i];
        }
    } else if (WF) {
        quantise();
    }
    if (j == 0 && blockIdx.x == 0 && wave == 0)
        wave_topk_weights(my_e, my_k, p.k, p.idx + (int64_t)t * p.k, p.w + (int64_t)t * p.k,
                          nullptr);
    lds_barrier();

    floatx4 acc[2][1];
    acc[0][0] = floatx4{0, 0, 0, 0};
    acc[1][0] = floatx4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
        uint4 b[2][1];
        int sb[2][1];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            b[m][0] = w[m].q[s];
            sb[m][0] = (int)(w[m].sc[s / 4] >> (8 * (s % 4)) & 0xFF);
        }
        mx_step<2, 1>(b, sb, ahi, alo, shi, slo, ld, nblk, s, 0, acc);
    }
    // Every row of C is the token's row (all lanes fed row 0), so every lane
    // stores its element 0 - four lanes the same value to each column -
    // and no lane condition can pull the MFMAs under a partial mask.
    const int n = (blockIdx.x * NW + wave) * 16 + (lane & 15);
    p.h[(int64_t)pr * p.I + n] = f2bf(silu(acc[0][0][0]) * acc[1][0][0]);
}

// Down projection and combine for decode rows, one workgroup per (16 CB
// output columns, token t): wave j takes pair (t, j) - its expert's 16 CB
// weight rows over the whole K, and its h row, quantised by the wave into its
// own LDS area - and rounds its outputs to bf16 as a staging row would be; then
// y[t] over those columns is the sum over j in order of w[t, j] times them,
// in fp32, rounded once: the same arithmetic as the down kernel followed by
// the combine, without the staging rows or the extra launch.  A few experts
// shared by two of the rows are streamed twice (a T=6 block has 47 experts
// for 48 pairs).
struct MxTokP {
    const uint16_t *h;           // [rows, ldh]
    const uint8_t *c, *s;        // down codes / scales, packed
    const int32_t *idx, *row_of;
    const float *w;
    uint16_t *y;                 // [T, H]
    int H, E, k, I, ldh;
};

template <int NQ, int CB>
__global__ __launch_bounds__(512) void expert_mxfp4_down_tok(MxTokP p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63, j = threadIdx.x >> 6;
    const int t = blockIdx.y, cb0 = blockIdx.x * CB;  // output columns 16*cb0 .. 16*(cb0+CB)-1
    const int K = p.I, nblk = K / 32, ld = K + MX_PAD;
    const int wst = (2 * ld + 2 * nblk + 15) & ~15;  // a wave's LDS area (16-byte aligned)
    const int pr = t * p.k + j;
    const int e = __builtin_amdgcn_readfirstlane(p.idx[pr]);
    // the h row of the pair: from the permutation, or the pair itself when
    // gate+up wrote its rows in pair order
    const int row = p.row_of ? __builtin_amdgcn_readfirstlane(p.row_of[pr]) : pr;
    uint8_t *ahi = smem + j * wst;
    uint8_t *alo = ahi + ld, *shi = alo + ld, *slo = shi + nblk;
    float *s_o = (float *)(smem + p.k * wst);  // [k][CB][64]
    // This pair's h row, one 32-element block per lane (nblk <= 64), and
    // the expert's 16-row weight blocks of these columns (scales first).
    // With one block per wave the weights are requested between the h row's
    // load and its quantisation, so they are in flight meanwhile (a wave's
    // loads complete in order for its wait counter: weights requested ahead
    // of the h row would make the quantiser wait for them too); with two,
    // holding them through the quantisation measured slower, and they
    // follow it (T=1, 2: down 10.5 -> 10.1 us; T=6, 8: 15.5 -> 16.0 us).
    uint4 raw[4];
    if (lane < nblk)
        block_load(raw, p.h + (int64_t)row * p.ldh + lane * 32);
    if (CB > 1 && lane < nblk)
        block_quantise(raw, 0, lane, K, ahi, alo, shi, slo);
    MxSlice<NQ> w[CB];
#pragma unroll
    for (int c = 0; c < CB; ++c) {
        const int64_t blk = (int64_t)e * (p.H / 16) + cb0 + c;
        slice_load<NQ>(w[c], p.c + blk * NQ * 1024 + 16 * lane, p.s + (blk * 64 + lane) * NQ, 0, 0,
                       NQ);
    }
    if (CB == 1 && lane < nblk)
        block_quantise(raw, 0, lane, K, ahi, alo, shi, slo);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's LDS rows
    __builtin_amdgcn_wave_barrier();
    floatx4 acc[1][CB];
#pragma unroll
    for (int c = 0; c < CB; ++c)
        acc[0][c] = floatx4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
        uint4 b[1][CB];
        int sb[1][CB];
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            b[0][c] = w[c].q[s];
            sb[0][c] = (int)(w[c].sc[s / 4] >> (8 * (s % 4)) & 0xFF);
        }
        mx_step<1, CB>(b, sb, ahi, alo, shi, slo, ld, nblk, s, 0, acc);
    }
    // Row 0 of C is in lanes 0..15, element 0 (column 16*cb + lane).  Every
    // lane stores its elements: a store under a lane condition would let the
    // compiler sink the MFMAs into that branch, where they would run with
    // part of the wave masked off.
#pragma unroll
    for (int c = 0; c < CB; ++c)
        s_o[(j * CB + c) * 64 + lane] = bf2f(f2bf(acc[0][c][0]));
    __syncthreads();
    if (j == 0 && lane < 16 * CB) {
        const int c = lane >> 4, n = lane & 15;
        float v = 0.0f;
        for (int q = 0; q < p.k; ++q)
            v = fmaf(p.w[t * p.k + q], s_o[(q * CB + c) * 64 + n], v);
        p.y[(int64_t)t * p.H + 16 * (cb0 + c) + n] = f2bf(v);
    }
}

// Repacking from the OCP row-major form: one thread per 16 code bytes, and
// one per scale byte.
__global__ void pack_codes(const uint8_t *__restrict__ in, uint8_t *__restrict__ out, int E, int N,
                           int K)
{
    const int Q = K / 128;
    const int64_t total = (int64_t)E * N * Q * 4;  // 16-byte chunks
    for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < total;
         o += (int64_t)gridDim.x * blockDim.x) {
        const int l = (int)(o & 63);
        const int64_t bq = o >> 6;  // (e*N/16 + nb) * Q + q
        const int q = (int)(bq % Q);
        const int64_t eb = bq / Q;  // e * N/16 + nb
        const int64_t row = eb * 16 + (l & 15);  // e * N + n
        const uint8_t *src = in + row * (K / 2) + (128 * q + 32 * (l >> 4)) / 2;
        *(uint4 *)(out + o * 16) = *(const uint4 *)src;
    }
}

__global__ void pack_scales(const uint8_t *__restrict__ in, uint8_t *__restrict__ out, int E, int N,
                            int K)
{
    const int Q = K / 128;
    const int64_t total = (int64_t)E * N * Q * 4;  // one byte per (row block, lane, step)
    for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < total;
         o += (int64_t)gridDim.x * blockDim.x) {
        const int q = (int)(o % Q);
        const int64_t bl = o / Q;  // (e*N/16 + nb) * 64 + l
        const int l = (int)(bl & 63);
        const int64_t row = (bl >> 6) * 16 + (l & 15);
        out[o] = in[row * (K / 32) + 4 * q + (l >> 4)];
    }
}

template <bool GU, int CPW, int NW, int NQ, bool ONE = false, bool WF = false>
void launch(const MxP &p, int N, int K, int tiles, hipStream_t st)
{
    const size_t lds = (size_t)p.cap * (2 * (K + MX_PAD) + 2 * (K / 32));
    // Dynamic LDS above the default limit is granted per size; a failure
    // here is left to the launch below to report.
    static size_t granted = 48 * 1024;
    if (lds > granted &&
        hipFuncSetAttribute((const void *)expert_mxfp4<GU, CPW, NW, NQ, ONE, WF>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) == hipSuccess)
        granted = lds;
    expert_mxfp4<GU, CPW, NW, NQ, ONE, WF>
        <<<dim3(N / (16 * CPW * NW), tiles), 64 * NW, lds, st>>>(p, p.ntiles, p.tiles, p.offsets,
                                                                   p.row_tok);
}

// Slab width (in 128-wide K steps): the largest of 16, 8, 6, 4, 2, 1 that
// divides K / 128; K of one slab of 16 or 6 steps has its own variant.
template <bool GU, int CPW, int NW>
void launch_k(const MxP &p, int N, int K, int tiles, hipStream_t st, bool wf = false)
{
    const int q = K / 128;
    if (NW == 2 && wf && q == 16)
        launch<GU, CPW, NW, 16, true, true>(p, N, K, tiles, st);
    else if (q == 16)
        launch<GU, CPW, NW, 16, true>(p, N, K, tiles, st);
    else if (q == 6)
        launch<GU, CPW, NW, 6, true>(p, N, K, tiles, st);
    else if (q % 16 == 0)
        launch<GU, CPW, NW, 16>(p, N, K, tiles, st);
    else if (q % 8 == 0)
        launch<GU, CPW, NW, 8>(p, N, K, tiles, st);
    else if (q % 6 == 0)
        launch<GU, CPW, NW, 6>(p, N, K, tiles, st);
    else if (q % 4 == 0)
        launch<GU, CPW, NW, 4>(p, N, K, tiles, st);
    else if (q % 2 == 0)
        launch<GU, CPW, NW, 2>(p, N, K, tiles, st);
    else
        launch<GU, CPW, NW, 1>(p, N, K, tiles, st);
}

template <bool GU>
void run(const ExpertArgs &a, hipStream_t st)
{
    MxP p;
    p.a = (const uint16_t *)(GU ? a.x : a.h);
    p.xq = GU ? a.xq : nullptr;
    p.c0 = (const uint8_t *)(GU ? a.w_gate : a.w_down);
    p.c1 = (const uint8_t *)(GU ? a.w_up : nullptr);
    p.s0 = GU ? a.s_gate : a.s_down;
    p.s1 = GU ? a.s_up : nullptr;
    p.row_tok = a.row_tok;
    p.offsets = a.offsets;
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
    const int tiles = GU ? a.max_tiles_gu : a.max_tiles_dc;
    if (tiles == 0)
        return;
    // N is a multiple of 128 (checked at the boundary).  Gate+up: 16 columns
    // of both matrices per wave; down: 32 columns per wave.  Tiles of at most
    // 8 rows (decode and verify) take two waves per workgroup: twice the
    // workgroups spread the weight bytes more evenly over the CUs (a CU
    // pulls its share at its own rate; at T=6 four waves leave a fifth of
    // the CUs a third more bytes than the rest), and the activation rows
    // each workgroup quantises are few.  Fuller tiles take four, which
    // quantise their rows once for 64 columns.  MOE_MX_NW (1, 2 or 4)
    // overrides the choice for tuning runs (read once per process).
    static const int forced = [] {
        const char *e = getenv("MOE_MX_NW");
        const int v = e ? atoi(e) : 0;
        return (v == 1 || v == 2 || v == 4) ? v : 0;
    }();
    constexpr int CPW = GU ? 1 : 2;
    const int nw = forced ? forced : p.cap <= 8 ? 2 : 4;
    // a single decode row: gate+up requests its weights right behind the
    // activation row (T=1: 11.7 -> 11.3 us; at T=2 the two-per-CU bound
    // costs more than the overlap saves, 13.9 -> 15.5 us)
    const bool wf = GU && p.cap <= 1;
    if (nw == 4)
        launch_k<GU, CPW, 4>(p, N, K, tiles, st);
    else if (nw == 2)
        launch_k<GU, CPW, 2>(p, N, K, tiles, st, wf);
    else
        launch_k<GU, CPW, 1>(p, N, K, tiles, st);
}

}  // namespace

void launch_pack_mxfp4(int E, int N, int K, const uint8_t *codes, const uint8_t *scales,
                       uint8_t *codes_out, uint8_t *scales_out, hipStream_t st)
{
    const int64_t chunks = (int64_t)E * N * (K / 128) * 4;
    const unsigned grid = (unsigned)std::min<int64_t>((chunks + 255) / 256, 65536);
    pack_codes<<<grid, 256, 0, st>>>(codes, codes_out, E, N, K);
    pack_scales<<<grid, 256, 0, st>>>(scales, scales_out, E, N, K);
}

bool down_combine_mxfp4_ok(const ExpertArgs &a)
{
    return a.wdt == W_MXFP4 && a.act == ACT_BF16 && a.T >= 1 && a.T <= 8 && a.I_shared == 0 &&
           a.k <= 8 && a.I % 128 == 0 && a.I <= 1024 && a.topk_idx && a.y;
}

constexpr int MX_DECODE_CUS = 256;  // compute units of an MI355X

template <int NQ>
static void down_tok(const MxTokP &p, int T, hipStream_t st)
{
    const size_t wst = (2 * (p.I + MX_PAD) + 2 * (p.I / 32) + 15) & ~(size_t)15;
    // Each workgroup costs its CU a fixed time (mostly its waves' h rows and
    // their latency), so once one 16-column block per wave would need more
    // workgroups than the device has CUs, a wave takes two blocks (measured
    // at H=2048, top-8: T=3 to 8 pass 14.4-22.6 -> 11.5-16.2 us; T <= 2
    // keep one block, which is slightly faster there).
    const int cb = (p.H / 16) * T > MX_DECODE_CUS && p.H % 32 == 0 ? 2 : 1;
    const size_t lds = (size_t)p.k * wst + (size_t)p.k * 64 * 4 * cb;
    if (cb == 2)
        expert_mxfp4_down_tok<NQ, 2><<<dim3(p.H / 32, T), 64 * p.k, lds, st>>>(p);
    else
        expert_mxfp4_down_tok<NQ, 1><<<dim3(p.H / 16, T), 64 * p.k, lds, st>>>(p);
}

void launch_down_combine_mxfp4(const ExpertArgs &a, hipStream_t st)
{
    MxTokP p;
    p.h = (const uint16_t *)a.h;
    p.c = (const uint8_t *)a.w_down;
    p.s = a.s_down;
    p.idx = a.topk_idx;
    p.row_of = a.row_of;
    p.w = a.topk_w;
    p.y = (uint16_t *)a.y;
    p.H = a.H;
    p.E = a.E;
    p.k = a.k;
    p.I = a.I;
    p.ldh = a.I;
    switch (a.I / 128) {  // the whole K in one slab (I <= 1024)
    case 1: down_tok<1>(p, a.T, st); break;
    case 2: down_tok<2>(p, a.T, st); break;
    case 3: down_tok<3>(p, a.T, st); break;
    case 4: down_tok<4>(p, a.T, st); break;
    case 5: down_tok<5>(p, a.T, st); break;
    case 6: down_tok<6>(p, a.T, st); break;
    case 7: down_tok<7>(p, a.T, st); break;
    default: down_tok<8>(p, a.T, st); break;
    }
}

namespace {

template <int NQ, int PER>
void pair_launch(const MxPairP &p, hipStream_t st)
{
    const size_t lds = (size_t)mx_row_bytes(p.H);
    constexpr int NW = 2;
    const dim3 grid(p.I / (16 * NW), p.T * p.k);
    if (p.xq)  // quantised rows from the router: weights requested before the row lands
        expert_mxfp4_pair<NW, NQ, PER, true, true><<<grid, 64 * NW, lds, st>>>(p);
    else if (p.T == 1)  // a single row: weights first (the grid is far smaller than the chip)
        expert_mxfp4_pair<NW, NQ, PER, true, false><<<grid, 64 * NW, lds, st>>>(p);
    else
        expert_mxfp4_pair<NW, NQ, PER, false, false><<<grid, 64 * NW, lds, st>>>(p);
}

template <int NQ>
void pair_per(const MxPairP &p, hipStream_t st)
{
    switch (topk_per(p.E)) {
    case 1: pair_launch<NQ, 1>(p, st); break;
    case 2: pair_launch<NQ, 2>(p, st); break;
    case 4: pair_launch<NQ, 4>(p, st); break;
    case 8: pair_launch<NQ, 8>(p, st); break;
    default: pair_launch<NQ, 16>(p, st); break;
    }
}

}  // namespace

bool gate_up_mxfp4_pair_ok(const ExpertArgs &a)
{
    const int q = a.H / 128;
    return a.wdt == W_MXFP4 && a.act == ACT_BF16 && a.T >= 1 && a.T <= 8 && a.I_shared == 0 &&
           a.k <= 8 && a.I % 128 == 0 && a.I <= 1024 && a.E <= 1023 && a.topk_idx &&
           a.topk_w && a.y && (q == 1 || q == 2 || q == 4 || q == 6 || q == 8 || q == 16);
}

void launch_gate_up_mxfp4_pair(const ExpertArgs &a, const float *logits, const float *bias,
                               int nparts, hipStream_t st)
{
    MxPairP p;
    p.x = (const uint16_t *)a.x;
    p.xq = a.xq;
    p.logits = logits;
    p.bias = bias;
    p.nparts = nparts;
    p.c0 = (const uint8_t *)a.w_gate;
    p.c1 = (const uint8_t *)a.w_up;
    p.s0 = a.s_gate;
    p.s1 = a.s_up;
    p.h = (uint16_t *)a.h;
    p.idx = const_cast<int32_t *>(a.topk_idx);
    p.w = const_cast<float *>(a.topk_w);
    p.T = a.T;
    p.H = a.H;
    p.E = a.E;
    p.k = a.k;
    p.I = a.I;
    switch (a.H / 128) {
    case 1: pair_per<1>(p, st); break;
    case 2: pair_per<2>(p, st); break;
    case 4: pair_per<4>(p, st); break;
    case 6: pair_per<6>(p, st); break;
    case 8: pair_per<8>(p, st); break;
    default: pair_per<16>(p, st); break;
    }
}

void launch_gate_up_mxfp4(const ExpertArgs &a, hipStream_t st) { run<true>(a, st); }
void launch_down_mxfp4(const ExpertArgs &a, hipStream_t st) { run<false>(a, st); }

}  // namespace moe
