// Grouped expert GEMMs on bf16 MFMA (gfx950), the fp32 variants, and the
// deterministic combine.
//
//  gate+up: for the rows of one expert, G = X Wg^T and U = X Wu^T; the
//           epilogue forms h = silu(G) * U and rounds it once to bf16
//           ("Jetson Orin Nano MoE ... expert cache", re-check and gate-first
//           sections: SwiGLU(gate, up), gate is the SiLU branch; "DeepSeek
//           V4.1F Q4 with native DSpark MTP", decode paragraph: fused
//           gate+up+SwiGLU and bf16 rounding inside the producing kernel).
//  down:    O = h Wd^T, rounded once into the grouped row's own staging row,
//           so no two pairs ever share an output location (same Jetson page,
//           nondeterminism section).
//  combine: y_t = sum_j w_tj * stage[row of (t, j)] (+ shared row) in fixed j
//           order: the routing-weight scale and the deterministic sum.
//
// A workgroup owns one tile of the permutation's tile list (one expert, up to
// BM consecutive grouped rows) and BN output columns.  X rows are gathered
// through row_src while staging the A tile; weights stream through double
// buffered LDS tiles, each weight element read once per tile.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace moe {

namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row (bf16): 144 bytes, conflict-free b128 reads

struct GemmP {
    const uint16_t *x;        // GU: activations [T, H]; DC: h [rows, ldh]
    const uint16_t *w0, *w1;  // routed: gate/up (GU) or down (DC), [E, N, K]
    const uint16_t *s0, *s1;  // shared expert matrices
    const int32_t *row_src, *offsets;
    const float *topk_w;
    uint16_t *out;            // GU: h; DC: stage
    const Tile *tiles;
    const int32_t *ntiles;
    int T, H, E, k, I, Is, ldh;
};

template <int BM, int BN, bool GU>
__global__ __launch_bounds__(256) void expert_gemm_bf16(GemmP p)
{
    constexpr int NB = GU ? 2 : 1;     // weight matrices per tile
    constexpr int WNC = BN / 4;        // columns per wave
    constexpr int MB = BM / 16;        // 16-row MFMA blocks
    constexpr int NBL = WNC / 16;      // 16-col MFMA blocks per wave and matrix
    constexpr int ACH = BM * BK / 8 / 256;       // A 16-byte chunks per thread
    constexpr int BCH = NB * BN * BK / 8 / 256;  // B chunks per thread
    static_assert(BM % 16 == 0 && WNC % 16 == 0, "tile shape");
    static_assert(ACH * 256 * 8 == BM * BK || BM == 16, "A chunking");

    __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][NB * BN * LDK];

    if ((int)blockIdx.y >= *p.ntiles)
        return;
    const Tile tile = p.tiles[blockIdx.y];
    const int g = tile.g, row0 = tile.row0;
    const bool routed = g < p.E;
    const int nrows = min(BM, p.offsets[g + 1] - row0);
    const int n_pairs = p.T * p.k;
    const int N = GU ? (routed ? p.I : p.Is) : p.H;
    const int K = GU ? p.H : (routed ? p.I : p.Is);
    const int n0 = blockIdx.x * BN;
    if (n0 >= N)
        return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t wstride = (int64_t)N * K;
    const uint16_t *W0 = routed ? p.w0 + (int64_t)g * wstride : p.s0;
    const uint16_t *W1 = GU ? (routed ? p.w1 + (int64_t)g * wstride : p.s1) : nullptr;

    // Global source of each A / B chunk this thread stages.
    constexpr int ACH_ = ACH > 0 ? ACH : 1;
    const uint16_t *asrc[ACH_];
    int aoff[ACH_];
    bool aon[ACH_];
#pragma unroll
    for (int i = 0; i < ACH_; ++i) {
        int c = tid + 256 * i;
        int r = c / (BK / 8), c8 = c % (BK / 8);
        aon[i] = (ACH > 0) || (c < BM * BK / 8);
        int rr = min(r, nrows - 1);
        int pos = row0 + rr;
        const uint16_t *row;
        if (GU) {
            int t = pair_token(p.row_src[pos], n_pairs, p.k);
            row = p.x + (int64_t)t * p.H;
        } else {
            row = p.x + (int64_t)pos * p.ldh;
        }
        asrc[i] = row + c8 * 8;
        aoff[i] = r * LDK + c8 * 8;
    }
    const uint16_t *bsrc[BCH];
    int boff[BCH];
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
        int c = tid + 256 * i;
        int m = c / (BN * BK / 8);
        int rem = c % (BN * BK / 8);
        int r = rem / (BK / 8), c8 = rem % (BK / 8);
        const uint16_t *W = (m == 0) ? W0 : W1;
        bsrc[i] = W + packed_bf16_off(n0 + r, c8 * 8, K);
        boff[i] = (m * BN + r) * LDK + c8 * 8;
    }

    floatx4 acc[NB][MB][NBL];
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int a = 0; a < MB; ++a)
#pragma unroll
            for (int b = 0; b < NBL; ++b)
                acc[m][a][b] = floatx4{0, 0, 0, 0};

    uint4 ra[ACH_], rb[BCH];
    auto gload = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < ACH_; ++i)
            if (aon[i])
                ra[i] = *(const uint4 *)(asrc[i] + k0);
#pragma unroll
        for (int i = 0; i < BCH; ++i)
            rb[i] = *(const uint4 *)(bsrc[i] + (int64_t)k0 * 32);  // k0 / 32 steps of 1024
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < ACH_; ++i)
            if (aon[i])
                *(uint4 *)(&sA[buf][aoff[i]]) = ra[i];
#pragma unroll
        for (int i = 0; i < BCH; ++i)
            *(uint4 *)(&sB[buf][boff[i]]) = rb[i];
    };

    const int nk = K / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    const int fr = lane & 15, fk = (lane >> 4) * 8;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk)
            gload(kt + 1);
#pragma unroll
        for (int ks = 0; ks < BK; ks += 32) {
            bf16x8 af[MB];
#pragma unroll
            for (int a = 0; a < MB; ++a)
                af[a] = as_bf16x8(*(const uint4 *)(&sA[cur][(a * 16 + fr) * LDK + ks + fk]));
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int b = 0; b < NBL; ++b) {
                    bf16x8 bfr = as_bf16x8(*(const uint4 *)(
                        &sB[cur][(m * BN + wave * WNC + b * 16 + fr) * LDK + ks + fk]));
#pragma unroll
                    for (int a = 0; a < MB; ++a)
                        acc[m][a][b] = mfma16(af[a], bfr, acc[m][a][b]);
                }
        }
        if (kt + 1 < nk)
            sstore(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = a * 16 + (lane >> 4) * 4 + i;
            if (m >= nrows)
                continue;
            const int pos = row0 + m;
            if (GU) {
#pragma unroll
                for (int b = 0; b < NBL; ++b) {
                    const int n = n0 + wave * WNC + b * 16 + fr;
                    float hv = silu(acc[0][a][b][i]) * acc[GU ? 1 : 0][a][b][i];
                    p.out[(int64_t)pos * p.ldh + n] = f2bf(hv);
                }
            } else {
#pragma unroll
                for (int b = 0; b < NBL; ++b) {
                    const int n = n0 + wave * WNC + b * 16 + fr;
                    p.out[(int64_t)pos * p.H + n] = f2bf(acc[0][a][b][i]);
                }
            }
        }
}

// ---- fp32 path: plain dot products, one thread per (row, column) --------

struct GemmF32 {
    const float *x, *w0, *w1, *s0, *s1;
    const int32_t *row_src, *offsets;
    const float *topk_w;
    float *out;
    const Tile *tiles;
    const int32_t *ntiles;
    int T, H, E, k, I, Is, ldh;
};

// Tile of 16 rows x 16 columns per 256-thread workgroup.
template <bool GU>
__global__ __launch_bounds__(256) void expert_gemm_f32(GemmF32 p)
{
    if ((int)blockIdx.y >= *p.ntiles)
        return;
    const Tile tile = p.tiles[blockIdx.y];
    const int g = tile.g, row0 = tile.row0;
    const bool routed = g < p.E;
    const int nrows = min(16, p.offsets[g + 1] - row0);
    const int n_pairs = p.T * p.k;
    const int N = GU ? (routed ? p.I : p.Is) : p.H;
    const int K = GU ? p.H : (routed ? p.I : p.Is);
    const int r = threadIdx.x / 16;
    const int n = blockIdx.x * 16 + threadIdx.x % 16;
    if (r >= nrows || n >= N)
        return;
    const int pos = row0 + r;
    const int64_t wstride = (int64_t)N * K;
    if (GU) {
        const float *wg = (routed ? p.w0 + g * wstride : p.s0) + (int64_t)n * K;
        const float *wu = (routed ? p.w1 + g * wstride : p.s1) + (int64_t)n * K;
        const int t = pair_token(p.row_src[pos], n_pairs, p.k);
        const float *a = p.x + (int64_t)t * p.H;
        float gs = 0.0f, us = 0.0f;
        for (int kk = 0; kk < K; ++kk) {
            gs = fmaf(a[kk], wg[kk], gs);
            us = fmaf(a[kk], wu[kk], us);
        }
        p.out[(int64_t)pos * p.ldh + n] = silu(gs) * us;
    } else {
        const float *wd = (routed ? p.w0 + g * wstride : p.s0) + (int64_t)n * K;
        const float *a = p.x + (int64_t)pos * p.ldh;
        float s = 0.0f;
        for (int kk = 0; kk < K; ++kk)
            s = fmaf(a[kk], wd[kk], s);
        p.out[(int64_t)pos * p.H + n] = s;
    }
}

// ---- combine ---------------------------------------------------------------

// y[t, c] = sum_j w[t*k + j] * stage[row_of[t*k + j], c] (+ stage[T*k + t, c]),
// fp32 sum in j order, rounded once.  Each thread handles 8 consecutive
// columns of one token; the row indices and weights of its (at most KM)
// rows are read first and then all the rows' 16-byte pieces together, so
// a thread's loads are in flight at once rather than one row at a time.
template <int KM>
__global__ __launch_bounds__(256) void combine_bf16(const uint16_t *__restrict__ stage,
                                                    const int32_t *__restrict__ row_of,
                                                    const float *__restrict__ topk_w,
                                                    uint16_t *__restrict__ y, int T, int H, int k,
                                                    int shared)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int per_row = H / 8;
    if (i >= (int64_t)T * per_row)
        return;
    const int t = (int)(i / per_row), c8 = (int)(i % per_row) * 8;
    const int n_rows = k + (shared ? 1 : 0);  // <= KM
    int64_t row[KM];
    float w[KM];
    if (per_row % 256 == 0) {
        // a workgroup lies within one token: its rows and weights are
        // uniform and come as scalar loads, off the vector memory path
        const int tu = __builtin_amdgcn_readfirstlane(t);
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            row[j] = j < k ? __builtin_amdgcn_readfirstlane(row_of[(int64_t)tu * k + j])
                           : (int64_t)T * k + tu;
            w[j] = j < k ? __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                         __builtin_bit_cast(int, topk_w[(int64_t)tu * k + j])))
                         : 1.0f;
        }
    } else {
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            row[j] = j < k ? row_of[(int64_t)t * k + j] : (int64_t)T * k + t;
            w[j] = j < k ? topk_w[(int64_t)t * k + j] : 1.0f;
        }
    }
    uint4 v[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j)
        if (j < n_rows)
        {
            // each staging row is read once: non-temporal (T=8192 with a
            // shared expert: 103.6 -> 91.8 us; T=2048: 16.5 -> 16.2 us)
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 t4 = __builtin_nontemporal_load((const u32x4 *)(stage + row[j] * H + c8));
            v[j] = uint4{t4[0], t4[1], t4[2], t4[3]};
        }
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < KM; ++j)
        if (j < n_rows) {
            const uint32_t w4[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = fmaf(w[j], bf2f((uint16_t)(w4[q] & 0xFFFF)), acc[2 * q]);
                acc[2 * q + 1] = fmaf(w[j], bf2f((uint16_t)(w4[q] >> 16)), acc[2 * q + 1]);
            }
        }
    *(uint4 *)(y + (int64_t)t * H + c8) =
        uint4{pack_bf2(acc[0], acc[1]), pack_bf2(acc[2], acc[3]), pack_bf2(acc[4], acc[5]),
              pack_bf2(acc[6], acc[7])};
}

__global__ __launch_bounds__(256) void combine_f32(const float *__restrict__ stage,
                                                   const int32_t *__restrict__ row_of,
                                                   const float *__restrict__ topk_w,
                                                   float *__restrict__ y, int T, int H, int k,
                                                   int shared)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * H)
        return;
    const int t = (int)(i / H), c = (int)(i % H);
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) {
        const int64_t q = (int64_t)t * k + j;
        acc = fmaf(topk_w[q], stage[(int64_t)row_of[q] * H + c], acc);
    }
    if (shared)
        acc += stage[((int64_t)T * k + t) * H + c];
    y[i] = acc;
}

// Tile shapes by the average rows per expert (the grids are upper bounds).
struct Shape {
    int bm, bn;
};
Shape pick(const ExpertArgs &a, bool gu)
{
    if (a.act == ACT_F32)
        return {16, 16};
    const int64_t avg = (int64_t)a.shape_T * a.k / a.E;
    const bool n128 = gu ? (a.I % 128 == 0 && a.I_shared % 128 == 0) : (a.H % 128 == 0);
    if (avg <= 16)
        return {16, 64};
    if (avg <= 64 || !n128)
        return {64, 64};
    return {128, 128};
}

template <int BM, int BN, bool GU>
void run_bf16(const ExpertArgs &a, hipStream_t st)
{
    GemmP p;
    p.x = (const uint16_t *)(GU ? a.x : a.h);
    p.w0 = (const uint16_t *)(GU ? a.w_gate : a.w_down);
    p.w1 = (const uint16_t *)(GU ? a.w_up : nullptr);
    p.s0 = (const uint16_t *)(GU ? a.sh_gate : a.sh_down);
    p.s1 = (const uint16_t *)(GU ? a.sh_up : nullptr);
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
    p.Is = a.I_shared;
    p.ldh = a.I > a.I_shared ? a.I : a.I_shared;
    const int N = GU ? (a.I > a.I_shared ? a.I : a.I_shared) : a.H;
    dim3 grid((N + BN - 1) / BN, GU ? a.max_tiles_gu : a.max_tiles_dc);
    if (grid.y == 0)
        return;
    expert_gemm_bf16<BM, BN, GU><<<grid, 256, 0, st>>>(p);
}

template <bool GU>
void run_f32(const ExpertArgs &a, hipStream_t st)
{
    GemmF32 p;
    p.x = (const float *)(GU ? a.x : a.h);
    p.w0 = (const float *)(GU ? a.w_gate : a.w_down);
    p.w1 = (const float *)(GU ? a.w_up : nullptr);
    p.s0 = (const float *)(GU ? a.sh_gate : a.sh_down);
    p.s1 = (const float *)(GU ? a.sh_up : nullptr);
    p.row_src = a.row_src;
    p.offsets = a.offsets;
    p.topk_w = a.topk_w;
    p.out = (float *)(GU ? a.h : a.stage);
    p.tiles = GU ? a.tiles_gu : a.tiles_dc;
    p.ntiles = GU ? a.ntiles_gu : a.ntiles_dc;
    p.T = a.T;
    p.H = a.H;
    p.E = a.E;
    p.k = a.k;
    p.I = a.I;
    p.Is = a.I_shared;
    p.ldh = a.I > a.I_shared ? a.I : a.I_shared;
    const int N = GU ? (a.I > a.I_shared ? a.I : a.I_shared) : a.H;
    dim3 grid((N + 15) / 16, GU ? a.max_tiles_gu : a.max_tiles_dc);
    if (grid.y == 0)
        return;
    expert_gemm_f32<GU><<<grid, 256, 0, st>>>(p);
}

template <bool GU>
void dispatch(const ExpertArgs &a, hipStream_t st)
{
    if (a.act == ACT_F32) {
        run_f32<GU>(a, st);
        return;
    }
    const Shape s = pick(a, GU);
    if (s.bm == 16)
        run_bf16<16, 64, GU>(a, st);
    else if (s.bm == 64)
        run_bf16<64, 64, GU>(a, st);
    else
        run_bf16<128, 128, GU>(a, st);
}

}  // namespace

int gemm_bm_gu(const ExpertArgs &a)
{
    if (stream_ok(a, true))
        return stream_bm(a);
    return a.wdt == W_MXFP4 ? mxfp4_bm() : pick(a, true).bm;
}
int gemm_bm_dc(const ExpertArgs &a)
{
    if (stream_ok(a, false))
        return stream_bm(a);
    return a.wdt == W_MXFP4 ? mxfp4_bm() : pick(a, false).bm;
}

void launch_gate_up(const ExpertArgs &a, hipStream_t st)
{
    if (stream_ok(a, true))
        launch_stream(a, true, st);
    else if (a.wdt == W_MXFP4)
        launch_gate_up_mxfp4(a, st);
    else
        dispatch<true>(a, st);
}

void launch_down(const ExpertArgs &a, hipStream_t st)
{
    if (stream_ok(a, false))
        launch_stream(a, false, st);
    else if (a.wdt == W_MXFP4)
        launch_down_mxfp4(a, st);
    else
        dispatch<false>(a, st);
}

namespace {

// Row-major [E, N, K] bf16 into the packed layout: one thread per 16 bytes
// out (the 8 elements of one lane of one block).
__global__ void pack_bf16(const uint16_t *__restrict__ in, uint16_t *__restrict__ out, int E, int N,
                          int K)
{
    const int64_t total = (int64_t)E * N * (K / 8);
    for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < total;
         o += (int64_t)gridDim.x * blockDim.x) {
        const int l = (int)(o & 63);
        const int c = (int)((o >> 6) & 1);
        const int64_t gs = o >> 7;  // (e * N/32 + g) * K/32 + s
        const int s = (int)(gs % (K / 32));
        const int64_t eg = gs / (K / 32);  // e * N/32 + g
        const int r = l & 15, b = l >> 4;
        const int64_t row = eg * 32 + 8 * (r >> 2) + 4 * c + (r & 3);  // e * N + n
        *(uint4 *)(out + o * 8) = *(const uint4 *)(in + row * K + 32 * s + 8 * b);
    }
}

}  // namespace

void launch_pack_bf16(int E, int N, int K, const uint16_t *w, uint16_t *out, hipStream_t st)
{
    const int64_t chunks = (int64_t)E * N * (K / 8);
    const unsigned grid = (unsigned)std::min<int64_t>((chunks + 255) / 256, 65536);
    pack_bf16<<<grid, 256, 0, st>>>(w, out, E, N, K);
}

void launch_combine(const CombineArgs &a, hipStream_t st)
{
    if (a.T == 0)
        return;
    if (a.act == ACT_BF16) {
        const int64_t n = (int64_t)a.T * (a.H / 8);
        const unsigned nb = (unsigned)((n + 255) / 256);
        if (a.k + (a.shared ? 1 : 0) <= 9)
            combine_bf16<9><<<nb, 256, 0, st>>>((const uint16_t *)a.stage, a.row_of, a.topk_w,
                                               (uint16_t *)a.y, a.T, a.H, a.k, a.shared);
        else
            combine_bf16<17><<<nb, 256, 0, st>>>((const uint16_t *)a.stage, a.row_of, a.topk_w,
                                                (uint16_t *)a.y, a.T, a.H, a.k, a.shared);
    } else {
        const int64_t n = (int64_t)a.T * a.H;
        combine_f32<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
            (const float *)a.stage, a.row_of, a.topk_w, (float *)a.y, a.T, a.H, a.k, a.shared);
    }
}

}  // namespace moe
