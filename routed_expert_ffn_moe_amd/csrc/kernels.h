// Launchers of the gfx950 kernels, called by the host orchestration in
// moe_api.cpp.  All pointers are device pointers; every launcher is
// asynchronous on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace moe {

enum { ACT_F32 = 0, ACT_BF16 = 1 };
enum { W_F32 = 0, W_BF16 = 1, W_MXFP4 = 2 };

struct RouterArgs {
    const void *x;        // [T, H] act
    const void *wr;       // [E, H] act
    const float *bias;    // [E] or null
    int nparts;           // 8: logits holds the split router's parts [T][E][8] (route_small)
    float *logits;        // [T, E] workspace
    int32_t *idx;         // [T, k]
    float *w;             // [T, k]
    int32_t *ticket;      // route_small's counter, cleared by router_small (or null)
    // With xq set, router_small also writes every token row as an MXFP8
    // hi / lo record of mx_row_bytes(H) bytes (mxfp8.h) at xq + t * that,
    // for the MXFP4 kernels; xq is ignored by the other routers, which
    // leave the expert kernels to quantise their rows themselves.
    uint8_t *xq;
    // With hist set, the segmented router also counts the pairs of each
    // permutation block per expert into hist [nblk, E] (cleared first).
    int32_t *hist;
    int nhist;
    int T, H, E, k, act;
};
void launch_router(const RouterArgs &a, hipStream_t st);         // logits + top-k
void launch_router_logits(const RouterArgs &a, hipStream_t st);  // logits only
// Logit planes the router writes for a pass: 8 (partial sums of the eighths
// of K, when the segmented router applies) or 1; the logits workspace holds
// that many [T, E] fp32 planes.
int router_parts(int T, int H, int E, int act);

// Permutation of one pass: counts, offsets and the grouped order of the
// (t, j) pairs, plus the GEMM tile lists.  Group E is the shared expert
// (all T tokens, in token order) when `shared` is set.
struct PermuteArgs {
    const int32_t *idx;   // [T, k]
    int32_t *blk;         // [nblk, E] workspace
    int32_t *counts;      // [E + 1]
    int32_t *offsets;     // [E + 2]
    int32_t *row_src;     // [T*k + T] pair id of each grouped row
    int32_t *row_tok;     // [T*k + T] token of each grouped row
    int32_t *row_of;      // [T*k] grouped row of each pair (inverse of row_src)
    Tile *tiles_a;        // tile list for row-block size bm_a
    int32_t *ntiles_a;
    Tile *tiles_b;        // tile list for row-block size bm_b
    int32_t *ntiles_b;
    int bm_a, bm_b;
    // Optional work-item lists of the streaming GEMMs (expert-major, then
    // column tile, then row tile): {group, first row, rows, first column}.
    int4 *items_a, *items_b;
    int ntn_a, ntn_b, max_tiles_a, max_tiles_b, wrows_a, wrows_b;
    int hist_done;        // blk already holds the per-block counts (from the router)
    int T, E, k, shared;
};
constexpr int PERMUTE_PAIRS_PER_BLOCK = 1024;  // pairs per histogram / scatter block
int permute_blocks(int n_pairs);  // number of histogram blocks
void launch_permute(const PermuteArgs &a, hipStream_t st);

// Short passes (route_small.hip): router logits, top-k and the whole
// permutation in two launches.
bool route_small_ok(int T, int k, int E, int H, int act);
int router_small_rw(int E, int H, int act);  // waves of router_small, 0 if it does not apply
// router_small can write the MXFP8 row records (RouterArgs::xq) for this
// shape, and the bytes they take for T tokens.
bool router_xq_ok(int E, int H, int act);
size_t router_xq_bytes(int T, int H);
void launch_router_small(const RouterArgs &r, hipStream_t st);  // logits only
// Short passes: the eight K-segment partial sums of router_small's logits as
// [T][E][8] floats at r.logits (no bias), for the decode gate+up kernel or
// route_small to add (T <= 64, bf16, router_small with 8 waves applicable);
// clears r.ticket (if given) as router_small does.
bool router_split_ok(int T, int E, int H, int act);
void launch_router_split(const RouterArgs &r, hipStream_t st);
void launch_route_small(const RouterArgs &r, const PermuteArgs &a, hipStream_t st);  // top-k + permutation

// Grouped gate+up GEMM with the SwiGLU epilogue: h[row] = silu(x_t Wg^T) *
// (x_t Wu^T) for every grouped row; and the grouped down GEMM writing
// stage[row] = h[row] Wd^T, one staging row per grouped row.
struct ExpertArgs {
    const void *x;                           // [T, H] act
    const uint8_t *xq;                       // x as MXFP8 row records (router_small), or null
    const void *w_gate, *w_up, *w_down;      // routed weights (codes for MXFP4)
    const uint8_t *s_gate, *s_up, *s_down;   // MXFP4 scales
    const void *sh_gate, *sh_up, *sh_down;   // shared expert (act dtype)
    const int32_t *row_src;                  // [rows] pair id
    const int32_t *row_tok;                  // [rows] token
    const int32_t *offsets;                  // [E + 2]
    const float *topk_w;                     // [T*k]
    void *h;                                 // [rows, max(I, I_shared)] act
    void *stage;                             // [rows, H] act
    const Tile *tiles_gu;
    const int32_t *ntiles_gu;
    const Tile *tiles_dc;
    const int32_t *ntiles_dc;
    const int4 *items_gu, *items_dc;       // work items of the streaming kernels
    const int32_t *topk_idx;                 // [T*k] expert of each pair
    const int32_t *row_of;                   // [T*k] grouped row of each pair
    void *y;                                 // [T, H] act: the layer output
    int max_tiles_gu, max_tiles_dc;
    int T, H, E, k, I, I_shared, act, wdt;
    int shape_T;  // tokens of a full pass: selects the tile shape
};
void launch_gate_up(const ExpertArgs &a, hipStream_t st);
void launch_down(const ExpertArgs &a, hipStream_t st);
int gemm_bm_gu(const ExpertArgs &a);  // row-block sizes of the tile lists
int gemm_bm_dc(const ExpertArgs &a);

// Weight-streaming bf16 kernels (expert_stream.hip), used when the shapes fit.
bool stream_ok(const ExpertArgs &a, bool gu);
int stream_bm(const ExpertArgs &a);
int stream_ntn(const ExpertArgs &a, bool gu);  // column tiles (0 if not streaming)
int stream_wrows(const ExpertArgs &a, bool gu);  // weight rows per streaming work item
void launch_stream(const ExpertArgs &a, bool gu, hipStream_t st);

// MXFP4 expert weights (bf16 activations, no shared expert).
int mxfp4_bm();
void launch_gate_up_mxfp4(const ExpertArgs &a, hipStream_t st);
void launch_down_mxfp4(const ExpertArgs &a, hipStream_t st);
// Decode rows (T <= 8, top_k <= 8, MXFP4, no shared expert, I <= 1024): the down
// projection of every (t, j) pair and the weighted combine in one kernel,
// writing y directly (the staging rows and the combine pass are skipped).
bool down_combine_mxfp4_ok(const ExpertArgs &a);
void launch_down_combine_mxfp4(const ExpertArgs &a, hipStream_t st);  // row_of null: pair order
// Decode rows without the permutation: gate+up of every (t, j) pair taking
// its expert from the router's logits (the same selection as the routing
// kernels), h in pair order, and the indices and weights into topk_idx /
// topk_w.  Followed by launch_down_combine_mxfp4 with row_of null.
bool gate_up_mxfp4_pair_ok(const ExpertArgs &a);
void launch_gate_up_mxfp4_pair(const ExpertArgs &a, const float *logits, const float *bias,
                               int nparts, hipStream_t st);
// OCP row-major MXFP4 (codes [E, N, K/2], scales [E, N, K/32]) into the
// packed layout the MXFP4 kernels read.
void launch_pack_mxfp4(int E, int N, int K, const uint8_t *codes, const uint8_t *scales,
                       uint8_t *codes_out, uint8_t *scales_out, hipStream_t st);

// y[t] = sum_j w[t*k + j] * stage[row_of[t*k + j]] (+ stage[T*k + t]) in
// j order: the routing-weight scale and the deterministic combine.
struct CombineArgs {
    const void *stage;
    const int32_t *row_of;
    const float *topk_w;
    void *y;
    int T, H, k, shared, act;
};
void launch_combine(const CombineArgs &a, hipStream_t st);

// Row-major bf16 [E, N, K] into the packed layout the bf16 GEMMs read
// (packed_bf16_off in common.h).
void launch_pack_bf16(int E, int N, int K, const uint16_t *w, uint16_t *out, hipStream_t st);

// Records `what` as the calling thread's last error (moe_last_error) and
// returns `code`: for entry points outside moe_api.cpp.
int api_fail(int code, const char *what);

// Measurement aids (probe.hip): the device's HBM read (sequential and
// scattered), MXFP4 dequantisation stream and bf16 MFMA ceilings.
void launch_probe_read(const void *buf, size_t bytes, int *sink, hipStream_t st);
void launch_probe_mfma(int waves, int iters, int *sink, hipStream_t st);
void launch_probe_gather(const void *pool, int pool_chunks, const int32_t *order, int nchunks,
                         size_t chunk_bytes, int wgs, int *sink, hipStream_t st);
void launch_probe_mxfp4(const void *codes, const uint8_t *scales, size_t nblocks, int wgs,
                        float *out, hipStream_t st);

}  // namespace moe
