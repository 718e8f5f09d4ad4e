// C ABI of the MoE layer: argument checks, workspace carving and the
// per-chunk launch sequence (router -> permutation -> gate+up -> down ->
// combine), all asynchronous on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

thread_local char g_last[256] = "";

int fail(int code, const char *what)
{
    std::snprintf(g_last, sizeof g_last, "%s", what);
    return code;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Device check: gfx950 only, cached per device.
int check_device()
{
    static std::mutex mu;
    static int cached[64];
    static bool init[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return fail(MOE_EHIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lock(mu);
    if (!init[dev]) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(MOE_EHIP, "hipGetDeviceProperties failed");
        cached[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? MOE_OK : MOE_EUNSUPPORTED;
        init[dev] = true;
    }
    if (cached[dev] != MOE_OK)
        return fail(cached[dev], "device is not gfx950");
    return MOE_OK;
}

int check_shape(const moe_shape_t *s)
{
    if (!s)
        return fail(MOE_EINVAL, "shape is NULL");
    if (s->T < 0)
        return fail(MOE_EINVAL, "T < 0");
    if (s->H <= 0 || s->H % 64)
        return fail(MOE_EINVAL, "H must be a positive multiple of 64");
    if (s->E < 1 || s->E > 1023)
        return fail(MOE_EINVAL, "E must be in 1..1023");
    if (s->top_k < 1 || s->top_k > s->E || s->top_k > 16)
        return fail(MOE_EINVAL, "top_k must be in 1..min(E, 16)");
    if (s->I <= 0 || s->I % 64)
        return fail(MOE_EINVAL, "I must be a positive multiple of 64");
    if (s->I_shared < 0 || s->I_shared % 64)
        return fail(MOE_EINVAL, "I_shared must be 0 or a positive multiple of 64");
    if (s->chunk_T < 0)
        return fail(MOE_EINVAL, "chunk_T < 0");
    const bool f32 = s->act_dtype == MOE_F32 && s->w_dtype == MOE_F32;
    const bool bf = s->act_dtype == MOE_BF16 && s->w_dtype == MOE_BF16;
    const bool mx = s->act_dtype == MOE_BF16 && s->w_dtype == MOE_MXFP4;
    if (!f32 && !bf && !mx) {
        if ((s->act_dtype < 0 || s->act_dtype > 2) || (s->w_dtype < 0 || s->w_dtype > 2))
            return fail(MOE_EINVAL, "unknown dtype");
        return fail(MOE_EUNSUPPORTED, "unsupported dtype combination");
    }
    if (mx && (s->H % 128 || s->I % 128))
        return fail(MOE_EINVAL, "MXFP4 needs H and I multiples of 128");
    if (mx && (s->H > 4096 || s->I > 4096))  // activation tile staged in LDS
        return fail(MOE_EUNSUPPORTED, "MXFP4 supports H and I up to 4096");
    if (mx && s->I_shared)
        return fail(MOE_EUNSUPPORTED, "MXFP4 with a shared expert is not supported");
    return MOE_OK;
}

// The kernels index token rows, staging rows and logit planes of one pass
// with 32-bit offsets: refuse passes whose largest offset would not fit.
int check_pass_size(const moe_shape_t *s, int64_t Tc)
{
    const int64_t lim = (int64_t)1 << 31;
    const int64_t rows = Tc * s->top_k + (s->I_shared > 0 ? Tc : 0);
    const int64_t width = std::max<int64_t>(s->H, std::max(s->I, s->I_shared));
    if (Tc * s->H >= lim || Tc * s->E * 8 >= lim || rows * width >= lim)
        return fail(MOE_EINVAL, "pass too large for 32-bit row offsets: lower T or chunk_T");
    return MOE_OK;
}

int check_weights(const moe_shape_t *s, const moe_weights_t *w)
{
    if (!w)
        return fail(MOE_EINVAL, "weights is NULL");
    if (!w->router_w || !w->w_gate || !w->w_up || !w->w_down)
        return fail(MOE_EINVAL, "router or expert weight pointer is NULL");
    if (!aligned16(w->router_w) || !aligned16(w->w_gate) || !aligned16(w->w_up) ||
        !aligned16(w->w_down))
        return fail(MOE_EINVAL, "weight pointer not 16-byte aligned");
    if (w->router_bias && ((uintptr_t)w->router_bias & 3u))
        return fail(MOE_EINVAL, "router_bias not 4-byte aligned");
    // bf16 / MXFP4 kernels read the packed layouts only; f32 ones row-major
    const int want = s->w_dtype == MOE_F32 ? MOE_LAYOUT_ROWMAJOR : MOE_LAYOUT_PACKED;
    if (w->layout != want)
        return fail(MOE_EINVAL, s->w_dtype == MOE_F32
                                    ? "f32 expert matrices must be row-major (layout ROWMAJOR)"
                                    : "bf16/MXFP4 expert matrices must be packed by moe_pack_bf16 / "
                                      "moe_pack_mxfp4 and declared with layout PACKED");
    if (s->w_dtype == MOE_MXFP4) {
        if (!w->s_gate || !w->s_up || !w->s_down)
            return fail(MOE_EINVAL, "MXFP4 scale pointer is NULL");
        if (!aligned16(w->s_gate) || !aligned16(w->s_up) || !aligned16(w->s_down))
            return fail(MOE_EINVAL, "MXFP4 scale pointer not 16-byte aligned");
    }
    if (s->I_shared > 0) {
        if (!w->sh_gate || !w->sh_up || !w->sh_down)
            return fail(MOE_EINVAL, "shared expert pointer is NULL");
        if (!aligned16(w->sh_gate) || !aligned16(w->sh_up) || !aligned16(w->sh_down))
            return fail(MOE_EINVAL, "shared expert pointer not 16-byte aligned");
    }
    return MOE_OK;
}

// Workspace layout of one pass of Tc tokens.
struct Layout {
    size_t logits, wts, blk, counts, offsets, row_src, row_tok, row_of, tiles_gu, ntiles, tiles_dc,
        items_gu, items_dc, h, stage, xq, total;
    bool has_xq;  // MXFP4 passes routed by router_small: x quantised once per token
    int max_tiles_gu, max_tiles_dc, bm_gu, bm_dc, ntn_gu, ntn_dc, wrows_gu, wrows_dc;
    int64_t logit_floats;  // capacity of the logits area
};

moe::ExpertArgs expert_shape(const moe_shape_t *s, int Tc)
{
    moe::ExpertArgs a{};
    a.T = Tc;
    a.shape_T = Tc;
    a.H = s->H;
    a.E = s->E;
    a.k = s->top_k;
    a.I = s->I;
    a.I_shared = s->I_shared;
    a.act = s->act_dtype == MOE_BF16 ? moe::ACT_BF16 : moe::ACT_F32;
    a.wdt = s->w_dtype;
    return a;
}

int max_tiles(int64_t Tc, const moe_shape_t *s, int bm)
{
    const int64_t pairs = Tc * s->top_k;
    int64_t n = cdiv(pairs, bm) + std::min<int64_t>(s->E, pairs);
    if (s->I_shared > 0)
        n += cdiv(Tc, bm);
    return (int)n;
}

Layout layout(const moe_shape_t *s, int Tc)
{
    Layout L{};
    const moe::ExpertArgs a = expert_shape(s, Tc);
    L.bm_gu = moe::gemm_bm_gu(a);
    L.bm_dc = moe::gemm_bm_dc(a);
    L.max_tiles_gu = max_tiles(Tc, s, L.bm_gu);
    L.max_tiles_dc = max_tiles(Tc, s, L.bm_dc);
    L.ntn_gu = moe::stream_ntn(a, true);
    L.ntn_dc = moe::stream_ntn(a, false);
    L.wrows_gu = moe::stream_wrows(a, true);
    L.wrows_dc = moe::stream_wrows(a, false);
    const int64_t pairs = (int64_t)Tc * s->top_k;
    const int64_t rows = pairs + (s->I_shared > 0 ? Tc : 0);
    const int64_t ldh = std::max(s->I, s->I_shared);
    const int64_t esz = s->act_dtype == MOE_F32 ? 4 : 2;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    // logits: one plane, or the eight partial-sum planes of the segmented
    // router (long passes) or of the split router (decode rows)
    const int ract = s->act_dtype == MOE_BF16 ? moe::ACT_BF16 : moe::ACT_F32;
    const int nplanes = moe::router_split_ok(Tc, s->E, s->H, ract)
                            ? 8
                            : moe::router_parts(Tc, s->H, s->E, ract);
    L.logit_floats = (int64_t)Tc * s->E * nplanes;
    L.logits = take((size_t)L.logit_floats * 4);
    L.wts = take((size_t)pairs * 4);
    L.blk = take((size_t)std::max(1, moe::permute_blocks((int)pairs)) * s->E * 4);
    L.counts = take((size_t)(s->E + 1) * 4);
    L.offsets = take((size_t)(s->E + 2) * 4);
    L.row_src = take((size_t)rows * 4);
    L.row_tok = take((size_t)rows * 4);
    L.row_of = take((size_t)pairs * 4);
    L.tiles_gu = take((size_t)L.max_tiles_gu * sizeof(moe::Tile));
    L.ntiles = take(2 * 4);
    L.tiles_dc = take((size_t)L.max_tiles_dc * sizeof(moe::Tile));
    L.items_gu = take((size_t)L.max_tiles_gu * L.ntn_gu * 16);
    L.items_dc = take((size_t)L.max_tiles_dc * L.ntn_dc * 16);
    L.h = take((size_t)rows * ldh * esz);
    L.stage = take((size_t)rows * s->H * esz);
    // decode, verify and other short passes with MXFP4 experts
    const int act = s->act_dtype == MOE_BF16 ? moe::ACT_BF16 : moe::ACT_F32;
    // The router quantising x once for all expert kernels is off unless
    // MOE_MX_XQ=1 (read at every call, so workspace sizing and calls agree
    // while it is unchanged): measured slower than each expert workgroup
    // quantising its own rows (the router's extra work lies on the decode
    // step's critical path, and copying a quantised row costs what
    // quantising it does).  The results are bit-identical either way.
    const char *xq_env = std::getenv("MOE_MX_XQ");
    const bool xq_on = xq_env && xq_env[0] == '1';
    L.has_xq = xq_on && s->w_dtype == MOE_MXFP4 && moe::router_xq_ok(s->E, s->H, act) &&
               moe::route_small_ok(Tc, s->top_k, s->E, s->H, act);
    L.xq = L.has_xq ? take(moe::router_xq_bytes(Tc, s->H)) : 0;
    L.total = off;
    return L;
}

// ---- optional stage timing (HIP events on the caller's stream) -----------

constexpr int N_STAGES = 5;
constexpr int MAX_TIMED = 4096;

struct Timing {
    std::mutex mu;
    bool on = false;
    int n = 0;                        // events pairs in use
    hipEvent_t ev[MAX_TIMED * N_STAGES][2];
    int stage[MAX_TIMED * N_STAGES];
    int calls = 0;
    int created = 0;
};
Timing g_timing;

// Event pair for one stage of the current call, or null when timing is off
// or the record is full.
hipEvent_t *timing_slot(int stage)
{
    if (!g_timing.on || g_timing.n >= MAX_TIMED * N_STAGES)
        return nullptr;
    const int i = g_timing.n;
    if (i >= g_timing.created) {
        if (hipEventCreate(&g_timing.ev[i][0]) != hipSuccess ||
            hipEventCreate(&g_timing.ev[i][1]) != hipSuccess)
            return nullptr;
        g_timing.created = i + 1;
    }
    g_timing.stage[i] = stage;
    g_timing.n = i + 1;
    return g_timing.ev[i];
}

struct StageScope {
    hipEvent_t *ev;
    hipStream_t st;
    StageScope(int stage, hipStream_t s) : ev(timing_slot(stage)), st(s)
    {
        if (ev)
            (void)hipEventRecord(ev[0], st);
    }
    ~StageScope()
    {
        if (ev)
            (void)hipEventRecord(ev[1], st);
    }
};

int pass_tokens(const moe_shape_t *s)
{
    return (s->chunk_T > 0 && s->chunk_T < s->T) ? s->chunk_T : s->T;
}

int launched(const char *what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        std::snprintf(g_last, sizeof g_last, "%s: %s", what, hipGetErrorString(e));
        return MOE_EHIP;
    }
    return MOE_OK;
}

// Router and permutation of one pass.
int route_pass(const moe_shape_t *s, const moe_weights_t *w, const void *x, int Tc,
               int32_t *idx, float *wts, char *ws, const Layout &L, hipStream_t st)
{
    moe::RouterArgs r{};
    r.x = x;
    r.wr = w->router_w;
    r.bias = w->router_bias;
    r.logits = (float *)(ws + L.logits);
    r.idx = idx;
    r.w = wts;
    r.T = Tc;
    r.H = s->H;
    r.E = s->E;
    r.k = s->top_k;
    r.act = s->act_dtype == MOE_BF16 ? moe::ACT_BF16 : moe::ACT_F32;
    const bool small = moe::route_small_ok(Tc, s->top_k, s->E, s->H, r.act);
    r.ticket = small ? (int32_t *)(ws + L.blk) : nullptr;
    r.xq = small && L.has_xq ? (uint8_t *)(ws + L.xq) : nullptr;
    // the segmented router counts the permutation's block histogram itself
    const bool seg = !small && moe::router_parts(Tc, s->H, s->E, r.act) == 8;
    r.hist = seg ? (int32_t *)(ws + L.blk) : nullptr;
    r.nhist = moe::permute_blocks(Tc * s->top_k) * s->E;
    // passes of up to 64 tokens: the split router, whose partial sums
    // route_small adds
    const bool split = small && !r.xq && moe::router_split_ok(Tc, s->E, s->H, r.act) &&
                       (int64_t)8 * Tc * s->E <= L.logit_floats;
    r.nparts = split ? 8 : 1;
    {
        StageScope sc(0, st);
        if (split)
            moe::launch_router_split(r, st);
        else if (small)
            moe::launch_router_small(r, st);  // top-k moves into the permutation pass
        else
            moe::launch_router(r, st);
    }
    int rc = launched("router");
    if (rc)
        return rc;
    moe::PermuteArgs p{};
    p.idx = idx;
    p.blk = (int32_t *)(ws + L.blk);
    p.counts = (int32_t *)(ws + L.counts);
    p.offsets = (int32_t *)(ws + L.offsets);
    p.row_src = (int32_t *)(ws + L.row_src);
    p.row_tok = (int32_t *)(ws + L.row_tok);
    p.row_of = (int32_t *)(ws + L.row_of);
    p.tiles_a = (moe::Tile *)(ws + L.tiles_gu);
    p.ntiles_a = (int32_t *)(ws + L.ntiles);
    p.tiles_b = (moe::Tile *)(ws + L.tiles_dc);
    p.ntiles_b = (int32_t *)(ws + L.ntiles) + 1;
    p.bm_a = L.bm_gu;
    p.bm_b = L.bm_dc;
    p.items_a = L.ntn_gu ? (int4 *)(ws + L.items_gu) : nullptr;
    p.items_b = L.ntn_dc ? (int4 *)(ws + L.items_dc) : nullptr;
    p.hist_done = seg ? 1 : 0;
    p.ntn_a = L.ntn_gu;
    p.ntn_b = L.ntn_dc;
    p.max_tiles_a = L.max_tiles_gu;
    p.max_tiles_b = L.max_tiles_dc;
    p.wrows_a = L.wrows_gu;
    p.wrows_b = L.wrows_dc;
    p.T = Tc;
    p.E = s->E;
    p.k = s->top_k;
    p.shared = s->I_shared > 0;
    if (small) {
        StageScope sc(1, st);  // top-k and the permutation
        moe::launch_route_small(r, p, st);
    } else {
        StageScope sc(1, st);
        moe::launch_permute(p, st);
    }
    return launched("permute");
}

}  // namespace

int moe::api_fail(int code, const char *what) { return fail(code, what); }

extern "C" {

size_t moe_workspace_bytes(const moe_shape_t *shape)
{
    if (check_shape(shape) != MOE_OK || check_pass_size(shape, pass_tokens(shape)) != MOE_OK)
        return 0;
    return layout(shape, pass_tokens(shape)).total;
}

int moe_forward(const moe_shape_t *s, const moe_weights_t *w, const void *x, void *y,
                int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes, void *stream)
{
    int rc = check_shape(s);
    if (rc)
        return rc;
    rc = check_weights(s, w);
    if (rc)
        return rc;
    if (s->T == 0)
        return MOE_OK;
    if (!x || !y || !topk_idx)
        return fail(MOE_EINVAL, "x, y or topk_idx is NULL");
    if (!aligned16(x) || !aligned16(y) || !aligned16(topk_idx) ||
        (topk_w && !aligned16(topk_w)))
        return fail(MOE_EINVAL, "x, y, topk_idx or topk_w not 16-byte aligned");
    const int Tc = pass_tokens(s);
    if ((rc = check_pass_size(s, Tc)))
        return rc;
    const Layout L = layout(s, Tc);
    if (!ws || ((uintptr_t)ws & 255u))
        return fail(MOE_EINVAL, "workspace NULL or not 256-byte aligned");
    if (ws_bytes < L.total)
        return fail(MOE_EWORKSPACE, "workspace too small");
    rc = check_device();
    if (rc)
        return rc;
    hipStream_t st = (hipStream_t)stream;
    char *wsb = (char *)ws;
    const int64_t esz = s->act_dtype == MOE_F32 ? 4 : 2;
    std::unique_lock<std::mutex> tlock(g_timing.mu, std::defer_lock);
    if (g_timing.on) {
        tlock.lock();
        g_timing.calls++;
    }
    for (int c0 = 0; c0 < s->T; c0 += Tc) {
        const int n = std::min(Tc, s->T - c0);
        const char *xc = (const char *)x + (int64_t)c0 * s->H * esz;
        char *yc = (char *)y + (int64_t)c0 * s->H * esz;
        int32_t *idx = topk_idx + (int64_t)c0 * s->top_k;
        float *wts = topk_w ? topk_w + (int64_t)c0 * s->top_k : (float *)(wsb + L.wts);
        // Tile shapes follow the full pass size Tc, so a shorter last pass
        // uses the carved layout with tighter grid bounds.
        Layout Lw = L;
        Lw.max_tiles_gu = max_tiles(n, s, L.bm_gu);
        Lw.max_tiles_dc = max_tiles(n, s, L.bm_dc);
        // Decode rows with MXFP4 experts: logits, then gate+up straight from
        // them (the pairs in token order, no permutation), then down + combine.
        {
            moe::ExpertArgs d = expert_shape(s, n);
            d.x = xc;
            d.w_gate = w->w_gate;
            d.w_up = w->w_up;
            d.w_down = w->w_down;
            d.s_gate = w->s_gate;
            d.s_up = w->s_up;
            d.s_down = w->s_down;
            d.topk_idx = idx;
            d.topk_w = wts;
            d.h = wsb + Lw.h;
            d.y = yc;
            d.xq = Lw.has_xq ? (const uint8_t *)(wsb + Lw.xq) : nullptr;
            if (moe::gate_up_mxfp4_pair_ok(d)) {
                moe::RouterArgs r{};
                r.x = xc;
                r.xq = const_cast<uint8_t *>(d.xq);
                r.wr = w->router_w;
                r.bias = w->router_bias;
                r.logits = (float *)(wsb + Lw.logits);
                r.T = n;
                r.H = s->H;
                r.E = s->E;
                r.k = s->top_k;
                r.act = moe::ACT_BF16;
                // the split router unless the router also quantises x
                const bool split = !d.xq && moe::router_split_ok(n, s->E, s->H, r.act) &&
                                   (int64_t)8 * n * s->E <= Lw.logit_floats;
                {
                    StageScope sc(0, st);
                    if (split)
                        moe::launch_router_split(r, st);
                    else
                        moe::launch_router_small(r, st);
                }
                if ((rc = launched("router")))
                    return rc;
                {
                    StageScope sc(2, st);
                    moe::launch_gate_up_mxfp4_pair(d, r.logits, w->router_bias, split ? 8 : 1, st);
                }
                if ((rc = launched("gate_up")))
                    return rc;
                d.row_of = nullptr;  // h rows in pair order
                {
                    StageScope sc(3, st);
                    moe::launch_down_combine_mxfp4(d, st);
                }
                if ((rc = launched("down")))
                    return rc;
                continue;
            }
        }
        rc = route_pass(s, w, xc, n, idx, wts, wsb, Lw, st);
        if (rc)
            return rc;
        moe::ExpertArgs a = expert_shape(s, n);
        a.shape_T = Tc;
        a.x = xc;
        // rows quantised by the short-pass router (route_pass set them up)
        a.xq = Lw.has_xq && moe::route_small_ok(n, s->top_k, s->E, s->H, a.act)
                   ? (const uint8_t *)(wsb + Lw.xq)
                   : nullptr;
        a.w_gate = w->w_gate;
        a.w_up = w->w_up;
        a.w_down = w->w_down;
        a.s_gate = w->s_gate;
        a.s_up = w->s_up;
        a.s_down = w->s_down;
        a.sh_gate = w->sh_gate;
        a.sh_up = w->sh_up;
        a.sh_down = w->sh_down;
        a.row_src = (const int32_t *)(wsb + Lw.row_src);
        a.row_tok = (const int32_t *)(wsb + Lw.row_tok);
        a.offsets = (const int32_t *)(wsb + Lw.offsets);
        a.topk_w = wts;
        a.h = wsb + Lw.h;
        a.stage = wsb + Lw.stage;
        a.tiles_gu = (const moe::Tile *)(wsb + Lw.tiles_gu);
        a.ntiles_gu = (const int32_t *)(wsb + Lw.ntiles);
        a.tiles_dc = (const moe::Tile *)(wsb + Lw.tiles_dc);
        a.items_gu = (const int4 *)(wsb + Lw.items_gu);
        a.items_dc = (const int4 *)(wsb + Lw.items_dc);
        a.ntiles_dc = (const int32_t *)(wsb + Lw.ntiles) + 1;
        a.topk_idx = idx;
        a.row_of = (const int32_t *)(wsb + Lw.row_of);
        a.y = yc;
        a.max_tiles_gu = Lw.max_tiles_gu;
        a.max_tiles_dc = Lw.max_tiles_dc;
        {
            StageScope sc(2, st);
            moe::launch_gate_up(a, st);
        }
        if ((rc = launched("gate_up")))
            return rc;
        if (moe::down_combine_mxfp4_ok(a)) {  // decode rows: y straight from the down kernel
            {
                StageScope sc(3, st);
                moe::launch_down_combine_mxfp4(a, st);
            }
            if ((rc = launched("down")))
                return rc;
            continue;
        }
        {
            StageScope sc(3, st);
            moe::launch_down(a, st);
        }
        if ((rc = launched("down")))
            return rc;
        moe::CombineArgs cb{};
        cb.stage = wsb + Lw.stage;
        cb.row_of = (const int32_t *)(wsb + Lw.row_of);
        cb.topk_w = wts;
        cb.y = yc;
        cb.T = n;
        cb.H = s->H;
        cb.k = s->top_k;
        cb.shared = s->I_shared > 0;
        cb.act = a.act;
        {
            StageScope sc(4, st);
            moe::launch_combine(cb, st);
        }
        if ((rc = launched("combine")))
            return rc;
    }
    return MOE_OK;
}

int moe_route(const moe_shape_t *s, const moe_weights_t *w, const void *x, int32_t *topk_idx,
              float *topk_w, int32_t *counts, int32_t *offsets, int32_t *row_src, void *ws,
              size_t ws_bytes, void *stream)
{
    int rc = check_shape(s);
    if (rc)
        return rc;
    rc = check_weights(s, w);
    if (rc)
        return rc;
    if (s->chunk_T > 0 && s->chunk_T < s->T)
        return fail(MOE_EINVAL, "moe_route handles one pass: chunk_T must be 0 or >= T");
    if (s->T == 0)
        return MOE_OK;
    if (!x || !topk_idx)
        return fail(MOE_EINVAL, "x or topk_idx is NULL");
    if (!aligned16(x) || !aligned16(topk_idx) || (topk_w && !aligned16(topk_w)))
        return fail(MOE_EINVAL, "x, topk_idx or topk_w not 16-byte aligned");
    if ((rc = check_pass_size(s, s->T)))
        return rc;
    const Layout L = layout(s, s->T);
    if (!ws || ((uintptr_t)ws & 255u))
        return fail(MOE_EINVAL, "workspace NULL or not 256-byte aligned");
    if (ws_bytes < L.total)
        return fail(MOE_EWORKSPACE, "workspace too small");
    rc = check_device();
    if (rc)
        return rc;
    hipStream_t st = (hipStream_t)stream;
    char *wsb = (char *)ws;
    float *wts = topk_w ? topk_w : (float *)(wsb + L.wts);
    rc = route_pass(s, w, x, s->T, topk_idx, wts, wsb, L, st);
    if (rc)
        return rc;
    const int64_t pairs = (int64_t)s->T * s->top_k;
    if (counts && hipMemcpyAsync(counts, wsb + L.counts, (size_t)s->E * 4,
                                 hipMemcpyDeviceToDevice, st) != hipSuccess)
        return launched("copy counts");
    if (offsets && hipMemcpyAsync(offsets, wsb + L.offsets, (size_t)(s->E + 1) * 4,
                                  hipMemcpyDeviceToDevice, st) != hipSuccess)
        return launched("copy offsets");
    if (row_src && hipMemcpyAsync(row_src, wsb + L.row_src, (size_t)pairs * 4,
                                  hipMemcpyDeviceToDevice, st) != hipSuccess)
        return launched("copy row_src");
    return MOE_OK;
}

int moe_pack_bf16(int E, int N, int K, const void *w, void *w_out, void *stream)
{
    if (E < 1 || N < 32 || N % 32 || K < 32 || K % 32)
        return fail(MOE_EINVAL, "moe_pack_bf16: E >= 1, N and K multiples of 32");
    if (!w || !w_out)
        return fail(MOE_EINVAL, "moe_pack_bf16: NULL pointer");
    if (!aligned16(w) || !aligned16(w_out))
        return fail(MOE_EINVAL, "moe_pack_bf16: pointer not 16-byte aligned");
    const size_t nb = (size_t)E * N * K * 2;
    const uintptr_t a = (uintptr_t)w, b = (uintptr_t)w_out;
    if (a < b + nb && b < a + nb)
        return fail(MOE_EINVAL, "moe_pack_bf16: output overlaps the input");
    moe::launch_pack_bf16(E, N, K, (const uint16_t *)w, (uint16_t *)w_out, (hipStream_t)stream);
    return launched("moe_pack_bf16");
}

int moe_pack_mxfp4(int E, int N, int K, const void *codes, const uint8_t *scales, void *codes_out,
                   uint8_t *scales_out, void *stream)
{
    if (E < 1 || N < 16 || N % 16 || K < 128 || K % 128)
        return fail(MOE_EINVAL, "moe_pack_mxfp4: E >= 1, N a multiple of 16, K of 128");
    if (!codes || !scales || !codes_out || !scales_out)
        return fail(MOE_EINVAL, "moe_pack_mxfp4: NULL pointer");
    if (!aligned16(codes) || !aligned16(scales) || !aligned16(codes_out) || !aligned16(scales_out))
        return fail(MOE_EINVAL, "moe_pack_mxfp4: pointer not 16-byte aligned");
    const size_t cb = (size_t)E * N * (K / 2), sb = (size_t)E * N * (K / 32);
    auto overlap = [](const void *a, size_t na, const void *b, size_t nb) {
        const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
        return x < y + nb && y < x + na;
    };
    if (overlap(codes_out, cb, codes, cb) || overlap(codes_out, cb, scales, sb) ||
        overlap(scales_out, sb, codes, cb) || overlap(scales_out, sb, scales, sb) ||
        overlap(codes_out, cb, scales_out, sb))
        return fail(MOE_EINVAL, "moe_pack_mxfp4: outputs overlap the inputs or each other");
    moe::launch_pack_mxfp4(E, N, K, (const uint8_t *)codes, scales, (uint8_t *)codes_out,
                           scales_out, (hipStream_t)stream);
    return launched("moe_pack_mxfp4");
}

const char *moe_strerror(int code)
{
    switch (code) {
    case MOE_OK:
        return "ok";
    case MOE_EINVAL:
        return "invalid argument";
    case MOE_EWORKSPACE:
        return "workspace too small";
    case MOE_EUNSUPPORTED:
        return "unsupported device or dtype combination";
    case MOE_EHIP:
        return "HIP runtime error";
    default:
        return "unknown error code";
    }
}

const char *moe_last_error(void) { return g_last; }

int moe_stage_timing_enable(int on)
{
    std::lock_guard<std::mutex> lock(g_timing.mu);
    g_timing.on = on != 0;
    g_timing.n = 0;
    g_timing.calls = 0;
    return MOE_OK;
}

int moe_stage_timing_read(float *ms, int n_stages, int *n_calls)
{
    std::lock_guard<std::mutex> lock(g_timing.mu);
    for (int i = 0; i < n_stages; ++i)
        if (ms)
            ms[i] = 0.0f;
    int rc = MOE_OK;
    for (int i = 0; i < g_timing.n; ++i) {
        float t = 0.0f;
        if (hipEventSynchronize(g_timing.ev[i][1]) != hipSuccess ||
            hipEventElapsedTime(&t, g_timing.ev[i][0], g_timing.ev[i][1]) != hipSuccess) {
            rc = fail(MOE_EHIP, "stage timing events failed");
            continue;
        }
        if (ms && g_timing.stage[i] < n_stages)
            ms[g_timing.stage[i]] += t;
    }
    if (n_calls)
        *n_calls = g_timing.calls;
    g_timing.n = 0;
    g_timing.calls = 0;
    return rc;
}

int moe_probe_read(const void *buf, size_t bytes, void *stream)
{
    if (!buf || bytes == 0 || bytes % 16 != 0)
        return fail(MOE_EINVAL, "moe_probe_read: buf and a positive multiple of 16 bytes");
    moe::launch_probe_read(buf, bytes, nullptr, (hipStream_t)stream);
    return launched("probe_read");
}

int moe_probe_gather(const void *pool, size_t pool_bytes, size_t chunk_bytes,
                     const int32_t *order, int nchunks, int wgs, void *stream)
{
    if (!pool || !order || chunk_bytes == 0 || chunk_bytes % 16 != 0 || nchunks <= 0 ||
        pool_bytes < chunk_bytes || pool_bytes / chunk_bytes > (size_t)INT32_MAX ||
        (uintptr_t)pool % 16 != 0 || wgs <= 0 || wgs > 65536)
        return fail(MOE_EINVAL, "moe_probe_gather: pool, order, chunk_bytes a positive multiple "
                                "of 16 within pool_bytes, nchunks > 0, 1 <= wgs <= 65536");
    moe::launch_probe_gather(pool, (int)(pool_bytes / chunk_bytes), order, nchunks, chunk_bytes,
                             wgs, nullptr, (hipStream_t)stream);
    return launched("probe_gather");
}

int moe_probe_mxfp4(const void *codes, const uint8_t *scales, size_t nblocks, int wgs, float *out,
                    void *stream)
{
    if (!codes || !scales || !out || nblocks == 0 || (uintptr_t)codes % 16 != 0 || wgs <= 0 ||
        wgs > 65536)
        return fail(MOE_EINVAL, "moe_probe_mxfp4: codes (16-byte aligned), scales, out, "
                                "nblocks > 0, 1 <= wgs <= 65536");
    moe::launch_probe_mxfp4(codes, scales, nblocks, wgs, out, (hipStream_t)stream);
    return launched("probe_mxfp4");
}

int moe_probe_mfma(int waves, int iters, int *sink, void *stream)
{
    if (waves <= 0 || waves % 4 != 0 || iters <= 0)
        return fail(MOE_EINVAL, "moe_probe_mfma: waves a positive multiple of 4, iters > 0");
    moe::launch_probe_mfma(waves, iters, sink, (hipStream_t)stream);
    return launched("probe_mfma");
}

}  // extern "C"
