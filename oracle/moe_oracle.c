/*
 * Plain CPU oracle for the top-k routed mixture-of-experts FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or helper with
 * the GPU library.
 *
 * Everything is computed in double precision from the exactly decoded
 * inputs, token by token, in the order the method defines.  Sources (the
 * pages are cited by title and section):
 *
 *  - "MoE prefill quantum" (artifacts.nacyot.com, section on the cause and
 *    the unique-expert equation): each token uses top_k of E experts.
 *  - "Jetson Orin Nano MoE: GPU clock floor and expert cache" (blog.gnu.or.kr,
 *    section re-checking part 1, and the gate-first section): an expert runs
 *    gate, then up, then down, and the activation is SwiGLU(gate, up), so the
 *    SiLU is applied to the gate branch.
 *  - same page, nondeterminism section: each expert writes its own output
 *    rows and the order in which they are summed never changes.
 *  - "DeepSeek V4.1F Q4 with native DSpark MTP on M3 Ultra" (aiwitness.kr,
 *    decode paragraph): an always-on shared expert runs gate+up+SwiGLU.
 *
 * Readings where the pages are silent (listed again in the design notes):
 *  - routing weights are a softmax over all E logits, restricted to the
 *    selected k and renormalised; this equals a softmax over the k selected
 *    logits, which is what is computed;
 *  - selection is on the logits (router bias included), descending, ties to
 *    the lower expert index;
 *  - the routing weight scales the expert's down-projection output;
 *  - the shared expert is added with weight 1;
 *  - MXFP4 follows the OCP MX v1.0 layout: E2M1 codes, two per byte with the
 *    even element in the low nibble, one E8M0 scale per 32 elements along K.
 *
 * Parity pins for every function live in tests/test_oracle.py (with the
 * page figures and format tables under tests/golden/).
 */
#include "moe_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* ---- input decoding ---------------------------------------------------- */

double or_bf16_to_f64(uint16_t v)
{
    /* bfloat16 is the upper half of an IEEE binary32. */
    uint32_t u = (uint32_t)v << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double or_e2m1_value(uint8_t code)
{
    /* E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
     * Exponent field 0 is subnormal: 0 or 0.5. */
    int sign = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -mag : mag;
}

double or_e8m0_value(uint8_t s)
{
    /* E8M0: an unsigned power-of-two exponent with bias 127; 0xFF is NaN. */
    if (s == 0xFF)
        return NAN;
    return ldexp(1.0, (int)s - 127);
}

/* Element (n, kk) of an [N, K] matrix stored in `dtype`. */
static double elem(const void *base, const uint8_t *scales, int dtype,
                   int64_t K, int64_t n, int64_t kk)
{
    switch (dtype) {
    case OR_F32:
        return (double)((const float *)base)[n * K + kk];
    case OR_BF16:
        return or_bf16_to_f64(((const uint16_t *)base)[n * K + kk]);
    default: {
        uint8_t byte = ((const uint8_t *)base)[n * (K / 2) + kk / 2];
        uint8_t code = (kk % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        return or_e2m1_value(code) * or_e8m0_value(scales[n * (K / 32) + kk / 32]);
    }
    }
}

/* Decode one [N, K] matrix into doubles. */
static void decode_matrix(const void *base, const uint8_t *scales, int dtype,
                          int64_t N, int64_t K, double *out)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t kk = 0; kk < K; ++kk)
            out[n * K + kk] = elem(base, scales, dtype, K, n, kk);
}

/* ---- router ------------------------------------------------------------ */

/* l_e = sum_h x[h] * Wr[e, h] + b_e, summed in h order. */
static void router_logits(const or_problem *p, const double *xt, double *l)
{
    for (int e = 0; e < p->E; ++e) {
        double acc = 0.0;
        for (int h = 0; h < p->H; ++h)
            acc += xt[h] * elem(p->router_w, NULL, p->act_dtype, p->H, e, h);
        if (p->router_bias)
            acc += (double)p->router_bias[e];
        l[e] = acc;
    }
}

/* Expert order: larger logit first, equal logits by lower index. */
static int before(const double *l, int a, int b)
{
    return l[a] > l[b] || (l[a] == l[b] && a < b);
}

/* Top-k of n logits by repeated selection of the best remaining expert. */
static void select_topk(const double *l, int n, int k, int32_t *idx)
{
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < n; ++e) {
            int taken = 0;
            for (int q = 0; q < j; ++q)
                if (idx[q] == e)
                    taken = 1;
            if (!taken && (best < 0 || before(l, e, best)))
                best = e;
        }
        idx[j] = best;
    }
}

/* Renormalised softmax weights of the k selected logits. */
static void topk_weights(const double *l, const int32_t *idx, int k, double *w)
{
    double m = l[idx[0]];
    double z = 0.0;
    for (int j = 0; j < k; ++j) {
        w[j] = exp(l[idx[j]] - m);
        z += w[j];
    }
    for (int j = 0; j < k; ++j)
        w[j] /= z;
}

/* ---- one expert FFN ---------------------------------------------------- */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* o = Wd * (silu(Wg x) .* (Wu x)); gate, up: [I, H]; down: [H, I]. */
static void expert_ffn(const double *xt, int H, int I, const void *wg,
                       const uint8_t *sg, const void *wu, const uint8_t *su,
                       const void *wd, const uint8_t *sd, int dtype,
                       double *a, double *o)
{
    for (int i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int h = 0; h < H; ++h)
            g += elem(wg, sg, dtype, H, i, h) * xt[h];
        for (int h = 0; h < H; ++h)
            u += elem(wu, su, dtype, H, i, h) * xt[h];
        a[i] = silu(g) * u;
    }
    for (int c = 0; c < H; ++c) {
        double acc = 0.0;
        for (int i = 0; i < I; ++i)
            acc += elem(wd, sd, dtype, I, c, i) * a[i];
        o[c] = acc;
    }
}

/* ---- public entry points ---------------------------------------------- */

static int check_problem(const or_problem *p)
{
    if (!p || !p->router_w)
        return OR_EINVAL;
    if (p->H <= 0 || p->E <= 0 || p->I <= 0 || p->top_k < 1 || p->top_k > p->E)
        return OR_EINVAL;
    if (p->act_dtype != OR_F32 && p->act_dtype != OR_BF16)
        return OR_EINVAL;
    if (p->w_dtype == OR_MXFP4 && (p->H % 32 || p->I % 32))
        return OR_EINVAL;
    if (p->I_shared < 0)
        return OR_EINVAL;
    return OR_OK;
}

int or_route(const or_problem *p, const void *x, int n_tok,
             const int32_t *tokens, int32_t *idx, double *w, double *logits)
{
    int rc = check_problem(p);
    if (rc != OR_OK || !x || !idx || n_tok < 0)
        return OR_EINVAL;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int i = 0; i < n_tok; ++i) {
        int t = tokens ? tokens[i] : i;
        double *xt = malloc(sizeof(double) * (size_t)p->H);
        double *l = malloc(sizeof(double) * (size_t)p->E);
        if (!xt || !l) {
            bad = 1;
        } else {
            for (int h = 0; h < p->H; ++h)
                xt[h] = elem(x, NULL, p->act_dtype, p->H, t, h);
            router_logits(p, xt, l);
            select_topk(l, p->E, p->top_k, idx + (int64_t)i * p->top_k);
            if (w)
                topk_weights(l, idx + (int64_t)i * p->top_k, p->top_k,
                             w + (int64_t)i * p->top_k);
            if (logits)
                memcpy(logits + (int64_t)i * p->E, l, sizeof(double) * (size_t)p->E);
        }
        free(xt);
        free(l);
    }
    return bad ? OR_ENOMEM : OR_OK;
}

int or_topk_margin(const or_problem *p, const void *x, int n_tok,
                   const int32_t *tokens, double *gap)
{
    /* Smallest difference between neighbours among the k+1 largest logits
     * (k if k == E): a positive gap means both the selected set and its
     * order are decided by a margin of at least `gap`. */
    int rc = check_problem(p);
    if (rc != OR_OK || !x || !gap || n_tok < 0)
        return OR_EINVAL;
    int k1 = p->top_k < p->E ? p->top_k + 1 : p->top_k;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int i = 0; i < n_tok; ++i) {
        int t = tokens ? tokens[i] : i;
        double *xt = malloc(sizeof(double) * (size_t)p->H);
        double *l = malloc(sizeof(double) * (size_t)p->E);
        int32_t *top = malloc(sizeof(int32_t) * (size_t)k1);
        if (!xt || !l || !top) {
            bad = 1;
        } else {
            for (int h = 0; h < p->H; ++h)
                xt[h] = elem(x, NULL, p->act_dtype, p->H, t, h);
            router_logits(p, xt, l);
            select_topk(l, p->E, k1, top);
            double g = INFINITY;
            for (int j = 0; j + 1 < k1; ++j)
                if (l[top[j]] - l[top[j + 1]] < g)
                    g = l[top[j]] - l[top[j + 1]];
            gap[i] = g;
        }
        free(xt);
        free(l);
        free(top);
    }
    return bad ? OR_ENOMEM : OR_OK;
}

int or_permute(int n_tok, int top_k, int E, const int32_t *idx,
               int32_t *counts, int32_t *offsets, int32_t *row_src)
{
    /* Stable counting sort of the (token, slot) pairs by expert id: pairs
     * keep the order t ascending, then j ascending, within each expert. */
    if (n_tok < 0 || top_k < 1 || E < 1 || !idx || !counts || !offsets || !row_src)
        return OR_EINVAL;
    int64_t pairs = (int64_t)n_tok * top_k;
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t q = 0; q < pairs; ++q) {
        if (idx[q] < 0 || idx[q] >= E)
            return OR_EINVAL;
        counts[idx[q]]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = calloc((size_t)E, sizeof(int32_t));
    if (!fill)
        return OR_ENOMEM;
    for (int64_t q = 0; q < pairs; ++q) {
        int e = idx[q];
        row_src[offsets[e] + fill[e]] = (int32_t)q;
        fill[e]++;
    }
    free(fill);
    return OR_OK;
}

int or_forward(const or_problem *p, const void *x, int n_tok,
               const int32_t *tokens, double *y, int32_t *idx, double *w)
{
    int rc = check_problem(p);
    if (rc != OR_OK || !x || !y || n_tok < 0)
        return OR_EINVAL;
    if (!p->w_gate || !p->w_up || !p->w_down)
        return OR_EINVAL;
    if (p->w_dtype == OR_MXFP4 && (!p->s_gate || !p->s_up || !p->s_down))
        return OR_EINVAL;
    if (p->I_shared > 0 && (!p->sh_gate || !p->sh_up || !p->sh_down))
        return OR_EINVAL;
    const int H = p->H, I = p->I, k = p->top_k;
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int i = 0; i < n_tok; ++i) {
        int t = tokens ? tokens[i] : i;
        int Imax = I > p->I_shared ? I : p->I_shared;
        double *xt = malloc(sizeof(double) * (size_t)H);
        double *l = malloc(sizeof(double) * (size_t)p->E);
        double *a = malloc(sizeof(double) * (size_t)Imax);
        double *o = malloc(sizeof(double) * (size_t)H);
        int32_t *sel = malloc(sizeof(int32_t) * (size_t)k);
        double *wt = malloc(sizeof(double) * (size_t)k);
        double *yt = y + (int64_t)i * H;
        if (!xt || !l || !a || !o || !sel || !wt) {
            bad = 1;
            goto done;
        }
        for (int h = 0; h < H; ++h)
            xt[h] = elem(x, NULL, p->act_dtype, H, t, h);

        /* Router: logits, top-k, renormalised softmax weights. */
        router_logits(p, xt, l);
        select_topk(l, p->E, k, sel);
        topk_weights(l, sel, k, wt);

        /* Routed experts, summed in slot order j = 0..k-1. */
        for (int c = 0; c < H; ++c)
            yt[c] = 0.0;
        for (int j = 0; j < k; ++j) {
            int e = sel[j];
            int64_t step_gu = p->w_dtype == OR_MXFP4 ? (int64_t)I * H / 2
                                                      : (int64_t)I * H;
            int64_t esz = p->w_dtype == OR_F32 ? 4 : p->w_dtype == OR_BF16 ? 2 : 1;
            const char *wg = (const char *)p->w_gate + (int64_t)e * step_gu * esz;
            const char *wu = (const char *)p->w_up + (int64_t)e * step_gu * esz;
            const char *wd = (const char *)p->w_down + (int64_t)e * step_gu * esz;
            const uint8_t *sg = NULL, *su = NULL, *sd = NULL;
            if (p->w_dtype == OR_MXFP4) {
                sg = p->s_gate + (int64_t)e * I * (H / 32);
                su = p->s_up + (int64_t)e * I * (H / 32);
                sd = p->s_down + (int64_t)e * H * (I / 32);
            }
            expert_ffn(xt, H, I, wg, sg, wu, su, wd, sd, p->w_dtype, a, o);
            for (int c = 0; c < H; ++c)
                yt[c] += wt[j] * o[c];
        }

        /* Shared expert, weight 1, after the routed sum. */
        if (p->I_shared > 0) {
            expert_ffn(xt, H, p->I_shared, p->sh_gate, NULL, p->sh_up, NULL,
                       p->sh_down, NULL, p->act_dtype, a, o);
            for (int c = 0; c < H; ++c)
                yt[c] += o[c];
        }
        if (idx)
            memcpy(idx + (int64_t)i * k, sel, sizeof(int32_t) * (size_t)k);
        if (w)
            memcpy(w + (int64_t)i * k, wt, sizeof(double) * (size_t)k);
    done:
        free(xt);
        free(l);
        free(a);
        free(o);
        free(sel);
        free(wt);
    }
    return bad ? OR_ENOMEM : OR_OK;
}

int or_decode(const void *base, const uint8_t *scales, int dtype, int64_t N,
              int64_t K, double *out)
{
    if (!base || !out || N < 0 || K < 0)
        return OR_EINVAL;
    if (dtype == OR_MXFP4 && (!scales || K % 32))
        return OR_EINVAL;
    if (dtype != OR_F32 && dtype != OR_BF16 && dtype != OR_MXFP4)
        return OR_EINVAL;
    decode_matrix(base, scales, dtype, N, K, out);
    return OR_OK;
}

/* ---- threads (timing only; results do not depend on the count) -------- */

int or_set_threads(int n)
{
    if (n < 1)
        return OR_EINVAL;
    omp_set_num_threads(n);
    return OR_OK;
}

int or_max_threads(void) { return omp_get_max_threads(); }
