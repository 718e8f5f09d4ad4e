/*
 * Drives every entry point of the C oracle on small problems, for a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer (test infrastructure:
 * tests/test_oracle_sanitized.py compiles and runs it).  Each buffer is its
 * own heap block of exactly the size the header states, so a read or write
 * past any of them stops the run; the checks below are invariants that hold
 * for any input (weights of a token sum to one, the permutation is a stable
 * grouping, a token's output does not depend on which other tokens are in
 * the call), not values.  Exit status 0 and "ok" on stdout when all hold.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void)  /* xorshift64*, input data only */
{
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

static float next_f(float scale)
{
    return scale * ((float)next_u32() / 4294967296.0f * 2.0f - 1.0f);
}

static void *fill(int dtype, int64_t n, float scale)
{
    /* n elements of dtype (MXFP4: n codes, two per byte) */
    if (dtype == OR_F32) {
        float *p = malloc(sizeof(float) * (size_t)n);
        for (int64_t i = 0; i < n; ++i)
            p[i] = next_f(scale);
        return p;
    }
    if (dtype == OR_BF16) {
        uint16_t *p = malloc(sizeof(uint16_t) * (size_t)n);
        for (int64_t i = 0; i < n; ++i) {
            float f = next_f(scale);
            uint32_t b;
            memcpy(&b, &f, 4);
            p[i] = (uint16_t)(b >> 16);
        }
        return p;
    }
    uint8_t *p = malloc((size_t)(n / 2));
    for (int64_t i = 0; i < n / 2; ++i)
        p[i] = (uint8_t)next_u32();
    return p;
}

static uint8_t *fill_scales(int64_t n)
{
    uint8_t *p = malloc((size_t)n);
    for (int64_t i = 0; i < n; ++i)
        p[i] = (uint8_t)(120 + next_u32() % 8);
    return p;
}

static int failures = 0;
#define CHECK(c, ...)                                         \
    do {                                                      \
        if (!(c)) {                                           \
            fprintf(stderr, "check failed: " __VA_ARGS__);    \
            fprintf(stderr, " (line %d)\n", __LINE__);        \
            ++failures;                                       \
        }                                                     \
    } while (0)

static void run_case(const char *name, int act, int wdt, int T, int H, int E, int k, int I,
                     int Is, int bias)
{
    or_problem p;
    memset(&p, 0, sizeof p);
    p.H = H;
    p.E = E;
    p.top_k = k;
    p.I = I;
    p.I_shared = Is;
    p.act_dtype = act;
    p.w_dtype = wdt;
    void *x = fill(act, (int64_t)T * H, 1.0f);
    void *rw = fill(act, (int64_t)E * H, 0.2f);
    float *rb = NULL;
    if (bias) {
        rb = malloc(sizeof(float) * (size_t)E);
        for (int e = 0; e < E; ++e)
            rb[e] = next_f(0.5f);
    }
    p.router_w = rw;
    p.router_bias = rb;
    void *wg = fill(wdt, (int64_t)E * I * H, 0.1f);
    void *wu = fill(wdt, (int64_t)E * I * H, 0.1f);
    void *wd = fill(wdt, (int64_t)E * H * I, 0.1f);
    uint8_t *sg = NULL, *su = NULL, *sd = NULL;
    if (wdt == OR_MXFP4) {
        sg = fill_scales((int64_t)E * I * (H / 32));
        su = fill_scales((int64_t)E * I * (H / 32));
        sd = fill_scales((int64_t)E * H * (I / 32));
    }
    p.w_gate = wg;
    p.w_up = wu;
    p.w_down = wd;
    p.s_gate = sg;
    p.s_up = su;
    p.s_down = sd;
    void *shg = NULL, *shu = NULL, *shd = NULL;
    if (Is) {
        shg = fill(act, (int64_t)Is * H, 0.1f);
        shu = fill(act, (int64_t)Is * H, 0.1f);
        shd = fill(act, (int64_t)H * Is, 0.1f);
    }
    p.sh_gate = shg;
    p.sh_up = shu;
    p.sh_down = shd;

    int32_t *idx = malloc(sizeof(int32_t) * (size_t)T * k);
    double *w = malloc(sizeof(double) * (size_t)T * k);
    double *logits = malloc(sizeof(double) * (size_t)T * E);
    CHECK(or_route(&p, x, T, NULL, idx, w, logits) == OR_OK, "%s: or_route", name);
    for (int t = 0; t < T; ++t) {
        double s = 0.0;
        for (int j = 0; j < k; ++j) {
            const int e = idx[t * k + j];
            CHECK(e >= 0 && e < E, "%s: expert id %d", name, e);
            s += w[t * k + j];
            if (j > 0)  /* selected in descending logit order */
                CHECK(logits[t * E + idx[t * k + j - 1]] >= logits[t * E + e],
                      "%s: selection order", name);
        }
        CHECK(fabs(s - 1.0) < 1e-12, "%s: weights of token %d sum to %.17g", name, t, s);
    }

    double *gap = malloc(sizeof(double) * (size_t)T);
    CHECK(or_topk_margin(&p, x, T, NULL, gap) == OR_OK, "%s: or_topk_margin", name);
    for (int t = 0; t < T; ++t)
        CHECK(gap[t] >= 0.0, "%s: margin", name);

    int32_t *counts = malloc(sizeof(int32_t) * (size_t)E);
    int32_t *offsets = malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *row_src = malloc(sizeof(int32_t) * (size_t)T * k);
    CHECK(or_permute(T, k, E, idx, counts, offsets, row_src) == OR_OK, "%s: or_permute", name);
    CHECK(offsets[E] == T * k, "%s: offsets end", name);
    for (int e = 0; e < E; ++e)
        for (int r = offsets[e]; r < offsets[e + 1]; ++r) {
            CHECK(idx[row_src[r]] == e, "%s: grouped row %d", name, r);
            if (r > offsets[e])
                CHECK(row_src[r - 1] < row_src[r], "%s: stable order", name);
        }

    double *y = malloc(sizeof(double) * (size_t)T * H);
    int32_t *idx2 = malloc(sizeof(int32_t) * (size_t)T * k);
    double *w2 = malloc(sizeof(double) * (size_t)T * k);
    CHECK(or_forward(&p, x, T, NULL, y, idx2, w2) == OR_OK, "%s: or_forward", name);
    CHECK(memcmp(idx, idx2, sizeof(int32_t) * (size_t)T * k) == 0, "%s: forward idx", name);
    for (int i = 0; i < T * H; ++i)
        CHECK(isfinite(y[i]), "%s: y finite", name);

    /* a token's row is the same alone, reordered or among others */
    const int nsub = T >= 3 ? 3 : T;
    int32_t *sub = malloc(sizeof(int32_t) * (size_t)nsub);
    for (int i = 0; i < nsub; ++i)
        sub[i] = T - 1 - 2 * i >= 0 ? T - 1 - 2 * i : i;
    double *ys = malloc(sizeof(double) * (size_t)nsub * H);
    CHECK(or_forward(&p, x, nsub, sub, ys, NULL, NULL) == OR_OK, "%s: or_forward subset", name);
    for (int i = 0; i < nsub; ++i)
        CHECK(memcmp(ys + (int64_t)i * H, y + (int64_t)sub[i] * H, sizeof(double) * (size_t)H) == 0,
              "%s: token %d differs in a subset call", name, sub[i]);

    /* decoders over each stored matrix */
    double *dec = malloc(sizeof(double) * (size_t)I * H);
    CHECK(or_decode(wg, sg, wdt, I, H, dec) == OR_OK, "%s: or_decode", name);
    for (int i = 0; i < I * H; ++i)
        CHECK(isfinite(dec[i]), "%s: decoded value", name);
    CHECK(or_decode(wd, sd, wdt, H, I, dec) == OR_OK, "%s: or_decode down", name);

    /* zero tokens: nothing read or written */
    CHECK(or_forward(&p, x, 0, NULL, y, NULL, NULL) == OR_OK, "%s: n_tok 0", name);
    CHECK(or_route(&p, x, 0, NULL, idx, NULL, NULL) == OR_OK, "%s: route n_tok 0", name);

    free(dec);
    free(ys);
    free(sub);
    free(w2);
    free(idx2);
    free(y);
    free(row_src);
    free(offsets);
    free(counts);
    free(gap);
    free(logits);
    free(w);
    free(idx);
    free(shd);
    free(shu);
    free(shg);
    free(sd);
    free(su);
    free(sg);
    free(wd);
    free(wu);
    free(wg);
    free(rb);
    free(rw);
    free(x);
}

static void run_errors(void)
{
    or_problem p;
    memset(&p, 0, sizeof p);
    float x[64] = {0}, rw[4 * 64] = {0};
    int32_t idx[8];
    double y[64], w[8];
    p.H = 64;
    p.E = 4;
    p.top_k = 2;
    p.I = 32;
    p.act_dtype = OR_F32;
    p.w_dtype = OR_F32;
    p.router_w = rw;
    CHECK(or_route(NULL, x, 1, NULL, idx, w, NULL) == OR_EINVAL, "NULL problem");
    CHECK(or_route(&p, NULL, 1, NULL, idx, w, NULL) == OR_EINVAL, "NULL x");
    CHECK(or_route(&p, x, -1, NULL, idx, w, NULL) == OR_EINVAL, "negative n_tok");
    CHECK(or_forward(&p, x, 1, NULL, y, NULL, NULL) == OR_EINVAL, "missing expert weights");
    p.top_k = 5;
    CHECK(or_route(&p, x, 1, NULL, idx, w, NULL) == OR_EINVAL, "top_k > E");
    p.top_k = 2;
    p.act_dtype = 7;
    CHECK(or_route(&p, x, 1, NULL, idx, w, NULL) == OR_EINVAL, "act dtype");
    p.act_dtype = OR_F32;
    p.w_dtype = OR_MXFP4;
    p.I = 48;
    CHECK(or_route(&p, x, 1, NULL, idx, w, NULL) == OR_EINVAL, "MXFP4 I not a multiple of 32");
    int32_t bad_idx[2] = {0, 4}, c[4], o[5], r[2];
    CHECK(or_permute(1, 2, 4, bad_idx, c, o, r) == OR_EINVAL, "expert id out of range");
    CHECK(or_decode(x, NULL, OR_MXFP4, 1, 32, y) == OR_EINVAL, "MXFP4 decode without scales");
    CHECK(or_decode(x, NULL, 9, 1, 32, y) == OR_EINVAL, "decode dtype");
    CHECK(or_set_threads(0) == OR_EINVAL, "zero threads");
}

int main(void)
{
    /*        name      act      w         T  H    E  k  I    I_s bias */
    run_case("f32", OR_F32, OR_F32, 7, 64, 8, 2, 32, 0, 0);
    run_case("bf16", OR_BF16, OR_BF16, 9, 64, 16, 4, 96, 0, 1);
    run_case("bf16+sh", OR_BF16, OR_BF16, 5, 128, 8, 3, 64, 64, 1);
    run_case("mxfp4", OR_BF16, OR_MXFP4, 6, 128, 8, 2, 64, 0, 1);
    run_case("mxfp4-f32x", OR_F32, OR_MXFP4, 1, 64, 4, 4, 32, 0, 0);
    run_case("k=E", OR_F32, OR_BF16, 4, 64, 3, 3, 32, 0, 0);
    run_errors();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
