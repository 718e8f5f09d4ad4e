/*
 * Plain CPU oracle for the top-k routed MoE FFN layer (test infrastructure
 * only; see moe_oracle.c for the passages each function follows).
 *
 * Layouts, all row-major:
 *   x [T, H]                         act_dtype (f32 or bf16 bit patterns)
 *   router_w [E, H]                  act_dtype
 *   router_bias [E]                  float, may be NULL
 *   w_gate, w_up [E, I, H]           w_dtype; for MXFP4: uint8 codes
 *   w_down [E, H, I]                 [E, I, H/2] / [E, H, I/2], scales
 *                                    [E, I, H/32] / [E, H, I/32]
 *   sh_gate, sh_up [I_shared, H]     act_dtype
 *   sh_down [H, I_shared]            act_dtype
 * Outputs are double precision.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_MXFP4 = 2 };
enum { OR_OK = 0, OR_EINVAL = -1, OR_ENOMEM = -2 };

typedef struct {
    int32_t H, E, top_k, I, I_shared;
    int32_t act_dtype, w_dtype;
    const void *router_w;
    const float *router_bias;
    const void *w_gate, *w_up, *w_down;
    const uint8_t *s_gate, *s_up, *s_down;
    const void *sh_gate, *sh_up, *sh_down;
} or_problem;

/* Decoders of the storage formats. */
double or_bf16_to_f64(uint16_t v);
double or_e2m1_value(uint8_t code);
double or_e8m0_value(uint8_t s);
int or_decode(const void *base, const uint8_t *scales, int dtype, int64_t N,
              int64_t K, double *out);

/* Routing of tokens `tokens[0..n_tok)` (all rows 0..n_tok-1 if NULL):
 * idx [n_tok, k], w [n_tok, k] (nullable), logits [n_tok, E] (nullable). */
int or_route(const or_problem *p, const void *x, int n_tok,
             const int32_t *tokens, int32_t *idx, double *w, double *logits);

/* Smallest neighbour gap among the k+1 largest logits, per token. */
int or_topk_margin(const or_problem *p, const void *x, int n_tok,
                   const int32_t *tokens, double *gap);

/* Stable counting sort of (t, j) pairs by expert: counts [E],
 * offsets [E+1], row_src [n_tok*k] = t*k + j in grouped order. */
int or_permute(int n_tok, int top_k, int E, const int32_t *idx,
               int32_t *counts, int32_t *offsets, int32_t *row_src);

/* y [n_tok, H] for the listed tokens, plus their idx and w (nullable). */
int or_forward(const or_problem *p, const void *x, int n_tok,
               const int32_t *tokens, double *y, int32_t *idx, double *w);

/* OpenMP threads of the calls above (for timing; results are the same for
 * every count) and the current count. */
int or_set_threads(int n);
int or_max_threads(void);

#ifdef __cplusplus
}
#endif

#endif
