/*
 * moe_oracle.h - CPU oracle of one sparse Mixture-of-Experts layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously-correct
 * definition the GPU library is checked against.  Only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load it; the product path
 * never does.  It shares no code with the GPU library.
 *
 * All pointers are HOST pointers.  Every call is synchronous, validates its
 * arguments first and returns MOE_REF_OK (0) or a nonzero status without
 * writing any output.
 *
 * What is computed (sources: "256 experts, 512 lines" blog post, sections
 * "Why GLM-5.2 in an engine built for DeepSeek" and "The constant that always
 * said 256"; NeutronStar README (main branch), Hy3 paragraph; NeutronStar
 * README, "The model"):
 *   logits  l[t,e] = sum_i x[t,i] * Wr[e,i], row stride n_expert
 *   score   s = sigmoid(l)  or  s = sqrt(softplus(l))
 *   select  top-k of key = s + bias[e] (bias optional), ties -> lower index
 *   weight  w_j = route_scale * s_j / sum_sel s   (bias never enters w)
 *   expert  FFN_e(x) = Wd[e] (silu(Wg[e] x) * (Wu[e] x))     (SwiGLU)
 *   output  y[t] = FFN_shared(x_t) + sum_j w_j FFN_{e_j}(x_t)
 * Arithmetic: fp64 accumulation in ascending index order, rounded once where a
 * stored value is produced (logits, scores, weights: fp32; the SwiGLU
 * intermediate h: bf16 for bf16/int8 layers, fp32 for fp32 layers; y: fp32).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MOE_REF_OK = 0, MOE_REF_ERR_INVALID = 1, MOE_REF_ERR_UNSUPPORTED = 2 };
enum { MOE_REF_SCORE_SIGMOID = 0, MOE_REF_SCORE_SQRT_SOFTPLUS = 1 };
enum { MOE_REF_DT_F32 = 0, MOE_REF_DT_BF16 = 1, MOE_REF_DT_Q8B32 = 2 };

typedef struct {
    int32_t n_tokens, d_model, n_expert, top_k, d_ff, n_shared, d_ff_shared;
    int32_t score;
    float route_scale;
    int32_t act_dtype, w_dtype;
} moe_ref_config;

/* A weight tensor [n, rows, cols], row-major, cols = reduction dimension.
 * F32: float; BF16: uint16 bit patterns; Q8B32: int8 quants in q and one fp16
 * scale (bit pattern) per 32 consecutive columns in scale [n, rows, cols/32]. */
typedef struct {
    const void *q;
    const uint16_t *scale;
} moe_ref_mat;

typedef struct {
    const float *w_router; /* [E, d] fp32 */
    const float *bias;     /* [E] fp32 or NULL */
    moe_ref_mat gate, up;  /* [E, F, d] */
    moe_ref_mat down;      /* [E, d, F] */
    moe_ref_mat s_gate, s_up, s_down; /* [S, Fs, d], [S, Fs, d], [S, d, Fs] */
} moe_ref_weights;

typedef struct {
    float *logits;     /* [T, E] */
    int32_t *topk_idx; /* [T, k] */
    float *topk_w;     /* [T, k] */
    int32_t *offsets;  /* [E+1] */
    int32_t *perm_rows, *inv_perm; /* [T*k] */
} moe_ref_debug;

/* Router: logits (optional output) and the top-k selection. */
int moe_ref_route(const moe_ref_config *cfg, const void *x, const float *w_router, const float *bias,
                  float *logits, int32_t *topk_idx, float *topk_w);
/* Selection from given logits. */
int moe_ref_select(const moe_ref_config *cfg, const float *logits, const float *bias,
                   int32_t *topk_idx, float *topk_w);
/* Stable counting sort of the flat assignments f = t*k + j by expert.
 * Assignments whose expert lies outside [0, E) are left out: they get
 * inv_perm = -1 and the unused tail of perm_rows is set to -1. */
int moe_ref_permute(const moe_ref_config *cfg, const int32_t *topk_idx, int32_t *offsets,
                    int32_t *perm_rows, int32_t *inv_perm);
/* slot_out[f, :] = w_f * FFN_{expert of f}(x_t), expert read from the
 * permutation; shared_out[t, :] = FFN_shared(x_t) (may be NULL iff n_shared==0). */
int moe_ref_expert_ffn(const moe_ref_config *cfg, const void *x, const moe_ref_weights *w,
                       const int32_t *offsets, const int32_t *perm_rows, const float *topk_w,
                       float *slot_out, float *shared_out);
/* y[t, :] = shared_out[t, :] + sum_j slot_out[t*k+j, :] (shared_out may be NULL). */
int moe_ref_combine(const moe_ref_config *cfg, const float *slot_out, const float *shared_out,
                    float *y);
/* The whole layer, token by token; dbg may be NULL and its fields may be NULL. */
int moe_ref_layer_forward(const moe_ref_config *cfg, const void *x, const moe_ref_weights *w,
                          float *y, moe_ref_debug *dbg);
/* Dense SwiGLU of every token through one expert (index `expert` of the given
 * tensors), written independently of the layer code; y64 [T, d] in fp64,
 * before any final rounding. */
int moe_ref_dense_swiglu(int32_t n_tokens, int32_t d_model, int32_t d_ff, int32_t act_dtype,
                         int32_t w_dtype, const void *x, moe_ref_mat gate, moe_ref_mat up,
                         moe_ref_mat down, int32_t expert, double *y64);

/* Row top-k: for each of `rows` rows of n scores, the k candidates that come
 * first under the selection order (larger value first, NaN after every number,
 * -0 == +0, equal values by lower index), written to idx[rows, k] in ascending
 * index order; vals[rows, k] (may be NULL) receives their scores.  1 <= k <= n. */
int moe_ref_topk_rows(int32_t rows, int32_t n, int32_t k, const float *scores, int32_t *idx,
                      float *vals);

/* Format helpers, exported so the tests can pin them. */
uint16_t moe_ref_bf16_from_f64(double v);
float moe_ref_f16_to_f32(uint16_t h);
float moe_ref_score(int32_t score, float logit);
const char *moe_ref_status_str(int status);
int moe_ref_mutant(void); /* which planted mistake this compiled copy carries (0 = none) */
int moe_ref_threads(void); /* OpenMP threads the token loops use */
int moe_ref_set_threads(int n); /* set them (n >= 1); returns the previous count */

#ifdef __cplusplus
}
#endif
#endif
