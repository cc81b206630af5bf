/*
 * moe_oracle.c - CPU oracle of one sparse MoE layer forward (see moe_oracle.h).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the product path.  Shares no code with
 * the GPU library.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp -shared -fPIC -lm.  No
 * fast-math: every sum below is evaluated in the order written.  The token
 * loops are split across OpenMP threads; each output element is computed by one
 * thread in a fixed order, so the results do not depend on the thread count.
 *
 * ORACLE_MUTANT (compile-time, default 0) plants one known mistake; the tests
 * build those variants to show that the pins detect each of them.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

int moe_ref_mutant(void) { return ORACLE_MUTANT; }

int moe_ref_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the token loops from now on (n >= 1); returns the previous count.
 * Results do not depend on it: every output element is computed by one thread
 * in a fixed order. */
int moe_ref_set_threads(int n) {
    const int prev = moe_ref_threads();
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
    return prev;
}

const char *moe_ref_status_str(int status) {
    switch (status) {
    case MOE_REF_OK: return "ok";
    case MOE_REF_ERR_INVALID: return "invalid argument";
    case MOE_REF_ERR_UNSUPPORTED: return "unsupported configuration";
    default: return "unknown status";
    }
}

/* ------------------------------------------------------------------------ */
/* Storage formats, from their definitions.                                  */
/* ------------------------------------------------------------------------ */

/* bf16 -> value: the bf16 bits are the upper half of an IEEE binary32. */
static double bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* IEEE binary16 -> value (normal, subnormal, zero, inf, NaN). */
static double f16_to_f64(uint16_t h) {
    int ex = (h >> 10) & 0x1F, fr = h & 0x3FF;
    double v;
    if (ex == 0) v = ldexp((double)fr, -24);
    else if (ex == 31) v = fr ? NAN : INFINITY;
    else v = ldexp((double)(fr | 0x400), ex - 25);
    return (h & 0x8000u) ? -v : v;
}

float moe_ref_f16_to_f32(uint16_t h) { return (float)f16_to_f64(h); }

/* Round a double to the nearest bf16 (ties to even), directly: bf16 keeps 8
 * significant bits, exponents down to 2^-126 for normals, then a fixed
 * quantum of 2^-133 for subnormals; beyond the largest finite value
 * (0x7F7F = (2 - 2^-7) * 2^127) rounding reaches 2^128 and gives infinity. */
uint16_t moe_ref_bf16_from_f64(double v) {
    if (isnan(v)) return 0x7FC0u;
    uint16_t sign = signbit(v) ? 0x8000u : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    int e;
    double m = frexp(a, &e); /* a = m * 2^e, m in [0.5, 1): leading bit 2^(e-1) */
    double r;
    if (e - 1 >= -126) r = ldexp(rint(ldexp(m, 8)), e - 8);
    else r = ldexp(rint(ldexp(a, 133)), -133);
    if (r >= 0x1.0p128) return (uint16_t)(sign | 0x7F80u);
    float f = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (u >> 16));
}

static double round_h(double a, int act_dtype) {
#if ORACLE_MUTANT == 5 /* planted: SwiGLU intermediate left unrounded */
    (void)act_dtype;
    return a;
#else
    if (act_dtype == MOE_REF_DT_F32) return (double)(float)a;
    return bf16_to_f64(moe_ref_bf16_from_f64(a));
#endif
}

static double act_at(const void *x, int act_dtype, size_t i) {
    if (act_dtype == MOE_REF_DT_F32) return (double)((const float *)x)[i];
    return bf16_to_f64(((const uint16_t *)x)[i]);
}

/* Element (row, col) of a weight tensor viewed as [rows_total, cols]. */
static double w_at(const moe_ref_mat *m, int w_dtype, size_t row, size_t col, size_t cols) {
    size_t i = row * cols + col;
    switch (w_dtype) {
    case MOE_REF_DT_F32: return (double)((const float *)m->q)[i];
    case MOE_REF_DT_BF16: return bf16_to_f64(((const uint16_t *)m->q)[i]);
    default: /* int8 quant times its block's fp16 scale; exact in fp64 */
        return f16_to_f64(m->scale[row * (cols / 32) + col / 32]) * (double)((const int8_t *)m->q)[i];
    }
}

/* ------------------------------------------------------------------------ */
/* Validation.                                                                */
/* ------------------------------------------------------------------------ */

static int check_config(const moe_ref_config *c) {
    if (!c) return MOE_REF_ERR_INVALID;
    if (c->n_tokens < 1 || c->d_model < 1 || c->d_ff < 1) return MOE_REF_ERR_INVALID;
    if (c->n_expert < 1 || c->n_expert > 1024) return MOE_REF_ERR_INVALID;
    if (c->top_k < 1 || c->top_k > c->n_expert || c->top_k > 32) return MOE_REF_ERR_INVALID;
    if (c->n_shared != 0 && c->n_shared != 1) return MOE_REF_ERR_INVALID;
    if (c->n_shared == 1 && c->d_ff_shared < 1) return MOE_REF_ERR_INVALID;
    if (c->score != MOE_REF_SCORE_SIGMOID && c->score != MOE_REF_SCORE_SQRT_SOFTPLUS)
        return MOE_REF_ERR_INVALID;
    if (!(c->route_scale > 0.0f) || isinf(c->route_scale)) return MOE_REF_ERR_INVALID;
    if (c->act_dtype < 0 || c->act_dtype > 1 || c->w_dtype < 0 || c->w_dtype > 2)
        return MOE_REF_ERR_INVALID;
    int ok = (c->act_dtype == MOE_REF_DT_F32 && c->w_dtype == MOE_REF_DT_F32) ||
             (c->act_dtype == MOE_REF_DT_BF16 && c->w_dtype == MOE_REF_DT_BF16) ||
             (c->act_dtype == MOE_REF_DT_BF16 && c->w_dtype == MOE_REF_DT_Q8B32);
    if (!ok) return MOE_REF_ERR_UNSUPPORTED;
    if (c->w_dtype == MOE_REF_DT_Q8B32 &&
        (c->d_model % 32 || c->d_ff % 32 || (c->n_shared && c->d_ff_shared % 32)))
        return MOE_REF_ERR_UNSUPPORTED;
    return MOE_REF_OK;
}

static int check_mat(const moe_ref_mat *m, int w_dtype) {
    if (!m->q) return 0;
    if (w_dtype == MOE_REF_DT_Q8B32 && !m->scale) return 0;
    return 1;
}

static int check_weights(const moe_ref_config *c, const moe_ref_weights *w, int need_router) {
    if (!w) return MOE_REF_ERR_INVALID;
    if (need_router && !w->w_router) return MOE_REF_ERR_INVALID;
    if (!check_mat(&w->gate, c->w_dtype) || !check_mat(&w->up, c->w_dtype) ||
        !check_mat(&w->down, c->w_dtype))
        return MOE_REF_ERR_INVALID;
    if (c->n_shared && (!check_mat(&w->s_gate, c->w_dtype) || !check_mat(&w->s_up, c->w_dtype) ||
                        !check_mat(&w->s_down, c->w_dtype)))
        return MOE_REF_ERR_INVALID;
    return MOE_REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Router: logits, scores, selection, weights.                               */
/* ------------------------------------------------------------------------ */

/* Logit of one (token, expert): fp64 sum in ascending i, rounded once.  Every
 * product (bf16 or fp32 times fp32) is exact in fp64. */
static float logit_of(const moe_ref_config *c, const void *x, const float *wr, int t, int e) {
    const size_t d = (size_t)c->d_model;
    double acc = 0.0;
    for (size_t i = 0; i < d; ++i)
        acc += act_at(x, c->act_dtype, (size_t)t * d + i) * (double)wr[(size_t)e * d + i];
    return (float)acc;
}

/* Score of one logit, evaluated in fp64 and rounded once to fp32.
 * sigmoid(l) = 1/(1+exp(-l)); softplus(l) = ln(1+exp(l)), written as
 * l + log1p(exp(-l)) for l > 0 so that large l does not overflow. */
float moe_ref_score(int32_t score, float logit) {
    double l = (double)logit;
    if (score == MOE_REF_SCORE_SIGMOID) {
#if ORACLE_MUTANT == 7 /* planted: sign error in the sigmoid */
        return (float)(1.0 / (1.0 + exp(l)));
#else
        return (float)(1.0 / (1.0 + exp(-l)));
#endif
    }
    double sp = l > 0.0 ? l + log1p(exp(-l)) : log1p(exp(l));
#if ORACLE_MUTANT == 8 /* planted: square root dropped */
    return (float)sp;
#else
    return (float)sqrt(sp);
#endif
}

/* Total order used for selection: a precedes b when its key is larger, or the
 * keys are equal and its index is lower.  NaN keys come after every number
 * (ordered among themselves by index); -0 and +0 compare equal. */
static int precedes(float ka, int a, float kb, int b) {
    int na = isnan(ka), nb = isnan(kb);
#if ORACLE_MUTANT == 11 /* planted: NaN ranked first */
    if (na != nb) return na;
#else
    if (na != nb) return nb;
#endif
    if (!na) {
        if (ka > kb) return 1;
        if (ka < kb) return 0;
    }
#if ORACLE_MUTANT == 1 /* planted: ties broken toward the higher index */
    return a > b;
#else
    return a < b;
#endif
}

/* Selection and weights of one token from its logits row. */
static void select_token(const moe_ref_config *c, const float *lrow, const float *bias,
                         int32_t *idx, float *wout, float *s, float *key, unsigned char *taken) {
    const int E = c->n_expert, k = c->top_k;
    for (int e = 0; e < E; ++e) {
        s[e] = moe_ref_score(c->score, lrow[e]);
        key[e] = bias ? s[e] + bias[e] : s[e]; /* one fp32 addition */
        taken[e] = 0;
    }
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e)
            if (!taken[e] && (best < 0 || precedes(key[e], e, key[best], best))) best = e;
        taken[best] = 1;
        idx[j] = best;
    }
    double S = 0.0;
    for (int j = 0; j < k; ++j) {
#if ORACLE_MUTANT == 3 /* planted: bias leaks into the weights */
        S += (double)key[idx[j]];
#else
        S += (double)s[idx[j]];
#endif
    }
    for (int j = 0; j < k; ++j) {
#if ORACLE_MUTANT == 3
        double sj = (double)key[idx[j]];
#else
        double sj = (double)s[idx[j]];
#endif
#if ORACLE_MUTANT == 4 /* planted: scale applied before renormalising (it cancels) */
        double Ss = 0.0;
        for (int m = 0; m < k; ++m) Ss += (double)s[idx[m]] * (double)c->route_scale;
        wout[j] = Ss > 0.0 ? (float)(sj * (double)c->route_scale / Ss) : 0.0f;
#else
        wout[j] = S > 0.0 ? (float)((sj / S) * (double)c->route_scale) : 0.0f;
#endif
    }
}

static int select_all(const moe_ref_config *c, const float *logits, const float *bias,
                      int32_t *topk_idx, float *topk_w) {
    const int T = c->n_tokens, E = c->n_expert, k = c->top_k;
    int fail = 0;
#pragma omp parallel
    {
        float *s = malloc(sizeof(float) * (size_t)E), *key = malloc(sizeof(float) * (size_t)E);
        unsigned char *taken = malloc((size_t)E);
        if (!s || !key || !taken) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(static)
            for (int t = 0; t < T; ++t)
                select_token(c, logits + (size_t)t * E, bias, topk_idx + (size_t)t * k,
                             topk_w + (size_t)t * k, s, key, taken);
        }
        free(s);
        free(key);
        free(taken);
    }
    return fail ? MOE_REF_ERR_INVALID : MOE_REF_OK;
}

int moe_ref_select(const moe_ref_config *cfg, const float *logits, const float *bias,
                   int32_t *topk_idx, float *topk_w) {
    int st = check_config(cfg);
    if (st) return st;
    if (!logits || !topk_idx || !topk_w) return MOE_REF_ERR_INVALID;
    return select_all(cfg, logits, bias, topk_idx, topk_w);
}

static void compute_logits(const moe_ref_config *c, const void *x, const float *wr, float *logits) {
    const int T = c->n_tokens, E = c->n_expert;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
#if ORACLE_MUTANT == 9 /* planted: router weights read transposed */
            const size_t d = (size_t)c->d_model;
            double acc = 0.0;
            for (size_t i = 0; i < d; ++i)
                acc += act_at(x, c->act_dtype, (size_t)t * d + i) *
                       (double)wr[(i * (size_t)E + (size_t)e) % ((size_t)E * d)];
            logits[(size_t)t * E + e] = (float)acc;
#else
            logits[(size_t)t * E + e] = logit_of(c, x, wr, t, e);
#endif
        }
}

int moe_ref_route(const moe_ref_config *cfg, const void *x, const float *w_router, const float *bias,
                  float *logits, int32_t *topk_idx, float *topk_w) {
    int st = check_config(cfg);
    if (st) return st;
    if (!x || !w_router || !topk_idx || !topk_w) return MOE_REF_ERR_INVALID;
    const size_t n = (size_t)cfg->n_tokens * (size_t)cfg->n_expert;
    float *lg = logits ? logits : malloc(sizeof(float) * n);
    if (!lg) return MOE_REF_ERR_INVALID;
    compute_logits(cfg, x, w_router, lg);
    st = select_all(cfg, lg, bias, topk_idx, topk_w);
    if (!logits) free(lg);
    return st;
}

/* Row top-k over long candidate rows (the sparse attention indexer's top-512 /
 * top-1024 selection, "256 experts, 512 lines" blog post, section "The constant
 * that always said 256").  Definition: under the selection order of precedes()
 * the k chosen candidates of a row are its first k; they are listed by
 * ascending candidate index. */
typedef struct { float v; int32_t i; } ref_cand;

static int cand_cmp(const void *pa, const void *pb) {
    const ref_cand *a = pa, *b = pb;
    if (precedes(a->v, a->i, b->v, b->i)) return -1;
    if (precedes(b->v, b->i, a->v, a->i)) return 1;
    return 0;
}

int moe_ref_topk_rows(int32_t rows, int32_t n, int32_t k, const float *scores, int32_t *idx,
                      float *vals) {
    if (rows < 0 || n < 1 || k < 1 || k > n) return MOE_REF_ERR_INVALID;
    if (rows > 0 && (!scores || !idx)) return MOE_REF_ERR_INVALID;
    int failed = 0;
#pragma omp parallel for schedule(dynamic)
    for (int r = 0; r < rows; ++r) {
        ref_cand *c = malloc(sizeof(ref_cand) * (size_t)n);
        unsigned char *taken = calloc((size_t)n, 1);
        if (!c || !taken) {
#pragma omp atomic write
            failed = 1;
        } else {
            const float *row = scores + (size_t)r * n;
            for (int i = 0; i < n; ++i) {
                c[i].v = row[i];
                c[i].i = i;
            }
            qsort(c, (size_t)n, sizeof(ref_cand), cand_cmp);
            for (int j = 0; j < k; ++j) {
#if ORACLE_MUTANT == 12 /* planted: the k-th and (k+1)-th candidates swapped */
                const int jj = (j == k - 1 && k < n) ? k : j;
                taken[c[jj].i] = 1;
#else
                taken[c[j].i] = 1;
#endif
            }
            int o = 0;
            for (int i = 0; i < n; ++i)
                if (taken[i]) {
                    idx[(size_t)r * k + o] = i;
                    if (vals) vals[(size_t)r * k + o] = row[i];
                    ++o;
                }
        }
        free(c);
        free(taken);
    }
    return failed ? MOE_REF_ERR_INVALID : MOE_REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Permutation: stable counting sort of assignments by expert.               */
/* ------------------------------------------------------------------------ */

int moe_ref_permute(const moe_ref_config *cfg, const int32_t *topk_idx, int32_t *offsets,
                    int32_t *perm_rows, int32_t *inv_perm) {
    int st = check_config(cfg);
    if (st) return st;
    if (!topk_idx || !offsets || !perm_rows || !inv_perm) return MOE_REF_ERR_INVALID;
    const int E = cfg->n_expert;
    const long n = (long)cfg->n_tokens * cfg->top_k;
    long pos = 0;
    for (int e = 0; e < E; ++e) {
        offsets[e] = (int32_t)pos;
#if ORACLE_MUTANT == 2 /* planted: unstable order inside an expert's segment */
        for (long f = n - 1; f >= 0; --f)
#else
        for (long f = 0; f < n; ++f)
#endif
            if (topk_idx[f] == e) perm_rows[pos++] = (int32_t)f;
    }
    offsets[E] = (int32_t)pos;
    for (long r = pos; r < n; ++r) perm_rows[r] = -1;
    for (long f = 0; f < n; ++f) inv_perm[f] = -1;
    for (long r = 0; r < pos; ++r) inv_perm[perm_rows[r]] = (int32_t)r;
    return MOE_REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Expert FFN (SwiGLU) and combine.                                           */
/* ------------------------------------------------------------------------ */

/* o[0..d) = FFN of one token through expert `e` of (gate, up, down), fp64.
 * g_r, u_r: fp64 sums over i ascending; a_r = silu(g_r) * u_r with
 * silu(g) = g / (1 + exp(-g)); h_r = a_r rounded to the activation format;
 * o_i: fp64 sum over r ascending.  h: scratch of f doubles. */
static void expert_ffn_token(const moe_ref_config *c, const void *x, int t, const moe_ref_mat *g,
                             const moe_ref_mat *u, const moe_ref_mat *dn, int e, int f, double *h,
                             double *o) {
    const size_t d = (size_t)c->d_model;
    for (int r = 0; r < f; ++r) {
        double gs = 0.0, us = 0.0;
        const size_t row = (size_t)e * (size_t)f + (size_t)r;
        for (size_t i = 0; i < d; ++i) {
            double xi = act_at(x, c->act_dtype, (size_t)t * d + i);
            gs += xi * w_at(g, c->w_dtype, row, i, d);
            us += xi * w_at(u, c->w_dtype, row, i, d);
        }
        double a = gs / (1.0 + exp(-gs)) * us;
        h[r] = round_h(a, c->act_dtype);
    }
    for (size_t i = 0; i < d; ++i) {
        double acc = 0.0;
        const size_t row = (size_t)e * d + i;
        for (int r = 0; r < f; ++r) {
#if ORACLE_MUTANT == 10 /* planted: down projection indexed transposed */
            acc += w_at(dn, c->w_dtype, ((size_t)e * d + (size_t)r % d), i % (size_t)f, (size_t)f) * h[r];
#else
            acc += w_at(dn, c->w_dtype, row, (size_t)r, (size_t)f) * h[r];
#endif
        }
        o[i] = acc;
    }
}

/* Expert of each flat assignment, recovered from the permutation. */
static int expert_of_slots(const moe_ref_config *c, const int32_t *offsets, const int32_t *perm_rows,
                           int32_t *eslot) {
    const long n = (long)c->n_tokens * c->top_k;
    for (long f = 0; f < n; ++f) eslot[f] = -1;
    if (offsets[0] != 0 || offsets[c->n_expert] > n) return MOE_REF_ERR_INVALID;
    for (int e = 0; e < c->n_expert; ++e) {
        if (offsets[e + 1] < offsets[e]) return MOE_REF_ERR_INVALID;
        for (long r = offsets[e]; r < offsets[e + 1]; ++r) {
            long f = perm_rows[r];
            if (f < 0 || f >= n) return MOE_REF_ERR_INVALID;
            eslot[f] = e;
        }
    }
    return MOE_REF_OK;
}

int moe_ref_expert_ffn(const moe_ref_config *cfg, const void *x, const moe_ref_weights *w,
                       const int32_t *offsets, const int32_t *perm_rows, const float *topk_w,
                       float *slot_out, float *shared_out) {
    int st = check_config(cfg);
    if (st) return st;
    if ((st = check_weights(cfg, w, 0))) return st;
    if (!x || !offsets || !perm_rows || !topk_w || !slot_out) return MOE_REF_ERR_INVALID;
    if (cfg->n_shared && !shared_out) return MOE_REF_ERR_INVALID;
    const int T = cfg->n_tokens, k = cfg->top_k, d = cfg->d_model;
    int32_t *eslot = malloc(sizeof(int32_t) * (size_t)T * (size_t)k);
    if (!eslot) return MOE_REF_ERR_INVALID;
    if ((st = expert_of_slots(cfg, offsets, perm_rows, eslot))) {
        free(eslot);
        return st;
    }
    const int fmax = cfg->d_ff > cfg->d_ff_shared ? cfg->d_ff : cfg->d_ff_shared;
#pragma omp parallel
    {
        double *h = malloc(sizeof(double) * (size_t)fmax), *o = malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic)
        for (int t = 0; t < T; ++t) {
            for (int j = 0; j < k; ++j) {
                const size_t f = (size_t)t * k + (size_t)j;
                float *dst = slot_out + f * (size_t)d;
                if (eslot[f] < 0) {
                    for (int i = 0; i < d; ++i) dst[i] = 0.0f;
                    continue;
                }
                expert_ffn_token(cfg, x, t, &w->gate, &w->up, &w->down, eslot[f], cfg->d_ff, h, o);
                for (int i = 0; i < d; ++i) dst[i] = (float)((double)topk_w[f] * o[i]);
            }
            if (cfg->n_shared) {
                expert_ffn_token(cfg, x, t, &w->s_gate, &w->s_up, &w->s_down, 0, cfg->d_ff_shared,
                                 h, o);
                for (int i = 0; i < d; ++i) shared_out[(size_t)t * d + i] = (float)o[i];
            }
        }
        free(h);
        free(o);
    }
    free(eslot);
    return MOE_REF_OK;
}

int moe_ref_combine(const moe_ref_config *cfg, const float *slot_out, const float *shared_out,
                    float *y) {
    int st = check_config(cfg);
    if (st) return st;
    if (!slot_out || !y) return MOE_REF_ERR_INVALID;
    const int T = cfg->n_tokens, k = cfg->top_k, d = cfg->d_model;
    for (int t = 0; t < T; ++t)
        for (int i = 0; i < d; ++i) {
            double acc = shared_out ? (double)shared_out[(size_t)t * d + i] : 0.0;
            for (int j = 0; j < k; ++j) acc += (double)slot_out[((size_t)t * k + j) * d + i];
            y[(size_t)t * d + i] = (float)acc;
        }
    return MOE_REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Whole layer, token-major, straight from the definition.                   */
/* ------------------------------------------------------------------------ */

int moe_ref_layer_forward(const moe_ref_config *cfg, const void *x, const moe_ref_weights *w,
                          float *y, moe_ref_debug *dbg) {
    int st = check_config(cfg);
    if (st) return st;
    if ((st = check_weights(cfg, w, 1))) return st;
    if (!x || !y) return MOE_REF_ERR_INVALID;
    const int T = cfg->n_tokens, E = cfg->n_expert, k = cfg->top_k, d = cfg->d_model;
    float *logits = malloc(sizeof(float) * (size_t)T * E);
    int32_t *idx = malloc(sizeof(int32_t) * (size_t)T * k);
    float *wt = malloc(sizeof(float) * (size_t)T * k);
    if (!logits || !idx || !wt) {
        free(logits);
        free(idx);
        free(wt);
        return MOE_REF_ERR_INVALID;
    }
    compute_logits(cfg, x, w->w_router, logits);
    st = select_all(cfg, logits, w->bias, idx, wt);
    const int fmax = cfg->d_ff > cfg->d_ff_shared ? cfg->d_ff : cfg->d_ff_shared;
    if (!st) {
#pragma omp parallel
        {
            double *h = malloc(sizeof(double) * (size_t)fmax);
            double *o = malloc(sizeof(double) * (size_t)d), *acc = malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic)
            for (int t = 0; t < T; ++t) {
                for (int i = 0; i < d; ++i) acc[i] = 0.0;
#if ORACLE_MUTANT != 6 /* planted (6): shared expert dropped */
                if (cfg->n_shared) {
                    expert_ffn_token(cfg, x, t, &w->s_gate, &w->s_up, &w->s_down, 0,
                                     cfg->d_ff_shared, h, o);
                    for (int i = 0; i < d; ++i) acc[i] = o[i];
                }
#endif
                for (int j = 0; j < k; ++j) {
                    const size_t f = (size_t)t * k + (size_t)j;
                    expert_ffn_token(cfg, x, t, &w->gate, &w->up, &w->down, idx[f], cfg->d_ff, h, o);
                    for (int i = 0; i < d; ++i) acc[i] += (double)wt[f] * o[i];
                }
                for (int i = 0; i < d; ++i) y[(size_t)t * d + i] = (float)acc[i];
            }
            free(h);
            free(o);
            free(acc);
        }
    }
    if (!st && dbg) {
        if (dbg->logits) memcpy(dbg->logits, logits, sizeof(float) * (size_t)T * E);
        if (dbg->topk_idx) memcpy(dbg->topk_idx, idx, sizeof(int32_t) * (size_t)T * k);
        if (dbg->topk_w) memcpy(dbg->topk_w, wt, sizeof(float) * (size_t)T * k);
        if (dbg->offsets && dbg->perm_rows && dbg->inv_perm)
            st = moe_ref_permute(cfg, idx, dbg->offsets, dbg->perm_rows, dbg->inv_perm);
    }
    free(logits);
    free(idx);
    free(wt);
    return st;
}

/* ------------------------------------------------------------------------ */
/* Dense SwiGLU through one expert, written out separately for the identity  */
/* (with one expert, top-1 and no shared expert the layer reduces to it).     */
/* ------------------------------------------------------------------------ */

int moe_ref_dense_swiglu(int32_t n_tokens, int32_t d_model, int32_t d_ff, int32_t act_dtype,
                         int32_t w_dtype, const void *x, moe_ref_mat gate, moe_ref_mat up,
                         moe_ref_mat down, int32_t expert, double *y64) {
    if (n_tokens < 1 || d_model < 1 || d_ff < 1 || expert < 0 || !x || !y64) return MOE_REF_ERR_INVALID;
    if (!check_mat(&gate, w_dtype) || !check_mat(&up, w_dtype) || !check_mat(&down, w_dtype))
        return MOE_REF_ERR_INVALID;
    const size_t D = (size_t)d_model, F = (size_t)d_ff;
    double *hid = malloc(sizeof(double) * F);
    if (!hid) return MOE_REF_ERR_INVALID;
    for (int t = 0; t < n_tokens; ++t) {
        for (size_t r = 0; r < F; ++r) {
            double gate_r = 0.0, up_r = 0.0;
            for (size_t i = 0; i < D; ++i) {
                const double xv = act_at(x, act_dtype, (size_t)t * D + i);
                gate_r += xv * w_at(&gate, w_dtype, (size_t)expert * F + r, i, D);
                up_r += xv * w_at(&up, w_dtype, (size_t)expert * F + r, i, D);
            }
            const double a = gate_r / (1.0 + exp(-gate_r)) * up_r; /* silu(g) * u */
            hid[r] = act_dtype == MOE_REF_DT_F32 ? (double)(float)a
                                                 : bf16_to_f64(moe_ref_bf16_from_f64(a));
        }
        for (size_t i = 0; i < D; ++i) {
            double s = 0.0;
            for (size_t r = 0; r < F; ++r) s += w_at(&down, w_dtype, (size_t)expert * D + i, r, F) * hid[r];
            y64[(size_t)t * D + i] = s;
        }
    }
    free(hid);
    return MOE_REF_OK;
}
