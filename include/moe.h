/*
 * moe.h - C ABI of the MI355X (gfx950) sparse Mixture-of-Experts layer forward.
 *
 * One MoE layer: a router scores every token against n_expert experts, keeps
 * the top-k, renormalises their weights; the token rows are grouped by expert;
 * each selected expert applies a SwiGLU FFN; an always-on shared expert is
 * added; the weighted results return to token order.
 *
 *   logits  l[t,e] = sum_i x[t,i] * Wr[e,i]            (row stride n_expert)
 *   score   s = sigmoid(l)  or  s = sqrt(softplus(l))
 *   key     s + bias[e]  (bias optional; it selects, it never weights)
 *   select  top-k keys; equal keys -> lower expert index first; NaN last
 *   weight  w_j = route_scale * s_j / sum over the selected s
 *   FFN_e   Wd[e] . (silu(Wg[e] x) * (Wu[e] x)),  silu(g) = g / (1 + e^-g)
 *   y[t]    FFN_shared(x_t) + sum_j w_j FFN_{e_j}(x_t)
 *
 * Sources: "256 experts, 512 lines" blog post - section "Why GLM-5.2 in an
 * engine built for DeepSeek" (sigmoid routing, top-8, MoE with a shared
 * expert) and section "The constant that always said 256" (sqrt(softplus)
 * scores, top-6, the 1.5 scale, logits addressed with stride n_expert and
 * n_expert a runtime value, a parallel top-k rather than a serial one);
 * NeutronStar README, main branch - Hy3 paragraph (sigmoid scores plus a
 * per-expert bias choosing 8 of 192 experts, and a shared expert); NeutronStar README - "The model"
 * (decision tensors kept at Q8_0/F32), "GLM-5.2 CUDA port" (gate/up and down
 * projection kernels) and the MTP paragraph (only the selected experts' weights
 * are read for small batches; batch kernels address whole [E, rows, cols]
 * expert tensors).
 *
 * Conventions for every entry point
 *  - Pointers are DEVICE pointers owned by the caller; the library never
 *    allocates, frees or synchronises.  `stream` is a hipStream_t (NULL = the
 *    null stream); all work is enqueued on it and the call returns at once.
 *  - Every call validates its arguments first.  On failure it returns a
 *    nonzero moe_status and enqueues nothing.  MOE_ERR_DEVICE reports a launch
 *    error seen right after enqueueing; faults inside kernels surface at the
 *    caller's next synchronisation.
 *  - Activations (x), weight tensors, router weights, slot_out, shared_out,
 *    y and the workspace must be 16-byte aligned; the per-element arrays
 *    (bias, logits, topk_idx, topk_w, offsets, perm_rows, inv_perm) need
 *    4-byte alignment.  Sizes are element counts.
 *  - Layouts are row-major.  Weight tensors are [n, rows, cols] with cols the
 *    reduction dimension.  bf16 and fp16 values are passed as their bit
 *    patterns (uint16).  Q8B32 = int8 quants [n, rows, cols] plus one fp16
 *    scale per 32 consecutive columns [n, rows, cols/32]; weight = scale * q.
 *  - Results: expert indices and the permutation are exact and do not depend
 *    on the path taken; logits and scores are accumulated in fp64 and rounded
 *    once to fp32; the SwiGLU intermediate is rounded to the activation format
 *    (bf16, or fp32 for fp32 layers); y is fp32.
 *  - The workspace (`ws`, `ws_bytes`) is caller-owned scratch of at least
 *    moe_workspace_bytes(cfg) bytes.  It needs no initialisation: every call
 *    writes each workspace word before reading it.  Calls that share a
 *    workspace must not overlap.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID = 1,     /* NULL/misaligned pointer, value out of range, bad enum */
    MOE_ERR_UNSUPPORTED = 2, /* valid but not provided: dtype pair, d/F not multiples of 64, path */
    MOE_ERR_WORKSPACE = 3,   /* ws_bytes < moe_workspace_bytes(cfg) */
    MOE_ERR_DEVICE = 4       /* the HIP runtime refused a launch */
} moe_status;

typedef enum { MOE_SCORE_SIGMOID = 0, MOE_SCORE_SQRT_SOFTPLUS = 1 } moe_score;
typedef enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1, MOE_DT_Q8B32 = 2 } moe_dtype;
typedef enum { MOE_PATH_AUTO = 0, MOE_PATH_DECODE = 1, MOE_PATH_PREFILL = 2 } moe_path;

/* Largest token count the decode path accepts (MOE_PATH_AUTO takes it for
 * n_tokens <= MOE_DECODE_MAX_TOKENS). */
#define MOE_DECODE_MAX_TOKENS 8

typedef struct {
    int32_t n_tokens;    /* T >= 1 */
    int32_t d_model;     /* d: multiple of 64 */
    int32_t n_expert;    /* E in [1, 1024], a runtime value */
    int32_t top_k;       /* k in [1, min(E, 32)] */
    int32_t d_ff;        /* F: routed expert hidden size, multiple of 64 */
    int32_t n_shared;    /* 0 or 1 shared expert */
    int32_t d_ff_shared; /* Fs: shared expert hidden size, multiple of 64 (if n_shared) */
    int32_t score;       /* moe_score */
    float route_scale;   /* finite, > 0: 1.5 for the sqrt(softplus) router, 1.0 for sigmoid */
    int32_t act_dtype;   /* moe_dtype of x and of the SwiGLU intermediate: F32 or BF16 */
    int32_t w_dtype;     /* moe_dtype of the expert weights: (F32,F32) (BF16,BF16) (BF16,Q8B32) */
    int32_t path;        /* moe_path, used by moe_layer_forward */
} moe_config;

typedef struct {
    const void *q;          /* [n, rows, cols] elements of w_dtype (int8 for Q8B32) */
    const uint16_t *scale;  /* Q8B32 only: fp16 bits [n, rows, cols/32]; else ignored */
} moe_mat;

typedef struct {
    const float *w_router;  /* [E, d] fp32 */
    const float *bias;      /* [E] fp32 or NULL */
    moe_mat gate, up;       /* [E, F, d] */
    moe_mat down;           /* [E, d, F] */
    moe_mat s_gate, s_up;   /* [1, Fs, d]   (ignored when n_shared == 0) */
    moe_mat s_down;         /* [1, d, Fs] */
} moe_weights;

/* Stages of moe_layer_forward whose kernels a caller can time: 0 router
 * logits, 1 top-k selection, 2 permutation, 3 gate/up (SwiGLU), 4 down
 * projection, 5 combine.  The decode path (n_tokens <= MOE_DECODE_MAX_TOKENS)
 * builds the permutation inside the selection kernel and the combine inside
 * the down kernel: it launches no kernel for stages 2 and 5 and leaves their
 * events unrecorded. */
#define MOE_STAGES 6
#define MOE_STAGE_EVENTS (2 * MOE_STAGES)

/* Optional outputs of moe_layer_forward; any field may be NULL. */
typedef struct {
    float *logits;      /* [T, E] */
    int32_t *topk_idx;  /* [T, k] */
    float *topk_w;      /* [T, k] */
    int32_t *offsets;   /* [E+1] */
    int32_t *perm_rows; /* [T*k] */
    int32_t *inv_perm;  /* [T*k] */
    void **stage_events; /* NULL, or MOE_STAGE_EVENTS hipEvent_t created by the caller (entries
                            may be NULL): [2s] receives the start timestamp of stage s's first
                            kernel dispatch, [2s+1] the end timestamp of its last (the dispatch's
                            own timestamps, via hipExtLaunchKernel), so the elapsed time between
                            them is the stage's kernel time without the launch gaps around it */
} moe_debug;

/* Bytes of workspace every entry point below may use for this config
 * (0 if the config is invalid).  Monotone in every size field. */
size_t moe_workspace_bytes(const moe_config *cfg);

/* Router: logits (optional, [T,E]) and the top-k selection.
 * x [T, d] act_dtype; w_router [E, d] fp32; bias [E] or NULL;
 * topk_idx [T, k] int32 in rank order; topk_w [T, k] fp32. */
int moe_route(const moe_config *cfg, const void *x, const float *w_router, const float *bias,
              float *logits, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
              void *stream);

/* Selection alone, from given fp32 logits [T, E] (row stride n_expert).
 * n_expert == 256 runs a compile-time 256-expert instantiation of the top-k;
 * cfg->path == MOE_PATH_PREFILL forces the runtime-n_expert kernel instead
 * (both give identical results; the switch exists so that can be checked). */
int moe_select(const moe_config *cfg, const float *logits, const float *bias, int32_t *topk_idx,
               float *topk_w, void *stream);

/* Token->expert grouping: a stable counting sort of the flat assignments
 * f = t*k + j by expert.  offsets [E+1] (exclusive prefix sum of the expert
 * counts); perm_rows [T*k]: the f of every assignment, ordered by (expert, f);
 * inv_perm [T*k]: position of f in perm_rows.  Indices outside [0, E) are left
 * out: inv_perm = -1, and the unused tail of perm_rows is -1. */
int moe_permute(const moe_config *cfg, const int32_t *topk_idx, int32_t *offsets,
                int32_t *perm_rows, int32_t *inv_perm, void *ws, size_t ws_bytes, void *stream);

/* Routed and shared experts.  slot_out [T*k, d] fp32: row f = w_f *
 * FFN_{expert of f}(x_t); shared_out [T, d] fp32 = FFN_shared(x_t), or NULL
 * when n_shared == 0.  offsets / perm_rows as produced by moe_permute; topk_w
 * [T, k].  Rows of assignments that perm_rows does not list are not written.
 * Offsets that are not a monotone split of [0, T*k] (checked on the device)
 * leave every slot row unwritten; the shared expert is still computed. */
int moe_expert_ffn(const moe_config *cfg, const void *x, const moe_weights *w,
                   const int32_t *offsets, const int32_t *perm_rows, const float *topk_w,
                   float *slot_out, float *shared_out, void *ws, size_t ws_bytes, void *stream);

/* y [T, d] fp32 = shared_out[t] (if not NULL) + sum_j slot_out[t*k + j]. */
int moe_combine(const moe_config *cfg, const float *slot_out, const float *shared_out, float *y,
                void *stream);

/* The whole layer: route, group, experts, combine.  y [T, d] fp32.
 * cfg->path picks the decode path (GEMV over the selected experts' weights,
 * combine fused; n_tokens <= MOE_DECODE_MAX_TOKENS) or the prefill path
 * (grouped GEMMs, bf16 on MFMA); MOE_PATH_AUTO chooses by n_tokens. */
int moe_layer_forward(const moe_config *cfg, const void *x, const moe_weights *w, float *y,
                      moe_debug *dbg, void *ws, size_t ws_bytes, void *stream);

/* moe_layer_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and kernels as moe_layer_forward, but
 * no caller workspace: the library's own static device array of
 * MOE_STATIC_SCRATCH_BYTES serves instead (one per GPU, held from the first
 * call on that GPU until the process ends; the current device's copy is used,
 * so `stream` must belong to the current device).  A config whose
 * moe_workspace_bytes exceeds MOE_STATIC_SCRATCH_BYTES returns
 * MOE_ERR_WORKSPACE and enqueues nothing (64 MiB covers every decode config
 * here and prefill batches of a few hundred tokens at d_model 4096-6144).
 * This call never allocates or frees.  Every call on one GPU shares that GPU's
 * array, which keeps the last call's contents (nothing in it needs to start
 * at zero: each call writes every word before reading it), so calls that
 * overlap on one GPU - on two streams, or from two host threads without
 * ordering - race and must not be issued.  MOE_ERR_DEVICE if the array's
 * device address cannot be obtained. */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)
int moe_layer_forward_noalloc(const moe_config *cfg, const void *x, const moe_weights *w, float *y,
                              moe_debug *dbg, void *stream);

/* Top-k over long candidate rows: the sparse attention indexer's selection of
 * the best 512 or 1024 entries of a long score row ("256 experts, 512 lines"
 * blog post, section "The constant that always said 256"), with the order of
 * the expert selection above.  For each of `rows` rows of scores [rows, n]
 * fp32, the k candidates that come first (larger score first, NaN after every
 * number, -0 equal to +0, equal scores by lower candidate index) go to
 * idx [rows, k] int32, listed by ascending candidate index, and their scores,
 * bit for bit, to vals [rows, k] fp32 (vals may be NULL).
 * 1 <= k <= n <= MOE_TOPK_ROWS_MAX_N and rows >= 0 (0 enqueues nothing), else
 * MOE_ERR_INVALID; scores, idx and vals need 4-byte alignment.  No workspace.
 * events: NULL, or 2 hipEvent_t created by the caller (entries may be NULL)
 * that receive the start and end timestamps of the kernel dispatch. */
#define MOE_TOPK_ROWS_MAX_N 65536
int moe_topk_rows(const float *scores, int32_t rows, int32_t n, int32_t k, int32_t *idx, float *vals,
                  void **events, void *stream);

/* Router look-ahead, its read half (NeutronStar fork page, "Cross-layer
 * expert prefetch": the next layer's router runs on this layer's hidden
 * state and the experts it predicts are read while the GPU still computes).
 * The predictions come from moe_route called with the next layer's router
 * weights on this layer's input x; this call then reads the weights of the
 * experts ids [n_ids] int32 (device memory, e.g. that topk_idx; entries
 * outside [0, n_expert) are skipped on the device) of the layer w: bit 0 of
 * `which` selects gate, bit 1 up, bit 2 down (for MOE_DT_Q8B32 the codes
 * and their scales), and `rows` > 0 limits the read to the leading rows of
 * each selected matrix (gate and up have d_ff rows, down d_model; 0: all).
 * It writes no memory, so no result of any call changes; the reads leave
 * those weights in the device's memory-side cache (the Infinity Cache),
 * where that layer's expert kernels find them if they run before other
 * traffic evicts them.  Meant for a second stream, beside the work of the
 * current layer: `workgroups` (1 .. MOE_PREFETCH_MAX_WORKGROUPS) fixes the
 * launch's size, so that it takes only part of the chip.
 * 0 <= n_ids <= MOE_PREFETCH_MAX_IDS (0 enqueues nothing), 1 <= which <= 7,
 * rows >= 0, the selected matrices as in moe_weights with their scale
 * arrays (MOE_DT_Q8B32) 16-byte aligned too, else MOE_ERR_INVALID;
 * an expert matrix of more than 2^31 - 1 bytes is MOE_ERR_UNSUPPORTED.  No
 * workspace.  events: NULL, or 2 hipEvent_t created by the caller (entries
 * may be NULL) that receive the start and end timestamps of the dispatch. */
#define MOE_PREFETCH_MAX_IDS 65536
#define MOE_PREFETCH_MAX_WORKGROUPS 4096
int moe_prefetch_experts(const moe_config *cfg, const moe_weights *w, const int32_t *ids, int32_t n_ids,
                         int32_t which, int32_t rows, int32_t workgroups, void **events, void *stream);

/* Human-readable name of a status code (static storage). */
const char *moe_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif
