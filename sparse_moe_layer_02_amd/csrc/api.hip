// api.hip - the C ABI of include/moe.h: argument validation (nothing is
// enqueued on failure), the workspace layout, and the choice between the
// decode path (GEMVs over the selected experts) and the prefill path (grouped
// MFMA GEMMs).  All device work is enqueued on the caller's stream; nothing
// here allocates, frees or synchronises.
#include <math.h>
#include <string.h>

#include <mutex>

#include "common.h"
#include "kernels.h"
#include "prefetch.h"
#include "topk_rows.h"

using namespace moe;

namespace {

constexpr int MAX_TOKENS = 1 << 20;

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Arrays read with 16-byte vector loads (activations, weights, the fp32 rows
// of slot/shared/y, the workspace) must be 16-byte aligned; per-element
// arrays (logits, indices, weights of the routing, offsets, permutation,
// bias) need only their element alignment.
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
bool ptr_ok(const void* p) { return p != nullptr && aligned16(p); }
bool opt_ptr_ok(const void* p) { return p == nullptr || aligned16(p); }
bool elt_ok(const void* p) { return p != nullptr && aligned4(p); }
bool opt_elt_ok(const void* p) { return p == nullptr || aligned4(p); }

int validate_config(const moe_config* c) {
    if (!c) return MOE_ERR_INVALID;
    if (c->n_tokens < 1 || c->n_tokens > MAX_TOKENS) return MOE_ERR_INVALID;
    if (c->d_model < 1 || c->d_ff < 1) return MOE_ERR_INVALID;
    if (c->n_expert < 1 || c->n_expert > 1024) return MOE_ERR_INVALID;
    if (c->top_k < 1 || c->top_k > c->n_expert || c->top_k > 32) return MOE_ERR_INVALID;
    if (c->n_shared != 0 && c->n_shared != 1) return MOE_ERR_INVALID;
    if (c->n_shared == 1 && c->d_ff_shared < 1) return MOE_ERR_INVALID;
    if (c->score != MOE_SCORE_SIGMOID && c->score != MOE_SCORE_SQRT_SOFTPLUS) return MOE_ERR_INVALID;
    if (!(c->route_scale > 0.0f) || isinf(c->route_scale)) return MOE_ERR_INVALID;
    if (c->act_dtype < 0 || c->act_dtype > 1 || c->w_dtype < 0 || c->w_dtype > 2) return MOE_ERR_INVALID;
    if (c->path < MOE_PATH_AUTO || c->path > MOE_PATH_PREFILL) return MOE_ERR_INVALID;
    const bool pair_ok = (c->act_dtype == MOE_DT_F32 && c->w_dtype == MOE_DT_F32) ||
                         (c->act_dtype == MOE_DT_BF16 && c->w_dtype == MOE_DT_BF16) ||
                         (c->act_dtype == MOE_DT_BF16 && c->w_dtype == MOE_DT_Q8B32);
    if (!pair_ok) return MOE_ERR_UNSUPPORTED;
    if (c->d_model % 64 || c->d_ff % 64 || (c->n_shared && c->d_ff_shared % 64)) return MOE_ERR_UNSUPPORTED;
    if ((size_t)c->d_model > (1u << 20) || (size_t)c->d_ff > (1u << 20) ||
        (c->n_shared && (size_t)c->d_ff_shared > (1u << 20)))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int ldh_of(const moe_config* c) {
    return c->n_shared ? (c->d_ff > c->d_ff_shared ? c->d_ff : c->d_ff_shared) : c->d_ff;
}

// Rows per grouped-GEMM tile.  256 (the LDS-copy kernels of
// grouped_gemm_dma.hip) once experts average 96 rows or more: a long or skewed
// prefill, where a few hot experts hold most rows (compute-bound) and the
// rest are bandwidth-bound; those kernels compute only the 32-row blocks of a
// tile that hold rows, so a short tile costs its weight stream, not a full
// 256-row product.  Fewer rows per expert: 64-row tiles (every expert
// bandwidth-bound; the register-staged kernels keep more loads in flight per
// CU).  int8 weights always take 64-row tiles (grouped_gemm_q8.hip).
int gemm_bm(const moe_config* c) {
    if (c->w_dtype == MOE_DT_Q8B32) return 64;
    const long n = (long)c->n_tokens * c->top_k;
    return n >= 96L * c->n_expert ? 256 : 64;
}

// Upper bound on the tiles of bm rows: every expert's last tile may be partial.
int max_tiles_of(const moe_config* c, int bm) {
    const long n = (long)c->n_tokens * c->top_k;
    long t = (n + bm - 1) / bm + (n < c->n_expert ? n : c->n_expert);
    if (c->n_shared) t += (c->n_tokens + bm - 1) / bm;
    return (int)t;
}

// Capacity of the decode slot table: the shared expert and at most
// min(E, T*k) routed experts (decode token counts only).
int n_dslots_of(const moe_config* c) {
    if (c->n_tokens > MOE_DECODE_MAX_TOKENS) return 0;
    const int n = c->n_tokens * c->top_k;
    return c->n_shared + (n < c->n_expert ? n : c->n_expert);
}

Layout make_layout(const moe_config* c) {
    Layout L;
    const size_t T = (size_t)c->n_tokens, E = (size_t)c->n_expert, k = (size_t)c->top_k;
    const size_t d = (size_t)c->d_model, n = T * k;
    const size_t hsz = c->act_dtype == MOE_DT_BF16 ? 2 : 4;
    L.n_blk = (int)((n + PERM_BLOCK - 1) / PERM_BLOCK);
    L.max_tiles = max_tiles_of(c, GEMM_BM);  // the smallest tile: capacity for any bm
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align256(o + bytes);
        return at;
    };
    L.logits = take(T * E * 4);
    L.topk_idx = take(n * 4);
    L.topk_w = take(n * 4);
    L.offsets = take((E + 1) * 4);
    L.perm_rows = take(n * 4);
    L.inv_perm = take(n * 4);
    L.blk_hist = take((size_t)L.n_blk * E * 4);
    L.blk_base = take((size_t)L.n_blk * E * 4);
    L.meta = take(META_WORDS * 4);
    L.active = take(E * 4);
    L.tiles = take((size_t)L.max_tiles * 8);
    L.h = take((n + (c->n_shared ? T : 0)) * (size_t)ldh_of(c) * hsz);
    L.slot_out = take(n * d * 4);
    L.shared_out = take(c->n_shared ? T * d * 4 : 0);
    L.scores = take(T * E * 4);
    L.dslots = take((size_t)n_dslots_of(c) * sizeof(DecodeSlot));
    L.total = o;
    return L;
}

template <class P>
P* at(void* ws, size_t off) {
    return reinterpret_cast<P*>(static_cast<uint8_t*>(ws) + off);
}

int check_ws(const moe_config* c, const void* ws, size_t ws_bytes) {
    if (!ws || !aligned16(ws)) return MOE_ERR_INVALID;
    if (ws_bytes < make_layout(c).total) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

bool mat_ok(const moe_config* c, const moe_mat& m) {
    if (!ptr_ok(m.q)) return false;
    if (c->w_dtype == MOE_DT_Q8B32 && (m.scale == nullptr || ((uintptr_t)m.scale & 3u))) return false;
    return true;
}

int check_weights(const moe_config* c, const moe_weights* w, bool router) {
    if (!w) return MOE_ERR_INVALID;
    if (router && (!ptr_ok(w->w_router) || !opt_elt_ok(w->bias))) return MOE_ERR_INVALID;
    if (!mat_ok(c, w->gate) || !mat_ok(c, w->up) || !mat_ok(c, w->down)) return MOE_ERR_INVALID;
    if (c->n_shared && (!mat_ok(c, w->s_gate) || !mat_ok(c, w->s_up) || !mat_ok(c, w->s_down)))
        return MOE_ERR_INVALID;
    return MOE_OK;
}

int device_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

MatRef ref(const moe_mat& m) { return MatRef{m.q, m.scale}; }

PermArgs perm_args(const moe_config* c, const Layout& L, void* ws, const int32_t* idx, int32_t* off,
                   int32_t* perm, int32_t* inv) {
    PermArgs p;
    p.topk_idx = idx;
    p.T = c->n_tokens;
    p.k = c->top_k;
    p.E = c->n_expert;
    p.n_shared = c->n_shared;
    p.offsets = off;
    p.perm_rows = perm;
    p.inv_perm = inv;
    p.blk_hist = at<int32_t>(ws, L.blk_hist);
    p.blk_base = at<int32_t>(ws, L.blk_base);
    p.meta = at<int32_t>(ws, L.meta);
    p.active = at<int32_t>(ws, L.active);
    p.tiles = at<int2>(ws, L.tiles);
    p.n_blk = L.n_blk;
    p.bm = gemm_bm(c);
    return p;
}

FfnArgs ffn_args(const moe_config* c, const Layout& L, void* ws, const void* x, const moe_weights* w,
                 const int32_t* off, const int32_t* perm, const float* topk_w) {
    FfnArgs f;
    f.x = x;
    f.gate = ref(w->gate);
    f.up = ref(w->up);
    f.down = ref(w->down);
    f.s_gate = ref(w->s_gate);
    f.s_up = ref(w->s_up);
    f.s_down = ref(w->s_down);
    f.offsets = off;
    f.perm_rows = perm;
    f.topk_w = topk_w;
    f.meta = at<int32_t>(ws, L.meta);
    f.active = at<int32_t>(ws, L.active);
    f.tiles = at<int2>(ws, L.tiles);
    f.T = c->n_tokens;
    f.d = c->d_model;
    f.E = c->n_expert;
    f.k = c->top_k;
    f.F = c->d_ff;
    f.Fs = c->n_shared ? c->d_ff_shared : 0;
    f.n_shared = c->n_shared;
    f.act = c->act_dtype;
    f.wdt = c->w_dtype;
    f.h = at<void>(ws, L.h);
    f.ldh = ldh_of(c);
    f.slot_out = at<float>(ws, L.slot_out);
    f.shared_out = c->n_shared ? at<float>(ws, L.shared_out) : nullptr;
    f.y = nullptr;
    f.bm = gemm_bm(c);
    f.max_tiles = max_tiles_of(c, f.bm);
    f.shared_done = 0;
    f.grid_has_shared = 0;
    f.dslots = at<DecodeSlot>(ws, L.dslots);
    f.n_dslots = n_dslots_of(c);
    return f;
}

// int8 prefill layers: each product goes to the grouped MFMA GEMM once the
// experts average enough rows for it, else to the GEMVs over the grouped rows
// (they read each weight once per row; the GEMMs widen every weight tile to
// bf16 and pad the tile to 32 rows).  Measured at c2's shape: the down GEMM
// wins from about half a row per expert (32 tokens: 0.32 against 0.37 ms),
// the gate/up GEMM from about 1.5 rows (64 tokens: 0.91 against 0.92 ms; 48
// tokens: 0.80 against 0.75 ms).  The two products may take different kinds
// of kernel: both read and write h and slot_out in the same layout.
bool q8_mfma_gateup(const FfnArgs& f) { return f.wdt == MOE_DT_Q8B32 && 2L * f.T * f.k >= 3L * f.E; }
bool q8_mfma_down(const FfnArgs& f) { return f.wdt == MOE_DT_Q8B32 && 2L * f.T * f.k >= (long)f.E; }

// Experts of the prefill path: MFMA for bf16 weights and for int8 weights with
// enough rows per expert, GEMVs otherwise.
// bf16 experts on the matrix cores: gate/up, then down.
hipError_t run_bf16_experts(const FfnArgs& f, hipStream_t st, const KTime& kg = KTime(),
                            const KTime& kd = KTime()) {
    hipError_t e;
    if ((e = launch_gateup_mfma(f, st, kg)) != hipSuccess) return e;
    return launch_down_mfma(f, st, kd);
}

hipError_t run_expert_kernels(const FfnArgs& f, hipStream_t st) {
    hipError_t e;
    if (f.wdt == MOE_DT_BF16) return run_bf16_experts(f, st);
    e = q8_mfma_gateup(f) ? launch_gateup_mfma_q8(f, st) : launch_gateup_gemv(f, st);
    if (e != hipSuccess) return e;
    return q8_mfma_down(f) ? launch_down_mfma_q8(f, st) : launch_down_slots_gemv(f, st);
}

// The caller's stage events (if any) as per-stage kernel timings.
void stage_timings(const moe_debug* dbg, KTime* kt) {
    for (int s = 0; s < MOE_STAGES; ++s) {
        kt[s] = KTime();
        if (dbg && dbg->stage_events) {
            kt[s].start = static_cast<hipEvent_t>(dbg->stage_events[2 * s]);
            kt[s].stop = static_cast<hipEvent_t>(dbg->stage_events[2 * s + 1]);
        }
    }
}

SelectArgs select_args(const moe_config* c, const float* logits, const float* bias, int32_t* idx,
                       float* w) {
    SelectArgs s;
    s.logits = logits;
    s.bias = bias;
    s.T = c->n_tokens;
    s.E = c->n_expert;
    s.k = c->top_k;
    s.score = c->score;
    s.route_scale = c->route_scale;
    s.topk_idx = idx;
    s.topk_w = w;
    s.generic_only = false;
    return s;
}


// Arguments of a whole-layer call other than its workspace.
int check_layer_args(const moe_config* cfg, const void* x, const moe_weights* w, const float* y,
                     const moe_debug* dbg) {
    int s = validate_config(cfg);
    if (s) return s;
    if ((s = check_weights(cfg, w, true))) return s;
    if (!ptr_ok(x) || !ptr_ok(y)) return MOE_ERR_INVALID;
    if (dbg && (!opt_elt_ok(dbg->logits) || !opt_elt_ok(dbg->topk_idx) || !opt_elt_ok(dbg->topk_w) ||
                !opt_elt_ok(dbg->offsets) || !opt_elt_ok(dbg->perm_rows) || !opt_elt_ok(dbg->inv_perm)))
        return MOE_ERR_INVALID;
    const bool decode = cfg->path == MOE_PATH_DECODE ||
                        (cfg->path == MOE_PATH_AUTO && cfg->n_tokens <= MOE_DECODE_MAX_TOKENS);
    if (decode && cfg->n_tokens > MOE_DECODE_MAX_TOKENS) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int enqueue_layer(const moe_config* cfg, const void* x, const moe_weights* w, float* y, moe_debug* dbg,
                  void* ws, void* stream);

// ---------------------------------------------------------------------------
// The library's own scratch for moe_layer_forward_noalloc: one array per GPU
// (every device that loads this code object holds its own copy, until the
// process ends).  In host code `scratch` only names the symbol; its device
// address is looked up once per device, with that device current, and only
// that address is ever handed to kernels.
// ---------------------------------------------------------------------------
__device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];

// Device address of the current device's scratch array (looked up on the
// first call made on that device).
int static_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return MOE_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return MOE_ERR_DEVICE;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_config* cfg) {
    if (validate_config(cfg) != MOE_OK) return 0;
    return make_layout(cfg).total;
}

const char* moe_status_str(int status) {
    switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_DEVICE: return "device launch failed";
    default: return "unknown status";
    }
}

int moe_route(const moe_config* cfg, const void* x, const float* w_router, const float* bias,
              float* logits, int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
    int s = validate_config(cfg);
    if (s) return s;
    if (!ptr_ok(x) || !ptr_ok(w_router) || !opt_elt_ok(bias) || !opt_elt_ok(logits) || !elt_ok(topk_idx) ||
        !elt_ok(topk_w))
        return MOE_ERR_INVALID;
    if (!logits && (s = check_ws(cfg, ws, ws_bytes))) return s;
    const Layout L = make_layout(cfg);
    float* lg = logits ? logits : at<float>(ws, L.logits);
    hipStream_t st = static_cast<hipStream_t>(stream);
    RouteArgs r{x, w_router, cfg->n_tokens, cfg->d_model, cfg->n_expert, cfg->act_dtype, lg,
                cfg->path == MOE_PATH_PREFILL};
    hipError_t e = launch_router_logits(r, st);
    if (e == hipSuccess) e = launch_topk(select_args(cfg, lg, bias, topk_idx, topk_w), st);
    return device_status(e);
}

int moe_select(const moe_config* cfg, const float* logits, const float* bias, int32_t* topk_idx,
               float* topk_w, void* stream) {
    int s = validate_config(cfg);
    if (s) return s;
    if (!elt_ok(logits) || !opt_elt_ok(bias) || !elt_ok(topk_idx) || !elt_ok(topk_w)) return MOE_ERR_INVALID;
    SelectArgs a = select_args(cfg, logits, bias, topk_idx, topk_w);
    a.generic_only = cfg->path == MOE_PATH_PREFILL;  // lets tests reach the generic kernel at E = 256
    return device_status(launch_topk(a, static_cast<hipStream_t>(stream)));
}

int moe_topk_rows(const float* scores, int32_t rows, int32_t n, int32_t k, int32_t* idx, float* vals,
                  void** events, void* stream) {
    static_assert(MOE_TOPK_ROWS_MAX_N == TOPK_ROWS_MAX_N, "row top-k limit");
    if (rows < 0 || n < 1 || n > MOE_TOPK_ROWS_MAX_N || k < 1 || k > n) return MOE_ERR_INVALID;
    if (rows == 0) return MOE_OK;
    if (!elt_ok(scores) || !elt_ok(idx) || !opt_elt_ok(vals)) return MOE_ERR_INVALID;
    KTime kt;
    if (events) {
        kt.start = static_cast<hipEvent_t>(events[0]);
        kt.stop = static_cast<hipEvent_t>(events[1]);
    }
    TopkRowsArgs a{scores, rows, n, k, idx, vals};
    return device_status(launch_topk_rows(a, static_cast<hipStream_t>(stream), kt));
}

int moe_prefetch_experts(const moe_config* cfg, const moe_weights* w, const int32_t* ids, int32_t n_ids,
                         int32_t which, int32_t rows, int32_t workgroups, void** events, void* stream) {
    int s = validate_config(cfg);
    if (s) return s;
    if (!w || n_ids < 0 || n_ids > MOE_PREFETCH_MAX_IDS || which < 1 || which > 7 || rows < 0 || workgroups < 1 ||
        workgroups > MOE_PREFETCH_MAX_WORKGROUPS)
        return MOE_ERR_INVALID;
    if ((which & 1 && !mat_ok(cfg, w->gate)) || (which & 2 && !mat_ok(cfg, w->up)) ||
        (which & 4 && !mat_ok(cfg, w->down)))
        return MOE_ERR_INVALID;
    if (cfg->w_dtype == MOE_DT_Q8B32 && ((which & 1 && !aligned16(w->gate.scale)) ||
                                         (which & 2 && !aligned16(w->up.scale)) ||
                                         (which & 4 && !aligned16(w->down.scale))))
        return MOE_ERR_INVALID;  // the scales are read with 16-byte loads too
    if (n_ids == 0) return MOE_OK;
    if (!elt_ok(ids)) return MOE_ERR_INVALID;
    // every matrix of an expert holds F * d elements: gate and up F rows of d,
    // down d rows of F
    const int64_t elems = (int64_t)cfg->d_ff * cfg->d_model;
    const int64_t esize = cfg->w_dtype == MOE_DT_F32 ? 4 : cfg->w_dtype == MOE_DT_BF16 ? 2 : 1;
    if (elems * esize > 0x7FFFFFFF) return MOE_ERR_UNSUPPORTED;  // one buffer descriptor per expert matrix
    const bool q8 = cfg->w_dtype == MOE_DT_Q8B32;
    const moe_mat* mats[3] = {&w->gate, &w->up, &w->down};
    PrefetchArgs a{};
    const int order[PF_SEGMENTS][2] = {{0, 0}, {1, 0}, {0, 1}, {1, 1}, {2, 0}, {2, 1}};  // (matrix, scales?)
    for (int g = 0; g < PF_SEGMENTS; ++g) {
        const int m = order[g][0];
        const bool sc = order[g][1] != 0;
        if (!(which >> m & 1) || (sc && !q8)) continue;
        const int64_t n_rows = m == 2 ? cfg->d_model : cfg->d_ff, row_elems = elems / n_rows;
        const int64_t r = rows == 0 || rows > n_rows ? n_rows : rows;  // leading rows read
        a.base[g] = sc ? reinterpret_cast<const uint8_t*>(mats[m]->scale) : static_cast<const uint8_t*>(mats[m]->q);
        a.stride[g] = sc ? elems / 32 * 2 : elems * esize;
        a.bytes[g] = sc ? r * (row_elems / 32) * 2 : r * row_elems * esize;
    }
    a.ids = ids;
    a.n_ids = n_ids;
    a.E = cfg->n_expert;
    KTime kt;
    if (events) {
        kt.start = static_cast<hipEvent_t>(events[0]);
        kt.stop = static_cast<hipEvent_t>(events[1]);
    }
    return device_status(launch_prefetch_experts(a, workgroups, static_cast<hipStream_t>(stream), kt));
}

int moe_permute(const moe_config* cfg, const int32_t* topk_idx, int32_t* offsets, int32_t* perm_rows,
                int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream) {
    int s = validate_config(cfg);
    if (s) return s;
    if (!elt_ok(topk_idx) || !elt_ok(offsets) || !elt_ok(perm_rows) || !elt_ok(inv_perm)) return MOE_ERR_INVALID;
    if ((s = check_ws(cfg, ws, ws_bytes))) return s;
    const Layout L = make_layout(cfg);
    PermArgs p = perm_args(cfg, L, ws, topk_idx, offsets, perm_rows, inv_perm);
    return device_status(launch_permute(p, static_cast<hipStream_t>(stream)));
}

int moe_expert_ffn(const moe_config* cfg, const void* x, const moe_weights* w, const int32_t* offsets,
                   const int32_t* perm_rows, const float* topk_w, float* slot_out, float* shared_out, void* ws,
                   size_t ws_bytes, void* stream) {
    int s = validate_config(cfg);
    if (s) return s;
    if ((s = check_weights(cfg, w, false))) return s;
    if (!ptr_ok(x) || !elt_ok(offsets) || !elt_ok(perm_rows) || !elt_ok(topk_w) || !ptr_ok(slot_out))
        return MOE_ERR_INVALID;
    if (cfg->n_shared && !ptr_ok(shared_out)) return MOE_ERR_INVALID;
    if ((s = check_ws(cfg, ws, ws_bytes))) return s;
    const Layout L = make_layout(cfg);
    hipStream_t st = static_cast<hipStream_t>(stream);
    PermArgs p = perm_args(cfg, L, ws, nullptr, const_cast<int32_t*>(offsets), const_cast<int32_t*>(perm_rows),
                           nullptr);
    hipError_t e = launch_lists_from_offsets(p, st);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
    FfnArgs f = ffn_args(cfg, L, ws, x, w, offsets, perm_rows, topk_w);
    f.slot_out = slot_out;
    f.shared_out = cfg->n_shared ? shared_out : nullptr;
    return device_status(run_expert_kernels(f, st));
}

int moe_combine(const moe_config* cfg, const float* slot_out, const float* shared_out, float* y, void* stream) {
    int s = validate_config(cfg);
    if (s) return s;
    if (!ptr_ok(slot_out) || !opt_ptr_ok(shared_out) || !ptr_ok(y)) return MOE_ERR_INVALID;
    CombineArgs c{slot_out, shared_out, y, cfg->n_tokens, cfg->top_k, cfg->d_model};
    return device_status(launch_combine(c, static_cast<hipStream_t>(stream)));
}

int moe_layer_forward(const moe_config* cfg, const void* x, const moe_weights* w, float* y, moe_debug* dbg,
                      void* ws, size_t ws_bytes, void* stream) {
    int s = check_layer_args(cfg, x, w, y, dbg);
    if (s) return s;
    if ((s = check_ws(cfg, ws, ws_bytes))) return s;
    return enqueue_layer(cfg, x, w, y, dbg, ws, stream);
}

int moe_layer_forward_noalloc(const moe_config* cfg, const void* x, const moe_weights* w, float* y,
                              moe_debug* dbg, void* stream) {
    int s = check_layer_args(cfg, x, w, y, dbg);
    if (s) return s;
    if (make_layout(cfg).total > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    void* scratch_ptr = nullptr;
    if ((s = static_scratch(&scratch_ptr))) return s;
    return enqueue_layer(cfg, x, w, y, dbg, scratch_ptr, stream);
}

}  // extern "C"

namespace {

// The layer's launches over a workspace `ws` already checked to be large enough.
int enqueue_layer(const moe_config* cfg, const void* x, const moe_weights* w, float* y, moe_debug* dbg,
                  void* ws, void* stream) {
    const bool decode = cfg->path == MOE_PATH_DECODE ||
                        (cfg->path == MOE_PATH_AUTO && cfg->n_tokens <= MOE_DECODE_MAX_TOKENS);
    const Layout L = make_layout(cfg);
    hipStream_t st = static_cast<hipStream_t>(stream);

    float* logits = dbg && dbg->logits ? dbg->logits : at<float>(ws, L.logits);
    int32_t* idx = dbg && dbg->topk_idx ? dbg->topk_idx : at<int32_t>(ws, L.topk_idx);
    float* wts = dbg && dbg->topk_w ? dbg->topk_w : at<float>(ws, L.topk_w);
    int32_t* off = dbg && dbg->offsets ? dbg->offsets : at<int32_t>(ws, L.offsets);
    int32_t* perm = dbg && dbg->perm_rows ? dbg->perm_rows : at<int32_t>(ws, L.perm_rows);
    int32_t* inv = dbg && dbg->inv_perm ? dbg->inv_perm : at<int32_t>(ws, L.inv_perm);

    // prefill: the token-grouped GEMV router up to 64 tokens, the tiled one beyond
    RouteArgs r{x, w->w_router, cfg->n_tokens, cfg->d_model, cfg->n_expert, cfg->act_dtype, logits, false};
    KTime kt[MOE_STAGES];
    stage_timings(dbg, kt);
    if (decode) {
        // router | selection + shared gate/up | routed gate/up | down with the combine
        DecodeRouteArgs dr;
        dr.r = r;
        dr.s = select_args(cfg, logits, w->bias, idx, wts);
        dr.p = perm_args(cfg, L, ws, idx, off, perm, inv);
        dr.f = ffn_args(cfg, L, ws, x, w, off, perm, wts);
        dr.f.y = y;
        dr.scores = at<float>(ws, L.scores);
        return device_status(launch_decode(dr, kt, st));
    }
    hipError_t e = launch_router_logits(r, st, kt[0]);
    if (e == hipSuccess) e = launch_topk(select_args(cfg, logits, w->bias, idx, wts), st, kt[1]);
    if (e == hipSuccess) e = launch_permute(perm_args(cfg, L, ws, idx, off, perm, inv), st, kt[2]);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
    FfnArgs f = ffn_args(cfg, L, ws, x, w, off, perm, wts);
    if (f.wdt == MOE_DT_BF16) {
        e = run_bf16_experts(f, st, kt[3], kt[4]);
    } else {
        e = q8_mfma_gateup(f) ? launch_gateup_mfma_q8(f, st, kt[3]) : launch_gateup_gemv(f, st, kt[3]);
        if (e == hipSuccess) e = q8_mfma_down(f) ? launch_down_mfma_q8(f, st, kt[4]) : launch_down_slots_gemv(f, st, kt[4]);
    }
    if (e == hipSuccess) {
        CombineArgs c{f.slot_out, f.shared_out, y, cfg->n_tokens, cfg->top_k, cfg->d_model};
        e = launch_combine(c, st, kt[5]);
    }
    return device_status(e);
}

}  // namespace
