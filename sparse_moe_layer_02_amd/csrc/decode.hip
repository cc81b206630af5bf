// decode.hip - the decode path (T <= MOE_DECODE_MAX_TOKENS) in four launches,
// with no hand-off between workgroups inside a launch (on this multi-die part
// an agent-scope release fence per workgroup writes back that die's L2 and
// the fences serialise; a kernel boundary publishes results once):
//
//   1. decode_router_kernel: one workgroup per expert computes that expert's
//      router logit and score for every token (fp64, rounded once).
//   2. decode_select_kernel: workgroup 0 runs the top-k of every token (one
//      wavefront each), then one wavefront builds the stable grouping and
//      publishes indices, weights, offsets, permutation and the active-expert
//      list; the other workgroups compute the shared expert's gate/up rows
//      meanwhile (they do not depend on the routing).
//   3. the routed experts' gate/up GEMV over the active list (gemv_ffn.hip).
//   4. decode_down_kernel: a workgroup owns a tile of rows of y; its
//      wavefronts take the expert slots (slot 0 the shared expert, then the
//      active experts in ascending index), stream each slot's down-projection
//      rows once and leave per-slot partial results in LDS, which are then
//      added in slot order - y is written once, deterministically, without
//      atomics and without a separate combine launch.
//
// The pages: the router with a runtime n_expert and a parallel (not
// single-thread) top-k ("256 experts, 512 lines", "The constant that always
// said 256"); decode reads only the selected experts' weights and is bound by
// memory bandwidth (NeutronStar README, MTP paragraph and closing paragraph).
#include "common.h"
#include "gemv_dev.h"
#include "kernels.h"
#include "permute_dev.h"
#include "route_dev.h"

#pragma clang fp contract(off)

namespace moe {

// ---------------------------------------------------------------------------
// 1. router logits + scores, one workgroup per expert
// ---------------------------------------------------------------------------
template <int AF>
__global__ __launch_bounds__(256) void decode_router_kernel(DecodeRouteArgs a) {
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_index();
    const int E = a.r.E, T = a.r.T, d = a.r.d;
    __shared__ double part[4][MOE_DECODE_MAX_TOKENS];
    const int e = blockIdx.x;
    double acc[MOE_DECODE_MAX_TOKENS];
#pragma unroll
    for (int t = 0; t < MOE_DECODE_MAX_TOKENS; ++t) acc[t] = 0.0;
    const float* wrow = a.r.wr + (size_t)e * d;
    for (int c = tid * 4; c < d; c += 1024) {
        const float4 w4 = *reinterpret_cast<const float4*>(wrow + c);
#pragma unroll
        for (int t = 0; t < MOE_DECODE_MAX_TOKENS; ++t) {
            if (t < T) {
                float x0, x1, x2, x3;
                if (AF == MOE_DT_BF16) {
                    const uint2 xv = *reinterpret_cast<const uint2*>(
                        static_cast<const uint16_t*>(a.r.x) + (size_t)t * d + c);
                    x0 = bf16_lo(xv.x); x1 = bf16_hi(xv.x); x2 = bf16_lo(xv.y); x3 = bf16_hi(xv.y);
                } else {
                    const float4 xv = *reinterpret_cast<const float4*>(
                        static_cast<const float*>(a.r.x) + (size_t)t * d + c);
                    x0 = xv.x; x1 = xv.y; x2 = xv.z; x3 = xv.w;
                }
                acc[t] = __fma_rn((double)x0, (double)w4.x, acc[t]);
                acc[t] = __fma_rn((double)x1, (double)w4.y, acc[t]);
                acc[t] = __fma_rn((double)x2, (double)w4.z, acc[t]);
                acc[t] = __fma_rn((double)x3, (double)w4.w, acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < MOE_DECODE_MAX_TOKENS; ++t) {
        if (t < T) {
            const double s = wave_sum_f64(acc[t]);
            if (lane == 0) part[wave][t] = s;
        }
    }
    __syncthreads();
    if (tid < T) {
        const double s = ((part[0][tid] + part[1][tid]) + part[2][tid]) + part[3][tid];
        const float logit = (float)s;
        a.r.logits[(size_t)tid * E + e] = logit;
        a.scores[(size_t)tid * E + e] = router_score(a.s.score, logit);
    }
}

// ---------------------------------------------------------------------------
// 2. selection + grouping (workgroup 0), shared gate/up rows (the others)
// ---------------------------------------------------------------------------
constexpr int DS_THREADS = 1024;
constexpr int DS_WAVES = DS_THREADS / WAVE;  // shared gate/up row pairs per workgroup

// Exclusive prefix sum of arr[0..n) in place by one wavefront (n <= 1024);
// returns the total.  Lane l owns the 16 consecutive entries from 16*l.
__device__ int wave_excl_scan_array(int* arr, int n) {
    const int lane = lane_id();
    int loc[16], s = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int i = lane * 16 + j;
        loc[j] = i < n ? arr[i] : 0;
        s += loc[j];
    }
    int inc = s;
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const int u = __shfl_up(inc, o);
        if (lane >= o) inc += u;
    }
    int run = inc - s;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int i = lane * 16 + j;
        if (i < n) arr[i] = run;
        run += loc[j];
    }
    return __builtin_amdgcn_readlane(inc, WAVE - 1);
}

template <int KPL, int EFIX, int WF, int AF, int MT>
__global__ __launch_bounds__(DS_THREADS) void decode_select_kernel(DecodeRouteArgs a) {
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_index();
    if (blockIdx.x > 0) {
        const int row0 = ((int)blockIdx.x - 1) * DS_WAVES + wave;
        if (row0 < a.f.Fs)
            gateup_wave<WF, AF, 1, MT, MT == 1 ? 4 : 2>(a.f, true, 0, a.f.Fs, a.f.T * a.f.k, a.f.T, row0,
                                                        nullptr);
        return;
    }
    __shared__ int32_t s_idx[MOE_DECODE_MAX_TOKENS * 32];
    __shared__ int cnt[1024];
    const int E = a.r.E, T = a.r.T, k = a.s.k, n = T * k;
    if (wave < T) {
        const int my = topk_token<KPL, EFIX, true>(a.scores + (size_t)wave * E, a.s.bias, E, k, a.s.score,
                                                   a.s.route_scale, a.s.topk_idx + (size_t)wave * k,
                                                   a.s.topk_w + (size_t)wave * k);
        if (lane < k) s_idx[wave * k + lane] = my;
    }
    __syncthreads();
    if (wave != 0) return;
    // one wavefront: counts, active list, offsets, stable scatter
    for (int e = lane; e < E; e += WAVE) cnt[e] = 0;
    for (int f = lane; f < n; f += WAVE) atomicAdd(&cnt[s_idx[f]], 1);
    int na = 0;
    for (int base = 0; base < E; base += WAVE) {
        const int e = base + lane;
        const bool act = e < E && cnt[e] > 0;
        const uint64_t b = __ballot(act);
        if (act) a.p.active[na + __popcll(b & lanemask_lt())] = e;
        na += __popcll(b);
    }
    const int total = wave_excl_scan_array(cnt, E);
    for (int e = lane; e < E; e += WAVE) a.p.offsets[e] = cnt[e];
    if (lane == 0) {
        a.p.offsets[E] = total;
        a.p.meta[0] = na;
        a.p.meta[1] = 0;
        a.p.meta[2] = total;
    }
    PermArgs p = a.p;
    p.topk_idx = s_idx;
    scatter_range(p, 0, n, cnt);
}

// ---------------------------------------------------------------------------
// 4. down projection + combine
// ---------------------------------------------------------------------------
constexpr int DD_THREADS = 512;
constexpr int DD_WAVES = DD_THREADS / WAVE;
constexpr int DD_R = 4;  // rows of y per workgroup
constexpr int DD_MAX_SLOTS = MOE_DECODE_MAX_TOKENS * 32 + 1;

template <int WF, int AF, int MT>
__global__ __launch_bounds__(DD_THREADS) void decode_down_kernel(FfnArgs a) {
    __shared__ float part[DD_MAX_SLOTS][MOE_DECODE_MAX_TOKENS][DD_R];
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_index();
    const int T = a.T, d = a.d, k = a.k;
    const int row0 = blockIdx.x * DD_R;
    const int n_sh = a.n_shared ? 1 : 0;
    const int n_slots = n_sh + a.meta[0];  // slot 0: the shared expert, then the active experts
    for (int q = tid; q < n_slots * MOE_DECODE_MAX_TOKENS * DD_R; q += DD_THREADS) (&part[0][0][0])[q] = 0.0f;
    __syncthreads();
    const int hsz = AF == MOE_DT_BF16 ? 2 : 4;
    for (int s = wave; s < n_slots; s += DD_WAVES) {
        const bool shared = s < n_sh;
        const int e = shared ? 0 : a.active[s - n_sh];
        const int F = shared ? a.Fs : a.F;
        const int r0 = shared ? T * k : a.offsets[e];
        const int m = shared ? T : a.offsets[e + 1] - r0;
        const MatRef& D = shared ? a.s_down : a.down;
        const uint8_t* wq[DD_R];
        const uint16_t* ws[DD_R];
#pragma unroll
        for (int r = 0; r < DD_R; ++r) row_ptrs<WF>(D, e, d, F, min(row0 + r, d - 1), wq[r], ws[r]);
        for (int tg = 0; tg < m; tg += MT) {
            const int nt = min(MT, m - tg);
            const void* hr[MT];
            int tok[MT];
            float wt[MT];
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int ii = min(i, nt - 1);
                hr[i] = static_cast<const uint8_t*>(a.h) + (size_t)(r0 + tg + ii) * a.ldh * hsz;
                tok[i] = tg + ii;
                wt[i] = 1.0f;
                if (!shared) {
                    const int f = a.perm_rows[r0 + tg + ii];
                    const bool ok = f >= 0 && f < T * k;
                    tok[i] = ok ? f / k : -1;
                    wt[i] = ok ? a.topk_w[f] : 0.0f;
                }
            }
            float acc[DD_R][MT];
#pragma unroll
            for (int r = 0; r < DD_R; ++r)
#pragma unroll
                for (int i = 0; i < MT; ++i) acc[r][i] = 0.0f;
            // one chunk of each of the DD_R rows in flight per lane: with four rows
            // per wavefront that already covers the latency (measured faster than two)
            wave_dot<WF, AF, DD_R, MT, 1>(wq, ws, hr, nt, F, acc);
#pragma unroll
            for (int r = 0; r < DD_R; ++r)
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const float v = wave_sum(acc[r][i]);
                    if (lane == r * MT + i && i < nt && tok[i] >= 0) part[s][tok[i]][r] = wt[i] * v;
                }
        }
    }
    __syncthreads();
    for (int q = tid; q < T * DD_R; q += DD_THREADS) {
        const int t = q / DD_R, r = q % DD_R;
        if (row0 + r >= d) continue;
        float acc = 0.0f;
        for (int s = 0; s < n_slots; ++s) acc += part[s][t][r];
        a.y[(size_t)t * d + row0 + r] = acc;
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static int mt_for(int T, int wdt) {
    const int mt = T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8;
    return (wdt == MOE_DT_Q8B32 && mt > 4) ? 4 : mt;
}

template <int WF, int AF>
static void down_launch(const FfnArgs& a, int mt, dim3 grid, hipStream_t st, const KTime& kt) {
    if (mt == 1) launch_kernel(decode_down_kernel<WF, AF, 1>, grid, DD_THREADS, st, kt, a);
    else if (mt == 2) launch_kernel(decode_down_kernel<WF, AF, 2>, grid, DD_THREADS, st, kt, a);
    else if (mt == 4) launch_kernel(decode_down_kernel<WF, AF, 4>, grid, DD_THREADS, st, kt, a);
    else launch_kernel(decode_down_kernel<WF, AF, 8>, grid, DD_THREADS, st, kt, a);
}

template <int KPL, int EFIX, int WF, int AF>
static void select_launch_mt(const DecodeRouteArgs& a, int mt, dim3 grid, hipStream_t st, const KTime& kt) {
    if (mt == 1) launch_kernel(decode_select_kernel<KPL, EFIX, WF, AF, 1>, grid, DS_THREADS, st, kt, a);
    else if (mt == 2) launch_kernel(decode_select_kernel<KPL, EFIX, WF, AF, 2>, grid, DS_THREADS, st, kt, a);
    else if (mt == 4) launch_kernel(decode_select_kernel<KPL, EFIX, WF, AF, 4>, grid, DS_THREADS, st, kt, a);
    else launch_kernel(decode_select_kernel<KPL, EFIX, WF, AF, 8>, grid, DS_THREADS, st, kt, a);
}

template <int KPL, int EFIX>
static void select_launch_fmt(const DecodeRouteArgs& a, int mt, dim3 grid, hipStream_t st, const KTime& kt) {
    if (a.f.wdt == MOE_DT_F32) select_launch_mt<KPL, EFIX, MOE_DT_F32, MOE_DT_F32>(a, mt, grid, st, kt);
    else if (a.f.wdt == MOE_DT_BF16) select_launch_mt<KPL, EFIX, MOE_DT_BF16, MOE_DT_BF16>(a, mt, grid, st, kt);
    else select_launch_mt<KPL, EFIX, MOE_DT_Q8B32, MOE_DT_BF16>(a, mt, grid, st, kt);
}

hipError_t launch_decode(const DecodeRouteArgs& a, const KTime* kt, hipStream_t st) {
    const int T = a.r.T, E = a.r.E;
    const int mt = mt_for(T, a.f.wdt);
    // 1. router
    if (a.r.act == MOE_DT_BF16) launch_kernel(decode_router_kernel<MOE_DT_BF16>, E, 256, st, kt[0], a);
    else launch_kernel(decode_router_kernel<MOE_DT_F32>, E, 256, st, kt[0], a);
    hipError_t e = hipGetLastError();
    // 2. selection + grouping, shared gate/up
    if (e == hipSuccess) {
        dim3 grid(1 + (a.f.n_shared ? (a.f.Fs + DS_WAVES - 1) / DS_WAVES : 0));
        const int kpl = (E + WAVE - 1) / WAVE;
        if (E == 256) select_launch_fmt<4, 256>(a, mt, grid, st, kt[1]);
        else if (kpl <= 1) select_launch_fmt<1, 0>(a, mt, grid, st, kt[1]);
        else if (kpl <= 2) select_launch_fmt<2, 0>(a, mt, grid, st, kt[1]);
        else if (kpl <= 3) select_launch_fmt<3, 0>(a, mt, grid, st, kt[1]);
        else if (kpl <= 4) select_launch_fmt<4, 0>(a, mt, grid, st, kt[1]);
        else if (kpl <= 8) select_launch_fmt<8, 0>(a, mt, grid, st, kt[1]);
        else select_launch_fmt<16, 0>(a, mt, grid, st, kt[1]);
        e = hipGetLastError();
    }
    // 3. routed gate/up
    FfnArgs f = a.f;
    f.shared_done = 1;
    if (e == hipSuccess) e = launch_gateup_gemv(f, st, kt[3]);
    // 4. down + combine
    if (e == hipSuccess) {
        dim3 grid((f.d + DD_R - 1) / DD_R);
        if (f.wdt == MOE_DT_F32) down_launch<MOE_DT_F32, MOE_DT_F32>(f, mt, grid, st, kt[4]);
        else if (f.wdt == MOE_DT_BF16) down_launch<MOE_DT_BF16, MOE_DT_BF16>(f, mt, grid, st, kt[4]);
        else down_launch<MOE_DT_Q8B32, MOE_DT_BF16>(f, mt, grid, st, kt[4]);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace moe
