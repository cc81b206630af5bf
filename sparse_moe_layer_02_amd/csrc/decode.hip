// decode.hip - the decode path (T <= MOE_DECODE_MAX_TOKENS) in four launches,
// with no hand-off between workgroups inside a launch (on this multi-die part
// an agent-scope release fence per workgroup writes back that die's L2 and
// the fences serialise; a kernel boundary publishes results once):
//
//   1. decode_router_kernel: one workgroup per expert computes that expert's
//      router logit and score for every token (fp64, rounded once); the
//      workgroups after the first E compute the shared expert's gate/up rows.
//   2. decode_select_kernel: workgroup 0 runs the top-k of every token (one
//      wavefront each), then one wavefront builds the stable grouping and
//      publishes indices, weights, offsets, permutation, the active-expert
//      list and the decode slot table; the other workgroups compute the
//      shared expert's down projection into shared_out.
//   3. the routed experts' gate/up GEMV over the slot table (gemv_ffn.hip).
//   4. decode_down_rows_kernel: a wavefront owns one row of y, starts from
//      shared_out and adds every routed slot's weighted down-projection row
//      in slot order - y is written once, deterministically, without atomics
//      and without a separate combine launch (decode_down_kernel, with
//      per-slot partials in LDS, covers the shapes outside its limits).
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
// 1. router logits + scores, one workgroup per expert; the workgroups after
//    the first E compute the shared expert's gate/up rows (one row pair per
//    wavefront), which do not depend on the routing
// ---------------------------------------------------------------------------
template <int WF, int AF, int MT>
__global__ __launch_bounds__(256) void decode_router_kernel(DecodeRouteArgs a) {
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_index();
    const int E = a.r.E, T = a.r.T, d = a.r.d;
    if ((int)blockIdx.x >= E) {
        const int row0 = ((int)blockIdx.x - E) * 4 + wave;
        if (row0 < a.f.Fs)
            gateup_wave<WF, AF, 1, MT, MT == 1 ? 4 : 2>(a.f, true, 0, a.f.Fs, a.f.T * a.f.k, a.f.T, row0,
                                                        nullptr);
        return;
    }
    __shared__ double part[4][MOE_DECODE_MAX_TOKENS];
    const int e = blockIdx.x;
    double acc[MOE_DECODE_MAX_TOKENS];
#pragma unroll
    for (int t = 0; t < MOE_DECODE_MAX_TOKENS; ++t) acc[t] = 0.0;
    const float* wrow = a.r.wr + (size_t)e * d;
    // Thread tid adds columns tid*4 .. tid*4+3 of every 1024-column stripe, in
    // ascending order; the W_r loads of four stripes are issued before the
    // first product (one memory round trip for d <= 4096).
    for (int c0 = tid * 4; c0 < d; c0 += 4 * 1024) {
        float4 w4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = c0 + j * 1024;
            w4[j] = c < d ? *reinterpret_cast<const float4*>(wrow + c) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = c0 + j * 1024;
            if (c >= d) break;
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
                    acc[t] = __fma_rn((double)x0, (double)w4[j].x, acc[t]);
                    acc[t] = __fma_rn((double)x1, (double)w4[j].y, acc[t]);
                    acc[t] = __fma_rn((double)x2, (double)w4[j].z, acc[t]);
                    acc[t] = __fma_rn((double)x3, (double)w4[j].w, acc[t]);
                }
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
// 2. selection + grouping (workgroup 0), shared expert's down projection
//    into shared_out (the others)
// ---------------------------------------------------------------------------
constexpr int DS_THREADS = 512;  // enough wavefronts for the top-k of MOE_DECODE_MAX_TOKENS tokens
constexpr int DS_WAVES = DS_THREADS / WAVE;
constexpr int DS_ROWS = 2;  // shared down rows per wavefront
constexpr int DS_MAX_N = MOE_DECODE_MAX_TOKENS * 32;  // assignments T*k at most

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

// Grouping of n = T*k <= 64 assignments by one wavefront, in registers: lane
// f holds assignment f = t*k + j (expert s_idx[f], weight s_w[f]).  Its row
// in the stable order by (expert, token) is the number of assignments that
// precede it, found by comparing against every other lane's key (n
// v_readlane steps); the same pass counts the earlier assignments of its own
// expert (its place in the expert's group) and the group size.  A group's
// first assignment writes the slot header; slot numbers count the distinct
// experts below.  Writes perm_rows, inv_perm, offsets, the active list, meta
// and the decode slot table.
__device__ void group_in_registers(const DecodeRouteArgs& a, const int32_t* s_idx, const float* s_w) {
    const int lane = lane_id();
    const int E = a.r.E, T = a.r.T, k = a.s.k, n = T * k;
    const bool v = lane < n;
    const int ef = v ? s_idx[lane] : 0x7FFFFFFF;
    const float wf = v ? s_w[lane] : 0.0f;
    const int tf = v ? lane / k : 0;
    const int keyf = v ? ef * MOE_DECODE_MAX_TOKENS + tf : 0x7FFFFFFF;
    int rank = 0, before = 0, same = 0;
    for (int g = 0; g < n; ++g) {
        const int kg = __builtin_amdgcn_readlane(keyf, g);
        const int eg = __builtin_amdgcn_readlane(ef, g);
        rank += kg < keyf;
        before += (eg == ef) & (kg < keyf);
        same += eg == ef;
    }
    const bool first = v && before == 0;
    const uint64_t fb = __ballot(first);
    const int na = __popcll(fb);
    int slot = 0;  // distinct experts below ef
    for (int g = 0; g < n; ++g) {
        const int eg = __builtin_amdgcn_readlane(ef, g);
        slot += (int)((fb >> g) & 1) & (eg < ef);
    }
    const int n_sh = a.f.n_shared ? 1 : 0;
    DecodeSlot* ds = a.f.dslots;
    if (v) {
        a.p.perm_rows[rank] = lane;
        a.p.inv_perm[lane] = rank;
        DecodeSlot* D = ds + n_sh + slot;
        D->tok[before] = tf;
        D->w[before] = wf;
        if (first) {
            a.p.active[slot] = ef;
            *reinterpret_cast<int4*>(D) = make_int4(ef, rank, same, 0);
        }
    }
    for (int e = lane; e <= E; e += WAVE) {
        int off = 0;
        for (int g = 0; g < n; ++g) off += __builtin_amdgcn_readlane(ef, g) < e;
        a.p.offsets[e] = off;
    }
    for (int j = n_sh + na + lane; j < a.f.n_dslots; j += WAVE)
        *reinterpret_cast<int4*>(ds + j) = make_int4(-1, 0, 0, 0);
    if (n_sh) {
        if (lane == 0) *reinterpret_cast<int4*>(ds) = make_int4(0, n, T, 1);
        if (lane < T) {
            ds[0].tok[lane] = lane;
            ds[0].w[lane] = 1.0f;
        }
    }
    if (lane == 0) {
        a.p.meta[0] = na;
        a.p.meta[1] = 0;
        a.p.meta[2] = n;
    }
}

template <int KPL, int EFIX, int WF, int AF, int MT>
__global__ __launch_bounds__(DS_THREADS) void decode_select_kernel(DecodeRouteArgs a) {
    const int lane = lane_id(), wave = wave_index();
    if (blockIdx.x > 0) {
        const int row0 = (((int)blockIdx.x - 1) * DS_WAVES + wave) * DS_ROWS;
        if (row0 < a.f.d) down_rows_wave<WF, AF, DS_ROWS, MT>(a.f, true, 0, a.f.Fs, a.f.T * a.f.k, a.f.T, row0);
        return;
    }
    __shared__ int32_t s_idx[DS_MAX_N];   // expert of assignment f = t*k + j
    __shared__ float s_w[DS_MAX_N];       // its routing weight
    __shared__ int32_t s_perm[DS_MAX_N];  // assignment of h row r
    __shared__ int32_t s_act[DS_MAX_N];   // active experts, ascending
    __shared__ int cnt[1024];             // counts, then scatter cursors (end offsets)
    __shared__ int s_off[1024];           // first h row of each expert
    __shared__ int s_slot[1024];          // routed slot of each active expert
    const int E = a.r.E, T = a.r.T, k = a.s.k, n = T * k;
    if (wave < T) {
        float wl;
        const int my = topk_token<KPL, EFIX, true>(a.scores + (size_t)wave * E, a.s.bias, E, k, a.s.score,
                                                   a.s.route_scale, a.s.topk_idx + (size_t)wave * k,
                                                   a.s.topk_w + (size_t)wave * k, &wl);
        if (lane < k) {
            s_idx[wave * k + lane] = my;
            s_w[wave * k + lane] = wl;
        }
    }
    __syncthreads();
    if (wave != 0) return;
    if (n <= WAVE) {
        group_in_registers(a, s_idx, s_w);
        return;
    }
    // one wavefront: counts, active list, offsets, stable scatter, slot table
    for (int e = lane; e < E; e += WAVE) cnt[e] = 0;
    for (int f = lane; f < n; f += WAVE) atomicAdd(&cnt[s_idx[f]], 1);
    int na = 0;
    for (int base = 0; base < E; base += WAVE) {
        const int e = base + lane;
        const bool act = e < E && cnt[e] > 0;
        const uint64_t b = __ballot(act);
        if (act) {
            const int pos = na + __popcll(b & lanemask_lt());
            a.p.active[pos] = e;
            s_act[pos] = e;
            s_slot[e] = pos;
        }
        na += __popcll(b);
    }
    const int total = wave_excl_scan_array(cnt, E);
    for (int e = lane; e < E; e += WAVE) {
        a.p.offsets[e] = cnt[e];
        s_off[e] = cnt[e];
    }
    if (lane == 0) {
        a.p.offsets[E] = total;
        a.p.meta[0] = na;
        a.p.meta[1] = 0;
        a.p.meta[2] = total;
    }
    PermArgs p = a.p;
    p.topk_idx = s_idx;
    p.perm_rows = s_perm;
    scatter_range(p, 0, n, cnt);
    const int n_sh = a.f.n_shared ? 1 : 0;
    DecodeSlot* ds = a.f.dslots;
    for (int r = lane; r < n; r += WAVE) {
        const int f = s_perm[r];
        const int e = s_idx[f];
        DecodeSlot* D = ds + n_sh + s_slot[e];
        const int i = r - s_off[e];
        a.p.perm_rows[r] = f;
        D->tok[i] = f / k;
        D->w[i] = s_w[f];
    }
    for (int j = lane; j < a.f.n_dslots; j += WAVE) {
        int4 hd = make_int4(-1, 0, 0, 0);
        if (j < n_sh) hd = make_int4(0, n, T, 1);
        else if (j - n_sh < na) {
            const int e = s_act[j - n_sh];
            hd = make_int4(e, s_off[e], cnt[e] - s_off[e], 0);
        }
        *reinterpret_cast<int4*>(ds + j) = hd;
    }
    if (n_sh && lane < T) {
        ds[0].tok[lane] = lane;
        ds[0].w[lane] = 1.0f;
    }
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
        if (shared) {  // computed by the selection launch
            for (int q = lane; q < T * DD_R; q += WAVE)
                if (row0 + q % DD_R < d) part[0][q / DD_R][q % DD_R] = a.shared_out[(size_t)(q / DD_R) * d + row0 + q % DD_R];
            continue;
        }
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
// 4'. down projection + combine, one row of y per wavefront
//
// A wavefront owns one row of y and walks every slot of the decode slot table
// in order (slot 0 the shared expert, then the active experts ascending),
// adding weight * (W_down[e] row) . h into the lane of each token; y is
// written once, in the same slot order as decode_down_kernel, so the two
// give the same bits.
//
// Latency: the slot headers come in with one lane-parallel load (lane s holds
// slot s) and are broadcast with v_readlane; the h rows of all slots are
// staged into LDS (four 16-byte loads per thread, all in flight together,
// then stored after the headers are read); then the weight row pieces of a
// whole batch of slots are loaded at once, unconditionally (slots past the
// last valid one repeat it), so the compiler's wait counts are exact and
// each slot is reduced as soon as its own pieces have landed.
// Used when F = F_s is 1-4 chunks of 64 lanes x 16 bytes, the table has at
// most 64 slots and h fits the staging buffer; decode_down_kernel otherwise.
// ---------------------------------------------------------------------------
constexpr int DR_WAVES = 16;  // rows of y per workgroup
constexpr int DR_THREADS = DR_WAVES * WAVE;
constexpr int DR_H_BYTES = 64 * 1024;  // LDS staging buffer for h

// Slot headers held across the wavefront: lane s has slot s.
struct SlotLanes {
    int e, r0, m, shared, tok0, tok1;
    float w0, w1;
    __device__ __forceinline__ int get(int v, int s) const { return __builtin_amdgcn_readlane(v, s); }
};

template <int WF, int NC>
struct DownBatch {
    static constexpr int NS = (WF == MOE_DT_Q8B32 ? 14 : 24) / NC;  // slots per batch
    uint4 w[NS][NC];
    uint16_t sc[NS][NC];
    static constexpr int LOADS = NS * NC * (WF == MOE_DT_Q8B32 ? 2 : 1);  // vector-memory ops per batch
};

template <int WF, int NC>
__device__ __forceinline__ void down_load_batch(DownBatch<WF, NC>& B, const FfnArgs& a, const SlotLanes& H,
                                                int s0, int n_valid, int row) {
    constexpr int EPL = WTraits<WF>::EPL, ESZ = WTraits<WF>::ESZ, NS = DownBatch<WF, NC>::NS;
    const int lane = lane_id();
#pragma unroll
    for (int g = 0; g < NS; ++g) {
        const int s = min(s0 + g, n_valid - 1);
        const int e = H.get(H.e, s);
        const bool sh = H.get(H.shared, s) != 0;
        const uint8_t* q;
        const uint16_t* sp;
        row_ptrs<WF>(sh ? a.s_down : a.down, e, a.d, sh ? a.Fs : a.F, row, q, sp);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int col = (c * WAVE + lane) * EPL;
            B.w[g][c] = ld_stream16(q + (size_t)col * ESZ);
            if constexpr (WF == MOE_DT_Q8B32) B.sc[g][c] = __builtin_nontemporal_load(&sp[col >> 5]);  // read once, as the row
        }
        __builtin_amdgcn_sched_barrier(0);  // issue order = slot order (reductions wait in that order)
    }
}

template <int WF, int AF, int NC>
__device__ __forceinline__ void down_reduce_batch(const DownBatch<WF, NC>& B, const FfnArgs& a,
                                                  const SlotLanes& H, int s0, int n_valid, const uint8_t* hs,
                                                  float& my) {
    constexpr int EPL = WTraits<WF>::EPL, NS = DownBatch<WF, NC>::NS;
    const int lane = lane_id();
    const size_t hrow_bytes = (size_t)a.ldh * (AF == MOE_DT_BF16 ? 2 : 4);
#pragma unroll
    for (int g = 0; g < NS; ++g) {
        const int s = s0 + g;
        if (s >= n_valid) break;
        float sc[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) sc[c] = WF == MOE_DT_Q8B32 ? f16_to_f32(B.sc[g][c]) : 1.0f;
        const int m = H.get(H.m, s), r0 = H.get(H.r0, s);
        for (int i = 0; i < m; ++i) {
            const uint8_t* hrow = hs + (size_t)(r0 + i) * hrow_bytes;
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                XChunk<AF, EPL> xc;
                xc.load(hrow, (c * WAVE + lane) * EPL);
                if constexpr (WF == MOE_DT_Q8B32)
                    acc = fmaf(Dot<WF, AF>::run_u(B.w[g][c], xc, Dot<WF, AF>::corr(xc)), sc[c], acc);
                else acc = Dot<WF, AF>::run(B.w[g][c], xc, acc);
            }
            const float v = wave_sum(acc);
            const int t = i == 0 ? H.get(H.tok0, s) : i == 1 ? H.get(H.tok1, s) : a.dslots[s].tok[i];
            const float w = i == 0   ? __int_as_float(H.get(__float_as_int(H.w0), s))
                            : i == 1 ? __int_as_float(H.get(__float_as_int(H.w1), s))
                                     : a.dslots[s].w[i];
            if (lane == t) my += w * v;
        }
    }
}

template <int WF, int AF, int NC>
__global__ __launch_bounds__(DR_THREADS) void decode_down_rows_kernel(FfnArgs a) {
    using Batch = DownBatch<WF, NC>;
    __shared__ uint4 s_h[DR_H_BYTES / 16];
    const int lane = lane_id(), wave = wave_index();
    const int row = blockIdx.x * DR_WAVES + wave;  // the grid covers d exactly
    // h rows [0, T*k + T) -> LDS, 1 KB per wavefront copy, together with the
    // slot headers; the workgroup barrier comes before any weight load:
    // the CU accepts only so many outstanding loads, so a barrier behind the
    // weight batch would release only once most weights had arrived, and the
    // reductions would then run after the stream instead of beside it
    const int hsz = AF == MOE_DT_BF16 ? 2 : 4;
    const int n16 = (int)((size_t)(a.T * a.k + (a.n_shared ? a.T : 0)) * a.ldh * hsz / 16);
    const uint4* hsrc = static_cast<const uint4*>(a.h);
    static_assert(DR_H_BYTES == 4 * 16 * DR_THREADS, "four staged pieces per thread");
    const int tq = threadIdx.x;
    const uint4 h0 = hsrc[min(tq, n16 - 1)], h1 = hsrc[min(tq + DR_THREADS, n16 - 1)];
    const uint4 h2 = hsrc[min(tq + 2 * DR_THREADS, n16 - 1)], h3 = hsrc[min(tq + 3 * DR_THREADS, n16 - 1)];
    __builtin_amdgcn_sched_barrier(0);  // all staging loads in flight together
    SlotLanes H{-1, 0, 0, 0, 0, 0, 0.0f, 0.0f};
    if (lane < a.n_dslots) {
        const DecodeSlot* D = a.dslots + lane;
        const int4 hd = *reinterpret_cast<const int4*>(D);
        const int2 tk = *reinterpret_cast<const int2*>(D->tok);
        const float2 wv = *reinterpret_cast<const float2*>(D->w);
        H.e = hd.x; H.r0 = hd.y; H.m = hd.z; H.shared = hd.w;
        H.tok0 = tk.x; H.tok1 = tk.y;
        H.w0 = wv.x; H.w1 = wv.y;
    }
    // valid slots form a prefix of the table (slot 0 is always valid); the
    // shared expert's slot 0 comes from shared_out (selection launch)
    const int n_valid = __popcll(__ballot(lane < a.n_dslots && H.e >= 0));
    const int first = a.n_shared ? 1 : 0;
    float my = (first && lane < a.T) ? a.shared_out[(size_t)lane * a.d + row] : 0.0f;  // lane t: y[t, row]
    s_h[tq] = h0;  // (entries past n16 hold unread copies)
    s_h[tq + DR_THREADS] = h1;
    s_h[tq + 2 * DR_THREADS] = h2;
    s_h[tq + 3 * DR_THREADS] = h3;
    __syncthreads();
    uint8_t* hdst = reinterpret_cast<uint8_t*>(s_h);
    Batch B;
    down_load_batch(B, a, H, first, n_valid, row);  // (k >= 1: there is a routed slot)
    down_reduce_batch<WF, AF, NC>(B, a, H, first, n_valid, hdst, my);
    for (int s0 = first + Batch::NS; s0 < n_valid; s0 += Batch::NS) {
        down_load_batch(B, a, H, s0, n_valid, row);
        down_reduce_batch<WF, AF, NC>(B, a, H, s0, n_valid, hdst, my);
    }
    if (lane < a.T) a.y[(size_t)lane * a.d + row] = my;
}

// Chunks of 64 lanes x 16 bytes in a down row when decode_down_rows_kernel
// applies, else 0.
static int down_rows_nc(const FfnArgs& f) {
    const int epl = f.wdt == MOE_DT_Q8B32 ? 16 : f.wdt == MOE_DT_BF16 ? 8 : 4;
    if (f.F % (WAVE * epl) || (f.n_shared && f.Fs != f.F) || f.d % DR_WAVES || f.n_dslots > WAVE) return 0;
    const int nc = f.F / (WAVE * epl);
    if (nc < 1 || nc > (f.wdt == MOE_DT_Q8B32 ? 2 : f.wdt == MOE_DT_F32 ? 3 : 4)) return 0;  // (more would spill)
    const size_t hb = (size_t)(f.T * f.k + (f.n_shared ? f.T : 0)) * f.ldh * (f.act == MOE_DT_BF16 ? 2 : 4);
    return hb <= (size_t)DR_H_BYTES ? nc : 0;
}

template <int WF, int AF>
static void down_rows_launch(const FfnArgs& a, int nc, hipStream_t st, const KTime& kt) {
    const dim3 grid(a.d / DR_WAVES);
    if (nc == 1) launch_kernel(decode_down_rows_kernel<WF, AF, 1>, grid, DR_THREADS, st, kt, a);
    else if (nc == 2) launch_kernel(decode_down_rows_kernel<WF, AF, 2>, grid, DR_THREADS, st, kt, a);
    else if (nc == 3) launch_kernel(decode_down_rows_kernel<WF, AF, 3>, grid, DR_THREADS, st, kt, a);
    else launch_kernel(decode_down_rows_kernel<WF, AF, 4>, grid, DR_THREADS, st, kt, a);
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

template <int WF, int AF>
static void router_launch_mt(const DecodeRouteArgs& a, int mt, dim3 grid, hipStream_t st, const KTime& kt) {
    if (mt == 1) launch_kernel(decode_router_kernel<WF, AF, 1>, grid, 256, st, kt, a);
    else if (mt == 2) launch_kernel(decode_router_kernel<WF, AF, 2>, grid, 256, st, kt, a);
    else if (mt == 4) launch_kernel(decode_router_kernel<WF, AF, 4>, grid, 256, st, kt, a);
    else launch_kernel(decode_router_kernel<WF, AF, 8>, grid, 256, st, kt, a);
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
    // 1. router, shared gate/up
    const dim3 rgrid(E + (a.f.n_shared ? (a.f.Fs + 3) / 4 : 0));
    if (a.f.wdt == MOE_DT_F32) router_launch_mt<MOE_DT_F32, MOE_DT_F32>(a, mt, rgrid, st, kt[0]);
    else if (a.f.wdt == MOE_DT_BF16) router_launch_mt<MOE_DT_BF16, MOE_DT_BF16>(a, mt, rgrid, st, kt[0]);
    else router_launch_mt<MOE_DT_Q8B32, MOE_DT_BF16>(a, mt, rgrid, st, kt[0]);
    hipError_t e = hipGetLastError();
    // 2. selection + grouping, shared down
    if (e == hipSuccess) {
        dim3 grid(1 + (a.f.n_shared ? (a.f.d + DS_WAVES * DS_ROWS - 1) / (DS_WAVES * DS_ROWS) : 0));
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
    if (e == hipSuccess) e = launch_gateup_gemv_decode(f, st, kt[3]);
    // 4. down + combine
    const int nc = down_rows_nc(f);
    if (e == hipSuccess && nc) {
        if (f.wdt == MOE_DT_F32) down_rows_launch<MOE_DT_F32, MOE_DT_F32>(f, nc, st, kt[4]);
        else if (f.wdt == MOE_DT_BF16) down_rows_launch<MOE_DT_BF16, MOE_DT_BF16>(f, nc, st, kt[4]);
        else down_rows_launch<MOE_DT_Q8B32, MOE_DT_BF16>(f, nc, st, kt[4]);
        e = hipGetLastError();
    } else if (e == hipSuccess) {
        dim3 grid((f.d + DD_R - 1) / DD_R);
        if (f.wdt == MOE_DT_F32) down_launch<MOE_DT_F32, MOE_DT_F32>(f, mt, grid, st, kt[4]);
        else if (f.wdt == MOE_DT_BF16) down_launch<MOE_DT_BF16, MOE_DT_BF16>(f, mt, grid, st, kt[4]);
        else down_launch<MOE_DT_Q8B32, MOE_DT_BF16>(f, mt, grid, st, kt[4]);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace moe
