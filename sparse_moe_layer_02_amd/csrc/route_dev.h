// route_dev.h - device building blocks of the router: the score functions
// (fp64, rounded once to fp32), the packed selection key and the one-
// wavefront top-k with renormalised weights.  Shared by the selection kernel
// and the fused decode routing kernel.
//
// Packed key: (orderable fp32 key) << 32 | (0xFFFFFFFF - e), so one unsigned
// maximum picks the larger key and, on equal keys, the lower expert index.
// NaN keys map below every number; -0 is folded onto +0.  k rounds of a
// wave-wide DPP maximum select the experts in rank order; the selected scores
// are summed in fp64 in that order and the weights formed in fp64.
#pragma once
#include "common.h"

#pragma clang fp contract(off)

namespace moe {

__device__ __forceinline__ float router_score(int kind, float logit) {
    const double l = (double)logit;
    if (kind == MOE_SCORE_SIGMOID) return (float)(1.0 / (1.0 + exp(-l)));
    const double sp = l > 0.0 ? l + log1p(exp(-l)) : log1p(exp(l));
    return (float)sqrt(sp);
}

__device__ __forceinline__ uint64_t pack_key(float key, int e) {
    uint32_t u = __float_as_uint(key);
    uint32_t ord;
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) ord = 0u;  // NaN: below -inf
    else {
        if (u == 0x80000000u) u = 0u;  // -0 == +0
        ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    }
    return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

// Selection for one token by one wavefront: lane l holds experts l, l+64, ...
// (KPL of them); writes topk_idx[0..k) and topk_w[0..k).  Returns with the
// selected experts' indices in `my_idx` of lanes 0..k-1.
// FROM_SCORES: `lrow` already holds the fp32 scores instead of the logits.
template <int KPL, int EFIX, bool FROM_SCORES = false>
__device__ __forceinline__ int topk_token(const float* __restrict__ lrow, const float* __restrict__ bias,
                                          int E_rt, int k, int score_kind, float route_scale,
                                          int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
    const int E = EFIX ? EFIX : E_rt;
    const int lane = lane_id();
    uint64_t key[KPL];
    float sc[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        const int e = lane + WAVE * j;
        if (e < E) {
            const float s = FROM_SCORES ? lrow[e] : router_score(score_kind, lrow[e]);
            const float kf = bias ? s + bias[e] : s;
            sc[j] = s;
            key[j] = pack_key(kf, e);
        } else {
            sc[j] = 0.0f;
            key[j] = 0ull;
        }
    }
    int my_idx = 0;
    float my_s = 0.0f;
    double S = 0.0;
    for (int r = 0; r < k; ++r) {
        uint64_t best = key[0];
#pragma unroll
        for (int j = 1; j < KPL; ++j) best = u64_max(best, key[j]);
        best = wave_max_u64(best);
        const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
        const int owner = e % WAVE, slot = e / WAVE;
        float s_owned = 0.0f;
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            if (lane == owner && j == slot) {
                s_owned = sc[j];
                key[j] = 0ull;
            }
        }
        const float s_sel = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(s_owned), owner));
        S += (double)s_sel;
        if (lane == r) {
            my_idx = e;
            my_s = s_sel;
        }
    }
    if (lane < k) {
        idx_out[lane] = my_idx;
        w_out[lane] = S > 0.0 ? (float)(((double)my_s / S) * (double)route_scale) : 0.0f;
    }
    return my_idx;
}

}  // namespace moe
