// route_dev.h - device building blocks of the router: the score functions
// (fp64, rounded once to fp32), the packed selection key and the one-
// wavefront top-k with renormalised weights.  Shared by the selection kernel
// and the fused decode routing kernel.
//
// Packed key: (orderable fp32 key) << 32 | (0xFFFFFFFF - e), so the unsigned
// order is the larger key first and, on equal keys, the lower expert index.
// NaN keys map below every number; -0 is folded onto +0.  k rounds of
// wave-wide DPP maxima select the experts in rank order; the selected scores
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
// (KPL of them); writes topk_idx[0..k) and topk_w[0..k).  Returns the
// expert of rank `lane` in lanes 0..k-1, and its weight in `w_lane`.
// FROM_SCORES: `lrow` already holds the fp32 scores instead of the logits.
//
// Each lane first sorts its KPL packed keys in descending order, so its
// candidate for the next rank is always its first key.  A round then takes
// the wave maximum of the candidates' upper halves (the orderable score; a
// 32-bit DPP maximum) and, only when several lanes hold that score, a second
// maximum of their lower halves (the inverted index: the lowest expert wins).
// The winning lane drops its first key.  Padding keys are 0 and real keys are
// never 0, so k <= E rounds never select padding.
template <int KPL, int EFIX, bool FROM_SCORES = false>
__device__ __forceinline__ int topk_token(const float* __restrict__ lrow, const float* __restrict__ bias,
                                          int E_rt, int k, int score_kind, float route_scale,
                                          int32_t* __restrict__ idx_out, float* __restrict__ w_out,
                                          float* w_lane = nullptr) {
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
    // insertion sort, descending
#pragma unroll
    for (int i = 1; i < KPL; ++i) {
#pragma unroll
        for (int j = i; j > 0; --j) {
            const bool sw = key[j] > key[j - 1];
            const uint64_t ka = key[j - 1], kb = key[j];
            const float sa = sc[j - 1], sb = sc[j];
            key[j - 1] = sw ? kb : ka;
            key[j] = sw ? ka : kb;
            sc[j - 1] = sw ? sb : sa;
            sc[j] = sw ? sa : sb;
        }
    }
    int my_idx = 0;
    float my_s = 0.0f;
    double S = 0.0;
    for (int r = 0; r < k; ++r) {
        const uint32_t hi = (uint32_t)(key[0] >> 32), lo = (uint32_t)key[0];
        const uint32_t M = wave_max_u32(hi);
        const uint64_t cand = __ballot(hi == M);
        int win;
        if (__popcll(cand) == 1) {
            win = __ffsll((unsigned long long)cand) - 1;
        } else {
            const uint32_t L = wave_max_u32(hi == M ? lo : 0u);
            win = __ffsll((unsigned long long)__ballot(hi == M && lo == L)) - 1;
        }
        const int e = (int)(0xFFFFFFFFu - (uint32_t)__builtin_amdgcn_readlane(lo, win));
        const float s_sel = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(sc[0]), win));
        if (lane == win) {
#pragma unroll
            for (int j = 0; j + 1 < KPL; ++j) {
                key[j] = key[j + 1];
                sc[j] = sc[j + 1];
            }
            key[KPL - 1] = 0ull;
            sc[KPL - 1] = 0.0f;
        }
        S += (double)s_sel;
        if (lane == r) {
            my_idx = e;
            my_s = s_sel;
        }
    }
    const float w = S > 0.0 ? (float)(((double)my_s / S) * (double)route_scale) : 0.0f;
    if (lane < k) {
        idx_out[lane] = my_idx;
        w_out[lane] = w;
    }
    if (w_lane) *w_lane = w;
    return my_idx;
}

}  // namespace moe
