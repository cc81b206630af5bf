// route.hip - the router of the MoE layer on gfx950.
//
//   logits[t, e] = sum_i x[t, i] * Wr[e, i]      (stride n_expert, fp64 sum)
//   score        = sigmoid(l) or sqrt(softplus(l)), fp64, rounded to fp32
//   key          = score + bias[e]  (fp32 add; bias optional)
//   top-k        by (key desc, index asc), NaN last
//   weight       = route_scale * s_j / sum_sel s   (fp64, rounded to fp32)
//
// Sources: "256 experts, 512 lines" blog post, "The constant that always said
// 256" (logit stride n_expert, n_expert a runtime value, sqrt(softplus) with
// top-6 and scale 1.5, a parallel top-k instead of a single-thread fallback)
// and "Why GLM-5.2 in an engine built for DeepSeek" (sigmoid, top-8);
// NeutronStar README (main branch), Hy3 paragraph (expert bias).
//
// Every product x*Wr (bf16 or fp32 times fp32) is exact in fp64, so the
// prefill kernel, which adds them in ascending i per output like the
// definition, reproduces the definition's fp32 logits bit for bit.  The decode
// kernel splits the sum across a workgroup (fixed order) for latency; its fp64
// sum rounds to the same fp32 value except in vanishingly rare cases.
#include "common.h"
#include "kernels.h"
#include "route_dev.h"

#pragma clang fp contract(off)

namespace moe {

// ---------------------------------------------------------------------------
// Decode router: one workgroup per expert, T <= MOE_DECODE_MAX_TOKENS.
// Thread j sums columns 4*(j + 256*r) .. +3 in ascending order, then the
// workgroup adds the 256 partials in a fixed tree order.
// ---------------------------------------------------------------------------
template <int AF>
__global__ __launch_bounds__(256) void router_gemv_kernel(const void* __restrict__ x,
                                                          const float* __restrict__ wr, int T, int d,
                                                          int E, float* __restrict__ logits) {
    const int e = blockIdx.x;
    const int tid = threadIdx.x;
    double acc[MOE_DECODE_MAX_TOKENS];
#pragma unroll
    for (int t = 0; t < MOE_DECODE_MAX_TOKENS; ++t) acc[t] = 0.0;
    const float* wrow = wr + (size_t)e * d;
    for (int c = tid * 4; c < d; c += 1024) {
        const float4 w4 = *reinterpret_cast<const float4*>(wrow + c);
#pragma unroll
        for (int t = 0; t < MOE_DECODE_MAX_TOKENS; ++t) {
            if (t < T) {
                float x0, x1, x2, x3;
                if (AF == MOE_DT_BF16) {
                    const uint2 xv = *reinterpret_cast<const uint2*>(
                        static_cast<const uint16_t*>(x) + (size_t)t * d + c);
                    x0 = bf16_lo(xv.x); x1 = bf16_hi(xv.x); x2 = bf16_lo(xv.y); x3 = bf16_hi(xv.y);
                } else {
                    const float4 xv = *reinterpret_cast<const float4*>(
                        static_cast<const float*>(x) + (size_t)t * d + c);
                    x0 = xv.x; x1 = xv.y; x2 = xv.z; x3 = xv.w;
                }
                acc[t] = __fma_rn((double)x0, (double)w4.x, acc[t]);
                acc[t] = __fma_rn((double)x1, (double)w4.y, acc[t]);
                acc[t] = __fma_rn((double)x2, (double)w4.z, acc[t]);
                acc[t] = __fma_rn((double)x3, (double)w4.w, acc[t]);
            }
        }
    }
    __shared__ double part[4][MOE_DECODE_MAX_TOKENS];
    const int wave = tid / WAVE;
#pragma unroll
    for (int t = 0; t < MOE_DECODE_MAX_TOKENS; ++t) {
        if (t < T) {
            double s = wave_sum_f64(acc[t]);
            if (lane_id() == 0) part[wave][t] = s;
        }
    }
    __syncthreads();
    if (tid < T) {
        double s = ((part[0][tid] + part[1][tid]) + part[2][tid]) + part[3][tid];
        logits[(size_t)tid * E + e] = (float)s;
    }
}

// ---------------------------------------------------------------------------
// Prefill router: 64 tokens x 64 experts per workgroup, each thread owns 4x4
// logits and adds x*Wr in ascending i (fp64 FMA; the product is exact so the
// FMA equals multiply-then-add).  K is staged through LDS in chunks of 32.
// ---------------------------------------------------------------------------
constexpr int RG_TM = 64, RG_TE = 64, RG_KC = 32;

template <int AF>
__global__ __launch_bounds__(256) void router_gemm_kernel(const void* __restrict__ x,
                                                          const float* __restrict__ wr, int T, int d,
                                                          int E, float* __restrict__ logits) {
    __shared__ float xs[RG_KC][RG_TM + 1];
    __shared__ float ws[RG_KC][RG_TE + 4];
    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * RG_TM, e0 = blockIdx.y * RG_TE;
    const int tx = tid % 16, ty = tid / 16;
    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;

    for (int k0 = 0; k0 < d; k0 += RG_KC) {
        // x tile: 64 rows x 32 columns; thread loads 8 consecutive columns of one row
        {
            const int r = tid / 4, c = (tid % 4) * 8;
            const int t = t0 + r;
            float v[8];
            if (t < T) {
                if (AF == MOE_DT_BF16) {
                    const uint4 q = *reinterpret_cast<const uint4*>(
                        static_cast<const uint16_t*>(x) + (size_t)t * d + k0 + c);
                    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
                    v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
                } else {
                    const float* p = static_cast<const float*>(x) + (size_t)t * d + k0 + c;
                    const float4 a = *reinterpret_cast<const float4*>(p);
                    const float4 b = *reinterpret_cast<const float4*>(p + 4);
                    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
                    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = 0.0f;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) xs[c + j][r] = v[j];
        }
        // Wr tile: 64 experts x 32 columns; two float4 per thread
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int r = tid / 8 + 32 * p, c = (tid % 8) * 4;
            const int e = e0 + r;
            float4 w4 = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e < E) w4 = *reinterpret_cast<const float4*>(wr + (size_t)e * d + k0 + c);
            ws[c + 0][r] = w4.x;
            ws[c + 1][r] = w4.y;
            ws[c + 2][r] = w4.z;
            ws[c + 3][r] = w4.w;
        }
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < RG_KC; ++kk) {
            double xv[4], wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) xv[i] = (double)xs[kk][ty + 16 * i];
#pragma unroll
            for (int j = 0; j < 4; ++j) wv[j] = (double)ws[kk][tx + 16 * j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __fma_rn(xv[i], wv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + ty + 16 * i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + tx + 16 * j;
            if (e < E) logits[(size_t)t * E + e] = (float)acc[i][j];
        }
    }
}

// ---------------------------------------------------------------------------
// Top-k: one wavefront per token (topk_token in route_dev.h).
// ---------------------------------------------------------------------------
template <int KPL, int EFIX>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                   const float* __restrict__ bias, int T, int E_rt,
                                                   int k, int score_kind, float route_scale,
                                                   int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w) {
    const int E = EFIX ? EFIX : E_rt;
    const int t = blockIdx.x * 4 + threadIdx.x / WAVE;
    if (t >= T) return;
    topk_token<KPL, EFIX>(logits + (size_t)t * E, bias, E, k, score_kind, route_scale,
                          topk_idx + (size_t)t * k, topk_w + (size_t)t * k);
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
hipError_t launch_router_logits(const RouteArgs& a, hipStream_t st, const KTime& kt) {
    if (a.T <= MOE_DECODE_MAX_TOKENS && !a.force_gemm) {
        dim3 grid(a.E);
        if (a.act == MOE_DT_BF16)
            launch_kernel(router_gemv_kernel<MOE_DT_BF16>, grid, 256, st, kt, a.x, a.wr, a.T, a.d, a.E, a.logits);
        else
            launch_kernel(router_gemv_kernel<MOE_DT_F32>, grid, 256, st, kt, a.x, a.wr, a.T, a.d, a.E, a.logits);
    } else {
        dim3 grid((a.T + RG_TM - 1) / RG_TM, (a.E + RG_TE - 1) / RG_TE);
        if (a.act == MOE_DT_BF16)
            launch_kernel(router_gemm_kernel<MOE_DT_BF16>, grid, 256, st, kt, a.x, a.wr, a.T, a.d, a.E, a.logits);
        else
            launch_kernel(router_gemm_kernel<MOE_DT_F32>, grid, 256, st, kt, a.x, a.wr, a.T, a.d, a.E, a.logits);
    }
    return hipGetLastError();
}

template <int KPL, int EFIX>
static void topk_launch(const SelectArgs& a, hipStream_t st, const KTime& kt) {
    dim3 grid((a.T + 3) / 4);
    launch_kernel(topk_kernel<KPL, EFIX>, grid, 256, st, kt, a.logits, a.bias, a.T, a.E, a.k, a.score,
                  a.route_scale, a.topk_idx, a.topk_w);
}

hipError_t launch_topk(const SelectArgs& a, hipStream_t st, const KTime& kt) {
    const int kpl = (a.E + WAVE - 1) / WAVE;
    if (a.E == 256 && !a.generic_only) topk_launch<4, 256>(a, st, kt);  // the common 256-expert router
    else if (kpl <= 1) topk_launch<1, 0>(a, st, kt);
    else if (kpl <= 2) topk_launch<2, 0>(a, st, kt);
    else if (kpl <= 3) topk_launch<3, 0>(a, st, kt);
    else if (kpl <= 4) topk_launch<4, 0>(a, st, kt);
    else if (kpl <= 8) topk_launch<8, 0>(a, st, kt);
    else topk_launch<16, 0>(a, st, kt);
    return hipGetLastError();
}

}  // namespace moe
