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
// Router for few tokens: workgroup (e, g) computes expert e's logits for the
// tokens 8g .. 8g+7.  Thread j sums columns 4*(j + 256*r) .. +3 in ascending
// order, then the workgroup adds the 256 partials in a fixed tree order.
// ---------------------------------------------------------------------------
constexpr int ROUTER_GEMV_MAX_T = 64;  // more tokens: the tiled kernel below

template <int AF>
__global__ __launch_bounds__(256) void router_gemv_kernel(const void* __restrict__ x,
                                                          const float* __restrict__ wr, int T, int d,
                                                          int E, float* __restrict__ logits) {
    const int e = blockIdx.x;
    const int tid = threadIdx.x;
    const int t0 = blockIdx.y * MOE_DECODE_MAX_TOKENS;
    T = min(T - t0, MOE_DECODE_MAX_TOKENS);
    x = static_cast<const uint8_t*>(x) + (size_t)t0 * d * (AF == MOE_DT_BF16 ? 2 : 4);
    logits += (size_t)t0 * E;
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
// Prefill router: a workgroup computes a TM-token x TE-expert tile of logits;
// each of its 256 threads owns RT tokens x RE experts and adds x*Wr in
// ascending i with fp64 FMA (the product is exact, so the FMA equals
// multiply-then-add, and the sum follows the definition's order).  K is staged
// through LDS in chunks of KC columns, widened to fp64 once at staging; the
// next chunk's global loads are issued before the current chunk is consumed,
// so their latency overlaps the arithmetic.  The inner loop reads two columns
// per 16-byte LDS read; the row pitch of KC + 2 doubles staggers consecutive
// rows by 4 dwords across the LDS banks.
// ---------------------------------------------------------------------------
template <int AF, int TM, int TE, int RT, int RE, int KC>
__global__ __launch_bounds__(256) void router_gemm_kernel(const void* __restrict__ x,
                                                          const float* __restrict__ wr, int T, int d,
                                                          int E, float* __restrict__ logits) {
    constexpr int NTX = TE / RE, NTY = TM / RT, PITCH = KC + 2;
    constexpr int NXQ = TM * KC / 8, NWQ = TE * KC / 4;  // staging items: 8 x values, 4 Wr values
    constexpr int NXI = (NXQ + 255) / 256, NWI = (NWQ + 255) / 256;  // items per thread
    static_assert(NTX * NTY == 256, "256 threads per tile");
    __shared__ __attribute__((aligned(16))) double xs[TM * PITCH];
    __shared__ __attribute__((aligned(16))) double ws[TE * PITCH];
    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * TM, e0 = blockIdx.y * TE;
    const int tx = tid % NTX, ty = tid / NTX;

    uint4 rx[NXI];  // 8 bf16 (or the first 4 of 8 fp32: rx2 holds the rest)
    uint4 rx2[NXI];
    float4 rw[NWI];
    auto gload = [&](int k0) {
#pragma unroll
        for (int it = 0; it < NXI; ++it) {
            const int q = tid + 256 * it, r = q / (KC / 8), c = (q % (KC / 8)) * 8;
            const int t = t0 + r;
            rx[it] = make_uint4(0, 0, 0, 0);
            rx2[it] = make_uint4(0, 0, 0, 0);
            if (q < NXQ && t < T) {
                if (AF == MOE_DT_BF16) {
                    rx[it] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + (size_t)t * d + k0 + c);
                } else {
                    const float* p = static_cast<const float*>(x) + (size_t)t * d + k0 + c;
                    rx[it] = *reinterpret_cast<const uint4*>(p);
                    rx2[it] = *reinterpret_cast<const uint4*>(p + 4);
                }
            }
        }
#pragma unroll
        for (int it = 0; it < NWI; ++it) {
            const int q = tid + 256 * it, r = q / (KC / 4), c = (q % (KC / 4)) * 4;
            const int e = e0 + r;
            rw[it] = (q < NWQ && e < E) ? *reinterpret_cast<const float4*>(wr + (size_t)e * d + k0 + c)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int it = 0; it < NXI; ++it) {
            const int q = tid + 256 * it, r = q / (KC / 8), c = (q % (KC / 8)) * 8;
            if (q >= NXQ) break;
            double* dst = &xs[r * PITCH + c];
            if (AF == MOE_DT_BF16) {
                const uint4 u = rx[it];
                dst[0] = bf16_lo(u.x); dst[1] = bf16_hi(u.x); dst[2] = bf16_lo(u.y); dst[3] = bf16_hi(u.y);
                dst[4] = bf16_lo(u.z); dst[5] = bf16_hi(u.z); dst[6] = bf16_lo(u.w); dst[7] = bf16_hi(u.w);
            } else {
                const uint4 a = rx[it], b = rx2[it];
                dst[0] = __uint_as_float(a.x); dst[1] = __uint_as_float(a.y);
                dst[2] = __uint_as_float(a.z); dst[3] = __uint_as_float(a.w);
                dst[4] = __uint_as_float(b.x); dst[5] = __uint_as_float(b.y);
                dst[6] = __uint_as_float(b.z); dst[7] = __uint_as_float(b.w);
            }
        }
#pragma unroll
        for (int it = 0; it < NWI; ++it) {
            const int q = tid + 256 * it, r = q / (KC / 4), c = (q % (KC / 4)) * 4;
            if (q >= NWQ) break;
            double* dst = &ws[r * PITCH + c];
            dst[0] = rw[it].x;
            dst[1] = rw[it].y;
            dst[2] = rw[it].z;
            dst[3] = rw[it].w;
        }
    };

    double acc[RT][RE];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < RE; ++j) acc[i][j] = 0.0;

    gload(0);
    for (int k0 = 0; k0 < d; k0 += KC) {
        lstore();
        __syncthreads();
        if (k0 + KC < d) gload(k0 + KC);
#pragma unroll 4
        for (int kk = 0; kk < KC; kk += 2) {
            double2 xv[RT], wv[RE];
#pragma unroll
            for (int i = 0; i < RT; ++i)
                xv[i] = *reinterpret_cast<const double2*>(&xs[(ty + NTY * i) * PITCH + kk]);
#pragma unroll
            for (int j = 0; j < RE; ++j)
                wv[j] = *reinterpret_cast<const double2*>(&ws[(tx + NTX * j) * PITCH + kk]);
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int j = 0; j < RE; ++j) {
                    acc[i][j] = __fma_rn(xv[i].x, wv[j].x, acc[i][j]);
                    acc[i][j] = __fma_rn(xv[i].y, wv[j].y, acc[i][j]);
                }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int t = t0 + ty + NTY * i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < RE; ++j) {
            const int e = e0 + tx + NTX * j;
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
template <int AF, int TM, int TE, int RT, int RE, int KC>
static void router_gemm_tile(const RouteArgs& a, hipStream_t st, const KTime& kt) {
    dim3 grid((a.T + TM - 1) / TM, (a.E + TE - 1) / TE);
    launch_kernel(router_gemm_kernel<AF, TM, TE, RT, RE, KC>, grid, 256, st, kt, a.x, a.wr, a.T, a.d, a.E,
                  a.logits);
}

// The largest tile that still gives every compute unit two workgroups; the
// smallest when none does (few tokens).
template <int AF>
static void router_gemm_launch(const RouteArgs& a, hipStream_t st, const KTime& kt) {
    auto blocks = [&](int tm, int te) { return (long)((a.T + tm - 1) / tm) * ((a.E + te - 1) / te); };
    if (a.d % 64 == 0 && blocks(64, 64) >= 512) router_gemm_tile<AF, 64, 64, 4, 4, 32>(a, st, kt);
    else if (a.d % 64 == 0 && blocks(32, 64) >= 512) router_gemm_tile<AF, 32, 64, 2, 4, 64>(a, st, kt);
    else if (a.d % 128 == 0) router_gemm_tile<AF, 16, 32, 1, 2, 128>(a, st, kt);
    else router_gemm_tile<AF, 16, 32, 1, 2, 64>(a, st, kt);
}

hipError_t launch_router_logits(const RouteArgs& a, hipStream_t st, const KTime& kt) {
    if (a.T <= ROUTER_GEMV_MAX_T && !a.force_gemm) {
        dim3 grid(a.E, (a.T + MOE_DECODE_MAX_TOKENS - 1) / MOE_DECODE_MAX_TOKENS);
        if (a.act == MOE_DT_BF16)
            launch_kernel(router_gemv_kernel<MOE_DT_BF16>, grid, 256, st, kt, a.x, a.wr, a.T, a.d, a.E, a.logits);
        else
            launch_kernel(router_gemv_kernel<MOE_DT_F32>, grid, 256, st, kt, a.x, a.wr, a.T, a.d, a.E, a.logits);
    } else if (a.act == MOE_DT_BF16) {
        router_gemm_launch<MOE_DT_BF16>(a, st, kt);
    } else {
        router_gemm_launch<MOE_DT_F32>(a, st, kt);
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
