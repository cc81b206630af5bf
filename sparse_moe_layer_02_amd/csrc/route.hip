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
#include "dma_dev.h"
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
// Prefill router on the fp64 matrix cores, for many tokens: a workgroup of eight
// wavefronts computes a 64-token x 64-expert tile of logits, each wavefront a
// 16 x 32 piece as 1 x 2 blocks of v_mfma_f64_16x16x4_f64 (A = x rows, B =
// Wr rows, widened to fp64 as they are read from LDS; every product is exact
// in fp64 and the unit accumulates in fp64, so only the order of the fp64
// additions differs from the definition's, far below the fp32 rounding of the
// result).  K is staged raw through three LDS stages of 64 columns, copied
// straight from global memory into LDS (1 KB per copy instruction: whole
// 128- or 256-byte rows), chunk c + 2 issued into the stage of chunk c - 1
// behind one barrier per chunk.  Inside a chunk the K order is free (the
// products are exact), so each 16-column group is split so that the lane
// with K slot lk takes columns 4 lk .. 4 lk + 3 of the group over four
// instructions: one 8-byte (x, bf16) and two 16-byte (Wr) LDS reads feed
// eight MFMAs.  The 16-byte chunks of a staged row are XOR-swizzled so the
// sixteen rows a read serves hit distinct banks.
//
// Operand layout of the 16x16x4 f64 instruction (checked on the device): lane l
// supplies A[l % 16][l / 16] and B[l / 16][l % 16]; its four results are
// D[l / 16 + 4 j][l % 16], j = 0..3.
// ---------------------------------------------------------------------------
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <int AF>
__global__ __launch_bounds__(512) void router_mfma_kernel(const void* __restrict__ x,
                                                          const float* __restrict__ wr, int T, int d,
                                                          int E, float* __restrict__ logits) {
    constexpr int TM = 64, TE = 64, KC = 64, NW = 8;
    constexpr int XRB = KC * (AF == MOE_DT_BF16 ? 2 : 4);  // bytes of one staged x row (128 or 256)
    constexpr int XS = TM * XRB, WS = TE * KC * 4;          // bytes of a stage's x and Wr rows
    constexpr int XCP = XS / 1024, NCP = (XS + WS) / 1024;  // 1 KB copies per stage (x, all)
    constexpr int NQ = NCP / NW, XQ = XCP / NW;             // per wavefront (all, x)
    static_assert(NQ * NW == NCP && XQ * NW == XCP, "copy geometry");
    constexpr int XCH = XRB / 16;                           // 16-byte chunks per x row
    // three stages of raw x and raw Wr rows (separate objects: reading one
    // stage does not wait for the copies into the others)
    __shared__ __attribute__((aligned(1024))) uint8_t xs0[XS];
    __shared__ __attribute__((aligned(1024))) uint8_t xs1[XS];
    __shared__ __attribute__((aligned(1024))) uint8_t xs2[XS];
    __shared__ __attribute__((aligned(1024))) uint8_t ws0[WS];
    __shared__ __attribute__((aligned(1024))) uint8_t ws1[WS];
    __shared__ __attribute__((aligned(1024))) uint8_t ws2[WS];
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
    const int t0 = blockIdx.x * TM, e0 = blockIdx.y * TE;
    // chunk c of row r sits at slot c ^ sw(r): x rows of 128 bytes sw = (r >> 1) & 7,
    // rows of 256 bytes sw = r & 15 (the sixteen rows one read serves hit distinct banks)
    auto xswz = [](int r) { return XCH == 8 ? (r >> 1) & 7 : r & 15; };
    // copy q of this wavefront: 1 KB = 1024 / row bytes rows, lane l at slot l % chunks
    // (rows past T or E read the last row; their results are never stored)
    const uint8_t* src[NQ];
    int dst[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int id = q * NW + wave;
        if (q < XQ) {
            const int r = id * (1024 / XRB) + lane / XCH, slot = lane % XCH;
            const int row = min(t0 + r, T - 1);
            src[q] = static_cast<const uint8_t*>(x) + (size_t)row * d * (XRB / KC) + 16 * (slot ^ xswz(r));
            dst[q] = id * 1024;
        } else {
            const int id2 = id - XCP;
            const int r = id2 * 4 + lane / 16, slot = lane % 16;
            const int row = min(e0 + r, E - 1);
            src[q] = reinterpret_cast<const uint8_t*>(wr + (size_t)row * d) + 16 * (slot ^ (r & 15));
            dst[q] = id2 * 1024;
        }
    }
    const int nch = d / KC;
    auto issue = [&](auto sc, int ch) {
        constexpr int S = decltype(sc)::value;
        uint8_t* X = S == 0 ? xs0 : S == 1 ? xs1 : xs2;
        uint8_t* W = S == 0 ? ws0 : S == 1 ? ws1 : ws2;
        const int c = ch < nch ? ch : nch - 1;  // chunks past the end re-read the last (unused)
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if (q < XQ) copy16(src[q] + (size_t)c * XRB, X + dst[q]);
            else copy16(src[q] + (size_t)c * 256, W + dst[q]);
        }
    };

    // wavefront w: tokens (w / 2) * 16 .. +15, experts (w % 2) * 32 .. +31 of the tile
    const int wm = (wave / 2) * 16, wn = (wave % 2) * 32;
    const int lr = lane % 16, lk = lane / 16;
    f64x4 acc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[j] = f64x4{0.0, 0.0, 0.0, 0.0};
    const int xm = wm + lr;
    // chunk ch in stage S: wait for it (chunk ch + 1 may still be in flight),
    // barrier (every wavefront has also finished the stage of chunk ch - 1),
    // issue chunk ch + 2 into that stage, then the products
    auto chunk = [&](auto sc, int ch) {
        constexpr int S = decltype(sc)::value;
        const uint8_t* X = S == 0 ? xs0 : S == 1 ? xs1 : xs2;
        const uint8_t* W = S == 0 ? ws0 : S == 1 ? ws1 : ws2;
        wait_vm<NQ>();
        barrier_nofence();
        issue(ic<(S + 2) % 3>(), ch + 2);
#pragma unroll
        for (int kg = 0; kg < KC; kg += 16) {  // K slot lk of instruction s: column kg + 4 lk + s
            double av[4];
            if constexpr (AF == MOE_DT_BF16) {
                const int c = kg / 8 + lk / 2;
                const uint2 p = *reinterpret_cast<const uint2*>(X + xm * XRB + 16 * (c ^ xswz(xm)) + 8 * (lk & 1));
                av[0] = (double)bf16_lo(p.x);
                av[1] = (double)bf16_hi(p.x);
                av[2] = (double)bf16_lo(p.y);
                av[3] = (double)bf16_hi(p.y);
            } else {
                const int c = kg / 4 + lk;
                const float4 p = *reinterpret_cast<const float4*>(X + xm * XRB + 16 * (c ^ xswz(xm)));
                av[0] = (double)p.x;
                av[1] = (double)p.y;
                av[2] = (double)p.z;
                av[3] = (double)p.w;
            }
            float4 wv[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int n = wn + 16 * j + lr;
                wv[j] = *reinterpret_cast<const float4*>(W + n * 256 + 16 * ((kg / 4 + lk) ^ (n & 15)));
            }
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float bw = s4 == 0 ? wv[j].x : s4 == 1 ? wv[j].y : s4 == 2 ? wv[j].z : wv[j].w;
                    acc[j] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[s4], (double)bw, acc[j], 0, 0, 0);
                }
            }
        }
        wait_lgkm0();  // this stage's reads done before the next barrier releases its refill
    };
    issue(ic<0>(), 0);
    issue(ic<1>(), 1);
    int ch = 0;
    for (; ch + 3 <= nch; ch += 3) {
        chunk(ic<0>(), ch);
        chunk(ic<1>(), ch + 1);
        chunk(ic<2>(), ch + 2);
    }
    if (ch < nch) chunk(ic<0>(), ch);
    if (ch + 1 < nch) chunk(ic<1>(), ch + 1);
    wait_vm<0>();  // no copy may still be writing LDS when the workgroup ends
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = e0 + wn + 16 * j + lr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + wm + lk + 4 * r;
            if (t < T && e < E) logits[(size_t)t * E + e] = (float)acc[j][r];
        }
    }
}

// ---------------------------------------------------------------------------
// The same on a 16-token x 32-expert tile, for token counts whose 64 x 64 tiles
// cannot fill the chip (c4: 32 of them): the eight wavefronts form four K
// groups of two, group g taking the 64-column chunks g, g + 4, ...; each
// wavefront owns one 16 x 16 block and alternates two accumulators, and the
// groups' partial sums are added in a fixed order at the end (deterministic;
// only the order of fp64 additions differs from the definition's).
// ---------------------------------------------------------------------------
template <int AF>
__global__ __launch_bounds__(512) void router_mfma_split_kernel(const void* __restrict__ x,
                                                                const float* __restrict__ wr, int T, int d,
                                                                int E, float* __restrict__ logits) {
    constexpr int TM = 16, TE = 32, KC = 64, KG = 4, GT = 128;  // GT threads per K group
    constexpr int XW = AF == MOE_DT_BF16 ? KC / 2 : KC;
    constexpr int XP = XW + 1, WP = KC + 1;
    constexpr int XQ = TM * XW / 4, WQ = TE * KC / 4;  // 16-byte staging items per chunk
    constexpr int XI = (XQ + GT - 1) / GT, WI = WQ / GT;
    static_assert(WQ % GT == 0 && XQ % GT == 0, "staging shape");
    __shared__ uint32_t xs[KG][2][TM * XP];
    __shared__ float ws[KG][2][TE * WP];
    __shared__ f64x4 red[KG - 1][2][WAVE];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / WAVE;
    const int kg = wave / 2, blk = wave % 2, gtid = tid % GT;
    const int t0 = blockIdx.x * TM, e0 = blockIdx.y * TE;
    uint4 rx[XI];
    float4 rw[WI];
    auto gload = [&](int k0) {
#pragma unroll
        for (int it = 0; it < XI; ++it) {
            const int q = gtid + GT * it, r = q / (XW / 4), c = (q % (XW / 4)) * 4;
            rx[it] = make_uint4(0, 0, 0, 0);
            if (t0 + r < T) {
                const uint32_t* row = AF == MOE_DT_BF16
                    ? reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(x) + (size_t)(t0 + r) * d + k0)
                    : reinterpret_cast<const uint32_t*>(static_cast<const float*>(x) + (size_t)(t0 + r) * d + k0);
                rx[it] = *reinterpret_cast<const uint4*>(row + c);
            }
        }
#pragma unroll
        for (int it = 0; it < WI; ++it) {
            const int q = gtid + GT * it, r = q / (KC / 4), c = (q % (KC / 4)) * 4;
            rw[it] = e0 + r < E ? *reinterpret_cast<const float4*>(wr + (size_t)(e0 + r) * d + k0 + c)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto lstore = [&](int stg) {
#pragma unroll
        for (int it = 0; it < XI; ++it) {
            const int q = gtid + GT * it, r = q / (XW / 4), c = (q % (XW / 4)) * 4;
            uint32_t* dst = &xs[kg][stg][r * XP + c];
            dst[0] = rx[it].x; dst[1] = rx[it].y; dst[2] = rx[it].z; dst[3] = rx[it].w;
        }
#pragma unroll
        for (int it = 0; it < WI; ++it) {
            const int q = gtid + GT * it, r = q / (KC / 4), c = (q % (KC / 4)) * 4;
            float* dst = &ws[kg][stg][r * WP + c];
            dst[0] = rw[it].x; dst[1] = rw[it].y; dst[2] = rw[it].z; dst[3] = rw[it].w;
        }
    };
    const int lr = lane % 16, lk = lane / 16;
    auto xval = [&](int stg, int kk) -> double {
        if (AF == MOE_DT_BF16) {
            const uint32_t pair = xs[kg][stg][lr * XP + (kk >> 1)];
            return (double)((kk & 1) ? bf16_hi(pair) : bf16_lo(pair));
        }
        return (double)__uint_as_float(xs[kg][stg][lr * XP + kk]);
    };

    f64x4 acc0 = f64x4{0.0, 0.0, 0.0, 0.0}, acc1 = acc0;
    const int nch = d / KC, rounds = (nch + KG - 1) / KG;
    if (kg < nch) {
        gload(kg * KC);
        lstore(0);
    }
    __syncthreads();
    for (int rd = 0; rd < rounds; ++rd) {
        const int ch = rd * KG + kg, stg = rd & 1;
        const bool have = ch < nch, have_next = ch + KG < nch;
        if (have_next) gload((ch + KG) * KC);
        if (have) {
#pragma unroll
            for (int ks = 0; ks < KC; ks += 8) {
                const double a0 = xval(stg, ks + lk), a1 = xval(stg, ks + 4 + lk);
                const double b0 = (double)ws[kg][stg][(16 * blk + lr) * WP + ks + lk];
                const double b1 = (double)ws[kg][stg][(16 * blk + lr) * WP + ks + 4 + lk];
                acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc1, 0, 0, 0);
            }
        }
        if (have_next) lstore(stg ^ 1);
        __syncthreads();
    }
    f64x4 acc = acc0 + acc1;
    if (kg > 0) red[kg - 1][blk][lane] = acc;
    __syncthreads();
    if (kg == 0) {
#pragma unroll
        for (int g = 0; g < KG - 1; ++g) acc += red[g][blk][lane];
        const int e = e0 + 16 * blk + lr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + lk + 4 * r;
            if (t < T && e < E) logits[(size_t)t * E + e] = (float)acc[r];
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

// The matrix-core kernels from 128 tiles on: 64 x 64 tiles with the whole K
// per workgroup, else 16 x 32 tiles with K split over four groups of
// wavefronts; below that the largest VALU tile that still gives every compute
// unit two workgroups, the smallest when none does.
constexpr long ROUTER_MFMA_MIN_TILES = 128;
template <int AF>
static void router_gemm_launch(const RouteArgs& a, hipStream_t st, const KTime& kt) {
    auto blocks = [&](int tm, int te) { return (long)((a.T + tm - 1) / tm) * ((a.E + te - 1) / te); };
    if (a.d % 64 == 0 && blocks(64, 64) >= ROUTER_MFMA_MIN_TILES) {
        dim3 grid((a.T + 63) / 64, (a.E + 63) / 64);
        launch_kernel(router_mfma_kernel<AF>, grid, 512, st, kt, a.x, a.wr, a.T, a.d, a.E, a.logits);
    } else if (a.d % 64 == 0 && blocks(16, 32) >= ROUTER_MFMA_MIN_TILES) {
        dim3 grid((a.T + 15) / 16, (a.E + 31) / 32);
        launch_kernel(router_mfma_split_kernel<AF>, grid, 512, st, kt, a.x, a.wr, a.T, a.d, a.E, a.logits);
    } else if (a.d % 64 == 0 && blocks(64, 64) >= 512) router_gemm_tile<AF, 64, 64, 4, 4, 32>(a, st, kt);
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
