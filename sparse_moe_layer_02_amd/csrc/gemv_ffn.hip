// gemv_ffn.hip - expert FFN as bandwidth-bound GEMVs over only the selected
// experts' weights (the decode path), on gfx950.
//
//   h[row, :]  = silu(Wg[e] x_t) * (Wu[e] x_t)        (rounded to the act format)
//   y[t, i]   += w_f * (Wd[e] h_row)[i]   (shared expert: weight 1, added first)
//
// The pages: decode reads only the selected experts (NeutronStar README, MTP
// paragraph: "only the selected experts load, per token"); the bottleneck is
// memory bandwidth, not compute (main branch, closing paragraph); decision
// tensors stay at Q8_0/F32 and experts are gate/up + down projections
// ("The model", "GLM-5.2 CUDA port").
//
// Mapping: a workgroup is 4 wavefronts; each wavefront owns a few weight rows
// and streams them once with 16-byte loads (lane l reads columns
// [l*EPL, l*EPL+EPL) of every 64*EPL-column chunk), applying each row to every
// token routed to that expert (an expert's token group is read from the
// permutation).  int8 blocks of 32 are dequantised in registers: the lane's
// 16 quants lie in one block, so the fp32 dot of quants and activations is
// scaled once by that block's fp16 scale.  Cross-lane sums use the DPP
// butterfly of common.h; every sum has a fixed order, so results are
// deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {

template <int WF> struct WTraits;
template <> struct WTraits<MOE_DT_F32> { static constexpr int EPL = 4, ESZ = 4; };
template <> struct WTraits<MOE_DT_BF16> { static constexpr int EPL = 8, ESZ = 2; };
template <> struct WTraits<MOE_DT_Q8B32> { static constexpr int EPL = 16, ESZ = 1; };

// Activation chunk of EPL values starting at column c of row `p`.
template <int AF, int EPL> struct XChunk;
template <int EPL> struct XChunk<MOE_DT_F32, EPL> {
    float v[EPL];
    __device__ __forceinline__ void load(const void* p, int c) {
        const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p) + c);
#pragma unroll
        for (int j = 0; j < EPL / 4; ++j) {
            const float4 a = q[j];
            v[4 * j] = a.x; v[4 * j + 1] = a.y; v[4 * j + 2] = a.z; v[4 * j + 3] = a.w;
        }
    }
};
template <int EPL> struct XChunk<MOE_DT_BF16, EPL> {
    uint32_t v[EPL / 2];  // packed bf16 pairs
    __device__ __forceinline__ void load(const void* p, int c) {
        const uint16_t* b = static_cast<const uint16_t*>(p) + c;
        if constexpr (EPL >= 8) {
#pragma unroll
            for (int j = 0; j < EPL / 8; ++j) {
                const uint4 a = reinterpret_cast<const uint4*>(b)[j];
                v[4 * j] = a.x; v[4 * j + 1] = a.y; v[4 * j + 2] = a.z; v[4 * j + 3] = a.w;
            }
        } else {
            const uint2 a = *reinterpret_cast<const uint2*>(b);
            v[0] = a.x; v[1] = a.y;
        }
    }
};

// Dot of one 16-byte weight chunk with an activation chunk (before the
// Q8 block scale).
template <int WF, int AF> struct Dot;
template <> struct Dot<MOE_DT_F32, MOE_DT_F32> {
    __device__ __forceinline__ static float run(uint4 w, const XChunk<MOE_DT_F32, 4>& x, float acc) {
        acc = fmaf(__uint_as_float(w.x), x.v[0], acc);
        acc = fmaf(__uint_as_float(w.y), x.v[1], acc);
        acc = fmaf(__uint_as_float(w.z), x.v[2], acc);
        acc = fmaf(__uint_as_float(w.w), x.v[3], acc);
        return acc;
    }
};
template <> struct Dot<MOE_DT_BF16, MOE_DT_BF16> {
    __device__ __forceinline__ static float run(uint4 w, const XChunk<MOE_DT_BF16, 8>& x, float acc) {
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.x), as_bf16x2(x.v[0]), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.y), as_bf16x2(x.v[1]), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.z), as_bf16x2(x.v[2]), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.w), as_bf16x2(x.v[3]), acc, false);
        return acc;
    }
};
template <> struct Dot<MOE_DT_Q8B32, MOE_DT_BF16> {
    __device__ __forceinline__ static float run(uint4 w, const XChunk<MOE_DT_BF16, 16>& x, float acc) {
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int32_t q = (int32_t)ww[j];
            acc = fmaf((float)((q << 24) >> 24), bf16_lo(x.v[2 * j]), acc);
            acc = fmaf((float)((q << 16) >> 24), bf16_hi(x.v[2 * j]), acc);
            acc = fmaf((float)((q << 8) >> 24), bf16_lo(x.v[2 * j + 1]), acc);
            acc = fmaf((float)(q >> 24), bf16_hi(x.v[2 * j + 1]), acc);
        }
        return acc;
    }
};

// acc[r][i] += <weight row r, activation row i> over `ncols` columns, partial
// per lane (not yet reduced across the wave).
template <int WF, int AF, int NR, int MT>
__device__ __forceinline__ void wave_dot(const uint8_t* const (&wq)[NR], const uint16_t* const (&wsc)[NR],
                                         const bool (&rv)[NR], const void* const (&xr)[MT], int nt,
                                         int ncols, float (&acc)[NR][MT]) {
    constexpr int EPL = WTraits<WF>::EPL, ESZ = WTraits<WF>::ESZ;
    const int lane = lane_id();
#pragma unroll 2
    for (int c = lane * EPL; c < ncols; c += WAVE * EPL) {
        uint4 w[NR];
        float sc[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            w[r] = rv[r] ? *reinterpret_cast<const uint4*>(wq[r] + (size_t)c * ESZ) : make_uint4(0, 0, 0, 0);
            if constexpr (WF == MOE_DT_Q8B32) sc[r] = rv[r] ? f16_to_f32(wsc[r][c >> 5]) : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            if (i < nt) {
                XChunk<AF, EPL> xc;
                xc.load(xr[i], c);
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    if constexpr (WF == MOE_DT_Q8B32)
                        acc[r][i] = fmaf(Dot<WF, AF>::run(w[r], xc, 0.0f), sc[r], acc[r][i]);
                    else
                        acc[r][i] = Dot<WF, AF>::run(w[r], xc, acc[r][i]);
                }
            }
        }
    }
}

template <int WF>
__device__ __forceinline__ void row_ptrs(const MatRef& m, int e, int rows, int cols, int row,
                                         const uint8_t*& q, const uint16_t*& s) {
    constexpr int ESZ = WTraits<WF>::ESZ;
    const size_t grow = (size_t)e * rows + row;
    q = static_cast<const uint8_t*>(m.q) + grow * cols * ESZ;
    s = (WF == MOE_DT_Q8B32) ? m.scale + grow * (cols / 32) : nullptr;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

template <int AF>
__device__ __forceinline__ void store_h(void* h, size_t idx, float v) {
    if (AF == MOE_DT_BF16) static_cast<uint16_t*>(h)[idx] = f32_to_bf16(v);
    else static_cast<float*>(h)[idx] = v;
}

// ---------------------------------------------------------------------------
// gate/up: grid (row tiles, slot).  Slot s < n_active is active[s]; the last
// slot (when there is a shared expert) is the shared expert over all tokens.
// ---------------------------------------------------------------------------
template <int WF, int AF, int RG, int MT>
__global__ __launch_bounds__(256) void gateup_gemv_kernel(FfnArgs a) {
    const int slot = blockIdx.y;
    const bool shared = a.n_shared && slot == (int)gridDim.y - 1;
    int e, F, r0, m;
    if (shared) {
        e = 0; F = a.Fs; r0 = a.T * a.k; m = a.T;
    } else {
        if (slot >= a.meta[0]) return;
        e = a.active[slot]; F = a.F; r0 = a.offsets[e]; m = a.offsets[e + 1] - r0;
    }
    const int lane = lane_id();
    const int row0 = (blockIdx.x * 4 + threadIdx.x / WAVE) * RG;
    if (row0 >= F) return;
    const MatRef& G = shared ? a.s_gate : a.gate;
    const MatRef& U = shared ? a.s_up : a.up;
    const uint8_t* wq[2 * RG];
    const uint16_t* ws[2 * RG];
    bool rv[2 * RG];
#pragma unroll
    for (int r = 0; r < RG; ++r) {
        const int row = min(row0 + r, F - 1);
        row_ptrs<WF>(G, e, F, a.d, row, wq[r], ws[r]);
        row_ptrs<WF>(U, e, F, a.d, row, wq[RG + r], ws[RG + r]);
        rv[r] = rv[RG + r] = row0 + r < F;
    }
    for (int tg = 0; tg < m; tg += MT) {
        const int nt = min(MT, m - tg);
        const void* xr[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int ii = min(i, nt - 1);
            int t = tg + ii;
            if (!shared) {
                const int f = a.perm_rows[r0 + tg + ii];
                t = (f >= 0 && f < a.T * a.k) ? f / a.k : 0;  // a caller's bad row reads token 0
            }
            xr[i] = static_cast<const uint8_t*>(a.x) + (size_t)t * a.d * (AF == MOE_DT_BF16 ? 2 : 4);
        }
        float acc[2 * RG][MT];
#pragma unroll
        for (int r = 0; r < 2 * RG; ++r)
#pragma unroll
            for (int i = 0; i < MT; ++i) acc[r][i] = 0.0f;
        wave_dot<WF, AF, 2 * RG, MT>(wq, ws, rv, xr, nt, a.d, acc);
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const float g = wave_sum(acc[r][i]);
                const float u = wave_sum(acc[RG + r][i]);
                if (lane == r * MT + i && i < nt && rv[r])
                    store_h<AF>(a.h, (size_t)(r0 + tg + i) * a.ldh + row0 + r, silu_mul(g, u));
            }
    }
}

// ---------------------------------------------------------------------------
// down + combine (T <= MOE_DECODE_MAX_TOKENS): each wavefront owns RD output
// rows and walks the shared expert, then the active experts in ascending
// order; lane t keeps token t's running sums, so y is written once, without
// atomics.
// ---------------------------------------------------------------------------
template <int WF, int AF, int RD, int MT>
__global__ __launch_bounds__(256) void down_combine_kernel(FfnArgs a) {
    const int lane = lane_id();
    const int row0 = (blockIdx.x * 4 + threadIdx.x / WAVE) * RD;
    if (row0 >= a.d) return;
    const int hsz = AF == MOE_DT_BF16 ? 2 : 4;
    float yacc[RD];
#pragma unroll
    for (int r = 0; r < RD; ++r) yacc[r] = 0.0f;
    bool rv[RD];
#pragma unroll
    for (int r = 0; r < RD; ++r) rv[r] = row0 + r < a.d;

    const int n_act = a.meta[0];
    for (int s = -1; s < n_act; ++s) {
        const bool shared = s < 0;
        if (shared && !a.n_shared) continue;
        const int e = shared ? 0 : a.active[s];
        const int F = shared ? a.Fs : a.F;
        const int r0 = shared ? a.T * a.k : a.offsets[e];
        const int m = shared ? a.T : a.offsets[e + 1] - r0;
        const MatRef& D = shared ? a.s_down : a.down;
        const uint8_t* wq[RD];
        const uint16_t* ws[RD];
#pragma unroll
        for (int r = 0; r < RD; ++r) row_ptrs<WF>(D, e, a.d, F, min(row0 + r, a.d - 1), wq[r], ws[r]);
        for (int tg = 0; tg < m; tg += MT) {
            const int nt = min(MT, m - tg);
            const void* hr[MT];
            int tok[MT];
            float wt[MT];
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int ii = min(i, nt - 1);
                hr[i] = static_cast<const uint8_t*>(a.h) + (size_t)(r0 + tg + ii) * a.ldh * hsz;
                if (shared) {
                    tok[i] = tg + ii;
                    wt[i] = 1.0f;
                } else {
                    const int f = a.perm_rows[r0 + tg + ii];
                    const bool ok = f >= 0 && f < a.T * a.k;
                    tok[i] = ok ? f / a.k : -1;
                    wt[i] = ok ? a.topk_w[f] : 0.0f;
                }
            }
            float acc[RD][MT];
#pragma unroll
            for (int r = 0; r < RD; ++r)
#pragma unroll
                for (int i = 0; i < MT; ++i) acc[r][i] = 0.0f;
            wave_dot<WF, AF, RD, MT>(wq, ws, rv, hr, nt, F, acc);
#pragma unroll
            for (int r = 0; r < RD; ++r)
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const float v = wave_sum(acc[r][i]);
                    if (i < nt && lane == tok[i]) yacc[r] = shared ? v : fmaf(wt[i], v, yacc[r]);
                }
        }
    }
    if (lane < a.T) {
#pragma unroll
        for (int r = 0; r < RD; ++r)
            if (rv[r]) a.y[(size_t)lane * a.d + row0 + r] = yacc[r];
    }
}

// ---------------------------------------------------------------------------
// down into slots: grid (row tiles, slot); writes slot_out[f] = w_f * down
// rows and shared_out[t] (weight 1).
// ---------------------------------------------------------------------------
template <int WF, int AF, int RD, int MT>
__global__ __launch_bounds__(256) void down_slots_kernel(FfnArgs a) {
    const int slot = blockIdx.y;
    const bool shared = a.n_shared && slot == (int)gridDim.y - 1;
    int e, F, r0, m;
    if (shared) {
        e = 0; F = a.Fs; r0 = a.T * a.k; m = a.T;
    } else {
        if (slot >= a.meta[0]) return;
        e = a.active[slot]; F = a.F; r0 = a.offsets[e]; m = a.offsets[e + 1] - r0;
    }
    const int lane = lane_id();
    const int row0 = (blockIdx.x * 4 + threadIdx.x / WAVE) * RD;
    if (row0 >= a.d) return;
    const int hsz = AF == MOE_DT_BF16 ? 2 : 4;
    const MatRef& D = shared ? a.s_down : a.down;
    const uint8_t* wq[RD];
    const uint16_t* ws[RD];
    bool rv[RD];
#pragma unroll
    for (int r = 0; r < RD; ++r) {
        row_ptrs<WF>(D, e, a.d, F, min(row0 + r, a.d - 1), wq[r], ws[r]);
        rv[r] = row0 + r < a.d;
    }
    for (int tg = 0; tg < m; tg += MT) {
        const int nt = min(MT, m - tg);
        const void* hr[MT];
        size_t dst[MT];
        float wt[MT];
        bool ok[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int ii = min(i, nt - 1);
            hr[i] = static_cast<const uint8_t*>(a.h) + (size_t)(r0 + tg + ii) * a.ldh * hsz;
            ok[i] = true;
            if (shared) {
                dst[i] = (size_t)(tg + ii) * a.d;
                wt[i] = 1.0f;
            } else {
                const int f = a.perm_rows[r0 + tg + ii];
                ok[i] = f >= 0 && f < a.T * a.k;
                dst[i] = ok[i] ? (size_t)f * a.d : 0;
                wt[i] = ok[i] ? a.topk_w[f] : 0.0f;
            }
        }
        float acc[RD][MT];
#pragma unroll
        for (int r = 0; r < RD; ++r)
#pragma unroll
            for (int i = 0; i < MT; ++i) acc[r][i] = 0.0f;
        wave_dot<WF, AF, RD, MT>(wq, ws, rv, hr, nt, F, acc);
        float* out = shared ? a.shared_out : a.slot_out;
#pragma unroll
        for (int r = 0; r < RD; ++r)
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const float v = wave_sum(acc[r][i]);
                if (lane == r * MT + i && i < nt && rv[r] && ok[i]) out[dst[i] + row0 + r] = shared ? v : wt[i] * v;
            }
    }
}

// ---------------------------------------------------------------------------
// combine: y[t] = shared_out[t] + sum_j slot_out[t*k + j], four columns per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
    const size_t n4 = (size_t)a.T * a.d / 4;
    for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < n4; q += (size_t)gridDim.x * blockDim.x) {
        const size_t t = q * 4 / a.d, c = q * 4 % a.d;
        float4 acc = a.shared_out ? *reinterpret_cast<const float4*>(a.shared_out + t * a.d + c)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j = 0; j < a.k; ++j) {
            const float4 s = *reinterpret_cast<const float4*>(a.slot_out + (t * a.k + j) * a.d + c);
            acc.x += s.x; acc.y += s.y; acc.z += s.z; acc.w += s.w;
        }
        *reinterpret_cast<float4*>(a.y + t * a.d + c) = acc;
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
constexpr int RG_ROWS = 4;  // gate (and up) rows per wavefront
constexpr int RD_ROWS = 4;  // down rows per wavefront

static int pick_mt(int max_rows) { return max_rows <= 1 ? 1 : max_rows <= 2 ? 2 : max_rows <= 4 ? 4 : 8; }

#define MOE_DISPATCH_MT(KERNEL, WF, AF, R, MTV, GRID, ARGS, ST)                                    \
    do {                                                                                           \
        if ((MTV) == 1) KERNEL<WF, AF, R, 1><<<GRID, 256, 0, ST>>>(ARGS);                          \
        else if ((MTV) == 2) KERNEL<WF, AF, R, 2><<<GRID, 256, 0, ST>>>(ARGS);                     \
        else if ((MTV) == 4 || (WF) == MOE_DT_Q8B32) KERNEL<WF, AF, R, 4><<<GRID, 256, 0, ST>>>(ARGS); \
        else KERNEL<WF, AF, R, 8><<<GRID, 256, 0, ST>>>(ARGS);                                     \
    } while (0)

#define MOE_DISPATCH_FMT(KERNEL, R, MTV, GRID, ARGS, ST)                                   \
    do {                                                                                   \
        if ((ARGS).wdt == MOE_DT_F32)                                                      \
            MOE_DISPATCH_MT(KERNEL, MOE_DT_F32, MOE_DT_F32, R, MTV, GRID, ARGS, ST);       \
        else if ((ARGS).wdt == MOE_DT_BF16)                                                \
            MOE_DISPATCH_MT(KERNEL, MOE_DT_BF16, MOE_DT_BF16, R, MTV, GRID, ARGS, ST);     \
        else                                                                               \
            MOE_DISPATCH_MT(KERNEL, MOE_DT_Q8B32, MOE_DT_BF16, R, MTV, GRID, ARGS, ST);    \
    } while (0)

hipError_t launch_gateup_gemv(const FfnArgs& a, hipStream_t st) {
    const int fmax = a.n_shared && a.Fs > a.F ? a.Fs : a.F;
    const int slots = (a.E < a.T * a.k ? a.E : a.T * a.k) + (a.n_shared ? 1 : 0);
    dim3 grid((fmax + 4 * RG_ROWS - 1) / (4 * RG_ROWS), slots);
    const int mt = pick_mt(a.T);
    MOE_DISPATCH_FMT(gateup_gemv_kernel, RG_ROWS, mt, grid, a, st);
    return hipGetLastError();
}

hipError_t launch_down_combine_gemv(const FfnArgs& a, hipStream_t st) {
    dim3 grid((a.d + 4 * RD_ROWS - 1) / (4 * RD_ROWS));
    const int mt = pick_mt(a.T);
    MOE_DISPATCH_FMT(down_combine_kernel, RD_ROWS, mt, grid, a, st);
    return hipGetLastError();
}

hipError_t launch_down_slots_gemv(const FfnArgs& a, hipStream_t st) {
    const int slots = (a.E < a.T * a.k ? a.E : a.T * a.k) + (a.n_shared ? 1 : 0);
    dim3 grid((a.d + 4 * RD_ROWS - 1) / (4 * RD_ROWS), slots);
    const int mt = pick_mt(a.T);
    MOE_DISPATCH_FMT(down_slots_kernel, RD_ROWS, mt, grid, a, st);
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
    const size_t n4 = (size_t)a.T * a.d / 4;
    const size_t want = (n4 + 255) / 256;
    const int blocks = (int)(want < 4096 ? want : 4096);
    combine_kernel<<<blocks, 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace moe
