// gemv_dev.h - device building blocks of the expert GEMVs: weight-format
// traits, activation chunks, per-chunk dot products (fp32 FMA, bf16 dot2,
// int8 blocks of 32 dequantised in registers) and the wavefront row-dot loop.
#pragma once
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
// int8 blocks: u = q ^ 0x80 = q + 128 lies in [1, 255], so v_cvt_f32_ubyteN
// turns it into an fp32 value whose low 16 bits are zero, i.e. an exact bf16;
// pairs of them go through v_dot2_f32_bf16 against the packed activations
// (about 2.25 VALU instructions per weight instead of sign-extract, convert
// and FMA), and sum(q*x) = sum(u*x) - 128*sum(x), the last term computed
// once per activation chunk (corr) and shared by every row that uses it.
template <> struct Dot<MOE_DT_Q8B32, MOE_DT_BF16> {
    __device__ __forceinline__ static float corr(const XChunk<MOE_DT_BF16, 16>& x) {
        const bf16x2_t one = as_bf16x2(0x3F803F80u);  // (1.0, 1.0)
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(x.v[j]), one, s, false);
        return 128.0f * s;
    }
    // upper halves of two fp32 values -> one bf16 pair (lo in bits 15:0); one v_perm_b32
    __device__ __forceinline__ static uint32_t pack_hi(float lo, float hi) {
        return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
    }
    // sum over the chunk of q * x (before the block scale); c128 = corr(x)
    __device__ __forceinline__ static float run_u(uint4 w, const XChunk<MOE_DT_BF16, 16>& x, float c128) {
        const uint32_t ww[4] = {w.x ^ 0x80808080u, w.y ^ 0x80808080u, w.z ^ 0x80808080u, w.w ^ 0x80808080u};
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float f0 = (float)(ww[j] & 0xFFu), f1 = (float)((ww[j] >> 8) & 0xFFu);
            const float f2 = (float)((ww[j] >> 16) & 0xFFu), f3 = (float)(ww[j] >> 24);
            acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pack_hi(f0, f1)), as_bf16x2(x.v[2 * j]), acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pack_hi(f2, f3)), as_bf16x2(x.v[2 * j + 1]), acc, false);
        }
        return acc - c128;
    }
};

// acc[r][i] += <weight row r, activation row i> over `ncols` columns, partial
// per lane (not yet reduced across the wave).  Every row pointer must address
// a readable row (callers clamp rows past the end onto the last one and drop
// their results), so all loads of a chunk are issued back to back, unguarded.
template <int WF, int AF, int NR, int MT, int UNR = 2>
__device__ __forceinline__ void wave_dot(const uint8_t* const (&wq)[NR], const uint16_t* const (&wsc)[NR],
                                         const void* const (&xr)[MT], int nt, int ncols,
                                         float (&acc)[NR][MT]) {
    constexpr int EPL = WTraits<WF>::EPL, ESZ = WTraits<WF>::ESZ;
    const int lane = lane_id();
#pragma unroll UNR
    for (int c = lane * EPL; c < ncols; c += WAVE * EPL) {
        uint4 w[NR];
        uint16_t sraw[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            w[r] = ld_stream16(wq[r] + (size_t)c * ESZ);
            if constexpr (WF == MOE_DT_Q8B32) sraw[r] = __builtin_nontemporal_load(&wsc[r][c >> 5]);  // read once, as the row
        }
        float sc[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) sc[r] = WF == MOE_DT_Q8B32 ? f16_to_f32(sraw[r]) : 1.0f;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            if (i < nt) {
                XChunk<AF, EPL> xc;
                xc.load(xr[i], c);
                if constexpr (WF == MOE_DT_Q8B32) {
                    const float c128 = Dot<WF, AF>::corr(xc);
#pragma unroll
                    for (int r = 0; r < NR; ++r) acc[r][i] = fmaf(Dot<WF, AF>::run_u(w[r], xc, c128), sc[r], acc[r][i]);
                } else {
#pragma unroll
                    for (int r = 0; r < NR; ++r) acc[r][i] = Dot<WF, AF>::run(w[r], xc, acc[r][i]);
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

__device__ __forceinline__ float silu_mul(float g, float u) { return silu_f32(g) * u; }

template <int AF>
__device__ __forceinline__ void store_h(void* h, size_t idx, float v) {
    if (AF == MOE_DT_BF16) static_cast<uint16_t*>(h)[idx] = f32_to_bf16(v);
    else static_cast<float*>(h)[idx] = v;
}

// Rows [row0, row0+RG) of gate and up for the m tokens of one expert group:
// h rows r0 .. r0+m-1, where row r0+q serves token fr[q] / k (routed rows in
// permutation order), token fr[q] itself when TOKS (a decode slot's token
// list), or token q when fr is null (the shared expert, whose h rows follow
// the routed ones).  h = silu(g) * u, rounded to the activation format.  One
// wavefront; rows past F are computed on the last row and not stored.
template <int WF, int AF, int RG, int MT, int UNR, bool TOKS = false>
__device__ __forceinline__ void gateup_wave(const FfnArgs& a, bool shared, int e, int F, int r0, int m,
                                            int row0, const int32_t* fr) {
    const int lane = lane_id();
    const MatRef& G = shared ? a.s_gate : a.gate;
    const MatRef& U = shared ? a.s_up : a.up;
    const uint8_t* wq[2 * RG];
    const uint16_t* ws[2 * RG];
    bool rv[RG];
#pragma unroll
    for (int r = 0; r < RG; ++r) {
        const int row = min(row0 + r, F - 1);
        row_ptrs<WF>(G, e, F, a.d, row, wq[r], ws[r]);
        row_ptrs<WF>(U, e, F, a.d, row, wq[RG + r], ws[RG + r]);
        rv[r] = row0 + r < F;
    }
    for (int tg = 0; tg < m; tg += MT) {
        const int nt = min(MT, m - tg);
        const void* xr[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int ii = min(i, nt - 1);
            int t = tg + ii;
            if constexpr (TOKS) t = fr[tg + ii];
            else if (fr) {
                const int f = fr[tg + ii];
                t = (f >= 0 && f < a.T * a.k) ? f / a.k : 0;  // a caller's bad row reads token 0
            }
            xr[i] = static_cast<const uint8_t*>(a.x) + (size_t)t * a.d * (AF == MOE_DT_BF16 ? 2 : 4);
        }
        float acc[2 * RG][MT];
#pragma unroll
        for (int r = 0; r < 2 * RG; ++r)
#pragma unroll
            for (int i = 0; i < MT; ++i) acc[r][i] = 0.0f;
        wave_dot<WF, AF, 2 * RG, MT, UNR>(wq, ws, xr, nt, a.d, acc);
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

// Rows [row0, row0+RD) of one expert's down projection for its m tokens
// (h rows r0 .. r0+m-1): routed rows write w_f * value to slot_out[f], the
// shared expert writes its value to shared_out[t].  One wavefront.
template <int WF, int AF, int RD, int MT>
__device__ __forceinline__ void down_rows_wave(const FfnArgs& a, bool shared, int e, int F, int r0, int m,
                                               int row0) {
    const int lane = lane_id();
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
        wave_dot<WF, AF, RD, MT>(wq, ws, hr, nt, F, acc);
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

}  // namespace moe
