// common.h - device helpers shared by the gfx950 kernels of the MoE layer:
// storage-format conversions, wavefront (64-lane) reductions built from DPP
// and LDS-crossbar swizzles, and the workspace layout the host code hands to
// the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int WAVE = 64;

// ---------------------------------------------------------------------------
// Formats
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// silu(g) = g / (1 + e^-g) in fp32 with the hardware exponential and
// reciprocal (a few ulp of fp32, far below the bf16 rounding of h).  Large
// negative g gives e^-g = inf, a reciprocal of 0 and silu = -0, as the
// division would.
__device__ __forceinline__ float silu_f32(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// IEEE binary16 bits -> fp32 (hardware conversion; subnormals preserved).
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }

// 16 bytes read or written once per launch (weights streamed by the GEMVs,
// slot rows on their way to the combine): non-temporal accesses, which pass
// the caches without displacing the data other accesses reuse.
typedef uint32_t stream_u4 __attribute__((ext_vector_type(4)));
typedef float stream_f4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
    const stream_u4 v = __builtin_nontemporal_load(static_cast<const stream_u4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream16(float* p, float4 v) {
    __builtin_nontemporal_store(stream_f4{v.x, v.y, v.z, v.w}, reinterpret_cast<stream_f4*>(p));
}

// ---------------------------------------------------------------------------
// Wavefront reductions, all on the VALU (no LDS-crossbar round trips): an
// inclusive scan inside each 16-lane row with DPP row_shr 1, 2, 4, 8 (lanes
// shifted in from outside the row read 0), then row_bcast15 (rows 1 and 3 add
// the last lane of the row below) and row_bcast31 (rows 2 and 3 add lane 31),
// which leaves the wavefront total in lane 63; v_readlane makes it uniform.
// The order of operations is fixed, so the result is deterministic.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, true);
}
constexpr int DPP_ROW_SHR1 = 0x111, DPP_ROW_SHR2 = 0x112, DPP_ROW_SHR4 = 0x114, DPP_ROW_SHR8 = 0x118;
constexpr int DPP_ROW_BCAST15 = 0x142, DPP_ROW_BCAST31 = 0x143;

template <class Op>
__device__ __forceinline__ float wave_reduce_f32(float v, Op op) {
    v = op(v, __uint_as_float(dpp_u32<DPP_ROW_SHR1>(__float_as_uint(v))));
    v = op(v, __uint_as_float(dpp_u32<DPP_ROW_SHR2>(__float_as_uint(v))));
    v = op(v, __uint_as_float(dpp_u32<DPP_ROW_SHR4>(__float_as_uint(v))));
    v = op(v, __uint_as_float(dpp_u32<DPP_ROW_SHR8>(__float_as_uint(v))));
    v = op(v, __uint_as_float(dpp_u32<DPP_ROW_BCAST15, 0xA>(__float_as_uint(v))));
    v = op(v, __uint_as_float(dpp_u32<DPP_ROW_BCAST31, 0xC>(__float_as_uint(v))));
    return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}
struct AddF { __device__ float operator()(float a, float b) const { return a + b; } };

// Sum over the 64 lanes; every lane receives the same total.
__device__ __forceinline__ float wave_sum(float v) { return wave_reduce_f32(v, AddF()); }

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t u = __double_as_longlong(v);
    const uint32_t lo = dpp_u32<CTRL, ROW_MASK>((uint32_t)u), hi = dpp_u32<CTRL, ROW_MASK>((uint32_t)(u >> 32));
    return __longlong_as_double(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double wave_sum_f64(double v) {
    v += dpp_f64<DPP_ROW_SHR1>(v);
    v += dpp_f64<DPP_ROW_SHR2>(v);
    v += dpp_f64<DPP_ROW_SHR4>(v);
    v += dpp_f64<DPP_ROW_SHR8>(v);
    v += dpp_f64<DPP_ROW_BCAST15, 0xA>(v);
    v += dpp_f64<DPP_ROW_BCAST31, 0xC>(v);
    const uint64_t u = __double_as_longlong(v);
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, 63), hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), 63);
    return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

// Wave-wide maximum of an unsigned 32-bit value (0 is the neutral element);
// every lane receives it.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<DPP_ROW_SHR1>(v));
    v = max(v, dpp_u32<DPP_ROW_SHR2>(v));
    v = max(v, dpp_u32<DPP_ROW_SHR4>(v));
    v = max(v, dpp_u32<DPP_ROW_SHR8>(v));
    v = max(v, dpp_u32<DPP_ROW_BCAST15, 0xA>(v));
    v = max(v, dpp_u32<DPP_ROW_BCAST31, 0xC>(v));
    return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Index of this wavefront in its workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_index() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / WAVE));
}

// Lanes below this one, as a 64-bit mask.
__device__ __forceinline__ uint64_t lanemask_lt() {
    int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// ---------------------------------------------------------------------------
// Workspace layout.  Computed on the host (api.cpp) from the config; every
// region is 256-byte aligned.  Kernels receive the individual pointers.
// ---------------------------------------------------------------------------
struct Layout {
    size_t logits, topk_idx, topk_w, offsets, perm_rows, inv_perm;
    size_t blk_hist, blk_base, meta, active, tiles, h, slot_out, shared_out, scores, dslots, total;
    int n_blk;       // permutation blocks of PERM_BLOCK assignments
    int max_tiles;   // capacity of the grouped-GEMM tile list
};

// Meta words at ws + meta: [0] n_active experts, [1] n_tiles, [2] valid
// assignments, the rest reserved.
constexpr int META_WORDS = 16;
constexpr int PERM_BLOCK = 256;     // assignments per permutation block (one wave)
constexpr int GEMM_BM = 64;         // rows per grouped-GEMM tile (tile list granularity)

}  // namespace moe
