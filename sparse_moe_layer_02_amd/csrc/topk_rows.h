// topk_rows.h - launch interface of the row top-k (topk_rows.hip) for the C-ABI
// host code, and the wavefront scan it uses.
#pragma once
#include "kernels.h"

namespace moe {

// Top-k over long candidate rows (one workgroup per row); n <= TOPK_ROWS_MAX_N.
constexpr int TOPK_ROWS_MAX_N = 65536;
struct TopkRowsArgs {
    const float* scores;  // [rows, n]
    int rows, n, k;
    int32_t* idx;     // [rows, k], ascending candidate index
    float* vals;      // [rows, k] or null
    int sample_rank;  // rank of the sampled threshold (0: no sampled pass); set by launch_topk_rows
};
hipError_t launch_topk_rows(const TopkRowsArgs& a, hipStream_t st, const KTime& kt = KTime());
int topk_rows_threads(int n);  // workgroup size of the launch that takes n candidates
int topk_rows_npt(int n);      // keys per thread of that launch (0: n out of range)

// Inclusive scan of an unsigned 32-bit value over the 64 lanes, with the DPP
// steps of the wavefront reductions in common.h: after them lane l holds the
// sum of lanes 0..l.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
    v += dpp_u32<DPP_ROW_SHR1>(v);
    v += dpp_u32<DPP_ROW_SHR2>(v);
    v += dpp_u32<DPP_ROW_SHR4>(v);
    v += dpp_u32<DPP_ROW_SHR8>(v);
    v += dpp_u32<DPP_ROW_BCAST15, 0xA>(v);
    v += dpp_u32<DPP_ROW_BCAST31, 0xC>(v);
    return v;
}

// Wave-wide sum of an unsigned 32-bit value; every lane receives it.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
    return __builtin_amdgcn_readlane(wave_incl_scan_u32(v), 63);
}

}  // namespace moe
