// prefetch.hip - the read half of the router look-ahead: run the next layer's
// router early (on this layer's input) and read the experts it predicts
// before that layer needs them (NeutronStar fork page, cross-layer expert
// prefetch, where the reads fill a host cache from disk).  Here the weights
// live in HBM, and the reads fill the device's memory-side cache (the 256 MB
// Infinity Cache, which every HBM read passes through), so that the next
// layer's expert GEMVs find part of their weight stream there.  The router
// half is moe_route with the next layer's router weights; this file is the
// read of the predicted experts' weights.
//
// One launch reads, for each predicted expert, any subset of its gate, up and
// down matrices (int8 codes and their fp16 scales, or the bf16 / fp32
// elements), or their leading rows only.  The work is a flat list of 64 KiB
// chunks ordered (segment, chunk, expert): the GEMVs of the next layer read
// all experts side by side.  A fixed number of workgroups walks the list, so the launch leaves most of
// the chip to the kernels that run beside it.  The loaded data feeds an empty
// asm statement only: nothing is written.  Ids outside [0, E) are skipped.
#include "prefetch.h"

namespace moe {
namespace {

typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

constexpr int PF_THREADS = 256;
constexpr int PF_UNROLL = 16;                                // 16-byte loads in flight per lane
constexpr int64_t PF_CHUNK = (int64_t)PF_THREADS * 16 * PF_UNROLL;  // 64 KiB per workgroup step

__global__ __launch_bounds__(PF_THREADS) void prefetch_experts_kernel(PrefetchArgs a) {
    // chunk list: segment s (in the order of a.base), then chunk, then expert
    int64_t seg_start[PF_SEGMENTS + 1];
    seg_start[0] = 0;
#pragma unroll
    for (int s = 0; s < PF_SEGMENTS; ++s)
        seg_start[s + 1] = seg_start[s] + (a.base[s] ? (a.bytes[s] + PF_CHUNK - 1) / PF_CHUNK * a.n_ids : 0);
    const int64_t total = seg_start[PF_SEGMENTS];
    for (int64_t c = blockIdx.x; c < total; c += gridDim.x) {
        int s = 0;
#pragma unroll
        for (int q = 1; q < PF_SEGMENTS; ++q) s += c >= seg_start[q] ? 1 : 0;
        const int64_t r = c - seg_start[s];
        const int j = (int)(r % a.n_ids);
        const int64_t chunk = r / a.n_ids;
        const int e = a.ids[j];
        if (e < 0 || e >= a.E) continue;
        // the expert's segment as a buffer: loads past its end return 0
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(a.base[s] + (int64_t)e * a.stride[s]), (short)0, (int)a.bytes[s], 0x00020000);
        // unsigned offsets: past 2^31 - 1 they stay past the buffer's end (bytes < 2^31)
        const uint32_t off0 = (uint32_t)(chunk * PF_CHUNK) + threadIdx.x * 16u;
        v4u32 v[PF_UNROLL];
#pragma unroll
        for (int u = 0; u < PF_UNROLL; ++u)
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(off0 + (uint32_t)(u * PF_THREADS * 16)), 0, 0);
#pragma unroll
        for (int u = 0; u < PF_UNROLL; ++u) asm volatile("" ::"v"(v[u]));
    }
}

}  // namespace

hipError_t launch_prefetch_experts(const PrefetchArgs& a, int workgroups, hipStream_t st, const KTime& kt) {
    if (a.n_ids <= 0) return hipSuccess;
    launch_kernel(prefetch_experts_kernel, dim3(workgroups), dim3(PF_THREADS), st, kt, a);
    return hipGetLastError();
}

}  // namespace moe
