// prefetch.h - launch interface of the router look-ahead's weight reads
// (prefetch.hip).
#pragma once

#include "kernels.h"

namespace moe {

// Reads of predicted experts' weights (the router look-ahead): segment s of
// expert e is the first bytes[s] bytes at base[s] + e * stride[s]; a null
// base skips the segment.  ids [n_ids] on the device; ids outside [0, E) are
// skipped.
constexpr int PF_SEGMENTS = 6;  // gate codes, up codes, gate scales, up scales, down codes, down scales
struct PrefetchArgs {
    const uint8_t* base[PF_SEGMENTS];
    int64_t stride[PF_SEGMENTS], bytes[PF_SEGMENTS];
    const int32_t* ids;
    int n_ids, E;
};
hipError_t launch_prefetch_experts(const PrefetchArgs& a, int workgroups, hipStream_t st, const KTime& kt = KTime());

}  // namespace moe
