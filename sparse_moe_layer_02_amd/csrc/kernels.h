// kernels.h - internal launch interface between the C-ABI host code (api.hip)
// and the kernel files.  Every launcher enqueues on the given stream and
// returns hipGetLastError().
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace moe {

// Kernel timing of one stage: `start` receives the start timestamp of the
// stage's first kernel dispatch, `stop` the end timestamp of its last
// (hipExtLaunchKernel events, taken from the dispatch itself, so launch gaps
// before and after the stage are not counted).  Either may be null.
struct KTime {
    hipEvent_t start = nullptr, stop = nullptr;
    KTime first() const { return KTime{start, nullptr}; }
    KTime last() const { return KTime{nullptr, stop}; }
};

template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kern)(KArgs...), dim3 grid, dim3 block, hipStream_t st, const KTime& kt,
                          Args... args) {
    if (kt.start || kt.stop) hipExtLaunchKernelGGL(kern, grid, block, 0, st, kt.start, kt.stop, 0, args...);
    else kern<<<grid, block, 0, st>>>(args...);
}

struct RouteArgs {
    const void* x;
    const float* wr;
    int T, d, E, act;
    float* logits;
    bool force_gemm;  // use the tiled prefill kernel even for few tokens
};
hipError_t launch_router_logits(const RouteArgs& a, hipStream_t st, const KTime& kt = KTime());

struct SelectArgs {
    const float* logits;
    const float* bias;
    int T, E, k, score;
    float route_scale;
    int32_t* topk_idx;
    float* topk_w;
    bool generic_only;  // skip the compile-time 256-expert instantiation
};
hipError_t launch_topk(const SelectArgs& a, hipStream_t st, const KTime& kt = KTime());

struct PermArgs {
    const int32_t* topk_idx;
    int T, k, E;
    int n_shared;
    int32_t* offsets;    // [E+1] (read-only for launch_lists_from_offsets)
    int32_t* perm_rows;  // [T*k]
    int32_t* inv_perm;   // [T*k]
    int32_t* blk_hist;   // [n_blk, E]
    int32_t* blk_base;   // [n_blk, E]
    int32_t* meta;       // META_WORDS
    int32_t* active;     // [E] experts with rows, ascending
    int2* tiles;         // [max_tiles] (group, first row) for the grouped GEMM
    int n_blk;
    int bm;              // tile rows for the tile list
};
hipError_t launch_permute(const PermArgs& a, hipStream_t st, const KTime& kt = KTime());
// active / tile lists from existing offsets (offsets and perm_rows untouched)
hipError_t launch_lists_from_offsets(const PermArgs& a, hipStream_t st, const KTime& kt = KTime());

// One expert slot of the decode path, written by the selection kernel and read
// by the decode expert kernels in a single dependent load.  Slot 0 is the
// shared expert when there is one (e = 0, shared = 1, tokens 0..T-1, weight
// 1); the routed slots follow in ascending expert index.  Slots past the last
// active expert carry e = -1.
struct DecodeSlot {
    int32_t e;       // expert index, -1 for an unused slot
    int32_t r0;      // first row of the slot in h
    int32_t m;       // tokens routed to the slot (h rows r0 .. r0+m-1)
    int32_t shared;  // 1 for the shared expert
    int32_t tok[MOE_DECODE_MAX_TOKENS];  // token of h row r0+i
    float w[MOE_DECODE_MAX_TOKENS];      // routing weight of that row (1 for the shared expert)
};

// One set of expert weights for the FFN kernels.
struct MatRef {
    const void* q;
    const uint16_t* scale;
};

struct FfnArgs {
    const void* x;          // [T, d]
    MatRef gate, up, down;  // routed [E, F, d], [E, F, d], [E, d, F]
    MatRef s_gate, s_up, s_down;
    const int32_t* offsets;
    const int32_t* perm_rows;
    const float* topk_w;
    const int32_t* meta;    // n_active at [0], n_tiles at [1]
    const int32_t* active;  // active experts, ascending
    const int2* tiles;
    int T, d, E, k, F, Fs, n_shared, act, wdt;
    void* h;                // [T*k + T*n_shared, ldh] in the activation format
    int ldh;                // max(F, Fs)
    float* slot_out;        // [T*k, d]
    float* shared_out;      // [T, d]
    float* y;               // [T, d] (fused combine)
    int max_tiles;          // grid bound of the grouped GEMMs (tiles of bm rows)
    int bm;                 // rows per grouped-GEMM tile: 64, 128 or 256
    int shared_done;        // the shared expert's h rows were already produced (decode route kernel)
    DecodeSlot* dslots;     // decode slot table (decode path only)
    int n_dslots;           // its capacity: n_shared + min(E, T*k)
    int grid_has_shared;    // set by the launchers: the last grid slot is the shared expert
};
// gate/up GEMV over the active experts (and the shared one) -> h
hipError_t launch_gateup_gemv(const FfnArgs& a, hipStream_t st, const KTime& kt = KTime());
// gate/up GEMV of the decode path over the routed slots of the decode slot table
hipError_t launch_gateup_gemv_decode(const FfnArgs& a, hipStream_t st, const KTime& kt = KTime());
// down GEMV writing weighted slot rows and the shared rows
hipError_t launch_down_slots_gemv(const FfnArgs& a, hipStream_t st, const KTime& kt = KTime());
// grouped bf16 MFMA GEMMs (prefill)
hipError_t launch_gateup_mfma(const FfnArgs& a, hipStream_t st, const KTime& kt = KTime());
hipError_t launch_down_mfma(const FfnArgs& a, hipStream_t st, const KTime& kt = KTime());
hipError_t launch_gateup_dma(const FfnArgs& a, hipStream_t st, const KTime& kt = KTime());
// grouped MFMA GEMMs for int8 (blocks of 32 + fp16 scale) weights, 64- or 128-row tiles
hipError_t launch_gateup_mfma_q8(const FfnArgs& a, hipStream_t st, const KTime& kt = KTime());
hipError_t launch_down_mfma_q8(const FfnArgs& a, hipStream_t st, const KTime& kt = KTime());
bool q8_dma_ok(const FfnArgs& a);
hipError_t launch_gateup_q8_dma(const FfnArgs& a, hipStream_t st, const KTime& kt = KTime());
hipError_t launch_down_q8_dma(const FfnArgs& a, hipStream_t st, const KTime& kt = KTime());
hipError_t launch_down_dma(const FfnArgs& a, hipStream_t st, const KTime& kt = KTime());

// The decode path (T <= MOE_DECODE_MAX_TOKENS) in four launches: router;
// selection + grouping beside the shared gate/up; routed gate/up; down +
// combine into f.y.  kt[s] times stage s (MOE_STAGES entries); the decode
// path launches nothing for the permutation and combine stages.
struct DecodeRouteArgs {
    RouteArgs r;
    SelectArgs s;
    PermArgs p;
    FfnArgs f;
    float* scores;  // [T, E] fp32 router scores (workspace)
};
hipError_t launch_decode(const DecodeRouteArgs& a, const KTime* kt, hipStream_t st);

struct CombineArgs {
    const float* slot_out;
    const float* shared_out;
    float* y;
    int T, k, d;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t st, const KTime& kt = KTime());

}  // namespace moe
