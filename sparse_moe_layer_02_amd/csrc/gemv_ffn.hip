// gemv_ffn.hip - expert FFN as bandwidth-bound GEMVs over only the selected
// experts' weights (the decode path), on gfx950.
//
//   h[row, :]      = silu(Wg[e] x_t) * (Wu[e] x_t)     (rounded to the act format)
//   slot[f, i]     = w_f * (Wd[e] h_row)[i]            (prefill GEMV fallback)
//
// The decode down projection and the combine are fused in decode.hip.
//
// The pages: a small batch reads the weights of its selected experts and no
// others (NeutronStar README, MTP paragraph); the limit is memory bandwidth
// rather than arithmetic (main branch, closing paragraph); decision tensors
// stay at Q8_0/F32 and experts are gate/up + down projections ("The model",
// "GLM-5.2 CUDA port").
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
#include "gemv_dev.h"

namespace moe {

// ---------------------------------------------------------------------------
// gate/up: grid (row tiles, slot).  Slot s < n_active is active[s]; the last
// slot (when there is a shared expert) is the shared expert over all tokens.
// ---------------------------------------------------------------------------
template <int WF, int AF, int RG, int MT>
__global__ __launch_bounds__(256) void gateup_gemv_kernel(FfnArgs a) {
    const int slot = blockIdx.y;
    const bool shared = a.grid_has_shared && slot == (int)gridDim.y - 1;
    int e, F, r0, m;
    if (shared) {
        e = 0; F = a.Fs; r0 = a.T * a.k; m = a.T;
    } else {
        if (slot >= a.meta[0]) return;
        e = a.active[slot]; F = a.F; r0 = a.offsets[e]; m = a.offsets[e + 1] - r0;
    }
    const int row0 = (blockIdx.x * 4 + wave_index()) * RG;
    if (row0 >= F) return;
    // two 16-byte loads per weight row in flight per lane (a 4096-wide int8
    // row is read in two halves): measured slightly faster than the whole row
    gateup_wave<WF, AF, RG, MT, 2>(a, shared, e, F, r0, m, row0, shared ? nullptr : a.perm_rows + r0);
}

// ---------------------------------------------------------------------------
// gate/up of the decode path: grid (row tiles, routed slot); a workgroup
// reads its slot's expert, h rows and tokens from the decode slot table in
// one load, so the weight stream starts one memory round trip after launch.
// ---------------------------------------------------------------------------
template <int WF, int AF, int RG, int MT>
__global__ __launch_bounds__(256) void gateup_gemv_decode_kernel(FfnArgs a) {
    const DecodeSlot* D = a.dslots + (a.n_shared ? 1 : 0) + blockIdx.y;
    const int4 hd = *reinterpret_cast<const int4*>(D);  // e, r0, m: one load, before any branch
    const int row0 = (blockIdx.x * 4 + wave_index()) * RG;
    if (hd.x < 0 || row0 >= a.F) return;
    gateup_wave<WF, AF, RG, MT, 4, true>(a, false, hd.x, a.F, hd.y, hd.z, row0, D->tok);
}

// ---------------------------------------------------------------------------
// down into slots: grid (row tiles, slot); writes slot_out[f] = w_f * down
// rows and shared_out[t] (weight 1).
// ---------------------------------------------------------------------------
template <int WF, int AF, int RD, int MT>
__global__ __launch_bounds__(256) void down_slots_kernel(FfnArgs a) {
    const int slot = blockIdx.y;
    const bool shared = a.grid_has_shared && slot == (int)gridDim.y - 1;
    int e, F, r0, m;
    if (shared) {
        e = 0; F = a.Fs; r0 = a.T * a.k; m = a.T;
    } else {
        if (slot >= a.meta[0]) return;
        e = a.active[slot]; F = a.F; r0 = a.offsets[e]; m = a.offsets[e + 1] - r0;
    }
    const int row0 = (blockIdx.x * 4 + wave_index()) * RD;
    if (row0 >= a.d) return;
    down_rows_wave<WF, AF, RD, MT>(a, shared, e, F, r0, m, row0);
}

// ---------------------------------------------------------------------------
// combine: y[t] = shared_out[t] + sum_j slot_out[t*k + j], four columns per thread.
// Every input is read once and y is written once, so the accesses are
// non-temporal: the slot rows stream past the caches instead of displacing
// what they hold (c5: 188 -> 161 us).  The additions keep their order.
// ---------------------------------------------------------------------------
typedef float cf4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
    const size_t n4 = (size_t)a.T * a.d / 4;
    for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < n4; q += (size_t)gridDim.x * blockDim.x) {
        const size_t t = q * 4 / a.d, c = q * 4 % a.d;
        cf4 acc = a.shared_out ? __builtin_nontemporal_load(reinterpret_cast<const cf4*>(a.shared_out + t * a.d + c))
                               : cf4{0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < a.k; ++j)
            acc += __builtin_nontemporal_load(reinterpret_cast<const cf4*>(a.slot_out + (t * a.k + j) * a.d + c));
        __builtin_nontemporal_store(acc, reinterpret_cast<cf4*>(a.y + t * a.d + c));
    }
}
// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
constexpr int RG_ROWS = 1;  // gate (and up) rows per wavefront
constexpr int RD_ROWS = 4;  // down rows per wavefront

static int pick_mt(int max_rows) { return max_rows <= 1 ? 1 : max_rows <= 2 ? 2 : max_rows <= 4 ? 4 : 8; }

#define MOE_DISPATCH_MT(KERNEL, WF, AF, R, MTV, GRID, ARGS, ST, KT)                                  \
    do {                                                                                          \
        if ((MTV) == 1) launch_kernel(KERNEL<WF, AF, R, 1>, GRID, 256, ST, KT, ARGS);             \
        else if ((MTV) == 2) launch_kernel(KERNEL<WF, AF, R, 2>, GRID, 256, ST, KT, ARGS);        \
        else if ((MTV) == 4 || (WF) == MOE_DT_Q8B32)                                              \
            launch_kernel(KERNEL<WF, AF, R, 4>, GRID, 256, ST, KT, ARGS);                         \
        else launch_kernel(KERNEL<WF, AF, R, 8>, GRID, 256, ST, KT, ARGS);                        \
    } while (0)

#define MOE_DISPATCH_FMT(KERNEL, R, MTV, GRID, ARGS, ST, KT)                                   \
    do {                                                                                       \
        if ((ARGS).wdt == MOE_DT_F32)                                                          \
            MOE_DISPATCH_MT(KERNEL, MOE_DT_F32, MOE_DT_F32, R, MTV, GRID, ARGS, ST, KT);       \
        else if ((ARGS).wdt == MOE_DT_BF16)                                                    \
            MOE_DISPATCH_MT(KERNEL, MOE_DT_BF16, MOE_DT_BF16, R, MTV, GRID, ARGS, ST, KT);     \
        else                                                                                   \
            MOE_DISPATCH_MT(KERNEL, MOE_DT_Q8B32, MOE_DT_BF16, R, MTV, GRID, ARGS, ST, KT);    \
    } while (0)

hipError_t launch_gateup_gemv(const FfnArgs& a0, hipStream_t st, const KTime& kt) {
    FfnArgs a = a0;
    a.grid_has_shared = a.n_shared && !a.shared_done;
    const int fmax = a.grid_has_shared && a.Fs > a.F ? a.Fs : a.F;
    const int slots = (a.E < a.T * a.k ? a.E : a.T * a.k) + (a.grid_has_shared ? 1 : 0);
    dim3 grid((fmax + 4 * RG_ROWS - 1) / (4 * RG_ROWS), slots);
    const int mt = pick_mt(a.T);
    MOE_DISPATCH_FMT(gateup_gemv_kernel, RG_ROWS, mt, grid, a, st, kt);
    return hipGetLastError();
}

hipError_t launch_gateup_gemv_decode(const FfnArgs& a, hipStream_t st, const KTime& kt) {
    const int slots = a.E < a.T * a.k ? a.E : a.T * a.k;
    dim3 grid((a.F + 4 * RG_ROWS - 1) / (4 * RG_ROWS), slots);
    const int mt = pick_mt(a.T);
    MOE_DISPATCH_FMT(gateup_gemv_decode_kernel, RG_ROWS, mt, grid, a, st, kt);
    return hipGetLastError();
}

hipError_t launch_down_slots_gemv(const FfnArgs& a0, hipStream_t st, const KTime& kt) {
    FfnArgs a = a0;
    a.grid_has_shared = a.n_shared && !a.shared_done;
    const int slots = (a.E < a.T * a.k ? a.E : a.T * a.k) + (a.grid_has_shared ? 1 : 0);
    dim3 grid((a.d + 4 * RD_ROWS - 1) / (4 * RD_ROWS), slots);
    const int mt = pick_mt(a.T);
    MOE_DISPATCH_FMT(down_slots_kernel, RD_ROWS, mt, grid, a, st, kt);
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t st, const KTime& kt) {
    const size_t n4 = (size_t)a.T * a.d / 4;
    const size_t want = (n4 + 255) / 256;
    const int blocks = (int)(want < 4096 ? want : 4096);
    launch_kernel(combine_kernel, blocks, 256, st, kt, a);
    return hipGetLastError();
}

}  // namespace moe
