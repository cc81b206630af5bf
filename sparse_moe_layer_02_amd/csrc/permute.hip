// permute.hip - token->expert grouping on gfx950: a stable counting sort of the
// flat assignments f = t*k + j by expert.
//
//   offsets[e]   = number of assignments to experts < e   (offsets[E] = total)
//   perm_rows[r] = the f of row r, ordered by (expert, f)
//   inv_perm[f]  = r with perm_rows[r] == f
//
// It also emits the lists the expert kernels are launched over: the experts
// that received rows (ascending) and the grouped-GEMM tiles (expert, first row)
// including the shared expert's tiles as group E.
//
// The pages motivate the grouping: small indexed batches read only the
// selected experts (NeutronStar README, MTP paragraph), and a prefill chunk's
// rows that route to one expert share one read of its weights (NeutronStar
// README, "Long-prompt prefill"; main branch, Hy3 batch prefill).
//
// Stability without ordered atomics: counts are LDS atomics (order-free); the
// scatter walks assignments in ascending f, 64 at a time, and ranks lanes with
// equal experts by a ballot per expert-index bit (multisplit, Ashkiani et al.,
// "GPU Multisplit", PPoPP 2016) followed by a popcount of the lower lanes.
#include "common.h"
#include "kernels.h"
#include "permute_dev.h"

namespace moe {

// Small problems (T*k <= 1024): everything in one 1024-thread workgroup.
__global__ __launch_bounds__(1024) void permute_small_kernel(PermArgs a) {
    __shared__ int cnt[1024];
    __shared__ int smem[17];
    const int tid = threadIdx.x, E = a.E, n = a.T * a.k;
    cnt[tid] = 0;
    __syncthreads();
    for (int f = tid; f < n; f += blockDim.x) {
        const int e = a.topk_idx[f];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    const int c = cnt[tid];
    int off;
    emit_lists(a, c, smem, &off);
    cnt[tid] = off;  // becomes the scatter cursor
    __syncthreads();
    if (tid < WAVE) scatter_range(a, 0, n, cnt);
}

// Large problems: per-block histograms, one scan workgroup, per-block scatter.
__global__ __launch_bounds__(256) void perm_hist_kernel(PermArgs a) {
    __shared__ int cnt[1024];
    const int tid = threadIdx.x, E = a.E, n = a.T * a.k, b = blockIdx.x;
    for (int e = tid; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    const int f = b * PERM_BLOCK + tid;
    if (f < n) {
        const int e = a.topk_idx[f];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) a.blk_hist[(size_t)b * E + e] = cnt[e];
}

// Column sums and column prefix sums of the [n_blk, E] block histogram.  The
// 1024 threads split into SCAN_PARTS groups of 1024 / SCAN_PARTS lanes; lane e
// of group p owns expert columns e, e + 1024 / SCAN_PARTS, ... and adds the
// blocks p, p + SCAN_PARTS, ... (independent loads, many in flight), so the
// per-expert totals come from SCAN_PARTS partial sums in LDS instead of one
// serial walk over the blocks.  The bases then walk the blocks again, each
// group over its own contiguous range of blocks, starting from the totals of
// the ranges before it.
constexpr int SCAN_PARTS = 4;

__global__ __launch_bounds__(1024) void perm_scan_kernel(PermArgs a) {
    __shared__ int smem[17];
    __shared__ int part[SCAN_PARTS][1024];  // partial column sums per block range
    const int tid = threadIdx.x, E = a.E, nb = a.n_blk;
    constexpr int LANES = 1024 / SCAN_PARTS;
    const int g = tid / LANES, l = tid % LANES;
    const int bper = (nb + SCAN_PARTS - 1) / SCAN_PARTS;  // blocks of group g: [g*bper, min(nb, (g+1)*bper))
    const int b0 = g * bper, b1 = min(nb, b0 + bper);
    for (int e = l; e < E; e += LANES) {
        int c = 0;
#pragma unroll 8
        for (int b = b0; b < b1; ++b) c += a.blk_hist[(size_t)b * E + e];
        part[g][e] = c;
    }
    __syncthreads();
    int c = 0;
    if (tid < E)
        for (int q = 0; q < SCAN_PARTS; ++q) c += part[q][tid];
    int off;
    emit_lists(a, c, smem, &off);  // (its block scans synchronise the workgroup)
    if (tid < E) {  // offset of expert tid, then the group prefixes: part[q] becomes the start of range q
        int run = off;
        for (int q = 0; q < SCAN_PARTS; ++q) {
            const int v = part[q][tid];
            part[q][tid] = run;
            run += v;
        }
    }
    __syncthreads();
    for (int e = l; e < E; e += LANES) {
        int run = part[g][e];
        for (int b = b0; b < b1; ++b) {
            const int h = a.blk_hist[(size_t)b * E + e];
            a.blk_base[(size_t)b * E + e] = run;
            run += h;
        }
    }
}

__global__ __launch_bounds__(64) void perm_scatter_kernel(PermArgs a) {
    __shared__ int cursor[1024];
    const int b = blockIdx.x, E = a.E, n = a.T * a.k;
    for (int e = lane_id(); e < E; e += WAVE) cursor[e] = a.blk_base[(size_t)b * E + e];
    __syncthreads();
    const int f0 = b * PERM_BLOCK;
    scatter_range(a, f0, min(f0 + PERM_BLOCK, n), cursor);
}

// Active-expert and tile lists from a caller's offsets (no permutation work).
// Offsets that are not a monotone split of [0, <= T*k] give empty expert lists
// (the shared expert is still computed), so no kernel indexes past a buffer.
__global__ __launch_bounds__(1024) void lists_from_offsets_kernel(PermArgs a) {
    __shared__ int smem[17];
    const int e = threadIdx.x, n = a.T * a.k;
    bool ok = true;
    if (e < a.E) {
        const int lo = a.offsets[e], hi = a.offsets[e + 1];
        ok = lo >= 0 && lo <= hi && hi <= n && (e > 0 || lo == 0);
    }
    const bool all_ok = __syncthreads_and(ok);
    const int c = (e < a.E && all_ok) ? a.offsets[e + 1] - a.offsets[e] : 0;
    int off;
    emit_lists(a, c, smem, &off, false);
}

hipError_t launch_lists_from_offsets(const PermArgs& a, hipStream_t st, const KTime& kt) {
    launch_kernel(lists_from_offsets_kernel, 1, 1024, st, kt, a);
    return hipGetLastError();
}

hipError_t launch_permute(const PermArgs& a, hipStream_t st, const KTime& kt) {
    const int n = a.T * a.k;
    if (n <= 1024) {
        launch_kernel(permute_small_kernel, 1, 1024, st, kt, a);
    } else {
        launch_kernel(perm_hist_kernel, a.n_blk, 256, st, kt.first(), a);
        launch_kernel(perm_scan_kernel, 1, 1024, st, KTime(), a);
        launch_kernel(perm_scatter_kernel, a.n_blk, 64, st, kt.last(), a);
    }
    return hipGetLastError();
}

}  // namespace moe
