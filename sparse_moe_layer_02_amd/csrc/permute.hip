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

namespace moe {

__device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = lane_id();
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const int u = __shfl_up(v, o);
        if (lane >= o) v += u;
    }
    return v;
}

// Exclusive scan of one int per thread over a 1024-thread block.
__device__ int block_excl_scan_1024(int v, int* smem /*[16]*/, int* total) {
    const int lane = lane_id(), wave = threadIdx.x / WAVE;
    const int inc = wave_incl_scan(v);
    if (lane == WAVE - 1) smem[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        int w = lane < 16 ? smem[lane] : 0;
        const int wi = wave_incl_scan(w);
        if (lane < 16) smem[lane] = wi - w;  // exclusive prefix of wave totals
        if (lane == 15) smem[16] = wi;
    }
    __syncthreads();
    const int out = smem[wave] + inc - v;
    *total = smem[16];
    __syncthreads();
    return out;
}

// Expert-index bits needed to tell E experts apart.
__device__ __forceinline__ int index_bits(int E) {
    int b = 0;
    while ((1 << b) < E) ++b;
    return b;
}

// Rank, among the lanes holding the same expert, of this lane (ascending lane
// order), and the number of such lanes.  Invalid lanes take no part.
__device__ __forceinline__ void multisplit_rank(int e, bool valid, int nbits, int* rank, int* count,
                                                int* leader) {
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t bb = __ballot(bit);
        peers &= bit ? bb : ~bb;
    }
    *rank = __popcll(peers & lanemask_lt());
    *count = __popcll(peers);
    *leader = __ffsll((unsigned long long)peers) - 1;
}

// Lists derived from the expert counts: offsets, active experts, GEMM tiles.
// Called by all 1024 threads; thread e < E holds count c.  `own` = this call
// produced the permutation (write offsets and the perm_rows tail), as opposed
// to deriving the lists from a caller's offsets.
__device__ void emit_lists(const PermArgs& a, int c, int* smem, int* off_out, bool own = true) {
    const int e = threadIdx.x, E = a.E;
    int total, n_active, n_rtiles;
    const int off = block_excl_scan_1024(e < E ? c : 0, smem, &total);
    const int act = (e < E && c > 0) ? 1 : 0;
    const int apos = block_excl_scan_1024(act, smem, &n_active);
    const int nt = e < E ? (c + a.bm - 1) / a.bm : 0;
    const int tbase = block_excl_scan_1024(nt, smem, &n_rtiles);
    if (e < E) {
        if (own) a.offsets[e] = off;
        if (act) a.active[apos] = e;
        for (int i = 0; i < nt; ++i) a.tiles[tbase + i] = make_int2(e, i * a.bm);
    }
    const int s_tiles = a.n_shared ? (a.T + a.bm - 1) / a.bm : 0;
    for (int i = e; i < s_tiles; i += blockDim.x) a.tiles[n_rtiles + i] = make_int2(E, i * a.bm);
    if (e == 0) {
        if (own) a.offsets[E] = total;
        a.meta[0] = n_active;
        a.meta[1] = n_rtiles + s_tiles;
        a.meta[2] = total;
    }
    if (own) {
        const int n = a.T * a.k;
        for (int r = total + e; r < n; r += blockDim.x) a.perm_rows[r] = -1;
    }
    *off_out = off;
}

// Stable scatter of assignments [f0, f1) by one wave, cursors in LDS.
__device__ void scatter_range(const PermArgs& a, int f0, int f1, int* cursor) {
    const int lane = lane_id(), E = a.E, nbits = index_bits(E);
    for (int c0 = f0; c0 < f1; c0 += WAVE) {
        const int f = c0 + lane;
        const int e = f < f1 ? a.topk_idx[f] : -1;
        const bool valid = f < f1 && e >= 0 && e < E;
        int rank, count, leader;
        multisplit_rank(e, valid, nbits, &rank, &count, &leader);
        const int base = valid ? cursor[e] : 0;
        if (valid && lane == leader) cursor[e] = base + count;
        const int pos = valid ? base + rank : -1;
        if (valid) a.perm_rows[pos] = f;
        if (f < f1) a.inv_perm[f] = pos;
    }
}

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

__global__ __launch_bounds__(1024) void perm_scan_kernel(PermArgs a) {
    __shared__ int smem[17];
    const int e = threadIdx.x, E = a.E;
    int c = 0;
    if (e < E)
        for (int b = 0; b < a.n_blk; ++b) c += a.blk_hist[(size_t)b * E + e];
    int off;
    emit_lists(a, c, smem, &off);
    if (e < E) {
        int run = off;
        for (int b = 0; b < a.n_blk; ++b) {
            a.blk_base[(size_t)b * E + e] = run;
            run += a.blk_hist[(size_t)b * E + e];
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

hipError_t launch_lists_from_offsets(const PermArgs& a, hipStream_t st) {
    lists_from_offsets_kernel<<<1, 1024, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_permute(const PermArgs& a, hipStream_t st) {
    const int n = a.T * a.k;
    if (n <= 1024) {
        permute_small_kernel<<<1, 1024, 0, st>>>(a);
    } else {
        perm_hist_kernel<<<a.n_blk, 256, 0, st>>>(a);
        perm_scan_kernel<<<1, 1024, 0, st>>>(a);
        perm_scatter_kernel<<<a.n_blk, 64, 0, st>>>(a);
    }
    return hipGetLastError();
}

}  // namespace moe
