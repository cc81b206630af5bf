// permute_dev.h - device building blocks of the token->expert grouping
// (stable counting sort by expert): block-wide scans, the ballot multisplit
// rank, the list emitter (offsets, active experts, grouped-GEMM tiles) and the
// stable scatter.  Shared by the permutation kernels and the fused decode
// routing kernel.
#pragma once
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
    const int nt = (e < E && a.bm > 0) ? (c + a.bm - 1) / a.bm : 0;  // bm == 0: no tile list
    const int tbase = block_excl_scan_1024(nt, smem, &n_rtiles);
    if (e < E) {
        if (own) a.offsets[e] = off;
        if (act) a.active[apos] = e;
        for (int i = 0; i < nt; ++i) a.tiles[tbase + i] = make_int2(e, i * a.bm);
    }
    const int s_tiles = (a.n_shared && a.bm > 0) ? (a.T + a.bm - 1) / a.bm : 0;
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

}  // namespace moe
