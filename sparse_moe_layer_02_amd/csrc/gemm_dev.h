// gemm_dev.h - tile bookkeeping shared by the grouped-GEMM kernels.
#pragma once
#include "common.h"
#include "kernels.h"

namespace moe {

// Rows of one tile: which source row to read and where the result goes.
struct TileRows {
    int g;        // group: expert, or E for the shared expert
    int rbeg;     // first row in permutation (h) order
    int nrows;    // valid rows (<= BM)
};

// Tiles in the list (the device-side count the permutation step wrote).
__device__ __forceinline__ int tile_count(const FfnArgs& a) { return a.meta[1]; }

template <int BM>
__device__ __forceinline__ bool tile_rows(const FfnArgs& a, int tile, TileRows& tr) {
    if (tile >= tile_count(a)) return false;
    const int2 t = a.tiles[tile];
    tr.g = t.x;
    if (t.x == a.E) {  // shared expert: rows are tokens
        tr.rbeg = a.T * a.k + t.y;
        tr.nrows = min(BM, a.T - t.y);
    } else {
        tr.rbeg = a.offsets[t.x] + t.y;
        tr.nrows = min(BM, a.offsets[t.x + 1] - tr.rbeg);
    }
    return true;
}
// 16 bytes as a vector value (kept in registers; a struct copy of uint4 can
// end up in scratch memory when staged across a loop).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
// A weight row piece that no other tile of the launch reads: non-temporal.
template <bool NT>
__device__ __forceinline__ u32x4 ld16w(const uint16_t* p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    else return ld16(p);
}
__device__ __forceinline__ void st16(uint8_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// The dispatcher deals consecutive workgroups to the 8 XCDs in turn, and each
// XCD has its own L2.  Only the first nt * gridDim.y workgroups have work (nt =
// the tile count the permutation step wrote; the grid is sized for the host's
// upper bound), and they are remapped so that every XCD receives an equal,
// contiguous range of the logical work order; the rest return false.  The
// logical order walks groups of NG N tiles; inside a group, M tile by M tile,
// all N tiles of the group.  The workgroups an XCD runs side by side then cover
// a block of M tiles x NG N tiles: each weight tile is read by the M tiles of
// its expert and each A tile (rows of x or h) by the group's N tiles, mostly
// from that XCD's L2.  NG = 4 pays off for tiles of 128 rows or more (experts
// with many rows).  With 64-row tiles (few rows per expert, bandwidth-bound)
// every weight tile is read by one M tile anyway, and NG = 16 lets the N
// tiles that share an activation tile run side by side (about 2-3% faster
// than NG = 1 at 512 tokens, bf16 and int8 weights).
constexpr int N_XCD = 8;

template <int NG>
__device__ __forceinline__ bool work_item(int nt, int& tile, int& ntile) {
    const int gy = gridDim.y;
    nt = min(nt, (int)gridDim.x);  // never more tiles than the grid was sized for
    const int L = blockIdx.x + blockIdx.y * gridDim.x, N = nt * gy;
    if (L >= N) return false;
    const int q = N / N_XCD, r = N % N_XCD, xcd = L % N_XCD, loc = L / N_XCD;
    const int logical = xcd < r ? xcd * (q + 1) + loc : r * (q + 1) + (xcd - r) * q + loc;
    const int group = logical / (nt * NG), rem = logical % (nt * NG);
    const int gsize = min(NG, gy - group * NG);
    tile = rem / gsize;
    ntile = group * NG + rem % gsize;
    return true;
}

}  // namespace moe
