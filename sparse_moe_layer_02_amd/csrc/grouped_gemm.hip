// grouped_gemm.hip - prefill expert FFN as grouped bf16 GEMMs on the gfx950
// matrix cores (v_mfma_f32_32x32x16_bf16), fp32 accumulation.
//
//   gate/up:  H_e = bf16( silu(A_e Wg[e]^T) * (A_e Wu[e]^T) ),  A_e = rows of x
//             gathered through the permutation (no gathered copy is written)
//   down:     slot_out[f, :] = w_f * (H_e Wd[e]^T)[row of f]   (weighted scatter)
// The shared expert runs as one more group (index E) over all T tokens with
// weight 1, writing shared_out.
//
// The pages: a prefill chunk's tokens collectively route to most experts, so
// one read of an expert's weights serves all of its rows (NeutronStar README,
// "Long-prompt prefill"; main branch, Hy3 batch prefill); the batch kernels
// are expert tiles over gate/up then down (the LUT bug note and "GLM-5.2 CUDA
// port").
//
// Work list: the permutation step writes tiles (group, first row) of GEMM_BM
// rows; the grid is (tile slot, N tile) and slots past the device-side count
// exit at once.  Tiles: 64 rows x 64 N columns (gate/up: 64 gate + 64 up
// columns; down: 128 columns), K staged through LDS in 64-wide double-buffered
// chunks; 16-byte chunks are XOR-swizzled by row so the MFMA operand reads are
// free of bank conflicts.  Each wavefront owns a 32-row half and 32 (gate/up)
// or 64 (down) columns, so gate and up for the same output columns meet in one
// wavefront's registers for the SiLU*mul epilogue.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int BM = GEMM_BM;  // 64
constexpr int BK = 64;
constexpr int ROWB = BK * 2;  // bytes per LDS tile row (128)

// Byte offset of 16-byte chunk `ch` (0..7) of tile row `row` in LDS.
__device__ __forceinline__ int lds_off(int row, int ch) { return row * ROWB + ((ch ^ (row & 7)) << 4); }

__device__ __forceinline__ bf16x8_t lds_frag(const uint8_t* base, int row, int ch) {
    return *reinterpret_cast<const bf16x8_t*>(base + lds_off(row, ch));
}

// Rows of one tile: which source row to read and where the result goes.
struct TileRows {
    int g;        // group: expert, or E for the shared expert
    int rbeg;     // first row in permutation (h) order
    int nrows;    // valid rows (<= BM)
};

__device__ __forceinline__ bool tile_rows(const FfnArgs& a, int tile, TileRows& tr) {
    if (tile >= a.meta[1]) return false;
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

// The dispatcher deals consecutive workgroups to the 8 XCDs in turn, and each
// XCD has its own L2.  Remap the linear workgroup index so that every XCD
// receives one contiguous range of the logical work order (M tile fastest,
// then N tile): the M tiles of one expert, which read the same weight tile,
// then run side by side on one XCD and share its L2.
constexpr int N_XCD = 8;
constexpr bool TILE_FASTEST = true;

__device__ __forceinline__ void work_item(int& tile, int& ntile) {
    const int gx = gridDim.x, gy = gridDim.y;
    const int L = blockIdx.x + blockIdx.y * gx, N = gx * gy;
    const int q = N / N_XCD, r = N % N_XCD, xcd = L % N_XCD, loc = L / N_XCD;
    const int logical = xcd < r ? xcd * (q + 1) + loc : r * (q + 1) + (xcd - r) * q + loc;
    if (TILE_FASTEST) {
        tile = logical % gx;
        ntile = logical / gx;
    } else {
        tile = logical / gy;
        ntile = logical % gy;
    }
}

// ---------------------------------------------------------------------------
// gate/up
// ---------------------------------------------------------------------------
constexpr int GU_BN = 64;  // columns of gate (and of up) per workgroup

__global__ __launch_bounds__(256) void gateup_mfma_kernel(FfnArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + 2 * GU_BN) * ROWB];
    __shared__ int src_row[BM];
    int tile, ntile;
    work_item(tile, ntile);
    TileRows tr;
    if (!tile_rows(a, tile, tr)) return;
    const bool shared = tr.g == a.E;
    const int F = shared ? a.Fs : a.F;
    const int n0 = ntile * GU_BN;
    if (n0 >= F) return;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / WAVE;
    const int K = a.d;
    if (tid < BM) {
        int t = -1;
        if (tid < tr.nrows) {
            if (shared) {
                t = tr.rbeg - a.T * a.k + tid;
            } else {
                const int f = a.perm_rows[tr.rbeg + tid];
                t = (f >= 0 && f < a.T * a.k) ? f / a.k : -1;
            }
        }
        src_row[tid] = t;
    }
    __syncthreads();

    const MatRef& G = shared ? a.s_gate : a.gate;
    const MatRef& U = shared ? a.s_up : a.up;
    const int ge = shared ? 0 : tr.g;
    const uint16_t* gbase = static_cast<const uint16_t*>(G.q) + ((size_t)ge * F + n0) * K;
    const uint16_t* ubase = static_cast<const uint16_t*>(U.q) + ((size_t)ge * F + n0) * K;
    const uint16_t* xbase = static_cast<const uint16_t*>(a.x);

    // global -> register staging: each thread moves 2 A chunks, 2 gate, 2 up chunks of 16 B
    const int ch = tid & 7, r_lo = tid >> 3;  // rows r_lo and r_lo + 32
    int arow[2];
    bool bval[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int r = r_lo + 32 * p;
        arow[p] = src_row[r];
        bval[p] = n0 + r < F;
    }
    uint4 ra[2], rg[2], ru[2];
    auto gload = [&](int k0) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int r = r_lo + 32 * p;
            ra[p] = arow[p] >= 0 ? *reinterpret_cast<const uint4*>(xbase + (size_t)arow[p] * K + k0 + ch * 8)
                                 : make_uint4(0, 0, 0, 0);
            rg[p] = bval[p] ? *reinterpret_cast<const uint4*>(gbase + (size_t)r * K + k0 + ch * 8)
                            : make_uint4(0, 0, 0, 0);
            ru[p] = bval[p] ? *reinterpret_cast<const uint4*>(ubase + (size_t)r * K + k0 + ch * 8)
                            : make_uint4(0, 0, 0, 0);
        }
    };
    auto lstore = [&](int s) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int r = r_lo + 32 * p;
            *reinterpret_cast<uint4*>(&lds[s][lds_off(r, ch)]) = ra[p];
            *reinterpret_cast<uint4*>(&lds[s][lds_off(BM + r, ch)]) = rg[p];
            *reinterpret_cast<uint4*>(&lds[s][lds_off(BM + GU_BN + r, ch)]) = ru[p];
        }
    };

    const int mh = wave & 1, nh = wave >> 1;
    f32x16_t accg = {}, accu = {};
    gload(0);
    lstore(0);
    __syncthreads();
    int cur = 0;
    for (int k0 = 0; k0 < K; k0 += BK) {
        const bool more = k0 + BK < K;
        if (more) gload(k0 + BK);
        const uint8_t* L = lds[cur];
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = 2 * kk + (lane >> 5);
            const bf16x8_t fa = lds_frag(L, 32 * mh + (lane & 31), c);
            const bf16x8_t fg = lds_frag(L, BM + 32 * nh + (lane & 31), c);
            const bf16x8_t fu = lds_frag(L, BM + GU_BN + 32 * nh + (lane & 31), c);
            accg = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fg, accg, 0, 0, 0);
            accu = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fu, accu, 0, 0, 0);
        }
        if (more) lstore(cur ^ 1);
        __syncthreads();
        cur ^= 1;
    }

    // epilogue: lane holds column (lane & 31) and rows 8*(v/4) + 4*(lane/32) + v%4
    const int col = n0 + 32 * nh + (lane & 31);
    if (col < F) {
        uint16_t* h = static_cast<uint16_t*>(a.h);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int row = 32 * mh + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (row < tr.nrows) {
                const float g = accg[v], u = accu[v];
                h[(size_t)(tr.rbeg + row) * a.ldh + col] = f32_to_bf16(g / (1.0f + expf(-g)) * u);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// down + weighted scatter
// ---------------------------------------------------------------------------
constexpr int DN_BN = 128;

__global__ __launch_bounds__(256) void down_mfma_kernel(FfnArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + DN_BN) * ROWB];
    __shared__ int dst_row[BM];
    __shared__ float wrow[BM];
    int tile, ntile;
    work_item(tile, ntile);
    TileRows tr;
    if (!tile_rows(a, tile, tr)) return;
    const bool shared = tr.g == a.E;
    const int K = shared ? a.Fs : a.F;
    const int N = a.d;
    const int n0 = ntile * DN_BN;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / WAVE;
    if (tid < BM) {
        int dst = -1;
        float w = 0.0f;
        if (tid < tr.nrows) {
            if (shared) {
                dst = tr.rbeg - a.T * a.k + tid;
                w = 1.0f;
            } else {
                const int f = a.perm_rows[tr.rbeg + tid];
                if (f >= 0 && f < a.T * a.k) {
                    dst = f;
                    w = a.topk_w[f];
                }
            }
        }
        dst_row[tid] = dst;
        wrow[tid] = w;
    }
    __syncthreads();

    const MatRef& D = shared ? a.s_down : a.down;
    const int ge = shared ? 0 : tr.g;
    const uint16_t* dbase = static_cast<const uint16_t*>(D.q) + ((size_t)ge * N + n0) * K;
    const uint16_t* hbase = static_cast<const uint16_t*>(a.h);

    const int ch = tid & 7, r_lo = tid >> 3;
    bool aval[2], bval[4];
#pragma unroll
    for (int p = 0; p < 2; ++p) aval[p] = r_lo + 32 * p < tr.nrows;
#pragma unroll
    for (int p = 0; p < 4; ++p) bval[p] = n0 + r_lo + 32 * p < N;
    uint4 ra[2], rb[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int r = r_lo + 32 * p;
            ra[p] = aval[p] ? *reinterpret_cast<const uint4*>(hbase + (size_t)(tr.rbeg + r) * a.ldh + k0 + ch * 8)
                            : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int r = r_lo + 32 * p;
            rb[p] = bval[p] ? *reinterpret_cast<const uint4*>(dbase + (size_t)r * K + k0 + ch * 8)
                            : make_uint4(0, 0, 0, 0);
        }
    };
    auto lstore = [&](int s) {
#pragma unroll
        for (int p = 0; p < 2; ++p)
            *reinterpret_cast<uint4*>(&lds[s][lds_off(r_lo + 32 * p, ch)]) = ra[p];
#pragma unroll
        for (int p = 0; p < 4; ++p)
            *reinterpret_cast<uint4*>(&lds[s][lds_off(BM + r_lo + 32 * p, ch)]) = rb[p];
    };

    const int mh = wave & 1, nh = wave >> 1;  // wave: 32 rows x 64 columns (two 32x32 tiles)
    f32x16_t acc0 = {}, acc1 = {};
    gload(0);
    lstore(0);
    __syncthreads();
    int cur = 0;
    for (int k0 = 0; k0 < K; k0 += BK) {
        const bool more = k0 + BK < K;
        if (more) gload(k0 + BK);
        const uint8_t* L = lds[cur];
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = 2 * kk + (lane >> 5);
            const bf16x8_t fa = lds_frag(L, 32 * mh + (lane & 31), c);
            const bf16x8_t f0 = lds_frag(L, BM + 64 * nh + (lane & 31), c);
            const bf16x8_t f1 = lds_frag(L, BM + 64 * nh + 32 + (lane & 31), c);
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, f0, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, f1, acc1, 0, 0, 0);
        }
        if (more) lstore(cur ^ 1);
        __syncthreads();
        cur ^= 1;
    }

    float* out = shared ? a.shared_out : a.slot_out;
    const int c0 = n0 + 64 * nh + (lane & 31);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int row = 32 * mh + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < tr.nrows && dst_row[row] >= 0) {
            const size_t base = (size_t)dst_row[row] * N;
            const float w = wrow[row];
            if (c0 < N) out[base + c0] = w * acc0[v];
            if (c0 + 32 < N) out[base + c0 + 32] = w * acc1[v];
        }
    }
}

hipError_t launch_gateup_mfma(const FfnArgs& a, hipStream_t st, const KTime& kt) {
    const int fmax = a.n_shared && a.Fs > a.F ? a.Fs : a.F;
    dim3 grid(a.max_tiles, (fmax + GU_BN - 1) / GU_BN);
    launch_kernel(gateup_mfma_kernel, grid, 256, st, kt, a);
    return hipGetLastError();
}

hipError_t launch_down_mfma(const FfnArgs& a, hipStream_t st, const KTime& kt) {
    dim3 grid(a.max_tiles, (a.d + DN_BN - 1) / DN_BN);
    launch_kernel(down_mfma_kernel, grid, 256, st, kt, a);
    return hipGetLastError();
}

}  // namespace moe
