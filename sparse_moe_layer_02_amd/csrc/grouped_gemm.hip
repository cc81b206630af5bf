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
// Work list: the permutation step writes tiles (group, first row) of bm rows
// (64; layers averaging 96 rows per expert or more take the LDS-copy
// kernels of grouped_gemm_dma.hip instead); the grid is (tile
// slot, N tile), remapped per XCD (work_item), and slots past the
// device-side count exit at once.  A workgroup computes bm rows by 64 gate
// + 64 up columns (gate/up) or by 128 output columns (down), K staged
// through LDS in 64-wide double-buffered chunks.  Global loads run two chunks
// ahead through two register sets and are unconditional (addresses clamped
// into the tensors, out-of-tile rows zeroed on the way into LDS).  16-byte
// chunks are XOR-swizzled by row so the MFMA operand reads do not pile onto
// the same banks.  Each wavefront owns bm/2 rows and 32 (gate/up) or 64
// (down) columns, so gate and up for the same output columns meet in one
// wavefront's registers for the SiLU*mul epilogue.
#include "common.h"
#include "kernels.h"
#include "gemm_dev.h"

namespace moe {

constexpr int BK = 64;
constexpr int ROWB = BK * 2;  // bytes per LDS tile row (128)

// Byte offset of 16-byte chunk `ch` (0..7) of tile row `row` in LDS.
__device__ __forceinline__ int lds_off(int row, int ch) { return row * ROWB + ((ch ^ (row & 7)) << 4); }

__device__ __forceinline__ bf16x8_t lds_frag(const uint8_t* base, int row, int ch) {
    return *reinterpret_cast<const bf16x8_t*>(base + lds_off(row, ch));
}

// ---------------------------------------------------------------------------
// gate/up
// ---------------------------------------------------------------------------
constexpr int GU_BN = 64;  // columns of gate (and of up) per workgroup

// BM rows x (64 gate + 64 up) columns per workgroup; wavefront (mh, nh) owns
// rows [BM/2 * mh, BM/2 * (mh + 1)) and columns [32 nh, 32 nh + 32) of both
// gate and up, as MT = BM/64 blocks of 32 rows.  NTW: weight loads
// non-temporal (experts of one tile: no other workgroup reads the rows).
template <int BM, bool NTW>
__global__ __launch_bounds__(256, 2) void gateup_mfma_kernel(FfnArgs a) {
    constexpr int MT = BM / 64, AP = BM / 32;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + 2 * GU_BN) * ROWB];
    __shared__ int src_row[BM];
    int tile, ntile;
    if (!work_item<BM == 128 ? 4 : 16>(tile_count(a), tile, ntile)) return;
    TileRows tr;
    if (!tile_rows<BM>(a, tile, tr)) return;
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

    // global -> register staging: each thread moves AP chunks of A and 2 of gate, 2 of up (16 B each)
    const int ch = tid & 7, r_lo = tid >> 3;  // rows r_lo + 32 p
    int arow[AP];
    bool bval[2];
#pragma unroll
    for (int p = 0; p < AP; ++p) arow[p] = src_row[r_lo + 32 * p];
#pragma unroll
    for (int p = 0; p < 2; ++p) bval[p] = n0 + r_lo + 32 * p < F;
    struct Stage {
        u32x4 a[AP], g[2], u[2];
    };
    // row pointers clamped into the tensors; rows past the tile read a valid
    // row and are zeroed
    const uint16_t* ap[AP];
    const uint16_t *gp[2], *up[2];
#pragma unroll
    for (int p = 0; p < AP; ++p) ap[p] = xbase + (size_t)(arow[p] >= 0 ? arow[p] : 0) * K + ch * 8;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int r = bval[p] ? r_lo + 32 * p : 0;
        gp[p] = gbase + (size_t)r * K + ch * 8;
        up[p] = ubase + (size_t)r * K + ch * 8;
    }
    auto gload = [&](Stage& R, int k0) {
#pragma unroll
        for (int p = 0; p < AP; ++p) R.a[p] = ld16(ap[p] + k0);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            R.g[p] = ld16w<NTW>(gp[p] + k0);
            R.u[p] = ld16w<NTW>(up[p] + k0);
        }
    };
    auto lstore = [&](const Stage& R, int s) {
#pragma unroll
        for (int p = 0; p < AP; ++p) st16(&lds[s][lds_off(r_lo + 32 * p, ch)], R.a[p]);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int r = r_lo + 32 * p;
            st16(&lds[s][lds_off(BM + r, ch)], R.g[p]);
            st16(&lds[s][lds_off(BM + GU_BN + r, ch)], R.u[p]);
        }
    };

    const int mh = wave & 1, nh = wave >> 1;
    f32x16_t accg[MT], accu[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        accg[i] = f32x16_t{};
        accu[i] = f32x16_t{};
    }
    // Half a chunk (two 16-wide steps of K): fragments first, then MFMAs.
    auto compute = [&](int s, int half) {
        const uint8_t* L = lds[s];
        bf16x8_t fg[2], fu[2], fa[2][MT];
        auto frags = [&](int j) {
            const int c = 2 * (2 * half + j) + (lane >> 5);
            fg[j] = lds_frag(L, BM + 32 * nh + (lane & 31), c);
            fu[j] = lds_frag(L, BM + GU_BN + 32 * nh + (lane & 31), c);
#pragma unroll
            for (int i = 0; i < MT; ++i) fa[j][i] = lds_frag(L, (BM / 2) * mh + 32 * i + (lane & 31), c);
        };
        frags(0);
        frags(1);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                accg[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[j][i], fg[j], accg[i], 0, 0, 0);
                accu[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[j][i], fu[j], accu[i], 0, 0, 0);
            }
    };
    // Two register sets: the loads of chunk j + 2 are issued while chunk j is
    // consumed, and stored to LDS one chunk later, so each load has two
    // chunks' worth of arithmetic to arrive.
    Stage R0, R1;
    gload(R0, 0);
    if (BK < K) gload(R1, BK);
    lstore(R0, 0);
    __syncthreads();
    for (int k0 = 0; k0 < K; k0 += 2 * BK) {
        if (k0 + 2 * BK < K) gload(R0, k0 + 2 * BK);
        compute(0, 0);
        compute(0, 1);
        if (k0 + BK < K) lstore(R1, 1);
        __syncthreads();
        if (k0 + BK >= K) break;
        if (k0 + 3 * BK < K) gload(R1, k0 + 3 * BK);
        compute(1, 0);
        compute(1, 1);
        if (k0 + 2 * BK < K) lstore(R0, 0);
        __syncthreads();
    }

    // epilogue: lane holds column (lane & 31) and rows 8*(v/4) + 4*(lane/32) + v%4 of each block
    const int col = n0 + 32 * nh + (lane & 31);
    if (col < F) {
        uint16_t* h = static_cast<uint16_t*>(a.h);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = (BM / 2) * mh + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row < tr.nrows) {
                    const float g = accg[i][v], u = accu[i][v];
                    h[(size_t)(tr.rbeg + row) * a.ldh + col] = f32_to_bf16(silu_f32(g) * u);
                }
            }
    }
}

// ---------------------------------------------------------------------------
// down + weighted scatter
// ---------------------------------------------------------------------------
constexpr int DN_BN = 128;

// BM rows x 128 output columns per workgroup; wavefront (mh, nh) owns rows
// [BM/2 * mh, BM/2 * (mh + 1)) as MT = BM/64 blocks of 32, and columns
// [64 nh, 64 nh + 64) as two 32-column blocks.  NTW as for gate/up.
template <int BM, bool NTW>
__global__ __launch_bounds__(256, 2) void down_mfma_kernel(FfnArgs a) {
    constexpr int MT = BM / 64, AP = BM / 32;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + DN_BN) * ROWB];
    __shared__ int dst_row[BM];
    __shared__ float wrow[BM];
    int tile, ntile;
    if (!work_item<BM == 128 ? 4 : 16>(tile_count(a), tile, ntile)) return;
    TileRows tr;
    if (!tile_rows<BM>(a, tile, tr)) return;
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
    bool aval[AP], bval[4];
#pragma unroll
    for (int p = 0; p < AP; ++p) aval[p] = r_lo + 32 * p < tr.nrows;
#pragma unroll
    for (int p = 0; p < 4; ++p) bval[p] = n0 + r_lo + 32 * p < N;
    struct Stage {
        u32x4 a[AP], b[4];
    };
    const uint16_t* ap[AP];
    const uint16_t* bp[4];
#pragma unroll
    for (int p = 0; p < AP; ++p) ap[p] = hbase + (size_t)(tr.rbeg + (aval[p] ? r_lo + 32 * p : 0)) * a.ldh + ch * 8;
#pragma unroll
    for (int p = 0; p < 4; ++p) bp[p] = dbase + (size_t)(bval[p] ? r_lo + 32 * p : 0) * K + ch * 8;
    auto gload = [&](Stage& R, int k0) {
#pragma unroll
        for (int p = 0; p < AP; ++p) R.a[p] = ld16(ap[p] + k0);
#pragma unroll
        for (int p = 0; p < 4; ++p) R.b[p] = ld16w<NTW>(bp[p] + k0);
    };
    auto lstore = [&](const Stage& R, int s) {
#pragma unroll
        for (int p = 0; p < AP; ++p) st16(&lds[s][lds_off(r_lo + 32 * p, ch)], R.a[p]);
#pragma unroll
        for (int p = 0; p < 4; ++p) st16(&lds[s][lds_off(BM + r_lo + 32 * p, ch)], R.b[p]);
    };

    const int mh = wave & 1, nh = wave >> 1;
    f32x16_t acc0[MT], acc1[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        acc0[i] = f32x16_t{};
        acc1[i] = f32x16_t{};
    }
    auto compute = [&](int s, int half) {
        const uint8_t* L = lds[s];
        bf16x8_t f0[2], f1[2], fa[2][MT];
        auto frags = [&](int j) {
            const int c = 2 * (2 * half + j) + (lane >> 5);
            f0[j] = lds_frag(L, BM + 64 * nh + (lane & 31), c);
            f1[j] = lds_frag(L, BM + 64 * nh + 32 + (lane & 31), c);
#pragma unroll
            for (int i = 0; i < MT; ++i) fa[j][i] = lds_frag(L, (BM / 2) * mh + 32 * i + (lane & 31), c);
        };
        frags(0);
        frags(1);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                acc0[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[j][i], f0[j], acc0[i], 0, 0, 0);
                acc1[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[j][i], f1[j], acc1[i], 0, 0, 0);
            }
    };
    Stage R0, R1;
    gload(R0, 0);
    if (BK < K) gload(R1, BK);
    lstore(R0, 0);
    __syncthreads();
    for (int k0 = 0; k0 < K; k0 += 2 * BK) {
        if (k0 + 2 * BK < K) gload(R0, k0 + 2 * BK);
        compute(0, 0);
        compute(0, 1);
        if (k0 + BK < K) lstore(R1, 1);
        __syncthreads();
        if (k0 + BK >= K) break;
        if (k0 + 3 * BK < K) gload(R1, k0 + 3 * BK);
        compute(1, 0);
        compute(1, 1);
        if (k0 + 2 * BK < K) lstore(R0, 0);
        __syncthreads();
    }

    float* out = shared ? a.shared_out : a.slot_out;
    const int c0 = n0 + 64 * nh + (lane & 31);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int row = (BM / 2) * mh + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (row < tr.nrows && dst_row[row] >= 0) {
                const size_t base = (size_t)dst_row[row] * N;
                const float w = wrow[row];
                if (c0 < N) out[base + c0] = w * acc0[i][v];
                if (c0 + 32 < N) out[base + c0 + 32] = w * acc1[i][v];
            }
        }
}

// Weight loads non-temporal when the experts average at most 32 rows (one
// 64-row tile each, mostly): c4 (16 rows) 3.50 -> 3.33 ms.  Experts of two or
// more tiles share their weight rows between tiles in L2, which non-temporal
// loads give up (87 rows per expert: 5.62 -> 7.25 ms).
static bool stream_weights(const FfnArgs& a) { return (long)a.T * a.k <= 32L * a.E; }

hipError_t launch_gateup_mfma(const FfnArgs& a, hipStream_t st, const KTime& kt) {
    if (a.bm == 256) return launch_gateup_dma(a, st, kt);
    if (a.bm != 64) return hipErrorInvalidValue;
    const int fmax = a.n_shared && a.Fs > a.F ? a.Fs : a.F;
    dim3 grid(a.max_tiles, (fmax + GU_BN - 1) / GU_BN);
    if (stream_weights(a)) launch_kernel(gateup_mfma_kernel<64, true>, grid, 256, st, kt, a);
    else launch_kernel(gateup_mfma_kernel<64, false>, grid, 256, st, kt, a);
    return hipGetLastError();
}

hipError_t launch_down_mfma(const FfnArgs& a, hipStream_t st, const KTime& kt) {
    if (a.bm == 256) return launch_down_dma(a, st, kt);
    if (a.bm != 64) return hipErrorInvalidValue;
    dim3 grid(a.max_tiles, (a.d + DN_BN - 1) / DN_BN);
    if (stream_weights(a)) launch_kernel(down_mfma_kernel<64, true>, grid, 256, st, kt, a);
    else launch_kernel(down_mfma_kernel<64, false>, grid, 256, st, kt, a);
    return hipGetLastError();
}

}  // namespace moe
