// grouped_gemm_q8.hip - the prefill grouped GEMMs for int8 expert weights
// (blocks of 32 along the reduction dimension, one fp16 scale per block) on
// the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16), fp32 accumulation.
//
//   gate/up:  H_e = bf16( silu(A_e Wg[e]^T) * (A_e Wu[e]^T) ),  A_e = rows of x
//   down:     slot_out[f, :] = w_f * (H_e Wd[e]^T)[row of f]
// with W[n, k] = scale[n, k / 32] * q[n, k]: the same operation as the bf16
// kernels of grouped_gemm.hip, whose tile list, work order and epilogues
// these kernels share.
//
// The pages: the batch path runs the experts as tiles over "dequantized
// gate/up" and down projections (NeutronStar README, "GLM-5.2 CUDA port" and
// the LUT bug note); decision tensors stay at Q8_0 ("The model").
//
// Exactness.  q (|q| <= 127) is exact in bf16, so the weight tile is staged
// into LDS as the integers q themselves and every MFMA product q * x is exact;
// the block scale is applied after the MFMAs: each 64-wide K chunk holds two
// blocks, each block's two 16-wide MFMA steps accumulate into fresh fp32
// registers, and every lane then adds scale[n, block] * partial into its
// accumulators.  (Rounding scale * q to bf16 instead would cost up to 2^-9
// relative per weight.)  In the 32 x 32 MFMA layout a lane holds one output
// column n, so it needs one scale per block, read from the chunk's scales
// staged in LDS beside the tile.
//
// Tiles: 64 rows x 64 gate + 64 up columns (gate/up) or x 128 output columns
// (down), K in double-buffered 64-wide chunks; the weight
// chunk is 64 bytes per row (four 16-byte pieces), read once per tile and
// widened to bf16 on its way into LDS.
#include "common.h"
#include "kernels.h"
#include "gemm_dev.h"

namespace moe {
namespace {

constexpr int BK = 64;
constexpr int ROWB = BK * 2;  // bytes per bf16 LDS tile row (128)

__device__ __forceinline__ int lds_off(int row, int ch) { return row * ROWB + ((ch ^ (row & 7)) << 4); }

__device__ __forceinline__ bf16x8_t lds_frag(const uint8_t* base, int row, int ch) {
    return *reinterpret_cast<const bf16x8_t*>(base + lds_off(row, ch));
}

// 16 int8 values -> two 16-byte pieces of bf16 (exact: |q| <= 127).
__device__ __forceinline__ void q8_to_bf16(u32x4 w, u32x4& lo, u32x4& hi) {
    uint32_t out[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int32_t v = (int32_t)w[j];
        const float f0 = (float)((v << 24) >> 24), f1 = (float)((v << 16) >> 24);
        const float f2 = (float)((v << 8) >> 24), f3 = (float)(v >> 24);
        out[2 * j] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
        out[2 * j + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
    }
    lo = u32x4{out[0], out[1], out[2], out[3]};
    hi = u32x4{out[4], out[5], out[6], out[7]};
}

__device__ __forceinline__ u32x4 ld16b(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// The K loop of both kernels.  Chunk c (BK wide) is computed from LDS buffer
// c & 1; meanwhile the loads of chunks c + 1 .. c + NR sit in a ring of NR
// register stages (the one of chunk c + 1 issued NR - 1 chunks ago).  After
// chunk c's MFMAs, stage (c + 1) % NR is widened into the other buffer and
// reloaded with chunk c + 1 + NR; one barrier per chunk then separates the
// reads of a buffer from its next fill.
#ifndef Q8_RING
#define Q8_RING 4
#endif
constexpr int NR = Q8_RING;

template <class St, class GL, class LS, class CP>
__device__ __forceinline__ void q8_k_loop(int nch, St (&R)[NR], GL gload, LS lstore, CP compute) {
#pragma unroll
    for (int i = 0; i < NR; ++i)
        if (i < nch) gload(R[i], i * BK);
    lstore(R[0], 0);
    if (NR < nch) gload(R[0], NR * BK);
    __syncthreads();
    for (int c0 = 0; c0 < nch; c0 += NR) {
#pragma unroll
        for (int q = 0; q < NR; ++q) {
            const int c = c0 + q;
            if (c < nch) {
                compute(q & 1);
                if (c + 1 < nch) lstore(R[(q + 1) % NR], (q + 1) & 1);
                if (c + 1 + NR < nch) gload(R[(q + 1) % NR], (c + 1 + NR) * BK);
                __syncthreads();
            }
        }
    }
}

// ---------------------------------------------------------------------------
// gate/up
// ---------------------------------------------------------------------------
constexpr int GU_BN = 64;  // columns of gate (and of up) per workgroup

template <int BM>
__global__ __launch_bounds__(256, 2) void gateup_mfma_q8_kernel(FfnArgs a) {
    constexpr int MT = BM / 64, AP = BM / 32;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + 2 * GU_BN) * ROWB];
    __shared__ float lsc[2][2 * GU_BN][2];  // per chunk: scale of (B row, block)
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
    const int K = a.d, KB = K / 32;
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
    const uint16_t* xbase = static_cast<const uint16_t*>(a.x);

    // A: AP 16-byte pieces of bf16 x per thread (rows r_lo + 32 p, piece ch);
    // B: one 16-byte piece of int8 per thread of gate and of up (row rb, piece cb);
    // scales: one per thread (B row tid / 2 of gate|up, block tid % 2).
    const int ch = tid & 7, r_lo = tid >> 3;
    const int cb = tid & 3, rb = tid >> 2;
    const int srow = tid >> 1, sblk = tid & 1;
    int arow[AP];
#pragma unroll
    for (int p = 0; p < AP; ++p) arow[p] = src_row[r_lo + 32 * p];
    const uint16_t* ap[AP];
#pragma unroll
    for (int p = 0; p < AP; ++p) ap[p] = xbase + (size_t)(arow[p] >= 0 ? arow[p] : 0) * K + ch * 8;
    const int brow = n0 + rb < F ? n0 + rb : n0;  // rows past F read a valid row (results not stored)
    const uint8_t* gp = static_cast<const uint8_t*>(G.q) + ((size_t)ge * F + brow) * K + cb * 16;
    const uint8_t* upp = static_cast<const uint8_t*>(U.q) + ((size_t)ge * F + brow) * K + cb * 16;
    const int s_n = n0 + (srow & (GU_BN - 1)) < F ? n0 + (srow & (GU_BN - 1)) : n0;
    const uint16_t* sp = (srow < GU_BN ? G.scale : U.scale) + ((size_t)ge * F + s_n) * KB + sblk;

    struct Stage {
        u32x4 a[AP], g, u;
        uint16_t s;
    };
    auto gload = [&](Stage& R, int k0) {
#pragma unroll
        for (int p = 0; p < AP; ++p) R.a[p] = ld16(ap[p] + k0);
        R.g = ld16b(gp + k0);
        R.u = ld16b(upp + k0);
        R.s = sp[k0 / 32];
    };
    auto lstore = [&](const Stage& R, int s) {
#pragma unroll
        for (int p = 0; p < AP; ++p) st16(&lds[s][lds_off(r_lo + 32 * p, ch)], R.a[p]);
        u32x4 lo, hi;
        q8_to_bf16(R.g, lo, hi);
        st16(&lds[s][lds_off(BM + rb, 2 * cb)], lo);
        st16(&lds[s][lds_off(BM + rb, 2 * cb + 1)], hi);
        q8_to_bf16(R.u, lo, hi);
        st16(&lds[s][lds_off(BM + GU_BN + rb, 2 * cb)], lo);
        st16(&lds[s][lds_off(BM + GU_BN + rb, 2 * cb + 1)], hi);
        lsc[s][srow][sblk] = f16_to_f32(R.s);
    };

    if (BM == 64 && tr.nrows <= 32) {
        // A tile of at most 32 rows: wavefront w computes every row for gate
        // columns 16w .. 16w + 15 and the same up columns, as one 32 x 32
        // block whose B rows are those 16 gate rows, then those 16 up rows
        // (lane l holds column l & 31 of the block: gate for l & 31 < 16),
        // so no wavefront computes an empty row block.
        const int r32 = lane & 31;
        const bool up = r32 >= 16;
        const int brow = (up ? GU_BN : 0) + 16 * wave + (r32 & 15);  // B row of this lane's column
        f32x16_t acc = f32x16_t{};
        auto compute1 = [&](int s, int blk) {
            const uint8_t* L = lds[s];
            bf16x8_t fb[2], fa[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int c = 2 * (2 * blk + j) + (lane >> 5);
                fb[j] = lds_frag(L, BM + brow, c);
                fa[j] = lds_frag(L, r32, c);
            }
            const float sc = lsc[s][brow][blk];
            f32x16_t p = f32x16_t{};
#pragma unroll
            for (int j = 0; j < 2; ++j) p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[j], fb[j], p, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[v] = fmaf(sc, p[v], acc[v]);
        };
        Stage R[NR];
        q8_k_loop(K / BK, R, gload, lstore, [&](int b) {
            compute1(b, 0);
            compute1(b, 1);
        });
        // lane l (l & 31 < 16) holds gate column 16w + (l & 15) of rows
        // 8*(v/4) + 4*(l/32) + v%4; lane l + 16 the same up column
        const int col = n0 + 16 * wave + (r32 & 15);
        uint16_t* h = static_cast<uint16_t*>(a.h);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float u = __shfl_xor(acc[v], 16);
            const int row = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (!up && col < F && row < tr.nrows)
                h[(size_t)(tr.rbeg + row) * a.ldh + col] = f32_to_bf16(silu_f32(acc[v]) * u);
        }
        return;
    }
    const int mh = wave & 1, nh = wave >> 1;
    f32x16_t accg[MT], accu[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        accg[i] = f32x16_t{};
        accu[i] = f32x16_t{};
    }
    // One int8 block (32 of K): two 16-wide MFMA steps into fresh registers,
    // then accumulate scale * partial.
    auto compute = [&](int s, int blk) {
        const uint8_t* L = lds[s];
        bf16x8_t fg[2], fu[2], fa[2][MT];
        auto frags = [&](int j) {
            const int c = 2 * (2 * blk + j) + (lane >> 5);
            fg[j] = lds_frag(L, BM + 32 * nh + (lane & 31), c);
            fu[j] = lds_frag(L, BM + GU_BN + 32 * nh + (lane & 31), c);
#pragma unroll
            for (int i = 0; i < MT; ++i) fa[j][i] = lds_frag(L, (BM / 2) * mh + 32 * i + (lane & 31), c);
        };
        frags(0);
        frags(1);
        const float sg = lsc[s][32 * nh + (lane & 31)][blk], su = lsc[s][GU_BN + 32 * nh + (lane & 31)][blk];
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            f32x16_t pg = f32x16_t{}, pu = f32x16_t{};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                pg = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[j][i], fg[j], pg, 0, 0, 0);
                pu = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[j][i], fu[j], pu, 0, 0, 0);
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                accg[i][v] = fmaf(sg, pg[v], accg[i][v]);
                accu[i][v] = fmaf(su, pu[v], accu[i][v]);
            }
        }
    };
    Stage R[NR];
    q8_k_loop(K / BK, R, gload, lstore, [&](int b) {
        compute(b, 0);
        compute(b, 1);
    });

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

template <int BM>
__global__ __launch_bounds__(256, 2) void down_mfma_q8_kernel(FfnArgs a) {
    constexpr int MT = BM / 64, AP = BM / 32;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + DN_BN) * ROWB];
    __shared__ float lsc[2][DN_BN][2];
    __shared__ int dst_row[BM];
    __shared__ float wrow[BM];
    int tile, ntile;
    if (!work_item<BM == 128 ? 4 : 16>(tile_count(a), tile, ntile)) return;
    TileRows tr;
    if (!tile_rows<BM>(a, tile, tr)) return;
    const bool shared = tr.g == a.E;
    const int K = shared ? a.Fs : a.F, KB = K / 32;
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
    const uint16_t* hbase = static_cast<const uint16_t*>(a.h);

    // A: AP pieces of bf16 h per thread; B: two 16-byte int8 pieces per thread
    // (rows rb and rb + 64, piece cb); scales: one per thread.
    const int ch = tid & 7, r_lo = tid >> 3;
    const int cb = tid & 3, rb = tid >> 2;
    const int srow = tid >> 1, sblk = tid & 1;
    bool aval[AP];
#pragma unroll
    for (int p = 0; p < AP; ++p) aval[p] = r_lo + 32 * p < tr.nrows;
    const uint16_t* ap[AP];
#pragma unroll
    for (int p = 0; p < AP; ++p) ap[p] = hbase + (size_t)(tr.rbeg + (aval[p] ? r_lo + 32 * p : 0)) * a.ldh + ch * 8;
    const uint8_t* bp[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int n = n0 + rb + 64 * p < N ? n0 + rb + 64 * p : n0;
        bp[p] = static_cast<const uint8_t*>(D.q) + ((size_t)ge * N + n) * K + cb * 16;
    }
    const int s_n = n0 + srow < N ? n0 + srow : n0;
    const uint16_t* sp = D.scale + ((size_t)ge * N + s_n) * KB + sblk;

    struct Stage {
        u32x4 a[AP], b[2];
        uint16_t s;
    };
    auto gload = [&](Stage& R, int k0) {
#pragma unroll
        for (int p = 0; p < AP; ++p) R.a[p] = ld16(ap[p] + k0);
#pragma unroll
        for (int p = 0; p < 2; ++p) R.b[p] = ld16b(bp[p] + k0);
        R.s = sp[k0 / 32];
    };
    auto lstore = [&](const Stage& R, int s) {
#pragma unroll
        for (int p = 0; p < AP; ++p) st16(&lds[s][lds_off(r_lo + 32 * p, ch)], R.a[p]);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            u32x4 lo, hi;
            q8_to_bf16(R.b[p], lo, hi);
            st16(&lds[s][lds_off(BM + rb + 64 * p, 2 * cb)], lo);
            st16(&lds[s][lds_off(BM + rb + 64 * p, 2 * cb + 1)], hi);
        }
        lsc[s][srow][sblk] = f16_to_f32(R.s);
    };

    float* out = shared ? a.shared_out : a.slot_out;
    if (BM == 64 && tr.nrows <= 32) {
        // A tile of at most 32 rows: wavefront w computes every row for
        // output columns 32w .. 32w + 31 (one 32 x 32 block), so no
        // wavefront computes an empty row block.
        const int r32 = lane & 31;
        f32x16_t acc = f32x16_t{};
        auto compute1 = [&](int s, int blk) {
            const uint8_t* L = lds[s];
            bf16x8_t fb[2], fa[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int c = 2 * (2 * blk + j) + (lane >> 5);
                fb[j] = lds_frag(L, BM + 32 * wave + r32, c);
                fa[j] = lds_frag(L, r32, c);
            }
            const float sc = lsc[s][32 * wave + r32][blk];
            f32x16_t p = f32x16_t{};
#pragma unroll
            for (int j = 0; j < 2; ++j) p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[j], fb[j], p, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[v] = fmaf(sc, p[v], acc[v]);
        };
        Stage R[NR];
        q8_k_loop(K / BK, R, gload, lstore, [&](int b) {
            compute1(b, 0);
            compute1(b, 1);
        });
        const int col = n0 + 32 * wave + r32;
        if (col < N) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row < tr.nrows && dst_row[row] >= 0) out[(size_t)dst_row[row] * N + col] = wrow[row] * acc[v];
            }
        }
        return;
    }
    const int mh = wave & 1, nh = wave >> 1;
    f32x16_t acc0[MT], acc1[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        acc0[i] = f32x16_t{};
        acc1[i] = f32x16_t{};
    }
    auto compute = [&](int s, int blk) {
        const uint8_t* L = lds[s];
        bf16x8_t f0[2], f1[2], fa[2][MT];
        auto frags = [&](int j) {
            const int c = 2 * (2 * blk + j) + (lane >> 5);
            f0[j] = lds_frag(L, BM + 64 * nh + (lane & 31), c);
            f1[j] = lds_frag(L, BM + 64 * nh + 32 + (lane & 31), c);
#pragma unroll
            for (int i = 0; i < MT; ++i) fa[j][i] = lds_frag(L, (BM / 2) * mh + 32 * i + (lane & 31), c);
        };
        frags(0);
        frags(1);
        const float s0 = lsc[s][64 * nh + (lane & 31)][blk], s1 = lsc[s][64 * nh + 32 + (lane & 31)][blk];
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            f32x16_t p0 = f32x16_t{}, p1 = f32x16_t{};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[j][i], f0[j], p0, 0, 0, 0);
                p1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[j][i], f1[j], p1, 0, 0, 0);
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                acc0[i][v] = fmaf(s0, p0[v], acc0[i][v]);
                acc1[i][v] = fmaf(s1, p1[v], acc1[i][v]);
            }
        }
    };
    Stage R[NR];
    q8_k_loop(K / BK, R, gload, lstore, [&](int b) {
        compute(b, 0);
        compute(b, 1);
    });

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

}  // namespace

// 64-row tiles (the tile rule gives int8 layers bm = 64; the 128-row
// variants of these kernels would need more than 256 VGPRs).  Layers whose
// experts average few rows take the LDS-copy kernels of
// grouped_gemm_q8_dma.hip instead (a 64-row tile there is two passes of 32
// rows, reading its weights twice): gate/up up to 28 rows per expert, down
// up to 20.  Measured at c2's shape (ms per launch, LDS-copy against these):
// gate/up 0.66 / 0.90 at 64 tokens, 1.08 / 1.28 at 1024 (24 rows), 1.50 /
// 1.38 at 1536 (36 rows); down 0.56 / 0.64 at 512 (12 rows), 0.61 / 0.65 at
// 768, 0.66 / 0.67 at 1024, 0.89 / 0.74 at 1536.
static bool dma_gateup(const FfnArgs& a) { return q8_dma_ok(a) && (long)a.T * a.k <= 28L * a.E; }
static bool dma_down(const FfnArgs& a) { return q8_dma_ok(a) && (long)a.T * a.k <= 20L * a.E; }

hipError_t launch_gateup_mfma_q8(const FfnArgs& a, hipStream_t st, const KTime& kt) {
    if (a.bm != 64) return hipErrorInvalidValue;
    if (dma_gateup(a)) return launch_gateup_q8_dma(a, st, kt);
    const int fmax = a.n_shared && a.Fs > a.F ? a.Fs : a.F;
    dim3 grid(a.max_tiles, (fmax + GU_BN - 1) / GU_BN);
    launch_kernel(gateup_mfma_q8_kernel<64>, grid, 256, st, kt, a);
    return hipGetLastError();
}

hipError_t launch_down_mfma_q8(const FfnArgs& a, hipStream_t st, const KTime& kt) {
    if (a.bm != 64) return hipErrorInvalidValue;
    if (dma_down(a)) return launch_down_q8_dma(a, st, kt);
    dim3 grid(a.max_tiles, (a.d + DN_BN - 1) / DN_BN);
    launch_kernel(down_mfma_q8_kernel<64>, grid, 256, st, kt, a);
    return hipGetLastError();
}

}  // namespace moe
