// grouped_gemm_dma.hip - the prefill grouped GEMMs for experts with many rows:
// one workgroup per CU, each wavefront a 64- or 128-row by 128-column block of
// v_mfma_f32_32x32x16_bf16 accumulators, operands fed straight from global
// memory into LDS.
//
//   gate/up:  H_e = bf16( silu(A_e Wg[e]^T) * (A_e Wu[e]^T) ),  A_e = rows of x
//             gathered through the permutation
//   down:     slot_out[f, :] = w_f * (H_e Wd[e]^T)[row of f]   (weighted scatter)
// (the same operation as grouped_gemm.hip; the shared expert is group E).
//
// Why a second design.  With 64x64 wavefront blocks every 32x32x16 MFMA needs
// one 16-byte LDS read per lane, and with operands staged through registers
// every tile byte is also written to LDS by the shader: the CU needs about 1.5x
// the LDS bandwidth its matrix cores can use.  Here a wavefront holds 128
// (or 64) rows x 128 columns, so four MFMAs share each fragment read by half,
// and the global->LDS copy is the buffer-load-to-LDS path (16 bytes per lane,
// written at M0 + 16 * lane), which costs no VGPRs and no LDS write
// instructions.
//
// Pipeline.  K advances in stages of 32.  Four stages live in four separate
// LDS arrays (separate objects, so the compiler can tell that reading one
// stage does not wait for the copies into the others).  Chunk j + 4 is copied
// into the stage of chunk j as soon as every wavefront has finished reading
// it, so each copy has three stages of MFMA work to land.  Inside a stage the
// two K16 steps alternate: while the MFMAs of one step run, the fragments of
// the next step are read; the copies of the next chunk and the first
// fragments of the next stage are issued between the MFMAs of the second step
// (instruction order pinned with scheduling barriers, since one wavefront per
// SIMD has no other wavefront to hide latency behind).
//
// LDS layout of a stage: rows of 64 bytes (32 bf16 of K), A rows first, then
// 256 B rows.  The four 16-byte chunks of row r sit at slot c ^ f(r),
// f(r) = ((r >> 1) & 3) ^ ((r >> 3) & 1): the sixteen lanes that a 128-bit LDS
// read serves per cycle (sixteen consecutive rows, one chunk) hit sixteen
// different 16-byte bank groups (measured: no bank-conflict cycles).
#include "common.h"
#include "kernels.h"
#include "gemm_dev.h"

namespace moe {
namespace {

constexpr int SK = 32;        // K per stage
constexpr int SROW = SK * 2;  // LDS bytes per row of a stage
constexpr int SBN = 256;      // B rows per tile

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediates (vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8);
// a field at its maximum does not wait.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// Workgroup barrier without a memory fence (a fence would wait for every copy
// in flight); the empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void barrier_nofence() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

__device__ __forceinline__ void pin() { __builtin_amdgcn_sched_barrier(0); }

// N items spread evenly over MFMAs [A, B) of a K16 step: the items issued with
// MFMA t are [spread(t), spread(t + 1)).
template <int N, int A, int B>
__device__ constexpr int spread(int t) {
    return t <= A ? 0 : t >= B ? N : ((t - A) * N + (B - A) - 1) / (B - A);
}

// 16 bytes per lane from global memory into LDS at dst + 16 * lane (dst
// wave-uniform).
__device__ __forceinline__ void copy16(const uint8_t* src, uint8_t* dst) {
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void*)(dst), 16, 0, 0);
}

// Tile geometry: BM rows x 256 B rows, WV wavefronts in an MW x (WV / MW)
// grid, each owning MI x NI blocks of 32 x 32.
template <int BM_, int MW, int WV>
struct Geo {
    static constexpr int BM = BM_, NW = WV / MW;
    static constexpr int MI = BM / (32 * MW);      // 32-row blocks per wavefront
    static constexpr int NI = SBN / (32 * NW);    // 32-column blocks per wavefront
    static constexpr int ROWS = BM + SBN;         // LDS rows per stage
    static constexpr int STAGE = ROWS * SROW;     // bytes per stage
    static constexpr int NCP = ROWS / (16 * WV);  // copies per wavefront per stage (16 rows each)
    static constexpr int NCA = BM / (16 * WV);    // ... of which A rows
    static constexpr int NF = MI + NI;            // fragments per K16 step
    static constexpr int NM = MI * NI;            // MFMAs per K16 step
    static_assert(MI >= 1 && NI >= 1 && NCA >= 1 && NCP * 16 * WV == ROWS && NCA * 16 * WV == BM, "geometry");
};

// One tile's operand sources (copy lane addresses, fragment offsets) and its
// accumulators.
template <class GEO>
struct Gemm {
    static constexpr int MI = GEO::MI, NI = GEO::NI, NCP = GEO::NCP, NF = GEO::NF;
    const uint8_t* src[NCP];  // per-lane source of each copy at K = 0
    int dst[NCP];             // wave-uniform LDS byte offset of each copy in a stage
    int fo[NF];               // per-lane LDS byte offset of each fragment (K16 step 0)
    f32x16_t acc[MI][NI];

    __device__ __forceinline__ void copy(uint8_t* S, int ci, size_t kb) const { copy16(src[ci] + kb, S + dst[ci]); }
    // step 1 reads logical chunk c + 2 of the same row: slot ^ 2
    __device__ __forceinline__ bf16x8_t frag(const uint8_t* S, int fi, int ks) const {
        return *reinterpret_cast<const bf16x8_t*>(S + (ks ? (fo[fi] ^ 32) : fo[fi]));
    }
    // MFMA t of a K16 step: block (i, j) = (t / NI, t % NI); fragments are
    // ordered A0, B0..B(NI-1), A1.. so that the first MFMAs wait least.
    static __device__ __forceinline__ int fa_idx(int i) { return i == 0 ? 0 : NI + i; }
    static __device__ __forceinline__ int fb_idx(int j) { return 1 + j; }
    __device__ __forceinline__ void mfma(const bf16x8_t (&f)[NF], int t) {
        const int i = t / NI, j = t % NI;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[fa_idx(i)], f[fb_idx(j)], acc[i][j], 0, 0, 0);
    }
};

// The K loop shared by both kernels.  nst = K / 32 stages; chunk c of the
// operands is at byte offset c * 64 of every row.
template <class GEO>
__device__ __forceinline__ void k_loop(Gemm<GEO>& g, int nst, uint8_t* L0, uint8_t* L1, uint8_t* L2,
                                       uint8_t* L3) {
    constexpr int NCP = GEO::NCP, NF = GEO::NF, NM = GEO::NM;
    bf16x8_t P[NF], Q[NF];
    const int last = nst - 1;
    auto kb = [&](int c) { return (size_t)(c < last ? c : last) * SROW; };
    // Fragment reads go with the first three quarters of a step's MFMAs, so
    // they have landed when the step ends; the copies go with the last three
    // quarters.
    constexpr int RD = (NM * 3 + 3) / 4, CP = NM / 4;

    // one stage: S holds chunk j, N is the stage of chunk j + 1
    auto stage = [&](uint8_t* S, uint8_t* N, int j) {
        // step 0 MFMAs (fragments P) with step 1's fragment reads (Q)
#pragma unroll
        for (int t = 0; t < NM; ++t) {
            g.mfma(P, t);
#pragma unroll
            for (int q = spread<NF, 0, RD>(t); q < spread<NF, 0, RD>(t + 1); ++q) Q[q] = g.frag(S, q, 1);
            pin();
        }
        // every read of S done, chunk j + 1 landed (two later chunks may be in flight)
        wait_lgkm0();
        wait_vm<2 * NCP>();
        barrier_nofence();
        // step 1 MFMAs (Q) with the copy of chunk j + 4 into S and the first
        // fragment reads of the next stage (P)
        const size_t k4 = kb(j + 4);
#pragma unroll
        for (int t = 0; t < NM; ++t) {
            g.mfma(Q, t);
#pragma unroll
            for (int q = spread<NF, 0, RD>(t); q < spread<NF, 0, RD>(t + 1); ++q) P[q] = g.frag(N, q, 0);
#pragma unroll
            for (int q = spread<NCP, CP, NM>(t); q < spread<NCP, CP, NM>(t + 1); ++q) g.copy(S, q, k4);
            pin();
        }
    };

    // prologue: chunks 0..3 into stages 0..3, wait for chunk 0
#pragma unroll
    for (int q = 0; q < NCP; ++q) g.copy(L0, q, kb(0));
#pragma unroll
    for (int q = 0; q < NCP; ++q) g.copy(L1, q, kb(1));
#pragma unroll
    for (int q = 0; q < NCP; ++q) g.copy(L2, q, kb(2));
#pragma unroll
    for (int q = 0; q < NCP; ++q) g.copy(L3, q, kb(3));
    wait_vm<3 * NCP>();
    barrier_nofence();
#pragma unroll
    for (int q = 0; q < NF; ++q) P[q] = g.frag(L0, q, 0);

    int j = 0;
    for (; j + 4 <= nst; j += 4) {
        stage(L0, L1, j);
        stage(L1, L2, j + 1);
        stage(L2, L3, j + 2);
        stage(L3, L0, j + 3);
    }
    if (j < nst) stage(L0, L1, j);
    if (j + 1 < nst) stage(L1, L2, j + 1);
    if (j + 2 < nst) stage(L2, L3, j + 2);
    // no copy may still be writing LDS when the workgroup ends
    wait_vm<0>();
}

// Copy lanes: lane l of copy q of wavefront w fills stage row
// r = (q * WV + w) * 16 + l / 4, slot l & 3, which holds logical chunk
// (l & 3) ^ f(r); f(r) = ((l >> 3) & 3) ^ ((l >> 5) & 1) since r = l / 4 mod 16.
__device__ __forceinline__ int copy_row(int q, int wv, int wave, int lane) { return (q * wv + wave) * 16 + (lane >> 2); }
__device__ __forceinline__ int copy_col(int lane) { return ((lane & 3) ^ ((lane >> 3) & 3) ^ ((lane >> 5) & 1)) * 8; }

// Per-lane fragment offsets: wavefront (mh, nh) reads A rows
// mh * MI * 32 + 32 i + (lane & 31) and B rows brow[j] + (lane & 31).
template <class GEO>
__device__ __forceinline__ void frag_offsets(Gemm<GEO>& g, int mh, const int (&brow)[GEO::NI], int lane) {
    using G = Gemm<GEO>;
    const int r = lane & 31;
    const int slot0 = (lane >> 5) ^ ((lane >> 1) & 3) ^ ((lane >> 3) & 1);  // chunk lane / 32 of row lane & 31
    const int base = r * SROW + slot0 * 16;
#pragma unroll
    for (int i = 0; i < GEO::MI; ++i) g.fo[G::fa_idx(i)] = (mh * GEO::MI * 32 + 32 * i) * SROW + base;
#pragma unroll
    for (int j = 0; j < GEO::NI; ++j) g.fo[G::fb_idx(j)] = (GEO::BM + brow[j]) * SROW + base;
}

}  // namespace

// ---------------------------------------------------------------------------
// gate/up: BM rows x (128 gate + 128 up) columns per workgroup
// ---------------------------------------------------------------------------
template <int BM, int MW, int WV>
__global__ __launch_bounds__(64 * WV, 1) void gateup_dma_kernel(FfnArgs a) {
    using GEO = Geo<BM, MW, WV>;
    using G = Gemm<GEO>;
    constexpr int MI = GEO::MI, NI = GEO::NI, NW = GEO::NW;
    __shared__ __attribute__((aligned(1024))) uint8_t L0[GEO::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t L1[GEO::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t L2[GEO::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t L3[GEO::STAGE];
    __shared__ int src_row[BM];
    int tile, ntile;
    if (!work_item<4>(tile_count(a), tile, ntile)) return;
    TileRows tr;
    if (!tile_rows<BM>(a, tile, tr)) return;
    const bool shared = tr.g == a.E;
    const int F = shared ? a.Fs : a.F;
    const int n0 = ntile * (SBN / 2);
    if (n0 >= F) return;
    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = a.d;
    for (int r = tid; r < BM; r += 64 * WV) {
        int t = -1;
        if (r < tr.nrows) {
            if (shared) {
                t = tr.rbeg - a.T * a.k + r;
            } else {
                const int f = a.perm_rows[tr.rbeg + r];
                t = (f >= 0 && f < a.T * a.k) ? f / a.k : -1;
            }
        }
        src_row[r] = t;
    }
    __syncthreads();

    G g;
    const int cch = copy_col(lane);
    const MatRef& Wg = shared ? a.s_gate : a.gate;
    const MatRef& Wu = shared ? a.s_up : a.up;
    const int ge = shared ? 0 : tr.g;
    const uint16_t* gbase = static_cast<const uint16_t*>(Wg.q) + ((size_t)ge * F + n0) * K;
    const uint16_t* ubase = static_cast<const uint16_t*>(Wu.q) + ((size_t)ge * F + n0) * K;
    const uint16_t* xbase = static_cast<const uint16_t*>(a.x);
#pragma unroll
    for (int q = 0; q < GEO::NCP; ++q) {
        g.dst[q] = (q * WV + wave) * 1024;
        const int row = copy_row(q, WV, wave, lane);
        if (q < GEO::NCA) {
            // rows past the tile read token 0; their results are never stored
            const int t = src_row[row];
            g.src[q] = reinterpret_cast<const uint8_t*>(xbase + (size_t)(t >= 0 ? t : 0) * K + cch);
        } else {
            const int br = row - BM;  // 0..255: gate rows, then up rows
            const int n = br & 127;
            const int rr = n0 + n < F ? n : 0;  // columns past F read row 0 and are never stored
            const uint16_t* b = br < 128 ? gbase : ubase;
            g.src[q] = reinterpret_cast<const uint8_t*>(b + (size_t)rr * K + cch);
        }
    }
    // wavefront (mh, nh): gate columns nh * 128/NW + 32 j' and the same up
    // columns (blocks j < NI/2 are gate, j >= NI/2 up)
    const int mh = wave % MW, nh = wave / MW;
    int brow[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) brow[j] = (j < NI / 2 ? 0 : 128) + nh * (128 / NW) + 32 * (j % (NI / 2));
    frag_offsets<GEO>(g, mh, brow, lane);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) g.acc[i][j] = f32x16_t{};

    k_loop(g, K / SK, L0, L1, L2, L3);

    // epilogue: lane holds column (lane & 31) and rows 8*(v/4) + 4*(lane/32) + v%4 of each block
    uint16_t* h = static_cast<uint16_t*>(a.h);
#pragma unroll
    for (int j = 0; j < NI / 2; ++j) {
        const int col = n0 + brow[j] + (lane & 31);
        if (col >= F) continue;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = mh * MI * 32 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row < tr.nrows) {
                    const float gv = g.acc[i][j][v], uv = g.acc[i][j + NI / 2][v];
                    h[(size_t)(tr.rbeg + row) * a.ldh + col] = f32_to_bf16(gv / (1.0f + expf(-gv)) * uv);
                }
            }
    }
}

// ---------------------------------------------------------------------------
// down + weighted scatter: BM rows x 256 output columns per workgroup
// ---------------------------------------------------------------------------
template <int BM, int MW, int WV>
__global__ __launch_bounds__(64 * WV, 1) void down_dma_kernel(FfnArgs a) {
    using GEO = Geo<BM, MW, WV>;
    using G = Gemm<GEO>;
    constexpr int MI = GEO::MI, NI = GEO::NI, NW = GEO::NW;
    __shared__ __attribute__((aligned(1024))) uint8_t L0[GEO::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t L1[GEO::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t L2[GEO::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t L3[GEO::STAGE];
    __shared__ int dst_row[BM];
    __shared__ float wrow[BM];
    int tile, ntile;
    if (!work_item<4>(tile_count(a), tile, ntile)) return;
    TileRows tr;
    if (!tile_rows<BM>(a, tile, tr)) return;
    const bool shared = tr.g == a.E;
    const int K = shared ? a.Fs : a.F;
    const int N = a.d;
    const int n0 = ntile * SBN;
    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int r = tid; r < BM; r += 64 * WV) {
        int dst = -1;
        float w = 0.0f;
        if (r < tr.nrows) {
            if (shared) {
                dst = tr.rbeg - a.T * a.k + r;
                w = 1.0f;
            } else {
                const int f = a.perm_rows[tr.rbeg + r];
                if (f >= 0 && f < a.T * a.k) {
                    dst = f;
                    w = a.topk_w[f];
                }
            }
        }
        dst_row[r] = dst;
        wrow[r] = w;
    }
    __syncthreads();

    G g;
    const int cch = copy_col(lane);
    const MatRef& D = shared ? a.s_down : a.down;
    const int ge = shared ? 0 : tr.g;
    const uint16_t* dbase = static_cast<const uint16_t*>(D.q) + ((size_t)ge * N + n0) * K;
    const uint16_t* hbase = static_cast<const uint16_t*>(a.h) + (size_t)tr.rbeg * a.ldh;
#pragma unroll
    for (int q = 0; q < GEO::NCP; ++q) {
        g.dst[q] = (q * WV + wave) * 1024;
        const int row = copy_row(q, WV, wave, lane);
        if (q < GEO::NCA) {
            const int rr = row < tr.nrows ? row : 0;  // rows past the tile: never stored
            g.src[q] = reinterpret_cast<const uint8_t*>(hbase + (size_t)rr * a.ldh + cch);
        } else {
            const int br = row - BM;
            const int rr = n0 + br < N ? br : 0;
            g.src[q] = reinterpret_cast<const uint8_t*>(dbase + (size_t)rr * K + cch);
        }
    }
    const int mh = wave % MW, nh = wave / MW;
    int brow[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) brow[j] = nh * (SBN / NW) + 32 * j;
    frag_offsets<GEO>(g, mh, brow, lane);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) g.acc[i][j] = f32x16_t{};

    k_loop(g, K / SK, L0, L1, L2, L3);

    float* out = shared ? a.shared_out : a.slot_out;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int row = mh * MI * 32 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (row < tr.nrows && dst_row[row] >= 0) {
                const size_t base = (size_t)dst_row[row] * N;
                const float w = wrow[row];
#pragma unroll
                for (int j = 0; j < NI; ++j) {
                    const int col = n0 + brow[j] + (lane & 31);
                    if (col < N) out[base + col] = w * g.acc[i][j][v];
                }
            }
        }
}

// wavefront grid of the kernels launched: DMA_MW x (DMA_WV / DMA_MW)
constexpr int DMA_MW = 2, DMA_WV = 8;

hipError_t launch_gateup_dma(const FfnArgs& a, hipStream_t st, const KTime& kt) {
    const int fmax = a.n_shared && a.Fs > a.F ? a.Fs : a.F;
    dim3 grid(a.max_tiles, (fmax + SBN / 2 - 1) / (SBN / 2));
    if (a.bm == 256) launch_kernel(gateup_dma_kernel<256, DMA_MW, DMA_WV>, grid, 64 * DMA_WV, st, kt, a);
    else launch_kernel(gateup_dma_kernel<128, DMA_MW, DMA_WV>, grid, 64 * DMA_WV, st, kt, a);
    return hipGetLastError();
}

hipError_t launch_down_dma(const FfnArgs& a, hipStream_t st, const KTime& kt) {
    dim3 grid(a.max_tiles, (a.d + SBN - 1) / SBN);
    if (a.bm == 256) launch_kernel(down_dma_kernel<256, DMA_MW, DMA_WV>, grid, 64 * DMA_WV, st, kt, a);
    else launch_kernel(down_dma_kernel<128, DMA_MW, DMA_WV>, grid, 64 * DMA_WV, st, kt, a);
    return hipGetLastError();
}

}  // namespace moe
