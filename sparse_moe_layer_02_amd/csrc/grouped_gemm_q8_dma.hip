// grouped_gemm_q8_dma.hip - the int8 grouped GEMMs for layers whose experts
// average few rows (a short prefill spreads its tokens over all experts: about
// a dozen rows each), weights copied straight from global memory into LDS.
//
//   gate/up:  H_e = bf16( silu(A_e Wg[e]^T) * (A_e Wu[e]^T) ),  A_e = rows of x
//   down:     slot_out[f, :] = w_f * (H_e Wd[e]^T)[row of f]
// with W[n, k] = scale[n, k / 32] * q[n, k] (blocks of 32 along K, one fp16
// scale each): the operation of grouped_gemm_q8.hip, on the same tile list.
//
// Why a second design.  The register-staged kernels widen every weight to
// bf16 through registers into LDS, one 64-wide K chunk per barrier, two
// workgroups per CU; on these tiles their matrix work is a sliver and that
// staging, not HBM, sets their pace.  Here the int8 rows go into LDS with the
// buffer-load-to-LDS path (no VGPRs, no LDS store instructions), eight
// 64-wide K stages deep, and each wavefront widens only the 8 bytes per lane
// its MFMA step reads.
//
// Pass: at most 32 rows (a 64-row tile of the list takes two) x 256 weight rows.  Gate/up: 128 gate columns and the
// same 128 up columns; wavefront w owns gate columns 16w .. 16w + 15 and the
// same up columns as one 32 x 32 MFMA block (B rows 32w .. 32w + 31: those
// 16 gate rows, then those 16 up rows).  Down: wavefront w owns output columns 32w .. 32w + 31.
// A (the tile's bf16 rows of x or h, 128 bytes per row and stage) is copied
// into LDS beside the weight rows by wavefronts 0-3, one 1 KB copy each, and
// read by all eight.
//
// Exactness as in grouped_gemm_q8.hip: q is exact in bf16, every MFMA
// product q * x is exact, each block's two K16 steps accumulate into fresh
// registers and the block's scale multiplies that partial sum.  In the
// 32 x 32 layout a lane holds one column (one weight row), so one scale per
// lane and block.
#include "common.h"
#include "dma_dev.h"
#include "gemm_dev.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int QWV = 8;                   // wavefronts per workgroup
constexpr int QSK = 64;                  // K per stage: 64 int8 = 64 bytes of each weight row
constexpr int QBN = 256;                 // weight rows per tile
constexpr int QXS = QBN * QSK;           // bytes of one stage's weight rows (16 KB)
constexpr int QNCB = QXS / (1024 * QWV); // 1 KB weight copies per wavefront per stage (2)
constexpr int QNCP = 2 * QNCB;           // ... per pair of stages (8 rows x 128 bytes each)
constexpr int QROWS = 32;                // rows of a tile these kernels take
constexpr int QAS = QROWS * QSK * 2;     // bytes of one stage's A rows (4 KB: 32 rows x 64 bf16)
constexpr int QAW = QAS / 1024;          // wavefronts that copy A rows (one 1 KB copy each)
static_assert(QNCB * 1024 * QWV == QXS && QAW <= QWV, "copy geometry");

// Eight int8 -> eight bf16 (exact: |q| <= 127).
__device__ __forceinline__ bf16x8_t widen8(uint32_t lo, uint32_t hi) {
    uint32_t out[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int32_t v = (int32_t)(j ? hi : lo);
        const float f0 = (float)((v << 24) >> 24), f1 = (float)((v << 16) >> 24);
        const float f2 = (float)((v << 8) >> 24), f3 = (float)(v >> 24);
        out[2 * j] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
        out[2 * j + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
    }
    bf16x8_t r;
    __builtin_memcpy(&r, out, 16);
    return r;
}

// Per-lane sources and LDS offsets of one tile.
struct QTile {
    const uint8_t* asrc;     // A bytes this copy lane fetches at K = 0 (wavefronts < QAW)
    int adst;                // wave-uniform offset of that copy in an A stage
    const uint8_t* src[QNCP];// weight-row bytes each copy lane fetches at K = 0
    int dst[QNCP];           // wave-uniform offset of each copy in its half of a pair
    const uint4* scp;        // the lane's weight row's block scales, eight (four stages) per 16 bytes
    int fo;                  // LDS offset of the lane's weight fragment (row, half h) in its half of a pair
    int fsw;                 // that row's chunk swizzle
    bool fhi;                // the lane's weight row lies in rows 128..255 of a pair
    int ao;                  // LDS offset of the lane's A row (lane & 31) in an A stage
    f32x16_t acc;
};

// A rows in LDS: 128 bytes (eight 16-byte chunks) per row; chunk c of row r
// sits at slot c ^ (r & 7), so the 32 rows a fragment read covers spread
// over the banks.  Copy lane l of A copy q fills row 8q + l / 8, slot l % 8.
__device__ __forceinline__ int a_copy_row(int q, int lane) { return 8 * q + (lane >> 3); }
__device__ __forceinline__ int a_copy_chunk(int lane) { return (lane & 7) ^ ((lane >> 3) & 7); }

// Weight rows of a pair of stages (K128: 128 bytes of each row, whole cache
// lines) in two arrays of 128 rows: a copy of 64 lanes x 16 bytes covers
// eight whole lines rather than sixteen half lines, which the copy path of a
// CU takes measurably faster (chunk swizzle: pair_swz).

// The K loop: nst = K / 64 stages (a multiple of 4) in eight slots; slot s
// holds the A rows (Y) of chunk c = s mod 8, slots 2m, 2m + 1 the weight rows
// of that pair of chunks (rows 0..127 in X[2m], 128..255 in X[2m + 1]).  The lane's
// block scales come 16 bytes (four chunks) per load: sc[0] serves slots 0-3
// and is reloaded at stage 4 for the next round, sc[1] serves slots 4-7 and
// is reloaded at stage 0 of its round; each load goes out after every use of
// the values it replaces.  Chunks are fetched in pairs (2m, 2m + 1).
// At an even stage j the pair (j, j + 1) has landed (the pairs of chunks
// j + 2 .. j + 5 may still be in flight) and every wavefront has finished
// reading slots j - 2 and j - 1, which then receive the pair (j + 6, j + 7).
// HASA: this wavefront copies A rows (one more vector-memory operation per
// chunk, so its wait counts differ); WNT: the weight copies are non-temporal.
template <bool HASA, bool WNT>
__device__ __forceinline__ void q8_k_loop_dma(QTile& g, int nst, uint8_t* const (&X)[8], uint8_t* const (&Y)[8]) {
    constexpr int NC = QNCB + (HASA ? 1 : 0);  // copies per chunk
    uint4 sc[2];
    const int last = nst - 1;
    auto kc = [&](int c) { return c < last ? c : last; };  // chunks past the end re-read the last (unused)
    auto issue_pair = [&](auto kk, int c) {
        constexpr int K = decltype(kk)::value;
        static_assert(K % 2 == 0, "pairs start at even slots");
        const int c0 = kc(c), c1 = kc(c + 1);
        if constexpr (HASA) {
            copy16(g.asrc + (size_t)c0 * 128, Y[K] + g.adst);
            copy16(g.asrc + (size_t)c1 * 128, Y[K + 1] + g.adst);
        }
        const size_t p0 = (size_t)(c0 & ~1) * QSK;  // the pair's 128 bytes of each weight row
#pragma unroll
        for (int q = 0; q < QNCP; ++q) {
            if constexpr (WNT) copy16_nt(g.src[q] + p0, (q < QNCP / 2 ? X[K] : X[K + 1]) + g.dst[q]);
            else copy16(g.src[q] + p0, (q < QNCP / 2 ? X[K] : X[K + 1]) + g.dst[q]);
        }
    };
    auto stage = [&](auto kk, int j) {
        constexpr int K = decltype(kk)::value;
        if constexpr (K % 2 == 0) {
            // the pair (j, j + 1) has landed, and at stages 0 and 4 also the
            // scale load before it: what may still be in flight is the two
            // later pairs, plus a scale load at stages 2 and 6
            wait_lgkm0();
            wait_vm<K % 4 == 0 ? 4 * NC : 4 * NC + 1>();
            barrier_nofence();
            if constexpr (K == 0) sc[1] = g.scp[kc(j + 4) >> 2];
            if constexpr (K == 4) sc[0] = g.scp[kc(j + 4) >> 2];
            issue_pair(ic<(K + 6) % 8>(), j + 6);
        }
        const uint8_t* S = g.fhi ? X[K | 1] : X[K & ~1];
        const uint8_t* A = Y[K];
        uint2 wq[4];
        bf16x8_t fa[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            wq[s] = *reinterpret_cast<const uint2*>(S + g.fo + (((4 * (K & 1) + s) ^ g.fsw) << 4));
            fa[s] = *reinterpret_cast<const bf16x8_t*>(A + g.ao + (((2 * s + (threadIdx.x >> 5 & 1)) ^ (threadIdx.x & 7)) << 4));
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            f32x16_t p = f32x16_t{};
#pragma unroll
            for (int s = 2 * b; s < 2 * b + 2; ++s)
                p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s], widen8(wq[s].x, wq[s].y), p, 0, 0, 0);
            const uint4 q4 = sc[K / 4];
            const uint32_t w2 = (K % 4 == 0) ? q4.x : (K % 4 == 1) ? q4.y : (K % 4 == 2) ? q4.z : q4.w;
            const float scv = f16_to_f32((uint16_t)(w2 >> (16 * b)));
#pragma unroll
            for (int v = 0; v < 16; ++v) g.acc[v] = fmaf(scv, p[v], g.acc[v]);
        }
    };
    sc[0] = g.scp[0];
    issue_pair(ic<0>(), 0);
    issue_pair(ic<2>(), 2);
    issue_pair(ic<4>(), 4);
    int j = 0;
    for (; j + 8 <= nst; j += 8) {
        stage(ic<0>(), j);
        stage(ic<1>(), j + 1);
        stage(ic<2>(), j + 2);
        stage(ic<3>(), j + 3);
        stage(ic<4>(), j + 4);
        stage(ic<5>(), j + 5);
        stage(ic<6>(), j + 6);
        stage(ic<7>(), j + 7);
    }
    if (j < nst) stage(ic<0>(), j);
    if (j + 1 < nst) stage(ic<1>(), j + 1);
    if (j + 2 < nst) stage(ic<2>(), j + 2);
    if (j + 3 < nst) stage(ic<3>(), j + 3);
    if (j + 4 < nst) stage(ic<4>(), j + 4);
    if (j + 5 < nst) stage(ic<5>(), j + 5);
    if (j + 6 < nst) stage(ic<6>(), j + 6);
    // no copy may still be writing LDS when the workgroup ends
    wait_vm<0>();
}

// Copy and fragment set-up shared by both kernels (the passes fill in the
// copy sources g.src, g.asrc and the scale row g.scp): br is the lane's
// fragment row (0..255) in a pair of stages.
__device__ __forceinline__ void q8_dma_setup(QTile& g, int wave, int lane, int br) {
#pragma unroll
    for (int q = 0; q < QNCP; ++q) g.dst[q] = (((q * QWV + wave) * 8) & 127) * 128;
    g.adst = (wave < QAW ? wave : 0) * 1024;
    g.fsw = pair_swz(br);
    g.fhi = br >= 128;
    g.fo = (br & 127) * 128 + 8 * (lane >> 5);
    g.ao = (lane & 31) * 128;
    g.acc = f32x16_t{};
}
// Weight copy q (8 rows x 128 bytes; copies 0 .. QNCP/2 - 1 fill rows 0..127
// of a pair): the stage row of this copy lane, and its byte offset in that
// row's 128 bytes.
__device__ __forceinline__ int q8_copy_row(int q, int wave, int lane) { return (q * QWV + wave) * 8 + (lane >> 3); }
__device__ __forceinline__ int q8_copy_byte(int sr, int lane) { return 16 * ((lane & 7) ^ pair_swz(sr)); }

// Eight weight stages of 16 KB and eight A stages of 4 KB: the whole 160 KB.
#define Q8_DMA_LDS                                                                 \
    __shared__ __attribute__((aligned(1024))) uint8_t X0[QXS];                     \
    __shared__ __attribute__((aligned(1024))) uint8_t X1[QXS];                     \
    __shared__ __attribute__((aligned(1024))) uint8_t X2[QXS];                     \
    __shared__ __attribute__((aligned(1024))) uint8_t X3[QXS];                     \
    __shared__ __attribute__((aligned(1024))) uint8_t X4[QXS];                     \
    __shared__ __attribute__((aligned(1024))) uint8_t X5[QXS];                     \
    __shared__ __attribute__((aligned(1024))) uint8_t X6[QXS];                     \
    __shared__ __attribute__((aligned(1024))) uint8_t X7[QXS];                     \
    __shared__ __attribute__((aligned(1024))) uint8_t Y0[QAS];                     \
    __shared__ __attribute__((aligned(1024))) uint8_t Y1[QAS];                     \
    __shared__ __attribute__((aligned(1024))) uint8_t Y2[QAS];                     \
    __shared__ __attribute__((aligned(1024))) uint8_t Y3[QAS];                     \
    __shared__ __attribute__((aligned(1024))) uint8_t Y4[QAS];                     \
    __shared__ __attribute__((aligned(1024))) uint8_t Y5[QAS];                     \
    __shared__ __attribute__((aligned(1024))) uint8_t Y6[QAS];                     \
    __shared__ __attribute__((aligned(1024))) uint8_t Y7[QAS];                     \
    uint8_t* const X[8] = {X0, X1, X2, X3, X4, X5, X6, X7};                        \
    uint8_t* const Y[8] = {Y0, Y1, Y2, Y3, Y4, Y5, Y6, Y7}

template <bool WNT>
__device__ __forceinline__ void q8_run(QTile& g, int nst, int wave, uint8_t* const (&X)[8], uint8_t* const (&Y)[8]) {
    if (wave < QAW) q8_k_loop_dma<true, WNT>(g, nst, X, Y);
    else q8_k_loop_dma<false, WNT>(g, nst, X, Y);
}

// One pass of a gate/up tile: rows [tr.rbeg, tr.rbeg + tr.nrows), at most 32.
template <bool WNT>
__device__ __forceinline__ void gateup_q8_dma_pass(const FfnArgs& a, const TileRows& tr, int F, int n0, int wave,
                                                   int lane, uint8_t* const (&X)[8], uint8_t* const (&Y)[8]) {
    const bool shared = tr.g == a.E;
    const int K = a.d, KB = K / 32;
    const int r32 = lane & 31;
    const uint8_t* gq = static_cast<const uint8_t*>(shared ? a.s_gate.q : a.gate.q);
    const uint8_t* uq = static_cast<const uint8_t*>(shared ? a.s_up.q : a.up.q);
    const uint16_t* gsc = shared ? a.s_gate.scale : a.gate.scale;
    const uint16_t* usc = shared ? a.s_up.scale : a.up.scale;
    const size_t e0 = (size_t)(shared ? 0 : tr.g) * F;
    QTile g;
    const int br = 32 * wave + r32;
    q8_dma_setup(g, wave, lane, br);
    // stage rows 32 m .. 32 m + 15: gate rows n0 + 16 m + (0..15), 32 m + 16 ..
    // 32 m + 31: the same up rows, so each wavefront's 32 fragment rows lie in
    // one half of a pair (rows past F read row n0)
#pragma unroll
    for (int q = 0; q < QNCP; ++q) {
        const int sr = q8_copy_row(q, wave, lane);
        const int n = n0 + 16 * (sr >> 5) + (sr & 15);
        const size_t row = e0 + (n < F ? n : n0);
        g.src[q] = ((sr & 31) < 16 ? gq : uq) + row * K + q8_copy_byte(sr, lane);
    }
    {
        const int n = n0 + 16 * wave + (r32 & 15);
        const size_t row = e0 + (n < F ? n : n0);
        g.scp = reinterpret_cast<const uint4*>((r32 < 16 ? gsc : usc) + row * KB);
    }
    {   // A row r: the token of tile row r (rows past the tile read token 0; their results are never stored)
        const int r = a_copy_row(wave < QAW ? wave : 0, lane);
        int t = 0;
        if (r < tr.nrows) {
            if (shared) {
                t = tr.rbeg - a.T * a.k + r;
            } else {
                const int f = a.perm_rows[tr.rbeg + r];
                t = (f >= 0 && f < a.T * a.k) ? f / a.k : 0;
            }
        }
        g.asrc = reinterpret_cast<const uint8_t*>(static_cast<const uint16_t*>(a.x) + (size_t)t * K) +
                 a_copy_chunk(lane) * 16;
    }
    q8_run<WNT>(g, K / QSK, wave, X, Y);

    // lane l (l & 31 < 16) holds gate column n0 + 16w + (l & 15) of rows
    // 8*(v/4) + 4*(l/32) + v%4; lane l ^ 16 the same up column
    const int col = n0 + 16 * wave + (r32 & 15);
    uint16_t* h = static_cast<uint16_t*>(a.h);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const float u = __shfl_xor(g.acc[v], 16);
        const int row = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (r32 < 16 && col < F && row < tr.nrows)
            h[(size_t)(tr.rbeg + row) * a.ldh + col] = f32_to_bf16(silu_f32(g.acc[v]) * u);
    }
}

// One pass of a down tile: rows [tr.rbeg, tr.rbeg + tr.nrows), at most 32.
__device__ __forceinline__ void down_q8_dma_pass(const FfnArgs& a, const TileRows& tr, int n0, int wave, int lane,
                                                 uint8_t* const (&X)[8], uint8_t* const (&Y)[8]) {
    const bool shared = tr.g == a.E;
    const int N = a.d;
    const int K = shared ? a.Fs : a.F, KB = K / 32;
    const int r32 = lane & 31;
    const uint8_t* dq = static_cast<const uint8_t*>(shared ? a.s_down.q : a.down.q);
    const uint16_t* dsc = shared ? a.s_down.scale : a.down.scale;
    const size_t e0 = (size_t)(shared ? 0 : tr.g) * N;
    QTile g;
    const int br = 32 * wave + r32;
    q8_dma_setup(g, wave, lane, br);
#pragma unroll
    for (int q = 0; q < QNCP; ++q) {  // stage row sr: output column n0 + sr (rows past N read row n0)
        const int sr = q8_copy_row(q, wave, lane);
        const size_t row = e0 + (n0 + sr < N ? n0 + sr : n0);
        g.src[q] = dq + row * K + q8_copy_byte(sr, lane);
    }
    g.scp = reinterpret_cast<const uint4*>(dsc + (e0 + (n0 + br < N ? n0 + br : n0)) * KB);
    {   // A row r (rows past the tile read row 0; never stored)
        const int r = a_copy_row(wave < QAW ? wave : 0, lane);
        g.asrc = reinterpret_cast<const uint8_t*>(static_cast<const uint16_t*>(a.h) +
                                                  (size_t)(tr.rbeg + (r < tr.nrows ? r : 0)) * a.ldh) +
                 a_copy_chunk(lane) * 16;
    }
    q8_run<false>(g, K / QSK, wave, X, Y);

    const int col = n0 + br;
    float* out = shared ? a.shared_out : a.slot_out;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int row = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row >= tr.nrows || col >= N) continue;
        int dst = -1;
        float w = 0.0f;
        if (shared) {
            dst = tr.rbeg - a.T * a.k + row;
            w = 1.0f;
        } else {
            const int f = a.perm_rows[tr.rbeg + row];
            if (f >= 0 && f < a.T * a.k) {
                dst = f;
                w = a.topk_w[f];
            }
        }
        if (dst >= 0) __builtin_nontemporal_store(w * g.acc[v], out + (size_t)dst * N + col);  // read once, by the combine
    }
}

// A 64-row tile of the list runs as passes of at most 32 rows (its weights
// are then read once per pass); the barrier between passes keeps the next
// pass's copies out of stages other wavefronts may still be reading.
__global__ __launch_bounds__(64 * QWV, 1) void gateup_q8_dma_kernel(FfnArgs a) {
    Q8_DMA_LDS;
    int tile, ntile;
    if (!work_item<16>(tile_count(a), tile, ntile)) return;
    TileRows t64;
    if (!tile_rows<64>(a, tile, t64)) return;
    const int F = t64.g == a.E ? a.Fs : a.F;
    const int n0 = ntile * (QBN / 2);
    if (n0 >= F) return;
    const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int erows = t64.g == a.E ? a.T : a.offsets[t64.g + 1] - a.offsets[t64.g];
    // an expert of at most 32 rows is one pass of one tile: no other pass or
    // tile reads its weight rows, which are then copied non-temporal (c2p
    // gate/up 1.00 -> 0.96 ms)
    if (erows <= QROWS) {
        gateup_q8_dma_pass<true>(a, t64, F, n0, wave, lane, X, Y);
        return;
    }
    for (int p = 0; p * QROWS < t64.nrows; ++p) {
        if (p) __syncthreads();
        const TileRows tr{t64.g, t64.rbeg + p * QROWS, min(QROWS, t64.nrows - p * QROWS)};
        gateup_q8_dma_pass<false>(a, tr, F, n0, wave, lane, X, Y);
    }
}

__global__ __launch_bounds__(64 * QWV, 1) void down_q8_dma_kernel(FfnArgs a) {
    Q8_DMA_LDS;
    int tile, ntile;
    if (!work_item<16>(tile_count(a), tile, ntile)) return;
    TileRows t64;
    if (!tile_rows<64>(a, tile, t64)) return;
    const int n0 = ntile * QBN;
    const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    for (int p = 0; p * QROWS < t64.nrows; ++p) {
        if (p) __syncthreads();
        const TileRows tr{t64.g, t64.rbeg + p * QROWS, min(QROWS, t64.nrows - p * QROWS)};
        down_q8_dma_pass(a, tr, n0, wave, lane, X, Y);
    }
}

}  // namespace

// The kernels apply when both products' K is a whole number of four-stage
// scale loads (K % 256 == 0: every weight row's scales then start on a
// 16-byte boundary, the scale arrays being 16-byte aligned).
bool q8_dma_ok(const FfnArgs& a) {
    const bool ks = a.d % 256 == 0 && a.F % 256 == 0 && (!a.n_shared || a.Fs % 256 == 0);
    return a.bm == 64 && ks;
}

hipError_t launch_gateup_q8_dma(const FfnArgs& a, hipStream_t st, const KTime& kt) {
    if (!q8_dma_ok(a)) return hipErrorInvalidValue;
    const int fmax = a.n_shared && a.Fs > a.F ? a.Fs : a.F;
    dim3 grid(a.max_tiles, (fmax + QBN / 2 - 1) / (QBN / 2));
    launch_kernel(gateup_q8_dma_kernel, grid, 64 * QWV, st, kt, a);
    return hipGetLastError();
}

hipError_t launch_down_q8_dma(const FfnArgs& a, hipStream_t st, const KTime& kt) {
    if (!q8_dma_ok(a)) return hipErrorInvalidValue;
    dim3 grid(a.max_tiles, (a.d + QBN - 1) / QBN);
    launch_kernel(down_q8_dma_kernel, grid, 64 * QWV, st, kt, a);
    return hipGetLastError();
}

}  // namespace moe
