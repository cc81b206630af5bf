// grouped_gemm_dma.hip - the prefill grouped GEMMs for layers whose experts
// average 96 rows or more (a long or skewed prefill: hot experts with
// hundreds of rows beside cold ones with a few): one workgroup per CU, each
// wavefront a 64- or 128-row by 128-column block of v_mfma_f32_32x32x16_bf16
// accumulators, operands fed straight from global memory into LDS.
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
// Pipeline.  K advances in stages of 32, the operands in pairs of stages
// (K64: 128-byte rows, so each copy instruction covers eight whole cache
// lines) through separate LDS arrays (separate objects, so the compiler can
// tell that reading one pair does not wait for the copies into the others):
// three A pair arrays, each A pair copied three stages before it is read, and
// two B (weight) pair arrays, two stages ahead (see k_loop).  Inside a stage the
// two K16 steps alternate: while the MFMAs of one step run, the fragments of
// the next step are read; the copies of the next chunk and the first
// fragments of the next stage are issued between the MFMAs of the second step
// (instruction order pinned with scheduling barriers, since one wavefront per
// SIMD has no other wavefront to hide latency behind).
//
// Short tiles.  A tile computes only its 32-row blocks that hold rows (an
// expert's last tile, or an expert with few rows): row blocks are dealt to the
// two wavefront rows in turn, so every SIMD keeps the same share of the
// remaining MFMAs, and A-row copies that reach no row are not issued.  Each
// wavefront runs the K loop instantiated for its number of live blocks
// (0 .. MI) and the workgroup's number of live A copies, so the copy counts
// the waits rely on stay compile-time constants.  A tile with one live block
// costs about its weight stream (3.1 MB at d = 6144) instead of a full
// 256-row product.
//
// LDS layout of a pair: rows of 128 bytes (64 bf16 of K).  The eight 16-byte
// chunks of row r sit at slot c ^ g(r), g(r) = (r >> 1) & 7: the sixteen
// lanes that a 128-bit LDS read serves per cycle (sixteen consecutive rows,
// one chunk) hit sixteen different 16-byte bank groups.
#include "common.h"
#include "dma_dev.h"
#include "gemm_dev.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int SK = 32;        // K per stage
constexpr int SROW = SK * 2;  // LDS bytes per row of a stage
constexpr int SBN = 256;      // B rows per tile
constexpr int XS = SBN * SROW;  // bytes of one LDS array (16 KB): half of a B pair, or two quarters of an A pair

// N items spread evenly over MFMAs [A, B) of a K16 step: the items issued with
// MFMA t are [spread(t), spread(t + 1)).
template <int N, int A, int B>
__device__ constexpr int spread(int t) {
    return t <= A ? 0 : t >= B ? N : ((t - A) * N + (B - A) - 1) / (B > A ? B - A : 1);
}

// Tile geometry: BM rows x 256 B rows, WV wavefronts in an MW x (WV / MW)
// grid, each owning MI x NI blocks of 32 x 32.  Row blocks are dealt to the
// MW wavefront rows in turn (wavefront row mh owns blocks mh, mh + MW, ...),
// so a tile with few rows leaves every SIMD the same share of matrix work.
template <int BM_, int MW, int WV>
struct Geo {
    static constexpr int BM = BM_, NW = WV / MW, NWV = WV;
    static constexpr int MI = BM / (32 * MW);      // 32-row blocks per wavefront
    static constexpr int NI = SBN / (32 * NW);    // 32-column blocks per wavefront
    static constexpr int NCA8 = BM / (8 * WV);    // A copies per wavefront per pair of stages (8 rows x 128 bytes)
    static_assert(MI >= 1 && NI >= 1 && NCA8 >= 1 && NCA8 * 8 * WV == BM, "geometry");
};

// First row of row block i of wavefront row mh.
template <int MW>
__device__ __forceinline__ int block_row(int i, int mh) { return 32 * (MW * i + mh); }

// Rows of a pair of K32 stages (K64): 128 bytes, so a copy of 64 lanes x 16
// bytes covers eight whole 128-byte lines (eight rows) rather than sixteen
// half lines: the copy path of a CU costs per instruction and per line, and
// whole lines take it measurably less (chunk swizzle: pair_swz).
constexpr int PROW = 2 * SROW;  // LDS bytes per row of a pair

// One tile's operand sources (copy lane addresses, fragment offsets) and its
// accumulators, for a wavefront that computes AI of its MI row blocks (the
// blocks that hold rows of the tile; AI = 0: copies only) and issues NCAA of
// the NCA8 A-row copies of a pair of stages (those that reach rows of the
// tile) and NCB B-row copies per pair.  A and B rows both travel in pairs of
// K32 stages (K64: 128-byte rows, eight whole lines per copy).  An A pair
// array is four quarters of 64 rows (copy q fills quarter q; row block i,
// rows 32 (2 i + mh), lies in quarter i), a B pair array two halves of 128
// rows (block j < NI / 2 in the first).  BNT: the weight (B) copies are
// non-temporal.
template <class GEO, int AI, int NCAA, bool BNT>
struct Gemm {
    static constexpr int NI = GEO::NI, NCA_ = NCAA;
    static constexpr int NCB = SBN / 8 / GEO::NWV;    // B copies per wavefront per pair (eight rows each)
    static_assert(NCB * 8 * GEO::NWV == SBN && NCB % 2 == 0, "B copies fill both halves of a pair");
    static_assert(NI == 2 && GEO::NW == 4 && GEO::MI == 4, "pair layout: two B blocks, four A quarters");
    static_assert(GEO::NCA8 == 4, "one A copy per quarter and wavefront");
    static constexpr int NCPA = NCAA + NCB;           // A copies, then B copies (per pair of stages)
    static constexpr int NF = AI > 0 ? AI + NI : 0;   // fragments per K16 step
    static constexpr int NM = AI * NI;                // MFMAs per K16 step
    static constexpr int AIS = AI > 0 ? AI : 1, NFS = NF > 0 ? NF : 1;
    const uint8_t* src[NCPA];  // per-lane source of each copy at K = 0
    int dst[NCPA];             // wave-uniform LDS byte offset (in its quarter / half of a pair)
    int fo[NFS];               // per-lane LDS byte offset of each fragment (first K16 step of a pair)
    f32x16_t acc[AIS][NI];

    // A copy ci (< NCAA) of the pair at byte offset pb into quarter ci
    __device__ __forceinline__ void copy_a(uint8_t* const (&AQ)[4], int ci, size_t pb) const {
        copy16(src[ci] + pb, AQ[ci] + dst[ci]);
    }
    // B copy ci (>= NCAA): the first NCB / 2 fill rows 0..127 (Blo), the rest rows 128..255
    __device__ __forceinline__ void copy_b(uint8_t* Blo, uint8_t* Bhi, int ci, size_t pb) const {
        if constexpr (BNT) copy16_nt(src[ci] + pb, (ci - NCAA < NCB / 2 ? Blo : Bhi) + dst[ci]);
        else copy16(src[ci] + pb, (ci - NCAA < NCB / 2 ? Blo : Bhi) + dst[ci]);
    }
    // fragment fi at K16 step sp (0..3) of its pair (logical chunk c + 2 sp: slot ^ 2 sp)
    __device__ __forceinline__ bf16x8_t frag(uint8_t* const (&AQ)[4], const uint8_t* Blo, const uint8_t* Bhi, int fi,
                                             int sp) const {
        if (fi == 0 || fi > NI) {
            const int i = fi == 0 ? 0 : fi - NI;
            return *reinterpret_cast<const bf16x8_t*>(AQ[i] + (fo[fi] ^ (32 * sp)));
        }
        return *reinterpret_cast<const bf16x8_t*>((fi - 1 < NI / 2 ? Blo : Bhi) + (fo[fi] ^ (32 * sp)));
    }
    // MFMA t of a K16 step: block (i, j) = (t / NI, t % NI); fragments are
    // ordered A0, B0..B(NI-1), A1.. so that the first MFMAs wait least.  The
    // weight fragment goes in as the instruction's first operand, so a lane's
    // accumulators hold one row of the tile (see the epilogues).
    static __device__ __forceinline__ int fa_idx(int i) { return i == 0 ? 0 : NI + i; }
    static __device__ __forceinline__ int fb_idx(int j) { return 1 + j; }
    __device__ __forceinline__ void mfma(const bf16x8_t (&f)[NFS], int t) {
        const int i = t / NI, j = t % NI;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[fb_idx(j)], f[fa_idx(i)], acc[i][j], 0, 0, 0);
    }
};

// The K loop shared by both kernels.  nst = K / 32 stages (even: K is a
// multiple of 64), in pairs p = (2p, 2p + 1).  A pair p lives in A pair array
// p mod 3, B pair p in B pair array p mod 2.  A pair p + 2 goes out at the
// barrier of stage 2p (every wavefront has then finished pair p - 1, whose
// arrays it takes), three stages before it is read; B pair p + 2 at the
// barrier of stage 2p + 1, into the arrays of pair p, two stages before.  Each stage has
// one barrier, between its two K16 steps: by then every fragment of the
// stage has been read (the second step's during the first), and the next
// stage's operands must have landed (its first fragments are read during the
// second step).  Vector-memory counts complete in issue order: at an odd
// stage's barrier only the A pair issued at the even stage before may still
// be in flight; even stages need nothing new.
template <class GM>
__device__ __forceinline__ void k_loop(GM& g, int nst, uint8_t* const (&A0)[4], uint8_t* const (&A1)[4],
                                       uint8_t* const (&A2)[4], uint8_t* B0lo, uint8_t* B0hi, uint8_t* B1lo,
                                       uint8_t* B1hi) {
    constexpr int NCAA = GM::NCA_, NCB = GM::NCB, NF = GM::NF, NM = GM::NM, NFS = GM::NFS;
    bf16x8_t P[NFS], Q[NFS];
    const int lastp = nst / 2 - 1;
    auto pb = [&](int p) { return (size_t)(p < lastp ? p : lastp) * PROW; };
    // Fragment reads go with the first three quarters of a step's MFMAs, so
    // they have landed when the step ends; the copies go with the last three
    // quarters.
    constexpr int RD = (NM * 3 + 3) / 4, CP = NM / 4;

    // stage J of twelve (chunk j): A pair array (J / 2) mod 3, B pair array
    // (J / 2) mod 2, K32 half J & 1 of the pair
    auto stage = [&](auto kc, int j) {
        constexpr int J = decltype(kc)::value;
        constexpr bool ODD = (J & 1) != 0;
        constexpr int PA = (J / 2) % 3, PB = (J / 2) % 2;
        constexpr int NJ = (J + 1) % 12, NPA = (NJ / 2) % 3, NPB = (NJ / 2) % 2;
        constexpr int NCS = ODD ? NCB : NCAA;  // copies issued this stage
        uint8_t* const (&AQ)[4] = PA == 0 ? A0 : PA == 1 ? A1 : A2;
        uint8_t* const (&NAQ)[4] = NPA == 0 ? A0 : NPA == 1 ? A1 : A2;
        uint8_t* Blo = PB == 0 ? B0lo : B1lo;
        uint8_t* Bhi = PB == 0 ? B0hi : B1hi;
        uint8_t* NBlo = NPB == 0 ? B0lo : B1lo;
        uint8_t* NBhi = NPB == 0 ? B0hi : B1hi;
        // step 0 MFMAs (fragments P) with step 1's fragment reads (Q)
#pragma unroll
        for (int t = 0; t < NM; ++t) {
            g.mfma(P, t);
#pragma unroll
            for (int q = spread<NF, 0, RD>(t); q < spread<NF, 0, RD>(t + 1); ++q)
                Q[q] = g.frag(AQ, Blo, Bhi, q, 2 * (J & 1) + 1);
            pin();
        }
        // every read of this stage done; chunk j + 1 landed
        wait_lgkm0();
        wait_vm<ODD ? NCAA : NCAA + NCB>();
        barrier_nofence();
        // step 1 MFMAs (Q) with the copies (even stages: A pair j / 2 + 2 into
        // the arrays of pair j / 2 - 1; odd stages: B pair (j + 3) / 2 into
        // this pair's B arrays) and the first fragment reads of the next stage
        const size_t pa = pb(j / 2 + 2), pbb = pb((j + 3) / 2);
        uint8_t* const (&FAQ)[4] = PA == 0 ? A2 : PA == 1 ? A0 : A1;  // arrays of pair j / 2 - 1 (= j / 2 + 2 mod 3)
        auto issue = [&](int q) {
            if constexpr (ODD) g.copy_b(Blo, Bhi, NCAA + q, pbb);
            else g.copy_a(FAQ, q, pa);
        };
        if constexpr (NM == 0) {
#pragma unroll
            for (int q = 0; q < NCS; ++q) issue(q);
        }
#pragma unroll
        for (int t = 0; t < NM; ++t) {
            g.mfma(Q, t);
#pragma unroll
            for (int q = spread<NF, 0, RD>(t); q < spread<NF, 0, RD>(t + 1); ++q)
                P[q] = g.frag(NAQ, NBlo, NBhi, q, 2 * ((J + 1) & 1));
#pragma unroll
            for (int q = spread<NCS, CP, NM>(t); q < spread<NCS, CP, NM>(t + 1); ++q) issue(q);
            pin();
        }
    };

    // prologue, in the steady state's issue order: A pair 0, B pair 0, A pair
    // 1, B pair 1; then wait for pair 0
#pragma unroll
    for (int q = 0; q < NCAA; ++q) g.copy_a(A0, q, pb(0));
#pragma unroll
    for (int q = NCAA; q < NCAA + NCB; ++q) g.copy_b(B0lo, B0hi, q, pb(0));
#pragma unroll
    for (int q = 0; q < NCAA; ++q) g.copy_a(A1, q, pb(1));
#pragma unroll
    for (int q = NCAA; q < NCAA + NCB; ++q) g.copy_b(B1lo, B1hi, q, pb(1));
    wait_vm<NCAA + NCB>();
    barrier_nofence();
#pragma unroll
    for (int q = 0; q < NF; ++q) P[q] = g.frag(A0, B0lo, B0hi, q, 0);

    int j = 0;
    for (; j + 12 <= nst; j += 12) {
        stage(ic<0>(), j);
        stage(ic<1>(), j + 1);
        stage(ic<2>(), j + 2);
        stage(ic<3>(), j + 3);
        stage(ic<4>(), j + 4);
        stage(ic<5>(), j + 5);
        stage(ic<6>(), j + 6);
        stage(ic<7>(), j + 7);
        stage(ic<8>(), j + 8);
        stage(ic<9>(), j + 9);
        stage(ic<10>(), j + 10);
        stage(ic<11>(), j + 11);
    }
    // (nst is even: an even number of stages left, at most ten)
    if (j < nst) stage(ic<0>(), j);
    if (j + 1 < nst) stage(ic<1>(), j + 1);
    if (j + 2 < nst) stage(ic<2>(), j + 2);
    if (j + 3 < nst) stage(ic<3>(), j + 3);
    if (j + 4 < nst) stage(ic<4>(), j + 4);
    if (j + 5 < nst) stage(ic<5>(), j + 5);
    if (j + 6 < nst) stage(ic<6>(), j + 6);
    if (j + 7 < nst) stage(ic<7>(), j + 7);
    if (j + 8 < nst) stage(ic<8>(), j + 8);
    if (j + 9 < nst) stage(ic<9>(), j + 9);
    // no copy may still be writing LDS when the workgroup ends
    wait_vm<0>();
}



// Per-lane fragment offsets: wavefront (mh, nh) reads A rows
// block_row(i, mh) + (lane & 31) (quarter i of an A pair) and B rows brow[j] +
// (lane & 31) (B block j < NI/2 lies in rows 0..127 of a pair, the other in
// rows 128..255).
template <class GEO, class GM, int MW>
__device__ __forceinline__ void frag_offsets(GM& g, int mh, const int (&brow)[GEO::NI], int lane) {
    if constexpr (GM::NF > 0) {
        const int r = lane & 31;
        // row r of a 32-row block of a pair (A: in its quarter, B: in its
        // half), logical chunk lane / 32
        const int bslot = (lane >> 5) ^ pair_swz(r);
#pragma unroll
        for (int i = 0; i < GM::AIS; ++i) g.fo[GM::fa_idx(i)] = ((block_row<MW>(i, mh) & 63) + r) * PROW + bslot * 16;
#pragma unroll
        for (int j = 0; j < GEO::NI; ++j) g.fo[GM::fb_idx(j)] = ((brow[j] & 127) + r) * PROW + bslot * 16;
    }
}

// Row blocks wavefront row mh computes for a tile of nrows rows, and A-row
// copies a stage needs.
template <class GEO, int MW, int WV>
__device__ __forceinline__ int active_blocks(int nrows, int mh) {
    const int mb = (nrows + 31) / 32;
    return min(GEO::MI, max(0, (mb - mh + MW - 1) / MW));
}
template <class GEO, int WV>
__device__ __forceinline__ int active_a_copies(int nrows) {
    const int rows = (nrows + 31) / 32 * 32;
    return min(GEO::NCA8, max(1, (rows + 8 * WV - 1) / (8 * WV)));
}

// Calls body.template run<AI, NCAA>() for the runtime pair (ai, ncaa); with
// two wavefront rows ai is ncaa or ncaa - 1 (copy q covers rows 64 q ..
// 64 q + 63, wavefront row mh blocks mh, mh + 2, ...).
template <class GEO, int NCAA, class B>
__device__ __forceinline__ void dispatch_pairs(int ai, int ncaa, B& body) {
    if (ncaa == NCAA) {
        if (ai == NCAA) body.template run<NCAA, NCAA>();
        else body.template run<NCAA - 1, NCAA>();
        return;
    }
    if constexpr (NCAA < GEO::NCA8) dispatch_pairs<GEO, NCAA + 1>(ai, ncaa, body);
}

// ---------------------------------------------------------------------------
// Cold tiles: tiles of at most COLD_WIDE rows (an expert with few rows, or
// the short tail of a hot one).  Their matrix work is a sliver of their weight
// stream, so what bounds them is how many weight bytes a CU keeps in flight.
// A cold tile uses the eight 16 KB LDS arrays as four B pair slots (K64 pairs
// of 128-byte rows, as in the hot loop), three pairs in flight while the
// fourth is read.  Its A rows (up to 64) go to the four 8 KB A pair arrays,
// in K64 pairs too, one copy of 8 rows per pair from each copying wavefront:
// the A rows cross the load path once per workgroup, in whole-line copies,
// rather than once per computing wavefront in fragment loads that each touch
// 32 rows.  Tiles of up to 32 rows are one row block, computed by the first
// wavefront row while the four wavefronts of the second copy its A rows;
// tiles of 33-64 rows give each wavefront row one block, and all eight
// wavefronts copy A rows.
// ---------------------------------------------------------------------------
#ifndef COLD_ROWS_MAX
#define COLD_ROWS_MAX 32
#endif
#ifndef COLD_WIDE_MAX
#define COLD_WIDE_MAX 64
#endif
constexpr int COLD_ROWS = COLD_ROWS_MAX;  // one row block
constexpr int COLD_WIDE = COLD_WIDE_MAX;  // two row blocks
static_assert(COLD_ROWS <= 32 && COLD_WIDE <= 64, "a cold tile is at most two 32-row blocks");
constexpr int YS = 64 * PROW;  // bytes of one A pair array of a cold tile: 64 rows x 128 bytes (8 KB)

// AI: row blocks this wavefront computes (0 or 1); NA: 8-row A copies it
// issues per pair of stages (0 or 1); BNT: the weight copies are non-temporal.
template <class GEO, int AI, int NA, bool BNT>
struct GemmCold {
    static constexpr bool BNT_ = BNT;
    static_assert(AI == 0 || AI == 1, "a cold tile gives a wavefront at most one row block");
    static_assert(NA == 0 || NA == 1, "at most one A copy per wavefront and pair");
    static constexpr int BLOCKS = AI, ACOPIES = NA;
    static constexpr int NI = GEO::NI, NCB = SBN / 8 / GEO::NWV;  // B-row copies per wavefront per pair (8 rows)
    static_assert(NI == 2 && GEO::NW == 4 && NCB % 2 == 0, "a wavefront's two B blocks lie in the two halves of a pair");
    static constexpr int NCPP = NA + NCB;                          // copies per wavefront per pair of stages
    const uint8_t* asrc;   // NA: this lane's A-row copy source at K = 0
    int adst;              // NA: wave-uniform offset of the copy in an A array
    int fa;                // AI: A fragment offset in an A pair array (first K16 step)
    const uint8_t* src[NCB];
    int dst[NCB];          // offsets in a half of a B pair
    int fo[NI];            // B fragment offsets (first K16 step of a pair)
    f32x16_t acc[NI];
};

// Array K of eight.
template <int K>
__device__ __forceinline__ uint8_t* pick8(uint8_t* a0, uint8_t* a1, uint8_t* a2, uint8_t* a3, uint8_t* a4,
                                          uint8_t* a5, uint8_t* a6, uint8_t* a7) {
    if constexpr (K == 0) return a0;
    else if constexpr (K == 1) return a1;
    else if constexpr (K == 2) return a2;
    else if constexpr (K == 3) return a3;
    else if constexpr (K == 4) return a4;
    else if constexpr (K == 5) return a5;
    else if constexpr (K == 6) return a6;
    else return a7;
}

// The K loop of a cold tile: nst = K / 32 stages in eight slots; slots 2m,
// 2m + 1 hold a pair of chunks (K64: 128-byte rows, laid out as the hot
// loop's pairs): the B rows in X arrays 2m (rows 0..127) and 2m + 1 (rows
// 128..255), the A rows in Y array m.
// Chunks are fetched in pairs (2m, 2m + 1): each B copy covers eight whole
// 128-byte lines (see the hot loop's B pairs).  At an even stage j: the pair (j, j + 1)
// has landed (the pairs of chunks j + 2 .. j + 5 may still be in flight) and
// every wavefront has finished reading slots j - 2 and j - 1, which then
// receive the pair (j + 6, j + 7); odd stages only compute.
template <class GC>
__device__ __forceinline__ void k_loop_cold(GC& g, int nst, uint8_t* X0, uint8_t* X1, uint8_t* X2, uint8_t* X3,
                                            uint8_t* X4, uint8_t* X5, uint8_t* X6, uint8_t* X7, uint8_t* Y0,
                                            uint8_t* Y1, uint8_t* Y2, uint8_t* Y3) {
    constexpr int NCPP = GC::NCPP, NI = GC::NI, NCB = GC::NCB;
    const int last = nst - 1;
    auto pb = [&](int c) { return (size_t)((c < last ? c : last) / 2) * PROW; };
    auto slot = [&](auto kc) { return pick8<decltype(kc)::value>(X0, X1, X2, X3, X4, X5, X6, X7); };
    auto aslot = [&](auto kc) {  // the A pair array of slot K
        constexpr int M = decltype(kc)::value / 2;
        return M == 0 ? Y0 : M == 1 ? Y1 : M == 2 ? Y2 : Y3;
    };
    // chunks c, c + 1 into slots K, K + 1 (K even, c even): A rows, then the
    // B pair (whole 128-byte lines)
    auto issue_pair = [&](auto kc, int c) {
        constexpr int K = decltype(kc)::value;
        static_assert(K % 2 == 0, "pairs start at even slots");
        const size_t p0 = pb(c);
        if constexpr (GC::ACOPIES == 1) copy16(g.asrc + p0, aslot(kc) + g.adst);
#pragma unroll
        for (int q = 0; q < NCB; ++q) {
            if constexpr (GC::BNT_) copy16_nt(g.src[q] + p0, (q < NCB / 2 ? slot(kc) : slot(ic<K + 1>())) + g.dst[q]);
            else copy16(g.src[q] + p0, (q < NCB / 2 ? slot(kc) : slot(ic<K + 1>())) + g.dst[q]);
        }
    };
    auto stage = [&](auto kc, int j) {
        constexpr int K = decltype(kc)::value;
        if constexpr (K % 2 == 0) {
            wait_lgkm0();
            wait_vm<2 * NCPP>();
            barrier_nofence();
            issue_pair(ic<(K + 6) % 8>(), j + 6);
        }
        if constexpr (GC::BLOCKS == 1) {
            const uint8_t* Blo = slot(ic<K & ~1>());
            const uint8_t* Bhi = slot(ic<K | 1>());
            const uint8_t* SA = aslot(kc);
            bf16x8_t af[2], b[2][NI];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                af[s] = *reinterpret_cast<const bf16x8_t*>(SA + (g.fa ^ (32 * (2 * (K & 1) + s))));
#pragma unroll
                for (int jj = 0; jj < NI; ++jj)
                    b[s][jj] = *reinterpret_cast<const bf16x8_t*>((jj < NI / 2 ? Blo : Bhi) +
                                                                  (g.fo[jj] ^ (32 * (2 * (K & 1) + s))));
            }
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int jj = 0; jj < NI; ++jj)
                    g.acc[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[s][jj], af[s], g.acc[jj], 0, 0, 0);
        }
    };
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

}  // namespace

// Cold tiles (see k_loop_cold): wavefront row mh computes row block mh (a
// tile of up to 32 rows is computed by wavefront row 0, one of up to 64 rows
// by rows 0 and 1), and the tile's A rows go in copies of 8 rows x 128 bytes
// per pair of stages: 4 of them by the wavefronts of row 1 (tiles of up to
// 32 rows) or 8 by all eight wavefronts.
template <int MW, int WV, class B>
__device__ __forceinline__ void cold_dispatch(B& body, int nrows, int wave) {
    static_assert(MW == 2 && WV == 8, "two wavefront rows of four");
    const int mh = wave % MW, nh = wave / MW;
    if (nrows <= COLD_ROWS) {
        if (mh == 0) body.template run_cold<1, 0>(0);
        else body.template run_cold<0, 1>(nh);
    } else {
        body.template run_cold<1, 1>(wave);
    }
}

// Epilogue layout.  With the weight fragment as the MFMA's first operand, the
// 32 x 32 block's lane l holds tile row (l & 31) of its row block and the 16
// columns 8 * (v / 4) + 4 * (l / 32) + v % 4, v = 0..15 of its column block:
// four runs of four adjacent columns, so each run leaves in one 8-byte (h,
// bf16) or 16-byte (slot_out, fp32) store, and the two lanes of a row
// together write 16 or 32 contiguous bytes per run pair.
__device__ __forceinline__ int run_col(int q, int lane) { return 8 * q + 4 * (lane >> 5); }

// A wavefront's 32 x 32 fp32 block stored as whole 128-byte row segments:
// lane l holds row l & 31 in runs of four columns (run_col), so a direct
// store instruction would write 32 rows x 32 bytes.  The block goes through
// the wavefront's own 4 KB of LDS (16-byte chunk c of row r at slot
// c ^ ((r >> 1) & 7): no bank conflicts either way), scaled by the lane row's
// w, then each lane stores 16 bytes of row 8 p + l / 8 (p = 0..3): eight whole
// rows per instruction.  dst(R) is row R's output address for the block, or
// null (row not stored).
template <class D>
__device__ __forceinline__ void store_block_rows(uint8_t* wl, const f32x16_t& v, float w, int lane, D dst) {
    const int r = lane & 31;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int slot = (2 * q + (lane >> 5)) ^ ((r >> 1) & 7);
        *reinterpret_cast<float4*>(wl + r * 128 + slot * 16) =
            make_float4(w * v[4 * q], w * v[4 * q + 1], w * v[4 * q + 2], w * v[4 * q + 3]);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int R = 8 * p + (lane >> 3), c = lane & 7;
        const float4 val = *reinterpret_cast<const float4*>(wl + R * 128 + ((c ^ ((R >> 1) & 7)) * 16));
        float* o = dst(R);
        if (o) st_stream16(o + 4 * c, val);
    }
}

// h = bf16(silu(g) * u) of four adjacent columns as one 8-byte store.
__device__ __forceinline__ void store_h4(uint16_t* dst, const f32x16_t& g, const f32x16_t& u, int q) {
    uint32_t w[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const float g0 = g[4 * q + 2 * e], u0 = u[4 * q + 2 * e];
        const float g1 = g[4 * q + 2 * e + 1], u1 = u[4 * q + 2 * e + 1];
        w[e] = (uint32_t)f32_to_bf16(silu_f32(g0) * u0) | ((uint32_t)f32_to_bf16(silu_f32(g1) * u1) << 16);
    }
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
}

// ---------------------------------------------------------------------------
// gate/up: BM rows x (128 gate + 128 up) columns per workgroup
// ---------------------------------------------------------------------------
// The expert owns a single tile of rows: its weight rows are read by this
// tile's workgroups only (and each by one of them), so the gate/up kernel
// copies them non-temporal (BNT) and leaves the caches to the rows that are
// shared: the A rows, and the weights of experts with several tiles (c5
// gate/up 2.83 -> 2.78 ms; marking every weight copy non-temporal cost 7%).
__device__ __forceinline__ bool one_tile_expert(const FfnArgs& a, const TileRows& tr) {
    const int rows = tr.g == a.E ? a.T : a.offsets[tr.g + 1] - a.offsets[tr.g];
    return rows <= 256;
}

template <int BM, int MW, int WV, bool BNT>
struct GateUpTile {
    using GEO = Geo<BM, MW, WV>;
    const FfnArgs& a;
    const TileRows& tr;
    const int* src_row;
    uint8_t *X0, *X1, *X2, *X3, *X4, *X5, *X6, *X7;
    uint8_t *Y0, *Y1, *Y2, *Y3;
    int F, n0, wave, lane;

    template <int AI, int NCAA>
    __device__ __forceinline__ void run() {
        using G = Gemm<GEO, AI, NCAA, BNT>;
        constexpr int NI = GEO::NI, NW = GEO::NW;
        const bool shared = tr.g == a.E;
        const int K = a.d;
        G g;
        const MatRef& Wg = shared ? a.s_gate : a.gate;
        const MatRef& Wu = shared ? a.s_up : a.up;
        const int ge = shared ? 0 : tr.g;
        const uint16_t* gbase = static_cast<const uint16_t*>(Wg.q) + ((size_t)ge * F + n0) * K;
        const uint16_t* ubase = static_cast<const uint16_t*>(Wu.q) + ((size_t)ge * F + n0) * K;
        const uint16_t* xbase = static_cast<const uint16_t*>(a.x);
#pragma unroll
        for (int qa = 0; qa < NCAA; ++qa) {  // A: 8 rows x 128 bytes per copy, rows 64 qa + 8 wave ..
            const int ar = 64 * qa + 8 * wave + (lane >> 3);
            g.dst[qa] = wave * 1024;
            // rows past the tile read token 0; their results are never stored
            const int t = src_row[ar];
            g.src[qa] = reinterpret_cast<const uint8_t*>(xbase + (size_t)(t >= 0 ? t : 0) * K) +
                        16 * ((lane & 7) ^ pair_swz(ar));
        }
#pragma unroll
        for (int b = 0; b < G::NCB; ++b) {  // B: 8 rows x 128 bytes per copy, rows 0..255 = gate, then up
            const int r0 = (b * WV + wave) * 8, br = r0 + (lane >> 3);
            g.dst[NCAA + b] = (r0 & 127) * PROW;
            const int n = br & 127;
            const int rr = n0 + n < F ? n : 0;  // columns past F read row 0 and are never stored
            const uint16_t* bb = br < 128 ? gbase : ubase;
            g.src[NCAA + b] =
                reinterpret_cast<const uint8_t*>(bb + (size_t)rr * K) + 16 * ((lane & 7) ^ pair_swz(br));
        }
        // wavefront (mh, nh): gate columns nh * 128/NW + 32 j' and the same up
        // columns (blocks j < NI/2 are gate, j >= NI/2 up)
        const int mh = wave % MW, nh = wave / MW;
        int brow[NI];
#pragma unroll
        for (int j = 0; j < NI; ++j) brow[j] = (j < NI / 2 ? 0 : 128) + nh * (128 / NW) + 32 * (j % (NI / 2));
        frag_offsets<GEO, G, MW>(g, mh, brow, lane);
#pragma unroll
        for (int i = 0; i < G::AIS; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j) g.acc[i][j] = f32x16_t{};

        uint8_t* const AQ0[4] = {X0, X0 + 8192, X2, X2 + 8192};
        uint8_t* const AQ1[4] = {X4, X4 + 8192, X6, X6 + 8192};
        uint8_t* const AQ2[4] = {Y0, Y1, Y2, Y3};
        k_loop(g, K / SK, AQ0, AQ1, AQ2, X1, X3, X5, X7);

        // epilogue: lane holds row (lane & 31) of each row block (see run_col)
        uint16_t* h = static_cast<uint16_t*>(a.h);
#pragma unroll
        for (int i = 0; i < AI; ++i) {
            const int row = block_row<MW>(i, mh) + (lane & 31);
            if (row >= tr.nrows) continue;
            uint16_t* hrow = h + (size_t)(tr.rbeg + row) * a.ldh + n0;
#pragma unroll
            for (int j = 0; j < NI / 2; ++j) {
                if (n0 + brow[j] >= F) continue;  // (F is a multiple of 64: whole blocks)
#pragma unroll
                for (int q = 0; q < 4; ++q) store_h4(hrow + brow[j] + run_col(q, lane), g.acc[i][j], g.acc[i][j + NI / 2], q);
            }
        }
    }

    // a tile of at most COLD_WIDE rows (see k_loop_cold); ac: the A rows this
    // wavefront copies when NA = 1 (rows 16 ac .. 16 ac + 15)
    template <int AI, int NA>
    __device__ __forceinline__ void run_cold(int ac) {
        using G = GemmCold<GEO, AI, NA, BNT>;
        constexpr int NI = GEO::NI, NW = GEO::NW;
        const bool shared = tr.g == a.E;
        const int K = a.d;
        G g;
        const MatRef& Wg = shared ? a.s_gate : a.gate;
        const MatRef& Wu = shared ? a.s_up : a.up;
        const int ge = shared ? 0 : tr.g;
        const uint16_t* gbase = static_cast<const uint16_t*>(Wg.q) + ((size_t)ge * F + n0) * K;
        const uint16_t* ubase = static_cast<const uint16_t*>(Wu.q) + ((size_t)ge * F + n0) * K;
        const uint16_t* xbase = static_cast<const uint16_t*>(a.x);
#pragma unroll
        for (int qb = 0; qb < G::NCB; ++qb) {  // B: 8 rows x 128 bytes per copy, rows 0..255 = gate, then up
            const int r0 = (qb * WV + wave) * 8, br = r0 + (lane >> 3);
            g.dst[qb] = (r0 & 127) * PROW;
            const int n = br & 127;
            const int rr = n0 + n < F ? n : 0;  // columns past F read row 0 and are never stored
            const uint16_t* b = br < 128 ? gbase : ubase;
            g.src[qb] = reinterpret_cast<const uint8_t*>(b + (size_t)rr * K) + 16 * ((lane & 7) ^ pair_swz(br));
        }
        const int mh = wave % MW, nh = wave / MW;
        if constexpr (NA == 1) {  // A rows 8 ac .. 8 ac + 7 (rows past the tile read token 0)
            const int ar = 8 * ac + (lane >> 3);
            const int t = src_row[ar];
            g.asrc = reinterpret_cast<const uint8_t*>(xbase + (size_t)(t >= 0 ? t : 0) * K) +
                     16 * ((lane & 7) ^ pair_swz(ar));
            g.adst = ac * 1024;
        }
        int brow[NI];
#pragma unroll
        for (int j = 0; j < NI; ++j) brow[j] = (j < NI / 2 ? 0 : 128) + nh * (128 / NW) + 32 * (j % (NI / 2));
        // fragment lanes: row lane & 31 (of block mh for A), logical chunk
        // lane / 32 (first K16 step of a pair)
        const int bslot = (lane >> 5) ^ pair_swz(lane & 31);
        g.fa = (block_row<MW>(0, mh) + (lane & 31)) * PROW + bslot * 16;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            g.fo[j] = ((brow[j] & 127) + (lane & 31)) * PROW + bslot * 16;
            g.acc[j] = f32x16_t{};
        }

        k_loop_cold(g, K / SK, X0, X1, X2, X3, X4, X5, X6, X7, Y0, Y1, Y2, Y3);

        if constexpr (AI == 1) {
            const int row = block_row<MW>(0, mh) + (lane & 31);
            if (row < tr.nrows) {
                uint16_t* hrow = static_cast<uint16_t*>(a.h) + (size_t)(tr.rbeg + row) * a.ldh + n0;
#pragma unroll
                for (int j = 0; j < NI / 2; ++j) {
                    if (n0 + brow[j] >= F) continue;
#pragma unroll
                    for (int q = 0; q < 4; ++q) store_h4(hrow + brow[j] + run_col(q, lane), g.acc[j], g.acc[j + NI / 2], q);
                }
            }
        }
    }
};

template <int BM, int MW, int WV>
__global__ __launch_bounds__(64 * WV, 1) void gateup_dma_kernel(FfnArgs a) {
    using GEO = Geo<BM, MW, WV>;
    static_assert(BM * SROW == XS, "a stage's A rows fill one LDS array");
    // eight separate arrays (separate objects, so the compiler can tell a
    // read of one from the copies still landing in the others): hot tiles
    // use them as four K32 stages of (A rows, B rows), cold tiles as eight
    // B-row stages
    __shared__ __attribute__((aligned(1024))) uint8_t X0[XS];
    __shared__ __attribute__((aligned(1024))) uint8_t X1[XS];
    __shared__ __attribute__((aligned(1024))) uint8_t X2[XS];
    __shared__ __attribute__((aligned(1024))) uint8_t X3[XS];
    __shared__ __attribute__((aligned(1024))) uint8_t X4[XS];
    __shared__ __attribute__((aligned(1024))) uint8_t X5[XS];
    __shared__ __attribute__((aligned(1024))) uint8_t X6[XS];
    __shared__ __attribute__((aligned(1024))) uint8_t X7[XS];
    // four 8 KB arrays: the hot loop's third A pair array (64 rows each), or a
    // cold tile's four A pair arrays
    __shared__ __attribute__((aligned(1024))) uint8_t Y0[YS];
    __shared__ __attribute__((aligned(1024))) uint8_t Y1[YS];
    __shared__ __attribute__((aligned(1024))) uint8_t Y2[YS];
    __shared__ __attribute__((aligned(1024))) uint8_t Y3[YS];
    // the tile's source tokens share Y3: both loops read them before their
    // first copy into Y3, which goes out after the first barrier of the loop
    // (issued after the first stage's barrier)
    static_assert(BM * sizeof(int) <= YS, "row table fits one A array");
    int* src_row = reinterpret_cast<int*>(Y3);
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
    const int ai = active_blocks<GEO, MW, WV>(tr.nrows, wave % MW);
    auto go = [&](auto bnt) {
        GateUpTile<BM, MW, WV, decltype(bnt)::value> body{a,  tr, src_row, X0, X1, X2, X3, X4, X5, X6,
                                                          X7, Y0, Y1,      Y2, Y3, F,  n0, wave, lane};
        if (tr.nrows <= COLD_WIDE) cold_dispatch<MW, WV>(body, tr.nrows, wave);
        else dispatch_pairs<GEO, 1>(ai, active_a_copies<GEO, WV>(tr.nrows), body);
    };
    if (one_tile_expert(a, tr)) go(std::true_type());
    else go(std::false_type());
}

// ---------------------------------------------------------------------------
// down + weighted scatter: BM rows x 256 output columns per workgroup
// ---------------------------------------------------------------------------
template <int BM, int MW, int WV, bool BNT>
struct DownTile {
    using GEO = Geo<BM, MW, WV>;
    const FfnArgs& a;
    const TileRows& tr;
    const int* dst_row;
    const float* wrow;
    uint8_t *X0, *X1, *X2, *X3, *X4, *X5, *X6, *X7;
    uint8_t *Y0, *Y1, *Y2, *Y3;
    int n0, wave, lane;

    template <int AI, int NCAA>
    __device__ __forceinline__ void run() {
        using G = Gemm<GEO, AI, NCAA, BNT>;
        constexpr int NI = GEO::NI, NW = GEO::NW;
        const bool shared = tr.g == a.E;
        const int K = shared ? a.Fs : a.F;
        const int N = a.d;
        G g;
        const MatRef& D = shared ? a.s_down : a.down;
        const int ge = shared ? 0 : tr.g;
        const uint16_t* dbase = static_cast<const uint16_t*>(D.q) + ((size_t)ge * N + n0) * K;
        const uint16_t* hbase = static_cast<const uint16_t*>(a.h) + (size_t)tr.rbeg * a.ldh;
#pragma unroll
        for (int qa = 0; qa < NCAA; ++qa) {  // A: 8 rows x 128 bytes per copy, rows 64 qa + 8 wave ..
            const int ar = 64 * qa + 8 * wave + (lane >> 3);
            g.dst[qa] = wave * 1024;
            const int rr = ar < tr.nrows ? ar : 0;  // rows past the tile: never stored
            g.src[qa] = reinterpret_cast<const uint8_t*>(hbase + (size_t)rr * a.ldh) + 16 * ((lane & 7) ^ pair_swz(ar));
        }
#pragma unroll
        for (int b = 0; b < G::NCB; ++b) {  // B: 8 rows x 128 bytes per copy
            const int r0 = (b * WV + wave) * 8, br = r0 + (lane >> 3);
            g.dst[NCAA + b] = (r0 & 127) * PROW;
            const int rr = n0 + br < N ? br : 0;
            g.src[NCAA + b] =
                reinterpret_cast<const uint8_t*>(dbase + (size_t)rr * K) + 16 * ((lane & 7) ^ pair_swz(br));
        }
        // wavefront (mh, nh): output columns nh * 32 + 128 j (one block in
        // each half of a B pair)
        const int mh = wave % MW, nh = wave / MW;
        int brow[NI];
#pragma unroll
        for (int j = 0; j < NI; ++j) brow[j] = 128 * j + nh * (128 / NW);
        frag_offsets<GEO, G, MW>(g, mh, brow, lane);
#pragma unroll
        for (int i = 0; i < G::AIS; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j) g.acc[i][j] = f32x16_t{};

        // the lane's rows' destinations and weights (their LDS table is
        // overwritten by the K loop's third A pair array)
        int drow[G::AIS];
        float dw[G::AIS];
#pragma unroll
        for (int i = 0; i < AI; ++i) {
            const int row = block_row<MW>(i, mh) + (lane & 31);
            drow[i] = row < tr.nrows ? dst_row[row] : -1;
            dw[i] = row < tr.nrows ? wrow[row] : 0.0f;
        }
        uint8_t* const AQ0[4] = {X0, X0 + 8192, X2, X2 + 8192};
        uint8_t* const AQ1[4] = {X4, X4 + 8192, X6, X6 + 8192};
        uint8_t* const AQ2[4] = {Y0, Y1, Y2, Y3};
        k_loop(g, K / SK, AQ0, AQ1, AQ2, X1, X3, X5, X7);

        // epilogue through LDS (store_block_rows): every wavefront has left
        // the K loop's LDS stages before any is reused; row R's destination
        // comes from lane R
        wait_lgkm0();
        barrier_nofence();
        float* out = shared ? a.shared_out : a.slot_out;
        uint8_t* wl = (wave < 4 ? X0 : X2) + (wave & 3) * 4096;
#pragma unroll
        for (int i = 0; i < AI; ++i) {
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                if (n0 + brow[j] >= N) continue;  // (d is a multiple of 64: whole blocks)
                store_block_rows(wl, g.acc[i][j], dw[i], lane, [&](int R) -> float* {
                    const int dr = __shfl(drow[i], R);
                    return dr >= 0 ? out + (size_t)dr * N + n0 + brow[j] : nullptr;
                });
            }
        }
    }

    // a tile of at most COLD_WIDE rows (see k_loop_cold); ac: the A rows this
    // wavefront copies when NA = 1 (rows 16 ac .. 16 ac + 15)
    template <int AI, int NA>
    __device__ __forceinline__ void run_cold(int ac) {
        using G = GemmCold<GEO, AI, NA, BNT>;
        constexpr int NI = GEO::NI, NW = GEO::NW;
        const bool shared = tr.g == a.E;
        const int K = shared ? a.Fs : a.F;
        const int N = a.d;
        G g;
        const MatRef& D = shared ? a.s_down : a.down;
        const int ge = shared ? 0 : tr.g;
        const uint16_t* dbase = static_cast<const uint16_t*>(D.q) + ((size_t)ge * N + n0) * K;
        const uint16_t* hbase = static_cast<const uint16_t*>(a.h) + (size_t)tr.rbeg * a.ldh;
#pragma unroll
        for (int qb = 0; qb < G::NCB; ++qb) {  // B: 8 rows x 128 bytes per copy
            const int r0 = (qb * WV + wave) * 8, br = r0 + (lane >> 3);
            g.dst[qb] = (r0 & 127) * PROW;
            const int rr = n0 + br < N ? br : 0;
            g.src[qb] = reinterpret_cast<const uint8_t*>(dbase + (size_t)rr * K) + 16 * ((lane & 7) ^ pair_swz(br));
        }
        const int mh = wave % MW, nh = wave / MW;
        if constexpr (NA == 1) {  // A rows 8 ac .. 8 ac + 7 (rows past the tile read row 0; never stored)
            const int ar = 8 * ac + (lane >> 3);
            const int rr = ar < tr.nrows ? ar : 0;
            g.asrc = reinterpret_cast<const uint8_t*>(hbase + (size_t)rr * a.ldh) + 16 * ((lane & 7) ^ pair_swz(ar));
            g.adst = ac * 1024;
        }
        // this lane's output row and weight, read before the K loop: the
        // LDS that holds them is reused by the A-row copies
        const int orow_i = block_row<MW>(0, mh) + (lane & 31);
        const int drow = AI == 1 && orow_i < tr.nrows ? dst_row[orow_i] : -1;
        const float dw = AI == 1 && orow_i < tr.nrows ? wrow[orow_i] : 0.0f;
        int brow[NI];
#pragma unroll
        for (int j = 0; j < NI; ++j) brow[j] = 128 * j + nh * (128 / NW);
        // fragment lanes: row lane & 31 (of block mh for A), logical chunk
        // lane / 32 (first K16 step of a pair)
        const int bslot = (lane >> 5) ^ pair_swz(lane & 31);
        g.fa = (block_row<MW>(0, mh) + (lane & 31)) * PROW + bslot * 16;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            g.fo[j] = ((brow[j] & 127) + (lane & 31)) * PROW + bslot * 16;
            g.acc[j] = f32x16_t{};
        }

        k_loop_cold(g, K / SK, X0, X1, X2, X3, X4, X5, X6, X7, Y0, Y1, Y2, Y3);

        if constexpr (AI == 1) {
            if (drow >= 0) {
                float* orow = (shared ? a.shared_out : a.slot_out) + (size_t)drow * N + n0;
                const float w = dw;
#pragma unroll
                for (int j = 0; j < NI; ++j) {
                    if (n0 + brow[j] >= N) continue;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<float4*>(orow + brow[j] + run_col(q, lane)) =
                            make_float4(w * g.acc[j][4 * q], w * g.acc[j][4 * q + 1], w * g.acc[j][4 * q + 2],
                                        w * g.acc[j][4 * q + 3]);
                }
            }
        }
    }
};

template <int BM, int MW, int WV>
__global__ __launch_bounds__(64 * WV, 1) void down_dma_kernel(FfnArgs a) {
    using GEO = Geo<BM, MW, WV>;
    static_assert(BM * SROW == XS, "a stage's A rows fill one LDS array");
    // eight separate arrays (separate objects, so the compiler can tell a
    // read of one from the copies still landing in the others): hot tiles
    // use them as four K32 stages of (A rows, B rows), cold tiles as eight
    // B-row stages
    __shared__ __attribute__((aligned(1024))) uint8_t X0[XS];
    __shared__ __attribute__((aligned(1024))) uint8_t X1[XS];
    __shared__ __attribute__((aligned(1024))) uint8_t X2[XS];
    __shared__ __attribute__((aligned(1024))) uint8_t X3[XS];
    __shared__ __attribute__((aligned(1024))) uint8_t X4[XS];
    __shared__ __attribute__((aligned(1024))) uint8_t X5[XS];
    __shared__ __attribute__((aligned(1024))) uint8_t X6[XS];
    __shared__ __attribute__((aligned(1024))) uint8_t X7[XS];
    // four 8 KB arrays: the hot loop's third A pair array (64 rows each), or a
    // cold tile's four A pair arrays
    __shared__ __attribute__((aligned(1024))) uint8_t Y0[YS];
    __shared__ __attribute__((aligned(1024))) uint8_t Y1[YS];
    __shared__ __attribute__((aligned(1024))) uint8_t Y2[YS];
    __shared__ __attribute__((aligned(1024))) uint8_t Y3[YS];
    // the tile's destinations and weights share Y3 (see gateup_dma_kernel):
    // each lane reads its rows' into registers before the K loop
    static_assert(BM * (sizeof(int) + sizeof(float)) <= YS, "row tables fit one A array");
    int* dst_row = reinterpret_cast<int*>(Y3);
    float* wrow = reinterpret_cast<float*>(Y3 + BM * sizeof(int));
    int tile, ntile;
    if (!work_item<4>(tile_count(a), tile, ntile)) return;
    TileRows tr;
    if (!tile_rows<BM>(a, tile, tr)) return;
    const bool shared = tr.g == a.E;
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
    // (non-temporal weight copies for one-tile experts help gate/up, not down:
    // c5 down 1.61 -> 1.65 ms with them)
    DownTile<BM, MW, WV, false> body{a, tr, dst_row, wrow, X0, X1, X2, X3, X4, X5, X6, X7, Y0, Y1, Y2, Y3, n0, wave, lane};
    const int ai = active_blocks<GEO, MW, WV>(tr.nrows, wave % MW);
    if (tr.nrows <= COLD_WIDE) {
        cold_dispatch<MW, WV>(body, tr.nrows, wave);
    } else {
        dispatch_pairs<GEO, 1>(ai, active_a_copies<GEO, WV>(tr.nrows), body);
    }
}

// wavefront grid of the kernels launched: DMA_MW x (DMA_WV / DMA_MW)
#ifndef DMA_MW_V
#define DMA_MW_V 2
#define DMA_WV_V 8
#endif
constexpr int DMA_MW = DMA_MW_V, DMA_WV = DMA_WV_V;

hipError_t launch_gateup_dma(const FfnArgs& a, hipStream_t st, const KTime& kt) {
    const int fmax = a.n_shared && a.Fs > a.F ? a.Fs : a.F;
    dim3 grid(a.max_tiles, (fmax + SBN / 2 - 1) / (SBN / 2));
    if (a.bm != 256) return hipErrorInvalidValue;
    launch_kernel(gateup_dma_kernel<256, DMA_MW, DMA_WV>, grid, 64 * DMA_WV, st, kt, a);
    return hipGetLastError();
}

hipError_t launch_down_dma(const FfnArgs& a, hipStream_t st, const KTime& kt) {
    dim3 grid(a.max_tiles, (a.d + SBN - 1) / SBN);
    if (a.bm != 256) return hipErrorInvalidValue;
    launch_kernel(down_dma_kernel<256, DMA_MW, DMA_WV>, grid, 64 * DMA_WV, st, kt, a);
    return hipGetLastError();
}

}  // namespace moe
