// topk_rows.hip - top-k over long candidate rows: for every row of n fp32
// scores, the k candidates that come first under the router's selection order
// (larger value first, NaN after every number, -0 == +0, equal values by lower
// index), written by ascending candidate index.  This is the selection of the
// sparse attention indexer (top-512 or top-1024 rows out of a long row; "256
// experts, 512 lines" blog post, section "The constant that always said 256").
//
// One workgroup per row; the row stays in registers (NPT keys per thread,
// element i = j * THREADS + tid, so every load instruction is coalesced).
//   1. Keys: the float is mapped to an unsigned key whose integer order is the
//      selection order (NaN -> 1, padding -> 0, -0 -> +0).
//   2. Radix select, 8 bits per pass from the top: a 256-bin histogram of the
//      keys that still match the resolved prefix, the bin where the running
//      count from the top reaches the number still needed, and the prefix
//      grows by that digit.  A pass ends the search early when the whole bin is
//      needed.  The histogram keeps one column per lane (two 16-bit counters
//      per word), so the LDS atomics of one instruction never share an
//      address, whatever the score distribution (floats in a narrow range put
//      nearly every key in one or two top-byte bins).
//   3. Compaction in index order: per (chunk, wavefront) group the counts of
//      keys above the threshold and equal to it, a block-wide exclusive scan
//      of both, then each chosen key's output position = keys above it with a
//      lower index + min(equal keys with a lower index, equal keys needed).
//      The tie at the threshold is thereby cut by index.
#include "kernels.h"
#include "permute_dev.h"

namespace moe {
namespace {

// Selection order as an unsigned integer order; 0 is reserved for padding.
// Integer operations only (subnormal scores keep their order), and every step
// works on the key itself, so the loaded value dies at once.
__device__ __forceinline__ uint32_t order_key(float x) {
    const uint32_t u = __float_as_uint(x);
    uint32_t k = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);  // negative: ~u; else u | sign bit
    k = k == 0x7FFFFFFFu ? 0x80000000u : k;                          // -0 ranks with +0
    // NaN: +NaN maps above +inf's key 0xFF800000, -NaN below -inf's 0x007FFFFF
    return k - 0x007FFFFFu <= 0xFF800000u - 0x007FFFFFu ? k : 1u;
}

struct TkState {
    uint32_t prefix, mask, need, done;
};

template <int THREADS, int NPT>
__global__ __launch_bounds__(THREADS, 2) void topk_rows_kernel(TopkRowsArgs a) {
    constexpr int WAVES = THREADS / WAVE;
    constexpr int GROUPS = NPT * WAVES;  // (chunk, wavefront) groups in index order
    constexpr int S = THREADS / 128;     // merge threads per histogram word
    constexpr int R = WAVE / S;          // lane columns each of them sums
    static_assert(GROUPS <= THREADS && S >= 1 && R * S == WAVE, "launch shape");

    __shared__ uint32_t hist[128][WAVE];  // word w: bins 2w (low half), 2w+1 (high half); column = lane
    __shared__ uint32_t tot[256];         // tot[r] = count of bin 255 - r
    __shared__ uint32_t cgt[GROUPS], ceq[GROUPS];
    __shared__ uint32_t wsum[2][WAVES];
    __shared__ TkState st;

    const int tid = threadIdx.x, lane = lane_id(), wave = wave_index();
    const int n = a.n, k = a.k;
    const float* row = a.scores + (size_t)blockIdx.x * n;

    for (int w = tid; w < 128 * WAVE; w += THREADS) (&hist[0][0])[w] = 0;

    // Every load is issued before the first key is formed.  Buffer loads: one
    // offset register for all chunks (the chunk goes in the scalar offset),
    // and the range check of the descriptor (n floats) returns 0 past the row.
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), (short)0, n * 4, 0x00020000);
    float v[NPT];
#pragma unroll
    for (int j = 0; j < NPT; ++j)
        v[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc, tid * 4, j * THREADS * 4, 0));
    uint32_t key[NPT];
#pragma unroll
    for (int j = 0; j < NPT; ++j) key[j] = tid < n - j * THREADS ? order_key(v[j]) : 0u;  // scalar bound per chunk
    __syncthreads();

    // ---- radix select ----------------------------------------------------
    uint32_t prefix = 0, mask = 0, need = (uint32_t)k;
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
        for (int j = 0; j < NPT; ++j) {
            const uint32_t kk = key[j];
            if ((kk & mask) == prefix) {
                const uint32_t b = (kk >> shift) & 255u;
                atomicAdd(&hist[b >> 1][lane], 1u << ((b & 1u) * 16u));
            }
        }
        __syncthreads();
        {
            const int w = tid / S, s = tid % S;
            uint32_t lo = 0, hi = 0;
            // not unrolled fully: the R column addresses would stay live in
            // registers for the whole kernel
#pragma unroll 4
            for (int i = 0; i < R; ++i) {
                const int l = s * R + ((i + w) % R);  // distinct columns across a wavefront: no bank conflicts
                const uint32_t c = hist[w][l];
                hist[w][l] = 0;
                lo += c & 0xFFFFu;
                hi += c >> 16;
            }
#pragma unroll
            for (int o = 1; o < S; o <<= 1) {
                lo += __shfl_xor(lo, o);
                hi += __shfl_xor(hi, o);
            }
            if (s == 0) {
                tot[255 - 2 * w] = lo;
                tot[254 - 2 * w] = hi;
            }
        }
        __syncthreads();
        if (wave == 0) {
            const uint32_t c0 = tot[4 * lane], c1 = tot[4 * lane + 1], c2 = tot[4 * lane + 2],
                           c3 = tot[4 * lane + 3];
            const uint32_t sum = c0 + c1 + c2 + c3;
            const uint32_t incl = (uint32_t)wave_incl_scan((int)sum);
            const uint64_t hit = __ballot(incl >= need);
            if (hit != 0ull && lane == __ffsll((unsigned long long)hit) - 1) {
                uint32_t above = incl - sum, c = c0;
                int r = 0;
                if (above + c0 < need) {
                    above += c0, c = c1, r = 1;
                    if (above + c1 < need) {
                        above += c1, c = c2, r = 2;
                        if (above + c2 < need) above += c2, c = c3, r = 3;
                    }
                }
                const uint32_t b = 255u - (uint32_t)(4 * lane + r);
                const uint32_t rem = need - above;
                st.prefix = prefix | (b << shift);
                st.mask = mask | (255u << shift);
                st.need = rem;
                // Padding keys (0) are counted only while the prefix is 0, i.e. in
                // the lowest bin; the search never stops on a zero prefix, so the
                // final threshold is never matched by padding.
                st.done = ((rem == c && st.prefix != 0u) || shift == 0) ? 1u : 0u;
            } else if (hit == 0ull && lane == 0) {
                // unreachable while k <= valid keys; keeps the exit uniform
                st.prefix = prefix, st.mask = mask, st.need = need, st.done = 1u;
            }
        }
        __syncthreads();
        prefix = __builtin_amdgcn_readfirstlane(st.prefix);
        mask = __builtin_amdgcn_readfirstlane(st.mask);
        need = __builtin_amdgcn_readfirstlane(st.need);
        if (__builtin_amdgcn_readfirstlane(st.done)) break;
    }

    // ---- compaction in index order ----------------------------------------
    // Chosen: key & mask > prefix (all of them), and the first `need` keys with
    // key & mask == prefix by index.  Padding (key 0) never passes either test.
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
        const uint32_t km = key[j] & mask;
        const uint64_t bg = __ballot(km > prefix), be = __ballot(km == prefix);
        if (lane == 0) {
            cgt[j * WAVES + wave] = (uint32_t)__popcll(bg);
            ceq[j * WAVES + wave] = (uint32_t)__popcll(be);
        }
    }
    __syncthreads();
    {
        const uint32_t g = tid < GROUPS ? cgt[tid] : 0u, e = tid < GROUPS ? ceq[tid] : 0u;
        const uint32_t gi = (uint32_t)wave_incl_scan((int)g), ei = (uint32_t)wave_incl_scan((int)e);
        if (lane == WAVE - 1) {
            wsum[0][wave] = gi;
            wsum[1][wave] = ei;
        }
        __syncthreads();
        uint32_t gb = 0, eb = 0;
        for (int w = 0; w < wave; ++w) {
            gb += wsum[0][w];
            eb += wsum[1][w];
        }
        if (tid < GROUPS) {
            cgt[tid] = gb + gi - g;
            ceq[tid] = eb + ei - e;
        }
    }
    __syncthreads();
    // The threshold is read again after the barrier, so the tests below are
    // recomputed instead of being held in registers since the count loop.
    const uint32_t M = __builtin_amdgcn_readfirstlane(st.mask), P = __builtin_amdgcn_readfirstlane(st.prefix),
                   NEED = __builtin_amdgcn_readfirstlane(st.need);
    const uint64_t below = lanemask_lt();
    int32_t* idx = a.idx + (size_t)blockIdx.x * k;
    float* vals = a.vals ? a.vals + (size_t)blockIdx.x * k : nullptr;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
        const uint32_t km = key[j] & M;
        const bool gt = km > P, eq = km == P;
        const uint64_t bg = __ballot(gt), be = __ballot(eq);
        if (bg == 0ull && be == 0ull) continue;
        const uint32_t g_before = cgt[j * WAVES + wave] + (uint32_t)__popcll(bg & below);
        const uint32_t e_before = ceq[j * WAVES + wave] + (uint32_t)__popcll(be & below);
        uint32_t pos = 0xFFFFFFFFu;
        if (gt) pos = g_before + min(e_before, NEED);
        else if (eq && e_before < NEED) pos = g_before + e_before;
        if (pos < (uint32_t)k && tid < n - j * THREADS) {  // both hold by construction
            const int i = j * THREADS + tid;
            idx[pos] = i;
            if (vals) vals[pos] = row[i];
        }
    }
}

template <int THREADS, int NPT>
hipError_t launch_shape(const TopkRowsArgs& a, hipStream_t st, const KTime& kt) {
    launch_kernel(topk_rows_kernel<THREADS, NPT>, dim3(a.rows), dim3(THREADS), st, kt, a);
    return hipGetLastError();
}

}  // namespace

// Launch shapes: up to 16384 candidates 512 threads with 1..32 keys each (a
// power of two); beyond that 1024 threads with 32 or 64 keys each.
int topk_rows_threads(int n) { return n > 512 * 32 ? 1024 : 512; }

int topk_rows_npt(int n) {
    if (n < 1 || n > TOPK_ROWS_MAX_N) return 0;
    const int threads = topk_rows_threads(n);
    int npt = 1;
    while (threads * npt < n) npt *= 2;
    return npt;
}

hipError_t launch_topk_rows(const TopkRowsArgs& a, hipStream_t st, const KTime& kt) {
    if (a.rows == 0) return hipSuccess;
    if (a.rows < 0 || a.n < 1 || a.n > TOPK_ROWS_MAX_N || a.k < 1 || a.k > a.n) return hipErrorInvalidValue;
    const int npt = topk_rows_npt(a.n);
    if (topk_rows_threads(a.n) == 1024) {
        if (npt == 32) return launch_shape<1024, 32>(a, st, kt);
        if (npt == 64) return launch_shape<1024, 64>(a, st, kt);
        return hipErrorInvalidValue;
    }
    switch (npt) {
        case 1: return launch_shape<512, 1>(a, st, kt);
        case 2: return launch_shape<512, 2>(a, st, kt);
        case 4: return launch_shape<512, 4>(a, st, kt);
        case 8: return launch_shape<512, 8>(a, st, kt);
        case 16: return launch_shape<512, 16>(a, st, kt);
        case 32: return launch_shape<512, 32>(a, st, kt);
    }
    return hipErrorInvalidValue;
}

}  // namespace moe
