// topk_rows.hip - top-k over long candidate rows: for every row of n fp32
// scores, the k candidates that come first under the router's selection order
// (larger value first, NaN after every number, -0 == +0, equal values by lower
// index), written by ascending candidate index.  This is the selection of the
// sparse attention indexer (top-512 or top-1024 rows out of a long row; "256
// experts, 512 lines" blog post, section "The constant that always said 256").
//
// One workgroup per row; the row stays in registers.  Wavefront w owns the
// contiguous candidates [w * NPT * 64, (w + 1) * NPT * 64): chunk j of it is
// the 64 candidates from w * NPT * 64 + j * 64, one per lane, so every load
// instruction reads 256 contiguous bytes and (chunk, lane) order is index order.
//   1. Keys: the float's bits mapped to an unsigned key whose integer order is
//      the selection order (padding -> 0).  NaN (-> 1) and -0 (-> the key of
//      +0) need a fix-up that only wavefronts holding one of them run.
//   2. Radix select, 8 bits per pass from the top: a 256-bin histogram of the
//      keys that still match the resolved prefix, the bin where the running
//      count from the top reaches the number still needed, and the prefix
//      grows by that digit.  A pass ends the search early when the whole bin is
//      needed.  The histogram keeps 32 columns per bin and lane l adds to
//      column l % 32, so the LDS atomics of one instruction never collide more
//      than two to an address, whatever the score distribution (floats in a
//      narrow range put nearly every key in one or two top-byte bins).
//   3. Output in index order: each wavefront counts its keys above the
//      threshold and equal to it; the wavefront totals give every wavefront the
//      number of chosen candidates before it.  Equal keys are chosen while their
//      rank among equal keys is below the number still needed, which cuts the
//      tie at the threshold by index; only the wavefront holding the cut tests
//      that rank.  A chosen candidate's position is the running count of its
//      wavefront plus its rank in the chunk's ballot; chosen candidates wait in
//      a ring in LDS private to the wavefront and leave 64 at a time, in one
//      coalesced store per output array.
#include <cmath>
#include <type_traits>

#include "topk_rows.h"

namespace moe {
namespace {

// Key of a float whose bits are u: negative -> ~u, else u with the sign bit
// set.  Integer order of keys is numeric order (integer operations only, so
// subnormal scores keep their order), except for NaN and -0 (fixed below).
__device__ __forceinline__ uint32_t raw_key(uint32_t u) {
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
// The fix-up: -0 (key 0x7FFFFFFF) ranks with +0, every NaN (+NaN above +inf's
// key 0xFF800000, -NaN below -inf's 0x007FFFFF) becomes 1, below every number.
__device__ __forceinline__ uint32_t fix_key(uint32_t k) {
    k = k == 0x7FFFFFFFu ? 0x80000000u : k;
    return k - 0x007FFFFFu <= 0xFF800000u - 0x007FFFFFu ? k : 1u;
}

// The score a key came from, branch-free: a key with the top bit set came from
// a non-negative float (clear the bit), any other from a negative one (invert).
// Exact except for the two keys that merge several bit patterns (0x80000000:
// +0 or -0; 1: any NaN), which the caller reloads.
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float(k ^ (~(uint32_t)((int32_t)k >> 31) | 0x80000000u));
}

struct TkState {
    uint32_t prefix, mask, need, done;
};

// Writes the chosen candidates of one wavefront.  CUT: this wavefront holds the
// cut of the tie at the threshold (equal keys are chosen while their rank among
// equal keys, erun + ballot rank, is below need); otherwise a key is chosen when
// key & mask >= pc.  SPECIAL: the row holds NaN or -0, whose values are reloaded.
// The wavefront's outputs are the contiguous positions [run, run + its count):
// chosen candidates go to a 128-entry ring in LDS (private to the wavefront, so
// no workgroup barrier), and every 64 of them leave in one coalesced store per
// output array.  The stores go through buffer descriptors of k entries.
constexpr int TK_RING = 128;
constexpr int TK_SAMPLES = 256;          // keys sampled per row for the threshold
constexpr int TK_CAND_PER_THREAD = 8;    // LDS room for candidates per thread
constexpr int TK_BIN_BITS = 12, TK_BINS = 1 << TK_BIN_BITS;  // bins of the candidates' counting pass

template <int NPT, bool CUT, bool SPECIAL>
__device__ __forceinline__ void emit_wave(const uint32_t* key, uint32_t mask, uint32_t pc, uint32_t prefix,
                                          uint32_t need, uint32_t run, uint32_t erun, int base0, bool with_vals,
                                          uint32_t* ring_i, uint32_t* ring_v, __amdgpu_buffer_rsrc_t out_idx,
                                          __amdgpu_buffer_rsrc_t out_vals, __amdgpu_buffer_rsrc_t rsrc) {
    const int lane = lane_id();
    const uint32_t start = run;  // outputs [start, flushed) are stored, [flushed, run) wait in the ring
    uint32_t flushed = start;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
        const uint32_t km = key[j] & mask;
        bool chosen;
        if (CUT) {
            const uint64_t em = __ballot(km == prefix);
            const uint32_t erank = (uint32_t)__builtin_amdgcn_mbcnt_hi(
                (uint32_t)(em >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)em, erun));
            chosen = km > prefix || (km == prefix && erank < need);
            erun += (uint32_t)__popcll(em);
        } else {
            chosen = km >= pc;
        }
        const uint64_t cm = __ballot(chosen);
        if (cm == 0ull) continue;
        const uint32_t pos =
            (uint32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(cm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)cm, run));
        run += (uint32_t)__popcll(cm);
        if (chosen) {
            const int i = base0 + j * WAVE + lane;
            const uint32_t kk = key[j];
            float v = key_value(kk);  // rebuilt from the key: no memory round trip per chosen score
            if (SPECIAL && with_vals && (kk == 0x80000000u || kk == 1u))
                v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc, i * 4, 0, 0));
            const uint32_t slot = (pos - start) % TK_RING;
            ring_i[slot] = (uint32_t)i;
            ring_v[slot] = __float_as_uint(v);
        }
        if (run - flushed >= (uint32_t)WAVE) {  // fewer than 64 wait before a chunk, so the ring never overruns
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            const uint32_t e = flushed + (uint32_t)lane, slot = (e - start) % TK_RING;
            __builtin_amdgcn_raw_buffer_store_b32(ring_i[slot], out_idx, (int)(e * 4u), 0, 0);
            if (with_vals) __builtin_amdgcn_raw_buffer_store_b32(ring_v[slot], out_vals, (int)(e * 4u), 0, 0);
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            flushed += WAVE;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const uint32_t e = flushed + (uint32_t)lane;
    if (e < run) {
        const uint32_t slot = (e - start) % TK_RING;
        __builtin_amdgcn_raw_buffer_store_b32(ring_i[slot], out_idx, (int)(e * 4u), 0, 0);
        if (with_vals) __builtin_amdgcn_raw_buffer_store_b32(ring_v[slot], out_vals, (int)(e * 4u), 0, 0);
    }
}

template <int THREADS, int NPT>
__global__ __launch_bounds__(THREADS, 2) void topk_rows_kernel(TopkRowsArgs a) {
    constexpr int WAVES = THREADS / WAVE;
    constexpr int SPAN = NPT * WAVE;  // candidates per wavefront
    constexpr int COLS = 32;          // histogram columns: lane l adds to column l % 32
    constexpr int S = THREADS / 256;  // merge threads per bin
    constexpr int R = COLS / S;       // columns each of them sums
    static_assert(S >= 1 && R * S == COLS && WAVES <= WAVE, "launch shape");

    // One LDS region serves the two paths, which never run in the same
    // workgroup at once (the sampled pass writes nothing here before it is
    // sure to finish the row): the full path's histogram and output rings, or
    // the sampled pass's TK_BINS counters (the histogram's first words, zero
    // as the full path needs them), candidate keys and 16-bit candidate
    // indices (n <= 65536).  Small enough for two 1024-thread workgroups of
    // 32 keys per thread on one CU.
    constexpr bool SAMPLED = NPT >= 16;  // rows of 16 or more keys per thread (see topk_rows_sample_rank)
    constexpr int CAP = SAMPLED ? TK_CAND_PER_THREAD * THREADS : 0;  // candidates the sampled pass can hold
    static_assert(TK_BINS % THREADS == 0 && TK_BINS <= 256 * COLS && TK_SAMPLES >= WAVE, "candidate bins");
    constexpr int FULL_WORDS = 256 * COLS + WAVES * 2 * TK_RING, SAMPLED_WORDS = TK_BINS + CAP + CAP / 2;
    __shared__ uint32_t lds[FULL_WORDS > SAMPLED_WORDS ? FULL_WORDS : SAMPLED_WORDS];
    uint32_t* const hist = lds;                      // [bin][column]
    uint32_t* const ring = lds + 256 * COLS;         // per wavefront: chosen indices, then values, on their way out
    uint32_t* const cand_key = lds + TK_BINS;        // sampled pass
    uint16_t* const cand_idx = (uint16_t*)(lds + TK_BINS + CAP);
    __shared__ uint32_t tot[256];         // tot[r] = count of bin 255 - r
    __shared__ uint32_t wtot[3][WAVES];   // per wavefront: keys above, equal, any NaN / -0
    __shared__ TkState st;
    __shared__ uint32_t samp[TK_SAMPLES];
    __shared__ uint32_t wmax[WAVES], wcnt[WAVES], fst[2];

    const int tid = threadIdx.x, lane = lane_id(), wave = wave_index();
    const int n = a.n, k = a.k;
    const int base0 = wave * SPAN;
    const float* row = a.scores + (size_t)blockIdx.x * n;

    for (int w = tid; w < 256 * COLS; w += THREADS) hist[w] = 0;

    // Every load is issued before the first key is formed.  Buffer loads: one
    // offset register (the chunk goes in the instruction's offset), and the
    // range check of the descriptor (n floats) returns 0 past the row.
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), (short)0, n * 4, 0x00020000);
    uint32_t key[NPT];
#pragma unroll
    for (int j = 0; j < NPT; ++j) key[j] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (base0 + lane) * 4, j * WAVE * 4, 0);
    uint64_t special = 0;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
        uint32_t u = key[j];
        asm volatile("" : "+v"(u));  // keeps every load ahead of all key arithmetic
        special |= __ballot(__builtin_amdgcn_classf(__uint_as_float(u), 0x23));  // NaN or -0
        key[j] = raw_key(u);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (special != 0ull) {
#pragma unroll
        for (int j = 0; j < NPT; ++j) key[j] = fix_key(key[j]);
    }
    if (base0 + SPAN > n) {  // the wavefront reaches past the row: padding keys are 0
#pragma unroll
        for (int j = 0; j < NPT; ++j) key[j] = lane < n - (base0 + j * WAVE) ? key[j] : 0u;
    }
    if (lane == 0) wtot[2][wave] = special != 0ull ? 1u : 0u;
    // Samples for the threshold: the middle chunk of every wavefront, every
    // LSTEP-th lane (TK_SAMPLES in all, spread over the row); and the row's
    // largest key.
    constexpr int SPW = TK_SAMPLES / WAVES, LSTEP = WAVE / SPW;
    static_assert(SPW * WAVES == TK_SAMPLES && LSTEP * SPW == WAVE, "sample layout");
    const bool sampled = SAMPLED && a.sample_rank > 0;
    if (sampled) {
        if (lane % LSTEP == 0) samp[wave * SPW + lane / LSTEP] = key[NPT / 2];
        uint32_t mx = 0;
#pragma unroll
        for (int j = 0; j < NPT; ++j) mx = max(mx, key[j]);
        mx = wave_max_u32(mx);
        if (lane == 0) wmax[wave] = mx;
    }
    __syncthreads();

    // ---- radix select ----------------------------------------------------
    // Passes of 8 bits from bit position shift down (the last one aligned at
    // bit 0; a pass may re-read bits already resolved, which are constant among
    // the matching keys).  count(mask, prefix, shift) adds every key with
    // key & mask == prefix to the histogram.  On return st holds the threshold
    // (prefix under mask) and the number of keys at it that are still needed.
    uint32_t* my_col = &hist[lane % COLS];
    // cols: the counts are spread over COLS columns per bin (keys of the whole
    // row, whose top bytes collide); otherwise one counter per bin in the first
    // 256 words (the few candidates of the sampled pass, spread over the bins).
    auto radix = [&](auto&& count, uint32_t prefix, uint32_t mask, int shift, uint32_t need, auto cols_tag) {
        constexpr bool cols = decltype(cols_tag)::value;
        for (;;) {
            count(mask, prefix, shift);
            __syncthreads();
            if constexpr (!cols) {
                if (tid < 256) {
                    tot[255 - tid] = hist[tid];
                    hist[tid] = 0;
                }
            } else {
                const int b = tid / S, s = tid % S;
                uint32_t c = 0;
                // not unrolled fully: the R column addresses would stay live in
                // registers for the whole kernel
#pragma unroll 4
                for (int i = 0; i < R; ++i) {
                    const int l = s * R + ((i + b) % R);  // distinct columns across a wavefront: no bank conflicts
                    c += hist[b * COLS + l];
                    hist[b * COLS + l] = 0;
                }
#pragma unroll
                for (int o = 1; o < S; o <<= 1) c += __shfl_xor(c, o);
                if (s == 0) tot[255 - b] = c;
            }
            __syncthreads();
            if (wave == 0) {
                const uint32_t c0 = tot[4 * lane], c1 = tot[4 * lane + 1], c2 = tot[4 * lane + 2],
                               c3 = tot[4 * lane + 3];
                const uint32_t sum = c0 + c1 + c2 + c3;
                const uint32_t incl = wave_incl_scan_u32(sum);
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
            shift = max(shift - 8, 0);
        }
    };
    const bool with_vals = a.vals != nullptr;
    const __amdgpu_buffer_rsrc_t out_idx =
        __builtin_amdgcn_make_buffer_rsrc(a.idx + (size_t)blockIdx.x * k, (short)0, k * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t out_vals = __builtin_amdgcn_make_buffer_rsrc(
        with_vals ? (void*)(a.vals + (size_t)blockIdx.x * k) : (void*)(a.idx + (size_t)blockIdx.x * k), (short)0,
        k * 4, 0x00020000);

    // ---- sampled pass ------------------------------------------------------
    // T = the sample_rank-th largest sample.  If between k and CAP keys are
    // >= T, the chosen candidates are all among them (every key below T has at
    // least k keys above it): they are compacted in index order into LDS and
    // the exact selection and the output run on them alone.  Otherwise (an
    // unlucky sample, heavy ties) the row takes the full radix path below.
    if constexpr (SAMPLED) if (sampled) {
        if (wave == 0) {
            // T: two 8-bit radix steps over the samples (one wavefront, four
            // samples per lane, the histogram in tot), which find the 16-bit
            // prefix of the sample_rank-th largest sample; T is the smallest key
            // with that prefix, so at least sample_rank samples are >= T.
            uint32_t sv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[i] = samp[4 * lane + i];
            uint32_t prefix = 0, mask = 0, need = (uint32_t)a.sample_rank;
#pragma unroll
            for (int pass = 0; pass < 2; ++pass) {
                const int shift = 24 - 8 * pass;
#pragma unroll
                for (int i = 0; i < 4; ++i) tot[4 * lane + i] = 0u;
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if ((sv[i] & mask) == prefix) atomicAdd(&tot[(sv[i] >> shift) & 255u], 1u);
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                const uint32_t c0 = tot[255 - 4 * lane], c1 = tot[254 - 4 * lane], c2 = tot[253 - 4 * lane],
                               c3 = tot[252 - 4 * lane];  // lane l: bins 255 - 4l down to 252 - 4l
                const uint32_t sum = c0 + c1 + c2 + c3, incl = wave_incl_scan_u32(sum);
                uint32_t above = incl - sum;
                int r = 0;
                if (above + c0 < need) {
                    above += c0, r = 1;
                    if (above + c1 < need) {
                        above += c1, r = 2;
                        if (above + c2 < need) above += c2, r = 3;
                    }
                }
                const int L = __ffsll((unsigned long long)__ballot(incl >= need)) - 1;  // exists: need <= matching samples
                const uint32_t b = 255u - (uint32_t)(4 * L + __builtin_amdgcn_readlane(r, L));
                need -= (uint32_t)__builtin_amdgcn_readlane((int)above, L);
                prefix |= b << shift;
                mask |= 255u << shift;
            }
            const uint32_t km = wave_max_u32(lane < WAVES ? wmax[lane] : 0u);
            if (lane == 0) fst[0] = prefix, fst[1] = km;
        }
        __syncthreads();
        const uint32_t T = __builtin_amdgcn_readfirstlane(fst[0]), KMAX = __builtin_amdgcn_readfirstlane(fst[1]);
        uint32_t c_w = 0;
#pragma unroll
        for (int j = 0; j < NPT; ++j) {
            c_w += (uint32_t)__popcll(__ballot(key[j] >= T));
            __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("" : "+s"(c_w));
        if (lane == 0) wcnt[wave] = c_w;
        __syncthreads();
        const uint32_t wc = lane < WAVES ? wcnt[lane] : 0u;
        const uint32_t C = wave_sum_u32(wc);
        if (T != 0u && C >= (uint32_t)k && C <= (uint32_t)CAP) {
            uint32_t run = wave_sum_u32(lane < wave ? wc : 0u);
            uint32_t TC = T;
            asm volatile("" : "+s"(TC));  // the tests are made again, not held in scalar registers since the count
#pragma unroll
            for (int j = 0; j < NPT; ++j) {
                const bool c = key[j] >= TC;
                const uint64_t m = __ballot(c);
                const uint32_t pos = (uint32_t)__builtin_amdgcn_mbcnt_hi(
                    (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, run));
                if (c) {
                    cand_key[pos] = key[j];
                    cand_idx[pos] = (uint16_t)(base0 + j * WAVE + lane);
                }
                run += (uint32_t)__popcll(m);
            }
            __syncthreads();
            // Exact selection among the candidates, which lie in [T, KMAX].  One
            // pass counts them in TK_BINS bins of 2^sh consecutive keys from T;
            // the bin where the count from the top reaches k holds the k-th key.
            // If it is needed whole, every key from its lower end is chosen;
            // else its keys (usually a handful) are gathered and one wavefront
            // takes the remaining rank among them.  A crossing bin of more than
            // 64 keys (dense ties) runs 8-bit radix passes on the candidates.
            uint32_t M = 0xFFFFFFFFu, P = T, NEED = (uint32_t)k;  // all candidates equal: the first k
            if (T != KMAX) {
                const uint32_t span = KMAX - T;
                const int sh = max(0, 32 - __builtin_clz(span) - TK_BIN_BITS);  // (span >> sh) < TK_BINS
                for (int i = tid; i < (int)C; i += THREADS) atomicAdd(&hist[(cand_key[i] - T) >> sh], 1u);
                __syncthreads();
                constexpr int BPT = TK_BINS / THREADS;  // bins per thread, highest first
                uint32_t cb[BPT], csum = 0;
#pragma unroll
                for (int q = 0; q < BPT; ++q) {
                    const int bin = TK_BINS - 1 - BPT * tid - q;
                    cb[q] = hist[bin];
                    hist[bin] = 0u;  // (zero again for the radix fallback)
                    csum += cb[q];
                }
                const uint32_t ci = wave_incl_scan_u32(csum);
                if (lane == WAVE - 1) wcnt[wave] = ci;
                __syncthreads();
                const uint32_t cincl = wave_sum_u32(lane < wave && lane < WAVES ? wcnt[lane] : 0u) + ci;
                if (cincl - csum < (uint32_t)k && cincl >= (uint32_t)k) {  // exactly one thread
                    uint32_t above = cincl - csum;
                    int q = 0;
                    while (q < BPT - 1 && above + cb[q] < (uint32_t)k) above += cb[q++];
                    st.prefix = (uint32_t)(TK_BINS - 1 - BPT * tid - q);  // the crossing bin
                    st.need = (uint32_t)k - above;                       // keys still needed from it
                    st.mask = cb[q];                                      // keys in it
                    st.done = 0u;                                         // gathered so far
                }
                __syncthreads();
                const uint32_t bstar = __builtin_amdgcn_readfirstlane(st.prefix), rem = __builtin_amdgcn_readfirstlane(st.need),
                               cbin = __builtin_amdgcn_readfirstlane(st.mask);
                const uint32_t lo = T + (bstar << sh);  // smallest key of the crossing bin
                if (rem == cbin) {
                    M = 0xFFFFFFFFu, P = lo - 1u, NEED = 0u;  // chosen: key >= lo (lo >= T >= 1)
                } else if (cbin <= (uint32_t)WAVE) {
                    for (int i = tid; i < (int)C; i += THREADS) {
                        const uint32_t kk = cand_key[i];
                        if (((kk - T) >> sh) == bstar) samp[atomicAdd(&st.done, 1u)] = kk;
                    }
                    __syncthreads();
                    if (wave == 0) {
                        // the rem-th largest of the bin's keys, taken one by one
                        uint32_t v = lane < (int)cbin ? samp[lane] : 0u, kth = 0u;
                        const uint32_t mine = v;
                        for (uint32_t it = 0; it < rem; ++it) {
                            kth = wave_max_u32(v);
                            const uint64_t who = __ballot(v == kth);
                            if (lane == __ffsll((unsigned long long)who) - 1) v = 0u;
                        }
                        const uint32_t greater = (uint32_t)__popcll(__ballot(lane < (int)cbin && mine > kth));
                        if (lane == 0) st.prefix = kth, st.need = rem - greater;
                    }
                    __syncthreads();
                    M = 0xFFFFFFFFu;
                    P = __builtin_amdgcn_readfirstlane(st.prefix);
                    NEED = __builtin_amdgcn_readfirstlane(st.need);
                } else {
                    const uint32_t diff = T ^ KMAX;
                    const int hb = 31 - __builtin_clz(diff);
                    const uint32_t m0 = ~((2u << hb) - 1u);  // 0 when hb = 31
                    radix(
                        [&](uint32_t mask, uint32_t prefix, int shift) {
                            for (int i = tid; i < (int)C; i += THREADS) {
                                const uint32_t kk = cand_key[i];
                                if ((kk & mask) == prefix) atomicAdd(&hist[(kk >> shift) & 255u], 1u);
                            }
                        },
                        T & m0, m0, max(hb - 7, 0), (uint32_t)k, std::false_type());
                    M = __builtin_amdgcn_readfirstlane(st.mask);
                    P = __builtin_amdgcn_readfirstlane(st.prefix);
                    NEED = __builtin_amdgcn_readfirstlane(st.need);
                }
            }
            // Output: thread t takes the candidates [t * per, (t + 1) * per);
            // block scans of its counts above and at the threshold give its
            // first output position.
            const int per = ((int)C + THREADS - 1) / THREADS;
            const int i0 = min(tid * per, (int)C), i1 = min(i0 + per, (int)C);
            uint32_t g = 0, e = 0;
            for (int i = i0; i < i1; ++i) {
                const uint32_t km = cand_key[i] & M;
                g += km > P ? 1u : 0u;
                e += km == P ? 1u : 0u;
            }
            const uint32_t gi = wave_incl_scan_u32(g), ei = wave_incl_scan_u32(e);
            if (lane == WAVE - 1) wtot[0][wave] = gi, wtot[1][wave] = ei;
            __syncthreads();
            const bool row_special = __ballot(lane < WAVES && wtot[2][lane] != 0u) != 0ull;
            uint32_t g_before = wave_sum_u32(lane < wave && lane < WAVES ? wtot[0][lane] : 0u) + gi - g;
            uint32_t e_before = wave_sum_u32(lane < wave && lane < WAVES ? wtot[1][lane] : 0u) + ei - e;
            for (int i = i0; i < i1; ++i) {
                const uint32_t kk = cand_key[i], km = kk & M;
                int off = -1;
                if (km > P) {
                    off = (int)((g_before + min(e_before, NEED)) * 4u);
                    ++g_before;
                } else if (km == P) {
                    if (e_before < NEED) off = (int)((g_before + e_before) * 4u);
                    ++e_before;
                }
                if (off >= 0) {
                    const uint32_t ci = cand_idx[i];
                    __builtin_amdgcn_raw_buffer_store_b32(ci, out_idx, off, 0, 0);
                    if (with_vals) {
                        float v = key_value(kk);
                        if (row_special && (kk == 0x80000000u || kk == 1u))
                            v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc, (int)(ci * 4u), 0, 0));
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), out_vals, off, 0, 0);
                    }
                }
            }
            return;
        }
    }

    // ---- full radix path over the keys in registers ------------------------
    radix(
        [&](uint32_t mask, uint32_t prefix, int shift) {
#pragma unroll
            for (int j = 0; j < NPT; ++j) {
                const uint32_t kk = key[j];
                if ((kk & mask) == prefix) atomicAdd(my_col + ((kk >> shift) & 255u) * COLS, 1u);
            }
        },
        0u, 0u, 24, (uint32_t)k, std::true_type());
    const uint32_t prefix = __builtin_amdgcn_readfirstlane(st.prefix), mask = __builtin_amdgcn_readfirstlane(st.mask),
                   need = __builtin_amdgcn_readfirstlane(st.need);

    // ---- output in index order --------------------------------------------
    // Chosen: key & mask > prefix (all of them), and the first `need` keys with
    // key & mask == prefix by index.  Padding (key 0) never passes either test.
    uint32_t g_w = 0, e_w = 0;  // this wavefront's keys above / at the threshold
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
        const uint32_t km = key[j] & mask;
        g_w += (uint32_t)__popcll(__ballot(km > prefix));
        e_w += (uint32_t)__popcll(__ballot(km == prefix));
        __builtin_amdgcn_sched_barrier(0);  // one chunk at a time: no scalar masks held across chunks
    }
    asm volatile("" : "+s"(g_w), "+s"(e_w));  // counted here, not inside the store's branch
    if (lane == 0) {
        wtot[0][wave] = g_w;
        wtot[1][wave] = e_w;
    }
    __syncthreads();
    // lane w < WAVES holds wavefront w's totals; DPP sums give the totals of the
    // wavefronts before this one
    const uint32_t wg = lane < WAVES ? wtot[0][lane] : 0u, we = lane < WAVES ? wtot[1][lane] : 0u;
    const bool row_special = __ballot(lane < WAVES && wtot[2][lane] != 0u) != 0ull;
    const uint32_t g_base = wave_sum_u32(lane < wave ? wg : 0u), e_base = wave_sum_u32(lane < wave ? we : 0u);
    // The threshold passes through an empty asm statement, so the tests below
    // are recomputed instead of being held in scalar registers since the counts.
    uint32_t M = mask, P = prefix, NEED = need;
    asm volatile("" : "+s"(M), "+s"(P), "+s"(NEED));
    const uint32_t run = g_base + min(e_base, NEED);  // chosen candidates before this wavefront
    const bool all_eq = e_base + e_w <= NEED, no_eq = e_base >= NEED;
    if (all_eq || no_eq) {
        if (no_eq && P == 0xFFFFFFFFu) return;  // nothing above the largest key: no output here
        const uint32_t pc = all_eq ? P : P + 1u;
        if (row_special)
            emit_wave<NPT, false, true>(key, M, pc, P, NEED, run, e_base, base0, with_vals, ring + wave * 2 * TK_RING, ring + (wave * 2 + 1) * TK_RING,
                                         out_idx, out_vals, rsrc);
        else
            emit_wave<NPT, false, false>(key, M, pc, P, NEED, run, e_base, base0, with_vals, ring + wave * 2 * TK_RING, ring + (wave * 2 + 1) * TK_RING,
                                         out_idx, out_vals, rsrc);
    } else {
        if (row_special)
            emit_wave<NPT, true, true>(key, M, P, P, NEED, run, e_base, base0, with_vals, ring + wave * 2 * TK_RING, ring + (wave * 2 + 1) * TK_RING,
                                        out_idx, out_vals, rsrc);
        else
            emit_wave<NPT, true, false>(key, M, P, P, NEED, run, e_base, base0, with_vals, ring + wave * 2 * TK_RING, ring + (wave * 2 + 1) * TK_RING,
                                        out_idx, out_vals, rsrc);
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

// Rank of the sampled threshold among the TK_SAMPLES samples: the expected
// number of samples above the k-th largest key plus four standard deviations
// and three, so that fewer than k keys reach it (and the row takes the full
// radix path) for about one row in 10^4 to 10^5 of random scores; 0 (no
// sampled pass) for rows of fewer than 16 keys per thread, where the full
// passes are short, and when the expected number of candidates would not fit
// comfortably in the LDS room for them.  (A margin of six deviations and four
// cost 3% more on the 512 x 32768, top-1024 and 1 x 65536, top-1024 indexer
// workloads: more candidates to select from and to write out.)
int topk_rows_sample_rank(int n, int k) {
    if (topk_rows_npt(n) < 16) return 0;
    // the samples are spread over the workgroup's key slots, those past n being padding
    const double slots = (double)topk_rows_threads(n) * topk_rows_npt(n);
    const double kf = (double)k * TK_SAMPLES / slots;
    const int r = (int)std::ceil(kf + 4.0 * std::sqrt(kf) + 3.0);
    const double expect = (double)r * slots / TK_SAMPLES;
    if (r > TK_SAMPLES / 2 || expect > 0.7 * TK_CAND_PER_THREAD * topk_rows_threads(n)) return 0;
    return r;
}

hipError_t launch_topk_rows(const TopkRowsArgs& a_in, hipStream_t st, const KTime& kt) {
    TopkRowsArgs a = a_in;
    if (a.rows == 0) return hipSuccess;
    if (a.rows < 0 || a.n < 1 || a.n > TOPK_ROWS_MAX_N || a.k < 1 || a.k > a.n) return hipErrorInvalidValue;
    a.sample_rank = topk_rows_sample_rank(a.n, a.k);
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
