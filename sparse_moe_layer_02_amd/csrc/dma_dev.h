// dma_dev.h - the global->LDS copy path and the waits and barriers that go
// with it, shared by the kernels that stage operands with
// global_load_lds_dwordx4 (grouped_gemm_dma.hip, grouped_gemm_q8_dma.hip).
#pragma once
#include <type_traits>

#include "common.h"

namespace moe {

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

// 16 bytes per lane from global memory into LDS at dst + 16 * lane (dst
// wave-uniform).  Vector-memory counters complete in issue order, so a wait
// for one copy waits for every load issued before it.
__device__ __forceinline__ void copy16(const uint8_t* src, uint8_t* dst) {
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void*)(dst), 16, 0, 0);
}

template <int K>
using ic = std::integral_constant<int, K>;

// LDS rows of 64 bytes: the four 16-byte chunks of row r sit at slot c ^ f(r),
// f(r) = ((r >> 1) & 3) ^ ((r >> 3) & 1), so that sixteen consecutive rows
// read at one chunk hit sixteen different 16-byte bank groups.
__device__ __forceinline__ int slot_swz(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }

// Copy lanes: lane l of copy q of wavefront w fills stage row
// r = (q * WV + w) * 16 + l / 4, slot l & 3, which holds logical chunk
// (l & 3) ^ f(r); f(r) = ((l >> 3) & 3) ^ ((l >> 5) & 1) since r = l / 4 mod 16.
__device__ __forceinline__ int copy_row(int q, int wv, int wave, int lane) { return (q * wv + wave) * 16 + (lane >> 2); }
__device__ __forceinline__ int copy_chunk(int lane) { return (lane & 3) ^ ((lane >> 3) & 3) ^ ((lane >> 5) & 1); }

}  // namespace moe
