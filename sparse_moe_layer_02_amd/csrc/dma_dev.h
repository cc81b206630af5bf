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

// The same copy marked non-temporal (rows no other workgroup reads).
__device__ __forceinline__ void copy16_nt(const uint8_t* src, uint8_t* dst) {
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void*)(dst), 16, 0, 2);
}

template <int K>
using ic = std::integral_constant<int, K>;

// LDS rows of 128 bytes (a copy instruction of 64 lanes x 16 bytes then
// covers eight whole cache lines): the eight 16-byte chunks of row r sit at
// slot c ^ g(r), g(r) = (r >> 1) & 7, so that sixteen consecutive rows read at
// one chunk hit sixteen different 16-byte bank groups.  Copy lane l of a copy
// of rows r0 .. r0 + 7 (r0 a multiple of 8) fills row r0 + l / 8, slot l & 7,
// which holds logical chunk (l & 7) ^ g(r0 + l / 8).
__device__ __forceinline__ int pair_swz(int r) { return (r >> 1) & 7; }

}  // namespace moe
