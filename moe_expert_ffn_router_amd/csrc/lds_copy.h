// Copies from global memory straight into LDS (global_load_lds), the waits
// on them, and the 16-byte-unit swizzles of LDS rows that keep fragment reads
// free of bank conflicts.  Shared by the prefill GEMMs.
#pragma once

#include "moe_internal.h"

namespace moe {

// Swizzles of the 16-byte units of a row, chosen so that the 16-byte
// fragment reads hit distinct banks both per 8 lanes (32 banks) and per
// 16 lanes (64 banks): 16 consecutive rows reading the same unit spread over
// all banks.  a_swz for 128-byte rows (8 units), b_swz for 64-byte rows (4).
__device__ __forceinline__ int a_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int b_swz(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }

// Copies of 16 bytes (4 bytes) per lane from base + off into LDS at lds +
// 16 * lane (4 * lane).  Issued as inline assembly: the compiler then sees no
// pending LDS write (it would otherwise wait for every copy in flight before
// any LDS read it cannot prove disjoint), and every wait on these copies is
// an explicit one (moe_lds_sync).  No register receives data (the address
// registers are read at issue).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t off, const void* lds) {
  const uint32_t l = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(l) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const uint8_t* base, uint32_t off, const void* lds) {
  const uint32_t l = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(off), "s"(base), "s"(l) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt immediate: at most `vm` vector memory operations outstanding
// (vmcnt is 6 bits, split over bits 3:0 and 15:14), no LDS operation
// outstanding (lgkmcnt 0), expcnt not waited.
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | 0x070; }

// Wait (as above), then a barrier that the compiler moves no memory access
// across.
#define MOE_DMA_SYNC(N)                                          \
  do {                                                           \
    __builtin_amdgcn_s_waitcnt(::moe::waitcnt_vm_lgkm0(N));      \
    asm volatile("s_barrier" ::: "memory");                      \
  } while (0)

}  // namespace moe
