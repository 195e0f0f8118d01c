// dma.h -- LDS DMA helpers shared by the GEMM kernels (gfx950).
//
// global_load_lds_dwordx4 moves 16 bytes per lane from global memory straight
// into LDS: lane i's bytes land at M0 + 16 * i.  The loads are issued from
// inline assembly (they have no register results), and their completion is
// awaited with explicit vmcnt waits, because the compiler would otherwise
// wait for every outstanding DMA before each LDS read.
#pragma once
#include "common.h"

namespace moe {

// XOR swizzle of the 16-byte chunks of an LDS tile row holding a BK-wide K
// step of bf16 (BK = 64: 128-byte rows; BK = 32: 64-byte rows): chunk c of
// row R sits in slot c ^ swz_slot<BK>(R).
template <int BK>
__device__ __forceinline__ int swz_slot(int R) {
  if constexpr (BK == 64)
    return (R & 7) ^ ((R >> 3) & 1);
  else
    return (R >> 2) & 3;
}

// NT: non-temporal (streamed once, e.g. expert weights: ~7.0 vs ~6.2 TB/s
// for plain streaming reads on MI355X).  The compiler treats m0 as reserved
// and ignores the clobber; that is safe here because compiler-generated code
// in these kernels never uses m0 (tests/test_isa_cpu.py checks the ISA).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool NT>
__device__ __forceinline__ void dma16(const void *gbase, uint32_t voff, uint32_t lds_addr) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(gbase)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(gbase)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// 32-row fragments of a wave's TM-fragment row band holding at least one
// valid row, given `left` = valid rows from the band's first row (uniform).
template <int TM>
__device__ __forceinline__ int live_frags(int64_t left) {
  if (left <= 0) return 0;
  const int64_t f = (left + 31) / 32;
  return f < TM ? (int)f : TM;
}

// s_waitcnt vmcnt(N) with the other counters left open (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}


}  // namespace moe
