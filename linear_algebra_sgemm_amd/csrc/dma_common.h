// Direct global -> LDS copies shared by the direct-to-LDS kernels (FP32 and the
// half products): the copy instruction, its waits and the LDS layout rule for
// tiles stored as 64-byte rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lasg {

// Chunk permutation of row r of a tile stored as 64-byte rows of four 16-byte
// chunks.  A fragment read takes the same chunk from 32 consecutive rows; four
// rows fill one 256-byte line of the 64 banks, so without a permutation rows r,
// r + 4, r + 8 ... would all hit the same 16-byte bank group (a 4-way conflict).
// Permuting the chunks by (r / 4) % 4 gives the rows of four consecutive lines
// four different groups.  Measured on gfx950 with SQ_LDS_BANK_CONFLICT: this
// form is conflict-free (4 LDS cycles per 16-byte read of a wave), while a
// permutation by ((r / 2) ^ (r / 8)) % 4 still costs 8 cycles.
__device__ __forceinline__ int row64_swizzle(int r) { return (r >> 2) & 3; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// All LDS reads of this wave are complete, then the workgroup barrier.  (HIP's
// __syncthreads would also wait for every outstanding global load, which would
// drain the prefetch pipeline.)  The wait is the compiler's own s_waitcnt so that
// its wait-count bookkeeping knows the LDS reads before it are done; the empty
// asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt left at their maxima
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One direct global -> LDS copy of 16 bytes per lane from address base + offset
// (a wave-uniform 64-bit base in scalar registers and a per-lane 32-bit byte
// offset: the instruction's saddr form, so the K loop only advances the scalar
// base); lane l writes LDS bytes [lds_base + 16 l, +16).  Written as inline
// assembly so that the compiler does not add its own "wait for every LDS-bound
// load" before later LDS reads; the kernel orders these copies itself with
// wait_vmcnt and the barriers.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // m0 is listed as clobbered on purpose
__device__ __forceinline__ void dma16_sbase(const void* base, uint32_t offset, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_base), "v"(offset), "s"(base) : "memory", "m0");
}
// The same with the LDS address passed through readfirstlane: for callers in
// which the compiler cannot see that the address is wave-uniform (it is), so
// that it stays in a scalar register.
__device__ __forceinline__ void dma16_sbase_u(const void* base, uint32_t offset, uint32_t lds_base) {
  dma16_sbase(base, offset, __builtin_amdgcn_readfirstlane(lds_base));
}
// The same with 4 bytes per lane (lane l writes LDS bytes [lds_base + 4 l, +4)):
// for sources whose rows are only 4-byte aligned.
__device__ __forceinline__ void dma4_sbase(const void* base, uint32_t offset, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(lds_base), "v"(offset), "s"(base) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

}  // namespace lasg
