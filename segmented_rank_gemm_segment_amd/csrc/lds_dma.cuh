// LDS staging helpers for the MFMA kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora_device.cuh"

namespace lora {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Direct global -> LDS loads (gfx950 global_load_lds_dwordx4).  Each
// instruction moves 64 lanes x 16 bytes into 1 KB of LDS starting at M0.
// Issued through inline asm so that the compiler does not add conservative
// waits on them; completion is tracked by hand with s_waitcnt vmcnt(0) only
// (a wave waits for all of its loads, never for a count of them, so no wait
// depends on the order in which loads complete).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

__device__ __forceinline__ void dma16(uint32_t m0, const void *src) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src)
               : "memory", "m0");
}

// The same with the source given as a 64-bit scalar base plus a 32-bit
// per-lane byte offset (the instruction's saddr form).
__device__ __forceinline__ void dma16_s(uint32_t m0, uint32_t off, const void *base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(off), "s"(base)
               : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding, then LDS-fence and barrier the workgroup.
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lgkm_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ mfma_bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(mfma_bf16x8, v); }

// Row of element v (0..15) of a 32x32 MFMA accumulator held by lane l
// (its column is l % 32).
__device__ __forceinline__ int acc_row(int v, int l) { return (v >> 2) * 8 + (l >> 5) * 4 + (v & 3); }

}  // namespace lora
