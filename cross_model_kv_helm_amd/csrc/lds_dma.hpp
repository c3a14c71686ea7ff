// lds_dma.hpp — gfx950 building blocks shared by the matrix-core kernels
// that stage operand tiles through LDS: raw buffer descriptors, the
// buffer -> LDS copy, the wait for this wave's copies and the LDS barrier.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace helm {
namespace lds {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_t;

// Offset past every descriptor's range: the load returns zeros and touches
// no memory (an offset plus up to 255 stays past every range).
constexpr uint32_t kSkip = 0xffffff00u;

// Raw buffer descriptor words: base, `bytes` in range (offsets at or past it
// read zeros), raw (unswizzled) dword format.  The arguments are wave-uniform;
// readfirstlane tells the compiler so, keeping the words in scalar registers
// (the copy's descriptor operand must be one).
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xffffu),
               (uint32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}

// Buffer -> LDS copy of 16 bytes per lane: lane i reads the 16 bytes at
// byte offset voff + soff of the buffer `rsrc` and they land at lds_base +
// 16*i.  rsrc, soff and lds_base are wave-uniform; only voff is range
// checked.  Inline assembly so that the compiler does not make later LDS
// accesses wait for the copy; the kernel waits for its copies itself
// (wait_vmcnt) before the barrier that publishes a tile.
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t voff, uint32_t soff, const void* lds_base) {
  const uint32_t m = (uint32_t)(uintptr_t)(lds_void_t)lds_base;
  asm("" : "+s"(soff));   // a constant offset above 64 is no inline operand: keep it in a register
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "s"(m)
               : "memory", "m0");
}

// Waits until at most N of this wave's vector memory operations (here only
// the copies) are outstanding; they complete in issue order.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace lds
}  // namespace helm
