// LDS staging helpers shared by the streaming kernels (decode and prefill attention, large-tile
// GEMM).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {
namespace lds {

// Wait until at most `n` vector-memory operations of this wave are outstanding (n a constant).
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(((n >> 4) << 14) | (0xF << 8) | (0x7 << 4) | (n & 0xF));
}

// Work-group barrier for LDS traffic only: waits for this wave's LDS operations, not for its
// outstanding global loads (prefetches stay in flight across it).
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One direct global->LDS load of 16 bytes per lane: lane i's bytes at base + off land at LDS
// byte lds + 16 i.  Inline assembly, so the compiler does not track it (its own tracking makes
// every later LDS read wait for all such loads); completion is awaited with wait_vm before the
// barrier that publishes the data.  No register results; the address operands are read at issue.
__device__ __forceinline__ void dma16(const char* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "{m0}"(lds) : "memory");
}

// The same with 4 bytes per lane: lane i's word at base + off lands at LDS byte lds + 4 i.
__device__ __forceinline__ void dma4(const char* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, %1" : : "v"(off), "s"(base), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ uint32_t addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}

}  // namespace lds
}  // namespace mla
