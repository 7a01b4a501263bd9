// Direct-to-LDS streaming helpers shared by the pipelined GEMMs: buffer
// resources, buffer_load ... lds wrappers, the vmcnt + barrier step fence, the
// LDS row swizzle and the per-sub-step instruction-order hint.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace moe {

typedef __attribute__((address_space(3))) char lds_char;

// 16 (dma16) or 4 (dma4) bytes per lane from a buffer straight into LDS at
// dst + size * lane; offsets past the buffer's range write zeros and move no
// data.  Kept out of the kernel templates: the host pass drops a kernel
// template whose body names this builtin.
__device__ __attribute__((always_inline)) inline void dma16(__amdgpu_buffer_rsrc_t r, lds_char* dst, uint32_t voff,
                                                            uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}
__device__ __attribute__((always_inline)) inline void dma4(__amdgpu_buffer_rsrc_t r, lds_char* dst, uint32_t voff,
                                                           uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, voff, soff, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes >= 0x7fffffffLL ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// Wait until at most n vector-memory operations of this wave are in flight,
// then meet the other waves at the barrier.  The asm block is also a compiler
// barrier for memory operations.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// XOR swizzle of the 16-byte chunk index of row r: conflict-free 128-bit reads
// of 8 and of 16 consecutive rows at one logical chunk.
template <int ROW>
__device__ __forceinline__ int swz(int r) {
  if constexpr (ROW == 64) return ((r >> 1) ^ (r >> 3)) & 3;
  else return (r & 7) ^ ((r >> 3) & 1);
}

// Instruction-order hint for one sub-step: MS MFMAs, with RS LDS reads (for the
// next sub-step) after the first RS of them and VS ring DMAs spread evenly.
template <int Q, int MS, int RS, int VS>
__device__ __forceinline__ void sub_schedule() {
  if constexpr (Q < MS) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                        // one MFMA
    if constexpr (Q < RS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one next-sub-step read
    constexpr int DE = VS > 0 ? (MS / VS > 0 ? MS / VS : 1) : 1;
    if constexpr (VS > 0 && (Q + 1) % DE == 0 && (Q + 1) / DE <= VS) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    sub_schedule<Q + 1, MS, RS, VS>();
  } else if constexpr (RS > MS) {
    __builtin_amdgcn_sched_group_barrier(0x100, RS - MS, 0);
  }
}

// Host side: opt kernel Kern into `bytes` of dynamic LDS, once per device (the
// attribute is kept per device; 64 devices at most are remembered).
template <auto Kern>
hipError_t allow_lds(int bytes) {
  static std::atomic<uint64_t> done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute((const void*)Kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

}  // namespace moe
