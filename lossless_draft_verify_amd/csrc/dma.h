// LDS-DMA copies (global_load_lds) and the waits that go with them, for kernels that stream
// their operands through LDS stages without holding them in registers.
#pragma once

#include "device.h"

namespace dspark {

typedef __attribute__((address_space(3))) void lds_void;

// Copy 16 bytes per lane from global memory into LDS at byte address lds + 16 * lane (lds
// wave-uniform). Written as inline asm so that the compiler does not see an LDS-DMA write: it
// tracks those only coarsely and would put a full vmcnt(0) wait (every copy in flight) before
// each LDS read it cannot tell apart from the copies. The kernel orders copies and reads itself:
// wait_copies<n>() + s_barrier before a stage is read, lds_barrier() before it is overwritten;
// the "memory" clobbers keep the compiler's LDS reads between those points.
__device__ __forceinline__ void copy16_to_lds(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}
// Same, with the non-temporal hint, for operands read once per round (U slices, target rows):
// they then displace less of what is re-read every step (the W2 columns).
__device__ __forceinline__ void copy16_to_lds_nt(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(lds)
               : "memory", "m0");
}
// Same, 4 bytes per lane, to lds + 4 * lane.
__device__ __forceinline__ void copy4_to_lds(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)p));
}

// Copy a row of N 16-byte pieces from global memory to LDS (bytes lds .. lds + 16 N) with the
// lanes of one wave: lane l copies piece l, and piece 64 + l when N > 64.
template <int N>
__device__ __forceinline__ void copy_row_to_lds(const uint16_t* src, uint32_t lds, int lane) {
  static_assert(N <= 128, "at most two copies per lane");
  if (lane < N) copy16_to_lds(src + 8 * lane, lds);
  if constexpr (N > 64) {
    if (lane < N - 64) copy16_to_lds(src + 8 * (64 + lane), lds + 1024);
  }
}

template <int N>
__device__ __forceinline__ void wait_copies() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait_copies<Base + Step * k>() for a wave-uniform k in [0, K] (the count of copies a wave
// issued per stage when it varies at run time).
template <int Base, int Step, int K>
__device__ __forceinline__ void wait_copies_upto(int k) {
  if constexpr (K > 0) {
    if (k >= K) {
      wait_copies<Base + Step * K>();
      return;
    }
    wait_copies_upto<Base, Step, K - 1>(k);
  } else {
    wait_copies<Base>();
  }
}

// Value of lane l ^ 32 (v_permlane32_swap exchanges the two half-waves).
__device__ __forceinline__ float other_half(float x, int half) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(half ? r[0] : r[1]);
}

__device__ __forceinline__ double other_half(double x, int half) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const auto lo = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(u),
                                                   static_cast<uint32_t>(u), false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(u >> 32),
                                                   static_cast<uint32_t>(u >> 32), false, false);
  const uint64_t v = (static_cast<uint64_t>(half ? hi[0] : hi[1]) << 32) | (half ? lo[0] : lo[1]);
  return __longlong_as_double(static_cast<long long>(v));
}

}  // namespace dspark
