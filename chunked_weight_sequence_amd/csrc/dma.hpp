// Direct copies from global memory into LDS, and waits on them, for gfx950.
//
// global_load_lds_dwordx4 moves 16 bytes per lane from any global address straight into LDS:
// lane l's bytes land at M0 + 16 * l (M0 wave-uniform). No registers hold the data on the way,
// so a kernel can keep several copies in flight per wave. The vector-memory counter (vmcnt)
// covers these copies together with ordinary vector loads and stores and counts them in issue
// order, so a wait for a given copy names how many of the wave's operations were issued after
// it; waiting with a smaller count only waits longer.
#pragma once

#include <stdint.h>

#include <type_traits>
#include <utility>

#include <hip/hip_runtime.h>

namespace ttt {

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}

// One 16-byte-per-lane copy into LDS at m0 + 16 * lane from sbase + voff (sbase and m0
// wave-uniform). M0 is written in the same statement; nothing else in these kernels uses it.
__device__ __forceinline__ void dma16(uint32_t voff, const char* sbase, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(m0));
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// s_waitcnt needs an immediate: wait with the largest listed count not above n (a smaller count
// only waits longer). The lists hold the counts a kernel's steady state and tail produce.
template <int... V>
struct WaitList;
template <>
struct WaitList<> {
  __device__ __forceinline__ static void wait(int) { wait_vm<0>(); }
};
template <int V0, int... V>
struct WaitList<V0, V...> {
  __device__ __forceinline__ static void wait(int n) {
    if (n >= V0) wait_vm<V0>();
    else WaitList<V...>::wait(n);
  }
};
// The steady-state counts first, by equality (one compare each), then the rounding list.
template <class Common, class Rest>
struct WaitFast;
template <int... C, class Rest>
struct WaitFast<std::integer_sequence<int, C...>, Rest> {
  __device__ __forceinline__ static void wait(int n) {
    bool done = false;
    ((!done && n == C ? (wait_vm<C>(), done = true) : false), ...);
    if (!done) Rest::wait(n);
  }
};
}  // namespace ttt
