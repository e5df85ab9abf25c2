// Direct-to-LDS global loads (global_load_lds_dwordx4) issued from inline assembly, and the
// explicit vmcnt waits that go with them. Shared by the GEMM and matvec kernels.
//
//  * One load moves 16 bytes per lane from (base + voff) into LDS at (lds_addr + 16 * lane): a
//    wave's load fills 1024 contiguous LDS bytes.
//  * The compiler cannot see which LDS bytes such a load writes; issuing it through the builtin
//    makes it wait for every outstanding load before any LDS read. From inline assembly it is
//    invisible to the compiler's wait insertion, so the kernel waits for it explicitly with
//    s_waitcnt vmcnt(N): vector memory loads complete in issue order, so vmcnt <= N means that
//    all but the N most recent loads (of any kind) have landed. Loads the compiler issues itself
//    only make such waits stricter, and the compiler's own waits for them can only over-wait.
//  * The destination is LDS only: no register is written by an unfinished load.
//  * M0 is listed as clobbered; the compiler keeps it reserved and does not otherwise use it in
//    these kernels (checked in the generated code).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

// A pointer every lane holds the same value of, moved to scalar registers.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// kStream marks bytes read once per launch (a matvec's weights): the load carries the nt
// (non-temporal) hint, so the caches favour keeping the data workgroups re-read, such as the
// activations.
template <bool kStream = false>
__device__ __forceinline__ void load_lds16(const void* base, uint32_t voff, uint32_t lds_addr) {
  if constexpr (kStream) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %0, %1 nt"
        :
        : "v"(voff), "s"(uniform_ptr(base)), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
        : "memory", "m0");
  } else {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(uniform_ptr(base)), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
        : "memory", "m0");
  }
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Waits until at most PER * min(later, L) of this wave's loads are outstanding: the loads of
// `later` groups of PER loads issued after the group being waited for stay in flight.
template <int PER, int L>
__device__ __forceinline__ void wait_groups(int later) {
  if constexpr (L == 0) {
    wait_vmcnt<0>();
  } else {
    if (later >= L) wait_vmcnt<PER * L>();
    else wait_groups<PER, L - 1>(later);
  }
}

// Waits until at most n (wave-uniform, 0 <= n) of this wave's loads are outstanding, for n known
// only at run time: takes the largest immediate not above n (n above MAX waits for MAX).
template <int MAX>
__device__ __forceinline__ void wait_at_most(int n) {
  if constexpr (MAX == 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= MAX) wait_vmcnt<MAX>();
    else wait_at_most<MAX - 1>(n);
  }
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const void __attribute__((address_space(3)))*)p));
}

}  // namespace wq
