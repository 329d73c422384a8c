// Helpers shared by the attention kernels (prefill, decode, float32 path).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsa_common.hpp"

namespace bsa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Number of valid entries in an attended-set row (the valid entries form a prefix; -1 pads).
// Each lane of the wave reads one entry, so a row costs one load per 64 entries instead of a
// chain of dependent loads.
__device__ __forceinline__ int count_valid(const int32_t* row, int NA) {
  const int lane = threadIdx.x % kWave;
  int n = 0;
  for (int i0 = 0; i0 < NA; i0 += kWave) {
    const int i = i0 + lane;
    const bool ok = i < NA && row[i] >= 0;
    const int cnt = __popcll(__ballot(ok));
    n += cnt;
    if (cnt < kWave) break;
  }
  return n;
}

// One copy from global memory straight into LDS, BYTES (4 or 16) per lane: lane l's bytes at
// gbase + voff land at LDS byte address lds_addr + BYTES * l (gbase and lds_addr wave-uniform;
// lanes outside the exec mask copy nothing).  Issued as inline assembly so the compiler does not
// treat the copy as an LDS write of unknown extent: its own tracking would otherwise wait for
// every copy in flight before each LDS read and at each barrier, which defeats copying several
// blocks ahead.  Completion is the caller's business (vmcnt); M0 is saved and restored around
// the copy.
template <int BYTES>
__device__ __forceinline__ void dma_lds(const char* gbase, uint32_t voff, uint32_t lds_addr) {
  static_assert(BYTES == 4 || BYTES == 16, "global_load_lds moves 4 or 16 bytes per lane here");
#if defined(__HIP_DEVICE_COMPILE__)
  // both addresses are wave-uniform; make that explicit so they live in scalar registers
  // (readfirstlane returns int: widen through uint32_t so the low half is not sign-extended)
  const uint32_t la = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr);
  const uint64_t ga = (uint64_t)(uintptr_t)gbase;
  const uint32_t g_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(ga >> 32));
  const uint32_t g_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)ga);
  const uint64_t gs = ((uint64_t)g_hi << 32) | (uint64_t)g_lo;
  uint32_t saved;
#if defined(BSA_SYNC_COPIES)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#endif
  if constexpr (BYTES == 16)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(la), "v"(voff), "s"(gs)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(la), "v"(voff), "s"(gs)
        : "memory");
#if defined(BSA_SYNC_COPIES)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#endif
#endif
}

// Race-check build (compiled with -DBSA_SYNC_COPIES, as libbsa_sync.so): every direct-to-LDS
// copy first waits for all of its wave's LDS reads in flight and then for its own completion, so
// no copy can overwrite a tile that the wave is still reading nor be read before it lands; the
// kernels whose waves all issue the same copies add a workgroup barrier on both sides as well
// (sync_copies_barrier).  The normal build must give the same bits.
__device__ __forceinline__ void sync_copies_barrier() {
#if defined(BSA_SYNC_COPIES)
  __syncthreads();
#endif
}

// LDS byte address of a shared-memory pointer
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

}  // namespace bsa
