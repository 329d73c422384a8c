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

}  // namespace bsa
