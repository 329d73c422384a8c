// Measured ceilings of the GPU for the two bounds the attention kernels are priced against, used
// by the benchmark beside the vendor peaks: the bf16 matrix-core rate (back-to-back 32x32x16
// MFMAs on independent accumulators) and the rate of gathering random 16 KB blocks straight from
// HBM into LDS (the access pattern of the kernels' K/V staging).  Built as its own library
// (libbsa_peak.so); not part of the attention path or of its C ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attend_common.hpp"

namespace bsa {
namespace {

constexpr int kPeakMfmaThreads = 256;   // one wave per SIMD of a CU
constexpr int kPeakGatherWaves = 4;
constexpr int kPeakGatherRing = 2;      // 16 KB blocks in flight per wave
constexpr int kPeakBlockBytes = 16384;

__global__ __launch_bounds__(kPeakMfmaThreads) void peak_mfma_kernel(float* out, int iters) {
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.0f;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = f2bf(1e-3f * (float)(threadIdx.x % 13));
    b[i] = f2bf(1e-3f * (float)i);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j % 4] = mfma32(a, b, acc[j % 4]);
  }
  float r = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) r += acc[j][i];
  out[blockIdx.x * kPeakMfmaThreads + threadIdx.x] = r;
}

__device__ __forceinline__ uint32_t peak_hash(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t h = a * 0x9E3779B1u ^ (b + 0x7F4A7C15u) * 0x85EBCA77u ^ (c + 0x165667B1u) * 0xC2B2AE3Du;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  h *= 0x297A2D39u;
  h ^= h >> 15;
  return h;
}

// each wave copies blocks_per_wave pseudo-random 16 KB blocks of src (n_blocks of them) into a
// ring of kPeakGatherRing block slots of its own LDS; a slot is reused once its copy has landed
__global__ __launch_bounds__(kPeakGatherWaves * 64) void peak_gather_kernel(
    const char* __restrict__ src, uint32_t n_blocks, int blocks_per_wave, unsigned* out) {
  __shared__ __attribute__((aligned(16))) char ring[kPeakGatherWaves * kPeakGatherRing * kPeakBlockBytes];
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const uint32_t base = lds_addr_of(ring) + (uint32_t)(w * kPeakGatherRing * kPeakBlockBytes);
  for (int t = 0; t < blocks_per_wave; ++t) {
    // at most kPeakGatherRing - 1 blocks (16 copies each) may still be in flight
    constexpr int kLeft = (kPeakGatherRing - 1) * 16;
    if (t >= kPeakGatherRing) __builtin_amdgcn_s_waitcnt(0x0F70 | (kLeft & 15) | ((kLeft >> 4) << 14));
    const uint32_t blk = peak_hash(blockIdx.x, (uint32_t)w, (uint32_t)t) % n_blocks;
    const char* g = src + (size_t)blk * kPeakBlockBytes;
    const uint32_t slot = base + (uint32_t)((t % kPeakGatherRing) * kPeakBlockBytes);
#pragma unroll
    for (int i = 0; i < kPeakBlockBytes / 1024; ++i)
      dma_lds<16>(g, (uint32_t)(i * 1024 + lane * 16), slot + (uint32_t)(i * 1024));
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  out[blockIdx.x * kPeakGatherWaves * 64 + threadIdx.x] =
      *reinterpret_cast<const unsigned*>(ring + threadIdx.x * 16);
}

static_assert((kPeakGatherRing - 1) * 16 <= 63, "the wait count must fit vmcnt");

}  // namespace
}  // namespace bsa

extern "C" {

// n_wg workgroups of 256 threads, each wave issuing iters x 16 MFMAs (32x32x16 bf16, 32768
// flops each); out holds n_wg * 256 floats.  Asynchronous on st.
hipError_t bsa_peak_mfma(float* out, int n_wg, int iters, hipStream_t st) {
  if (out == nullptr || n_wg <= 0 || iters <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bsa::peak_mfma_kernel, dim3(n_wg), dim3(bsa::kPeakMfmaThreads), 0, st, out,
                     iters);
  return hipGetLastError();
}

// n_wg workgroups of 4 waves, each wave copying blocks_per_wave random 16 KB blocks of src
// (n_blocks x 16 KB bytes, device memory) into LDS; out holds n_wg * 256 unsigned.
// Asynchronous on st.
hipError_t bsa_peak_gather(const void* src, uint32_t n_blocks, int n_wg, int blocks_per_wave,
                           unsigned* out, hipStream_t st) {
  if (src == nullptr || out == nullptr || n_blocks == 0 || n_wg <= 0 || blocks_per_wave <= 0)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(bsa::peak_gather_kernel, dim3(n_wg), dim3(bsa::kPeakGatherWaves * 64), 0, st,
                     static_cast<const char*>(src), n_blocks, blocks_per_wave, out);
  return hipGetLastError();
}

}  // extern "C"
