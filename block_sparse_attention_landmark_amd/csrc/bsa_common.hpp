// Shared device helpers for the block-sparse landmark attention kernels (gfx950 / CDNA4).
//
// Conventions used by every kernel:
//  * tensors are contiguous and head-major: q [B,Hq,T,D], k/v [B,Hkv,T,D], landmarks
//    [B,Hkv,NB,D]; one 64-token block of one head is a contiguous 64*D*elem-size chunk;
//  * query head h belongs to kv group h / (Hq / Hkv);
//  * bf16 is handled as the clang __bf16 type (gfx950 converts with v_cvt_pk_bf16_f32, RNE);
//  * wave size is 64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

constexpr int kBlock = 64;      // tokens per key block / query block / chunk
constexpr int kWave = 64;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }
__device__ __forceinline__ bf16 f2bf(float x) { return (bf16)x; }

// Round a float64 value to the nearest bf16 (ties to even) in one step, without passing through
// float32 (which could round twice).  Finite inputs only; values here are far from overflow.
__device__ __forceinline__ bf16 f64_to_bf16_rne(double x) {
  uint64_t u = __double_as_longlong(x);
  // bf16 keeps the top 7 of float64's 52 fraction bits after renormalising the exponent; do the
  // rounding on the float64 bit pattern, then convert the exactly representable result.
  const uint64_t drop = 52 - 7;
  uint64_t lsb = (u >> drop) & 1ull;
  uint64_t bias = (1ull << (drop - 1)) - 1ull + lsb;
  uint64_t r = (u + bias) & ~((1ull << drop) - 1ull);
  // r is exactly representable in float32 and bf16 (subnormal bf16 results are not produced
  // by the workloads; they would be flushed by the float32 cast below)
  return (bf16)(float)__longlong_as_double(r);
}

// one 32x32x16 bf16 MFMA step: acc += A(32x16) * B(16x32)
//   A fragment: lane l holds A[m = l%32][k = 8*(l/32) .. +8]
//   B fragment: lane l holds B[k = 8*(l/32) .. +8][n = l%32]
//   acc:        lane l, register i holds C[m = 8*(i/4) + 4*(l/32) + i%4][n = l%32]
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Transposed 8-byte LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16 lanes, lane l
// receives element l%4 of the four-element chunks addressed by lanes 4e + (l%16)/4 of its group,
// for e = 0..3.  With lane s of a group pointing at row (base + (s%16)/4), columns 4*(s%4)..+3 of
// a row-major tile, lane l therefore gets column (l%16) of rows base..base+3: a column read.
__device__ __forceinline__ i16x4 lds_read_tr16(const bf16* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  typedef __attribute__((address_space(3))) bf16 lds_bf16;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_bf16*)p);
}

// Combine a value with the one held 32 lanes away (lanes l and l^32 hold the same query row in
// the MFMA layouts used here).  v_permlane32_swap exchanges the upper half of its first operand
// with the lower half of its second; given x twice, the two results hold x of both halves.
__device__ __forceinline__ float wave_max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the 64 lanes of a wave, the result in every lane, without LDS round trips: two DPP
// steps within quads (quad_perm [1,0,3,2], [2,3,0,1]), two rotations within 16-lane rows
// (row_ror 4, 8; each lane then holds its row's sum), and the four row sums read by readlane.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum64(float x) {
  x += dpp_f32<0xB1>(x);
  x += dpp_f32<0x4E>(x);
  x += dpp_f32<0x124>(x);
  x += dpp_f32<0x128>(x);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// log(sigmoid(x)) without overflow: min(x, 0) - log1p(exp(-|x|))
__device__ __forceinline__ float log_sigmoid(float x) {
  return fminf(x, 0.0f) - log1pf(expf(-fabsf(x)));
}

// order-preserving map from float to uint32 (larger float -> larger key); -0 and +0 differ,
// which is harmless: they never decide a top-K boundary differently from the float compare
// except between -0 and +0, whose scores are equal and then ordered by index by the caller.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f == 0.0f) u = 0u;  // fold -0 onto +0 so equal scores get equal keys
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

}  // namespace bsa
