// Device-side helpers for gfx950: bf16 bit conversions, MFMA operand types, wave sums.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// float32 -> bfloat16, round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two float32 -> bfloat16 with the conversion instruction (round to nearest, ties to even),
// packed a | b << 16.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, h2));
}

// a = hi + lo (and b) in bfloat16 to about 16 bits: hi the nearest bfloat16, lo the nearest
// bfloat16 to the exact remainder; both pairs packed as in cvt_pk_bf16.
__device__ __forceinline__ void split_bf16_pk(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = cvt_pk_bf16(a, b);
  lo = cvt_pk_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// Row m of a 32-row MFMA operand block -> channel within the block, chosen so that the
// 16 accumulator registers of lane l of a 32x32 result hold 16 consecutive channels
// (16 * (l / 32) + i).  The result layout of the 32x32 MFMAs puts register i of lane l
// at row 8 * (i / 4) + 4 * (l / 32) + (i % 4); inverting that gives this bijection.
__device__ __forceinline__ int cmap32(int m) {
  return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sum over the 32 lanes that share bit 5 of the lane id (one half of the wave).
__device__ __forceinline__ float half_wave_sum(float v) {
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// bf16 MFMA 32x32x16 (gfx950): a, b carry 8 consecutive k per lane; k group = lane / 32.
__device__ __forceinline__ floatx16 mfma_bf16(const u32x4& a, const u32x4& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp32 MFMA 32x32x2: one k per lane, k = lane / 32.
__device__ __forceinline__ floatx16 mfma_f32(float a, float b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

}  // namespace kvc
