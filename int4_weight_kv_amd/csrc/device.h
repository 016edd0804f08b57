// Device helpers for the gfx950 kernels (wave64, bf16 MFMA).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "layout.h"

namespace futx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kMagic = 0x43004300u;  // bf16 pair (128, 128)
constexpr float kBias = 136.0f;           // 128 + nibble offset 8

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One word of 8 nibbles -> 8 bf16 operand elements with values 136 + code.
__device__ __forceinline__ bf16x8 widen_word(uint32_t w) {
  u32x4 r;
  r.x = (w & 0x000F000Fu) | kMagic;
  r.y = ((w >> 4) & 0x000F000Fu) | kMagic;
  r.z = ((w >> 8) & 0x000F000Fu) | kMagic;
  r.w = ((w >> 12) & 0x000F000Fu) | kMagic;
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  u32x4 r = {v.x, v.y, v.z, v.w};
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ uint32_t word_of(uint4 v, int s) {
  return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace futx
