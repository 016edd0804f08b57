// Device helpers for the gfx950 kernels (wave64, bf16 MFMA).
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "layout.h"

namespace futx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kMagic = 0x41804180u;  // bf16 pair (16, 16): exponent 2^4
constexpr uint32_t kNibMask = 0x00780078u; // mantissa bits 3..6 of both halves
constexpr float kBias = 24.0f;             // 16 + nibble offset 8

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16h(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// One word of 8 nibbles -> 8 bf16 operand elements with values 24 + code
// (encoding in layout.h).
__device__ __forceinline__ bf16x8 widen_word(uint32_t w) {
  u32x4 r;
  r.x = (w & kNibMask) | kMagic;
  r.y = ((w >> 4) & kNibMask) | kMagic;
  r.z = ((w >> 8) & kNibMask) | kMagic;
  r.w = (__builtin_amdgcn_alignbit(w, w, 12) & kNibMask) | kMagic;
  return __builtin_bit_cast(bf16x8, r);
}

// The same word -> 8 fp16 elements equal to the signed codes exactly: the
// nibble widens to fp16 128 + n (exponent 2^7, mantissa bits 3..6) and one
// packed fp16 subtraction of 136 per pair leaves code = n - 8, which is
// exactly representable.  Used where the operand offset must not enter the
// fp32 accumulation (attention).
// widen_word with three shifts and four 3-operand and-or ops (7 VALU ops per
// word).  gfx9 VOP3 encodings take no literal operand, so with the mask and
// magic as literals the compiler emits a separate and + or; the caller
// passes them as opaque registers (mask scalar, magic vector: one scalar
// operand per instruction), made with nib_regs().  No instruction is written
// in inline asm: the compiler must see every VALU write that feeds a matrix
// core instruction to insert its wait states.
struct NibRegs {
  uint32_t mask, magic;
};
__device__ __forceinline__ NibRegs nib_regs() {
  NibRegs r{kNibMask, kMagic};
  asm volatile("" : "+s"(r.mask));  // no instruction: hides the constant
  asm volatile("" : "+v"(r.magic));
  return r;
}
__device__ __forceinline__ bf16x8 widen_word_fast(uint32_t w, NibRegs k) {
  u32x4 r;
  r.x = (w & k.mask) | k.magic;
  r.y = ((w >> 4) & k.mask) | k.magic;
  r.z = ((w >> 8) & k.mask) | k.magic;
  r.w = (__builtin_amdgcn_alignbit(w, w, 12) & k.mask) | k.magic;
  return __builtin_bit_cast(bf16x8, r);
}

// The same widening to exact fp16 codes: (n | 128-exponent) is the fp16
// value 128 + n = 136 + code, and one packed fp16 subtraction of 136 per
// pair leaves the code itself.  The mask and the magic constant sit in
// registers (nib_regs_f16()), so each pair takes one v_and_or_b32: a VOP3
// instruction on gfx950 cannot carry literal constants, and with literals
// the AND and the OR would be two instructions.
__device__ __forceinline__ NibRegs nib_regs_f16() {
  NibRegs r{kNibMask, 0x58005800u};
  asm volatile("" : "+s"(r.mask));  // no instruction: hides the constant
  asm volatile("" : "+v"(r.magic));
  return r;
}
__device__ __forceinline__ f16x8 widen_word_exact_f16(uint32_t w, NibRegs k) {
  u32x4 r;
  r.x = (w & k.mask) | k.magic;
  r.y = ((w >> 4) & k.mask) | k.magic;
  r.z = ((w >> 8) & k.mask) | k.magic;
  r.w = (__builtin_amdgcn_alignbit(w, w, 12) & k.mask) | k.magic;
  const f16x8 v = __builtin_bit_cast(f16x8, r);
  return v - (f16x8)(_Float16)136.0f;
}

__device__ __forceinline__ uint32_t rotl_dev(uint32_t x, int r) {
  r &= 31;
  return r ? __builtin_amdgcn_alignbit(x, x, 32 - r) : x;
}

// element e of a word holding nibble n, other bits zero
__device__ __forceinline__ uint32_t nibble_bits(int e, uint32_t n) {
  return rotl_dev(n << 3, 4 * (e >> 1) + 16 * (e & 1));
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

// fp32 -> bf16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// two fp32 -> packed bf16 pair (a in the low half), round to nearest even
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}

// The value held by lane ^ LB (LB = 16 or 32), for every lane, through the
// gfx950 cross-row swaps instead of an LDS permute.  With both operands x,
// v_permlane16_swap returns, for each pair of 16-lane rows, x of the even
// row in its first result and x of the odd row in its second (in every lane
// of the pair); v_permlane32_swap does the same for the lower and upper 32
// lanes (checked lane by lane on MI355X).
template <int LB>
__device__ __forceinline__ float xor_lanes(float v) {
  static_assert(LB == 16 || LB == 32, "rows of 16 or halves of 32 lanes");
  const uint32_t x = __float_as_uint(v);
  const bool upper = (threadIdx.x & LB) != 0;
  if constexpr (LB == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return __uint_as_float(upper ? r[0] : r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return __uint_as_float(upper ? r[0] : r[1]);
  }
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

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Cross-lane moves within a row of 16 lanes through the DPP modifier (a VALU
// operand form: no LDS round trip).  Controls: quad_perm [1,0,3,2] and
// [2,3,0,1] swap neighbours at distance 1 and 2; row_half_mirror maps lane i
// of each 8 to 7 - i, row_mirror lane i of 16 to 15 - i.
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}

// Sum over aligned groups of N consecutive lanes (N = 1, 2, 4, 8 or 16); every
// lane of a group gets the group's sum.  After the two quad steps all lanes
// of a quad hold its sum, so each mirror step adds the partner quad's (or
// half-row's) sum: the same pairing as an xor butterfly, hence the same value
// in every lane.
template <int N, typename T>
__device__ __forceinline__ T group_sum(T v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group of 1..16 lanes");
  auto mv = [](auto ctrl, T x) -> T {
    if constexpr (sizeof(T) == 8) return dpp_f64<decltype(ctrl)::value>(x);
    else return dpp_f32<decltype(ctrl)::value>(x);
  };
  if constexpr (N >= 2) v += mv(std::integral_constant<int, kDppQuadXor1>{}, v);
  if constexpr (N >= 4) v += mv(std::integral_constant<int, kDppQuadXor2>{}, v);
  if constexpr (N >= 8) v += mv(std::integral_constant<int, kDppHalfMirror>{}, v);
  if constexpr (N >= 16) v += mv(std::integral_constant<int, kDppMirror>{}, v);
  return v;
}

// An fp64 value as an unevaluated fp32 pair hi + lo.  Sums of bf16 operands
// are formed exactly in fp64 and carried as such pairs, so that removing the
// nibble offset (24 * sum) costs two fp32 FMAs and no precision.
__device__ __forceinline__ float2 split_f64(double v) {
  const float hi = (float)v;
  return float2{hi, (float)(v - (double)hi)};
}

// d - 24 * (hi + lo) with one rounding per step
__device__ __forceinline__ float remove_offset(float d, float2 s) {
  return fmaf(-kBias, s.y, fmaf(-kBias, s.x, d));
}

}  // namespace futx
