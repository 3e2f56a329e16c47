// Device helpers shared by the libspear_ec kernels (gfx950 / CDNA4).
//
// Integer-code operands.  The matrix cores take bf16 operands.  An int4 code c
// is turned into the bf16 value 128 + c with one bit operation: 0x4300 is
// 128.0 in bf16 and the low 7 mantissa bits then count units, so OR-ing a
// nibble into them gives 128 + c exactly.  Eight codes of a 32-bit word become
// four packed bf16 pairs with four AND-OR operations and three shifts.  The
// products (128 + c) * x are exact in fp32; the offset is removed with the
// per-block sums of x:
//     sum_k (c_k - z) x_k = sum_k (128 + c_k) x_k - (128 + z) * sum_k x_k,
// and the group scale s is applied in fp32.  Nothing is rounded to bf16 on
// the weight side, so the dequantized weight the layer sees is the exact
// (c - z) * s of the format.
//
// K order.  The pairs built from a word hold columns (0,4), (1,5), (2,6),
// (3,7) of its eight, so a matrix-core operand carries the columns of an
// 8-column block in the order 0,4,1,5,2,6,3,7.  A dot product does not depend
// on the order of its terms, so the activations are permuted the same way
// (x_permute8) and the packed weights keep their canonical layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spear {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kBf16Offset128 = 0x43004300u;  // bf16 pair (128.0, 128.0)
constexpr uint32_t kBf16One = 0x3F803F80u;        // bf16 pair (1.0, 1.0)

// Eight codes (nibble j = column j of the block) -> bf16 pairs of 128 + c in
// the operand order 0,4,1,5,2,6,3,7.
__device__ __forceinline__ u32x4 codes_to_bf16_offset(uint32_t w) {
  const uint32_t m = 0x000F000Fu;
  u32x4 o;
  o.x = (w & m) | kBf16Offset128;
  o.y = ((w >> 4) & m) | kBf16Offset128;
  o.z = ((w >> 8) & m) | kBf16Offset128;
  o.w = ((w >> 12) & m) | kBf16Offset128;
  return o;
}

// Eight consecutive bf16 activations (packed in 4 words) -> the same operand
// order 0,4,1,5,2,6,3,7 as codes_to_bf16_offset.
__device__ __forceinline__ u32x4 x_permute8(u32x4 d) {
  u32x4 o;
  o.x = (d.x & 0xFFFFu) | (d.z << 16);
  o.y = (d.x >> 16) | (d.z & 0xFFFF0000u);
  o.z = (d.y & 0xFFFFu) | (d.w << 16);
  o.w = (d.y >> 16) | (d.w & 0xFFFF0000u);
  return o;
}

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Logistic function in the form whose exp() argument is never positive.
__device__ __forceinline__ float sigmoidf_safe(float z) {
  if (z >= 0.f) return 1.f / (1.f + expf(-z));
  const float e = expf(z);
  return e / (1.f + e);
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

}  // namespace spear
