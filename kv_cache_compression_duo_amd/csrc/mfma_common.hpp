// Matrix-core helpers shared by the flash kernel and the grouped-query decode:
// operand types of v_mfma_f32_32x32x16_bf16 / _f16, the element-generic
// product, row sums of packed softmax weights and the transposed LDS reads
// that turn row-major V tiles into V^T operands.
#pragma once
#include <type_traits>

#include "device_common.hpp"

namespace duo {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Element-generic pieces: the kernels take K/V tiles (and P) as bf16, or as
// fp16 for layers with an fp16 or 4-bit cache (Q, given as bf16, is converted;
// every bf16 value with a normal fp16 exponent converts exactly).
template <bool F16>
using elem8 = std::conditional_t<F16, f16x8, bf16x8>;
template <bool F16>
__device__ __forceinline__ elem8<F16> as_elem8(const u32x4& v) {
  return __builtin_bit_cast(elem8<F16>, v);
}
__device__ __forceinline__ f32x16 mma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma32(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// c + a.x + a.y for a pair of softmax weights (v_dot2c against ones)
__device__ __forceinline__ float add_pair(bf16x2 a, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, bf16x2{(__bf16)1.0f, (__bf16)1.0f}, c, false);
}
__device__ __forceinline__ float add_pair(f16x2 a, float c) {
  return __builtin_amdgcn_fdot2(a, f16x2{(_Float16)1.0f, (_Float16)1.0f}, c, false);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ __attribute__((address_space(3))) void* lds_ptr(const void* p) {
  return (__attribute__((address_space(3))) void*)(const_cast<void*>(p));
}

// Two transposed 8-byte LDS reads (ds_read_b64_tr_b16) joined into one MFMA
// operand. In each group of 16 lanes, lane i receives element i % 4 of the
// 4-element chunks read by lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4:
// when lane c reads row c / 4 (of four consecutive rows) at columns
// 4 (c % 4) .. 4 (c % 4) + 3 of a 16-column strip, lane i gets column i of
// the four rows.
__device__ __forceinline__ bf16x8 lds_tr_pair(const char* lo, const char* hi) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<char*>(lo)));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<char*>(hi)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace duo
