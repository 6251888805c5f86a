// Device-side building blocks shared by the attention kernels (gfx950 / CDNA4).
//
// Layout facts used throughout (wave64, v_mfma_f32_32x32x16_bf16):
//   A operand  lane l holds A[l % 32][8 * (l / 32) + e], e = 0..7
//   B operand  lane l holds B[8 * (l / 32) + e][l % 32]
//   C/D        lane l, accumulator a (0..15) holds C[8 * (a / 4) + 4 * (l / 32) + a % 4][l % 32]
// v_mfma_f32_32x32x2_f32 uses the same C layout with A[l % 32][l / 32], B[l / 32][l % 32].
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element e (0..3) =
//   mem16[addr(lane 4 * e + i / 4) + i % 4]  — a 16x4 -> 4x16 transpose of the group's rows.
// v_permlane32_swap(x, x) returns {x[l], x[l ^ 32]} (in lane-dependent order).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum of a value with its partner in the other half of the wave (lane ^ 32)
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f32_32x32x2(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 4 x bf16 transposed read (see layout note above); `p` points into LDS.
__device__ __forceinline__ bf16x4 lds_read_tr4(const __bf16* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cvt_bf16x8(f32x8 x) { return __builtin_convertvector(x, bf16x8); }
__device__ __forceinline__ bf16x4 cvt_bf16x4(f32x4 x) { return __builtin_convertvector(x, bf16x4); }

}  // namespace swa
