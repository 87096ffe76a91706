// Device-side helpers shared by the gfx950 attention kernels: vector types, the
// 32x32x16 MFMA wrappers for fp16/bf16 inputs with fp32 accumulation, and
// fp32 -> 16-bit packing with round-to-nearest-even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum { DT_F16 = 0, DT_BF16 = 1 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// acc += A * B for a 32x32 output block and a 16-deep contraction.  Each lane holds
// eight 16-bit elements of A and of B; the lane -> (row, k) assignment is the
// hardware's, and only needs to be the same for A and B.
template <int DT>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 acc);

template <>
__device__ __forceinline__ f32x16 mfma32x32x16<DT_BF16>(u32x4 a, u32x4 b, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x16 mfma32x32x16<DT_F16>(u32x4 a, u32x4 b, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc, 0,
                                                0, 0);
}

// Two fp32 values -> one dword of two 16-bit values (lo = x, hi = y), nearest-even.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float x, float y);

template <>
__device__ __forceinline__ uint32_t pack2<DT_BF16>(float x, float y) {
  bf16x2 v;
  v[0] = (__bf16)x;
  v[1] = (__bf16)y;
  return __builtin_bit_cast(uint32_t, v);
}

template <>
__device__ __forceinline__ uint32_t pack2<DT_F16>(float x, float y) {
  f16x2 v;
  v[0] = (_Float16)x;
  v[1] = (_Float16)y;
  return __builtin_bit_cast(uint32_t, v);
}

// 16-bit storage value -> fp32 (exact).
template <int DT>
__device__ __forceinline__ float to_f32(uint32_t bits16);

template <>
__device__ __forceinline__ float to_f32<DT_BF16>(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

template <>
__device__ __forceinline__ float to_f32<DT_F16>(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace attn
