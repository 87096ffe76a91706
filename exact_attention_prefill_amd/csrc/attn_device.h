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

// Work-item and workgroup indices from the compiler's builtins.  HIP's threadIdx and
// blockIdx read them through device-library functions that are compiled with the
// default IEEE mode; this library is compiled with it off (-mno-amdgpu-ieee), and the
// inliner does not inline across that difference, which would leave real calls (and a
// stack) at every kernel's entry.  Grid sizes come from each kernel's parameters.
__device__ __forceinline__ int thread_x() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ int group_x() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int group_y() { return (int)__builtin_amdgcn_workgroup_id_y(); }
__device__ __forceinline__ int group_z() { return (int)__builtin_amdgcn_workgroup_id_z(); }

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

// ---- LDS staging and cross-lane helpers shared by the attention kernels ----

// LDS row pitch of a staged K/V tile: rows of d = 32 and d = 96 are padded to the
// pitch of d = 64 and d = 128, so every head size uses one of two swizzle families
// (rows of 128 bytes, or a multiple of 256).
template <int D>
constexpr int lds_row_bytes() {
  return D == 32 ? 128 : D == 96 ? 256 : 2 * D;
}

// s_waitcnt immediate that waits until at most n vector-memory operations of this
// wave are outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt at their "no wait" maxima).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// ... until every LDS operation of this wave has completed (vmcnt and expcnt not waited).
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t* lds_base, uint32_t byte_off) {
  const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) char*)lds_base + byte_off));
  return __builtin_bit_cast(u32x2, t);
}

__device__ __forceinline__ u32x4 lds_read_b128(const uint16_t* lds_base, uint32_t byte_off) {
  return *(const u32x4*)((const char*)lds_base + byte_off);
}

// One 16-byte-per-lane buffer load that writes LDS directly: lane i's 16 bytes from
// rsrc + voff land at LDS byte address lds_addr + 16 i.  Issued from inline assembly
// so the compiler does not track it: its own tracking cannot tell which LDS array a
// transpose read touches and would drain every load in flight before each such read.
// A kernel using it orders these loads itself: every buffer is read only after an
// s_waitcnt vmcnt(0) and a barrier that follow the loads into it, and is reloaded
// only after a barrier that follows every read of it.
// m0 is a reserved register that nothing else in these kernels reads or writes; the
// clobber records that the assembly overwrites it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const u32x4& rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %0, 0 offen lds"
      :
      : "s"(rsrc), "v"(voff), "s"(lds_addr)
      : "memory", "m0");
}
// The same with 4 bytes per lane: lane i's dword lands at lds_addr + 4 i.
__device__ __forceinline__ void lds_dma4(const u32x4& rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %0, 0 offen lds"
      :
      : "s"(rsrc), "v"(voff), "s"(lds_addr)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// Raw buffer descriptor over [base, base + nrec): stride 0, dword format; offsets at or
// past nrec read nothing.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t nrec) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return (u32x4){(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, nrec, 0x00020000u};
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// max(x, x of the lane 32 apart) and the sum likewise, from one v_permlane32_swap:
// it returns (x with its upper half replaced by the partner's lower half, and the
// partner half's view), so the two results hold {x, partner} in some order.
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row sum of packed 16-bit P pairs: sum += lo + hi (v_dot2 with (1, 1)).
template <int DT>
__device__ __forceinline__ float add_pair(uint32_t pair, float acc);
template <>
__device__ __forceinline__ float add_pair<DT_BF16>(uint32_t pair, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                         acc, false);
}
template <>
__device__ __forceinline__ float add_pair<DT_F16>(uint32_t pair, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), __builtin_bit_cast(f16x2, 0x3c003c00u), acc, false);
}


}  // namespace attn
