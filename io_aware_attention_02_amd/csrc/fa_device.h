// fa_device.h -- device-side building blocks for the gfx950 attention kernels.
//
// Vector types that map onto the CDNA4 matrix-core operands, thin wrappers over the MFMA
// builtins, lane-exchange helpers and bf16 packing.  Only kernel sources include this file.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// D[32x32] += A[32x16] * B[16x32], bf16 in, fp32 accumulate.  Lane l holds A row (l & 31)
// and B column (l & 31), k-slots 8*(l >> 5) .. +7.  Output lane l holds column (l & 31),
// rows 8*(r >> 2) + 4*(l >> 5) + (r & 3) for r = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D[16x16] += A[16x32] * B[32x16].  Lane l holds A row (l & 15) / B column (l & 15),
// k-slots 8*(l >> 4) .. +7.  Output lane l holds column (l & 15), rows 4*(l >> 4) + r.
__device__ __forceinline__ f32x4 mfma16k32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D[16x16] += A[16x16] * B[16x16].  Lane l holds A row (l & 15) / B column (l & 15),
// k-slots 4*(l >> 4) .. +3.  Output as for mfma16k32.
__device__ __forceinline__ f32x4 mfma16k16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Combine a value with the one held by lane l ^ 32 (v_permlane32_swap exchanges the upper
// half-wave of its first operand with the lower half-wave of its second; with both operands
// equal, the two results hold {own, partner} in some order, so max/add of them is symmetric).
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Exchange with lane l ^ 16 through the LDS crossbar (used off the hot loop).
__device__ __forceinline__ float shfl_xor(float x, int mask) {
  return __shfl_xor(x, mask, 64);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* x) {
  u32x4 u;
  u[0] = pack_bf16x2(x[0], x[1]);
  u[1] = pack_bf16x2(x[2], x[3]);
  u[2] = pack_bf16x2(x[4], x[5]);
  u[3] = pack_bf16x2(x[6], x[7]);
  return __builtin_bit_cast(bf16x8, u);
}

// Workgroup id -> logical work index, so that consecutive logical indices run on the same XCD.
// Workgroups are dispatched round-robin over the 8 XCDs (id % 8); logical index ranges of
// about total/8 are given to one XCD each, so tiles that share K/V share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int w, int total) {
  constexpr int kXcd = 8;
  const int q = total / kXcd, r = total % kXcd;
  const int xcd = w % kXcd, slot = w / kXcd;
  return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

}  // namespace fa
