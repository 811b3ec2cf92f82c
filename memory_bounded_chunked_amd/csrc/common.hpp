// Shared device-side types and helpers for the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

enum DType : int { F32 = 0, BF16 = 1, W8_BF16 = 2 };

// bf16 <-> fp32. The hardware conversion (v_cvt_pk_bf16_f32) rounds to
// nearest even; it is what a (__bf16) cast lowers to on gfx950.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
// Two fp32 -> packed pair of bf16 (low half = a), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// 32x32x16 bf16 MFMA, fp32 accumulate. Operand lane layout (checked on gfx950):
// lane l supplies A[m = l%32][k = 8*(l/32) .. +7] and B[k = 8*(l/32) .. +7][n = l%32];
// result register r of lane l is C[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 32x32x2 fp32 MFMA: lane l supplies A[l%32][l/32], B[l/32][l%32]; same C layout.
__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Workgroups are dealt round-robin to the 8 XCDs (each with its own L2):
// hardware id b runs on XCD b % 8. This maps b to a logical id so that every
// XCD owns one contiguous range of logical ids (a bijection on [0, total)).
__device__ __forceinline__ int64_t xcd_contiguous(int64_t b, int64_t total) {
  constexpr int64_t XCDS = 8;
  const int64_t xcd = b % XCDS, j = b / XCDS;
  const int64_t base = total / XCDS, rem = total % XCDS;
  return xcd * base + (xcd < rem ? xcd : rem) + j;
}

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

}  // namespace dit
