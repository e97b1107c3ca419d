// Shared device helpers for the gfx950 kernels of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Weight element encodings (values match moe_dtype).
enum WDtype : int { W_BF16 = 1, W_E4M3 = 3, W_E2M1 = 4 };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// An E8M0 scale byte as the fp32 operand of the scaled conversions: those
// instructions read only the exponent field of the scale, so placing the
// byte there gives 2^(b - 127), with b = 0 -> 2^-127 and b = 255 -> NaN.
__device__ __forceinline__ float e8m0_as_scale(uint32_t b) {
  return __uint_as_float((b & 0xffu) << 23);
}

// 8 E2M1 codes (one dword, element 2i in the low nibble of byte i) scaled
// by 2^(b-127) -> 8 bf16 in K order.
__device__ __forceinline__ bf16x8_t dequant_e2m1x8(uint32_t codes, float scale) {
  bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  bf16x8_t r;
  uint32_t w[4];
  __builtin_memcpy(&w[0], &p0, 4);
  __builtin_memcpy(&w[1], &p1, 4);
  __builtin_memcpy(&w[2], &p2, 4);
  __builtin_memcpy(&w[3], &p3, 4);
  __builtin_memcpy(&r, w, 16);
  return r;
}

// 8 E4M3 codes (two dwords, K order) scaled by 2^(b-127) -> 8 bf16.
__device__ __forceinline__ bf16x8_t dequant_e4m3x8(uint32_t lo, uint32_t hi, float scale) {
  bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false);
  bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true);
  bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false);
  bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true);
  bf16x8_t r;
  uint32_t w[4];
  __builtin_memcpy(&w[0], &p0, 4);
  __builtin_memcpy(&w[1], &p1, 4);
  __builtin_memcpy(&w[2], &p2, 4);
  __builtin_memcpy(&w[3], &p3, 4);
  __builtin_memcpy(&r, w, 16);
  return r;
}

// Workgroups are dispatched round-robin over the 8 XCDs (id i runs on XCD
// i % 8). Remap the hardware id so that each XCD receives one contiguous
// range of logical ids: neighbouring logical tiles (which share operands)
// then share that XCD's L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t hw_id, uint32_t grid) {
  constexpr uint32_t kXcd = 8;
  uint32_t xcd = hw_id % kXcd;
  uint32_t q = grid / kXcd, r = grid % kXcd;
  uint32_t base = xcd * q + (xcd < r ? xcd : r);
  return base + hw_id / kXcd;
}

// The non-gated squared ReLU epilogue: max(z, 0)^2 (NaN -> 0, as z > 0 fails).
__device__ __forceinline__ float relu2_f32(float z) { return z > 0.0f ? z * z : 0.0f; }

__device__ __forceinline__ float silu_f32(float z) {
  return z / (1.0f + __expf(-z));
}

}  // namespace moe
