// MXFP8 conversion of bf16 activations: E4M3 codes plus one E8M0 scale per
// 32 consecutive K elements of a row, the operand form of the MXFP8 grouped
// GEMM of ROCm/aiter PR #5310 "Add MoE GEMM variants and weight-gradient
// kernel" (Summary; its second review's kernel excerpt decodes an a_scale and
// a b_scale byte per K block). The pages do not give the conversion; this is
// the one of the OCP Microscaling Formats v1.0 specification:
//   X = floor(log2(max |v|)) - 8 over the block (8: largest E4M3 exponent),
//       clamped to [-127, 127]; an all-zero block takes -127; byte X + 127;
//   code = E4M3 nearest to v / 2^X, ties to even, saturating at +-448,
//       sign bit set when v < 0.
// A block holding a NaN or an infinity has no finite shared exponent: it is
// written as a NaN block (scale byte 0xFF, every code 0x7F), so the
// non-finite input never turns into finite codes or leaks into the bytes of
// its neighbours.
//
// HBM-bound: one thread per (row, 32-element block) reads 64 bytes, writes
// 32 code bytes and one scale byte; a wave covers 4 KB of contiguous input.
// The codes come from gfx950's scaled conversion v_cvt_scalef32_pk_fp8_bf16
// (two elements per instruction), which divides by the power of two given
// as an E8M0 exponent and rounds to the nearest E4M3 value, ties to even,
// but turns results past 448 into NaN and keeps the sign of -0 (measured).
// So each element's magnitude is first clamped to 448 * 2^X (bf16 bits are
// ordered like magnitudes: one packed 16-bit min for two elements) and the
// sign of a zero is cleared; the conversion of v / 2^X is then exact up to
// its single rounding, which is the definition's.
#include "common.h"
#include "params.h"

namespace moe {

constexpr int kQuantThreads = 256;

typedef short q_v2s __attribute__((ext_vector_type(2)));
typedef __bf16 q_v2bf __attribute__((ext_vector_type(2)));
typedef unsigned short q_v2u16 __attribute__((ext_vector_type(2)));

// Two bf16 elements (bits of one dword) -> the dword with their magnitudes
// clamped to `lim2` (448 * 2^X in both halves) and the sign of a zero
// element cleared. Each half's magnitude plus 0x7FFF has bit 15 set exactly
// when the magnitude is non-zero, and never carries into the other half.
__device__ __forceinline__ uint32_t clamp_pair(uint32_t d, uint32_t lim2) {
  const uint32_t mag = d & 0x7FFF7FFFu;
  const uint32_t sgn = d & 0x80008000u & (mag + 0x7FFF7FFFu);
  const q_v2u16 m = __builtin_elementwise_min(__builtin_bit_cast(q_v2u16, mag), __builtin_bit_cast(q_v2u16, lim2));
  return __builtin_bit_cast(uint32_t, m) | sgn;
}

__global__ __launch_bounds__(kQuantThreads) void quant_mxfp8_kernel(
    const uint16_t* __restrict__ x, int64_t x_ld, int64_t rows, int32_t kb, uint8_t* __restrict__ q,
    int64_t q_ld, uint8_t* __restrict__ s, int64_t s_ld) {
  const int64_t total = rows * kb;
  for (int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kQuantThreads) {
    const int64_t row = i / kb;
    const int b = (int)(i % kb);
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + row * x_ld + (int64_t)b * 32);
    u32x4_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = src[j];
    // block maximum of |v| on the bf16 bits (order of magnitudes = order of bits)
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        amax = max(amax, v[j][w] & 0x7FFFu);
        amax = max(amax, (v[j][w] >> 16) & 0x7FFFu);
      }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(q + row * q_ld + (int64_t)b * 32);
    if (amax >= 0x7F80u) {  // exponent field all ones: a NaN or an infinity in the block
      const uint32_t nan4 = 0x7F7F7F7Fu;
      dst[0] = u32x4_t{nan4, nan4, nan4, nan4};
      dst[1] = u32x4_t{nan4, nan4, nan4, nan4};
      s[row * s_ld + b] = (uint8_t)0xFF;
      continue;
    }
    // floor(log2(max)) from the exponent field; a zero or subnormal maximum
    // (below 2^-126) gives X below -127, so the clamp decides
    const int e = (int)(amax >> 7);
    const int X = e == 0 ? -127 : min(max(e - 127 - 8, -127), 127);
    // the conversion's scale operand: E8M0 byte X + 127 in the exponent
    // field (byte 0 is 2^-127); X <= 119 for finite inputs, so 448 * 2^X
    // (bf16 exponent 135 + X, mantissa 0x60) is a finite bf16
    const float scale = __uint_as_float((uint32_t)(X + 127) << 23);
    const uint32_t lim = ((uint32_t)(135 + X) << 7) | 0x60u;
    const uint32_t lim2 = lim | (lim << 16);
    uint32_t out[8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w = 0; w < 4; w += 2) {
        // elements 8j + 2w .. 8j + 2w + 3 -> the four bytes of dword 2j + w/2
        const uint32_t lo = clamp_pair(v[j][w], lim2), hi = clamp_pair(v[j][w + 1], lim2);
        q_v2s r = {0, 0};
        r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(q_v2bf, lo), scale, false);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(q_v2bf, hi), scale, true);
        out[2 * j + w / 2] = __builtin_bit_cast(uint32_t, r);
      }
    dst[0] = u32x4_t{out[0], out[1], out[2], out[3]};
    dst[1] = u32x4_t{out[4], out[5], out[6], out[7]};
    s[row * s_ld + b] = (uint8_t)(X + 127);
  }
}

hipError_t launch_quant_mxfp8(const uint16_t* x, int64_t x_ld, int64_t rows, int64_t k, uint8_t* q, int64_t q_ld,
                              uint8_t* s, int64_t s_ld, hipStream_t stream) {
  const int64_t total = rows * (k / 32);
  if (total == 0) return hipSuccess;
  const int64_t want = (total + kQuantThreads - 1) / kQuantThreads;
  const uint32_t grid = (uint32_t)(want < 65536 * 8 ? want : 65536 * 8);
  hipLaunchKernelGGL(quant_mxfp8_kernel, dim3(grid), dim3(kQuantThreads), 0, stream, x, x_ld, rows,
                     (int32_t)(k / 32), q, q_ld, s, s_ld);
  return hipGetLastError();
}

}  // namespace moe
