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
// Every step is exact in fp32 (bf16 times a power of two inside the normal
// range, then an integer rounding on the bits), so the codes are the same
// as a float64 evaluation of the definition.
#include "common.h"
#include "params.h"

namespace moe {

constexpr int kQuantThreads = 256;

// |a| (a finite, non-negative fp32) -> E4M3 magnitude code, round to nearest
// even, saturating at 448 (code 0x7E).
__device__ __forceinline__ uint32_t e4m3_magnitude(float a) {
  if (a >= 448.0f) return 0x7Eu;
  if (a < 0.015625f) return (uint32_t)__builtin_rintf(a * 512.0f);  // subnormals: m * 2^-9
  const uint32_t bits = __float_as_uint(a);
  // keep 3 mantissa bits: round at bit 20 (ties to even), carries move into
  // the exponent; rebias the exponent from 127 to 7
  const uint32_t r = bits + 0x7FFFFu + ((bits >> 20) & 1u);
  return (r >> 20) - ((127u - 7u) << 3);
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
    const float inv = __uint_as_float((uint32_t)(127 - X) << 23);  // 2^-X, X in [-127, 120]
    uint32_t out[8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t pair = 0;
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
          const uint32_t h = (v[j][w] >> (16 * hlf)) & 0xFFFFu;
          const float a = bf16_bits_to_f32(h & 0x7FFFu) * inv;
          const uint32_t sign = (h & 0x8000u) && (h & 0x7FFFu) ? 0x80u : 0u;  // v < 0 (not -0)
          pair |= (e4m3_magnitude(a) | sign) << (8 * hlf);
        }
        // elements 8j + 2w, 8j + 2w + 1 -> bytes 2w, 2w + 1 of dword j / 2 half j % 2
        out[2 * j + w / 2] = (w % 2 == 0) ? pair : (out[2 * j + w / 2] | (pair << 16));
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
