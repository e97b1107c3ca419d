// moe_combine: y[t] = sum_j w[t, j] * C[t * top_k + j], fp32, j ascending,
// one bf16 rounding. The method's last step (top-k routing weights applied to
// the expert outputs); it runs after the padded rows were computed and writes
// only the rows it is asked for, which is the slice-back of TensorRT-LLM PR
// #15311 "Bound Triton MoE JIT specializations via token-dim bucketing and
// warmup", Description.
//
// HBM-bound: each thread owns 8 output columns of one token (one 16-byte load
// per expert slot, one 16-byte store).
#include "common.h"
#include "params.h"

namespace moe {

constexpr int kCombineThreads = 256;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const uint16_t* __restrict__ c, int64_t c_ld, const float* __restrict__ w,
    int64_t T, int32_t top_k, int32_t n8, uint16_t* __restrict__ y, int64_t y_ld) {
  const int64_t gid = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x;
  const int64_t t = gid / n8;
  const int col = (int)(gid % n8) * 8;
  if (t >= T) return;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  for (int j = 0; j < top_k; ++j) {
    const float wj = w[t * top_k + j];
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(c + (t * top_k + j) * c_ld + col);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += wj * bf16_bits_to_f32(v[q] & 0xffffu);
      acc[2 * q + 1] += wj * bf16_bits_to_f32(v[q] >> 16);
    }
  }
  u32x4_t o;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = f32_to_bf16_bits(acc[2 * q]) | (f32_to_bf16_bits(acc[2 * q + 1]) << 16);
  *reinterpret_cast<u32x4_t*>(y + t * y_ld + col) = o;
}

hipError_t launch_combine(const uint16_t* c, int64_t c_ld, const float* w, int64_t T,
                          int32_t top_k, int64_t N, uint16_t* y, int64_t y_ld,
                          hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int32_t n8 = (int32_t)(N / 8);
  const int64_t threads = T * n8;
  const int64_t blocks = (threads + kCombineThreads - 1) / kCombineThreads;
  hipLaunchKernelGGL(combine_kernel, dim3((uint32_t)blocks), dim3(kCombineThreads), 0, stream,
                     c, c_ld, w, T, top_k, n8, y, y_ld);
  return hipGetLastError();
}

}  // namespace moe
