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

constexpr int kCombineBatch = 8;  // slots whose loads are issued together

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
  // up to 8 slots' weights and rows are loaded before any is used (one
  // memory round trip instead of one per slot); the sum runs over j in order
  for (int j0 = 0; j0 < top_k; j0 += kCombineBatch) {
    float wj[kCombineBatch];
    u32x4_t v[kCombineBatch];
#pragma unroll
    for (int jj = 0; jj < kCombineBatch; ++jj) {
      const int64_t sl = t * top_k + j0 + jj;
      const bool ok = j0 + jj < top_k;
      wj[jj] = ok ? w[sl] : 0.0f;
      v[jj] = ok ? *reinterpret_cast<const u32x4_t*>(c + sl * c_ld + col) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int jj = 0; jj < kCombineBatch; ++jj) {
      if (j0 + jj >= top_k) break;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += wj[jj] * bf16_bits_to_f32(v[jj][q] & 0xffffu);
        acc[2 * q + 1] += wj[jj] * bf16_bits_to_f32(v[jj][q] >> 16);
      }
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
