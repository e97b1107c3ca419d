// Kernel parameter blocks and launcher entry points shared by the host API
// (api.cpp) and the kernels (*.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct GemmParams {
  const uint16_t* a;   // bf16 activation rows
  int64_t a_ld;        // elements
  int64_t a_rows;      // rows of A that slots can address: ceil(S / a_row_div)
  int32_t a_row_div;   // slot s reads row s / a_row_div
  const uint8_t* w;    // weight codes
  int64_t w_stride_e;  // bytes
  int64_t w_ld;        // bytes
  const uint8_t* ws;   // E8M0 scales
  int64_t ws_stride_e;
  int64_t ws_ld;
  const uint16_t* bias;  // bf16 or null
  int64_t bias_se, bias_sn;
  uint16_t* c;         // bf16 output rows
  int64_t c_ld;
  const int32_t* sorted;
  const int32_t* expert_ids;
  int32_t S;           // PAD value (= number of slots)
  int32_t N, K;
  int32_t max_blocks;
};

struct WgradParams {
  const uint16_t* x;
  int64_t x_ld;
  const uint16_t* grad;
  int64_t grad_ld;
  const int32_t* sorted;
  const int32_t* expert_ids;
  int32_t S, top_k, E;
  int32_t N, K;
  int32_t max_blocks;
  int32_t tiles_n, tiles_k;
  float* dw;
};

hipError_t launch_align(const int32_t* ids, int32_t S, int32_t E, int32_t B, int32_t* sorted_ids,
                        int32_t* expert_ids, int32_t* post_pad, int32_t max_blocks, hipStream_t stream);
hipError_t launch_gemm_large(const GemmParams& p, int wdt, bool swiglu, bool bias, hipStream_t stream);
hipError_t launch_gemm_decode(const GemmParams& p, int wdt, bool swiglu, bool bias, hipStream_t stream);
hipError_t launch_combine(const uint16_t* c, int64_t c_ld, const float* w, int64_t T, int32_t top_k,
                          int64_t N, uint16_t* y, int64_t y_ld, hipStream_t stream);
hipError_t launch_wgrad(const WgradParams& p, hipStream_t stream);
int gemm_block_m_large();
int gemm_block_m_decode();
int wgrad_block_m();

}  // namespace moe
