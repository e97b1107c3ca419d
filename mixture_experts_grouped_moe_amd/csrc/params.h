// Kernel parameter blocks and launcher entry points shared by the host API
// (api.cpp) and the kernels (*.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct GemmParams {
  const uint16_t* a;   // bf16 activation rows (E4M3 code rows for the MXFP8-activation kernel)
  int64_t a_ld;        // elements
  const uint8_t* as;   // E8M0 activation scales [a_rows][K/32] (MXFP8 activations only)
  int64_t as_ld;       // bytes
  int64_t a_rows;      // rows of A that slots can address: ceil(S / a_row_div)
  int32_t a_row_div;   // slot s reads row s / a_row_div
  // Weight codes of (e, n, 64-element K block kb) start at byte
  // e * w_stride_e + n * w_row + kb * w_blk, and the block's two scale bytes
  // at e * ws_stride_e + n * ws_row + kb * ws_blk (+0, +1); both layouts of
  // the API are these strides. w_span / ws_span bound one expert's bytes.
  const uint8_t* w;
  int64_t w_stride_e;
  int64_t w_row, w_blk;
  int64_t w_span;
  const uint8_t* ws;
  int64_t ws_stride_e;
  int64_t ws_row, ws_blk;
  int64_t ws_span;
  const uint16_t* bias;  // bf16 or null
  int64_t bias_se, bias_sn;
  uint16_t* c;         // bf16 output rows
  int64_t c_ld;
  const int32_t* sorted;
  const int32_t* expert_ids;
  const int32_t* post_pad;  // moe_align's padded row count: blocks past post_pad / block_m are unused
  int32_t S;           // PAD value (= number of slots)
  int32_t N, K;
  int32_t max_blocks;
  int32_t relu2;       // non-SwiGLU epilogue: store max(pre, 0)^2 instead of pre
  int32_t E;           // experts: a block naming another expert is skipped
  // Per-token mode of the fp8 kernel (group_sizes interface): block b covers
  // rows [blk_off[b], min(blk_off[b] + 64, blk_end[b], S)) of A and C, and
  // the accumulator is scaled by tok_scale[row] * exp_scale[e].
  const int32_t* blk_off;
  const int32_t* blk_end;
  const float* tok_scale;
  const float* exp_scale;
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
  uint32_t topk_magic;  // slot s's token row s / top_k = (s * topk_magic) >> topk_shift
  int32_t topk_shift;
  float* dw;
};

hipError_t launch_align(const int32_t* ids, int32_t S, int32_t E, int32_t B, int32_t* sorted_ids,
                        int32_t* expert_ids, int32_t* post_pad, int32_t max_blocks, hipStream_t stream);
hipError_t launch_block_map(const int32_t* group_sizes, int32_t E, int32_t B, int32_t rows, int32_t* expert_ids,
                            int32_t* offsets, int32_t* ends, int32_t max_blocks, int32_t* total_out,
                            hipStream_t stream);
hipError_t launch_gemm_large(const GemmParams& p, int wdt, bool swiglu, bool bias, hipStream_t stream);
hipError_t launch_gemm_decode(const GemmParams& p, int wdt, bool swiglu, bool bias, hipStream_t stream);
// MXFP8 activations x MXFP8 (E4M3) weights on the scaled fp8 MFMA
hipError_t launch_gemm_f8(const GemmParams& p, bool swiglu, bool bias, hipStream_t stream);
// E4M3 x E4M3 with per-token and per-expert fp32 scales over a block mapping
hipError_t launch_gemm_per_token(const GemmParams& p, bool bias, hipStream_t stream);
hipError_t launch_combine(const uint16_t* c, int64_t c_ld, const float* w, int64_t T, int32_t top_k,
                          int64_t N, uint16_t* y, int64_t y_ld, hipStream_t stream);
hipError_t launch_wgrad(const WgradParams& p, hipStream_t stream);
// Copy one block of rows-layout codes/scales into the K-block layout.
hipError_t launch_pack(const uint8_t* w, int64_t w_stride_e, int64_t w_ld, const uint8_t* ws,
                       int64_t ws_stride_e, int64_t ws_ld, int32_t E, int32_t N, int32_t K, int32_t row_bytes,
                       uint8_t* w_out, uint8_t* ws_out, hipStream_t stream);
hipError_t launch_quant_mxfp8(const uint16_t* x, int64_t x_ld, int64_t rows, int64_t k, uint8_t* q, int64_t q_ld,
                              uint8_t* s, int64_t s_ld, hipStream_t stream);
int gemm_block_m_large();
int gemm_block_m_f8();
int gemm_block_m_decode();
int wgrad_block_m();

}  // namespace moe
