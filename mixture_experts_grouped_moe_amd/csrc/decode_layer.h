// Parameter block and launcher of the fused decode layer (decode_layer.hip),
// shared with the host API (api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// The decode MoE step in one launch (routing, grouped GEMM, combine).
struct DecodeLayerParams {
  const uint16_t* x;     // bf16 token rows [T][K]
  int64_t x_ld;          // elements
  const int32_t* topk_ids;  // [T * top_k]
  const float* topk_w;      // [T * top_k]
  // weight codes of (e, n, 64-element K block kb) at byte
  // e * w_stride_e + n * w_row + kb * w_blk; E8M0 scale bytes likewise
  const uint8_t* w;
  int64_t w_stride_e, w_row, w_blk;
  const uint8_t* ws;     // E8M0 scales (block-scaled weights), else unused
  int64_t ws_stride_e, ws_row, ws_blk;
  const uint16_t* bias;  // bf16 [E][N] or null
  int64_t bias_se, bias_sn;
  uint16_t* c;           // bf16 [S][N] expert outputs, or null (not written)
  int64_t c_ld;
  uint16_t* y;           // bf16 [T][N]
  int64_t y_ld;
  int32_t S, top_k, E, N, K;
  int32_t relu2;
  // byte ranges of the buffer loads (each < 2^31): the T token rows, one
  // weight row's codes and scale bytes (from the row's first byte), the bias
  uint32_t x_bytes, w_rspan, ws_rspan, bias_bytes;
};

hipError_t launch_decode_layer(const DecodeLayerParams& p, int wdt, bool bias, hipStream_t stream);
int decode_layer_max_slots();
int decode_layer_max_experts();
int decode_layer_max_k();

}  // namespace moe
