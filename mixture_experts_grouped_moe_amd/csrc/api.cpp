// Host side of libmoe: the C ABI declared in include/moe.h. Argument
// validation (before anything touches the GPU), variant dispatch and the
// pure host helpers.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "moe.h"

#include "decode_layer.h"
#include "params.h"

namespace {

constexpr int64_t kDecodeMaxTokens = 32;
constexpr int32_t kAlignMaxExperts = 1024;

thread_local std::string g_last_error;

moe_status fail(moe_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status ok() {
  g_last_error.clear();
  return MOE_OK;
}

// The kernels are written for gfx950 only: refuse any other device.
moe_status check_device() {
  static int cached[64] = {0};  // 0 unknown, 1 gfx950, -1 other
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(err));
  if (dev >= 0 && dev < 64 && cached[dev] != 0)
    return cached[dev] == 1 ? MOE_OK : fail(MOE_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  hipDeviceProp_t prop;
  err = hipGetDeviceProperties(&prop, dev);
  if (err != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(err));
  const bool is950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) cached[dev] = is950 ? 1 : -1;
  if (!is950) return fail(MOE_ERR_UNSUPPORTED, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  return MOE_OK;
}

moe_status hip_status(hipError_t err, const char* what) {
  if (err != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
  return ok();
}

int64_t bucket(int64_t m) {
  if (m < 0) return -1;
  if (m < 16) return m;
  int bits = 64 - __builtin_clzll((unsigned long long)m);
  int64_t step = (int64_t)1 << (bits - 4);
  return ((m + step - 1) / step) * step;
}

bool valid_w_dtype(int32_t d) { return d == MOE_BF16 || d == MOE_E4M3 || d == MOE_E2M1X2; }

// The weight, scale and bias arguments of a routed GEMM (everything the two
// entry points that take moe_gemm_args share): layout, strides and the byte
// geometry the kernels address them with.
struct WeightGeom {
  bool kblock;
  int64_t elem_bytes;  // bytes per storage unit of the codes
  int64_t blk_units;   // storage units per row per 64-element K block
  int64_t nblk;        // 64-element K blocks
  int64_t w_span;      // bytes of one expert's codes, ws_span of its scales
  int64_t ws_span;
};

moe_status check_weights(const moe_gemm_args& a, WeightGeom* g) {
  if (a.w_layout != MOE_LAYOUT_ROWS && a.w_layout != MOE_LAYOUT_KBLOCK)
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown w_layout %d", a.w_layout);
  const bool kblock = a.w_layout == MOE_LAYOUT_KBLOCK;
  const int64_t w_elem_bytes = a.w_dtype == MOE_BF16 ? 2 : 1;
  const int64_t blk_units = a.w_dtype == MOE_E2M1X2 ? 32 : 64;
  const int64_t nblk = (a.k + 63) / 64;
  if ((a.w_ld * w_elem_bytes) % 16 != 0 || (a.w_stride_e * w_elem_bytes) % 16 != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "w_ld and w_stride_e must be multiples of 16 bytes");
  if (!kblock) {
    if (a.w_ld < a.k * blk_units / 64) return fail(MOE_ERR_INVALID_ARGUMENT, "w_ld must cover a row");
    if (a.w_stride_e < a.n * a.w_ld) return fail(MOE_ERR_INVALID_ARGUMENT, "w_stride_e < n * w_ld");
  } else {
    if (a.w_ld < a.n * blk_units) return fail(MOE_ERR_INVALID_ARGUMENT, "w_ld must cover a K block of n rows");
    if (a.w_stride_e < nblk * a.w_ld) return fail(MOE_ERR_INVALID_ARGUMENT, "w_stride_e < ceil(k/64) * w_ld");
  }
  if (a.w_dtype != MOE_BF16) {
    if (a.w_scale == nullptr) return fail(MOE_ERR_INVALID_ARGUMENT, "w_scale is null");
    const bool ok = !kblock ? (a.w_scale_ld >= a.k / 32 && a.w_scale_stride_e >= a.n * a.w_scale_ld)
                            : (a.w_scale_ld >= 2 * a.n && a.w_scale_stride_e >= nblk * a.w_scale_ld);
    if (!ok) return fail(MOE_ERR_INVALID_ARGUMENT, "w_scale strides too small");
  }
  if (a.bias != nullptr && (a.bias_stride_e < 0 || a.bias_stride_n < 0))
    return fail(MOE_ERR_INVALID_ARGUMENT, "negative bias stride");
  g->kblock = kblock;
  g->elem_bytes = w_elem_bytes;
  g->blk_units = blk_units;
  g->nblk = nblk;
  g->w_span = (kblock ? nblk : a.n) * a.w_ld * w_elem_bytes;
  g->ws_span = a.w_dtype == MOE_BF16 ? 0 : (kblock ? nblk : a.n) * a.w_scale_ld;
  return MOE_OK;
}

}  // namespace

extern "C" {

int64_t moe_bucket_round_up(int64_t m) { return bucket(m); }

int64_t moe_bucket_enumerate(int64_t max_tokens, int64_t* out, int64_t cap) {
  if (max_tokens < 0 || cap < 0 || (cap > 0 && out == nullptr)) return -1;
  int64_t n = 0;
  for (int64_t b = bucket(1); max_tokens >= 1 && b <= max_tokens; b = bucket(b + 1)) {
    if (n < cap) out[n] = b;
    ++n;
  }
  if (max_tokens >= 1) {
    const int64_t top = bucket(max_tokens);
    if (top > max_tokens) {
      if (n < cap) out[n] = top;
      ++n;
    }
  }
  return n;
}

int32_t moe_padding_supported(int32_t a_dtype, int32_t w_dtype, int32_t dynamic_act_scale) {
  return (a_dtype == MOE_BF16 && w_dtype == MOE_E2M1X2 && dynamic_act_scale == 0) ? 1 : 0;
}

int64_t moe_align_max_blocks(int64_t num_slots, int32_t num_experts, int32_t block_m) {
  if (num_slots < 0 || num_experts < 1 || block_m < 1) return -1;
  const int64_t used = num_slots < num_experts ? num_slots : num_experts;
  return (num_slots + used * (block_m - 1)) / block_m;
}

int32_t moe_gemm_block_m(int32_t a_dtype, int32_t w_dtype, int64_t num_tokens) {
  if (num_tokens < 0) return -1;
  if (a_dtype == MOE_E4M3 && w_dtype == MOE_E4M3) return moe::gemm_block_m_f8();  // one kernel for every T
  if (a_dtype != MOE_BF16 || !valid_w_dtype(w_dtype)) return -1;
  return num_tokens <= kDecodeMaxTokens ? moe::gemm_block_m_decode() : moe::gemm_block_m_large();
}

int32_t moe_wgrad_block_m(void) { return moe::wgrad_block_m(); }

int64_t moe_decode_max_tokens(void) { return kDecodeMaxTokens; }

const char* moe_status_string(int32_t status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_align(const int32_t* topk_ids, int64_t num_tokens, int32_t top_k, int32_t num_experts,
                     int32_t block_m, int32_t* sorted_token_ids, int32_t* expert_ids,
                     int32_t* num_tokens_post_pad, int64_t max_blocks, moe_stream_t stream) {
  if (num_tokens < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "num_tokens < 0");
  if (top_k < 1 || num_experts < top_k)
    return fail(MOE_ERR_INVALID_ARGUMENT, "need 1 <= top_k (%d) <= num_experts (%d)", top_k, num_experts);
  if (num_experts > kAlignMaxExperts)
    return fail(MOE_ERR_UNSUPPORTED, "num_experts %d > %d", num_experts, kAlignMaxExperts);
  if (block_m < 1 || block_m > 256) return fail(MOE_ERR_INVALID_ARGUMENT, "block_m %d not in [1, 256]", block_m);
  const int64_t S = num_tokens * top_k;
  // the kernel's slot indices run up to 512 past the last slot
  if (S > INT32_MAX - 65536) return fail(MOE_ERR_INVALID_ARGUMENT, "num_tokens * top_k must be <= 2^31 - 2^16");
  const int64_t need = moe_align_max_blocks(S, num_experts, block_m);
  if (max_blocks < need)
    return fail(MOE_ERR_INVALID_ARGUMENT, "max_blocks %lld < required %lld", (long long)max_blocks,
                (long long)need);
  if (max_blocks * block_m >= INT32_MAX) return fail(MOE_ERR_INVALID_ARGUMENT, "max_blocks * block_m too large");
  if ((S > 0 && topk_ids == nullptr) || num_tokens_post_pad == nullptr ||
      (max_blocks > 0 && (sorted_token_ids == nullptr || expert_ids == nullptr)))
    return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer argument");
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_align(topk_ids, (int32_t)S, num_experts, block_m, sorted_token_ids,
                                      expert_ids, num_tokens_post_pad, (int32_t)max_blocks,
                                      (hipStream_t)stream),
                    "moe_align launch");
}

moe_status moe_grouped_gemm(const moe_gemm_args* g, moe_stream_t stream) {
  if (g == nullptr) return fail(MOE_ERR_INVALID_ARGUMENT, "args is null");
  const moe_gemm_args& a = *g;
  if (a.num_tokens < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "num_tokens < 0");
  if (a.top_k < 1 || a.num_experts < a.top_k)
    return fail(MOE_ERR_INVALID_ARGUMENT, "need 1 <= top_k (%d) <= num_experts (%d)", a.top_k, a.num_experts);
  const bool a_f8 = a.a_dtype == MOE_E4M3;
  if (a.a_dtype != MOE_BF16 && !a_f8) return fail(MOE_ERR_UNSUPPORTED, "a_dtype must be MOE_BF16 or MOE_E4M3");
  if (!valid_w_dtype(a.w_dtype)) return fail(MOE_ERR_UNSUPPORTED, "w_dtype %d not supported", a.w_dtype);
  if (a_f8 && a.w_dtype != MOE_E4M3)
    return fail(MOE_ERR_UNSUPPORTED, "MXFP8 activations need MOE_E4M3 weights");
  if (a.n < 1 || a.n >= INT32_MAX) return fail(MOE_ERR_INVALID_ARGUMENT, "n out of range");
  if (a.k < 32 || a.k % 32 != 0 || a.k >= INT32_MAX)
    return fail(MOE_ERR_INVALID_ARGUMENT, "k (%lld) must be a positive multiple of 32", (long long)a.k);
  if (a.epilogue != MOE_EPILOGUE_NONE && a.epilogue != MOE_EPILOGUE_SWIGLU && a.epilogue != MOE_EPILOGUE_RELU2)
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown epilogue %d", a.epilogue);
  const bool swiglu = a.epilogue == MOE_EPILOGUE_SWIGLU;
  if (swiglu && a.n % 2 != 0) return fail(MOE_ERR_INVALID_ARGUMENT, "SwiGLU needs an even n");
  const int64_t out_w = swiglu ? a.n / 2 : a.n;
  const int64_t S = a.num_tokens * a.top_k;
  if (S >= INT32_MAX) return fail(MOE_ERR_INVALID_ARGUMENT, "num_tokens * top_k must be < 2^31");
  if (a.a_row_div != 1 && a.a_row_div != a.top_k)
    return fail(MOE_ERR_INVALID_ARGUMENT, "a_row_div must be 1 or top_k");
  if (a.a_ld < a.k || a.a_ld % (a_f8 ? 16 : 8) != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "a_ld must be >= k and a multiple of %d", a_f8 ? 16 : 8);
  if (a_f8 && (a.a_scale == nullptr || a.a_scale_ld < a.k / 32))
    return fail(MOE_ERR_INVALID_ARGUMENT, "MXFP8 activations need a_scale with a_scale_ld >= k / 32");
  WeightGeom wg;
  moe_status wst = check_weights(a, &wg);
  if (wst != MOE_OK) return wst;
  const bool kblock = wg.kblock;
  const int64_t w_elem_bytes = wg.elem_bytes;
  const int64_t blk_units = wg.blk_units;
  if (a.c_ld < out_w) return fail(MOE_ERR_INVALID_ARGUMENT, "c_ld must be >= the output width");
  const int32_t bm = moe_gemm_block_m(a.a_dtype, a.w_dtype, a.num_tokens);
  if (a.block_m != bm)
    return fail(MOE_ERR_INVALID_ARGUMENT, "block_m %d, expected %d for this call", a.block_m, bm);
  const int64_t need = moe_align_max_blocks(S, a.num_experts, a.block_m);
  if (a.max_blocks < need)
    return fail(MOE_ERR_INVALID_ARGUMENT, "max_blocks %lld < required %lld", (long long)a.max_blocks,
                (long long)need);
  if (a.max_blocks * a.block_m >= INT32_MAX) return fail(MOE_ERR_INVALID_ARGUMENT, "max_blocks too large");
  if (S > 0 && (a.a == nullptr || a.w == nullptr || a.c == nullptr || a.sorted_token_ids == nullptr ||
                a.expert_ids == nullptr || a.num_tokens_post_pad == nullptr))
    return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (((uintptr_t)a.a | (uintptr_t)a.w) % 16 != 0 || (uintptr_t)a.c % 2 != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "a and w must be 16-byte aligned, c 2-byte aligned");
  // the large-M kernel addresses A, one expert's weights and one expert's
  // scales through 32-bit buffer offsets
  const int64_t a_rows = S > 0 ? (S - 1) / a.a_row_div + 1 : 0;
  constexpr int64_t kBufMax = (int64_t)0x80000000;
  const int64_t w_span = wg.w_span, ws_span = wg.ws_span;
  if (a_rows * a.a_ld * (a_f8 ? 1 : 2) >= kBufMax || w_span >= kBufMax || ws_span >= kBufMax ||
      (a_f8 && a_rows * a.a_scale_ld >= kBufMax))
    return fail(MOE_ERR_UNSUPPORTED, "A, its scales, one expert's weights or its scales span 2 GB or more");
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  if (S == 0 || a.max_blocks == 0) return ok();
  const int64_t grid_guess = a.max_blocks * ((out_w + 7) / 8);
  if (grid_guess >= (int64_t)UINT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "grid too large");

  moe::GemmParams p{};
  p.a = static_cast<const uint16_t*>(a.a);
  p.a_ld = a.a_ld;
  p.a_rows = a_rows;
  p.as = a_f8 ? a.a_scale : nullptr;
  p.as_ld = a_f8 ? a.a_scale_ld : 0;
  p.a_row_div = a.a_row_div;
  p.w = static_cast<const uint8_t*>(a.w);
  p.w_stride_e = a.w_stride_e * w_elem_bytes;
  p.w_row = kblock ? blk_units * w_elem_bytes : a.w_ld * w_elem_bytes;
  p.w_blk = kblock ? a.w_ld * w_elem_bytes : blk_units * w_elem_bytes;
  p.w_span = w_span;
  p.ws = a.w_scale;
  p.ws_stride_e = a.w_scale_stride_e;
  p.ws_row = kblock ? 2 : a.w_scale_ld;
  p.ws_blk = kblock ? a.w_scale_ld : 2;
  p.ws_span = ws_span;
  p.bias = static_cast<const uint16_t*>(a.bias);
  p.bias_se = a.bias_stride_e;
  p.bias_sn = a.bias_stride_n;
  p.c = static_cast<uint16_t*>(a.c);
  p.c_ld = a.c_ld;
  p.sorted = a.sorted_token_ids;
  p.expert_ids = a.expert_ids;
  p.post_pad = a.num_tokens_post_pad;
  p.S = (int32_t)S;
  p.N = (int32_t)a.n;
  p.K = (int32_t)a.k;
  // at most `need` blocks are in use (one per started BLOCK_M rows of each
  // touched expert); the rest are sentinels, so the grid stops there
  p.max_blocks = (int32_t)need;
  p.relu2 = a.epilogue == MOE_EPILOGUE_RELU2 ? 1 : 0;
  p.E = a.num_experts;
  const bool bias = a.bias != nullptr;
  if (a_f8) return hip_status(moe::launch_gemm_f8(p, swiglu, bias, (hipStream_t)stream), "moe_grouped_gemm launch");
  const bool decode = a.num_tokens <= kDecodeMaxTokens;
  return hip_status(decode ? moe::launch_gemm_decode(p, a.w_dtype, swiglu, bias, (hipStream_t)stream)
                           : moe::launch_gemm_large(p, a.w_dtype, swiglu, bias, (hipStream_t)stream),
                    "moe_grouped_gemm launch");
}

int32_t moe_decode_layer_fits(int64_t num_tokens, int32_t top_k, int32_t num_experts, int64_t k) {
  return num_tokens >= 0 && num_tokens <= kDecodeMaxTokens && top_k >= 1 &&
         num_tokens * top_k <= moe::decode_layer_max_slots() && num_experts >= 1 &&
         num_experts <= moe::decode_layer_max_experts() && k >= 32 && k % 32 == 0 &&
         k <= moe::decode_layer_max_k();
}

moe_status moe_decode_layer(const moe_gemm_args* g, const int32_t* topk_ids, const float* topk_w, void* y,
                            int64_t y_ld, moe_stream_t stream) {
  if (g == nullptr) return fail(MOE_ERR_INVALID_ARGUMENT, "args is null");
  const moe_gemm_args& a = *g;
  if (a.num_tokens < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "num_tokens < 0");
  if (a.top_k < 1 || a.num_experts < a.top_k)
    return fail(MOE_ERR_INVALID_ARGUMENT, "need 1 <= top_k (%d) <= num_experts (%d)", a.top_k, a.num_experts);
  if (a.a_dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "the decode layer takes bf16 activations");
  if (!valid_w_dtype(a.w_dtype)) return fail(MOE_ERR_UNSUPPORTED, "w_dtype %d not supported", a.w_dtype);
  if (a.n < 1 || a.n >= INT32_MAX) return fail(MOE_ERR_INVALID_ARGUMENT, "n out of range");
  if (a.k < 32 || a.k % 32 != 0 || a.k >= INT32_MAX)
    return fail(MOE_ERR_INVALID_ARGUMENT, "k (%lld) must be a positive multiple of 32", (long long)a.k);
  if (a.epilogue == MOE_EPILOGUE_SWIGLU)
    return fail(MOE_ERR_UNSUPPORTED, "the decode layer has no SwiGLU epilogue");
  if (a.epilogue != MOE_EPILOGUE_NONE && a.epilogue != MOE_EPILOGUE_RELU2)
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown epilogue %d", a.epilogue);
  if (a.a_row_div != a.top_k) return fail(MOE_ERR_INVALID_ARGUMENT, "a_row_div must be top_k (A holds token rows)");
  if (a.a_ld < a.k || a.a_ld % 8 != 0) return fail(MOE_ERR_INVALID_ARGUMENT, "a_ld must be >= k and a multiple of 8");
  WeightGeom wg;
  moe_status wst = check_weights(a, &wg);
  if (wst != MOE_OK) return wst;
  if (a.c != nullptr && a.c_ld < a.n) return fail(MOE_ERR_INVALID_ARGUMENT, "c_ld must be >= n");
  if (y_ld < a.n) return fail(MOE_ERR_INVALID_ARGUMENT, "y_ld must be >= n");
  if (!moe_decode_layer_fits(a.num_tokens, a.top_k, a.num_experts, a.k))
    return fail(MOE_ERR_UNSUPPORTED,
                "the decode layer takes num_tokens <= %lld, num_tokens * top_k <= %d, num_experts <= %d "
                "and k <= %d",
                (long long)kDecodeMaxTokens, moe::decode_layer_max_slots(), moe::decode_layer_max_experts(),
                moe::decode_layer_max_k());
  if (a.num_tokens > 0 &&
      (a.a == nullptr || a.w == nullptr || topk_ids == nullptr || topk_w == nullptr || y == nullptr))
    return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (((uintptr_t)a.a | (uintptr_t)a.w) % 16 != 0 || ((uintptr_t)a.c | (uintptr_t)y) % 2 != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "a and w must be 16-byte aligned, c and y 2-byte aligned");
  // the kernel reads the token rows, each weight row's codes and scales and
  // the bias through 32-bit buffer ranges
  const int64_t x_bytes = a.num_tokens > 0 ? ((a.num_tokens - 1) * a.a_ld + a.k) * 2 : 0;
  const int64_t w_row = wg.kblock ? wg.blk_units * wg.elem_bytes : a.w_ld * wg.elem_bytes;
  const int64_t w_blk = wg.kblock ? a.w_ld * wg.elem_bytes : wg.blk_units * wg.elem_bytes;
  const int64_t piece = 8 * wg.blk_units * wg.elem_bytes / 64;  // bytes of 8 codes
  const int64_t w_rspan = ((a.k - 8) / 64) * w_blk + ((a.k - 8) % 64) * piece / 8 + piece;
  const int64_t ws_row = wg.kblock ? 2 : a.w_scale_ld, ws_blk = wg.kblock ? a.w_scale_ld : 2;
  const int64_t ws_rspan = a.w_dtype == MOE_BF16 ? 0 : ((a.k - 1) / 64) * ws_blk + ((a.k - 1) % 64) / 32 + 1;
  const int64_t bias_bytes =
      a.bias != nullptr ? ((a.num_experts - 1) * a.bias_stride_e + (a.n - 1) * a.bias_stride_n + 1) * 2 : 0;
  constexpr int64_t kBufMax = (int64_t)0x80000000;
  if (x_bytes >= kBufMax || w_rspan >= kBufMax || ws_rspan >= kBufMax || bias_bytes >= kBufMax)
    return fail(MOE_ERR_UNSUPPORTED, "A, one weight row, its scales or the bias spans 2 GB or more");
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  if (a.num_tokens == 0) return ok();

  moe::DecodeLayerParams p{};
  p.x = static_cast<const uint16_t*>(a.a);
  p.x_ld = a.a_ld;
  p.topk_ids = topk_ids;
  p.topk_w = topk_w;
  p.w = static_cast<const uint8_t*>(a.w);
  p.w_stride_e = a.w_stride_e * wg.elem_bytes;
  p.w_row = w_row;
  p.w_blk = w_blk;
  p.ws = a.w_scale;
  p.ws_stride_e = a.w_scale_stride_e;
  p.ws_row = ws_row;
  p.ws_blk = ws_blk;
  p.bias = static_cast<const uint16_t*>(a.bias);
  p.bias_se = a.bias_stride_e;
  p.bias_sn = a.bias_stride_n;
  p.c = static_cast<uint16_t*>(a.c);
  p.c_ld = a.c_ld;
  p.y = static_cast<uint16_t*>(y);
  p.y_ld = y_ld;
  p.S = (int32_t)(a.num_tokens * a.top_k);
  p.top_k = a.top_k;
  p.E = a.num_experts;
  p.N = (int32_t)a.n;
  p.K = (int32_t)a.k;
  p.relu2 = a.epilogue == MOE_EPILOGUE_RELU2 ? 1 : 0;
  p.x_bytes = (uint32_t)x_bytes;
  p.w_rspan = (uint32_t)w_rspan;
  p.ws_rspan = (uint32_t)ws_rspan;
  p.bias_bytes = (uint32_t)bias_bytes;
  return hip_status(moe::launch_decode_layer(p, a.w_dtype, a.bias != nullptr, (hipStream_t)stream),
                    "moe_decode_layer launch");
}

moe_status moe_packed_sizes(int32_t w_dtype, int64_t n, int64_t k, int64_t* w_units, int64_t* scale_bytes) {
  if (!valid_w_dtype(w_dtype)) return fail(MOE_ERR_INVALID_ARGUMENT, "w_dtype %d not supported", w_dtype);
  if (n < 1 || n >= INT32_MAX || k < 32 || k % 32 != 0 || k >= INT32_MAX)
    return fail(MOE_ERR_INVALID_ARGUMENT, "need n >= 1 and k a positive multiple of 32");
  const int64_t nblk = (k + 63) / 64;
  if (w_units) *w_units = nblk * n * (w_dtype == MOE_E2M1X2 ? 32 : 64);
  if (scale_bytes) *scale_bytes = w_dtype == MOE_BF16 ? 0 : nblk * 2 * n;
  return ok();
}

moe_status moe_pack_weights(int32_t w_dtype, int32_t num_experts, int64_t n, int64_t k, const void* w,
                            int64_t w_stride_e, int64_t w_ld, const uint8_t* w_scale, int64_t w_scale_stride_e,
                            int64_t w_scale_ld, void* w_out, uint8_t* w_scale_out, moe_stream_t stream) {
  int64_t out_units = 0, out_scale = 0;
  moe_status st = moe_packed_sizes(w_dtype, n, k, &out_units, &out_scale);
  if (st != MOE_OK) return st;
  if (num_experts < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "num_experts < 0");
  const int64_t eb = w_dtype == MOE_BF16 ? 2 : 1;
  const int64_t row_units = w_dtype == MOE_E2M1X2 ? k / 2 : k;
  if (w_ld < row_units || w_stride_e < n * w_ld || (w_ld * eb) % 16 != 0 || (w_stride_e * eb) % 16 != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "w strides must cover the rows and be multiples of 16 bytes");
  if (w_dtype == MOE_E4M3 && w_scale == nullptr && w_scale_out == nullptr) {
    // E4M3 codes without block scales (the per-token path's weights)
  } else if (w_dtype != MOE_BF16) {
    if (w_scale == nullptr || w_scale_out == nullptr)
      return fail(MOE_ERR_INVALID_ARGUMENT, "scales are required for block-scaled weights");
    if (w_scale_ld < k / 32 || w_scale_stride_e < n * w_scale_ld)
      return fail(MOE_ERR_INVALID_ARGUMENT, "w_scale strides too small");
  }
  if (num_experts == 0) return ok();
  if (w == nullptr || w_out == nullptr) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (((uintptr_t)w | (uintptr_t)w_out) % 16 != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "w and w_out must be 16-byte aligned");
  const uint8_t* wi = static_cast<const uint8_t*>(w);
  const uint8_t* wo = static_cast<const uint8_t*>(w_out);
  const int64_t in_bytes = ((int64_t)num_experts - 1) * w_stride_e * eb + n * w_ld * eb;
  const int64_t out_bytes = (int64_t)num_experts * out_units * eb;
  if (wi < wo + out_bytes && wo < wi + in_bytes) return fail(MOE_ERR_INVALID_ARGUMENT, "w and w_out overlap");
  st = check_device();
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_pack(wi, w_stride_e * eb, w_ld * eb, w_scale, w_scale_stride_e, w_scale_ld,
                                     num_experts, (int32_t)n, (int32_t)k, (int32_t)((w_dtype == MOE_E2M1X2 ? 32 : 64) * eb),
                                     static_cast<uint8_t*>(w_out), w_scale_out, (hipStream_t)stream),
                    "moe_pack_weights launch");
}

moe_status moe_combine(const void* c, int64_t c_ld, const float* topk_w, int64_t num_tokens, int32_t top_k,
                       int64_t n, void* y, int64_t y_ld, moe_stream_t stream) {
  if (num_tokens < 0 || top_k < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "num_tokens < 0 or top_k < 1");
  if (n < 8 || n % 8 != 0 || n >= INT32_MAX) return fail(MOE_ERR_INVALID_ARGUMENT, "n must be a positive multiple of 8");
  if (c_ld < n || c_ld % 8 != 0 || y_ld < n || y_ld % 8 != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "c_ld and y_ld must be >= n and multiples of 8");
  if (num_tokens > 0 && (c == nullptr || topk_w == nullptr || y == nullptr))
    return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (((uintptr_t)c | (uintptr_t)y) % 16 != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "c and y must be 16-byte aligned");
  if (num_tokens * (n / 8) >= (int64_t)INT32_MAX * 128)
    return fail(MOE_ERR_UNSUPPORTED, "problem too large for one launch");
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_combine(static_cast<const uint16_t*>(c), c_ld, topk_w, num_tokens, top_k, n,
                                        static_cast<uint16_t*>(y), y_ld, (hipStream_t)stream),
                    "moe_combine launch");
}

moe_status moe_quantize_mxfp8(const void* x, int64_t x_ld, int64_t rows, int64_t k, void* q, int64_t q_ld,
                              uint8_t* scales, int64_t scales_ld, moe_stream_t stream) {
  if (rows < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "rows < 0");
  if (k < 32 || k % 32 != 0 || k >= INT32_MAX) return fail(MOE_ERR_INVALID_ARGUMENT, "k must be a positive multiple of 32");
  if (x_ld < k || x_ld % 8 != 0) return fail(MOE_ERR_INVALID_ARGUMENT, "x_ld must be >= k and a multiple of 8");
  if (q_ld < k || q_ld % 16 != 0) return fail(MOE_ERR_INVALID_ARGUMENT, "q_ld must be >= k and a multiple of 16");
  if (scales_ld < k / 32) return fail(MOE_ERR_INVALID_ARGUMENT, "scales_ld must be >= k / 32");
  if (rows > 0 && (x == nullptr || q == nullptr || scales == nullptr))
    return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (((uintptr_t)x | (uintptr_t)q) % 16 != 0) return fail(MOE_ERR_INVALID_ARGUMENT, "x and q must be 16-byte aligned");
  if (rows > INT64_MAX / k) return fail(MOE_ERR_INVALID_ARGUMENT, "rows * k overflows");
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_quant_mxfp8(static_cast<const uint16_t*>(x), x_ld, rows, k, static_cast<uint8_t*>(q),
                                            q_ld, scales, scales_ld, (hipStream_t)stream),
                    "moe_quantize_mxfp8 launch");
}

moe_status moe_wgrad(const void* x, int64_t x_ld, const void* grad, int64_t grad_ld,
                     const int32_t* sorted_token_ids, const int32_t* expert_ids,
                     const int32_t* num_tokens_post_pad, int64_t num_tokens, int32_t top_k,
                     int32_t num_experts, int64_t n, int64_t k, int32_t block_m, int64_t max_blocks,
                     float* dw, moe_stream_t stream) {
  if (num_tokens < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "num_tokens < 0");
  if (top_k < 1 || num_experts < top_k)
    return fail(MOE_ERR_INVALID_ARGUMENT, "need 1 <= top_k (%d) <= num_experts (%d)", top_k, num_experts);
  if (num_experts > kAlignMaxExperts)
    return fail(MOE_ERR_UNSUPPORTED, "num_experts %d > %d", num_experts, kAlignMaxExperts);
  if (n < 32 || n % 32 != 0 || k < 32 || k % 32 != 0 || n >= INT32_MAX || k >= INT32_MAX)
    return fail(MOE_ERR_INVALID_ARGUMENT, "n and k must be positive multiples of 32");
  if (x_ld < k || x_ld % 8 != 0 || grad_ld < n || grad_ld % 8 != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "x_ld / grad_ld must cover a row and be multiples of 8");
  if (block_m != moe::wgrad_block_m())
    return fail(MOE_ERR_INVALID_ARGUMENT, "block_m %d, expected %d", block_m, moe::wgrad_block_m());
  const int64_t S = num_tokens * top_k;
  if (S >= INT32_MAX) return fail(MOE_ERR_INVALID_ARGUMENT, "num_tokens * top_k must be < 2^31");
  const int64_t need = moe_align_max_blocks(S, num_experts, block_m);
  if (max_blocks < need)
    return fail(MOE_ERR_INVALID_ARGUMENT, "max_blocks %lld < required %lld", (long long)max_blocks,
                (long long)need);
  if (max_blocks * block_m >= INT32_MAX) return fail(MOE_ERR_INVALID_ARGUMENT, "max_blocks too large");
  // the kernel runs even with no slots (it writes dW as zeros) and reads the
  // routing arrays whenever they have blocks
  if (dw == nullptr || (S > 0 && (x == nullptr || grad == nullptr)) ||
      (max_blocks > 0 && (sorted_token_ids == nullptr || expert_ids == nullptr)))
    return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (((uintptr_t)x | (uintptr_t)grad | (uintptr_t)dw) % 16 != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "x, grad and dw must be 16-byte aligned");
  const int64_t tiles = (int64_t)num_experts * ((n + 255) / 256) * ((k + 255) / 256);
  if (tiles >= (int64_t)INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "too many dW tiles");
  // x and grad are read through 32-bit buffer offsets
  if (num_tokens * x_ld * 2 >= (int64_t)0x80000000 || S * grad_ld * 2 >= (int64_t)0x80000000 ||
      n * k * 4 >= (int64_t)0x80000000)
    return fail(MOE_ERR_UNSUPPORTED, "x, grad or one expert's dW spans 2 GB or more");
  (void)num_tokens_post_pad;
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  moe::WgradParams p;
  p.x = static_cast<const uint16_t*>(x);
  p.x_ld = x_ld;
  p.grad = static_cast<const uint16_t*>(grad);
  p.grad_ld = grad_ld;
  p.sorted = sorted_token_ids;
  p.expert_ids = expert_ids;
  p.S = (int32_t)S;
  p.top_k = top_k;
  p.E = num_experts;
  p.N = (int32_t)n;
  p.K = (int32_t)k;
  p.max_blocks = (int32_t)max_blocks;
  p.tiles_n = 0;
  p.tiles_k = 0;
  p.dw = dw;
  return hip_status(moe::launch_wgrad(p, (hipStream_t)stream), "moe_wgrad launch");
}

moe_status moe_block_mapping(const int32_t* group_sizes, int32_t num_experts, int64_t rows, int32_t block_m,
                             int32_t* block_expert_ids, int32_t* block_token_offsets, int32_t* block_token_ends,
                             int64_t max_blocks, int32_t* total_rows, moe_stream_t stream) {
  if (num_experts < 1 || num_experts > 1024) return fail(MOE_ERR_INVALID_ARGUMENT, "need 1 <= num_experts <= 1024");
  if (rows < 0 || rows >= INT32_MAX) return fail(MOE_ERR_INVALID_ARGUMENT, "rows must be in [0, 2^31)");
  if (block_m < 1 || block_m > 256) return fail(MOE_ERR_INVALID_ARGUMENT, "need 1 <= block_m <= 256");
  const int64_t need = moe_align_max_blocks(rows, num_experts, block_m);
  if (max_blocks < need)
    return fail(MOE_ERR_INVALID_ARGUMENT, "max_blocks %lld < required %lld", (long long)max_blocks,
                (long long)need);
  if (max_blocks * block_m >= INT32_MAX) return fail(MOE_ERR_INVALID_ARGUMENT, "max_blocks * block_m too large");
  if (group_sizes == nullptr ||
      (max_blocks > 0 && (block_expert_ids == nullptr || block_token_offsets == nullptr || block_token_ends == nullptr)))
    return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer argument");
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_block_map(group_sizes, num_experts, block_m, (int32_t)rows, block_expert_ids,
                                          block_token_offsets, block_token_ends, (int32_t)max_blocks, total_rows,
                                          (hipStream_t)stream),
                    "moe_block_mapping launch");
}

moe_status moe_grouped_gemm_per_token(const moe_per_token_args* g, moe_stream_t stream) {
  if (g == nullptr) return fail(MOE_ERR_INVALID_ARGUMENT, "args is null");
  const moe_per_token_args& a = *g;
  if (a.rows < 0 || a.rows >= INT32_MAX) return fail(MOE_ERR_INVALID_ARGUMENT, "rows must be in [0, 2^31)");
  if (a.num_experts < 1 || a.num_experts > 1024) return fail(MOE_ERR_INVALID_ARGUMENT, "need 1 <= num_experts <= 1024");
  if (a.n < 1 || a.n >= INT32_MAX) return fail(MOE_ERR_INVALID_ARGUMENT, "n out of range");
  if (a.k < 16 || a.k % 16 != 0 || a.k >= INT32_MAX)
    return fail(MOE_ERR_INVALID_ARGUMENT, "k (%lld) must be a positive multiple of 16", (long long)a.k);
  if (a.a_ld < a.k || a.a_ld % 16 != 0) return fail(MOE_ERR_INVALID_ARGUMENT, "a_ld must be >= k and a multiple of 16");
  if (a.w_layout != MOE_LAYOUT_ROWS && a.w_layout != MOE_LAYOUT_KBLOCK)
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown w_layout %d", a.w_layout);
  const bool kblock = a.w_layout == MOE_LAYOUT_KBLOCK;
  if (kblock && a.k % 32 != 0) return fail(MOE_ERR_INVALID_ARGUMENT, "the K-block layout needs k %% 32 == 0");
  const int64_t nblk = (a.k + 63) / 64;
  if (a.w_ld % 16 != 0 || a.w_stride_e % 16 != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "w_ld and w_stride_e must be multiples of 16 bytes");
  if (!kblock) {
    if (a.w_ld < a.k) return fail(MOE_ERR_INVALID_ARGUMENT, "w_ld must cover a row");
    if (a.w_stride_e < a.n * a.w_ld) return fail(MOE_ERR_INVALID_ARGUMENT, "w_stride_e < n * w_ld");
  } else {
    if (a.w_ld < a.n * 64) return fail(MOE_ERR_INVALID_ARGUMENT, "w_ld must cover a K block of n rows");
    if (a.w_stride_e < nblk * a.w_ld) return fail(MOE_ERR_INVALID_ARGUMENT, "w_stride_e < ceil(k/64) * w_ld");
  }
  if (a.bias != nullptr && (a.bias_stride_e < 0 || a.bias_stride_n < 0))
    return fail(MOE_ERR_INVALID_ARGUMENT, "negative bias stride");
  if (a.c_ld < a.n) return fail(MOE_ERR_INVALID_ARGUMENT, "c_ld must be >= n");
  if (a.block_m != moe::gemm_block_m_f8())
    return fail(MOE_ERR_INVALID_ARGUMENT, "block_m %d, expected %d", a.block_m, moe::gemm_block_m_f8());
  const int64_t need = moe_align_max_blocks(a.rows, a.num_experts, a.block_m);
  if (a.max_blocks < need)
    return fail(MOE_ERR_INVALID_ARGUMENT, "max_blocks %lld < required %lld", (long long)a.max_blocks,
                (long long)need);
  if (a.max_blocks * a.block_m >= INT32_MAX) return fail(MOE_ERR_INVALID_ARGUMENT, "max_blocks too large");
  if (a.rows > 0 && (a.a == nullptr || a.a_scale == nullptr || a.w == nullptr || a.w_scale == nullptr ||
                     a.c == nullptr || a.block_expert_ids == nullptr || a.block_token_offsets == nullptr ||
                     a.block_token_ends == nullptr))
    return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (((uintptr_t)a.a | (uintptr_t)a.w) % 16 != 0 || (uintptr_t)a.c % 2 != 0 ||
      ((uintptr_t)a.a_scale | (uintptr_t)a.w_scale) % 4 != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "a and w must be 16-byte aligned, c 2-byte, the scales 4-byte");
  constexpr int64_t kBufMax = (int64_t)0x80000000;
  const int64_t w_span = (kblock ? nblk : a.n) * a.w_ld;
  if (a.rows * a.a_ld >= kBufMax || w_span >= kBufMax)
    return fail(MOE_ERR_UNSUPPORTED, "A or one expert's weights span 2 GB or more");
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  if (a.rows == 0 || a.max_blocks == 0) return ok();
  if (a.max_blocks * ((a.n + 511) / 512) >= (int64_t)UINT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "grid too large");

  moe::GemmParams p{};
  p.a = static_cast<const uint16_t*>(static_cast<const void*>(a.a));
  p.a_ld = a.a_ld;
  p.a_rows = a.rows;
  p.a_row_div = 1;
  p.w = a.w;
  p.w_stride_e = a.w_stride_e;
  p.w_row = kblock ? 64 : a.w_ld;
  p.w_blk = kblock ? a.w_ld : 64;
  p.w_span = w_span;
  p.bias = static_cast<const uint16_t*>(a.bias);
  p.bias_se = a.bias_stride_e;
  p.bias_sn = a.bias_stride_n;
  p.c = static_cast<uint16_t*>(a.c);
  p.c_ld = a.c_ld;
  p.expert_ids = a.block_expert_ids;
  p.blk_off = a.block_token_offsets;
  p.blk_end = a.block_token_ends;
  p.tok_scale = a.a_scale;
  p.exp_scale = a.w_scale;
  p.S = (int32_t)a.rows;
  p.N = (int32_t)a.n;
  p.K = (int32_t)a.k;
  p.E = a.num_experts;
  p.max_blocks = (int32_t)a.max_blocks;
  return hip_status(moe::launch_gemm_per_token(p, a.bias != nullptr, (hipStream_t)stream),
                    "moe_grouped_gemm_per_token launch");
}

}  // extern "C"
