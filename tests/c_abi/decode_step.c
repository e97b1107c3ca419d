/*
 * A plain C99 caller of libmoe (no C++, no Python, no torch): one decode step
 * of three tokens through moe_align -> moe_grouped_gemm -> moe_combine and
 * through moe_decode_layer, on device buffers from hipMalloc, checked against
 * the closed form of its inputs.
 *
 * Inputs (every value exact in bf16): x[t][k] = (t + 1) / 2, expert weights
 * W[e][n][k] = (e + 1 + n % 2) / 4, token t routed to experts t and t + 1
 * with weights 3/4 and 1/4. Then every product sum is exact:
 *   C[t * 2 + j][n] = 16 (t + 1) (t + j + 1 + n % 2)       (K = 128)
 *   y[t][n]         = 16 (t + 1) (t + 5/4 + n % 2)
 * and both paths must give exactly these bf16 values.
 *
 * Exit status 0 and "ok" on success; 1 and a message otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe.h"

enum { T = 3, TOPK = 2, E = 4, N = 64, K = 128 };

static uint16_t to_bf16(float f) {  /* truncation: exact for the values used here */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

static float from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

#define HIP_OK(call)                                                     \
  do {                                                                   \
    hipError_t e_ = (call);                                              \
    if (e_ != hipSuccess) {                                              \
      printf("%s failed: %s\n", #call, hipGetErrorString(e_));           \
      return 1;                                                          \
    }                                                                    \
  } while (0)

#define MOE_OK(call)                                                     \
  do {                                                                   \
    moe_status s_ = (call);                                              \
    if (s_ != MOE_OK) {                                                  \
      printf("%s failed: %s (%s)\n", #call, moe_status_string(s_),       \
             moe_last_error());                                          \
      return 1;                                                          \
    }                                                                    \
  } while (0)

int main(void) {
  static uint16_t x[T * K], w[E * N * K], c[T * TOPK * N], y3[T * N], y1[T * N];
  int32_t ids[T * TOPK];
  float topk_w[T * TOPK];
  for (int t = 0; t < T; ++t)
    for (int k = 0; k < K; ++k) x[t * K + k] = to_bf16(0.5f * (float)(t + 1));
  for (int e = 0; e < E; ++e)
    for (int n = 0; n < N; ++n)
      for (int k = 0; k < K; ++k) w[(e * N + n) * K + k] = to_bf16(0.25f * (float)(e + 1 + n % 2));
  for (int t = 0; t < T; ++t) {
    ids[t * TOPK] = t;
    ids[t * TOPK + 1] = t + 1;
    topk_w[t * TOPK] = 0.75f;
    topk_w[t * TOPK + 1] = 0.25f;
  }

  const int32_t block_m = moe_gemm_block_m(MOE_BF16, MOE_BF16, T);
  const int64_t max_blocks = moe_align_max_blocks(T * TOPK, E, block_m);
  if (block_m <= 0 || max_blocks <= 0) {
    printf("block_m %d, max_blocks %lld\n", block_m, (long long)max_blocks);
    return 1;
  }

  void *x_d, *w_d, *c_d, *y3_d, *y1_d, *ids_d, *tw_d, *sorted_d, *eids_d, *npad_d;
  HIP_OK(hipMalloc(&x_d, sizeof x));
  HIP_OK(hipMalloc(&w_d, sizeof w));
  HIP_OK(hipMalloc(&c_d, sizeof c));
  HIP_OK(hipMalloc(&y3_d, sizeof y3));
  HIP_OK(hipMalloc(&y1_d, sizeof y1));
  HIP_OK(hipMalloc(&ids_d, sizeof ids));
  HIP_OK(hipMalloc(&tw_d, sizeof topk_w));
  HIP_OK(hipMalloc(&sorted_d, (size_t)(max_blocks * block_m) * sizeof(int32_t)));
  HIP_OK(hipMalloc(&eids_d, (size_t)max_blocks * sizeof(int32_t)));
  HIP_OK(hipMalloc(&npad_d, sizeof(int32_t)));
  HIP_OK(hipMemcpy(x_d, x, sizeof x, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(w_d, w, sizeof w, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(ids_d, ids, sizeof ids, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(tw_d, topk_w, sizeof topk_w, hipMemcpyHostToDevice));

  moe_gemm_args a;
  memset(&a, 0, sizeof a);
  a.num_tokens = T;
  a.top_k = TOPK;
  a.num_experts = E;
  a.n = N;
  a.k = K;
  a.a_dtype = MOE_BF16;
  a.a_row_div = TOPK;
  a.a = x_d;
  a.a_ld = K;
  a.w_dtype = MOE_BF16;
  a.w_layout = MOE_LAYOUT_ROWS;
  a.w = w_d;
  a.w_stride_e = (int64_t)N * K;
  a.w_ld = K;
  a.epilogue = MOE_EPILOGUE_NONE;
  a.c = c_d;
  a.c_ld = N;
  a.sorted_token_ids = (const int32_t*)sorted_d;
  a.expert_ids = (const int32_t*)eids_d;
  a.num_tokens_post_pad = (const int32_t*)npad_d;
  a.block_m = block_m;
  a.max_blocks = max_blocks;

  /* the three launches, then the fused layer, all on the null stream */
  MOE_OK(moe_align((const int32_t*)ids_d, T, TOPK, E, block_m, (int32_t*)sorted_d, (int32_t*)eids_d,
                   (int32_t*)npad_d, max_blocks, NULL));
  MOE_OK(moe_grouped_gemm(&a, NULL));
  MOE_OK(moe_combine(c_d, N, (const float*)tw_d, T, TOPK, N, y3_d, N, NULL));
  a.c = NULL; /* the fused layer writes y only */
  MOE_OK(moe_decode_layer(&a, (const int32_t*)ids_d, (const float*)tw_d, y1_d, N, NULL));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(c, c_d, sizeof c, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(y3, y3_d, sizeof y3, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(y1, y1_d, sizeof y1, hipMemcpyDeviceToHost));

  int bad = 0;
  for (int t = 0; t < T; ++t)
    for (int n = 0; n < N; ++n) {
      for (int j = 0; j < TOPK; ++j) {
        const float want = 16.0f * (float)(t + 1) * (float)(t + j + 1 + n % 2);
        const float got = from_bf16(c[(t * TOPK + j) * N + n]);
        if (got != want && bad++ < 5) printf("C[%d][%d] = %g, expected %g\n", t * TOPK + j, n, got, want);
      }
      const float want = 16.0f * (float)(t + 1) * ((float)t + 1.25f + (float)(n % 2));
      const float got3 = from_bf16(y3[t * N + n]), got1 = from_bf16(y1[t * N + n]);
      if (got3 != want && bad++ < 5) printf("y (three launches)[%d][%d] = %g, expected %g\n", t, n, got3, want);
      if (got1 != want && bad++ < 5) printf("y (fused layer)[%d][%d] = %g, expected %g\n", t, n, got1, want);
    }

  hipFree(x_d);
  hipFree(w_d);
  hipFree(c_d);
  hipFree(y3_d);
  hipFree(y1_d);
  hipFree(ids_d);
  hipFree(tw_d);
  hipFree(sorted_d);
  hipFree(eids_d);
  hipFree(npad_d);
  if (bad) {
    printf("%d values differ\n", bad);
    return 1;
  }
  printf("ok\n");
  return 0;
}
