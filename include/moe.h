/*
 * moe.h - C ABI of libmoe: the routed, block-scaled MoE expert-layer hot path
 * on one AMD Instinct MI355X (gfx950).
 *
 * Pages the operations come from (cited by title and section):
 *   [TRT]  TensorRT-LLM PR #15311 "Bound Triton MoE JIT specializations via
 *          token-dim bucketing and warmup"
 *   [TA]   torchada PR #115 "tune the Nemotron MTP decode row on S5000 with a
 *          checked-in recipe"
 *   [AIT]  ROCm/aiter PR #5310 "[Triton/Gluon] Add MoE GEMM variants and
 *          weight-gradient kernel"
 *
 * Conventions for every entry point:
 *   - Pointers marked (device) are caller-owned device memory; (host) is host
 *     memory. The library never allocates, frees or synchronizes: every device
 *     call is asynchronous on `stream` (a hipStream_t; NULL = null stream).
 *   - Arguments are validated on the host before anything is launched; a
 *     rejected call returns an error code, touches no memory and launches
 *     nothing. moe_last_error() then holds a message (thread-local).
 *   - Device-resident data (routing ids, scale bytes) is not inspected: expert
 *     ids outside [0, E) are not routed; an E8M0 byte of 0xFF yields NaN.
 *   - Device faults are asynchronous and surface at the caller's next
 *     synchronization; the library does not catch them.
 *   - Slot s = t * top_k + j indexes the flattened routing [T, top_k].
 *   - PAD = T * top_k marks an unused position of sorted_token_ids.
 *   - All element offsets are formed in 64-bit arithmetic ([AIT] Notes: expert
 *     255 of a 256-expert layer with N*K = 14.7M starts past INT32_MAX).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* moe_stream_t; /* a hipStream_t */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1, /* a null pointer, a bad size, stride or combination */
  MOE_ERR_UNSUPPORTED = 2,      /* valid but not implemented (e.g. not a gfx950 device) */
  MOE_ERR_HIP = 4               /* a HIP runtime call failed; see moe_last_error() */
} moe_status;

/* Element encodings. */
typedef enum {
  MOE_BF16 = 1,   /* bfloat16 */
  MOE_FP32 = 2,   /* float */
  MOE_E4M3 = 3,   /* OCP E4M3 "FN" byte (MXFP8 element) */
  MOE_E2M1X2 = 4, /* two OCP E2M1 codes per byte (MXFP4): element 2i in the low nibble */
  MOE_E8M0 = 5,   /* MX scale byte b: 2^(b - 127); 0xFF = NaN */
  MOE_I32 = 6
} moe_dtype;

/* Weight layouts (a storage unit is an element, or a byte of two codes for
 * MOE_E2M1X2; R = 64 elements = 64 units, 32 for MOE_E2M1X2).
 *   MOE_LAYOUT_ROWS:   code (e, n, k) at unit e*w_stride_e + n*w_ld + k (k/2
 *                      for E2M1X2); scale byte (e, n, k/32) at
 *                      e*w_scale_stride_e + n*w_scale_ld + k/32. The layout
 *                      the pages' kernels read.
 *   MOE_LAYOUT_KBLOCK: 64-element K blocks outermost: code (e, n, k) at unit
 *                      e*w_stride_e + (k/64)*w_ld + n*R + (k%64) (halved for
 *                      E2M1X2), i.e. for every K block all N rows' 64 codes
 *                      back to back; scale byte (e, n, k/32) at
 *                      e*w_scale_stride_e + (k/64)*w_scale_ld + 2n + (k/32)%2.
 *                      Made by moe_pack_weights. A K block's codes for a run
 *                      of consecutive rows are one contiguous piece, so the
 *                      large-M kernel's weight loads are whole cache lines.
 *                      A library layout, not one from the pages; the values
 *                      are the same, so every result is identical. */
typedef enum {
  MOE_LAYOUT_ROWS = 0,
  MOE_LAYOUT_KBLOCK = 1
} moe_layout;

typedef enum {
  MOE_EPILOGUE_NONE = 0,
  /* h[:, j] = silu(pre[:, j]) * pre[:, N/2 + j], silu(z) = z / (1 + e^-z);
     output width N/2. Gate = first half of the N weight rows, up = second. */
  MOE_EPILOGUE_SWIGLU = 1,
  /* h = max(pre, 0)^2 elementwise, output width N: the non-gated squared
     ReLU ("relu2_no_mul") of [TA] "Follow-up on this table" (the Nemotron
     decode shape, E=128, hidden 2688, N=1856, top-6) */
  MOE_EPILOGUE_RELU2 = 2
} moe_epilogue;

/* ------------------------------------------------------------------------
 * Host helpers (pure, thread-safe, no GPU needed)
 * ---------------------------------------------------------------------- */

/* Token-dimension bucket of m ([TRT] Description and Test Coverage: eight
 * buckets per power-of-two octave, at most 12.5% padding, fixed points,
 * monotonic): m for m < 16, else m rounded up to a multiple of
 * 2^(bitlen(m) - 4). Returns 0 for m = 0 and -1 for m < 0. */
int64_t moe_bucket_round_up(int64_t m);

/* The sorted closure {bucket(m) : 1 <= m <= max_tokens}. Writes up to `cap`
 * values to out (host; may be NULL when cap = 0) and returns the closure's
 * size (so a call with cap = 0 sizes the buffer); -1 if max_tokens < 0. */
int64_t moe_bucket_enumerate(int64_t max_tokens, int64_t* out, int64_t cap);

/* 1 when padding the token dimension cannot change real tokens' outputs:
 * bf16 activations x MXFP4 weights with no dynamic activation scale ([TRT]
 * Description: the padding is restricted to W4A16 MXFP4). 0 otherwise. */
int32_t moe_padding_supported(int32_t a_dtype, int32_t w_dtype, int32_t dynamic_act_scale);

/* Size of the block list for `num_slots` routed slots:
 * floor((S + min(E, S) * (B - 1)) / B), an upper bound on the blocks any
 * routing uses ([AIT] second review: the block list is sized above the real
 * block count; the rest is sentinel blocks). -1 on bad arguments. */
int64_t moe_align_max_blocks(int64_t num_slots, int32_t num_experts, int32_t block_m);

/* BLOCK_M that moe_grouped_gemm expects the routing to be padded to. It
 * depends only on the dtypes and on whether num_tokens <= 32 (the decode
 * variant, [TA] "Follow-up on this table": the tiny-M default for M <= 32).
 * 32 is itself a token bucket, so a padded and an unpadded run of the same
 * tokens always take the same variant. -1 for an unsupported combination. */
int32_t moe_gemm_block_m(int32_t a_dtype, int32_t w_dtype, int64_t num_tokens);

/* BLOCK_M that moe_wgrad expects. */
int32_t moe_wgrad_block_m(void);

/* Largest number of tokens that takes the decode variant (32). */
int64_t moe_decode_max_tokens(void);

const char* moe_status_string(int32_t status);
const char* moe_last_error(void);

/* ------------------------------------------------------------------------
 * Routing ([AIT] Summary: moe_align_block_size's sorted_token_ids and
 * expert_ids; [AIT] second review: sentinel blocks hold expert id -1;
 * [TA] "Follow-up on this table": moe_align_block_size runs before the
 * fused MoE GEMM).
 *
 * topk_ids            (device) int32 [num_tokens, top_k], row-major.
 * sorted_token_ids    (device) int32 [max_blocks * block_m]: for expert e,
 *                     positions [o_e, o_e + c_e) hold e's slots in ascending
 *                     order, where c_e = #slots routed to e, p_e = c_e rounded
 *                     up to a multiple of block_m, o_e = sum of p_e' (e' < e);
 *                     every other position holds PAD.
 * expert_ids          (device) int32 [max_blocks]: block b's expert; -1 for
 *                     every block at or past num_tokens_post_pad / block_m.
 * num_tokens_post_pad (device) int32 [1]: sum of p_e.
 * max_blocks          the length of expert_ids; must be at least
 *                     moe_align_max_blocks(num_tokens * top_k, E, block_m).
 * The result is unique (a stable counting sort), and bit-identical run to run.
 * num_tokens = 0 is legal: writes 0 and max_blocks sentinel blocks.
 * Requirements: 1 <= top_k <= num_experts <= 1024, 1 <= block_m <= 256,
 * num_tokens * top_k <= 2^31 - 2^16. No workspace. */
moe_status moe_align(const int32_t* topk_ids, int64_t num_tokens, int32_t top_k,
                     int32_t num_experts, int32_t block_m,
                     int32_t* sorted_token_ids, int32_t* expert_ids,
                     int32_t* num_tokens_post_pad, int64_t max_blocks,
                     moe_stream_t stream);

/* ------------------------------------------------------------------------
 * Routed grouped GEMM ([AIT] Summary: moe_gemm_mxfp8, every expert's GEMM in
 * one launch, E8M0 microscales per 32 K-elements applied per K-step, optional
 * per-expert bias; [AIT] Notes: K-steps aligned to the 32-element scale
 * blocks, int64 expert offsets; [AIT] second review: sentinel blocks exit at
 * once, bias read through explicit strides; [TRT] Description: W4A16 MXFP4,
 * rows independent; [TA] What it does: bf16 decode at M <= 32).
 *
 * For every block b with 0 <= e = expert_ids[b] < num_experts (a block naming
 * another id is skipped) and every position r of it with slot
 * s = sorted_token_ids[b * block_m + r] < PAD:
 *   pre[n] = sum_k A_hat[s / a_row_div][k] * W_hat[e][n][k] + bias[e][n]
 *   W_hat[e][n][k] = dec(W[e][n][k]) * 2^(w_scale[e][n][k / 32] - 127)
 *   A_hat = A (bf16), or dec(A[r][k]) * 2^(a_scale[r][k / 32] - 127) for
 *   MOE_E4M3 activations (both operands MXFP8: the kernel feeds codes and
 *   scale bytes to gfx950's scaled fp8 MFMA, the a_scale / b_scale form of
 *   [AIT]'s kernel; moe_quantize_mxfp8 makes such activations)
 *   C[s][:] = bf16(pre) (MOE_EPILOGUE_NONE), bf16(swiglu(pre)) (width N/2)
 *             or bf16(max(pre, 0)^2) (MOE_EPILOGUE_RELU2)
 * accumulated in fp32, rounded once to bf16 (nearest-even) at the store.
 * Rows of C for PAD positions and unrouted slots are not written.
 * Weights are dequantized exactly into bf16 (the scale is a power of two)
 * except that products below bf16's subnormal range round to zero.
 * ---------------------------------------------------------------------- */
typedef struct {
  int64_t num_tokens;     /* T: routing rows; slots S = T * top_k; PAD = S */
  int32_t top_k;
  int32_t num_experts;    /* E */
  int64_t n;              /* N: weight rows per expert (pre-epilogue width) */
  int64_t k;              /* K: contraction length */

  int32_t a_dtype;        /* MOE_BF16, or MOE_E4M3 (MXFP8 activations, with
                             MOE_E4M3 weights only) */
  int32_t a_row_div;      /* slot s reads A row s / a_row_div: top_k (A = token
                             rows) or 1 (A = slot rows, e.g. the second GEMM) */
  const void* a;          /* (device) A rows, row r at a + r * a_ld elements */
  int64_t a_ld;           /* >= k */
  const uint8_t* a_scale; /* (device) MOE_E4M3 activations: E8M0 [rows][k/32],
                             row r at a_scale + r * a_scale_ld; else ignored */
  int64_t a_scale_ld;     /* >= k / 32 */

  int32_t w_dtype;        /* MOE_BF16, MOE_E4M3 or MOE_E2M1X2 */
  int32_t w_layout;       /* moe_layout of w and w_scale */
  const void* w;          /* (device) codes of [E][N][K]; strides in storage
                             units (elements; bytes of two codes for E2M1X2) */
  int64_t w_stride_e;     /* ROWS: >= n * w_ld; KBLOCK: >= ceil(k/64) * w_ld */
  int64_t w_ld;           /* ROWS: row stride >= k (k/2 for E2M1X2);
                             KBLOCK: K-block stride >= n * R */
  const uint8_t* w_scale; /* (device) E8M0 of [E][N][K/32]; NULL for MOE_BF16 */
  int64_t w_scale_stride_e; /* ROWS: >= n * w_scale_ld; KBLOCK: >= ceil(k/64) * w_scale_ld */
  int64_t w_scale_ld;     /* ROWS: >= k / 32; KBLOCK: K-block stride >= 2n */

  const void* bias;       /* (device) bf16 [E][N] or NULL */
  int64_t bias_stride_e;  /* in elements; any non-negative strides */
  int64_t bias_stride_n;

  int32_t epilogue;       /* moe_epilogue */
  void* c;                /* (device) bf16 [S][N or N/2], row s at c + s * c_ld */
  int64_t c_ld;           /* >= output width, in elements */

  const int32_t* sorted_token_ids; /* (device) from moe_align */
  const int32_t* expert_ids;       /* (device) */
  const int32_t* num_tokens_post_pad; /* (device) moe_align's padded row count; the
                             large-M bf16-activation kernel takes the number of
                             blocks in use from it (blocks at or past
                             num_tokens_post_pad / block_m must hold -1) */
  int32_t block_m;        /* must equal moe_gemm_block_m(a_dtype, w_dtype, T) */
  int64_t max_blocks;     /* length of expert_ids; only the first
                             moe_align_max_blocks(S, E, block_m) blocks
                             (every block moe_align can fill) are read */
} moe_gemm_args;

/* Requirements: k % 32 == 0 and k >= 32; n >= 1 (even with SwiGLU);
 * a_row_div in {1, top_k}; 16-byte aligned a and w rows (a_ld a multiple of
 * 8; w_ld a multiple of 16 bytes); c_ld >= the output width; A, one
 * expert's weights and one expert's scales each span less than 2 GB.
 * MOE_E4M3 activations: w_dtype MOE_E4M3, a_ld a multiple of 16, a_scale
 * non-null with a_scale_ld >= k / 32, the scales under 2 GB; every token
 * count runs the one scaled-fp8 kernel (no decode variant), whose block_m
 * (128 rows) is the same for every num_tokens. Other combinations:
 * MOE_ERR_UNSUPPORTED.
 * No workspace. */
moe_status moe_grouped_gemm(const moe_gemm_args* args, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * The decode MoE step in one launch: routing, the routed grouped GEMM and the
 * top-k combine for a few tokens ([TA] What it does: the M <= 32 bucket
 * dominates the decode step, where the launches around the GEMM are a fixed
 * cost of every call; "Follow-up on this table": moe_align_block_size and the
 * fused MoE GEMM on the tiny-M path). For token t < T and slot s = t*top_k + j
 * routed to expert e = topk_ids[s] (device, int32 [T][top_k]):
 *   C[s][n] = bf16( epilogue( A[t] . W_hat[e][n] + bias[e][n] ) )
 *   y[t][n] = bf16( sum_{j < top_k, ascending} topk_w[s] * C[s][n] )   (fp32)
 * with the arithmetic of moe_align -> moe_grouped_gemm (decode variant) ->
 * moe_combine, so C and y are bit-identical to those three calls (for
 * T * k <= 76288, see below). A slot
 * whose id lies outside [0, E) contributes 0 to y (and its C row is not
 * written).
 * args describes A (bf16 token rows: a_dtype MOE_BF16, a_row_div = top_k),
 * the weights, scales and bias exactly as for moe_grouped_gemm; epilogue
 * MOE_EPILOGUE_NONE or MOE_EPILOGUE_RELU2. args->c (device, bf16 [S][n], row
 * stride c_ld >= n) receives C when not NULL; no other memory is written
 * besides y. The routing fields (sorted_token_ids, expert_ids,
 * num_tokens_post_pad, block_m, max_blocks) are not read. topk_w (device)
 * fp32 [T][top_k]; y (device) bf16 [T][n], row stride y_ld >= n; every row
 * t < T is written.
 * Limits (moe_decode_layer_fits): T <= 32, T * top_k <= 256, E <= 1024,
 * k <= 4096. The activations of all tokens are held on chip; when T * k >
 * 76288 they are taken in two passes over halves of K (K/2 rounded up to a
 * multiple of 32, then the rest) and each output is the sum of its passes'
 * partial sums, so C and y may then differ
 * from the three launches' in the last bit (both within the parity bar of
 * the exact result). Outside the limits, with SwiGLU or with MOE_E4M3
 * activations: MOE_ERR_UNSUPPORTED. Other requirements as for
 * moe_grouped_gemm.
 * No workspace.
 * ---------------------------------------------------------------------- */
moe_status moe_decode_layer(const moe_gemm_args* args, const int32_t* topk_ids, const float* topk_w,
                            void* y, int64_t y_ld, moe_stream_t stream);

/* 1 when moe_decode_layer takes T tokens of top_k slots over num_experts
 * experts with contraction length k (the limits above), else 0. */
int32_t moe_decode_layer_fits(int64_t num_tokens, int32_t top_k, int32_t num_experts, int64_t k);

/* ------------------------------------------------------------------------
 * Weight repacking (a one-time step at weight-load time, outside the
 * method: it moves codes and scale bytes, computes nothing).
 * Copies E experts' codes and scales from MOE_LAYOUT_ROWS (w, w_scale with
 * the strides of moe_gemm_args) into MOE_LAYOUT_KBLOCK with dense strides:
 *   w_out:       K-block stride n*R units, expert stride ceil(k/64)*n*R units
 *   w_scale_out: K-block stride 2n bytes, expert stride ceil(k/64)*2n bytes
 * (moe_packed_sizes returns both expert strides). When k % 64 == 32 the
 * unused upper half of the last K block is written as zero codes and zero
 * scale bytes; no kernel reads it. w_scale / w_scale_out are NULL for
 * MOE_BF16, and may both be NULL for MOE_E4M3 (codes alone: the weights of
 * moe_grouped_gemm_per_token). Input and output must not overlap. Requirements as for
 * moe_grouped_gemm's weights (k % 32 == 0, 16-byte aligned rows). */
moe_status moe_pack_weights(int32_t w_dtype, int32_t num_experts, int64_t n, int64_t k,
                            const void* w, int64_t w_stride_e, int64_t w_ld,
                            const uint8_t* w_scale, int64_t w_scale_stride_e,
                            int64_t w_scale_ld, void* w_out, uint8_t* w_scale_out,
                            moe_stream_t stream);

/* Expert strides of moe_pack_weights' dense output: *w_units =
 * ceil(k/64) * n * R storage units, *scale_bytes = ceil(k/64) * 2n (0 for
 * MOE_BF16). Either pointer (host) may be NULL. Returns MOE_OK, or
 * MOE_ERR_INVALID_ARGUMENT for a bad dtype or size. */
moe_status moe_packed_sizes(int32_t w_dtype, int64_t n, int64_t k, int64_t* w_units,
                            int64_t* scale_bytes);

/* ------------------------------------------------------------------------
 * MXFP8 conversion of bf16 activations ([AIT] Summary and second review:
 * moe_gemm_mxfp8 takes both operands as E4M3 codes with one E8M0 scale per
 * 32 K-elements, a_scale and b_scale; the pages do not give the conversion,
 * this is the OCP Microscaling v1.0 one). For every row r < rows and block
 * b < k/32, with v = x[r][32b .. 32b+31]:
 *   X = floor(log2(max |v|)) - 8, clamped to [-127, 127]; -127 if all zero
 *   scales[r][b] = X + 127
 *   q[r][32b + i] = E4M3 nearest to v_i / 2^X (ties to even, saturating at
 *                   +-448, sign bit when v_i < 0)
 * x (device) bf16 rows with stride x_ld elements; q (device) uint8 rows with
 * stride q_ld bytes; scales (device) uint8 rows with stride scales_ld.
 * A block holding a NaN or an infinity is written as a NaN block: scale byte
 * 0xFF and every code 0x7F (its dequantised values are all NaN; the other
 * blocks are unaffected).
 * Requirements: k % 32 == 0, k >= 32; x_ld >= k and a multiple of 8; q_ld >= k
 * and a multiple of 16; scales_ld >= k / 32; x and q 16-byte aligned.
 * Otherwise MOE_ERR_INVALID_ARGUMENT, nothing launched.
 * ---------------------------------------------------------------------- */
moe_status moe_quantize_mxfp8(const void* x, int64_t x_ld, int64_t rows, int64_t k,
                              void* q, int64_t q_ld, uint8_t* scales, int64_t scales_ld,
                              moe_stream_t stream);

/* ------------------------------------------------------------------------
 * Top-k combine (the method's final step; [TRT] Description: the padded
 * rows are sliced off after the grouped GEMMs).
 *   y[t][n] = bf16( sum_{j < top_k, ascending} topk_w[t][j] * C[t*top_k + j][n] )
 * in fp32. c (device) bf16 [T*top_k][n] with row stride c_ld; topk_w (device)
 * fp32 [T][top_k]; y (device) bf16 [T][n] with row stride y_ld. Every row
 * t < num_tokens is written. n % 8 == 0, c_ld and y_ld multiples of 8.
 * ---------------------------------------------------------------------- */
moe_status moe_combine(const void* c, int64_t c_ld, const float* topk_w,
                       int64_t num_tokens, int32_t top_k, int64_t n,
                       void* y, int64_t y_ld, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * Expert weight gradient ([AIT] Summary: moe_wgrad, dW[e] = sum over the
 * tokens routed to e of grad[t]^T x input[t], straight from
 * sorted_token_ids / expert_ids; its trial-to-trial corruption came from
 * atomics accumulating into an un-reset dW. Here each output tile is owned by
 * one workgroup and written exactly once, so dW is overwritten, never
 * accumulated into, and repeated calls give identical bits.)
 *   dW[e][n][k] = sum_{slots s routed to e} grad[s][n] * x[s / top_k][k]
 * in fp32; experts with no slots are written as zeros; PAD positions are
 * skipped. x (device) bf16 [T][K], row stride x_ld; grad (device) bf16 [S][N],
 * row stride grad_ld; dw (device) fp32 [E][N][K] contiguous.
 * Requirements: block_m == moe_wgrad_block_m(); num_experts <= 1024;
 * n % 32 == 0, k % 32 == 0; x_ld, grad_ld multiples of 8; x, grad and dw
 * 16-byte aligned; x and grad each span less than 2 GB; the routing arrays
 * non-null whenever max_blocks > 0 (also with no tokens: dW is then written
 * as zeros); x and grad may be NULL when num_tokens = 0.
 * No workspace.
 * ---------------------------------------------------------------------- */
moe_status moe_wgrad(const void* x, int64_t x_ld, const void* grad, int64_t grad_ld,
                     const int32_t* sorted_token_ids, const int32_t* expert_ids,
                     const int32_t* num_tokens_post_pad,
                     int64_t num_tokens, int32_t top_k, int32_t num_experts,
                     int64_t n, int64_t k, int32_t block_m, int64_t max_blocks,
                     float* dw, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * Expert block mapping of the group_sizes interface ([AIT] Summary:
 * moe_gemm_per_token takes a 1-D tensor of per-expert row counts; [AIT]
 * Notes: one block-mapping builder shared by the GEMM wrappers; [AIT] second
 * review: block_expert_ids / block_token_offsets / block_token_ends, -1
 * sentinel blocks past the used ones).
 * Rows are grouped by expert: expert e owns rows [o_e, o_e + g_e) with
 * g_e = group_sizes[e] and o_e = g_0 + ... + g_{e-1}. Its ceil(g_e / block_m)
 * blocks follow in expert order; block i of e has
 *   block_expert_ids[b] = e, block_token_offsets[b] = o_e + i * block_m,
 *   block_token_ends[b] = o_e + g_e (the end of e's rows, not of the block).
 * Every block b past the used ones: expert -1, offset = end = total rows.
 * group_sizes (device) int32 [num_experts]; the three outputs (device) int32
 * [max_blocks]; total_rows (device) int32 [1] or NULL receives
 * sum(max(g_e, 0)) (capped at 2^31 - 1), which the caller may compare with
 * rows. The counts are expected to sum to rows; negative counts count as 0
 * and segments are clipped to [0, rows), so a mapping never names a row at
 * or past rows (blocks beyond max_blocks are dropped).
 * Requirements: 1 <= num_experts <= 1024, 0 <= rows < 2^31,
 * 1 <= block_m <= 256, max_blocks >= moe_align_max_blocks(rows, num_experts,
 * block_m) (the same bound as moe_align: both cut per-expert groups into
 * blocks), max_blocks * block_m < 2^31. One workgroup, no workspace.
 * ---------------------------------------------------------------------- */
moe_status moe_block_mapping(const int32_t* group_sizes, int32_t num_experts, int64_t rows, int32_t block_m,
                             int32_t* block_expert_ids, int32_t* block_token_offsets,
                             int32_t* block_token_ends, int64_t max_blocks, int32_t* total_rows,
                             moe_stream_t stream);

/* ------------------------------------------------------------------------
 * Per-token-scaled FP8 grouped GEMM ([AIT] Summary: moe_gemm_per_token,
 * E4M3 operands, per-token activation scales and per-expert weight scales
 * applied after the fp8 dot-product accumulation, a group_sizes interface;
 * [AIT] Tests & Benchmarks: a bias variant, empty-token guards).
 * For every block b with 0 <= e = block_expert_ids[b] < num_experts and
 * every row r in [block_token_offsets[b], min(+block_m, block_token_ends[b], rows)):
 *   C[r][n] = bf16( (sum_k dec(A[r][k]) * dec(W[e][n][k])) * a_scale[r] * w_scale[e]
 *                   + bias[e][n] )
 * with the dot product accumulated in fp32 (each E4M3 product is exact in
 * fp32), the two scales multiplied in fp32 and one bf16 rounding
 * (nearest-even). Rows no block covers are not written.
 * ---------------------------------------------------------------------- */
typedef struct {
  int64_t rows;            /* R: rows of A and C, the sum of the group sizes */
  int32_t num_experts;     /* E */
  int64_t n;               /* N: weight rows per expert, the output width */
  int64_t k;               /* K: contraction length */
  const uint8_t* a;        /* (device) E4M3 codes [R][K], row r at a + r * a_ld */
  int64_t a_ld;            /* bytes, >= k, a multiple of 16 */
  const float* a_scale;    /* (device) fp32 [R]: the scale of each row of A */
  int32_t w_layout;        /* MOE_LAYOUT_ROWS or MOE_LAYOUT_KBLOCK (E4M3 codes
                              only; moe_pack_weights with both scale pointers
                              NULL makes the latter) */
  const uint8_t* w;        /* (device) E4M3 codes of [E][N][K] */
  int64_t w_stride_e;      /* bytes; ROWS: >= n * w_ld; KBLOCK: >= ceil(k/64) * w_ld */
  int64_t w_ld;            /* bytes; ROWS: row stride >= k; KBLOCK: K-block stride >= 64n */
  const float* w_scale;    /* (device) fp32 [E]: one scale per expert */
  const void* bias;        /* (device) bf16 [E][N] or NULL */
  int64_t bias_stride_e;   /* in elements; any non-negative strides */
  int64_t bias_stride_n;
  void* c;                 /* (device) bf16 [R][N], row r at c + r * c_ld */
  int64_t c_ld;            /* >= n, in elements */
  const int32_t* block_expert_ids;    /* (device) from moe_block_mapping */
  const int32_t* block_token_offsets; /* (device) */
  const int32_t* block_token_ends;    /* (device) */
  int32_t block_m;         /* must equal moe_gemm_block_m(MOE_E4M3, MOE_E4M3, rows) */
  int64_t max_blocks;      /* length of the mapping, >= moe_align_max_blocks(rows, E, block_m) */
} moe_per_token_args;

/* Requirements: k % 16 == 0 (k % 32 == 0 for KBLOCK); w_ld, w_stride_e
 * multiples of 16; a and w 16-byte aligned, c 2-byte, the scales 4-byte; A
 * and one expert's weights each span less than 2 GB. rows = 0 or an empty
 * mapping launch nothing. Otherwise MOE_ERR_INVALID_ARGUMENT or
 * MOE_ERR_UNSUPPORTED, nothing launched. No workspace. */
moe_status moe_grouped_gemm_per_token(const moe_per_token_args* args, moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
