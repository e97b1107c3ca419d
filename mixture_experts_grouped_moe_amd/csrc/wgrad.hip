// moe_wgrad: dW[e] = sum over the slots s routed to e of grad[s]^T x[s / top_k],
// fp32, straight from moe_align's sorted_token_ids / expert_ids.
//
// Follows ROCm/aiter PR #5310 "Add MoE GEMM variants and weight-gradient
// kernel": Summary (moe_wgrad replaces sort + pad + bmm and a host sync; its
// atomics needed dW reset between benchmark trials or results were corrupted)
// and Tests & Benchmarks (constant input, linearity, zero-padded tokens).
//
// Design for gfx950: every workgroup owns one (expert, 128 x 128) tile of dW
// and loops over that expert's routing blocks (64 slots each), contracting
// over slots on v_mfma_f32_32x32x16_bf16; it writes its tile once, so dW is
// overwritten (never accumulated into), empty experts get zeros, nothing is
// atomic and repeated calls give identical bits. The contraction runs over
// the slot dimension, which is strided in both operands, so the slot-major
// tiles are transposed on their way into LDS. The expert's block range is
// found by a 64-way search of expert_ids by one wave.
#include "common.h"
#include "params.h"

namespace moe {

constexpr int kWgBM = 64;   // routing block (contraction step)
constexpr int kWgTN = 128;  // dW rows (N) per workgroup
constexpr int kWgTK = 128;  // dW columns (K) per workgroup
constexpr int kWgPitch = kWgBM + 8;  // LDS row pitch (bf16) of the transposed tiles


// First block index b in [0, nb) whose expert is >= target (sentinel -1
// blocks count as +infinity); nb when there is none. Called by one full wave.
__device__ int first_block_at_least(const int32_t* expert_ids, int nb, int target, int lane) {
  int lo = 0, hi = nb;  // answer in [lo, hi]
  while (hi - lo > kWave) {
    const int step = (hi - lo + kWave - 1) / kWave;
    const int idx = lo + lane * step;
    bool ge = true;
    if (idx < hi) {
      const int v = expert_ids[idx];
      ge = (v < 0) || (v >= target);
    }
    const uint64_t m = __ballot(ge);
    const int f = m ? __ffsll((unsigned long long)m) - 1 : kWave;  // first sample >= target
    if (f == 0) return lo;  // key(lo) >= target
    const int new_lo = lo + (f - 1) * step + 1;
    const int new_hi = min(hi, lo + f * step);
    lo = new_lo;
    hi = new_hi;
  }
  const int idx = lo + lane;
  bool ge = true;
  if (idx < hi) {
    const int v = expert_ids[idx];
    ge = (v < 0) || (v >= target);
  }
  const uint64_t m = __ballot(ge && idx < hi);
  return m ? lo + __ffsll((unsigned long long)m) - 1 : hi;
}

__global__ __launch_bounds__(256) void wgrad_kernel(WgradParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t gt[kWgTN][kWgPitch];  // grad^T tile [n][slot]
  __shared__ __attribute__((aligned(16))) uint16_t xt[kWgTK][kWgPitch];  // x^T tile [k][slot]
  __shared__ int32_t s_slot[kWgBM];
  __shared__ int32_t s_range[2];

  const uint32_t L = xcd_remap(blockIdx.x, gridDim.x);
  const int per_e = p.tiles_n * p.tiles_k;
  const int e = L / per_e;
  const int rem = L % per_e;
  const int tn = rem / p.tiles_k, tk = rem % p.tiles_k;
  const int n0 = tn * kWgTN, k0 = tk * kWgTK;

  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int l32 = lane % 32, h = lane / 32;
  if (wave == 0) {
    const int b0 = first_block_at_least(p.expert_ids, p.max_blocks, e, lane);
    if (lane == 0) s_range[0] = b0;
  } else if (wave == 1) {
    const int b1 = first_block_at_least(p.expert_ids, p.max_blocks, e + 1, lane);
    if (lane == 0) s_range[1] = b1;
  }
  __syncthreads();
  const int b0 = s_range[0], b1 = s_range[1];

  // waves 2 x 2: wave (wn, wk) computes rows n0 + wn*64 .. and cols k0 + wk*64 ..
  const int wn = wave / 2, wk = wave % 2;
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  for (int b = b0; b < b1; ++b) {
    __syncthreads();
    if (tid < kWgBM) s_slot[tid] = p.sorted[(int64_t)b * kWgBM + tid];
    __syncthreads();
    // load 64 slot rows x 128 columns of grad and of x (16-byte chunks),
    // write them transposed: gt[n][m], xt[k][m]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // 1024 chunks: 64 slot rows x 16 column chunks; a wave takes one chunk
      // column of all 64 rows so its transposed LDS writes are consecutive.
      const int m = lane, c = wave + 4 * i;
      const int s = s_slot[m];
      u32x4_t gv = {0, 0, 0, 0}, xv = {0, 0, 0, 0};
      if (s < p.S) {
        const int gn = n0 + c * 8, xk = k0 + c * 8;
        if (gn < p.N) gv = *reinterpret_cast<const u32x4_t*>(p.grad + (int64_t)s * p.grad_ld + gn);
        if (xk < p.K) xv = *reinterpret_cast<const u32x4_t*>(p.x + (int64_t)(s / p.top_k) * p.x_ld + xk);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        gt[c * 8 + 2 * q][m] = (uint16_t)(gv[q] & 0xffffu);
        gt[c * 8 + 2 * q + 1][m] = (uint16_t)(gv[q] >> 16);
        xt[c * 8 + 2 * q][m] = (uint16_t)(xv[q] & 0xffffu);
        xt[c * 8 + 2 * q + 1][m] = (uint16_t)(xv[q] >> 16);
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int m0 = ks * 16 + h * 8;
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&gt[wn * 64 + i * 32 + l32][m0]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&xt[wk * 64 + j * 32 + l32][m0]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  float* out = p.dw + (int64_t)e * p.N * p.K;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int k = k0 + wk * 64 + j * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = n0 + wn * 64 + i * 32 + (r / 4) * 8 + h * 4 + (r % 4);
        if (n < p.N && k < p.K) out[(int64_t)n * p.K + k] = acc[i][j][r];
      }
    }
}

int wgrad_block_m() { return kWgBM; }

hipError_t launch_wgrad(const WgradParams& p_in, hipStream_t stream) {
  WgradParams p = p_in;
  p.tiles_n = (p.N + kWgTN - 1) / kWgTN;
  p.tiles_k = (p.K + kWgTK - 1) / kWgTK;
  const int64_t grid = (int64_t)p.E * p.tiles_n * p.tiles_k;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(wgrad_kernel, dim3((uint32_t)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace moe
