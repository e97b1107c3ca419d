// Decode variant of the routed grouped GEMM (at most 32 tokens): weight
// streaming at HBM speed.
#include "common.h"
#include "params.h"

namespace moe {

constexpr int kThreadsDec = 256;

// ---------------------------------------------------------------------------
// Decode variant (at most 32 tokens): each touched expert's weight rows are
// streamed once from HBM. A workgroup owns (routing block of 8 slots, 16 weight
// rows); each wave streams 4 full rows with 16-byte loads spread over its 64
// lanes, so each lane holds a K-slice of every row, and keeps one fp32 partial
// per (row, slot). The slots' activations are staged in LDS, 2048 K-elements
// at a time. Partials are reduced across the wave at the end (a fixed order,
// so results are reproducible). Splitting N this finely gives thousands of
// workgroups even at one token, enough bytes in flight to fill HBM.
// Follows torchada PR #115 "tune the Nemotron MTP decode row on S5000 with a
// checked-in recipe": What it does (the tiny-M bucket, M <= 32, dominates the
// decode step) and "Follow-up on this table" (the tiny-M path is chosen by
// M <= 32, never by a tuned table).
// ---------------------------------------------------------------------------
constexpr int kDecBM = 8;         // routing block for decode
constexpr int kDecRowsPerWave = 4;
constexpr int kDecRows = 4 * kDecRowsPerWave;  // weight rows per workgroup
constexpr int kDecKC = 2048;      // K elements staged per pass

// Four waves per SIMD (at most 128 VGPRs; the LDS allows four workgroups per
// CU): more weight rows in flight per CU. For bf16 weights this took the
// decode sweep (M = 1 .. 28) from 70% to 74% of HBM bandwidth, same bits.
// The weight codes are read once per call and streamed with non-temporal
// loads: on a cold cache (weights evicted between calls, as in serving) that
// took the bf16 decode GEMM from 74.6 to 50.0 us at M = 7 and from 146 to
// 116 us at M = 28 (a plain streaming read of the same bytes measured alike:
// 74 against 51 us for 278 MB). The weight loads are issued before the
// block's slot list is read, so the list's latency overlaps theirs.
template <int WDT, bool SWIGLU, bool BIAS>
__global__ __launch_bounds__(kThreadsDec, 4) void moe_decode_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[kDecBM][kDecKC];
  __shared__ int32_t s_slot[kDecBM];

  const int b = blockIdx.x % p.max_blocks;
  const int chunk = blockIdx.x / p.max_blocks;
  const int e = p.expert_ids[b];
  if (e < 0 || e >= p.E) return;  // sentinel block (or an id outside this layer's experts)

  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  __shared__ int32_t s_nv;
  int nv = 0;

  // this wave's weight rows (and output columns)
  int32_t wrow[kDecRowsPerWave], ocol[kDecRowsPerWave];
#pragma unroll
  for (int r = 0; r < kDecRowsPerWave; ++r) {
    if (!SWIGLU) {
      const int n = chunk * kDecRows + wave * kDecRowsPerWave + r;
      wrow[r] = n < p.N ? n : -1;
      ocol[r] = wrow[r];
    } else {
      const int half = p.N / 2;
      const int hcol = chunk * (kDecRows / 2) + wave * (kDecRowsPerWave / 2) + (r % 2);
      const bool up = r >= 2;
      wrow[r] = hcol < half ? (up ? half + hcol : hcol) : -1;
      ocol[r] = hcol < half ? hcol : -1;
    }
  }
  const uint8_t* w_base = p.w + (int64_t)e * p.w_stride_e;
  const uint8_t* ws_base = (WDT != W_BF16) ? p.ws + (int64_t)e * p.ws_stride_e : nullptr;

  float acc[kDecRowsPerWave][kDecBM];
#pragma unroll
  for (int r = 0; r < kDecRowsPerWave; ++r)
#pragma unroll
    for (int j = 0; j < kDecBM; ++j) acc[r][j] = 0.0f;

  // raw weight codes of one 8-element piece: 16 B (bf16), 8 B (E4M3), 4 B (E2M1)
  constexpr int kWords = (WDT == W_BF16) ? 4 : (WDT == W_E4M3 ? 2 : 1);
  constexpr int kPer = kDecKC / 8 / kWave;  // 8-element pieces per lane per pass
  for (int kc = 0; kc < p.K; kc += kDecKC) {
    // 1. this wave's weight pieces for the pass ([row][i] holds elements
    //    kc + 8 * (lane + 64 i) .. +8): issued first, so their latency
    //    overlaps the activation staging below
    uint32_t wraw[kDecRowsPerWave][kPer][kWords];
    uint32_t sraw[kDecRowsPerWave][kPer];
#pragma unroll
    for (int r = 0; r < kDecRowsPerWave; ++r) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int k = kc + 8 * (lane + kWave * i);
        const bool ok = wrow[r] >= 0 && k < p.K;
        // codes of row wrow[r], K block k / 64, element k % 64
        const int64_t wb = (int64_t)(ok ? wrow[r] : 0) * p.w_row + (int64_t)(k / 64) * p.w_blk;
        if constexpr (WDT == W_BF16) {
          const u32x4_t v = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(w_base + wb + (k % 64) * 2))
                               : u32x4_t{0, 0, 0, 0};
#pragma unroll
          for (int q = 0; q < 4; ++q) wraw[r][i][q] = v[q];
        } else if constexpr (WDT == W_E4M3) {
          const u32x2_t v = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(w_base + wb + k % 64))
                               : u32x2_t{0, 0};
          wraw[r][i][0] = v[0];
          wraw[r][i][1] = v[1];
        } else {
          wraw[r][i][0] = ok ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(w_base + wb + (k % 64) / 2))
                             : 0u;
        }
        if constexpr (WDT != W_BF16)
          sraw[r][i] = ok ? __builtin_nontemporal_load(
                                &ws_base[(int64_t)wrow[r] * p.ws_row + (int64_t)(k / 64) * p.ws_blk + (k % 64) / 32])
                          : 127u;
      }
    }
    // (first pass) the block's real slots, compacted: s_slot[0 .. nv) (PAD
    // positions dropped), read once the weight loads are on their way
    if (kc == 0 && tid < kWave) {
      const int32_t s = tid < kDecBM ? p.sorted[(int64_t)b * kDecBM + tid] : p.S;
      const bool real = tid < kDecBM && s < p.S;
      const uint64_t m = __ballot(real);
      if (real) s_slot[__popcll(m & ((1ull << tid) - 1ull))] = s;
      if (tid == 0) s_nv = __popcll(m);
    }
    // 2. stage the real slots' activations for this pass
    __syncthreads();
    nv = s_nv;
    for (int q = tid; q < nv * (kDecKC / 8); q += kThreadsDec) {
      const int j = q / (kDecKC / 8), c = q % (kDecKC / 8);
      u32x4_t v = {0, 0, 0, 0};
      if (kc + c * 8 < p.K)
        v = *reinterpret_cast<const u32x4_t*>(p.a + (int64_t)(s_slot[j] / p.a_row_div) * p.a_ld + kc + c * 8);
      *reinterpret_cast<u32x4_t*>(&xs[j][c * 8]) = v;
    }
    __syncthreads();
    // 3. dequantise and accumulate one fp32 partial per (row, slot)
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = lane + kWave * i;
      bf16x8_t wv[kDecRowsPerWave];
#pragma unroll
      for (int r = 0; r < kDecRowsPerWave; ++r) {
        if constexpr (WDT == W_BF16) {
          __builtin_memcpy(&wv[r], wraw[r][i], 16);
        } else if constexpr (WDT == W_E4M3) {
          wv[r] = dequant_e4m3x8(wraw[r][i][0], wraw[r][i][1], e8m0_as_scale(sraw[r][i]));
        } else {
          wv[r] = dequant_e2m1x8(wraw[r][i][0], e8m0_as_scale(sraw[r][i]));
        }
      }
#pragma unroll
      for (int j = 0; j < kDecBM; ++j) {
        if (j < nv) {
          const bf16x8_t xv = *reinterpret_cast<const bf16x8_t*>(&xs[j][c * 8]);
#pragma unroll
          for (int r = 0; r < kDecRowsPerWave; ++r) {
            float a = acc[r][j];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              bf16x2_t x2, w2;
              __builtin_memcpy(&x2, reinterpret_cast<const char*>(&xv) + 4 * q, 4);
              __builtin_memcpy(&w2, reinterpret_cast<const char*>(&wv[r]) + 4 * q, 4);
              a = __builtin_amdgcn_fdot2_f32_bf16(x2, w2, a, false);
            }
            acc[r][j] = a;
          }
        }
      }
    }
  }

  // reduce each partial over the wave's 64 lanes (butterfly, fixed order)
#pragma unroll
  for (int r = 0; r < kDecRowsPerWave; ++r)
#pragma unroll
    for (int j = 0; j < kDecBM; ++j) {
      if (j < nv) {
        float v = acc[r][j];
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
        acc[r][j] = v;
      }
    }

  if (lane < nv) {
    const int s = s_slot[lane];
    uint16_t* crow = p.c + (int64_t)s * p.c_ld;
    float bvals[kDecRowsPerWave];
#pragma unroll
    for (int r = 0; r < kDecRowsPerWave; ++r)
      bvals[r] = (BIAS && wrow[r] >= 0)
                     ? bf16_bits_to_f32(p.bias[(int64_t)e * p.bias_se + (int64_t)wrow[r] * p.bias_sn])
                     : 0.0f;
    // select this lane's slot column from the (uniform) partials
    float v[kDecRowsPerWave];
#pragma unroll
    for (int r = 0; r < kDecRowsPerWave; ++r) {
      v[r] = 0.0f;
#pragma unroll
      for (int j = 0; j < kDecBM; ++j) v[r] = (j == lane) ? acc[r][j] : v[r];
      v[r] += bvals[r];
    }
    if (!SWIGLU) {
#pragma unroll
      for (int r = 0; r < kDecRowsPerWave; ++r)
        if (ocol[r] >= 0) crow[ocol[r]] = (uint16_t)f32_to_bf16_bits(p.relu2 ? relu2_f32(v[r]) : v[r]);
    } else {
#pragma unroll
      for (int r = 0; r < 2; ++r)
        if (ocol[r] >= 0) crow[ocol[r]] = (uint16_t)f32_to_bf16_bits(silu_f32(v[r]) * v[r + 2]);
    }
  }
}

// ---------------------------------------------------------------------------

#define MOE_LAUNCH_DEC(WDT, SW, BI) \
  hipLaunchKernelGGL((moe_decode_kernel<WDT, SW, BI>), grid, dim3(kThreadsDec), 0, stream, p)

template <int WDT>
static void launch_decode_wdt(const GemmParams& p, bool swiglu, bool bias, dim3 grid, hipStream_t stream) {
  if (swiglu) {
    if (bias) MOE_LAUNCH_DEC(WDT, true, true);
    else MOE_LAUNCH_DEC(WDT, true, false);
  } else {
    if (bias) MOE_LAUNCH_DEC(WDT, false, true);
    else MOE_LAUNCH_DEC(WDT, false, false);
  }
}

int gemm_block_m_decode() { return kDecBM; }

hipError_t launch_gemm_decode(const GemmParams& p, int wdt, bool swiglu, bool bias, hipStream_t stream) {
  if (p.max_blocks <= 0) return hipSuccess;
  const int rows = swiglu ? kDecRows / 2 : kDecRows;
  const int out_w = swiglu ? p.N / 2 : p.N;
  const int64_t chunks = (out_w + rows - 1) / rows;
  dim3 grid((uint32_t)(chunks * p.max_blocks));
  if (wdt == W_E2M1) launch_decode_wdt<W_E2M1>(p, swiglu, bias, grid, stream);
  else if (wdt == W_E4M3) launch_decode_wdt<W_E4M3>(p, swiglu, bias, grid, stream);
  else launch_decode_wdt<W_BF16>(p, swiglu, bias, grid, stream);
  return hipGetLastError();
}

}  // namespace moe
