// Routed grouped GEMM over block-scaled expert weights (large M), on MFMA.
//
// Follows ROCm/aiter PR #5310 "Add MoE GEMM variants and weight-gradient
// kernel": Summary (moe_gemm_mxfp8: all experts in one launch; an E8M0 byte per
// 32 K-elements turned into a power of two and applied per K-step; optional
// per-expert bias), Notes (K-steps aligned to the 32-element scale blocks;
// int64 expert offsets) and the second review (sentinel blocks return at once;
// E8M0 0x00 is 2^-127 and 0xFF is NaN; bias read through explicit strides).
// The W4A16 form (bf16 activations x MXFP4 weights) is the one of
// TensorRT-LLM PR #15311 "Bound Triton MoE JIT specializations via token-dim
// bucketing and warmup", Description.
//
// Design for gfx950:
//  * One workgroup (4 waves) per (routing block of 64 rows, N tile). The
//    routing block is the M tile, so padding waste is at most 63 rows per
//    expert and tiles never straddle two experts.
//  * The N tile holds 16 KB of weight codes per 64-wide K-step whatever the
//    element type (512 rows of E2M1, 256 of E4M3 or bf16 at 32 KB), staged in
//    LDS as raw codes. Each wave owns N/4 of the tile and dequantises only its
//    own fragments, once, with the gfx950 scaled conversions
//    (v_cvt_scalef32_pk_bf16_{fp4,fp8}); the E8M0 byte rides in the exponent
//    field of the conversion's scale operand, which gives exactly 2^(b-127)
//    including the 0x00 and 0xFF codes.
//  * v_mfma_f32_32x32x16_bf16, fp32 accumulators, one bf16 rounding at the
//    store. Each wave: 64 rows x (32 * NT) columns.
//  * LDS rows are split in 8 units (one 8-element fragment piece each) whose
//    position is XOR-swizzled by row so that the 32 lanes reading one unit of
//    32 different rows hit distinct banks.
//  * Double-buffered LDS, global loads for step k+1 issued before step k's
//    MFMAs, one barrier per K-step.
//  * Workgroup ids are remapped so each XCD walks all routing blocks of one
//    N tile in order: consecutive blocks of one expert reuse the weight tile
//    from that XCD's L2.
//  * SwiGLU: a tile's weight rows are the gate rows of its h columns followed
//    by the matching up rows, arranged so that a lane holds gate and up of the
//    same output element in the same accumulator register.
#include "common.h"
#include "params.h"

namespace moe {

template <int WDT> struct WTraits;
template <> struct WTraits<W_E2M1> { static constexpr int kRowBytes = 32, kUnit = 4, kNT = 4; };
template <> struct WTraits<W_E4M3> { static constexpr int kRowBytes = 64, kUnit = 8, kNT = 2; };
template <> struct WTraits<W_BF16> { static constexpr int kRowBytes = 128, kUnit = 16, kNT = 2; };


constexpr int kBM = 64;
constexpr int kBK = 64;
constexpr int kThreads = 256;

// Row swizzle of the 8 units of an LDS row of `unit` bytes: the rows that
// share a 128-byte bank window get different XOR keys.
template <int U>
__device__ __forceinline__ int unit_swz(int row) {
  constexpr int rows_per_window = 16 / U;  // 128 B / (8 units * U)
  return (row / rows_per_window) & 7;
}

// Global weight row of local tile row r, or -1 beyond N.
template <int NT, bool SWIGLU>
__device__ __forceinline__ int32_t tile_w_row(int r, int tile_n, int N) {
  constexpr int WN = NT * 32;
  constexpr int BN = 4 * WN;
  if (!SWIGLU) {
    int n = tile_n * BN + r;
    return n < N ? n : -1;
  } else {
    const int half = N / 2;
    const int w = r / WN, q = r % WN;
    const bool up = q >= WN / 2;
    const int hcol = tile_n * (BN / 2) + w * (WN / 2) + (up ? q - WN / 2 : q);
    if (hcol >= half) return -1;
    return up ? half + hcol : hcol;
  }
}

template <int WDT, bool SWIGLU, bool BIAS>
__global__ __launch_bounds__(kThreads) void moe_gemm_kernel(GemmParams p) {
  using Tr = WTraits<WDT>;
  constexpr int NT = Tr::kNT, U = Tr::kUnit, RB = Tr::kRowBytes;
  constexpr int WN = NT * 32, BN = 4 * WN;
  constexpr int A_STAGE = kBM * 128;
  constexpr int W_STAGE = BN * RB;
  constexpr int STAGE = A_STAGE + W_STAGE;
  constexpr int W_CHUNKS = W_STAGE / 16 / kThreads;
  constexpr int CHUNKS_PER_ROW = RB / 16;
  constexpr int UNITS_PER_CHUNK = 16 / U;

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  __shared__ int32_t s_slot[kBM];

  const uint32_t L = xcd_remap(blockIdx.x, gridDim.x);
  const int b = L % p.max_blocks;
  const int tile_n = L / p.max_blocks;
  const int e = p.expert_ids[b];
  if (e < 0) return;  // sentinel block

  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int l32 = lane % 32, h = lane / 32;

  if (tid < kBM) s_slot[tid] = p.sorted[(int64_t)b * kBM + tid];
  __syncthreads();

  // ---- per-thread load descriptors
  const uint16_t* a_src[2];
  int a_dst[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int id = tid + kThreads * i;
    const int row = id >> 3, c = id & 7;
    const int s = s_slot[row];
    a_src[i] = s < p.S ? p.a + (int64_t)(s / p.a_row_div) * p.a_ld + c * 8 : nullptr;
    a_dst[i] = row * 128 + ((c ^ (row & 7)) * 16);
  }
  const uint8_t* w_base = p.w + (int64_t)e * p.w_stride_e;
  const uint8_t* w_src[W_CHUNKS];
  int w_dst_row[W_CHUNKS], w_chunk[W_CHUNKS];
#pragma unroll
  for (int j = 0; j < W_CHUNKS; ++j) {
    const int id = tid + kThreads * j;
    const int row = id / CHUNKS_PER_ROW, c = id % CHUNKS_PER_ROW;
    const int32_t wr = tile_w_row<NT, SWIGLU>(row, tile_n, p.N);
    w_src[j] = wr >= 0 ? w_base + (int64_t)wr * p.w_ld + c * 16 : nullptr;
    w_dst_row[j] = row;
    w_chunk[j] = c;
  }
  // scale bytes and bias for this lane's weight rows (one per N sub-tile)
  const uint8_t* sc_src[NT];
  int32_t my_wrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = wave * WN + nt * 32 + l32;
    my_wrow[nt] = tile_w_row<NT, SWIGLU>(r, tile_n, p.N);
    sc_src[nt] = (WDT != W_BF16 && my_wrow[nt] >= 0)
                     ? p.ws + (int64_t)e * p.ws_stride_e + (int64_t)my_wrow[nt] * p.ws_ld
                     : nullptr;
  }

  const int nsteps = (p.K + kBK - 1) / kBK;
  u32x4_t ra[2];
  u32x4_t rw[W_CHUNKS];
  uint32_t rs[NT];  // two scale bytes (blocks 2*step, 2*step+1), packed

  auto load_global = [&](int step) {
    const int k0 = step * kBK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = (tid + kThreads * i) & 7;
      const bool ok = a_src[i] != nullptr && (k0 + c * 8) < p.K;
      ra[i] = ok ? *reinterpret_cast<const u32x4_t*>(a_src[i] + k0) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < W_CHUNKS; ++j) {
      constexpr int elems_per_chunk = (WDT == W_E2M1) ? 32 : (WDT == W_E4M3 ? 16 : 8);
      const bool ok = w_src[j] != nullptr && (k0 + w_chunk[j] * elems_per_chunk) < p.K;
      rw[j] = ok ? *reinterpret_cast<const u32x4_t*>(w_src[j] + (int64_t)step * RB)
                 : u32x4_t{0, 0, 0, 0};
    }
    if (WDT != W_BF16) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        uint32_t s0 = 127, s1 = 127;
        if (sc_src[nt] != nullptr) {
          const int blk = 2 * step;
          if (blk * 32 < p.K) s0 = sc_src[nt][blk];
          if ((blk + 1) * 32 < p.K) s1 = sc_src[nt][blk + 1];
        }
        rs[nt] = s0 | (s1 << 8);
      }
    }
  };

  auto store_lds = [&](int buf) {
    uint8_t* As = smem + buf * STAGE;
    uint8_t* Ws = As + A_STAGE;
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4_t*>(As + a_dst[i]) = ra[i];
#pragma unroll
    for (int j = 0; j < W_CHUNKS; ++j) {
      const int row = w_dst_row[j];
      const int sw = unit_swz<U>(row);
      uint8_t* dst = Ws + row * RB;
      if constexpr (U == 16) {
        *reinterpret_cast<u32x4_t*>(dst + ((w_chunk[j] ^ sw) * 16)) = rw[j];
      } else if constexpr (U == 8) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int u = w_chunk[j] * UNITS_PER_CHUNK + q;
          *reinterpret_cast<u32x2_t*>(dst + ((u ^ sw) * 8)) = u32x2_t{rw[j][2 * q], rw[j][2 * q + 1]};
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int u = w_chunk[j] * UNITS_PER_CHUNK + q;
          *reinterpret_cast<uint32_t*>(dst + ((u ^ sw) * 4)) = rw[j][q];
        }
      }
    }
  };

  f32x16_t acc[2][NT];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.0f;

  load_global(0);
  store_lds(0);
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const int cur = step & 1;
    float scale[NT][2];
    if (WDT != W_BF16) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        scale[nt][0] = e8m0_as_scale(rs[nt] & 0xff);
        scale[nt][1] = e8m0_as_scale(rs[nt] >> 8);
      }
    }
    if (step + 1 < nsteps) load_global(step + 1);

    const uint8_t* As = smem + cur * STAGE;
    const uint8_t* Ws = As + A_STAGE;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int u = 2 * ks + h;
      bf16x8_t af[2], bfr[NT];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int row = mt * 32 + l32;
        af[mt] = *reinterpret_cast<const bf16x8_t*>(As + row * 128 + ((u ^ (row & 7)) * 16));
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int row = wave * WN + nt * 32 + l32;
        const uint8_t* src = Ws + row * RB + ((u ^ unit_swz<U>(row)) * U);
        if constexpr (WDT == W_E2M1) {
          bfr[nt] = dequant_e2m1x8(*reinterpret_cast<const uint32_t*>(src), scale[nt][ks >> 1]);
        } else if constexpr (WDT == W_E4M3) {
          const u32x2_t v = *reinterpret_cast<const u32x2_t*>(src);
          bfr[nt] = dequant_e4m3x8(v[0], v[1], scale[nt][ks >> 1]);
        } else {
          bfr[nt] = *reinterpret_cast<const bf16x8_t*>(src);
        }
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mt], bfr[nt], acc[mt][nt], 0, 0, 0);
    }
    if (step + 1 < nsteps) store_lds(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: bias, SwiGLU, one bf16 rounding, store real rows only
  float bv[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    bv[nt] = 0.0f;
    if (BIAS && my_wrow[nt] >= 0)
      bv[nt] = bf16_bits_to_f32(p.bias[(int64_t)e * p.bias_se + (int64_t)my_wrow[nt] * p.bias_sn]);
  }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = mt * 32 + (i / 4) * 8 + h * 4 + (i % 4);
      const int s = s_slot[row];
      if (s >= p.S) continue;
      uint16_t* crow = p.c + (int64_t)s * p.c_ld;
      if constexpr (!SWIGLU) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if (my_wrow[nt] >= 0) crow[my_wrow[nt]] = (uint16_t)f32_to_bf16_bits(acc[mt][nt][i] + bv[nt]);
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < NT / 2; ++nt) {
          if (my_wrow[nt] >= 0) {
            const float g = acc[mt][nt][i] + bv[nt];
            const float up = acc[mt][nt + NT / 2][i] + bv[nt + NT / 2];
            crow[my_wrow[nt]] = (uint16_t)f32_to_bf16_bits(silu_f32(g) * up);
          }
        }
      }
    }
  }
}

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

template <int WDT, bool SWIGLU, bool BIAS>
__global__ __launch_bounds__(kThreads) void moe_decode_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[kDecBM][kDecKC];
  __shared__ int32_t s_slot[kDecBM];

  const int b = blockIdx.x % p.max_blocks;
  const int chunk = blockIdx.x / p.max_blocks;
  const int e = p.expert_ids[b];
  if (e < 0) return;  // sentinel block

  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  if (tid < kDecBM) s_slot[tid] = p.sorted[(int64_t)b * kDecBM + tid];
  __syncthreads();
  // which of the block's positions hold a real slot (PAD marks the rest)
  uint32_t vmask = 0;
#pragma unroll
  for (int j = 0; j < kDecBM; ++j) vmask |= (s_slot[j] < p.S ? 1u : 0u) << j;

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

  constexpr int kPer = kDecKC / 8 / kWave;  // 8-element pieces per lane per pass
  for (int kc = 0; kc < p.K; kc += kDecKC) {
    __syncthreads();
    // stage the real slots' activations: kDecBM rows x kDecKC (zeros for PAD)
    for (int q = tid; q < kDecBM * (kDecKC / 8); q += kThreads) {
      const int j = q / (kDecKC / 8), c = q % (kDecKC / 8);
      u32x4_t v = {0, 0, 0, 0};
      if (((vmask >> j) & 1u) && kc + c * 8 < p.K)
        v = *reinterpret_cast<const u32x4_t*>(p.a + (int64_t)(s_slot[j] / p.a_row_div) * p.a_ld + kc + c * 8);
      *reinterpret_cast<u32x4_t*>(&xs[j][c * 8]) = v;
    }
    __syncthreads();

    // weight pieces: [row][i] holds elements kc + 8 * (lane + 64 i) .. +8
    bf16x8_t wv[kDecRowsPerWave][kPer];
#pragma unroll
    for (int r = 0; r < kDecRowsPerWave; ++r) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int k = kc + 8 * (lane + kWave * i);
        const bool ok = wrow[r] >= 0 && k < p.K;
        const uint8_t* rowp = w_base + (int64_t)(ok ? wrow[r] : 0) * p.w_ld;
        if constexpr (WDT == W_BF16) {
          u32x4_t v = ok ? *reinterpret_cast<const u32x4_t*>(rowp + (int64_t)k * 2) : u32x4_t{0, 0, 0, 0};
          __builtin_memcpy(&wv[r][i], &v, 16);
        } else {
          const uint8_t sb = ok ? ws_base[(int64_t)wrow[r] * p.ws_ld + k / 32] : 127;
          const float sc = e8m0_as_scale(sb);
          if constexpr (WDT == W_E4M3) {
            u32x2_t v = ok ? *reinterpret_cast<const u32x2_t*>(rowp + k) : u32x2_t{0, 0};
            wv[r][i] = dequant_e4m3x8(v[0], v[1], sc);
          } else {
            uint32_t v = ok ? *reinterpret_cast<const uint32_t*>(rowp + k / 2) : 0u;
            wv[r][i] = dequant_e2m1x8(v, sc);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = lane + kWave * i;
#pragma unroll
      for (int j = 0; j < kDecBM; ++j) {
        if ((vmask >> j) & 1u) {
          const bf16x8_t xv = *reinterpret_cast<const bf16x8_t*>(&xs[j][c * 8]);
#pragma unroll
          for (int r = 0; r < kDecRowsPerWave; ++r) {
            float a = acc[r][j];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              bf16x2_t x2, w2;
              __builtin_memcpy(&x2, reinterpret_cast<const char*>(&xv) + 4 * q, 4);
              __builtin_memcpy(&w2, reinterpret_cast<const char*>(&wv[r][i]) + 4 * q, 4);
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
      if ((vmask >> j) & 1u) {
        float v = acc[r][j];
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
        acc[r][j] = v;
      }
    }

  if (lane < kDecBM && ((vmask >> lane) & 1u)) {
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
        if (ocol[r] >= 0) crow[ocol[r]] = (uint16_t)f32_to_bf16_bits(v[r]);
    } else {
#pragma unroll
      for (int r = 0; r < 2; ++r)
        if (ocol[r] >= 0) crow[ocol[r]] = (uint16_t)f32_to_bf16_bits(silu_f32(v[r]) * v[r + 2]);
    }
  }
}

// ---------------------------------------------------------------------------
#define MOE_LAUNCH(KERNEL, WDT, SW, BI) \
  hipLaunchKernelGGL((KERNEL<WDT, SW, BI>), grid, dim3(kThreads), 0, stream, p)

template <int WDT>
static void launch_gemm_wdt(const GemmParams& p, bool swiglu, bool bias, dim3 grid, hipStream_t stream) {
  if (swiglu) {
    if (bias) MOE_LAUNCH(moe_gemm_kernel, WDT, true, true);
    else MOE_LAUNCH(moe_gemm_kernel, WDT, true, false);
  } else {
    if (bias) MOE_LAUNCH(moe_gemm_kernel, WDT, false, true);
    else MOE_LAUNCH(moe_gemm_kernel, WDT, false, false);
  }
}

template <int WDT>
static void launch_decode_wdt(const GemmParams& p, bool swiglu, bool bias, dim3 grid, hipStream_t stream) {
  if (swiglu) {
    if (bias) MOE_LAUNCH(moe_decode_kernel, WDT, true, true);
    else MOE_LAUNCH(moe_decode_kernel, WDT, true, false);
  } else {
    if (bias) MOE_LAUNCH(moe_decode_kernel, WDT, false, true);
    else MOE_LAUNCH(moe_decode_kernel, WDT, false, false);
  }
}

int gemm_block_m_large() { return kBM; }
int gemm_block_m_decode() { return kDecBM; }

// Number of N tiles of the large-M kernel for this weight type.
static int gemm_tiles_n(int wdt, int N, bool swiglu) {
  const int nt = wdt == W_E2M1 ? WTraits<W_E2M1>::kNT : (wdt == W_E4M3 ? WTraits<W_E4M3>::kNT : WTraits<W_BF16>::kNT);
  const int bn = 4 * 32 * nt;
  return swiglu ? (N / 2 + bn / 2 - 1) / (bn / 2) : (N + bn - 1) / bn;
}

hipError_t launch_grouped_gemm(const GemmParams& p, int wdt, bool swiglu, bool bias, bool decode,
                               hipStream_t stream) {
  if (p.max_blocks <= 0) return hipSuccess;
  if (decode) {
    const int rows = swiglu ? kDecRows / 2 : kDecRows;
    const int out_w = swiglu ? p.N / 2 : p.N;
    const int64_t chunks = (out_w + rows - 1) / rows;
    dim3 grid((uint32_t)(chunks * p.max_blocks));
    if (wdt == W_E2M1) launch_decode_wdt<W_E2M1>(p, swiglu, bias, grid, stream);
    else if (wdt == W_E4M3) launch_decode_wdt<W_E4M3>(p, swiglu, bias, grid, stream);
    else launch_decode_wdt<W_BF16>(p, swiglu, bias, grid, stream);
  } else {
    const int64_t tiles = gemm_tiles_n(wdt, p.N, swiglu);
    dim3 grid((uint32_t)(tiles * p.max_blocks));
    if (wdt == W_E2M1) launch_gemm_wdt<W_E2M1>(p, swiglu, bias, grid, stream);
    else if (wdt == W_E4M3) launch_gemm_wdt<W_E4M3>(p, swiglu, bias, grid, stream);
    else launch_gemm_wdt<W_BF16>(p, swiglu, bias, grid, stream);
  }
  return hipGetLastError();
}

}  // namespace moe
