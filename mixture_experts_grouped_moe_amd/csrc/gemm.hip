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
//  * One workgroup of 4 waves (each 64 rows x 32*NT columns) per (routing
//    block of 64 rows, N tile); two workgroups per CU. The routing block is
//    the M tile, so no tile straddles two experts. A wave whose columns lie
//    past N, or whose 64 rows hold only padding (real rows come first in a
//    block), skips its MFMAs but still loads its share and joins every
//    barrier.
//  * Each 64-wide K step moves 8 KB of activations and the weight codes of
//    the N tile (512 rows: 16 KB of E2M1, 32 KB of E4M3; 256 rows: 32 KB of
//    bf16) straight from global memory into LDS with buffer_load ... lds (no
//    registers; rows past N, PAD rows and the K tail read as zeros through
//    the buffer bounds), three stages deep (two for E4M3), one barrier per
//    step. The E8M0 bytes of a lane's
//    weight rows arrive in registers with byte loads issued one step ahead
//    of their step's tiles, right after the compute that frees their
//    registers (issued with the tiles, last, they held up each step's wait:
//    3% on the MXFP8 workload; a variant that brought them by DMA into LDS
//    measured no faster).
//  * K order inside a step: lane half h of a wave handles K elements
//    [32h, 32h + 32) and MFMA substep ks takes [32h + 8ks, 32h + 8ks + 8).
//    Any order common to both operands gives the same dot product; this one
//    makes a lane's weight codes for the whole step one contiguous piece
//    (16 B of E2M1, 32 B of E4M3) governed by a single E8M0 scale (block
//    2*step + h), read with one or two ds_read_b128.
//  * Codes are dequantised by the waves that use them, with the gfx950 scaled
//    conversions (v_cvt_scalef32_pk_bf16_{fp4,fp8}), one MFMA pair ahead of
//    their use; the E8M0 byte rides in the exponent field of the conversion's
//    scale operand, which gives exactly 2^(b-127) including 0x00 and 0xFF.
//  * v_mfma_f32_32x32x16_bf16, fp32 accumulators, one bf16 rounding at the
//    store. Each wave: 64 rows x (32 * NT) columns. C is written in 16-byte
//    row pieces staged through LDS (store_tile_rows), or element by element
//    when C is not 16-byte aligned.
//  * LDS rows are made of 16-byte units XOR-swizzled by row so that each
//    16-lane group of a read instruction spreads over all 64 banks.
//  * Workgroup ids are remapped so each XCD walks all routing blocks of one
//    N tile in order: consecutive blocks of one expert reuse the weight tile
//    from that XCD's L2. Only the blocks in use (moe_align's padded row
//    count) are dealt out, in equal ranges per XCD.
//  * SwiGLU: a tile's weight rows are the gate rows of its h columns followed
//    by the matching up rows, arranged so that a lane holds gate and up of the
//    same output element in the same accumulator register.
#include "gemm_util.h"

namespace moe {

template <int WDT> struct WTraits;
template <> struct WTraits<W_E2M1> { static constexpr int kRowBytes = 32, kNT = 4, kStages = 3; };
template <> struct WTraits<W_E4M3> { static constexpr int kRowBytes = 64, kNT = 4, kStages = 2; };
template <> struct WTraits<W_BF16> { static constexpr int kRowBytes = 128, kNT = 2, kStages = 2; };

template <int WDT, bool SWIGLU, bool BIAS>
__global__ __launch_bounds__(kThreads, kMinBlocks) void moe_gemm_kernel(GemmParams p) {
  using Tr = WTraits<WDT>;
  constexpr int NT = Tr::kNT, RB = Tr::kRowBytes, STAGES = Tr::kStages;
  constexpr int WN = NT * 32, BN = kWavesN * WN;
  constexpr int NWAVES = kWavesM * kWavesN;
  constexpr int UW = RB / 16;                       // 16-byte units per weight row per step
  constexpr int KPU = 64 / UW;                      // K elements per weight unit
  constexpr int A_BYTES = kBM * 128;                // 8 KB
  constexpr int W_BYTES = BN * RB;                  // 16 KB (E2M1), 32 KB (E4M3, bf16)
  constexpr int A_LOADS = A_BYTES / 1024 / NWAVES;  // one 1 KB wave-wide load per instruction
  constexpr int W_LOADS = W_BYTES / 1024 / NWAVES;
  constexpr int S_LOADS = (WDT == W_BF16) ? 0 : NT;  // scale bytes per lane per step
  constexpr int SC_REGS = (WDT == W_BF16) ? 1 : NT;
  constexpr int LOADS = A_LOADS + W_LOADS;            // DMA loads per step per wave
  // Before computing a step a wave may leave in flight the DMA loads of the
  // next STAGES - 2 steps and the scale loads of the next STAGES - 1 (the
  // scale bytes of a step are loaded one step earlier than its tiles).
  constexpr int WAIT_N = LOADS * (STAGES - 2) + S_LOADS * (STAGES - 1);
  constexpr int PIECES = (WDT == W_BF16) ? 4 : (WDT == W_E4M3 ? 2 : 1);  // 16-byte code pieces per lane-row
  static_assert(A_LOADS * NWAVES * 1024 == A_BYTES && W_LOADS * NWAVES * 1024 == W_BYTES, "tile split");
  static_assert(WAIT_N < 64, "vmcnt range");

  // LDS: STAGES x [A tile | weight tile] (E4M3 and bf16: two 40 KB stages,
  // so two workgroups fill a CU's 160 KB exactly; with three stages a bf16
  // workgroup had the CU to itself and ran 19% slower. The block's slot list
  // is read from global memory until the epilogue, which keeps it in stage 0)
  constexpr int STAGE_BYTES = A_BYTES + W_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[STAGES][STAGE_BYTES];
  static_assert(kMinBlocks * STAGES * STAGE_BYTES <= 160 * 1024, "two workgroups per CU");

  // The grid covers every block moe_align could fill; the R blocks in use
  // (its padded row count / 64) times the N tiles are the real work. The
  // hardware deals workgroup ids round robin to the 8 XCDs: the real work is
  // split into 8 contiguous ranges of equal size, one per XCD, each walked in
  // order (all blocks of one N tile, then the next, so an expert's weight
  // tile is reused from the XCD's L2); the other workgroups return at once.
  // (Dealing out the whole grid instead gave the XCDs whose ranges held no
  // unused blocks up to 14% more real workgroups than the others.)
  const int R = min(p.max_blocks, max(*p.post_pad, 0) / kBM);
  const uint32_t work = (uint32_t)(gridDim.x / p.max_blocks) * (uint32_t)R;
  if (blockIdx.x / 8 >= work / 8 + (blockIdx.x % 8 < work % 8 ? 1u : 0u)) return;
  const uint32_t L = xcd_remap(blockIdx.x, work);
  const int b = L % R;
  const int tile_n = L / R;
  const int e = p.expert_ids[b];
  if (e < 0 || e >= p.E) return;  // sentinel block (or an id outside this layer's experts)

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: keeps derived addresses scalar
  const int wm = wave / kWavesN, wn = wave % kWavesN;              // this wave's rows / columns of the tile
  const int l32 = lane % 32, h = lane / 32;

  const int32_t* blk_slots = p.sorted + (int64_t)b * kBM;  // the block's slot ids

  // A wave computes nothing when its 64 rows hold only PAD positions (with
  // moe_align's routing the real rows of a block come first, so this skips
  // the padding past the last real row in 64-row steps) or when all its
  // columns lie past N; it still loads its share of the tiles and joins
  // every barrier. When its upper 32 rows are all PAD (an expert's last,
  // short block) it runs the MFMAs of the lower 32 only.
  const uint64_t live_rows = __ballot(blk_slots[wm * 64 + lane] < p.S);
  const bool rows_live = live_rows != 0;
  const bool upper_live = (live_rows >> 32) != 0;
  const bool cols_live = tile_w_row<NT, SWIGLU>(wn * WN, tile_n, p.N) >= 0;
  const bool wave_live = rows_live && cols_live;

  // ---- buffer resources (bounds give zeros for PAD rows, rows past N, K tail)
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.a, 0, (int)(uint32_t)(p.a_rows * p.a_ld * 2), 0x00020000);
  const uint8_t* w_base = p.w + (int64_t)e * p.w_stride_e;
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)w_base, 0, (int)(uint32_t)p.w_span, 0x00020000);
  __amdgpu_buffer_rsrc_t s_rsrc = w_rsrc;
  if constexpr (WDT != W_BF16)
    s_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(p.ws + (int64_t)e * p.ws_stride_e), 0,
                                               (int)(uint32_t)p.ws_span, 0x00020000);

  // ---- per-lane load descriptors: each load instruction of a wave fills one
  //      1 KB block of the stage, 16 bytes per lane in lane order
  uint32_t a_off[A_LOADS];
  int a_k[A_LOADS];  // first K element of the unit within the step (tail check)
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int q = (wave * A_LOADS + i) * 64 + lane;  // physical unit in the stage
    const int row = q / 8, pu = q % 8;
    const int u = swz<8>(row, pu);
    const int s = blk_slots[row];
    a_k[i] = u * 8;
    a_off[i] = s < p.S ? (uint32_t)((int64_t)(s / p.a_row_div) * p.a_ld * 2 + u * 16) : kOOB;
  }
  uint32_t w_off[W_LOADS];
  int w_k[W_LOADS];
#pragma unroll
  for (int i = 0; i < W_LOADS; ++i) {
    const int q = (wave * W_LOADS + i) * 64 + lane;
    const int row = q / UW, pu = q % UW;
    const int u = swz<UW>(row, pu);
    const int32_t wr = tile_w_row<NT, SWIGLU>(row, tile_n, p.N);
    w_k[i] = u * KPU;
    w_off[i] = wr >= 0 ? (uint32_t)((int64_t)wr * p.w_row + u * 16) : kOOB;
  }
  int32_t my_wrow[NT];
  uint32_t s_off[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    my_wrow[nt] = tile_w_row<NT, SWIGLU>(wn * WN + nt * 32 + l32, tile_n, p.N);
    s_off[nt] = my_wrow[nt] >= 0 ? (uint32_t)((int64_t)my_wrow[nt] * p.ws_row + h) : kOOB;
  }
  const uint32_t w_blk = (uint32_t)p.w_blk, ws_blk = (uint32_t)p.ws_blk;

  const int nsteps = (p.K + kBK - 1) / kBK;
  const int nsteps_pad = ((nsteps + STAGES - 1) / STAGES) * STAGES;

  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_u8_t*)&lds[0][0];
  // scale bytes of this lane's weight rows (one per N sub-tile), per stage
  uint32_t sc[STAGES][SC_REGS];

  // Issue the DMA loads of K step `step` into stage ST. A step wholly inside
  // K uses the per-lane offsets as they are, advanced by a scalar offset; the
  // K tail and the look-ahead steps past the last one (every step issues the
  // same number of loads) take the checked path, whose lanes past K read
  // zeros.
  auto issue = [&](int step, auto stage_tag) {
    constexpr int ST = decltype(stage_tag)::value;
    const int k0 = step * kBK;
    const uint32_t base = lds_base + ST * STAGE_BYTES;
    if (k0 + kBK <= p.K) {
      const uint32_t sa = (uint32_t)k0 * 2, sw = (uint32_t)step * w_blk;
#pragma unroll
      for (int i = 0; i < A_LOADS; ++i) dma16(a_rsrc, a_off[i], sa, base + (wave * A_LOADS + i) * 1024);
#pragma unroll
      for (int i = 0; i < W_LOADS; ++i) dma16(w_rsrc, w_off[i], sw, base + A_BYTES + (wave * W_LOADS + i) * 1024);
    } else {
      const bool live = k0 < p.K;
      const uint32_t sa = live ? (uint32_t)k0 * 2 : 0u, sw = live ? (uint32_t)step * w_blk : 0u;
#pragma unroll
      for (int i = 0; i < A_LOADS; ++i)
        dma16(a_rsrc, (live && k0 + a_k[i] < p.K) ? a_off[i] : kOOB, sa, base + (wave * A_LOADS + i) * 1024);
#pragma unroll
      for (int i = 0; i < W_LOADS; ++i)
        dma16(w_rsrc, (live && k0 + w_k[i] < p.K) ? w_off[i] : kOOB, sw,
              base + A_BYTES + (wave * W_LOADS + i) * 1024);
    }
  };
  // The scale bytes of K step `step` into register set ST (the set of the
  // step just computed, step - STAGES); a block past K reads 0.
  auto issue_scales = [&](int step, auto stage_tag) {
    constexpr int ST = decltype(stage_tag)::value;
    if constexpr (WDT != W_BF16) {
      const int k0 = step * kBK;
      const bool hl = k0 + 32 * h < p.K;
      const uint32_t ss = k0 < p.K ? (uint32_t)step * ws_blk : 0u;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sc[ST][nt] = load_byte(s_rsrc, hl ? s_off[nt] : kOOB, ss);
    }
  };

  f32x16_t acc[2][NT];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.0f;

  // Compute one K step from stage ST for the first NMT 32-row quarters of
  // this wave's rows (all of them: NMT = 2).
  auto compute = [&](auto stage_tag, auto nmt_tag) {
    constexpr int ST = decltype(stage_tag)::value;
    constexpr int NMT = decltype(nmt_tag)::value;
    const lds_u8_t* As = (const lds_u8_t*)&lds[ST][0];
    const lds_u8_t* Ws = As + A_BYTES;
    // this lane's weight codes for the whole step, one piece per N sub-tile
    u32x4_t wcode[NT][PIECES];
    float scl[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int row = wn * WN + nt * 32 + l32;
#pragma unroll
      for (int j = 0; j < PIECES; ++j)
        wcode[nt][j] = lds_read<u32x4_t>(Ws + row * RB + swz<UW>(row, PIECES * h + j) * 16);
      if constexpr (WDT != W_BF16) scl[nt] = e8m0_as_scale(sc[ST][nt]);
    }
    // activation fragments of substep ks (one per live 32-row quarter), read
    // one substep ahead of their use
    bf16x8_t af[2][NMT];
    auto read_a = [&](int ks, bf16x8_t(&dst)[NMT]) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const int row = wm * 64 + mt * 32 + l32;
        dst[mt] = lds_read<bf16x8_t>(As + row * 128 + swz<8>(row, 4 * h + ks) * 16);
      }
    };
    // weight operand of pair j = (substep j / NT, N sub-tile j % NT), in bf16
    auto operand = [&](int j) -> bf16x8_t {
      const int ks = j / NT, nt = j % NT;
      bf16x8_t bfr;
      if constexpr (WDT == W_E2M1) {
        bfr = dequant_e2m1x8(wcode[nt][0][ks], scl[nt]);
      } else if constexpr (WDT == W_E4M3) {
        const u32x4_t& v = wcode[nt][ks / 2];
        bfr = dequant_e4m3x8(v[2 * (ks % 2)], v[2 * (ks % 2) + 1], scl[nt]);
      } else {
        __builtin_memcpy(&bfr, &wcode[nt][ks], 16);
      }
      return bfr;
    };
    // Pairs j = 0 .. 4*NT-1, NMT MFMAs each. The weight operand of pair j+1
    // is dequantised while pair j's MFMAs run: a conversion feeding the very
    // next MFMA stalls it, one pair ahead it overlaps (measured on gfx950).
    read_a(0, af[0]);
    bf16x8_t bq[2];
    bq[0] = operand(0);
#pragma unroll
    for (int j = 0; j < 4 * NT; ++j) {
      const int ks = j / NT, nt = j % NT;
      if (nt == 0 && ks < 3) read_a(ks + 1, af[(ks + 1) % 2]);
      if (j + 1 < 4 * NT) bq[(j + 1) % 2] = operand(j + 1);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks % 2][mt], bq[j % 2], acc[mt][nt], 0, 0, 0);
    }
    if constexpr (WDT != W_BF16) {
      // the schedule above, pinned: the step's LDS reads for the weight codes
      // and the first activation fragments, the scale and first-operand VALU
      // work, then per pair: (the next substep's activation reads,) the next
      // operand's four conversions, the pair's MFMAs
      constexpr int kDsRead = 0x100, kValu = 0x002, kMfma = 0x008;
      __builtin_amdgcn_sched_group_barrier(kDsRead, NT * PIECES + NMT, 0);
      __builtin_amdgcn_sched_group_barrier(kValu, 2 * NT + 4, 0);
#pragma unroll
      for (int j = 0; j < 4 * NT; ++j) {
        if (j % NT == 0 && j / NT < 3) __builtin_amdgcn_sched_group_barrier(kDsRead, NMT, 0);
        if (j + 1 < 4 * NT) __builtin_amdgcn_sched_group_barrier(kValu, 4, 0);
        __builtin_amdgcn_sched_group_barrier(kMfma, NMT, 0);
      }
    }
  };

  using One = std::integral_constant<int, 1>;
  using Two = std::integral_constant<int, 2>;

  // Stage s holds steps s, s + STAGES, ... Before computing a step, the wave
  // waits until only the loads issued after this step's tiles are
  // outstanding (WAIT_N), so this step's tiles and scale bytes are done; the
  // barrier then makes every wave's loads visible and guarantees all waves
  // finished the previous step, whose stage the loads issued next overwrite.
  // Issue order: scales(0), then per step t < STAGES - 1 tiles(t) and
  // scales(t + 1); in the loop, tiles(step + STAGES - 1) before the compute
  // and scales(step + STAGES) after it, into the register set just read.
  // (the loop, with its first loads, is instantiated once per row count and
  // chosen before any load is issued: the scale bytes arrive by loads the
  // compiler does not track, so no register they write may be live across
  // the choice, where the compiler could copy it before the data lands)
  auto k_loop = [&](auto nmt_tag) {
    issue_scales(0, std::integral_constant<int, 0>{});
    static_for<0, STAGES - 1>([&](auto st) {
      constexpr int ST = decltype(st)::value;
      issue(ST, st);
      issue_scales(ST + 1, std::integral_constant<int, ST + 1>{});
    });
    for (int step = 0; step < nsteps_pad; step += STAGES) {
      static_for<0, STAGES>([&](auto st) {
        constexpr int ST = decltype(st)::value;
        wait_loads_barrier<WAIT_N>(sc[ST]);
        issue(step + ST + STAGES - 1, std::integral_constant<int, (ST + STAGES - 1) % STAGES>{});
        if (wave_live) compute(st, nmt_tag);
        issue_scales(step + ST + STAGES, st);
      });
    }
  };
  if (upper_live) k_loop(Two{});
  else k_loop(One{});
  // drain the look-ahead loads (all of them read as zeros past the last step),
  // then keep the slot list in stage 0 once every wave is done with it
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int32_t* s_slot = reinterpret_cast<int32_t*>(&lds[0][0]);
  if (tid < kBM) s_slot[tid] = blk_slots[tid];
  __syncthreads();

  // ---- epilogue: bias, SwiGLU, one bf16 rounding, store real rows only
  float bv[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    bv[nt] = 0.0f;
    if (BIAS && my_wrow[nt] >= 0)
      bv[nt] = bf16_bits_to_f32(p.bias[(int64_t)e * p.bias_se + (int64_t)my_wrow[nt] * p.bias_sn]);
  }
  // Aligned C (the usual case): whole 16-byte row pieces staged through LDS
  // (after the slot list); a workgroup's stores took a fifth of its time when
  // each lane wrote its 2-byte values itself.
  if (p.c_ld % 8 == 0 && ((uintptr_t)p.c & 15) == 0) {
    constexpr int OC = SWIGLU ? WN / 2 : WN;  // output columns of this wave
    static_assert(kBM * 4 + NWAVES * stage_rows_bytes<OC>() <= STAGES * STAGE_BYTES, "staging fits");
    lds_u8_t* const lds0 = (lds_u8_t*)&lds[0][0];
    const int col0 = SWIGLU ? tile_n * (BN / 2) + wn * (WN / 2) : tile_n * BN + wn * WN;
    const int out_w = SWIGLU ? p.N / 2 : p.N;
    store_tile_rows<OC>(
        [&](int mt, int j, int i) {
          if constexpr (!SWIGLU) {
            const float v = acc[mt][j][i] + bv[j];
            return p.relu2 ? relu2_f32(v) : v;
          } else {
            const float g = acc[mt][j][i] + bv[j];
            const float up = acc[mt][j + NT / 2][i] + bv[j + NT / 2];
            return silu_f32(g) * up;
          }
        },
        lds0 + kBM * 4 + wave * stage_rows_bytes<OC>(), lds0, wm * 64, p.c, p.c_ld, p.S, col0, out_w, lane);
    return;
  }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = wm * 64 + mt * 32 + (i / 4) * 8 + h * 4 + (i % 4);
      const int s = s_slot[row];
      if (s >= p.S) continue;
      uint16_t* crow = p.c + (int64_t)s * p.c_ld;
      if constexpr (!SWIGLU) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if (my_wrow[nt] >= 0) {
            const float v = acc[mt][nt][i] + bv[nt];
            crow[my_wrow[nt]] = (uint16_t)f32_to_bf16_bits(p.relu2 ? relu2_f32(v) : v);
          }
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
#define MOE_LAUNCH(WDT, SW, BI) \
  hipLaunchKernelGGL((moe_gemm_kernel<WDT, SW, BI>), grid, dim3(kThreads), 0, stream, p)

template <int WDT>
static void launch_gemm_wdt(const GemmParams& p, bool swiglu, bool bias, dim3 grid, hipStream_t stream) {
  if (swiglu) {
    if (bias) MOE_LAUNCH(WDT, true, true);
    else MOE_LAUNCH(WDT, true, false);
  } else {
    if (bias) MOE_LAUNCH(WDT, false, true);
    else MOE_LAUNCH(WDT, false, false);
  }
}

int gemm_block_m_large() { return kBM; }

// Number of N tiles of the large-M kernel for this weight type.
static int gemm_tiles_n(int wdt, int N, bool swiglu) {
  const int nt = wdt == W_E2M1 ? WTraits<W_E2M1>::kNT : (wdt == W_E4M3 ? WTraits<W_E4M3>::kNT : WTraits<W_BF16>::kNT);
  const int bn = kWavesN * 32 * nt;
  return swiglu ? (N / 2 + bn / 2 - 1) / (bn / 2) : (N + bn - 1) / bn;
}

hipError_t launch_gemm_large(const GemmParams& p, int wdt, bool swiglu, bool bias, hipStream_t stream) {
  if (p.max_blocks <= 0) return hipSuccess;
  const int64_t tiles = gemm_tiles_n(wdt, p.N, swiglu);
  dim3 grid((uint32_t)(tiles * p.max_blocks));
  if (wdt == W_E2M1) launch_gemm_wdt<W_E2M1>(p, swiglu, bias, grid, stream);
  else if (wdt == W_E4M3) launch_gemm_wdt<W_E4M3>(p, swiglu, bias, grid, stream);
  else launch_gemm_wdt<W_BF16>(p, swiglu, bias, grid, stream);
  return hipGetLastError();
}

}  // namespace moe
