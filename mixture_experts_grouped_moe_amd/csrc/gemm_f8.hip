// Routed grouped GEMM with MXFP8 activations and MXFP8 (E4M3) weights: both
// operands E4M3 codes with one E8M0 scale per 32 K-elements, the form of
// moe_gemm_mxfp8 in ROCm/aiter PR #5310 "Add MoE GEMM variants and
// weight-gradient kernel" (Summary: all experts in one launch, microscales
// applied per K step, optional per-expert bias; second review: the kernel
// decodes an a_scale and a b_scale byte per K block, sentinel blocks return at
// once, E8M0 0x00 is 2^-127 and 0xFF NaN, bias through explicit strides).
//
// Design for gfx950 (the routing and load pipeline of the bf16 large-M kernel
// in gemm.hip, on a taller tile):
//  * One workgroup of 8 waves (2 along M x 4 along N, each 64 rows x 128
//    columns) per (routing block of 128 rows, N tile of 512 weight rows); one
//    workgroup per CU. The kernel is bound by the bytes moved from L2 into
//    LDS: a 128-row block reads each weight tile once for twice the rows of a
//    64-row block, which took the MXFP8 workload from 2.24 to 2.05 ms.
//  * Each 64-wide K step moves 8 KB of activation codes and 32 KB of weight
//    codes straight into LDS with buffer_load ... lds, three stages deep (two
//    steps in flight), and the step's E8M0 bytes by byte (or 2-byte) DMA
//    into a ring of scale sets in LDS, one step ahead of the tiles; with
//    packed weights one wave fetches the N tile's weight scale bytes of a
//    step in a single 16-byte-per-lane DMA (1 KB).
//  * The contraction is v_mfma_scale_f32_32x32x64_f8f6f4: one instruction
//    per 32 x 32 output tile and K step, with the E8M0 bytes fed to it as they
//    are (no dequantisation). Its operand layout (measured on gfx950): lane l
//    holds row (or column) l % 32; bytes 0-15 are K elements 16h .. 16h+15
//    and bytes 16-31 are 32 + 16h .. 32 + 16h + 15 (h = l / 32), and the
//    scale operand of lane l is that of K block h: its 32 elements are bytes
//    0-15 of both lane halves (h = 0) or bytes 16-31 (h = 1). So a lane reads
//    16-byte units h and 2 + h of its row's 64-byte step piece.
//  * fp32 accumulators, bias and SwiGLU in the epilogue, one bf16 rounding;
//    C is written in 16-byte row pieces staged through LDS (store_tile_rows),
//    or element by element when C is not 16-byte aligned.
//
// The same kernel in per-token mode is moe_gemm_per_token of that PR
// (Summary: E4M3 operands with one fp32 scale per activation row and one per
// expert, both applied after the fp8 dot product; a group_sizes interface):
// the routing block is a run of consecutive rows of one expert taken from the
// block mapping (block_expert_ids / block_token_offsets / block_token_ends of
// the second review), the MFMA's scale bytes are the constant 127 (2^0), no
// scale bytes are loaded, and the epilogue multiplies the fp32 accumulator by
// a_scale[row] * w_scale[e] before the bias.
#include "gemm_util.h"

namespace moe {

constexpr int kF8NT = 4;                        // 32-column MFMA tiles per wave
constexpr int kF8WavesM = 2;                    // waves along M (64 rows each)
constexpr int kF8Stages = 3;
constexpr int kF8RowBytes = 64;                 // one row's codes per K step
constexpr int kF8BM = 64 * kF8WavesM;           // the routing block
constexpr int kF8Threads = kWave * kF8WavesM * kWavesN;
constexpr int kF8MinBlocks = kF8WavesM == 1 ? 2 : 1;  // workgroups per CU

typedef int f8_v8i __attribute__((ext_vector_type(8)));

// Two bytes per lane from buffer `rsrc` at `voff` + `soff` into LDS, written
// zero-extended as the dword at `lds_base` + 4 * lane (the byte at `voff` in
// bits 0-7); a lane whose `voff` is kOOB writes 0. `voff` + `soff` is even.
__device__ __forceinline__ void dma_ushort(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_ushort %0, %2, %3 offen lds"
               :: "v"(voff), "s"(__builtin_amdgcn_readfirstlane(lds_base)), "s"(rsrc),
                  "s"(__builtin_amdgcn_readfirstlane(soff)) : "m0");
}

constexpr int kE8M0One = 127;                   // E8M0 code of 2^0

// How the weight scale bytes of a step reach LDS (WSM):
//  kWsByte  one byte per lane, 32 rows per DMA, every wave;
//  kWsPair  a row's two bytes of a step adjacent and 2-byte aligned (even
//           scale strides): one 2-byte DMA per lane, 64 rows per DMA, every
//           wave;
//  kWsPiece the K-block layout with 16-byte aligned strides: the tile's 512
//           rows' byte pairs of a step are 64 aligned 16-byte pieces of 8
//           consecutive rows each (a SwiGLU tile's gate and up runs are 64
//           rows long and start at multiples of 8 when N/2 is), so one wave
//           fetches them all with a single 16-byte DMA. The activation
//           scale DMAs are then issued once per 32-row group too, by waves
//           0 .. 3, where the other modes have two waves load each group.
// The load path pays per DMA instruction more than per byte, so fewer
// scale DMAs leave more of it to the tiles.
constexpr int kWsByte = 0, kWsPair = 1, kWsPiece = 2;

template <bool SWIGLU, bool BIAS, bool PT, int WSM>
__global__ __launch_bounds__(kF8Threads, kF8MinBlocks) void moe_gemm_f8_kernel(GemmParams p) {
  constexpr int NT = kF8NT, STAGES = kF8Stages, RB = kF8RowBytes, BM = kF8BM;
  constexpr int WN = NT * 32, BN = kWavesN * WN;
  constexpr int NWAVES = kF8WavesM * kWavesN;
  constexpr int U = RB / 16;                        // 16-byte units per row per step
  constexpr int A_BYTES = BM * RB;                  // 4 KB per 64 rows
  constexpr int W_BYTES = BN * RB;                  // 32 KB
  constexpr int A_LOADS = A_BYTES / 1024 / NWAVES;  // 1
  constexpr int W_LOADS = W_BYTES / 1024 / NWAVES;  // 4
  constexpr bool WS2 = WSM == kWsPair, WSP = WSM == kWsPiece;
  constexpr int AS_BYTES = PT ? 0 : BM * 2 * 4;     // the step's activation scale bytes, one dword each
  // the step's weight scale bytes: one dword per row (kWsPair) or per byte
  // (kWsByte), or the rows' byte pairs as they lie in memory (kWsPiece)
  constexpr int WS_BYTES = PT ? 0 : (WSP ? BN * 2 : BN * (WS2 ? 1 : 2) * 4);
  constexpr int AS_GROUPS = BM / 32;                // 32-row groups, one scale DMA each
  constexpr int WS_ROWS = WS2 ? 64 : 32;            // weight rows per scale DMA (per-wave modes)
  constexpr int WS_DMAS = WSP ? 0 : BN / WS_ROWS / NWAVES;  // weight-scale DMAs per wave (per-wave modes)
  static_assert(NWAVES % AS_GROUPS == 0, "every wave issues one activation-scale DMA");
  static_assert(WSP || WS_DMAS * NWAVES * WS_ROWS == BN, "weight-scale split");
  static_assert(!WSP || (BN * 2 == 64 * 16 && AS_GROUPS < NWAVES), "one 16-byte piece per lane of one wave");
  constexpr int T_LOADS = A_LOADS + W_LOADS;        // tile DMAs per step per wave
  // scale DMAs per step of a wave: every wave the same in the per-wave
  // modes; with kWsPiece one for waves 0 .. AS_GROUPS (activation groups,
  // then the weight pieces) and none for the others
  constexpr int S_DMAS = PT ? 0 : (WSP ? 1 : WS_DMAS + 1);
  // A step's scale bytes are loaded one step before its tiles, into their
  // own ring of SR sets; before computing a step a wave may leave in flight
  // the tiles of the next STAGES - 2 steps and the scales of the next
  // STAGES - 1.
  constexpr int SR = STAGES + 1;
  constexpr int SC_BYTES = AS_BYTES + WS_BYTES;
  constexpr int WAIT_N = T_LOADS * (STAGES - 2) + S_DMAS * (STAGES - 1);
  constexpr int WAIT_N0 = T_LOADS * (STAGES - 2);   // a wave that loads no scale bytes
  static_assert(A_LOADS * NWAVES * 1024 == A_BYTES && W_LOADS * NWAVES * 1024 == W_BYTES, "tile split");
  static_assert(WAIT_N < 64, "vmcnt range");
  constexpr int STAGE_BYTES = A_BYTES + W_BYTES;
  static_assert(kF8MinBlocks * (STAGES * STAGE_BYTES + SR * SC_BYTES) <= 160 * 1024, "LDS of the workgroups of one CU");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[STAGES][STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_sc[PT ? 1 : SR][PT ? 16 : SC_BYTES];

  const uint32_t L = xcd_remap(blockIdx.x, gridDim.x);
  const int b = L % p.max_blocks;
  const int tile_n = L / p.max_blocks;
  const int e = p.expert_ids[b];
  if (e < 0 || e >= p.E) return;  // sentinel block

  // PT: rows row0 .. row_end - 1 of A and C (at most 64, clipped to S)
  int row0 = 0, row_end = 0;
  if constexpr (PT) {
    row0 = max(p.blk_off[b], 0);
    row_end = min(min(p.blk_end[b], p.S), row0 + min(p.S - row0, BM));
  }

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wn = wave % kWavesN;
  const int wm = wave / kWavesN;                   // the wave's 64 rows: wm * 64 ..
  const int l32 = lane % 32, h = lane / 32;
  const int32_t* blk_slots = p.sorted + (int64_t)b * BM;
  // slot (output row) of block row r: S (= PAD) for none
  auto slot_of = [&](int r) -> int {
    if constexpr (PT) return row0 + r < row_end ? row0 + r : p.S;
    else return blk_slots[r];
  };
  // A row of slot s
  auto a_row = [&](int s) -> int64_t {
    if constexpr (PT) return s;
    else return s / p.a_row_div;
  };

  // a wave with only PAD rows or only columns past N computes nothing (it
  // still loads its share and joins every barrier)
  const bool rows_live = __ballot(slot_of(wm * 64 + lane) < p.S) != 0;
  const bool cols_live = tile_w_row<NT, SWIGLU>(wn * WN, tile_n, p.N) >= 0;
  const bool wave_live = rows_live && cols_live;

  const uint8_t* a8 = reinterpret_cast<const uint8_t*>(p.a);
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a8, 0, (int)(uint32_t)(p.a_rows * p.a_ld), 0x00020000);
  const __amdgpu_buffer_rsrc_t as_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.as, 0, (int)(uint32_t)(p.a_rows * p.as_ld), 0x00020000);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.w + (int64_t)e * p.w_stride_e), 0, (int)(uint32_t)p.w_span, 0x00020000);
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.ws + (int64_t)e * p.ws_stride_e), 0, (int)(uint32_t)p.ws_span, 0x00020000);

  // ---- per-lane load descriptors (a load instruction fills one 1 KB block
  //      of the stage, 16 bytes per lane in lane order)
  uint32_t a_off[A_LOADS];
  int a_k[A_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int q = (wave * A_LOADS + i) * 64 + lane;
    const int row = q / U, u = swz<U>(row, q % U);
    const int s = slot_of(row);
    a_k[i] = u * 16;
    a_off[i] = s < p.S ? (uint32_t)(a_row(s) * p.a_ld + u * 16) : kOOB;
  }
  uint32_t w_off[W_LOADS];
  int w_k[W_LOADS];
#pragma unroll
  for (int i = 0; i < W_LOADS; ++i) {
    const int q = (wave * W_LOADS + i) * 64 + lane;
    const int row = q / U, u = swz<U>(row, q % U);
    const int32_t wr = tile_w_row<NT, SWIGLU>(row, tile_n, p.N);
    w_k[i] = u * 16;
    w_off[i] = wr >= 0 ? (uint32_t)((int64_t)wr * p.w_row + u * 16) : kOOB;
  }
  // Scale bytes of K block 2 * step + h go by DMA into a scale set (one zero-
  // extended dword per byte, lane order: 32-row group, then h, then the
  // row's place in the group), where each wave reads those of its own rows
  // and columns: the waves of a row group or of a column group would
  // otherwise each load the same bytes. Activation rows: group
  // wave % AS_GROUPS (in the per-wave modes two waves write each group
  // alike); weight rows: groups WS_DMAS * wave + i (kWsPair: 64-row groups,
  // one dword per row holding both bytes), or (kWsPiece) the byte pairs of
  // the tile's rows in row order, 2 bytes per row.
  int32_t my_wrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) my_wrow[nt] = tile_w_row<NT, SWIGLU>(wn * WN + nt * 32 + l32, tile_n, p.N);
  uint32_t ws_off[WS_DMAS > 0 ? WS_DMAS : 1];
#pragma unroll
  for (int i = 0; i < WS_DMAS; ++i) {
    const int r = WS2 ? (WS_DMAS * wave + i) * 64 + lane : (WS_DMAS * wave + i) * 32 + l32;
    const int32_t wr = tile_w_row<NT, SWIGLU>(r, tile_n, p.N);
    ws_off[i] = !PT && wr >= 0 ? (uint32_t)((int64_t)wr * p.ws_row + (WS2 ? 0 : h)) : kOOB;
  }
  // kWsPiece: lane l fetches tile rows 8l .. 8l + 7 (their first row's byte
  // pair; the other seven follow it in memory). A piece whose first row lies
  // past N (or past N/2 gate columns) holds no row in use and reads zeros;
  // the pairs of rows past N inside a used piece feed only columns that are
  // never stored.
  uint32_t wsp_off = kOOB;
  if constexpr (WSP) {
    const int32_t wr = tile_w_row<NT, SWIGLU>(8 * lane, tile_n, p.N);
    wsp_off = wr >= 0 ? (uint32_t)((int64_t)wr * p.ws_row) : kOOB;
  }
  // waves 0 .. AS_GROUPS - 1 load the activation scales, wave AS_GROUPS the
  // weight pieces (kWsPiece); in the per-wave modes every wave loads both
  const bool as_wave = !WSP || wave < AS_GROUPS;
  const bool wsp_wave = WSP && wave == AS_GROUPS;
  const int as_group = wave % AS_GROUPS;
  uint32_t as_off;
  {
    const int s = slot_of(as_group * 32 + l32);
    as_off = !PT && s < p.S ? (uint32_t)(a_row(s) * p.as_ld + h) : kOOB;
  }
  const uint32_t w_blk = (uint32_t)p.w_blk, ws_blk = (uint32_t)p.ws_blk;

  const int nsteps = (p.K + kBK - 1) / kBK;
  const int nsteps_pad = ((nsteps + STAGES - 1) / STAGES) * STAGES;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_u8_t*)&lds[0][0];
  const uint32_t lds_sc_base = (uint32_t)(uintptr_t)(lds_u8_t*)&lds_sc[0][0];
  uint32_t no_regs[1];      // the loads below write no registers the waits must hold

  // Issue the tile loads of K step `step` into stage ST; the K tail and the
  // look-ahead steps past the last one take the checked path (lanes past K
  // read zeros).
  auto issue = [&](int step, auto stage_tag) {
    constexpr int ST = decltype(stage_tag)::value;
    const int k0 = step * kBK;
    const uint32_t base = lds_base + ST * STAGE_BYTES;
    const bool full = k0 + kBK <= p.K;
    const bool live = k0 < p.K;
    const uint32_t sa = live ? (uint32_t)k0 : 0u, sw = live ? (uint32_t)step * w_blk : 0u;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      dma16(a_rsrc, (full || (live && k0 + a_k[i] < p.K)) ? a_off[i] : kOOB, sa,
            base + (wave * A_LOADS + i) * 1024);
#pragma unroll
    for (int i = 0; i < W_LOADS; ++i)
      dma16(w_rsrc, (full || (live && k0 + w_k[i] < p.K)) ? w_off[i] : kOOB, sw,
            base + A_BYTES + (wave * W_LOADS + i) * 1024);
  };
  // The scale bytes of K step `step` into scale set step % SR (a block past
  // K reads 0).
  auto issue_scales = [&](int step) {
    if constexpr (!PT) {
      const int k0 = step * kBK;
      const bool live = k0 < p.K;
      const uint32_t ss = live ? (uint32_t)step * ws_blk : 0u, sas = live ? (uint32_t)step * 2 : 0u;
      const bool h_live = live && k0 + 32 * h < p.K;
      const uint32_t base = lds_sc_base + (uint32_t)(step % SR) * SC_BYTES;
#pragma unroll
      for (int i = 0; i < WS_DMAS; ++i) {
        if constexpr (WS2) dma_ushort(s_rsrc, live ? ws_off[i] : kOOB, ss, base + AS_BYTES + (WS_DMAS * wave + i) * 256);
        else dma_byte(s_rsrc, h_live ? ws_off[i] : kOOB, ss, base + AS_BYTES + (WS_DMAS * wave + i) * 256);
      }
      if constexpr (WSP) {
        if (wsp_wave) dma16(s_rsrc, live ? wsp_off : kOOB, ss, base + AS_BYTES);
      }
      if (as_wave) dma_byte(as_rsrc, h_live ? as_off : kOOB, sas, base + as_group * 256);
    }
  };

  f32x16_t acc[2][NT];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.0f;

  // operand of LDS row `row`: units h and 2 + h of its 64-byte step piece
  auto operand = [&](const lds_u8_t* part, int row) -> f8_v8i {
    const u32x4_t lo = lds_read<u32x4_t>(part + row * RB + swz<U>(row, h) * 16);
    const u32x4_t hi = lds_read<u32x4_t>(part + row * RB + swz<U>(row, 2 + h) * 16);
    f8_v8i r;
    r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
    r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
    return r;
  };

  auto compute = [&](auto stage_tag, int step) {
    constexpr int ST = decltype(stage_tag)::value;
    const lds_u8_t* As = (const lds_u8_t*)&lds[ST][0];
    const lds_u8_t* Ws = As + A_BYTES;
    f8_v8i af[2];
    int sa[2] = {kE8M0One, kE8M0One};
    const lds_u8_t* Sa = (const lds_u8_t*)&lds_sc[0][0] + (step % SR) * SC_BYTES;  // activation scale dwords
    const lds_u8_t* Ss = Sa + AS_BYTES;                                              // weight scale dwords
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      af[mt] = operand(As, wm * 64 + mt * 32 + l32);
      if constexpr (!PT) sa[mt] = (int)lds_read<uint32_t>(Sa + ((2 * wm + mt) * 64 + lane) * 4);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const f8_v8i bf = operand(Ws, wn * WN + nt * 32 + l32);
      int sw = kE8M0One;
      if constexpr (!PT && WSP) {
        // the row's byte of K block 2 * step + h; the second block of a half
        // K step lies past K
        const int sb = lds_read<uint8_t>(Ss + (wn * WN + nt * 32 + l32) * 2 + h);
        sw = (h && step * kBK + 32 >= p.K) ? 0 : sb;
      } else if constexpr (!PT && WS2) {
        // both bytes of the row; the second block of a half K step lies past K
        const uint32_t d = lds_read<uint32_t>(Ss + (wn * WN + nt * 32 + l32) * 4);
        sw = (h && step * kBK + 32 >= p.K) ? 0 : (int)((d >> (8 * h)) & 0xffu);
      } else if constexpr (!PT) {
        sw = (int)lds_read<uint32_t>(Ss + ((wn * NT + nt) * 64 + lane) * 4);
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            af[mt], bf, acc[mt][nt], 0, 0, 0, sa[mt], 0, sw);
    }
  };

  // STAGES - 1 steps in flight: wait for this step's loads (the younger
  // look-ahead ones may still run), barrier, load the tiles of step +
  // STAGES - 1 into the stage every wave has finished computing on, compute
  // this one, then load the scales of step + STAGES into the set of the step
  // before this one (every wave is past it: it computed before the barrier).
  // Issue order: scales(0), then per step t < STAGES - 1 tiles(t) and
  // scales(t + 1).
  issue_scales(0);
  static_for<0, STAGES - 1>([&](auto st) {
    constexpr int ST = decltype(st)::value;
    issue(ST, st);
    issue_scales(ST + 1);
  });
  // (kWsPiece: the waves that load no scale bytes have fewer loads in flight)
  const bool scale_wave = !WSP || as_wave || wsp_wave;
  for (int step = 0; step < nsteps_pad; step += STAGES) {
    static_for<0, STAGES>([&](auto st) {
      constexpr int ST = decltype(st)::value;
      if (scale_wave) wait_loads_barrier<WAIT_N>(no_regs);
      else wait_loads_barrier<WAIT_N0>(no_regs);
      issue(step + ST + STAGES - 1, std::integral_constant<int, (ST + STAGES - 1) % STAGES>{});
      if (wave_live) compute(st, step + ST);
      issue_scales(step + ST + STAGES);
    });
  }
  // drain the look-ahead loads, then keep the slot list (PT: each row's
  // combined scale) in stage 0
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int32_t* s_slot = reinterpret_cast<int32_t*>(&lds[0][0]);
  float* s_scale = reinterpret_cast<float*>(&lds[0][0]) + BM;
  if (tid < BM) {
    const int s = slot_of(tid);
    s_slot[tid] = s;
    if constexpr (PT) s_scale[tid] = s < p.S ? p.tok_scale[s] * p.exp_scale[e] : 0.0f;
  }
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
  // (after the slot list and the row scales)
  if (p.c_ld % 8 == 0 && ((uintptr_t)p.c & 15) == 0) {
    constexpr int OC = SWIGLU ? WN / 2 : WN;  // output columns of this wave
    static_assert(BM * 8 + NWAVES * stage_rows_bytes<OC>() <= STAGES * STAGE_BYTES, "staging fits");
    lds_u8_t* const lds0 = (lds_u8_t*)&lds[0][0];
    const int col0 = SWIGLU ? tile_n * (BN / 2) + wn * (WN / 2) : tile_n * BN + wn * WN;
    const int out_w = SWIGLU ? p.N / 2 : p.N;
    store_tile_rows<OC>(
        [&](int mt, int j, int i) {
          if constexpr (!SWIGLU) {
            const float rs = PT ? s_scale[wm * 64 + mt * 32 + (i / 4) * 8 + h * 4 + (i % 4)] : 1.0f;
            const float v = (PT ? acc[mt][j][i] * rs : acc[mt][j][i]) + bv[j];
            return p.relu2 ? relu2_f32(v) : v;
          } else {
            static_assert(!PT, "the per-token mode has no SwiGLU epilogue");
            const float g = acc[mt][j][i] + bv[j];
            const float up = acc[mt][j + NT / 2][i] + bv[j + NT / 2];
            return silu_f32(g) * up;
          }
        },
        lds0 + BM * 8 + wave * stage_rows_bytes<OC>(), lds0, wm * 64, p.c, p.c_ld, p.S, col0, out_w, lane);
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
      const float rs = PT ? s_scale[row] : 1.0f;
      if constexpr (!SWIGLU) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if (my_wrow[nt] >= 0) {
            const float v = (PT ? acc[mt][nt][i] * rs : acc[mt][nt][i]) + bv[nt];
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

hipError_t launch_gemm_f8(const GemmParams& p, bool swiglu, bool bias, hipStream_t stream) {
  if (p.max_blocks <= 0) return hipSuccess;
  const int bn = kWavesN * 32 * kF8NT;
  const int64_t tiles = swiglu ? (p.N / 2 + bn / 2 - 1) / (bn / 2) : (p.N + bn - 1) / bn;
  const dim3 grid((uint32_t)(tiles * p.max_blocks));
  // the K-block layout with 16-byte aligned pieces of 8 rows' byte pairs
  // (a SwiGLU tile's up rows start at N/2 + a multiple of 8)?
  const bool wsp = p.ws_row == 2 && p.ws_blk % 16 == 0 && p.ws_stride_e % 16 == 0 &&
                   ((uintptr_t)p.ws & 15) == 0 && (!swiglu || (p.N / 2) % 8 == 0);
  // else both scale bytes of a row's step in one aligned 2-byte load?
  const bool ws2 = p.ws_row % 2 == 0 && p.ws_blk % 2 == 0 && p.ws_stride_e % 2 == 0 && (uintptr_t)p.ws % 2 == 0;
  const int wsm = wsp ? kWsPiece : (ws2 ? kWsPair : kWsByte);
#define MOE_LAUNCH_F8(SW, BI) \
  do { \
    if (wsm == kWsPiece) hipLaunchKernelGGL((moe_gemm_f8_kernel<SW, BI, false, kWsPiece>), grid, dim3(kF8Threads), 0, stream, p); \
    else if (wsm == kWsPair) hipLaunchKernelGGL((moe_gemm_f8_kernel<SW, BI, false, kWsPair>), grid, dim3(kF8Threads), 0, stream, p); \
    else hipLaunchKernelGGL((moe_gemm_f8_kernel<SW, BI, false, kWsByte>), grid, dim3(kF8Threads), 0, stream, p); \
  } while (0)
  if (swiglu) {
    if (bias) MOE_LAUNCH_F8(true, true);
    else MOE_LAUNCH_F8(true, false);
  } else {
    if (bias) MOE_LAUNCH_F8(false, true);
    else MOE_LAUNCH_F8(false, false);
  }
#undef MOE_LAUNCH_F8
  return hipGetLastError();
}

hipError_t launch_gemm_per_token(const GemmParams& p, bool bias, hipStream_t stream) {
  if (p.max_blocks <= 0) return hipSuccess;
  const int bn = kWavesN * 32 * kF8NT;
  const dim3 grid((uint32_t)((p.N + bn - 1) / bn * (int64_t)p.max_blocks));
  if (bias) hipLaunchKernelGGL((moe_gemm_f8_kernel<false, true, true, kWsByte>), grid, dim3(kF8Threads), 0, stream, p);
  else hipLaunchKernelGGL((moe_gemm_f8_kernel<false, false, true, kWsByte>), grid, dim3(kF8Threads), 0, stream, p);
  return hipGetLastError();
}

int gemm_block_m_f8() { return kF8BM; }

}  // namespace moe
