// Building blocks of the large-M grouped GEMM kernels (bf16 activations in
// gemm.hip, MXFP8 activations in gemm_f8.hip): the workgroup shape, the
// LDS-DMA and byte loads issued with inline assembly, the wait-and-barrier of
// the K loop, the LDS swizzle, the staged store of an output tile and the
// weight rows of an N tile.
#pragma once

#include <type_traits>

#include "common.h"
#include "params.h"

namespace moe {

constexpr int kWavesM = 1;                        // waves along M
constexpr int kWavesN = 4;                        // waves along N
constexpr int kBM = 64 * kWavesM;                 // the routing block
constexpr int kBK = 64;
constexpr int kThreads = kWave * kWavesM * kWavesN;  // 256
constexpr int kMinBlocks = 2;                     // workgroups per CU (LDS and registers allow two)
// A per-lane buffer offset past every buffer the kernel reads (each is below
// 2 GB, checked by the host API), also after a scalar step offset below 2 GB
// is added: such a lane reads zeros.
constexpr uint32_t kOOB = 0x80000000u;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

// Typed reads from an LDS address (kept in the LDS address space so the
// compiler can tell the stages apart).
template <typename T>
__device__ __forceinline__ T lds_read(const lds_u8_t* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(p);
}

// The K loop's loads are issued with inline assembly, so the compiler does
// not track them: it inserts no waits of its own (its alias analysis cannot
// tell the LDS stages apart and would wait for every load in flight), and the
// loop's explicit waits below are the whole synchronisation.
//
// 16 bytes per lane from buffer `rsrc` at byte offset `voff` + `soff` into
// LDS at `lds_base` + 16 * lane; a lane whose `voff` is kOOB reads zeros.
// `soff` (the step's advance) and `lds_base` are wave-uniform.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, %3 offen lds"
               :: "v"(voff), "s"(__builtin_amdgcn_readfirstlane(lds_base)), "s"(rsrc),
                  "s"(__builtin_amdgcn_readfirstlane(soff)) : "m0");
}

// One byte per lane from buffer `rsrc` at `voff` + `soff` into LDS, written
// zero-extended as the dword at `lds_base` + 4 * lane (measured on gfx950); a
// lane whose `voff` is kOOB writes 0.
__device__ __forceinline__ void dma_byte(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_ubyte %0, %2, %3 offen lds"
               :: "v"(voff), "s"(__builtin_amdgcn_readfirstlane(lds_base)), "s"(rsrc),
                  "s"(__builtin_amdgcn_readfirstlane(soff)) : "m0");
}

// One byte from buffer `rsrc` at `voff` + `soff` into a register (zero for a
// lane whose `voff` is kOOB).
__device__ __forceinline__ uint32_t load_byte(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff) {
  uint32_t v;
  asm volatile("buffer_load_ubyte %0, %1, %2, %3 offen"
               : "=v"(v) : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)));
  return v;
}

// Wait until at most N of this wave's loads are in flight and its LDS
// operations are done, then barrier. The registers passed in are loads whose
// values must not be used before this point; the "memory" clobber keeps LDS
// accesses on their side of the barrier.
template <int N, int R>
__device__ __forceinline__ void wait_loads_barrier(uint32_t (&regs)[R]) {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  if constexpr (R == 6) {
    asm volatile("s_waitcnt vmcnt(%6) lgkmcnt(0)\n\ts_barrier"
                 : "+v"(regs[0]), "+v"(regs[1]), "+v"(regs[2]), "+v"(regs[3]), "+v"(regs[4]), "+v"(regs[5])
                 : "n"(N) : "memory");
  } else if constexpr (R == 4) {
    asm volatile("s_waitcnt vmcnt(%4) lgkmcnt(0)\n\ts_barrier"
                 : "+v"(regs[0]), "+v"(regs[1]), "+v"(regs[2]), "+v"(regs[3]) : "n"(N) : "memory");
  } else if constexpr (R == 2) {
    asm volatile("s_waitcnt vmcnt(%2) lgkmcnt(0)\n\ts_barrier"
                 : "+v"(regs[0]), "+v"(regs[1]) : "n"(N) : "memory");
  } else {
    static_assert(R == 1, "registers to hold until the wait: 1 (none), 2, 4 or 6");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
  }
}

// Physical 16-byte unit of logical unit u in LDS row `row` (rows of U units).
// gfx950's LDS serves a ds_read_b128 16 lanes at a time from 64 banks
// (256 bytes); the 16 rows one such group reads get distinct 16-byte slots
// of that window (measured: conflict-free, where a 32-bank layout conflicts
// two-way).
template <int U>
__device__ __forceinline__ int swz(int row, int u) {
  return u ^ ((row / (16 / U)) % U);
}

// Bytes of LDS a wave needs to stage 32 rows of OC output columns
// (row stride OC * 2 + 16 bytes: the 16 spread the rows over the banks).
template <int OC>
constexpr int stage_rows_bytes() { return 32 * (OC * 2 + 16); }

// Stores a wave's output tile (two 32-row MFMA row tiles of OC columns) to
// the bf16 rows of C in 16-byte pieces. In the 32x32 MFMA layout a lane
// holds one column and 16 rows of a tile, so storing straight from the
// accumulators writes 2 bytes per lane and instruction; instead, per 32-row
// tile, adjacent lanes pair their columns (one DPP swap: the even lane keeps
// row i, the odd lane row i + 1), the 4-byte pairs go to this wave's LDS
// area `stg` (stage_rows_bytes<OC>() bytes, 16-byte aligned), and each lane
// reads back 8 consecutive columns of one row and stores them whole.
//   val(mt, j, i): the output value (fp32, before its one bf16 rounding) of
//     row mt * 32 + (i / 4) * 8 + h * 4 + i % 4 and column j * 32 + l32 of
//     the wave's tile (lane = 32 h + l32);
//   slots: LDS list of the tile's slot ids, row r of the wave at slots[r0 + r];
//     C row = slot id, none when it is >= S;
//   columns col0 .. col0 + OC - 1 of C, those >= out_w not stored.
// c must be 16-byte aligned and c_ld a multiple of 8 (16-byte row pieces).
template <int OC, class F>
__device__ __forceinline__ void store_tile_rows(F&& val, lds_u8_t* stg, const lds_u8_t* slots, int r0, uint16_t* c,
                                                int64_t c_ld, int S, int col0, int out_w, int lane) {
  constexpr int XS = OC * 2 + 16;  // staging row stride, bytes
  constexpr int PR = OC / 8;       // 16-byte pieces per row
  static_assert(OC % 32 == 0 && 64 % PR == 0, "columns per wave");
  const int l32 = lane % 32, h = lane / 32, odd = lane & 1;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int j = 0; j < OC / 32; ++j) {
#pragma unroll
      for (int ip = 0; ip < 8; ++ip) {
        const int i0 = 2 * ip;
        const uint32_t v0 = f32_to_bf16_bits(val(mt, j, i0));
        const uint32_t v1 = f32_to_bf16_bits(val(mt, j, i0 + 1));
        // the even lane receives its odd neighbour's row i0, the odd lane its
        // even neighbour's row i0 + 1
        const uint32_t nb = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(odd ? v0 : v1), 0xB1, 0xF, 0xF, false);
        const uint32_t word = odd ? (nb | (v1 << 16)) : (v0 | (nb << 16));
        const int row = (i0 / 4) * 8 + h * 4 + i0 % 4 + odd;
        const int col = j * 32 + (l32 & ~1);
        *reinterpret_cast<__attribute__((address_space(3))) uint32_t*>(stg + row * XS + col * 2) = word;
      }
    }
    // (a wave's LDS operations complete in order: the pieces read below see
    // the pairs written above, and the next tile's pairs are written after
    // these reads; the empty asm keeps the compiler from reordering them)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int it = 0; it < 32 * PR / 64; ++it) {
      const int q = it * 64 + lane;
      const int row = q / PR, pc = q % PR;
      const u32x4_t v = lds_read<u32x4_t>(stg + row * XS + pc * 16);
      const int s = lds_read<int32_t>(slots + (r0 + mt * 32 + row) * 4);
      const int col = col0 + pc * 8;
      if (s < S && col < out_w) {
        uint16_t* dst = c + (int64_t)s * c_ld + col;
        if (col + 8 <= out_w) {
          *reinterpret_cast<u32x4_t*>(dst) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (col + e < out_w) dst[e] = (uint16_t)(v[e / 2] >> (16 * (e % 2)));
        }
      }
    }
    asm volatile("" ::: "memory");
  }
}

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Global weight row of local tile row r, or -1 beyond N.
template <int NT, bool SWIGLU>
__device__ __forceinline__ int32_t tile_w_row(int r, int tile_n, int N) {
  constexpr int WN = NT * 32;
  constexpr int BN = kWavesN * WN;
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

}  // namespace moe
