// moe_wgrad: dW[e] = sum over the slots s routed to e of grad[s]^T x[s / top_k],
// fp32, straight from moe_align's sorted_token_ids / expert_ids.
//
// Follows ROCm/aiter PR #5310 "Add MoE GEMM variants and weight-gradient
// kernel": Summary (moe_wgrad replaces sort + pad + bmm and a host sync; its
// atomics needed dW reset between benchmark trials or results were corrupted)
// and Tests & Benchmarks (constant input, linearity, zero-padded tokens).
//
// Design for gfx950:
//  * dW is cut into (expert, 256 x 256) tiles. A persistent grid (one
//    workgroup of 8 waves per CU) walks them; each tile is accumulated over
//    its expert's routing blocks on v_mfma_f32_32x32x16_bf16 and written
//    once, so dW is overwritten (never accumulated into), empty experts get
//    zeros, nothing is atomic and repeated calls give identical bits.
//  * Slot rows of grad (256 columns) and x (256 columns), 512 bytes each, go
//    straight from global memory into LDS with buffer_load ... lds,
//    slot-major as they lie in memory, 32 slots per pipeline unit in four
//    32 KB stages. Units go in pairs (one 64-slot routing block): one
//    barrier per pair, after which the next pair's loads are issued (across
//    tile boundaries) and the pair is computed (one barrier per unit with
//    three stages measured 2% slower). Each wave computes 64 x 128 of the
//    tile: 16 MFMAs per unit. The
//    tile size is what the operand traffic asks for: loading both operands
//    costs (rows + columns) bytes per slot for rows x columns products, and
//    256 x 256 measured faster than 128 x 256 at two workgroups per CU
//    (5.7 against 6.5 ms on the E=256 gradient); larger tiles would need
//    more accumulator registers than two waves per SIMD allow.
//  * The contraction runs over slots, so an MFMA operand needs 8 consecutive
//    slots of one column: gfx950's transposing LDS read (ds_read_b64_tr_b16)
//    gathers them. Within each 16-lane group, lane j receives element j % 4
//    of the 8-byte reads of lanes j/4, j/4 + 4, j/4 + 8, j/4 + 12 (measured);
//    lane s of the group therefore points at slot (s / 4) and columns
//    4 (s % 4) .. + 3, and lane j ends up with column j of four consecutive
//    slots. Two such reads make one operand.
//  * A finished tile goes out through LDS: the MFMA output holds one column
//    per lane, so each wave passes 8 rows at a time through a scratch area
//    (the stage the next unit's loads will fill, free at that point; rows
//    4..7 of a pass XOR their columns with 32 so both halves of a write hit
//    distinct banks) and writes whole 512-byte row pieces with 16-byte
//    non-temporal stores.
//    Storing the MFMA output as it lies (one dword per lane, 128-byte row
//    stretches) issues four times the store instructions; four adjacent
//    columns per lane from swapped operands (32-byte stretches) measured
//    slower still.
//  * The 16-byte units of each LDS row are XOR-swizzled by slot.
//  * Tiles are numbered expert-major, then in groups of 8 N tiles walked
//    N-fastest, and each XCD takes consecutive tiles: the 64 workgroups an
//    XCD runs at once cover 8 x 8 tiles of one expert, whose grad and x
//    slices stay in its L2.
//  * Every expert's block range comes from one pass over expert_ids (sorted
//    by expert, sentinels last) into an LDS table at the start; slot ids are
//    read with scalar loads one unit ahead of their use and turned into row
//    offsets on the scalar unit (the token row s / top_k by a multiply-high),
//    so a load costs each lane only a select and an add. PAD slots and the
//    look-ahead past the last tile read zeros through the buffer bounds;
//    columns past N or K read whatever follows in memory and only reach dW
//    rows and columns that are never stored.
#include "common.h"
#include "params.h"

namespace moe {

constexpr int kWgBM = 64;                    // routing block
constexpr int kWgUM = 32;                    // slots per pipeline unit
constexpr int kWgTN = 256;                   // dW rows (N) per tile
constexpr int kWgTK = 256;                   // dW columns (K) per tile
constexpr int kWgGRowB = kWgTN * 2;          // 512 B: a slot's grad piece
constexpr int kWgXRowB = kWgTK * 2;          // 512 B: a slot's x piece
constexpr int kWgGUnitB = kWgUM * kWgGRowB;  // 16 KB
constexpr int kWgXUnitB = kWgUM * kWgXRowB;  // 16 KB
constexpr int kWgStageB = kWgGUnitB + kWgXUnitB;
constexpr int kWgStages = 4;                 // two pairs of units
constexpr int kWgWaves = 8;
constexpr int kWgThreads = kWgWaves * 64;
constexpr int kWgGLoads = kWgGUnitB / 1024 / kWgWaves;  // DMA instructions per wave per unit: 2 grad
constexpr int kWgXLoads = kWgXUnitB / 1024 / kWgWaves;  //   + 2 x (2 rows each)
constexpr int kWgStores = 8 * 4;             // 16-byte stores per lane per tile
constexpr int kWgPerCU = 1;                  // resident workgroups per CU
constexpr int kWgMaxExperts = 1024;
constexpr int kWgGroupN = 8;                 // N tiles per group of the tile order
constexpr uint32_t kWgOOB = 0x80000000u;     // buffer offset past x, grad and one expert's dW (each below 2 GB)
constexpr int kWgStoreNT = 2;                // cache-policy bits of the dW stores: non-temporal
static_assert(kWgGLoads == 2 && kWgXLoads == 2, "each wave loads the same 4 slot rows of both parts");

typedef __attribute__((address_space(3))) uint8_t wg_lds_u8_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short wg_s16x4_t;

// Physical 16-byte unit of logical unit u in LDS row (slot) m. A
// transposing read covers 4 consecutive slots x 2 consecutive units per
// 16-lane group; XOR-ing the unit with 4 (m % 4) moves the four slots' pieces
// 64 bytes apart, onto distinct banks (rows are 256 or 512 bytes long).
__device__ __forceinline__ int wg_swz(int m, int u) { return u ^ ((m % 4) * 4); }

// 16 bytes per lane from `rsrc` at `voff` into LDS at lds_base + 16 * lane.
__device__ __forceinline__ void wg_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
               :: "v"(voff), "s"(__builtin_amdgcn_readfirstlane(lds_base)), "s"(rsrc) : "m0");
}

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int wg_i32x4_t;

// 4 consecutive int32 at byte `off` of buffer `rsrc` through the scalar
// cache (a read). Asynchronous: the result must not be used before an
// lgkmcnt(0) wait that lists it (wg_wait_barrier).
__device__ __forceinline__ wg_i32x4_t wg_scalar_ids4(__amdgpu_buffer_rsrc_t rsrc, uint32_t off) {
  wg_i32x4_t v;
  asm volatile("s_buffer_load_dwordx4 %0, %1, %2"
               : "=s"(v) : "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(off)));
  return v;
}

// Wait until at most N of this wave's vector-memory operations are in
// flight and every LDS and scalar-memory operation is done, then barrier;
// `a` and `b` (prefetched scalar loads) are final from here on.
template <int N>
__device__ __forceinline__ void wg_wait_barrier(wg_i32x4_t& a, wg_i32x4_t& b) {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%2) lgkmcnt(0)\n\ts_barrier" : "+s"(a), "+s"(b) : "n"(N) : "memory");
}

// Operand of 8 consecutive slots [m0, m0 + 8) of tile column c0 + lane % 32,
// for the 32-wide MFMA fragment: lane l takes column c0 + l % 32 and slots
// m0 + 8 (l / 32) + i. Built from two transposing reads (slots +0..3, +4..7)
// of an LDS part whose rows are ROWB bytes.
template <int ROWB>
__device__ __forceinline__ bf16x8_t wg_operand(const wg_lds_u8_t* part, int c0, int m0, int lane) {
  const int g = lane / 16, s = lane % 16;
  const int col = c0 + 16 * (g % 2) + 4 * (s % 4);
  const int slot = m0 + 8 * (g / 2) + s / 4;
  bf16x8_t r;
  wg_s16x4_t v[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int m = slot + 4 * half;
    const int byte = m * ROWB + wg_swz(m, col / 8) * 16 + (col % 8) * 2;
    v[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) wg_s16x4_t*)(part + byte));
  }
  __builtin_memcpy(&r, v, 16);
  return r;
}

// A tile of dW and its expert's block range.
struct WgTile {
  int e, n0, k0, b0, b1;
};

__global__ __launch_bounds__(kWgThreads, kWgPerCU) void wgrad_kernel(WgradParams p) {
  // four stages of [grad unit | x unit], slot-major
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kWgStages][kWgStageB];
  __shared__ int32_t s_start[kWgMaxExperts + 1];  // first block of expert e (s_start[E] = end)

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l32 = lane % 32, h = lane / 32;

  // ---- expert block ranges: experts (lo, hi] start at every block b where
  //      the expert id changes (lo = previous id, hi = this id, or E for the
  //      first sentinel); experts past the last boundary start at max_blocks
  for (int e = tid; e <= p.E; e += kWgThreads) s_start[e] = p.max_blocks;
  __syncthreads();
  for (int b = tid; b < p.max_blocks; b += kWgThreads) {
    const int cur = p.expert_ids[b];
    const int prev = b > 0 ? p.expert_ids[b - 1] : -1;
    const int hi = (cur < 0 || cur > p.E) ? p.E : cur;
    const int lo = (b == 0 || prev < 0) ? -1 : prev;
    if ((b == 0 || prev != cur) && !(prev < 0 && cur < 0 && b > 0))
      for (int e = lo + 1; e <= hi; ++e) s_start[e] = b;
  }
  __syncthreads();

  // Tile order: expert-major; within an expert, groups of kWgGroupN N tiles
  // walked N-fastest then K, so any kWgGroupN x (64 / kWgGroupN) consecutive
  // tiles share a few grad and x slices. XCD x (= hardware id % 8) owns the
  // x-th eighth of the sequence, and its G/8 workgroups take consecutive
  // tiles of it round by round (G = gridDim.x).
  const int per_e = p.tiles_n * p.tiles_k;
  const int total = p.E * per_e;  // below 2^31 (checked by the host API)
  const int G = gridDim.x;
  const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
  const int chunk = (total + 7) / 8;
  auto tile_index = [&](int it) -> int {
    const int q = it * (G / 8) + local;
    const int T = xcd * chunk + q;
    return (q < chunk && T < total) ? T : total;
  };
  auto tile_at = [&](int T) {
    WgTile t;
    t.e = T / per_e;
    const int r = T % per_e;
    const int in_group = kWgGroupN * p.tiles_k;
    const int first_n = (r / in_group) * kWgGroupN;
    const int gsize = min(p.tiles_n - first_n, kWgGroupN);
    t.n0 = (first_n + (r % in_group) % gsize) * kWgTN;
    t.k0 = ((r % in_group) / gsize) * kWgTK;
    t.b0 = __builtin_amdgcn_readfirstlane(s_start[t.e]);
    t.b1 = __builtin_amdgcn_readfirstlane(s_start[t.e + 1]);
    return t;
  };

  const __amdgpu_buffer_rsrc_t g_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.grad, 0, (int)(uint32_t)((int64_t)p.S * p.grad_ld * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t x_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.x, 0, (int)(uint32_t)((int64_t)(p.S / p.top_k) * p.x_ld * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t sorted_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.sorted, 0, (int)(uint32_t)((int64_t)p.max_blocks * kWgBM * 4), 0x00020000);
  const uint32_t lds_base = (uint32_t)(uintptr_t)(wg_lds_u8_t*)&lds[0][0];
  const uint32_t g_row = (uint32_t)(p.grad_ld * 2), x_row = (uint32_t)(p.x_ld * 2);

  // ---- loader: walks the same tiles' units one pair ahead of the
  //      computation. Unit u of a tile is slots [32u, 32u + 32) of its block
  //      list; wave w loads slot rows 4w .. 4w + 3 of both parts (two
  //      instructions of 2 rows x 32 lanes each).
  //      Past the last tile it issues loads that read zeros, so every unit
  //      costs the same number of loads.
  // The 16-byte unit each lane fetches, as a byte offset within the row
  // piece (the LDS side is lane order, the global side the swizzled unit):
  // load i of either part has row % 4 = 2 (i % 2) + lane / 32.
  const uint32_t x_col0 = (uint32_t)wg_swz(lane / 32, lane % 32) * 16;
  const uint32_t x_col1 = (uint32_t)wg_swz(2 + lane / 32, lane % 32) * 16;
  // all-ones mask of the lanes that take the second row of a load (a
  // select by bit logic, one VALU operation)
  const uint32_t xm1 = lane >= 32 ? ~0u : 0u;
  auto pick = [](uint32_t mask, uint32_t a, uint32_t b) { return (a & mask) | (b & ~mask); };

  int ld_it = 0;
  WgTile ld = tile_at(tile_index(0));
  int ld_u = 0;
  bool ld_live = tile_index(0) < total;
  auto ld_skip_empty = [&]() {  // move to the next tile with a unit left (empty experts have none)
    while (ld_live && ld_u >= 2 * (ld.b1 - ld.b0)) {
      ++ld_it;
      ld_u = 0;
      const int T = tile_index(ld_it);
      ld_live = T < total;
      if (ld_live) ld = tile_at(T);
    }
  };
  // the ids of the pair of units the loader points at (a pair is one
  // 64-slot routing block, never split across tiles)
  auto ld_ids_pair = [&](wg_i32x4_t& a, wg_i32x4_t& b) {
    a = wg_i32x4_t{0, 0, 0, 0};
    b = a;
    if (ld_live) {
      const uint32_t off = (uint32_t)((ld.b0 * kWgBM + ld_u * kWgUM + wave * 4) * 4);
      a = wg_scalar_ids4(sorted_rsrc, off);
      b = wg_scalar_ids4(sorted_rsrc, off + kWgUM * 4);
    }
  };
  ld_skip_empty();
  wg_i32x4_t ids, ids_b;
  ld_ids_pair(ids, ids_b);
  wg_wait_barrier<0>(ids, ids_b);

  auto issue_unit = [&](int stage, const wg_i32x4_t& uid) {
    // scalar row offsets of the wave's 8 slots within the tile's column
    // range (a PAD slot s = S lands at or past the end of both buffers)
    // (past the last tile the ids are 0 and the bases put every lane past
    // the buffers: s * row + kWgOOB stays below 2^32)
    const uint32_t g_base = ld_live ? (uint32_t)ld.n0 * 2 : kWgOOB;
    const uint32_t x_base = ld_live ? (uint32_t)ld.k0 * 2 : kWgOOB;
    uint32_t go[4], xo[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t s = (uint32_t)uid[r];
      const uint64_t prod = ((uint64_t)__umulhi(s, p.topk_magic) << 32) | (s * p.topk_magic);
      const uint32_t xrow = (uint32_t)(prod >> p.topk_shift);
      go[r] = s * g_row + g_base;
      xo[r] = xrow * x_row + x_base;
    }
    const uint32_t dst = lds_base + (uint32_t)(stage * kWgStageB);
#pragma unroll
    for (int i = 0; i < kWgGLoads; ++i)
      wg_dma16(g_rsrc, pick(xm1, go[2 * i + 1], go[2 * i]) + (i % 2 ? x_col1 : x_col0),
               dst + (uint32_t)((wave * kWgGLoads + i) * 1024));
#pragma unroll
    for (int i = 0; i < kWgXLoads; ++i)
      wg_dma16(x_rsrc, pick(xm1, xo[2 * i + 1], xo[2 * i]) + (i % 2 ? x_col1 : x_col0),
               dst + (uint32_t)(kWgGUnitB + (wave * kWgXLoads + i) * 1024));
  };
  auto issue_pair = [&](int stage) {  // stages stage, stage + 1
    issue_unit(stage, ids);
    issue_unit(stage + 1, ids_b);
    if (ld_live) {
      ld_u += 2;
      ld_skip_empty();
      ld_ids_pair(ids, ids_b);  // complete by the next wait
    }
  };

  // waves 4 x 2: wave (wn, wk) computes dW rows n0 + wn*64 .. + 63 and
  // columns k0 + wk*128 .. + 127
  const int wn = wave / 2, wk = wave % 2;
  f32x16_t acc[2][4];  // [n sub-tile][k sub-tile]
  auto contract = [&](int stage) {
    const wg_lds_u8_t* gt = (const wg_lds_u8_t*)&lds[stage][0];
    const wg_lds_u8_t* xt = gt + kWgGUnitB;
    // every operand of the unit first (their LDS latency overlaps), then the MFMAs
    constexpr int KS = kWgUM / 16;
    bf16x8_t af[KS][2], bfr[KS][4];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int i = 0; i < 2; ++i) af[ks][i] = wg_operand<kWgGRowB>(gt, wn * 64 + i * 32, ks * 16, lane);
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[ks][j] = wg_operand<kWgXRowB>(xt, wk * 128 + j * 32, ks * 16, lane);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][i], bfr[ks][j], acc[i][j], 0, 0, 0);
  };

  // ---- computation, a pair of units (one routing block) per barrier:
  //      before a pair the wave waits until only the stores of a tile
  //      finished just before are in flight (the pair's loads were issued
  //      before them); the barrier makes every wave's DMA visible and
  //      guarantees all waves finished the previous pair, whose two stages
  //      the loads issued next overwrite.
  issue_pair(0);
  int st = 0;  // first stage of the next pair computed
  bool stored = false;
  for (int it = 0; tile_index(it) < total; ++it) {
    const WgTile t = tile_at(tile_index(it));
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    const int nu = 2 * (t.b1 - t.b0);
    for (int u = 0; u < nu; u += 2) {
      if (stored) {
        wg_wait_barrier<kWgStores>(ids, ids_b);
        stored = false;
      } else {
        wg_wait_barrier<0>(ids, ids_b);
      }
      issue_pair(st ^ 2);  // the pair computed last, now free
      contract(st);
      contract(st + 1);
      st ^= 2;
    }
    // store the tile through LDS: the first stage of the pair computed last
    // is free once every wave is past its last contraction (the next
    // pair's loads go to the other two). Each wave
    // passes 8 rows at a time through its own 4 KB of it and writes whole
    // 512-byte row pieces with 16-byte stores.
    __syncthreads();
    {
      // every lane issues its kWgStores stores, also at the N and K edges
      // (lanes past them write through an offset past the expert's dW, which
      // the buffer drops), so the waits above, which count them, stay exact
      const __amdgpu_buffer_rsrc_t dw_rsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.dw + (int64_t)t.e * p.N * p.K), 0, (int)(uint32_t)((int64_t)p.N * p.K * 4), 0x00020000);
      const int free_stage = st ^ 2;  // the last pair's first stage
      __attribute__((address_space(3))) float* scr =
          (__attribute__((address_space(3))) float*)&lds[free_stage][wave * 8 * 512];
#pragma unroll
      for (int pass = 0; pass < 8; ++pass) {
        const int i = pass / 4, q = pass % 4;
        // lane (l32, h) holds rows i*32 + 8q + 4h + (0..3) of columns j*32 + l32;
        // rows 4..7 of the scratch are stored with columns XOR 32 (distinct banks)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) scr[(4 * h + r) * 128 + ((j * 32 + l32) ^ (32 * h))] = acc[i][j][4 * q + r];
#pragma unroll
        for (int rd = 0; rd < 4; ++rd) {
          const int lr = 2 * rd + h;  // local row 0..7 of the pass
          const f32x4_t v = *(const __attribute__((address_space(3))) f32x4_t*)&scr[lr * 128 + ((4 * l32) ^ (32 * (lr / 4)))];
          const int n = t.n0 + wn * 64 + i * 32 + 8 * q + lr;
          const int k = t.k0 + wk * 128 + 4 * l32;
          const uint32_t off = (n < p.N && k < p.K) ? (uint32_t)(((int64_t)n * p.K + k) * 4) : kWgOOB;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(wg_i32x4_t, v), dw_rsrc, off, 0, kWgStoreNT);
        }
      }
    }
    stored = true;
  }
  // drain the look-ahead loads (past the last tile they read zeros)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

int wgrad_block_m() { return kWgBM; }

hipError_t launch_wgrad(const WgradParams& p_in, hipStream_t stream) {
  WgradParams p = p_in;
  p.tiles_n = (p.N + kWgTN - 1) / kWgTN;
  p.tiles_k = (p.K + kWgTK - 1) / kWgTK;
  // division by top_k as a multiply-high: with l = ceil(log2 d) and
  // m = ceil(2^(31+l) / d), floor(s / d) = (s m) >> (31 + l) for every
  // s < 2^31 (Granlund and Montgomery, "Division by invariant integers using
  // multiplication", 1994, Theorem 4.2 with N = 31)
  int l = 0;
  while ((1 << l) < p.top_k) ++l;
  p.topk_magic = (uint32_t)((((uint64_t)1 << (31 + l)) + (uint64_t)p.top_k - 1) / (uint64_t)p.top_k);
  p.topk_shift = 31 + l;
  const int64_t tiles = (int64_t)p.E * p.tiles_n * p.tiles_k;
  if (tiles == 0) return hipSuccess;
  int dev = 0, cus = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  // a persistent grid: kWgPerCU workgroups per CU, a multiple of 8 (one
  // stretch of tiles per XCD per round)
  int64_t grid = (int64_t)cus * kWgPerCU;
  grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL(wgrad_kernel, dim3((uint32_t)grid), dim3(kWgThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace moe
