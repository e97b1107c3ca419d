// The decode MoE step in one launch: routing, the grouped GEMM and the top-k
// combine for at most 32 tokens, with the same bits as moe_align ->
// moe_grouped_gemm (decode variant) -> moe_combine.
//
// Follows torchada PR #115 "tune the Nemotron MTP decode row on S5000 with a
// checked-in recipe": What it does (the M <= 32 decode bucket dominates the
// decode step, whose launches around the GEMM are fixed costs at every call)
// and "Follow-up on this table" (moe_align_block_size, the fused MoE GEMM);
// the combine is the method's last step (top-k weights applied to the expert
// outputs).
//
// Design for gfx950:
//  * Token-major: a workgroup of 8 waves owns 8 output columns (one weight
//    row per wave) for every touched expert, so each token's top-k outputs
//    of those columns end in one workgroup and the combine needs no
//    cross-workgroup step and no scratch memory. Each wave streams its row of
//    every touched expert in ascending expert order with non-temporal loads,
//    two experts ahead; every expert's weights are read once.
//  * Every weight, scale and bias load is a buffer load whose out-of-range
//    pieces read as zero, so none sits under a branch: the compiler can then
//    wait for exactly the oldest row of the prefetch ring (memory counters
//    retire in order) instead of for all loads in flight. The activation
//    loads stop at the last piece the token rows hold (a workgroup-uniform
//    bound); the first wait on the ids then covers them too, which costs
//    nothing, as the first weight rows wait for the routing anyway.
//  * The routing is done by every workgroup from the at most 256 ids. Up to
//    8 slots (one token's top-k), every wave does it on its own in registers
//    (lane s holds slot s: its rank among the routed slots by (expert,
//    slot), its expert's slot count and its place in the touched list, each
//    counted over the other lanes; the tables are then read with ballots),
//    so no barrier stands between the ids and the first weight rows; the
//    count loops take a few hundred cycles per slot, so beyond that it is
//    done in LDS: per-expert counts (LDS atomics), one scan giving each
//    touched expert its slot range and its place in the touched list, a
//    scatter of the slots. The order of slots inside an expert does not
//    matter: each output is computed on its own. The activation rows of all tokens are loaded while
//    the routing runs and written to LDS (M x K bf16, at most 149 KB) once
//    the first weight rows are on their way; when they do not fit (M x K >
//    76288, e.g. 32 tokens of 2688) they are staged in two passes over the
//    halves of K, the weight rows are streamed in the same halves, and each
//    output is the sum of its passes' wave sums.
//  * Each output C[s, n] is computed with exactly the arithmetic of the decode
//    kernel: lane l accumulates K pieces k = 8 (l + 64 i) in ascending i with
//    v_dot2_f32_bf16 (pieces past K as zeros, so the instruction count per
//    lane matches that kernel's 2048-element passes), then the sum across
//    the wave with the butterfly's pairing, bias, epilogue, one bf16
//    rounding. The combine sums w[t, j] * C[t k + j] over j ascending in
//    fp32 from the bf16 values, as moe_combine does. The results are
//    therefore bit-identical to the three launches (with passes, the sum is
//    grouped by pass, so the last bit may differ); a slot whose expert id
//    lies outside [0, E) contributes 0.
#include <type_traits>

#include "common.h"
#include "decode_layer.h"

namespace moe {

constexpr int kDlWaves = 8;                      // weight rows (output columns) per workgroup
constexpr int kDlThreads = kDlWaves * kWave;
constexpr int kDlMaxE = 1024;
constexpr int kDlMaxS = 256;                     // slots (tokens x top_k)
constexpr int kDlRegSlots = 8;                   // routed in registers up to this many slots
// M x K activation elements in LDS (149 KB: 28 tokens of 2688 fit); with
// the other arrays the workgroup uses all but ~1 KB of the CU's 160 KB
constexpr int kDlMaxXElems = 76288;
constexpr int kDlXLoads = (kDlMaxXElems / 8 + kDlThreads - 1) / kDlThreads;  // 16-byte pieces per thread
constexpr int kDlPass = 2048;                    // the decode kernel's K elements per pass
constexpr int kDlPassPieces = kDlPass / 8 / kWave;  // 8-element pieces per lane per pass
constexpr int kDlMaxPieces = 2 * kDlPassPieces;  // K <= 4096
constexpr uint32_t kDlOOB = 0x80000000u;         // an offset past every range: reads as zero
constexpr int kDlNT = 2;                         // buffer-load cache policy: non-temporal
constexpr int kDlRsrcWord3 = 0x00020000;         // raw 32-bit buffer

__device__ __forceinline__ float dl_bits_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t dl_f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// Sum over the wave with the pairing of v += shfl_xor(v, d) for d = 32, 16,
// 8, 4, 2, 1: each step adds every lane's value to that of the lane whose
// index differs in bit log2(d). fp32 addition is commutative, so every lane
// ends with the bits of that butterfly. The swaps exchange half-waves and
// 16-lane rows; the 8-step rotates a 16-lane row by 8 (exactly the xor);
// after it a lane's value depends only on its index mod 8, so rotating by 4
// reads a lane holding the xor-4 partner's value; the last two steps permute
// within quads.
__device__ __forceinline__ float dl_wave_sum(float v) {
  const auto h = __builtin_amdgcn_permlane32_swap(dl_f32_bits(v), dl_f32_bits(v), false, false);
  v = dl_bits_f32(h[0]) + dl_bits_f32(h[1]);
  const auto r = __builtin_amdgcn_permlane16_swap(dl_f32_bits(v), dl_f32_bits(v), false, false);
  v = dl_bits_f32(r[0]) + dl_bits_f32(r[1]);
  v = v + dl_bits_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)dl_f32_bits(v), 0x128, 0xF, 0xF, false));
  v = v + dl_bits_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)dl_f32_bits(v), 0x124, 0xF, 0xF, false));
  v = v + dl_bits_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)dl_f32_bits(v), 0x4E, 0xF, 0xF, false));
  v = v + dl_bits_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)dl_f32_bits(v), 0xB1, 0xF, 0xF, false));
  return v;
}

// f(integral_constant<int, R>) for R = R0 .. PF - 1, in order (the ring
// slots are compile-time indices, so the rows stay in registers)
template <int R0, int PF, class F>
__device__ __forceinline__ void dl_for_slots(F&& f) {
  if constexpr (R0 < PF) {
    f(std::integral_constant<int, R0>{});
    dl_for_slots<R0 + 1, PF>(f);
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dl_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kDlRsrcWord3);
}

// NP: 8-element pieces per lane per weight row and pass (4 for K <= 2048,
// else 8 in one pass, or 4 in each of two passes when SPLIT).
// PF: rows in flight per wave (the ring's depth).
// SPLIT: the activations of all tokens do not fit in LDS at once (M x K >
// kDlMaxXElems): K is taken in two halves of KH = K/2 rounded up to 32 elements
// (KH <= 2048), the activations are staged and the weight rows streamed one
// half at a time, and each output's sum is formed per half (wave sum of
// each half, the halves added in order), so the bits may differ from the
// three launches' in the last place.
// RR: at most kDlRegSlots slots, routed in registers by every wave (no LDS
// tables).
template <int WDT, bool BIAS, int NP, int PF, bool SPLIT, bool RR>
__global__ __launch_bounds__(kDlThreads, 1) void moe_decode_layer_kernel(DecodeLayerParams p) {
  // token rows, K elements each. Its last 4 KB hold the per-expert counts
  // (then the scatter cursors) during the routing, before any row is
  // written.
  // (SPLIT: 32 tokens of at most kDlPass elements per pass, and room for
  // the per-pass sums below)
  constexpr int kXElems = SPLIT ? 32 * kDlPass : kDlMaxXElems;
  __shared__ __attribute__((aligned(16))) uint32_t lds_x[kXElems / 2];
  uint16_t* const xs = reinterpret_cast<uint16_t*>(lds_x);
  int32_t* const s_cnt = reinterpret_cast<int32_t*>(&lds_x[kXElems / 2 - kDlMaxE]);
  __shared__ int32_t s_tl[kDlMaxS];     // touched experts, ascending
  __shared__ int32_t s_toff[kDlMaxS];   // first position of each touched expert's slots
  __shared__ int32_t s_tcnt[kDlMaxS];   // its slot count
  __shared__ int32_t s_slot[kDlMaxS];   // slots grouped by expert
  __shared__ int32_t s_xoff[kDlMaxS];   // xs offset of each grouped slot's token row
  __shared__ int32_t s_id[kDlMaxS];     // routed expert of each slot (-1: none)
  __shared__ uint16_t s_c[kDlMaxS][kDlWaves];  // bf16 C of each slot, per column of the workgroup
  __shared__ float s_acc[SPLIT ? kDlMaxS : 1][kDlWaves];  // (SPLIT) the sums of the earlier passes
  __shared__ int32_t s_part[2][kDlWaves];
  __shared__ int32_t s_ntouched;

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int S = p.S, E = p.E, K = p.K, top_k = p.top_k;
  const int M = S / top_k;

  // ---- 1. the routing ids, then every token's activations (of the first
  //      pass) into registers. xs holds row t at t * XK: K elements, or a
  //      pass of kDlPass when SPLIT (zeros past K).
  // (RR: every wave reads all ids, lane s slot s; else thread s slot s)
  const uint32_t id_raw = __builtin_amdgcn_raw_buffer_load_b32(dl_rsrc(p.topk_ids, (uint32_t)S * 4u),
                                                               (uint32_t)(RR ? lane : tid) * 4u, 0, 0);
  const int XK = SPLIT ? ((K / 2 + 31) / 32) * 32 : K;  // K elements per pass (and xs row stride)
  const int k8 = XK / 8;
  const int npass = SPLIT ? 2 : 1;
  const __amdgpu_buffer_rsrc_t x_rsrc = dl_rsrc(p.x, p.x_bytes);
  // pieces per thread that hold activations (the rest would read zeros)
  const int xl = (M * k8 + kDlThreads - 1) / kDlThreads;
  u32x4_t xr[kDlXLoads];
  // f(i, t, c) for this thread's pieces i: 16 bytes at row t, element 8 c
  // (piece tid + kDlThreads * i; t and c stepped, not divided, per piece)
  auto x_pieces = [&](auto&& f) {
    const int dt = kDlThreads / k8, dc = kDlThreads % k8;
    int t = tid / k8, c = tid % k8;
#pragma unroll
    for (int i = 0; i < kDlXLoads; ++i) {
      f(i, t, c);
      t += dt;
      c += dc;
      if (c >= k8) {
        c -= k8;
        ++t;
      }
    }
  };
  auto x_load = [&](int kbase) {
    x_pieces([&](int i, int t, int c) {
      if (i >= xl) return;
      const uint32_t off = (t < M && kbase + c * 8 < K) ? (uint32_t)(((int64_t)t * p.x_ld + kbase + c * 8) * 2)
                                                        : kDlOOB;
      xr[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, off, 0, 0));
    });
  };
  auto x_store = [&]() {
    x_pieces([&](int i, int t, int c) {
      if (i < xl && t < M) *reinterpret_cast<u32x4_t*>(&xs[t * XK + c * 8]) = xr[i];
    });
  };
  x_load(0);

  // ---- 2. routing
  // RR: lane s (s < S) holds slot s: its expert (-1: not routed), its
  // position among the routed slots ordered by (expert, slot), its expert's
  // slot count, whether it is that expert's first slot, and then the
  // expert's place among the touched experts (ascending)
  int rr_e = -1, rr_pos = 0, rr_cnt = 0, rr_ti = 0, rr_xoff = 0;
  bool rr_first = false;
  int nt;
  if constexpr (RR) {
    if (lane < S) {
      const int id = (int)id_raw;
      rr_e = (id >= 0 && id < E) ? id : -1;
    }
    int before = 0;
    for (int j = 0; j < S; ++j) {
      const int ej = __builtin_amdgcn_readlane(rr_e, j);
      const bool same = ej == rr_e;
      rr_pos += (ej >= 0 && (ej < rr_e || (same && j < lane))) ? 1 : 0;
      rr_cnt += same ? 1 : 0;
      before += (same && j < lane) ? 1 : 0;
    }
    rr_first = rr_e >= 0 && before == 0;
    const uint64_t firsts = __builtin_amdgcn_ballot_w64(rr_first);
    for (uint64_t m = firsts; m != 0; m &= m - 1)
      rr_ti += (__builtin_amdgcn_readlane(rr_e, (int)__builtin_ctzll(m)) < rr_e) ? 1 : 0;
    nt = __builtin_popcountll(firsts);
    rr_xoff = (lane / top_k) * XK;
    if (wave == 0 && lane < S) s_id[lane] = rr_e;  // for the combine (barriers follow)
  } else {
    // counts, scan, scatter
    for (int e = tid; e < E; e += kDlThreads) s_cnt[e] = 0;
    __syncthreads();
    if (tid < S) {
      const int id = (int)id_raw;
      const int r = (id >= 0 && id < E) ? id : -1;  // ids outside [0, E) are not routed
      s_id[tid] = r;
      if (r >= 0) atomicAdd(&s_cnt[r], 1);
    }
    __syncthreads();
    // experts 2 tid, 2 tid + 1: exclusive scans of the slot counts and of the
    // touched flags over all experts (E <= 1024 = 2 x 512)
    int c0 = 0, c1 = 0;
    if (2 * tid < E) c0 = s_cnt[2 * tid];
    if (2 * tid + 1 < E) c1 = s_cnt[2 * tid + 1];
    const int csum = c0 + c1, tsum = (c0 > 0) + (c1 > 0);
    int ci = csum, ti = tsum;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int a = __shfl_up(ci, d, kWave), b = __shfl_up(ti, d, kWave);
      if (lane >= d) {
        ci += a;
        ti += b;
      }
    }
    if (lane == kWave - 1) {
      s_part[0][wave] = ci;
      s_part[1][wave] = ti;
    }
    __syncthreads();
    int cbase = 0, tbase = 0, ttot = 0;
    for (int w = 0; w < kDlWaves; ++w) {
      if (w < wave) {
        cbase += s_part[0][w];
        tbase += s_part[1][w];
      }
      ttot += s_part[1][w];
    }
    int co = cbase + ci - csum, to = tbase + ti - tsum;
    if (c0 > 0) {
      s_tl[to] = 2 * tid;
      s_toff[to] = co;
      s_tcnt[to] = c0;
      ++to;
    }
    if (2 * tid < E) s_cnt[2 * tid] = co;  // the cursor of the scatter
    co += c0;
    if (c1 > 0) {
      s_tl[to] = 2 * tid + 1;
      s_toff[to] = co;
      s_tcnt[to] = c1;
    }
    if (2 * tid + 1 < E) s_cnt[2 * tid + 1] = co;
    if (tid == 0) s_ntouched = ttot;
    __syncthreads();
    if (tid < S && s_id[tid] >= 0) {
      const int pos = atomicAdd(&s_cnt[s_id[tid]], 1);
      s_slot[pos] = tid;
      s_xoff[pos] = (tid / top_k) * XK;
    }
    __syncthreads();
    nt = __builtin_amdgcn_readfirstlane(s_ntouched);
  }
  // touched expert idx < nt: its id, its slots' first position, their count
  auto touched = [&](int idx, int& e, int& o, int& c) {
    if constexpr (RR) {
      const uint64_t m = __builtin_amdgcn_ballot_w64(rr_first && rr_ti == idx);
      const int l = m != 0 ? (int)__builtin_ctzll(m) : 0;
      e = __builtin_amdgcn_readlane(rr_e, l);
      o = __builtin_amdgcn_readlane(rr_pos, l);
      c = __builtin_amdgcn_readlane(rr_cnt, l);
    } else {
      e = __builtin_amdgcn_readfirstlane(s_tl[idx]);
      o = __builtin_amdgcn_readfirstlane(s_toff[idx]);
      c = __builtin_amdgcn_readfirstlane(s_tcnt[idx]);
    }
  };
  // the slot at grouped position q and the xs offset of its token's row
  auto slot_at = [&](int q, int& sl, int& xo) {
    if constexpr (RR) {
      const uint64_t m = __builtin_amdgcn_ballot_w64(rr_e >= 0 && rr_pos == q);
      sl = m != 0 ? (int)__builtin_ctzll(m) : 0;
      xo = __builtin_amdgcn_readlane(rr_xoff, sl);
    } else {
      sl = __builtin_amdgcn_readfirstlane(s_slot[q]);
      xo = __builtin_amdgcn_readfirstlane(s_xoff[q]);
    }
  };

  // ---- 3. this wave's weight row of every touched expert, through a ring
  const int n = blockIdx.x * kDlWaves + wave;
  const bool row_live = n < p.N;
  constexpr int kWords = (WDT == W_BF16) ? 4 : (WDT == W_E4M3 ? 2 : 1);
  uint32_t wraw[PF][NP][kWords];
  uint32_t sraw[PF][NP];
  uint32_t braw[PF];
  const __amdgpu_buffer_rsrc_t b_rsrc = dl_rsrc(p.bias, BIAS ? p.bias_bytes : 0u);
  auto load_row = [&](int idx, auto slot_tag, int kbase) {
    constexpr int R = decltype(slot_tag)::value;
    const int kend = kbase + XK < K ? kbase + XK : K;
    const bool live = row_live && idx < nt;
    int e = 0, o_unused, c_unused;
    if (live) touched(idx, e, o_unused, c_unused);
    const int nn = live ? n : 0;
    const __amdgpu_buffer_rsrc_t w_rsrc =
        dl_rsrc(p.w + (int64_t)e * p.w_stride_e + (int64_t)nn * p.w_row, live ? p.w_rspan : 0u);
    const __amdgpu_buffer_rsrc_t s_rsrc =
        dl_rsrc(WDT != W_BF16 ? p.ws + (int64_t)e * p.ws_stride_e + (int64_t)nn * p.ws_row : p.ws,
                (WDT != W_BF16 && live) ? p.ws_rspan : 0u);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int k = kbase + 8 * (lane + kWave * i);
      const bool kin = k < kend;
      const uint32_t kb = (uint32_t)(k / 64);
      if constexpr (WDT == W_BF16) {
        const uint32_t off = kin ? kb * (uint32_t)p.w_blk + (uint32_t)(k % 64) * 2u : kDlOOB;
        const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, off, 0, kDlNT));
#pragma unroll
        for (int q = 0; q < 4; ++q) wraw[R][i][q] = v[q];
      } else if constexpr (WDT == W_E4M3) {
        const uint32_t off = kin ? kb * (uint32_t)p.w_blk + (uint32_t)(k % 64) : kDlOOB;
        const u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(w_rsrc, off, 0, kDlNT));
        wraw[R][i][0] = v[0];
        wraw[R][i][1] = v[1];
      } else {
        const uint32_t off = kin ? kb * (uint32_t)p.w_blk + (uint32_t)(k % 64) / 2u : kDlOOB;
        wraw[R][i][0] = __builtin_amdgcn_raw_buffer_load_b32(w_rsrc, off, 0, kDlNT);
      }
      if constexpr (WDT != W_BF16) {
        const uint32_t soff = kin ? kb * (uint32_t)p.ws_blk + (uint32_t)(k % 64) / 32u : kDlOOB;
        sraw[R][i] = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, soff, 0, kDlNT);
      }
    }
    if constexpr (BIAS) {
      const uint32_t boff = live ? (uint32_t)(((int64_t)e * p.bias_se + (int64_t)n * p.bias_sn) * 2) : kDlOOB;
      braw[R] = __builtin_amdgcn_raw_buffer_load_b16(b_rsrc, boff, 0, 0);
    }
  };
  auto compute_row = [&](int idx, auto slot_tag, int kbase, int pass) {
    constexpr int R = decltype(slot_tag)::value;
    if (idx >= nt) return;
    const int kend = kbase + XK < K ? kbase + XK : K;
    // this lane's dequantised pieces of the row (zeros past K)
    bf16x8_t wv[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if constexpr (WDT == W_BF16) {
        __builtin_memcpy(&wv[i], wraw[R][i], 16);
      } else if constexpr (WDT == W_E4M3) {
        wv[i] = dequant_e4m3x8(wraw[R][i][0], wraw[R][i][1], e8m0_as_scale(sraw[R][i]));
      } else {
        wv[i] = dequant_e2m1x8(wraw[R][i][0], e8m0_as_scale(sraw[R][i]));
      }
    }
    const float bv = BIAS ? bf16_bits_to_f32(braw[R] & 0xffffu) : 0.0f;
    int e_unused, o, cnt;
    touched(idx, e_unused, o, cnt);
    // two slots at a time: two independent accumulation chains
    for (int j = 0; j < cnt; j += 2) {
      const bool two = j + 1 < cnt;
      const int jb = two ? j + 1 : j;
      int sa, sb, xa, xb;
      slot_at(o + j, sa, xa);
      slot_at(o + jb, sb, xb);
      float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int k = kbase + 8 * (lane + kWave * i);
        const bool kin = k < kend;
        const int kk = kin ? k - kbase : 0;
        bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(&xs[xa + kk]);
        bf16x8_t vb = *reinterpret_cast<const bf16x8_t*>(&xs[xb + kk]);
        const bf16x8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
        va = kin ? va : z;
        vb = kin ? vb : z;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf16x2_t x2a, x2b, w2;
          __builtin_memcpy(&x2a, reinterpret_cast<const char*>(&va) + 4 * q, 4);
          __builtin_memcpy(&x2b, reinterpret_cast<const char*>(&vb) + 4 * q, 4);
          __builtin_memcpy(&w2, reinterpret_cast<const char*>(&wv[i]) + 4 * q, 4);
          a0 = __builtin_amdgcn_fdot2_f32_bf16(x2a, w2, a0, false);
          a1 = __builtin_amdgcn_fdot2_f32_bf16(x2b, w2, a1, false);
        }
      }
      a0 = dl_wave_sum(a0);
      a1 = dl_wave_sum(a1);
      if constexpr (SPLIT) {
        if (pass > 0) {
          a0 = s_acc[sa][wave] + a0;
          a1 = s_acc[sb][wave] + a1;
        }
        if (pass + 1 < npass) {
          if (lane == 0) {
            s_acc[sa][wave] = a0;
            if (two) s_acc[sb][wave] = a1;
          }
          continue;
        }
      }
      a0 += bv;
      a1 += bv;
      const uint16_t ca = (uint16_t)f32_to_bf16_bits(p.relu2 ? relu2_f32(a0) : a0);
      const uint16_t cb = (uint16_t)f32_to_bf16_bits(p.relu2 ? relu2_f32(a1) : a1);
      if (lane == 0) {
        s_c[sa][wave] = ca;
        if (two) s_c[sb][wave] = cb;
      }
    }
  };
  for (int pass = 0; pass < npass; ++pass) {
    const int kbase = pass * XK;
    if (pass > 0) {
      __syncthreads();  // every wave is done with the previous pass's activations
      x_load(kbase);
    }
    dl_for_slots<0, PF>([&](auto r) { load_row(decltype(r)::value, r, kbase); });
    // the activations into LDS (their loads were issued before the rows')
    x_store();
    __syncthreads();
    // row idx lives in ring slot idx % PF; its slot is refilled with row
    // idx + PF as soon as it has been used
    for (int idx = 0; idx < nt; idx += PF) {
      dl_for_slots<0, PF>([&](auto r) {
        constexpr int R = decltype(r)::value;
        compute_row(idx + R, r, kbase, pass);
        load_row(idx + R + PF, r, kbase);
      });
    }
  }
  __syncthreads();

  // ---- 4. the expert outputs (when asked for) and the combine
  const int n0 = blockIdx.x * kDlWaves;
  if (p.c != nullptr) {
    for (int q = tid; q < S * kDlWaves; q += kDlThreads) {
      const int s = q / kDlWaves, r = q % kDlWaves;
      if (s_id[s] >= 0 && n0 + r < p.N) p.c[(int64_t)s * p.c_ld + n0 + r] = s_c[s][r];
    }
  }
  // y[t, n] = sum_j w[t, j] * C[t k + j, n], j ascending
  for (int q = tid; q < M * kDlWaves; q += kDlThreads) {
    const int t = q / kDlWaves, r = q % kDlWaves;
    if (n0 + r >= p.N) continue;
    float acc = 0.0f;
    for (int j = 0; j < top_k; ++j) {
      const int s = t * top_k + j;
      const float cv = s_id[s] >= 0 ? bf16_bits_to_f32(s_c[s][r]) : 0.0f;
      acc += p.topk_w[s] * cv;
    }
    p.y[(int64_t)t * p.y_ld + n0 + r] = (uint16_t)f32_to_bf16_bits(acc);
  }
}

int decode_layer_max_slots() { return kDlMaxS; }
int decode_layer_max_experts() { return kDlMaxE; }
int decode_layer_max_k() { return kDlMaxPieces / kDlPassPieces * kDlPass; }

template <int WDT, int NP, bool SPLIT, bool RR>
static void launch_dl(const DecodeLayerParams& p, bool bias, dim3 grid, hipStream_t stream) {
  // Two rows in flight per wave (8 KB per wave at K = 2048, 64 KB per CU):
  // on a cold cache, depths 1, 2, 3, 4, 6 and 8 gave about 134, 121, 124, 123, 123
  // and 124 us at M = 28 (K = 2048) and 172, 152, 154, 160 us at M = 24,
  // K = 2688 (depths 1-4); deeper rings only lengthen the memory queues.
  // With two passes each row is half as long, so twice as many rows are
  // kept in flight.
  constexpr int PF = SPLIT ? 4 : 2;
  if (bias)
    hipLaunchKernelGGL((moe_decode_layer_kernel<WDT, true, NP, PF, SPLIT, RR>), grid, dim3(kDlThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((moe_decode_layer_kernel<WDT, false, NP, PF, SPLIT, RR>), grid, dim3(kDlThreads), 0, stream, p);
}

template <int WDT>
static void launch_dl_wdt(const DecodeLayerParams& p, bool bias, dim3 grid, hipStream_t stream) {
  const int64_t act = (int64_t)(p.S / p.top_k) * p.K;  // activation elements of all tokens
  const bool rr = p.S <= kDlRegSlots;  // routed in registers
  if (p.K <= kDlPass) {
    if (rr) launch_dl<WDT, kDlPassPieces, false, true>(p, bias, grid, stream);
    else launch_dl<WDT, kDlPassPieces, false, false>(p, bias, grid, stream);
  } else if (act <= kDlMaxXElems) {
    if (rr) launch_dl<WDT, kDlMaxPieces, false, true>(p, bias, grid, stream);
    else launch_dl<WDT, kDlMaxPieces, false, false>(p, bias, grid, stream);
  } else {
    launch_dl<WDT, kDlPassPieces, true, false>(p, bias, grid, stream);
  }
}

hipError_t launch_decode_layer(const DecodeLayerParams& p, int wdt, bool bias, hipStream_t stream) {
  const dim3 grid((uint32_t)((p.N + kDlWaves - 1) / kDlWaves));
  if (wdt == W_E2M1) launch_dl_wdt<W_E2M1>(p, bias, grid, stream);
  else if (wdt == W_E4M3) launch_dl_wdt<W_E4M3>(p, bias, grid, stream);
  else launch_dl_wdt<W_BF16>(p, bias, grid, stream);
  return hipGetLastError();
}

}  // namespace moe
