// moe_align: per-expert histogram, scan of the BLOCK_M-padded counts, and a
// stable scatter of slot ids into sorted_token_ids, with expert_ids per block
// and -1 sentinel blocks past the used ones.
//
// Follows ROCm/aiter PR #5310 "Add MoE GEMM variants and weight-gradient
// kernel" (Summary: sorted_token_ids / expert_ids of moe_align_block_size;
// second review: sentinel blocks hold -1) and torchada PR #115 ("Follow-up on
// this table": moe_align_block_size runs ahead of the fused MoE GEMM).
//
// G workgroups of 1024 threads (G = 1 up to 8K slots, then one per 8K
// slots, at most 16); no workspace and no cross-workgroup synchronisation.
// The slots are cut into 16 G contiguous runs, run r = 16 g + w owned by
// wave w of workgroup g. Every workgroup reads all ids: its waves count
// every run, into the per-expert totals, the counts of the runs before the
// workgroup's own, and each wave's count of its own run. A scan over
// experts of the padded totals then gives every wave its first position per
// expert (the expert's offset, the runs before this workgroup, the earlier
// waves of this workgroup), and each wave scatters its own run 64 slots at
// a time, ranking equal expert ids with ballots and advancing its own
// per-expert counters. The order within an expert is therefore ascending
// slot order (runs in slot order, batches in order, lanes in order): the
// result is unique and the same for any G. The scattered 4-byte stores of a
// run were what one workgroup spent most of its time on (one CU's memory
// pipeline), so they are spread over G CUs; the histogram is repeated in
// each workgroup instead of exchanged, which needs no scratch memory.
#include <algorithm>

#include "common.h"
#include "params.h"

namespace moe {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;
constexpr int kAlignMaxExperts = 1024;
constexpr int kAlignBatch = 8;  // 64-slot batches whose ids a wave loads together
constexpr int kAlignSlotsPerWg = 8192;  // slots per additional workgroup
constexpr int kAlignMaxWgs = 16;

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int32_t S, int32_t E, int32_t B,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_ids,
    int32_t* __restrict__ post_pad, int32_t max_blocks) {
  __shared__ int32_t tot[kAlignMaxExperts];   // per-expert slot counts (all runs)
  __shared__ int32_t bef[kAlignMaxExperts];   // ... of the runs before this workgroup's
  __shared__ int32_t off[kAlignMaxExperts];   // exclusive scan of padded counts
  // per wave and expert: the count of the wave's own run, then its next position
  __shared__ int32_t wave_pos[kAlignWaves][kAlignMaxExperts];
  __shared__ int32_t wave_sum[kAlignWaves];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int G = gridDim.x, g = blockIdx.x;
  // runs: one per 64 slots, at most 16 per workgroup, so small inputs leave
  // most waves (and their counters) idle
  const int runs = min(kAlignWaves * G, S / kWave + 1);
  const int run_len = S / runs + (S % runs != 0);
  const int own = g * kAlignWaves + wave;  // this wave's run
  // waves of this workgroup that own a run (only their counter rows are used)
  const int nw = max(0, min(kAlignWaves, runs - g * kAlignWaves));

  for (int i = tid; i < nw * kAlignMaxExperts; i += kAlignThreads)
    (&wave_pos[0][0])[i] = 0;
  for (int e = tid; e < E; e += kAlignThreads) {
    tot[e] = 0;
    bef[e] = 0;
  }
  __syncthreads();

  // 1. histograms: wave w counts runs w, w + 16, ... (all of them, across
  //    the workgroups' ranges)
  for (int r = wave; r < runs; r += kAlignWaves) {
    const int r0 = min(r * run_len, S), r1 = min(r0 + run_len, S);
    const bool mine = r == own, before = r < g * kAlignWaves;
    for (int base = r0; base < r1; base += kWave * kAlignBatch) {
      int ev[kAlignBatch];
#pragma unroll
      for (int i = 0; i < kAlignBatch; ++i) {
        const int s = base + i * kWave + lane;
        ev[i] = s < r1 ? ids[s] : -1;
      }
#pragma unroll
      for (int i = 0; i < kAlignBatch; ++i) {
        if (base + i * kWave >= r1) break;  // uniform across the wave
        const int e = ev[i];
        if (e >= 0 && e < E) {
          atomicAdd(&tot[e], 1);
          if (before) atomicAdd(&bef[e], 1);
          if (mine) atomicAdd(&wave_pos[wave][e], 1);
        }
      }
    }
  }
  __syncthreads();

  // 2. exclusive scan of p_e = ceil(c_e / B) * B over experts (E <= 1024:
  //    one value per thread; wave-level inclusive scan, then across waves),
  //    and each wave's first position per expert
  int c = 0;
  if (tid < E) c = tot[tid];
  const int p = ((c + B - 1) / B) * B;
  int incl = p;
  for (int d = 1; d < kWave; d <<= 1) {
    int v = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += v;
  }
  if (lane == kWave - 1) wave_sum[wave] = incl;
  __syncthreads();
  int before_sum = 0;
  for (int w = 0; w < wave; ++w) before_sum += wave_sum[w];
  int total = 0;
  for (int w = 0; w < kAlignWaves; ++w) total += wave_sum[w];
  const int o_e = before_sum + incl - p;
  if (tid < E) {
    off[tid] = o_e;
    int next = o_e + bef[tid];
    for (int w = 0; w < nw; ++w) {
      const int t = wave_pos[w][tid];
      wave_pos[w][tid] = next;
      next += t;
    }
  }
  if (g == 0 && tid == 0) *post_pad = total;
  __syncthreads();

  // 3. expert id per block: the largest e with off[e] <= b * B (that expert
  //    is never empty when b * B < total); -1 past the used blocks. Blocks
  //    are dealt to the workgroups in turn.
  for (int b = g * kAlignThreads + tid; b < max_blocks; b += G * kAlignThreads) {
    int pos = b * B;
    int e = -1;
    if (pos < total) {
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= pos) lo = mid; else hi = mid - 1;
      }
      e = lo;
    }
    expert_ids[b] = e;
  }
  // 4. PAD: the tail of each expert's segment (under 32 positions: one
  //    thread per expert; otherwise one wave per expert, lanes on
  //    consecutive positions) and everything past `total`; experts and
  //    positions are dealt to the workgroups in turn.
  const int32_t pad = S;
  if (B <= 32) {
    if (tid < E && tid % G == g)
      for (int q = o_e + c; q < o_e + p; ++q) sorted_ids[q] = pad;
  } else {
    for (int e = g * kAlignWaves + wave; e < E; e += G * kAlignWaves) {
      const int o = off[e], c_e = tot[e];
      const int end = o + ((c_e + B - 1) / B) * B;
      for (int q = o + c_e + lane; q < end; q += kWave) sorted_ids[q] = pad;
    }
  }
  const int64_t len = (int64_t)max_blocks * B;
  for (int64_t q = total + (int64_t)g * kAlignThreads + tid; q < len; q += (int64_t)G * kAlignThreads)
    sorted_ids[q] = pad;

  // 5. each wave scatters its own run in order, 64 slots at a time
  const int r0 = min(own * run_len, S), r1 = own < runs ? min(r0 + run_len, S) : r0;
  for (int base = r0; base < r1; base += kWave * kAlignBatch) {
    int ev[kAlignBatch];
#pragma unroll
    for (int i = 0; i < kAlignBatch; ++i) {
      const int s = base + i * kWave + lane;
      ev[i] = s < r1 ? ids[s] : -1;
    }
#pragma unroll
    for (int i = 0; i < kAlignBatch; ++i) {
      if (base + i * kWave >= r1) break;  // uniform across the wave
      const int s = base + i * kWave + lane;
      const int e = ev[i];
      const bool valid = e >= 0 && e < E;
      // lanes of this batch holding the same expert id
      uint64_t m = __ballot(valid);
#pragma unroll
      for (int bit = 0; bit < 10; ++bit) {
        const bool one = (e >> bit) & 1;
        const uint64_t bal = __ballot(one);
        m &= one ? bal : ~bal;
      }
      const int rank = __popcll(m & ((1ull << lane) - 1ull));
      int pos = 0;
      if (valid) pos = wave_pos[wave][e] + rank;
      // the lowest lane of each expert advances the wave's counter; its
      // write depends on its own read, and one wave's LDS operations run in
      // order, so every lane has read the position first
      if (valid && rank == 0) wave_pos[wave][e] = pos + __popcll(m);
      if (valid) sorted_ids[pos] = s;
    }
  }
}

// Expert block mapping of the group_sizes interface (ROCm/aiter PR #5310,
// Summary: moe_gemm_per_token takes a 1-D tensor of per-expert row counts;
// Notes: one block-mapping builder serves the GEMM wrappers; second review:
// block_expert_ids / block_token_offsets / block_token_ends with -1 sentinel
// blocks). Expert e owns rows [o_e, o_e + g_e), o_e the exclusive prefix sum
// of the counts; its ceil(g_e / B) blocks follow in expert order, block i
// starting at o_e + i * B, all ending at o_e + g_e. Negative counts count as
// zero, and segments are clipped to [0, rows), so no block ever names a row
// past the caller's buffers. One workgroup, one expert per thread: two
// 64-bit/32-bit scans, then a binary search per block.
__global__ __launch_bounds__(kAlignThreads) void block_map_kernel(
    const int32_t* __restrict__ group_sizes, int32_t E, int32_t B, int32_t rows,
    int32_t* __restrict__ expert_ids, int32_t* __restrict__ offsets, int32_t* __restrict__ ends,
    int32_t max_blocks, int32_t* __restrict__ total_out) {
  __shared__ int32_t seg_beg[kAlignMaxExperts];
  __shared__ int32_t seg_end[kAlignMaxExperts];
  __shared__ int32_t blk_beg[kAlignMaxExperts];
  __shared__ long long wave_rows[kAlignWaves];
  __shared__ int32_t wave_blks[kAlignWaves];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;

  // 1. row segments: exclusive scan of the counts in 64 bits
  const long long g = tid < E ? (long long)max(group_sizes[tid], 0) : 0ll;
  long long incl = g;
  for (int d = 1; d < kWave; d <<= 1) {
    const long long v = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += v;
  }
  if (lane == kWave - 1) wave_rows[wave] = incl;
  __syncthreads();
  long long before = 0, sum = 0;
  for (int w = 0; w < kAlignWaves; ++w) {
    if (w < wave) before += wave_rows[w];
    sum += wave_rows[w];
  }
  const long long o = before + incl - g;
  const int32_t beg = (int32_t)min(o, (long long)rows);
  const int32_t end = (int32_t)min(o + g, (long long)rows);
  const int32_t total = (int32_t)min(sum, (long long)rows);

  // 2. block counts and their exclusive scan
  const int32_t nb = (end - beg + B - 1) / B;
  int32_t bincl = nb;
  for (int d = 1; d < kWave; d <<= 1) {
    const int32_t v = __shfl_up(bincl, d, kWave);
    if (lane >= d) bincl += v;
  }
  if (lane == kWave - 1) wave_blks[wave] = bincl;
  __syncthreads();
  int32_t bbefore = 0, nblocks = 0;
  for (int w = 0; w < kAlignWaves; ++w) {
    if (w < wave) bbefore += wave_blks[w];
    nblocks += wave_blks[w];
  }
  if (tid < E) {
    seg_beg[tid] = beg;
    seg_end[tid] = end;
    blk_beg[tid] = bbefore + bincl - nb;
  }
  if (tid == 0 && total_out != nullptr) *total_out = (int32_t)min(sum, (long long)INT32_MAX);
  __syncthreads();

  // 3. per block: the largest e with blk_beg[e] <= b owns it (and is not
  //    empty while b < nblocks); sentinels past the used blocks
  for (int b = tid; b < max_blocks; b += kAlignThreads) {
    int32_t e = -1, off = total, en = total;
    if (b < nblocks) {
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (blk_beg[mid] <= b) lo = mid; else hi = mid - 1;
      }
      e = lo;
      off = seg_beg[e] + (b - blk_beg[e]) * B;
      en = seg_end[e];
    }
    expert_ids[b] = e;
    offsets[b] = off;
    ends[b] = en;
  }
}

hipError_t launch_block_map(const int32_t* group_sizes, int32_t E, int32_t B, int32_t rows, int32_t* expert_ids,
                            int32_t* offsets, int32_t* ends, int32_t max_blocks, int32_t* total_out,
                            hipStream_t stream) {
  hipLaunchKernelGGL(block_map_kernel, dim3(1), dim3(kAlignThreads), 0, stream, group_sizes, E, B, rows,
                     expert_ids, offsets, ends, max_blocks, total_out);
  return hipGetLastError();
}

hipError_t launch_align(const int32_t* ids, int32_t S, int32_t E, int32_t B,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* post_pad,
                        int32_t max_blocks, hipStream_t stream) {
  const int G = std::max(1, std::min(kAlignMaxWgs, S / kAlignSlotsPerWg));
  hipLaunchKernelGGL(align_kernel, dim3((uint32_t)G), dim3(kAlignThreads), 0, stream,
                     ids, S, E, B, sorted_ids, expert_ids, post_pad, max_blocks);
  return hipGetLastError();
}

}  // namespace moe
