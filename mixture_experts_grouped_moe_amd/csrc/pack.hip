// Weight repacking from the rows layout into the K-block layout (64-element K
// blocks outermost, every row's piece of a block back to back). A one-time
// copy at weight-load time: codes and scale bytes move, nothing is computed.
#include "common.h"
#include "params.h"

namespace moe {

constexpr int kThreadsPack = 256;

// One thread per 16-byte unit of the output. Output unit index
// ((e * nblk + kb) * N + n) * upr + u, upr = row_bytes / 16 units per row piece.
// The thread with u == 0 also moves the piece's two scale bytes.
__global__ __launch_bounds__(kThreadsPack) void moe_pack_kernel(const uint8_t* __restrict__ w, int64_t w_stride_e,
                                                                 int64_t w_ld, const uint8_t* __restrict__ ws,
                                                                 int64_t ws_stride_e, int64_t ws_ld, int32_t N,
                                                                 int32_t K, int32_t nblk, int32_t row_bytes,
                                                                 int32_t code_row_bytes, int64_t total,
                                                                 uint8_t* __restrict__ w_out, uint8_t* __restrict__ ws_out) {
  const int upr = row_bytes / 16;
  for (int64_t q = (int64_t)blockIdx.x * kThreadsPack + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * kThreadsPack) {
    const int u = (int)(q % upr);
    int64_t r = q / upr;
    const int n = (int)(r % N);
    r /= N;
    const int kb = (int)(r % nblk);
    const int64_t e = r / nblk;
    const int64_t src_byte = (int64_t)kb * row_bytes + u * 16;  // byte within the source row
    u32x4_t v = {0, 0, 0, 0};
    if (src_byte < code_row_bytes)  // the upper half of a last, half-filled block stays zero
      v = *reinterpret_cast<const u32x4_t*>(w + e * w_stride_e + (int64_t)n * w_ld + src_byte);
    *reinterpret_cast<u32x4_t*>(w_out + q * 16) = v;
    if (ws != nullptr && u == 0) {
      const uint8_t* srow = ws + e * ws_stride_e + (int64_t)n * ws_ld;
      uint8_t* drow = ws_out + (e * nblk + kb) * 2 * (int64_t)N + 2 * (int64_t)n;
      drow[0] = srow[2 * kb];
      drow[1] = 2 * kb + 1 < K / 32 ? srow[2 * kb + 1] : (uint8_t)0;
    }
  }
}

hipError_t launch_pack(const uint8_t* w, int64_t w_stride_e, int64_t w_ld, const uint8_t* ws, int64_t ws_stride_e,
                       int64_t ws_ld, int32_t E, int32_t N, int32_t K, int32_t row_bytes, uint8_t* w_out,
                       uint8_t* ws_out, hipStream_t stream) {
  const int32_t nblk = (K + 63) / 64;
  const int64_t total = (int64_t)E * nblk * N * (row_bytes / 16);
  if (total == 0) return hipSuccess;
  const int32_t code_row_bytes = (int32_t)((int64_t)K * row_bytes / 64);
  const int64_t want = (total + kThreadsPack - 1) / kThreadsPack;
  const uint32_t grid = (uint32_t)(want < 65536 * 16 ? want : 65536 * 16);
  hipLaunchKernelGGL(moe_pack_kernel, dim3(grid), dim3(kThreadsPack), 0, stream, w, w_stride_e, w_ld, ws,
                     ws_stride_e, ws_ld, N, K, nblk, row_bytes, code_row_bytes, total, w_out, ws_out);
  return hipGetLastError();
}

}  // namespace moe
