// Staging kernels for bf16 (16-bit, unquantized) base weights. The layer is
// the same as with NF4 weights; only the dequantization step becomes a copy
// (gate/up interleave for the MLP) or a transpose (backward dX GEMMs). Both
// kernels are HBM-bound: 2 B in, 2 B out per weight.
#include "common.hpp"
#include "kernels.hpp"

namespace qlora {

__device__ __forceinline__ int64_t w16_dest_row(int64_t n, int interleave) {
  if (interleave == 0) return n;
  return 64 * (n >> 5) + 32 * (interleave - 1) + (n & 31);
}

// out[dest_row(i)][j] = W[i][j]; one thread per 8 weights (16 B in, 16 B out),
// 2D grid: blockIdx.y = row block of 1, blockIdx.x * 256 + tid = 16-byte chunk.
__global__ __launch_bounds__(256) void w16_rows_kernel(const uint16_t* __restrict__ src, int64_t n,
                                                       int64_t k, uint16_t* __restrict__ out,
                                                       int64_t ld_out, int interleave) {
  const int64_t row = blockIdx.y;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 8-element chunk
  if (row >= n || c >= (k >> 3)) return;
  const u32x4_t v = *(const u32x4_t*)(src + row * k + c * 8);
  *(u32x4_t*)(out + w16_dest_row(row, interleave) * ld_out + c * 8) = v;
}

// out[kk][col_ofs + nn] = W[nn][kk] for a 64 x 64 block through LDS; thread t
// reads 16 B of a source row and writes 16 B of an output row.
__global__ __launch_bounds__(256) void w16_transpose_kernel(const uint16_t* __restrict__ src,
                                                            int64_t n, int64_t k,
                                                            uint16_t* __restrict__ out,
                                                            int64_t ld_out, int64_t col_ofs) {
  __shared__ uint16_t tile[64][64 + 2];
  const int tid = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.y * 64, k0 = (int64_t)blockIdx.x * 64;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int r = p * 32 + (tid >> 3), c = (tid & 7) * 8;   // source row r, columns c..c+7
    const u32x4_t v = *(const u32x4_t*)(src + (n0 + r) * k + k0 + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[r][c + 2 * e] = (uint16_t)(v[e] & 0xFFFFu);
      tile[r][c + 2 * e + 1] = (uint16_t)(v[e] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int kk = p * 32 + (tid >> 3), c = (tid & 7) * 8;  // output row kk, weight rows c..c+7
    u32x4_t v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = (uint32_t)tile[c + 2 * e][kk] | ((uint32_t)tile[c + 2 * e + 1][kk] << 16);
    *(u32x4_t*)(out + (k0 + kk) * ld_out + col_ofs + n0 + c) = v;
  }
}

hipError_t launch_w16_rows(const uint16_t* src, int64_t n, int64_t k, uint16_t* out, int64_t ld_out,
                           int interleave, hipStream_t stream) {
  if (n == 0 || k == 0) return hipSuccess;
  const dim3 grid((unsigned)(((k >> 3) + 255) / 256), (unsigned)n);
  w16_rows_kernel<<<grid, dim3(256), 0, stream>>>(src, n, k, out, ld_out, interleave);
  return hipGetLastError();
}

hipError_t launch_w16_transpose(const uint16_t* src, int64_t n, int64_t k, uint16_t* out,
                                int64_t ld_out, int64_t col_ofs, hipStream_t stream) {
  if (n == 0 || k == 0) return hipSuccess;
  const dim3 grid((unsigned)(k / 64), (unsigned)(n / 64));
  w16_transpose_kernel<<<grid, dim3(256), 0, stream>>>(src, n, k, out, ld_out, col_ofs);
  return hipGetLastError();
}

}  // namespace qlora
