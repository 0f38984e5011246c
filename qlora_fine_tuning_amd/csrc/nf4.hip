// NF4 (4-bit NormalFloat) dequantization kernels for gfx950.
//
// Format (the pages only say "QLoRA nf4" for every projection - Mistral
// benchmark page, configuration block - and that dequantizing straight to
// bfloat16 saved a copy - same page, breakdown item 2): a weight [n][k] is
// stored as 4-bit codes packed two per byte (element 2j of a row in the high
// nibble of byte j) plus one fp32 absmax per 64 consecutive weights of a row.
// Dequantized value: bf16_rne(fp32_rne(level[code] * absmax)).
//
// The 16 levels and their construction are in nf4_table.hpp.
//
// Kernels here are HBM-bound: 0.5 B of codes + 4/64 B of absmax in, 2 B of
// bf16 out per weight.
#include "common.hpp"
#include "kernels.hpp"
#include "nf4_table.hpp"

namespace qlora {

__constant__ uint32_t c_nf4_levels[16] = {QLORA_NF4_LEVEL_BITS};
static const uint32_t h_nf4_levels[16] = {QLORA_NF4_LEVEL_BITS};

void nf4_levels_host(float out[16]) {
  for (int i = 0; i < 16; ++i) {
    uint32_t b = h_nf4_levels[i];
    __builtin_memcpy(&out[i], &b, 4);
  }
}

// Dequantize 8 consecutive weights (one 32-bit word of codes, bytes in
// memory order) with the same absmax; returns them as 4 packed bf16 pairs.
__device__ __forceinline__ u32x4_t dequant8(uint32_t word, float amax, const float* lut) {
  u32x4_t o;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    uint32_t byte = (word >> (8 * b)) & 0xFFu;
    float w0 = lut[byte >> 4] * amax;    // element 2j   (high nibble)
    float w1 = lut[byte & 0xFu] * amax;  // element 2j+1 (low nibble)
    o[b] = pack_bf16x2(w0, w1);
  }
  return o;
}

// out row for weight row n: plain (n) or, with interleave32 = 1 + which,
// the 32-row interleave of two matrices: 64 * (n / 32) + 32 * which + n % 32.
__device__ __forceinline__ int64_t dest_row(int64_t n, int interleave) {
  if (interleave == 0) return n;
  return 64 * (n >> 5) + 32 * (interleave - 1) + (n & 31);
}

// One thread per 8 weights. Grid-stride over n * k / 8 groups.
__global__ __launch_bounds__(256) void nf4_dequant_rows_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ absmax, int64_t n, int64_t k,
    uint16_t* __restrict__ out, int64_t ld_out, int interleave) {
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = __uint_as_float(c_nf4_levels[threadIdx.x]);
  __syncthreads();
  const int64_t groups_per_row = k >> 3;
  const int64_t total = n * groups_per_row;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    int64_t row = t / groups_per_row;
    int64_t grp = t - row * groups_per_row;
    uint32_t word = *(const uint32_t*)(codes + row * (k >> 1) + grp * 4);
    float amax = absmax[row * (k >> 6) + (grp >> 3)];
    u32x4_t v = dequant8(word, amax, lut);
    *(u32x4_t*)(out + dest_row(row, interleave) * ld_out + grp * 8) = v;
  }
}

// Transposing dequant: out[kk][col_ofs + nn] = W[nn][kk]. One 64 x 64 tile
// per block, staged through LDS so both the code reads and the bf16 writes
// are row-contiguous.
__global__ __launch_bounds__(256) void nf4_dequant_transpose_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ absmax, int64_t n, int64_t k,
    uint16_t* __restrict__ out, int64_t ld_out, int64_t col_ofs) {
  __shared__ float lut[16];
  __shared__ uint16_t tile[64][64 + 2];
  const int tid = threadIdx.x;
  if (tid < 16) lut[tid] = __uint_as_float(c_nf4_levels[tid]);
  __syncthreads();
  const int64_t n0 = (int64_t)blockIdx.y * 64, k0 = (int64_t)blockIdx.x * 64;
  {
    // thread: row n0 + tid/4, 16 consecutive k starting at (tid%4)*16
    const int r = tid >> 2, c16 = (tid & 3) * 16;
    const int64_t row = n0 + r;
    const uint8_t* src = codes + row * (k >> 1) + ((k0 + c16) >> 1);
    float amax = absmax[row * (k >> 6) + (k0 >> 6)];
    u32x2_t words = *(const u32x2_t*)src;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      u32x4_t v = dequant8(words[w], amax, lut);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        tile[c16 + w * 8 + 2 * q][r] = (uint16_t)(v[q] & 0xFFFFu);
        tile[c16 + w * 8 + 2 * q + 1][r] = (uint16_t)(v[q] >> 16);
      }
    }
  }
  __syncthreads();
  {
    // thread: output row k0 + tid/4, 16 consecutive n starting at (tid%4)*16
    const int kk = tid >> 2, c16 = (tid & 3) * 16;
    u32x4_t a, b;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[q] = (uint32_t)tile[kk][c16 + 2 * q] | ((uint32_t)tile[kk][c16 + 2 * q + 1] << 16);
      b[q] = (uint32_t)tile[kk][c16 + 8 + 2 * q] | ((uint32_t)tile[kk][c16 + 8 + 2 * q + 1] << 16);
    }
    uint16_t* dst = out + (k0 + kk) * ld_out + col_ofs + n0 + c16;
    *(u32x4_t*)dst = a;
    *(u32x4_t*)(dst + 8) = b;
  }
}

hipError_t launch_nf4_dequant_rows(const uint8_t* codes, const float* absmax, int64_t n, int64_t k,
                                   uint16_t* out, int64_t ld_out, int interleave,
                                   hipStream_t stream) {
  const int64_t total = n * (k >> 3);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  nf4_dequant_rows_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
      codes, absmax, n, k, out, ld_out, interleave);
  return hipGetLastError();
}

hipError_t launch_nf4_dequant_transpose(const uint8_t* codes, const float* absmax, int64_t n,
                                        int64_t k, uint16_t* out, int64_t ld_out, int64_t col_ofs,
                                        hipStream_t stream) {
  if (n == 0 || k == 0) return hipSuccess;
  dim3 grid((unsigned)(k / 64), (unsigned)(n / 64));
  nf4_dequant_transpose_kernel<<<grid, dim3(256), 0, stream>>>(codes, absmax, n, k, out, ld_out,
                                                              col_ofs);
  return hipGetLastError();
}

}  // namespace qlora
