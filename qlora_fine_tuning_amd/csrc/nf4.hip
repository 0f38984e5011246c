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

// One thread per 16 weights of one row (8 code bytes and one absmax in, 32
// bf16 bytes out); blockIdx.y walks the rows (strided when there are more
// than the grid's y extent), blockIdx.x the 4096-weight chunks of a row.
__global__ __launch_bounds__(256) void nf4_dequant_rows_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ absmax, int64_t n, int64_t k,
    uint16_t* __restrict__ out, int64_t ld_out, int interleave) {
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = __uint_as_float(c_nf4_levels[threadIdx.x]);
  __syncthreads();
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // 16-weight group
  if (g * 16 >= k) return;
  for (int64_t row = blockIdx.y; row < n; row += gridDim.y) {
    const uint2 cw = *(const uint2*)(codes + row * (k >> 1) + g * 8);
    const float amax = absmax[row * (k >> 6) + (g >> 2)];
    uint16_t* o = out + dest_row(row, interleave) * ld_out + g * 16;
    *(u32x4_t*)o = dequant8(cw.x, amax, lut);
    *(u32x4_t*)(o + 8) = dequant8(cw.y, amax, lut);
  }
}

// Transposing dequant: out[kk][col_ofs + nn] = W[nn][kk]. A block covers 64
// weight rows x 128 input features: the 4 KB of codes go through LDS, then
// thread t dequantizes 8 weight rows x 4 features and writes 4 output rows
// of 8 consecutive values; 8 lanes cover one 128-byte output row segment.
__global__ __launch_bounds__(256) void nf4_dequant_transpose_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ absmax, int64_t n, int64_t k,
    uint16_t* __restrict__ out, int64_t ld_out, int64_t col_ofs) {
  __shared__ float lut[16];
  __shared__ __attribute__((aligned(16))) uint8_t ct[64 * 64];
  __shared__ float at[64][2];
  const int tid = threadIdx.x;
  if (tid < 16) lut[tid] = __uint_as_float(c_nf4_levels[tid]);
  const int64_t n0 = (int64_t)blockIdx.y * 64, k0 = (int64_t)blockIdx.x * 128;
  const int kvalid = (int)min((int64_t)128, k - k0);   // 64 or 128 (k is a multiple of 64)
  {
    const int r = tid >> 2, c = (tid & 3) * 16;   // 64 rows x 64 code bytes
    if (2 * c < kvalid)
      *(u32x4_t*)&ct[r * 64 + c] = *(const u32x4_t*)(codes + (n0 + r) * (k >> 1) + (k0 >> 1) + c);
    if (tid < 128 && 64 * (tid & 1) < kvalid)
      at[tid >> 1][tid & 1] = absmax[(n0 + (tid >> 1)) * (k >> 6) + (k0 >> 6) + (tid & 1)];
  }
  __syncthreads();
  const int qg = tid & 7, kq = tid >> 3;          // rows 8qg..8qg+7, features 4kq..4kq+3
  if (4 * kq >= kvalid) return;
  float w[8][4];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int r = 8 * qg + q;
    const uint32_t two = *(const uint16_t*)&ct[r * 64 + 2 * kq];
    const float amax = at[r][kq >> 4];
    w[q][0] = lut[(two >> 4) & 0xFu] * amax;
    w[q][1] = lut[two & 0xFu] * amax;
    w[q][2] = lut[(two >> 12) & 0xFu] * amax;
    w[q][3] = lut[(two >> 8) & 0xFu] * amax;
  }
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    u32x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(w[2 * e][f], w[2 * e + 1][f]);
    *(u32x4_t*)(out + (k0 + 4 * kq + f) * ld_out + col_ofs + n0 + 8 * qg) = o;
  }
}

// Quantizer (bf16 weights -> NF4). A lane takes 8 consecutive weights (16 B)
// and 8 lanes a 64-weight block, so a wave reads 1 KB contiguously. Per
// block: absmax = max |w| (exact: a bf16 value, stored as fp32), reduced over
// the block's 8 lanes. The code of w is the level nearest to w / absmax with
// ties to the lower code, found as the number of level midpoints
// mu_i = (L_i + L_{i+1}) / 2 with w > mu_i * absmax, compared in fp64: both
// mu_i and the product are exact there (24 + 8 significant bits), so the
// comparison is the exact one. A quotient of two bf16 values is either on a
// midpoint or at least 2^-34 (relative) away from it, so a nearest-level search
// on the fp64 quotient gives the same codes. An all-zero block gets absmax 0
// and code 7 (the exact zero) everywhere. Weights must be finite. Packing as
// for the dequant: element 2j in the high nibble of byte j.
__global__ __launch_bounds__(256) void nf4_quantize_kernel(const uint16_t* __restrict__ w,
                                                           int64_t nblocks,
                                                           uint8_t* __restrict__ codes,
                                                           float* __restrict__ absmax) {
  double mu[15];
#pragma unroll
  for (int i = 0; i < 15; ++i)
    mu[i] = 0.5 * ((double)__uint_as_float(c_nf4_levels[i]) + (double)__uint_as_float(c_nf4_levels[i + 1]));
  const int lane = threadIdx.x & 63;
  const int64_t groups = nblocks * 8;   // 8-weight groups
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // base is wave-aligned, so the loop condition is uniform across the wave and
  // a block's 8 lanes are either all in range or all out of it
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x + (threadIdx.x & ~63); base < groups;
       base += stride) {
    const int64_t g = base + lane;
    const bool in = g < groups;
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    if (in) v = *(const u32x4_t*)(w + g * 8);
    float wf[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wf[2 * e] = bf16_to_f32(v[e] & 0xFFFFu);
      wf[2 * e + 1] = bf16_to_f32(v[e] >> 16);
    }
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(wf[e]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    amax = fmaxf(amax, __shfl_xor(amax, 4));
    double t[15];
#pragma unroll
    for (int i = 0; i < 15; ++i) t[i] = mu[i] * (double)amax;
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double x = (double)wf[e];
      uint32_t c = 0;
#pragma unroll
      for (int i = 0; i < 15; ++i) c += x > t[i] ? 1u : 0u;
      if (amax == 0.0f) c = 7;
      // element 2j -> high nibble of byte j
      word |= c << (8 * (e >> 1) + ((e & 1) ? 0 : 4));
    }
    if (in) {
      *(uint32_t*)(codes + g * 4) = word;
      if ((lane & 7) == 0) absmax[g >> 3] = amax;
    }
  }
}

hipError_t launch_nf4_quantize(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                               float* absmax, hipStream_t stream) {
  const int64_t nblocks = n * (k / 64);
  if (nblocks == 0) return hipSuccess;
  int64_t grid = (nblocks * 8 + 255) / 256;   // a thread per 8 weights
  if (grid > 256 * 32) grid = 256 * 32;
  nf4_quantize_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(w, nblocks, codes, absmax);
  return hipGetLastError();
}

hipError_t launch_nf4_dequant_rows(const uint8_t* codes, const float* absmax, int64_t n, int64_t k,
                                   uint16_t* out, int64_t ld_out, int interleave,
                                   hipStream_t stream) {
  if (n == 0 || k == 0) return hipSuccess;
  const int64_t gx = (k / 16 + 255) / 256;
  const int64_t gy = n < 65535 ? n : 65535;
  nf4_dequant_rows_kernel<<<dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, stream>>>(
      codes, absmax, n, k, out, ld_out, interleave);
  return hipGetLastError();
}

hipError_t launch_nf4_dequant_transpose(const uint8_t* codes, const float* absmax, int64_t n,
                                        int64_t k, uint16_t* out, int64_t ld_out, int64_t col_ofs,
                                        hipStream_t stream) {
  if (n == 0 || k == 0) return hipSuccess;
  dim3 grid((unsigned)((k + 127) / 128), (unsigned)(n / 64));
  nf4_dequant_transpose_kernel<<<grid, dim3(256), 0, stream>>>(codes, absmax, n, k, out, ld_out,
                                                              col_ofs);
  return hipGetLastError();
}

}  // namespace qlora
