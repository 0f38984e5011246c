// Diagnostic: sustained dense bf16 MFMA rate and shader clock of this GPU.
//
// Every wave runs 8 independent accumulation chains of
// v_mfma_f32_32x32x16_bf16 on operands with random bits (random data draws
// more power than zeros, which the clock reacts to). Wave 0 of block 0 reads
// the shader-clock counter (s_memtime) and the 100 MHz constant clock
// (s_memrealtime) around its loop, which gives the clock under this load.
// Nothing is allocated: the clock readings land in a file-scope device array.
#include "common.hpp"
#include "kernels.hpp"

namespace qlora {

__device__ long long g_probe_clk[2];
__device__ float g_probe_sink[1];

__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, uint32_t seed) {
  const int lane = threadIdx.x & 63;
  uint32_t x = seed ^ (uint32_t)(blockIdx.x * 256 + threadIdx.x) * 2654435761u;
  auto rnd = [&]() {
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    // bf16 pairs with exponents near 1.0 and random mantissas and signs
    return (x & 0x807F807Fu) | 0x3F003F00u;
  };
  u32x4_t av[2], bv[2];
  for (int i = 0; i < 2; ++i) {
    av[i] = u32x4_t{rnd(), rnd(), rnd(), rnd()};
    bv[i] = u32x4_t{rnd(), rnd(), rnd(), rnd()};
  }
  bf16x8_t a[2], b[2];
  for (int i = 0; i < 2; ++i) {
    a[i] = __builtin_bit_cast(bf16x8_t, av[i]);
    b[i] = __builtin_bit_cast(bf16x8_t, bv[i]);
  }
  f32x16_t acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;
  const long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c & 1], b[(c >> 1) & 1], acc[c], 0, 0, 0);
  }
  const long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  if (s == 1234.5678f && lane == 0) g_probe_sink[0] = s;   // keeps the chains alive
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    g_probe_clk[0] = t1 - t0;
    g_probe_clk[1] = r1 - r0;
  }
}

hipError_t probe_mfma_peak(int iters, hipStream_t stream, double* tflops, double* ghz) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int blocks = 8 * cus;   // 8 blocks of 4 waves per CU
  hipEvent_t e0, e1;
  if ((e = hipEventCreate(&e0)) != hipSuccess) return e;
  if ((e = hipEventCreate(&e1)) != hipSuccess) return e;
  float best = 1e30f;
  for (int rep = 0; rep < 4 && e == hipSuccess; ++rep) {   // first rep warms the clock
    e = hipEventRecord(e0, stream);
    if (e == hipSuccess) {
      mfma_peak_kernel<<<dim3(blocks), dim3(256), 0, stream>>>(iters, 0x9E3779B9u + rep);
      e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e1, stream);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e == hipSuccess && rep > 0 && ms < best) best = ms;
  }
  long long clk[2] = {0, 1};
  if (e == hipSuccess) e = hipMemcpyFromSymbol(clk, HIP_SYMBOL(g_probe_clk), sizeof(clk));
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (e != hipSuccess) return e;
  const double flops = (double)blocks * 4 * iters * 8 * (32.0 * 32 * 16 * 2);
  *tflops = flops / (best * 1e-3) / 1e12;
  *ghz = clk[1] > 0 ? (double)clk[0] / ((double)clk[1] / 100e6) / 1e9 : 0.0;
  return hipSuccess;
}

}  // namespace qlora
