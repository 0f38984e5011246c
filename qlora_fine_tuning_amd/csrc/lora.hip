// Rank-r LoRA side-path kernels for gfx950 (HBM-bound "skinny" products).
//
// The chained-matmul bracketing of the Mistral benchmark page (items 10-11,
// "manual autograd") puts the rank-r product first: X A^T and dY B are
// [m][r] and cheap; the LoRA weight gradients dA = s T^T X and dB = s dY^T U
// are reductions over tokens of one big operand against an [m][r] one. All of
// these read one large bf16 operand once (X, dY, H, dg|du: 2 B per element)
// and are bound by HBM bandwidth, not by arithmetic.
//
//  rowdot     : U = G L^T  ([M][K] x [R][K]^T -> [M][R]) on MFMA 16x16x32 with
//               operand fragments loaded straight from global memory; K split
//               across the 8 waves of a block, partials summed in LDS in a
//               fixed order. Also emits the K-extension operand of the big
//               GEMM: [hi(sU) | lo(sU)] in bf16.
//  colreduce  : part[c][col][j] = sum_{i in chunk c} G[i][col] V[i][j]; each
//               lane owns two columns, V's row is wave-uniform (scalar loads).
//               G may be H = act(g) * u recomputed on the fly from g, u.
//  finish     : fixed-order sum over chunks, scale, bf16, any output stride.
#include "common.hpp"
#include "kernels.hpp"

namespace qlora {

// ------------------------------------------------------------------ rowdot --
template <int RT>
__global__ __launch_bounds__(512) void rowdot_kernel(const uint16_t* __restrict__ G, int64_t ldg,
                                                     const uint16_t* __restrict__ L, int64_t ldl,
                                                     int M, int K, int R, float s,
                                                     float* __restrict__ Uf,
                                                     float* __restrict__ Uf2, int split,
                                                     int64_t ldu, uint16_t* __restrict__ Ue,
                                                     int64_t ldue, int KE) {
  constexpr int RW = RT * 16;
  __shared__ float red[8][16][RW + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i0 = blockIdx.x * 16;
  const int nsteps = K >> 5;
  const int per = (nsteps + 7) >> 3;
  const int s0 = wave * per;
  const int s1 = min(nsteps, s0 + per);
  const int row = min(i0 + (lane & 15), M - 1);
  const int kq = (lane >> 4) * 8;
  const uint16_t* gp = G + (int64_t)row * ldg + kq;
  const uint16_t* lp[RT];
  bool lv[RT];
  f32x4_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int j = t * 16 + (lane & 15);
    lv[t] = j < R;
    lp[t] = L + (int64_t)min(j, R - 1) * ldl + kq;
    acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
#pragma unroll 4
  for (int st = s0; st < s1; ++st) {
    const int k0 = st * 32;
    const bf16x8_t a = *(const bf16x8_t*)(gp + k0);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      bf16x8_t b = *(const bf16x8_t*)(lp[t] + k0);
      if (!lv[t]) b = bf16x8_t{};
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[t], 0, 0, 0);
    }
  }
  // acc[t][v] = partial U[i0 + 4*(lane/16) + v][t*16 + lane%16]
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][4 * (lane >> 4) + v][t * 16 + (lane & 15)] = acc[t][v];
  __syncthreads();
  for (int e = tid; e < 16 * RW; e += 512) {
    const int i = e / RW, j = e - (e / RW) * RW;
    const int gi = i0 + i;
    if (gi >= M || j >= R) continue;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < 8; ++w) sum += red[w][i][j];
    if (j < split) {
      if (Uf) Uf[(int64_t)gi * ldu + j] = sum;
    } else if (Uf2) {
      Uf2[(int64_t)gi * ldu + (j - split)] = sum;
    }
    if (Ue) {
      const float su = s * sum;
      const uint32_t hi = f32_to_bf16(su);
      const float lo = su - bf16_to_f32(hi);
      Ue[(int64_t)gi * ldue + j] = (uint16_t)hi;
      Ue[(int64_t)gi * ldue + R + j] = (uint16_t)f32_to_bf16(lo);
    }
  }
  if (Ue) {
    const int pad = KE - 2 * R;
    for (int e = tid; e < 16 * pad; e += 512) {
      const int i = e / pad, j = 2 * R + (e - (e / pad) * pad);
      const int gi = i0 + i;
      if (gi < M) Ue[(int64_t)gi * ldue + j] = 0;
    }
  }
}

hipError_t launch_rowdot(const uint16_t* G, int64_t ldg, const uint16_t* L, int64_t ldl, int M,
                         int K, int R, float s, float* Uf, float* Uf2, int split, int64_t ldu,
                         uint16_t* Ue, int64_t ldue, int KE, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  dim3 grid((unsigned)((M + 15) / 16)), block(512);
  const int rt = (R + 15) / 16;
  switch (rt) {
    case 1: rowdot_kernel<1><<<grid, block, 0, stream>>>(G, ldg, L, ldl, M, K, R, s, Uf, Uf2, split, ldu, Ue, ldue, KE); break;
    case 2: rowdot_kernel<2><<<grid, block, 0, stream>>>(G, ldg, L, ldl, M, K, R, s, Uf, Uf2, split, ldu, Ue, ldue, KE); break;
    case 3: rowdot_kernel<3><<<grid, block, 0, stream>>>(G, ldg, L, ldl, M, K, R, s, Uf, Uf2, split, ldu, Ue, ldue, KE); break;
    case 4: rowdot_kernel<4><<<grid, block, 0, stream>>>(G, ldg, L, ldl, M, K, R, s, Uf, Uf2, split, ldu, Ue, ldue, KE); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// --------------------------------------------------------------- colreduce --
int colreduce_chunks(int M) {
  int c = (M + 255) / 256;
  if (c < 1) c = 1;
  if (c > 32) c = 32;
  return c;
}

template <int RT, bool HMODE>
__global__ __launch_bounds__(256) void colreduce_kernel(const uint16_t* __restrict__ G,
                                                        const uint16_t* __restrict__ gate,
                                                        const uint16_t* __restrict__ up, int act,
                                                        int64_t ldg, int M, int C,
                                                        const float* __restrict__ V, int64_t ldv,
                                                        int R, int rows_per_chunk,
                                                        float* __restrict__ part) {
  const int c = (blockIdx.x * 256 + threadIdx.x) * 2;
  const int chunk = blockIdx.y;
  const int r0 = chunk * rows_per_chunk;
  const int r1 = min(M, r0 + rows_per_chunk);
  const bool valid = c < C;
  const int cc = valid ? c : 0;
  float acc0[RT], acc1[RT];
#pragma unroll
  for (int j = 0; j < RT; ++j) acc0[j] = acc1[j] = 0.0f;
  for (int i = r0; i < r1; ++i) {
    float x0, x1;
    if (HMODE) {
      const uint32_t gw = *(const uint32_t*)(gate + (int64_t)i * ldg + cc);
      const uint32_t uw = *(const uint32_t*)(up + (int64_t)i * ldg + cc);
      const float h0 = act_fwd(act, bf16_to_f32(gw & 0xFFFFu)) * bf16_to_f32(uw & 0xFFFFu);
      const float h1 = act_fwd(act, bf16_to_f32(gw >> 16)) * bf16_to_f32(uw >> 16);
      x0 = bf16_to_f32(f32_to_bf16(h0));
      x1 = bf16_to_f32(f32_to_bf16(h1));
    } else {
      const uint32_t w = *(const uint32_t*)(G + (int64_t)i * ldg + cc);
      x0 = bf16_to_f32(w & 0xFFFFu);
      x1 = bf16_to_f32(w >> 16);
    }
    const float* vr = V + (int64_t)i * ldv;
#pragma unroll
    for (int j = 0; j < RT; ++j) {
      if (j < R) {
        const float vj = vr[j];
        acc0[j] = fmaf(x0, vj, acc0[j]);
        acc1[j] = fmaf(x1, vj, acc1[j]);
      }
    }
  }
  if (valid) {
    float* o = part + ((int64_t)chunk * C + c) * R;
    for (int j = 0; j < R && j < RT; ++j) {
      o[j] = acc0[j];
      o[R + j] = acc1[j];
    }
  }
}

hipError_t launch_colreduce(const uint16_t* G, const uint16_t* gate, const uint16_t* up, int act,
                            int64_t ldg, int M, int C, const float* V, int64_t ldv, int R,
                            float* part, hipStream_t stream) {
  if (M <= 0 || C <= 0) return hipSuccess;
  const int chunks = colreduce_chunks(M);
  const int rpc = (M + chunks - 1) / chunks;
  dim3 grid((unsigned)((C + 511) / 512), (unsigned)chunks), block(256);
  const bool hm = gate != nullptr;
#define QL_CR(RTV)                                                                              \
  do {                                                                                          \
    if (hm)                                                                                     \
      colreduce_kernel<RTV, true><<<grid, block, 0, stream>>>(G, gate, up, act, ldg, M, C, V,   \
                                                              ldv, R, rpc, part);               \
    else                                                                                        \
      colreduce_kernel<RTV, false><<<grid, block, 0, stream>>>(G, gate, up, act, ldg, M, C, V,  \
                                                               ldv, R, rpc, part);              \
  } while (0)
  if (R <= 8) QL_CR(8);
  else if (R <= 16) QL_CR(16);
  else if (R <= 32) QL_CR(32);
  else if (R <= 64) QL_CR(64);
  else return hipErrorInvalidValue;
#undef QL_CR
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void colreduce_finish_kernel(const float* __restrict__ part,
                                                               int chunks, int C, int R, int j0,
                                                               int nj, float s,
                                                               uint16_t* __restrict__ out,
                                                               int64_t ocs, int64_t ojs) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)C * nj) return;
  const int col = (int)(e / nj);
  const int jj = (int)(e - (int64_t)col * nj);
  float sum = 0.0f;
  for (int ch = 0; ch < chunks; ++ch) sum += part[((int64_t)ch * C + col) * R + j0 + jj];
  out[(int64_t)col * ocs + (int64_t)jj * ojs] = (uint16_t)f32_to_bf16(s * sum);
}

hipError_t launch_colreduce_finish(const float* part, int chunks, int C, int R, int j0, int nj,
                                   float s, uint16_t* out, int64_t ocs, int64_t ojs,
                                   hipStream_t stream) {
  const int64_t total = (int64_t)C * nj;
  if (total <= 0) return hipSuccess;
  colreduce_finish_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream>>>(
      part, chunks, C, R, j0, nj, s, out, ocs, ojs);
  return hipGetLastError();
}

// ---------------------------------------------------------------- layout --
__global__ __launch_bounds__(256) void copy2d_kernel(const uint16_t* __restrict__ src, int64_t s_rs,
                                                     int64_t s_cs, int rows, int cols,
                                                     uint16_t* __restrict__ dst, int64_t d_rs,
                                                     int64_t d_cs, int interleave) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)rows * cols) return;
  const int r = (int)(e / cols);
  const int c = (int)(e - (int64_t)r * cols);
  int64_t dr = r;
  if (interleave) dr = 64 * (r >> 5) + 32 * (interleave - 1) + (r & 31);
  dst[dr * d_rs + (int64_t)c * d_cs] = src[(int64_t)r * s_rs + (int64_t)c * s_cs];
}

hipError_t launch_copy2d(const uint16_t* src, int64_t s_rs, int64_t s_cs, int rows, int cols,
                         uint16_t* dst, int64_t d_rs, int64_t d_cs, int interleave,
                         hipStream_t stream) {
  const int64_t total = (int64_t)rows * cols;
  if (total <= 0) return hipSuccess;
  copy2d_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream>>>(
      src, s_rs, s_cs, rows, cols, dst, d_rs, d_cs, interleave);
  return hipGetLastError();
}

// Zero-fill by a kernel (not hipMemsetAsync) so callers may capture the
// sequence in a graph.
__global__ __launch_bounds__(256) void zero_kernel(uint8_t* __restrict__ dst, size_t bytes) {
  const size_t n16 = bytes >> 4;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
    ((u32x4_t*)dst)[i] = u32x4_t{0u, 0u, 0u, 0u};
  const size_t tail = bytes & 15;
  if (blockIdx.x == 0 && threadIdx.x < tail) dst[(n16 << 4) + threadIdx.x] = 0;
}

hipError_t launch_zero(void* dst, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  size_t blocks = ((bytes >> 4) + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  zero_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>((uint8_t*)dst, bytes);
  return hipGetLastError();
}

}  // namespace qlora
