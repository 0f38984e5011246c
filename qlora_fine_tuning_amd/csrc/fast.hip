// RMS layernorm, RoPE and cross-entropy kernels for gfx950 (forward and
// backward), the pages' other hand-derived training kernels (Mistral
// benchmark page, breakdown items 7-9; Gemma page, "+1 to RMS LayerNorm" and
// "256K vocabulary"). All three are HBM-bound: each reads its operands once
// with 16-byte loads and does its arithmetic in fp32.
//
//  rmsnorm : one wave per row. Pass 1 sums x^2 (bwd: (dy * w') * x), a wave
//            reduction finishes it; pass 2 re-reads the row, which is still in
//            cache, and writes y (bwd: dx). Forward saves r = 1/rms in fp32.
//  rope    : a thread takes 8 angle pairs (j, j + hd/2) of one token and up to
//            8 heads, so each sine/cosine serves every head it covers. Angles
//            are pos * base^(-2j/hd) in fp64, reduced to [-pi, pi] in fp64,
//            then sin/cos in fp32. Backward rotates by the opposite angle.
//  xent    : one workgroup per row; online max / sum-exp over the row in
//            16-byte chunks (any vocabulary size), then lse = max + log(sum)
//            and CE = lse - x[label]. The mean over labelled rows is a single
//            workgroup's fixed-order sum. Backward writes
//            (exp(x - lse) - onehot) * dloss / n, in place if asked.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace qlora {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ void unpack8(const u32x4_t& v, float* f) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf16_to_f32(v[e] & 0xFFFFu);
    f[2 * e + 1] = bf16_to_f32(v[e] >> 16);
  }
}

__device__ __forceinline__ u32x4_t pack8(const float* f) {
  u32x4_t o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(f[2 * e], f[2 * e + 1]);
  return o;
}

}  // namespace

// ------------------------------------------------------------ RMS layernorm --
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const uint16_t* __restrict__ X, int64_t m,
                                                          int64_t d, const uint16_t* __restrict__ w,
                                                          float eps, int gemma,
                                                          uint16_t* __restrict__ Y,
                                                          float* __restrict__ rstd) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= m) return;   // whole wave leaves together
  const uint16_t* x = X + row * d;
  const int64_t nc = d / 8;
  float ss = 0.0f;
  for (int64_t c = lane; c < nc; c += 64) {
    float f[8];
    unpack8(*(const u32x4_t*)(x + c * 8), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  const float wo = gemma ? 1.0f : 0.0f;
  for (int64_t c = lane; c < nc; c += 64) {
    float f[8], g[8];
    unpack8(*(const u32x4_t*)(x + c * 8), f);
    unpack8(*(const u32x4_t*)(w + c * 8), g);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = f[e] * r * (g[e] + wo);
    *(u32x4_t*)(Y + row * d + c * 8) = pack8(f);
  }
  if (lane == 0 && rstd) rstd[row] = r;
}

__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const uint16_t* __restrict__ dY,
                                                          const uint16_t* __restrict__ X,
                                                          const float* __restrict__ rstd, int64_t m,
                                                          int64_t d, const uint16_t* __restrict__ w,
                                                          int gemma, uint16_t* __restrict__ dX) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= m) return;
  const uint16_t* x = X + row * d;
  const uint16_t* dy = dY + row * d;
  const int64_t nc = d / 8;
  const float wo = gemma ? 1.0f : 0.0f;
  float dot = 0.0f;
  for (int64_t c = lane; c < nc; c += 64) {
    float f[8], g[8], ww[8];
    unpack8(*(const u32x4_t*)(x + c * 8), f);
    unpack8(*(const u32x4_t*)(dy + c * 8), g);
    unpack8(*(const u32x4_t*)(w + c * 8), ww);
#pragma unroll
    for (int e = 0; e < 8; ++e) dot += g[e] * (ww[e] + wo) * f[e];
  }
  dot = wave_sum(dot);
  const float r = rstd[row];
  const float k = r * r * dot / (float)d;
  for (int64_t c = lane; c < nc; c += 64) {
    float f[8], g[8], ww[8];
    unpack8(*(const u32x4_t*)(x + c * 8), f);
    unpack8(*(const u32x4_t*)(dy + c * 8), g);
    unpack8(*(const u32x4_t*)(w + c * 8), ww);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = r * (g[e] * (ww[e] + wo) - f[e] * k);
    *(u32x4_t*)(dX + row * d + c * 8) = pack8(f);
  }
}

hipError_t launch_rmsnorm_fwd(const uint16_t* X, int64_t m, int64_t d, const uint16_t* w, float eps,
                              int gemma, uint16_t* Y, float* rstd, hipStream_t stream) {
  if (m == 0) return hipSuccess;
  rmsnorm_fwd_kernel<<<dim3((unsigned)((m + 3) / 4)), dim3(256), 0, stream>>>(X, m, d, w, eps, gemma,
                                                                               Y, rstd);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const uint16_t* dY, const uint16_t* X, const float* rstd, int64_t m,
                              int64_t d, const uint16_t* w, int gemma, uint16_t* dX,
                              hipStream_t stream) {
  if (m == 0) return hipSuccess;
  rmsnorm_bwd_kernel<<<dim3((unsigned)((m + 3) / 4)), dim3(256), 0, stream>>>(dY, X, rstd, m, d, w,
                                                                               gemma, dX);
  return hipGetLastError();
}

// -------------------------------------------------------------------- RoPE --
constexpr int ROPE_HEADS_PER_THREAD = 8;

// Thread e covers token t, angle group q (8 consecutive j of the first half)
// and heads [hb, hb + 8). X and Y may be the same buffer (each element is
// read and written by one thread only).
__global__ __launch_bounds__(256) void rope_kernel(const uint16_t* X, int64_t ldx, uint16_t* Y,
                                                   int64_t ldy, int64_t m, int heads, int hd,
                                                   const int64_t* __restrict__ pos, RopeFreq fr,
                                                   float sign) {
  const int groups = hd / 16;   // 8-wide angle groups per head
  const int hblocks = (heads + ROPE_HEADS_PER_THREAD - 1) / ROPE_HEADS_PER_THREAD;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= m * hblocks * groups) return;
  const int q = (int)(e % groups);
  const int64_t rest = e / groups;
  const int hb = (int)(rest % hblocks) * ROPE_HEADS_PER_THREAD;
  const int64_t t = rest / hblocks;
  const double p = (double)pos[t];
  const double two_pi = 6.283185307179586476925286766559;
  float c[8], s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double a = p * fr.inv_freq[q * 8 + i];
    const double red = a - rint(a / two_pi) * two_pi;   // |red| <= pi
    sincosf((float)red, &s[i], &c[i]);
    s[i] *= sign;
  }
  const int half = hd / 2;
  const int hend = min(heads, hb + ROPE_HEADS_PER_THREAD);
  for (int h = hb; h < hend; ++h) {
    const uint16_t* xs = X + t * ldx + (int64_t)h * hd + q * 8;
    float a[8], b[8], ya[8], yb[8];
    unpack8(*(const u32x4_t*)xs, a);
    unpack8(*(const u32x4_t*)(xs + half), b);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ya[i] = a[i] * c[i] - b[i] * s[i];
      yb[i] = b[i] * c[i] + a[i] * s[i];
    }
    uint16_t* ys = Y + t * ldy + (int64_t)h * hd + q * 8;
    *(u32x4_t*)ys = pack8(ya);
    *(u32x4_t*)(ys + half) = pack8(yb);
  }
}

hipError_t launch_rope(const uint16_t* X, int64_t ldx, uint16_t* Y, int64_t ldy, int64_t m, int heads,
                       int hd, const int64_t* pos, const RopeFreq& fr, int backward,
                       hipStream_t stream) {
  if (m == 0) return hipSuccess;
  const int hblocks = (heads + ROPE_HEADS_PER_THREAD - 1) / ROPE_HEADS_PER_THREAD;
  const int64_t total = m * hblocks * (hd / 16);
  rope_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream>>>(
      X, ldx, Y, ldy, m, heads, hd, pos, fr, backward ? -1.0f : 1.0f);
  return hipGetLastError();
}

// ----------------------------------------------------------- cross entropy --
namespace {

constexpr int XENT_THREADS = 256;

// online (max, sum of exp(x - max)) of one value folded into (mx, sm)
__device__ __forceinline__ void lse_merge(float& mx, float& sm, float m2, float s2) {
  if (m2 > mx) {
    sm = sm * __expf(mx - m2) + s2;
    mx = m2;
  } else if (m2 > -INFINITY) {
    sm += s2 * __expf(m2 - mx);
  }
}

// workgroup-wide (max, sum) reduction; every thread gets the result
__device__ __forceinline__ void block_lse(float& mx, float& sm) {
  __shared__ float smx[XENT_THREADS / 64], ssm[XENT_THREADS / 64];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(mx, o), s2 = __shfl_xor(sm, o);
    lse_merge(mx, sm, m2, s2);
  }
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    smx[wv] = mx;
    ssm[wv] = sm;
  }
  __syncthreads();
  mx = smx[0];
  sm = ssm[0];
#pragma unroll
  for (int i = 1; i < XENT_THREADS / 64; ++i) lse_merge(mx, sm, smx[i], ssm[i]);
}

}  // namespace

// One workgroup per row of logits X [m][V] (row pitch ld, a multiple of 8).
// Labels outside [0, V) are treated as ignored (no target, CE 0).
__global__ __launch_bounds__(XENT_THREADS) void xent_fwd_kernel(const uint16_t* __restrict__ X,
                                                                int64_t ld, int64_t V,
                                                                const int64_t* __restrict__ labels,
                                                                float* __restrict__ lse_out,
                                                                float* __restrict__ ce_out) {
  const int64_t row = blockIdx.x;
  const uint16_t* x = X + row * ld;
  const int64_t nc = V / 8;
  float mx = -INFINITY, sm = 0.0f;
  for (int64_t c = threadIdx.x; c < nc; c += XENT_THREADS) {
    float f[8];
    unpack8(*(const u32x4_t*)(x + c * 8), f);
    float cm = f[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = fmaxf(cm, f[e]);
    float cs = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) cs += __expf(f[e] - cm);
    lse_merge(mx, sm, cm, cs);
  }
  for (int64_t j = nc * 8 + threadIdx.x; j < V; j += XENT_THREADS)   // tail of V % 8
    lse_merge(mx, sm, bf16_to_f32(x[j]), 1.0f);
  block_lse(mx, sm);
  if (threadIdx.x == 0) {
    const float lse = mx + __logf(sm);
    const int64_t lab = labels[row];
    lse_out[row] = lse;
    ce_out[row] = (lab >= 0 && lab < V) ? lse - bf16_to_f32(x[lab]) : 0.0f;
  }
}

// loss = sum of CE over rows with a target / their number (0 when there are
// none); fixed summation order: thread t takes rows t, t + 256, ...; then a
// tree over the 256 partial sums.
__global__ __launch_bounds__(256) void xent_mean_kernel(const float* __restrict__ ce,
                                                        const int64_t* __restrict__ labels,
                                                        int64_t m, int64_t V,
                                                        float* __restrict__ loss,
                                                        int32_t* __restrict__ n_valid) {
  __shared__ double ps[256];
  __shared__ int pn[256];
  double s = 0.0;
  int n = 0;
  for (int64_t i = threadIdx.x; i < m; i += 256) {
    const int64_t lab = labels[i];
    if (lab >= 0 && lab < V) {
      s += (double)ce[i];
      ++n;
    }
  }
  ps[threadIdx.x] = s;
  pn[threadIdx.x] = n;
  __syncthreads();
  for (int o = 128; o >= 1; o >>= 1) {
    if ((int)threadIdx.x < o) {
      ps[threadIdx.x] += ps[threadIdx.x + o];
      pn[threadIdx.x] += pn[threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    *n_valid = pn[0];
    *loss = pn[0] ? (float)(ps[0] / (double)pn[0]) : 0.0f;
  }
}

// dX = (exp(x - lse) - onehot(label)) * dloss / n for rows with a target, 0
// otherwise. dX may be X itself (each element is read, then written, by one
// thread).
__global__ __launch_bounds__(XENT_THREADS) void xent_bwd_kernel(const uint16_t* X, int64_t ld,
                                                                int64_t V,
                                                                const int64_t* __restrict__ labels,
                                                                const float* __restrict__ lse_in,
                                                                const float* __restrict__ dloss,
                                                                const int32_t* __restrict__ n_valid,
                                                                uint16_t* dX, int64_t ldd) {
  const int64_t row = blockIdx.x;
  const int64_t lab = labels[row];
  const int n = *n_valid;
  const bool on = lab >= 0 && lab < V && n > 0;
  const float scale = on ? (dloss ? *dloss : 1.0f) / (float)n : 0.0f;
  const float lse = lse_in[row];
  const uint16_t* x = X + row * ld;
  uint16_t* dx = dX + row * ldd;
  const int64_t nc = V / 8;
  for (int64_t c = threadIdx.x; c < nc; c += XENT_THREADS) {
    float f[8];
    unpack8(*(const u32x4_t*)(x + c * 8), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = on ? __expf(f[e] - lse) : 0.0f;
      f[e] = (p - (c * 8 + e == lab ? 1.0f : 0.0f)) * scale;
    }
    *(u32x4_t*)(dx + c * 8) = pack8(f);
  }
  for (int64_t j = nc * 8 + threadIdx.x; j < V; j += XENT_THREADS) {
    const float p = on ? __expf(bf16_to_f32(x[j]) - lse) : 0.0f;
    dx[j] = (uint16_t)f32_to_bf16((p - (j == lab ? 1.0f : 0.0f)) * scale);
  }
}

hipError_t launch_xent_fwd(const uint16_t* X, int64_t ld, int64_t m, int64_t V, const int64_t* labels,
                           float* lse, float* ce, float* loss, int32_t* n_valid, hipStream_t stream) {
  if (m > 0) {
    xent_fwd_kernel<<<dim3((unsigned)m), dim3(XENT_THREADS), 0, stream>>>(X, ld, V, labels, lse, ce);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  xent_mean_kernel<<<dim3(1), dim3(256), 0, stream>>>(ce, labels, m, V, loss, n_valid);
  return hipGetLastError();
}

hipError_t launch_xent_bwd(const uint16_t* X, int64_t ld, int64_t m, int64_t V, const int64_t* labels,
                           const float* lse, const float* dloss, const int32_t* n_valid, uint16_t* dX,
                           int64_t ldd, hipStream_t stream) {
  if (m == 0) return hipSuccess;
  xent_bwd_kernel<<<dim3((unsigned)m), dim3(XENT_THREADS), 0, stream>>>(X, ld, V, labels, lse, dloss,
                                                                       n_valid, dX, ldd);
  return hipGetLastError();
}

}  // namespace qlora
