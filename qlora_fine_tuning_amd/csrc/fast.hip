// RMS layernorm, RoPE and cross-entropy kernels for gfx950 (forward and
// backward), the pages' other hand-derived training kernels (Mistral
// benchmark page, breakdown items 7-9; Gemma page, "+1 to RMS LayerNorm" and
// "256K vocabulary"). All three are HBM-bound: each reads its operands once
// with 16-byte loads and does its arithmetic in fp32.
//
//  rmsnorm : one wave per row. The row is loaded into registers at once (rows
//            up to 8192; longer rows re-read it from cache in a second pass),
//            x^2 (bwd: (dy * w') * x) is summed by a wave reduction, then y
//            (bwd: dx) is written. Forward saves r = 1/rms in fp32.
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
// Rows of up to RN_MAX * 512 elements stay in registers: every load of the
// row is issued at once and the row is read once. Longer rows take a loop
// that re-reads the row (from cache) in the second pass.
constexpr int RN_MAX = 16;   // 16-byte chunks per lane, at most

// NCH > 0: the row is register-resident as NCH chunks per lane (d <= NCH * 512);
// NCH == 0: the looping form for any d.
template <int NCH>
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
  const float wo = gemma ? 1.0f : 0.0f;
  float ss = 0.0f;
  if constexpr (NCH > 0) {
    // the weight's chunks are loaded with the row's (up to 8 per lane), so
    // that the scaling pass does not wait for them after the reduction
    constexpr bool WPRE = NCH <= 8;
    u32x4_t v[NCH], vw[WPRE ? NCH : 1];
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      if (lane + 64 * i < nc) {
        v[i] = *(const u32x4_t*)(x + (lane + 64 * i) * 8);
        if constexpr (WPRE) vw[i] = *(const u32x4_t*)(w + (lane + 64 * i) * 8);
      }
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      if (lane + 64 * i < nc) {
        float f[8];
        unpack8(v[i], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
      }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int64_t c = lane + 64 * i;
      if (c < nc) {
        float f[8], g[8];
        unpack8(v[i], f);
        if constexpr (WPRE) unpack8(vw[i], g);
        else unpack8(*(const u32x4_t*)(w + c * 8), g);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = f[e] * r * (g[e] + wo);
        *(u32x4_t*)(Y + row * d + c * 8) = pack8(f);
      }
    }
    if (lane == 0) rstd[row] = r;
  } else {
#pragma unroll 4
    for (int64_t c = lane; c < nc; c += 64) {
      float f[8];
      unpack8(*(const u32x4_t*)(x + c * 8), f);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll 4
    for (int64_t c = lane; c < nc; c += 64) {
      float f[8], g[8];
      unpack8(*(const u32x4_t*)(x + c * 8), f);
      unpack8(*(const u32x4_t*)(w + c * 8), g);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = f[e] * r * (g[e] + wo);
      *(u32x4_t*)(Y + row * d + c * 8) = pack8(f);
    }
    if (lane == 0) rstd[row] = r;
  }
}

template <int NCH>
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
  const float r = rstd[row];
  float dot = 0.0f;
  if constexpr (NCH > 0) {
    // the weight's chunks are loaded once, with the row's (up to 8 per lane)
    constexpr bool WPRE = NCH <= 8;
    u32x4_t vx[NCH], vg[NCH], vw[WPRE ? NCH : 1];
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      if (lane + 64 * i < nc) {
        vx[i] = *(const u32x4_t*)(x + (lane + 64 * i) * 8);
        vg[i] = *(const u32x4_t*)(dy + (lane + 64 * i) * 8);
        if constexpr (WPRE) vw[i] = *(const u32x4_t*)(w + (lane + 64 * i) * 8);
      }
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      if (lane + 64 * i < nc) {
        float f[8], g[8], ww[8];
        unpack8(vx[i], f);
        unpack8(vg[i], g);
        if constexpr (WPRE) unpack8(vw[i], ww);
        else unpack8(*(const u32x4_t*)(w + (lane + 64 * i) * 8), ww);
#pragma unroll
        for (int e = 0; e < 8; ++e) dot += g[e] * (ww[e] + wo) * f[e];
      }
    dot = wave_sum(dot);
    const float k = r * r * dot / (float)d;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int64_t c = lane + 64 * i;
      if (c < nc) {
        float f[8], g[8], ww[8];
        unpack8(vx[i], f);
        unpack8(vg[i], g);
        if constexpr (WPRE) unpack8(vw[i], ww);
        else unpack8(*(const u32x4_t*)(w + c * 8), ww);   // w is small and cached
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = r * (g[e] * (ww[e] + wo) - f[e] * k);
        *(u32x4_t*)(dX + row * d + c * 8) = pack8(f);
      }
    }
  } else {
#pragma unroll 4
    for (int64_t c = lane; c < nc; c += 64) {
      float f[8], g[8], ww[8];
      unpack8(*(const u32x4_t*)(x + c * 8), f);
      unpack8(*(const u32x4_t*)(dy + c * 8), g);
      unpack8(*(const u32x4_t*)(w + c * 8), ww);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += g[e] * (ww[e] + wo) * f[e];
    }
    dot = wave_sum(dot);
    const float k = r * r * dot / (float)d;
#pragma unroll 4
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
}

hipError_t launch_rmsnorm_fwd(const uint16_t* X, int64_t m, int64_t d, const uint16_t* w, float eps,
                              int gemma, uint16_t* Y, float* rstd, hipStream_t stream) {
  if (m == 0) return hipSuccess;
  const dim3 grid((unsigned)((m + 3) / 4));
  if (d <= 8 * 512)
    rmsnorm_fwd_kernel<8><<<grid, dim3(256), 0, stream>>>(X, m, d, w, eps, gemma, Y, rstd);
  else if (d <= RN_MAX * 512)
    rmsnorm_fwd_kernel<RN_MAX><<<grid, dim3(256), 0, stream>>>(X, m, d, w, eps, gemma, Y, rstd);
  else
    rmsnorm_fwd_kernel<0><<<grid, dim3(256), 0, stream>>>(X, m, d, w, eps, gemma, Y, rstd);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const uint16_t* dY, const uint16_t* X, const float* rstd, int64_t m,
                              int64_t d, const uint16_t* w, int gemma, uint16_t* dX,
                              hipStream_t stream) {
  if (m == 0) return hipSuccess;
  const dim3 grid((unsigned)((m + 3) / 4));
  if (d <= 8 * 512)
    rmsnorm_bwd_kernel<8><<<grid, dim3(256), 0, stream>>>(dY, X, rstd, m, d, w, gemma, dX);
  else if (d <= RN_MAX * 512)
    rmsnorm_bwd_kernel<RN_MAX><<<grid, dim3(256), 0, stream>>>(dY, X, rstd, m, d, w, gemma, dX);
  else
    rmsnorm_bwd_kernel<0><<<grid, dim3(256), 0, stream>>>(dY, X, rstd, m, d, w, gemma, dX);
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
  const int half = hd / 2;
  const int nh = min(heads - hb, ROPE_HEADS_PER_THREAD);
  // All loads are issued before the angles are formed: first the position and
  // the group's 8 inverse frequencies (64 bytes of the argument block), which
  // the angles wait for, then the head values, which stay in flight meanwhile
  // (X and Y may be one buffer, so the compiler could not move a later head's
  // loads above an earlier head's stores by itself). Formed one after
  // another, each angle had waited for its own frequency's load first.
  const double p = (double)pos[t];
  double fi[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) fi[i] = fr.inv_freq[q * 8 + i];
  __builtin_amdgcn_sched_barrier(0);
  // (heads past the last one reload that one: no branch between the loads,
  // so the wait for the frequencies leaves the head loads in flight)
  u32x4_t va[ROPE_HEADS_PER_THREAD], vb[ROPE_HEADS_PER_THREAD];
#pragma unroll
  for (int i = 0; i < ROPE_HEADS_PER_THREAD; ++i) {
    const uint16_t* xs = X + t * ldx + (int64_t)(hb + min(i, nh - 1)) * hd + q * 8;
    va[i] = *(const u32x4_t*)xs;
    vb[i] = *(const u32x4_t*)(xs + half);
  }
  __builtin_amdgcn_sched_barrier(0);
  const double two_pi = 6.283185307179586476925286766559;
  float c[8], s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double a = p * fi[i];
    const double red = a - rint(a / two_pi) * two_pi;   // |red| <= pi
    sincosf((float)red, &s[i], &c[i]);
    s[i] *= sign;
  }
#pragma unroll
  for (int i = 0; i < ROPE_HEADS_PER_THREAD; ++i) {
    if (i < nh) {
      float a[8], b[8], ya[8], yb[8];
      unpack8(va[i], a);
      unpack8(vb[i], b);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        ya[k] = a[k] * c[k] - b[k] * s[k];
        yb[k] = b[k] * c[k] + a[k] * s[k];
      }
      uint16_t* ys = Y + t * ldy + (int64_t)(hb + i) * hd + q * 8;
      *(u32x4_t*)ys = pack8(ya);
      *(u32x4_t*)(ys + half) = pack8(yb);
    }
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
// 16-byte loads a thread issues before it uses any of them (the row passes
// are bound by how many bytes each workgroup keeps in flight)
constexpr int XENT_LOADS = 8;

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// 2^x by the hardware instruction (v_exp_f32, about 1 ulp; results below the
// normal range flush to 0, which a sum of exponentials cannot resolve anyway).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// The running state is kept in base 2: mx is the maximum of x * log2(e) and
// sm the sum of 2^(x log2(e) - mx), so each exponential is one fused
// multiply-add and one v_exp_f32. (mx, sm) <- merge with (m2, s2); either
// side may be empty (max -inf, sum 0).
__device__ __forceinline__ void lse_merge(float& mx, float& sm, float m2, float s2) {
  if (m2 > mx) {
    sm = sm * exp2_hw(mx - m2) + s2;
    mx = m2;
  } else if (m2 > -INFINITY) {
    sm += s2 * exp2_hw(m2 - mx);
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

// One thread's online (max, sum) over its chunks c = threadIdx.x + k *
// XENT_THREADS of a row, XENT_LOADS chunk loads in flight (the forward and
// the fused kernel share this pass, so they give the same bits).
__device__ __forceinline__ void row_lse_pass(const uint16_t* x, int64_t nc, float& mx, float& sm) {
  auto fold = [&](const u32x4_t& v, float& m_, float& s_) {
    float f[8];
    unpack8(v, f);
    float cm = f[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = fmaxf(cm, f[e]);
    const float mn = fmaxf(m_, cm * LOG2E);
    float cs = s_ * exp2_hw(m_ - mn);
#pragma unroll
    for (int e = 0; e < 8; ++e) cs += exp2_hw(fmaf(f[e], LOG2E, -mn));
    m_ = mn;
    s_ = cs;
  };
  int64_t c = threadIdx.x;
  for (; c + (XENT_LOADS - 1) * XENT_THREADS < nc; c += XENT_LOADS * XENT_THREADS) {   // loads in flight
    u32x4_t v[XENT_LOADS];
#pragma unroll
    for (int u = 0; u < XENT_LOADS; ++u) v[u] = *(const u32x4_t*)(x + (c + u * XENT_THREADS) * 8);
#pragma unroll
    for (int u = 0; u < XENT_LOADS; ++u) fold(v[u], mx, sm);
  }
  for (; c < nc; c += XENT_THREADS) fold(*(const u32x4_t*)(x + c * 8), mx, sm);
}

// The gradient of one row's 8-value chunks, c = threadIdx.x + k * XENT_THREADS:
// dx = (2^(x log2(e) - l2) - onehot(lab)) * scale. Each chunk is read and
// written by the same thread, so dx may be x; the loads of a batch of chunks
// are issued before any of its stores (a store to dx could otherwise alias
// the next load, and the loop would keep one load in flight).
__device__ __forceinline__ void xent_grad_chunks(const uint16_t* x, uint16_t* dx, int64_t nc,
                                                 int64_t lab, float l2, float scale, bool on) {
  auto grad = [&](const u32x4_t& v, int64_t c) {
    float f[8];
    unpack8(v, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = on ? exp2_hw(fmaf(f[e], LOG2E, -l2)) : 0.0f;
      f[e] = (p - (c * 8 + e == lab ? 1.0f : 0.0f)) * scale;
    }
    *(u32x4_t*)(dx + c * 8) = pack8(f);
  };
  constexpr int U = 4;
  int64_t c = threadIdx.x;
  for (; c + (U - 1) * XENT_THREADS < nc; c += U * XENT_THREADS) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = *(const u32x4_t*)(x + (c + u * XENT_THREADS) * 8);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) grad(v[u], c + u * XENT_THREADS);
  }
  for (; c < nc; c += XENT_THREADS) grad(*(const u32x4_t*)(x + c * 8), c);
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
  // fold 8 finite values at a time: rescale the running sum to the new
  // maximum (no branch; 2^(-inf) = 0 covers the empty start), then add their
  // exponentials
  float mx = -INFINITY, sm = 0.0f;
  row_lse_pass(x, nc, mx, sm);
  for (int64_t j = nc * 8 + threadIdx.x; j < V; j += XENT_THREADS)   // tail of V % 8
    lse_merge(mx, sm, bf16_to_f32(x[j]) * LOG2E, 1.0f);
  block_lse(mx, sm);
  if (threadIdx.x == 0) {
    const float lse = (mx + __log2f(sm)) * LN2;
    const int64_t lab = labels[row];
    lse_out[row] = lse;
    ce_out[row] = (lab >= 0 && lab < V) ? lse - bf16_to_f32(x[lab]) : 0.0f;
  }
}

// loss = sum of CE over rows with a target / their number (0 when there are
// none). One workgroup of 1024 threads; fixed summation order: thread t adds
// rows t, t + 1024, ... in order (fp64), then a tree over the 1024 partials.
__global__ __launch_bounds__(1024) void xent_mean_kernel(const float* __restrict__ ce,
                                                         const int64_t* __restrict__ labels,
                                                         int64_t m, int64_t V,
                                                         float* __restrict__ loss,
                                                         int32_t* __restrict__ n_valid) {
  __shared__ double ps[1024];
  __shared__ int pn[1024];
  double s = 0.0;
  int n = 0;
#pragma unroll 8
  for (int64_t i = threadIdx.x; i < m; i += 1024) {
    const int64_t lab = labels[i];
    const float c = ce[i];
    if (lab >= 0 && lab < V) {
      s += (double)c;
      ++n;
    }
  }
  ps[threadIdx.x] = s;
  pn[threadIdx.x] = n;
  __syncthreads();
  for (int o = 512; o >= 1; o >>= 1) {
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
                                                                float dloss_val,
                                                                const int32_t* __restrict__ n_valid,
                                                                uint16_t* dX, int64_t ldd) {
  const int64_t row = blockIdx.x;
  const int64_t lab = labels[row];
  const int n = *n_valid;
  const bool on = lab >= 0 && lab < V && n > 0;
  const float scale = on ? (dloss ? *dloss : dloss_val) / (float)n : 0.0f;
  const float l2 = lse_in[row] * LOG2E;
  const uint16_t* x = X + row * ld;
  uint16_t* dx = dX + row * ldd;
  const int64_t nc = V / 8;
  xent_grad_chunks(x, dx, nc, lab, l2, scale, on);
  for (int64_t j = nc * 8 + threadIdx.x; j < V; j += XENT_THREADS) {
    const float p = on ? exp2_hw(fmaf(bf16_to_f32(x[j]), LOG2E, -l2)) : 0.0f;
    dx[j] = (uint16_t)f32_to_bf16((p - (j == lab ? 1.0f : 0.0f)) * scale);
  }
}

// number of rows with a target (one 1024-thread workgroup, fixed order)
__global__ __launch_bounds__(1024) void xent_count_kernel(const int64_t* __restrict__ labels,
                                                          int64_t m, int64_t V,
                                                          int32_t* __restrict__ n_valid) {
  __shared__ int pn[1024];
  int n = 0;
#pragma unroll 8
  for (int64_t i = threadIdx.x; i < m; i += 1024) {
    const int64_t lab = labels[i];
    n += (lab >= 0 && lab < V) ? 1 : 0;
  }
  pn[threadIdx.x] = n;
  __syncthreads();
  for (int o = 512; o >= 1; o >>= 1) {
    if ((int)threadIdx.x < o) pn[threadIdx.x] += pn[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *n_valid = pn[0];
}

// Forward and backward of one row in one visit: the online (max, sum) pass of
// xent_fwd_kernel, then the gradient of xent_bwd_kernel with scale dloss / n
// (n from xent_count_kernel); the second pass re-reads the row from cache.
// Same arithmetic as the two separate kernels, so the same bits. dX may be X.
__global__ __launch_bounds__(XENT_THREADS) void xent_fused_kernel(const uint16_t* X, int64_t ld,
                                                                  int64_t V,
                                                                  const int64_t* __restrict__ labels,
                                                                  float dloss,
                                                                  const int32_t* __restrict__ n_valid,
                                                                  float* __restrict__ lse_out,
                                                                  float* __restrict__ ce_out,
                                                                  uint16_t* dX, int64_t ldd) {
  const int64_t row = blockIdx.x;
  const uint16_t* x = X + row * ld;
  const int64_t nc = V / 8;
  float mx = -INFINITY, sm = 0.0f;
  row_lse_pass(x, nc, mx, sm);
  for (int64_t j = nc * 8 + threadIdx.x; j < V; j += XENT_THREADS)
    lse_merge(mx, sm, bf16_to_f32(x[j]) * LOG2E, 1.0f);
  block_lse(mx, sm);   // ends with every thread past the block's barrier
  const float lse = (mx + __log2f(sm)) * LN2;
  const int64_t lab = labels[row];
  if (threadIdx.x == 0) {
    lse_out[row] = lse;
    ce_out[row] = (lab >= 0 && lab < V) ? lse - bf16_to_f32(x[lab]) : 0.0f;
  }
  __syncthreads();   // x[lab] is read before any thread overwrites the row
  const int n = *n_valid;
  const bool on = lab >= 0 && lab < V && n > 0;
  const float scale = on ? dloss / (float)n : 0.0f;
  const float l2 = lse * LOG2E;
  uint16_t* dx = dX + row * ldd;
  xent_grad_chunks(x, dx, nc, lab, l2, scale, on);
  for (int64_t j = nc * 8 + threadIdx.x; j < V; j += XENT_THREADS) {
    const float p = on ? exp2_hw(fmaf(bf16_to_f32(x[j]), LOG2E, -l2)) : 0.0f;
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
  xent_mean_kernel<<<dim3(1), dim3(1024), 0, stream>>>(ce, labels, m, V, loss, n_valid);
  return hipGetLastError();
}

hipError_t launch_xent_bwd(const uint16_t* X, int64_t ld, int64_t m, int64_t V, const int64_t* labels,
                           const float* lse, const float* dloss, const int32_t* n_valid, uint16_t* dX,
                           int64_t ldd, hipStream_t stream) {
  if (m == 0) return hipSuccess;
  xent_bwd_kernel<<<dim3((unsigned)m), dim3(XENT_THREADS), 0, stream>>>(X, ld, V, labels, lse, dloss,
                                                                       1.0f, n_valid, dX, ldd);
  return hipGetLastError();
}

}  // namespace qlora

namespace qlora {

// Rows of up to 64 KB take the one-visit kernel: with about 2048 rows in
// flight the re-read hits cache. Longer rows (Gemma's 256K vocabulary) would
// be read twice from HBM, so they take the forward and backward kernels in
// turn, which give the same bits.
constexpr int64_t XENT_FUSED_MAX_ROW_BYTES = 65536;

hipError_t launch_xent_fused(const uint16_t* X, int64_t ld, int64_t m, int64_t V, const int64_t* labels,
                             float dloss, float* lse, float* ce, float* loss, int32_t* n_valid,
                             uint16_t* dX, int64_t ldd, hipStream_t stream) {
  if (V * 2 > XENT_FUSED_MAX_ROW_BYTES) {
    hipError_t e = launch_xent_fwd(X, ld, m, V, labels, lse, ce, loss, n_valid, stream);
    if (e != hipSuccess || m == 0) return e;
    xent_bwd_kernel<<<dim3((unsigned)m), dim3(XENT_THREADS), 0, stream>>>(X, ld, V, labels, lse, nullptr,
                                                                         dloss, n_valid, dX, ldd);
    return hipGetLastError();
  }
  xent_count_kernel<<<dim3(1), dim3(1024), 0, stream>>>(labels, m, V, n_valid);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || m == 0) return e;
  xent_fused_kernel<<<dim3((unsigned)m), dim3(XENT_THREADS), 0, stream>>>(X, ld, V, labels, dloss,
                                                                         n_valid, lse, ce, dX, ldd);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  xent_mean_kernel<<<dim3(1), dim3(1024), 0, stream>>>(ce, labels, m, V, loss, n_valid);
  return hipGetLastError();
}

}  // namespace qlora
