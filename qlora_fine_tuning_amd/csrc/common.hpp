// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// Two fp32 -> packed bf16x2 (lo in bits 0..15), round to nearest even: one
// two-source v_cvt_pk_bf16_f32 (two one-value conversions would also need a
// shift and an OR).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }

// Logistic function with the hardware reciprocal (v_rcp_f32, ~1 ulp), which
// the bf16 outputs cannot resolve; saturates cleanly: exp(-x) -> inf gives
// rcp(inf) = 0, exp(-x) -> 0 gives 1.
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + fast_exp(-x)); }

// Activations of the gated MLP and their derivatives (fp32).
//   act 0: silu(g) = g * sig(g);  silu'(g) = sig * (1 + g * (1 - sig))
//          = sig + silu(g) * (1 - sig)
//   act 1: gelu_tanh(g) = g/2 * (1 + tanh z), z = sqrt(2/pi) (g + 0.044715 g^3)
//          gelu'(g) = (1 + tanh z)/2 + g/2 (1 - tanh^2 z) sqrt(2/pi) (1 + 3*0.044715 g^2)
//   With 1 + tanh z = 2 sig(2z) and 1 - tanh^2 z = 4 sig(2z) (1 - sig(2z)),
//   writing S = sig(2z):  gelu_tanh(g) = g * S,
//          gelu'(g) = S + g S (1 - S) (2 sqrt(2/pi) + 6 sqrt(2/pi) 0.044715 g^2).
//   The exponent of sig(2z), -2z log2(e), is g (c1 + c2 g^2) with folded
//   constants, so one v_exp_f32 (2^x) and one reciprocal form S; the forms
//   with S avoid the cancellation in 1 + tanh z for large negative z.
// ACT is a compile-time constant here so that code applying it to many values
// has no branch per value; the int overloads pick one of the two.
namespace actc {
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kS2pi = 0.7978845608028654f;          // sqrt(2/pi)
constexpr float kGk = 0.044715f;
constexpr float kC1 = -2.0f * 1.4426950408889634f * 0.7978845608028654f;            // -2 log2(e) sqrt(2/pi)
constexpr float kC2 = -2.0f * 1.4426950408889634f * 0.7978845608028654f * 0.044715f;
constexpr float kD0 = 2.0f * 0.7978845608028654f;                                   // 2 sqrt(2/pi)
constexpr float kD2 = 6.0f * 0.7978845608028654f * 0.044715f;
}  // namespace actc

// sig(2z) for the tanh-GELU, from g and g^2
__device__ __forceinline__ float gelu_sig2z(float g, float g2) {
  const float x = g * __builtin_fmaf(g2, actc::kC2, actc::kC1);
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x));
}

template <int ACT>
__device__ __forceinline__ void act_fwd_bwd_t(float g, float* a, float* da) {
  if (ACT == 0) {
    const float sg = sigmoidf_(g);
    const float av = g * sg;
    *a = av;
    *da = __builtin_fmaf(av, 1.0f - sg, sg);
  } else {
    const float g2 = g * g;
    const float S = gelu_sig2z(g, g2);
    const float av = g * S;
    *a = av;
    *da = __builtin_fmaf(av * (1.0f - S), __builtin_fmaf(g2, actc::kD2, actc::kD0), S);
  }
}

template <int ACT>
__device__ __forceinline__ float act_fwd_t(float g) {
  if (ACT == 0) return g * sigmoidf_(g);
  return g * gelu_sig2z(g, g * g);
}

__device__ __forceinline__ void act_fwd_bwd(int act, float g, float* a, float* da) {
  if (act == 0) act_fwd_bwd_t<0>(g, a, da);
  else act_fwd_bwd_t<1>(g, a, da);
}

__device__ __forceinline__ float act_fwd(int act, float g) {
  return act == 0 ? act_fwd_t<0>(g) : act_fwd_t<1>(g);
}

}  // namespace qlora
