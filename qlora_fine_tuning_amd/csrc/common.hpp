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
//   act 0: silu(g) = g * sigmoid(g);  silu'(g) = sig * (1 + g * (1 - sig))
//   act 1: gelu_tanh(g) = g/2 * (1 + tanh z), z = sqrt(2/pi) (g + 0.044715 g^3)
//          gelu'(g) = (1 + tanh z)/2 + g/2 (1 - tanh^2 z) sqrt(2/pi) (1 + 3*0.044715 g^2)
// tanh z is formed as 2 * sigmoid(2z) - 1.
// ACT is a compile-time constant here so that code applying it to many values
// has no branch per value; the int overloads pick one of the two.
template <int ACT>
__device__ __forceinline__ void act_fwd_bwd_t(float g, float* a, float* da) {
  if (ACT == 0) {
    float sg = sigmoidf_(g);
    *a = g * sg;
    *da = sg * (1.0f + g * (1.0f - sg));
  } else {
    const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
    const float k1 = 0.044715f;
    float g2 = g * g;
    float z = k0 * (g + k1 * g2 * g);
    float th = 2.0f * sigmoidf_(2.0f * z) - 1.0f;
    *a = 0.5f * g * (1.0f + th);
    *da = 0.5f * (1.0f + th) + 0.5f * g * (1.0f - th * th) * k0 * (1.0f + 3.0f * k1 * g2);
  }
}

template <int ACT>
__device__ __forceinline__ float act_fwd_t(float g) {
  if (ACT == 0) return g * sigmoidf_(g);
  const float k0 = 0.7978845608028654f;
  const float k1 = 0.044715f;
  float z = k0 * (g + k1 * g * g * g);
  float th = 2.0f * sigmoidf_(2.0f * z) - 1.0f;
  return 0.5f * g * (1.0f + th);
}

__device__ __forceinline__ void act_fwd_bwd(int act, float g, float* a, float* da) {
  if (act == 0) act_fwd_bwd_t<0>(g, a, da);
  else act_fwd_bwd_t<1>(g, a, da);
}

__device__ __forceinline__ float act_fwd(int act, float g) {
  return act == 0 ? act_fwd_t<0>(g) : act_fwd_t<1>(g);
}

}  // namespace qlora
