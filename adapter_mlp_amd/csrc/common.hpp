// Shared device helpers and kernel-argument structs of the LoRA / QLoRA
// library for gfx950 (CDNA4).  Written for 64-wide wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora_mi355x.h"

namespace lora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  Conversions to bf16 round to nearest, ties to even, and keep
// NaN quiet; they are written out on the bit pattern so the result does not
// depend on compiler flags.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 -> one dword of two bf16 (lo = a, hi = b), one v_cvt_pk_bf16_f32
// (round to nearest even, the same result as f2bf for every input).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------------------
// Activations of the gated MLP, h = phi(e) * g.
//   SwiGLU:     phi(x) = x sigmoid(x),  phi'(x) = s (1 + x (1 - s))
//   GeGLU-tanh: phi(x) = x/2 (1 + tanh u), u = sqrt(2/pi) (x + 0.044715 x^3)
//               phi'(x) = (1 + tanh u)/2 + x/2 (1 - tanh^2 u) sqrt(2/pi) (1 + 3*0.044715 x^2)
// tanh is formed from exp so both ends saturate cleanly: tanh u = 1 - 2/(e^{2u}+1).
// ---------------------------------------------------------------------------
// The bf16 epilogues (ACCURATE = false) round phi and phi' to bf16, so they
// take the hardware exponential and reciprocal (v_exp_f32, v_rcp_f32, about
// 1 ulp of fp32 each) instead of a correctly rounded division, which expands
// to some ten instructions.  1 / inf = 0 keeps both ends of the sigmoid and
// of tanh finite.
template <bool ACCURATE>
__device__ __forceinline__ float dev_exp(float x) {
  if constexpr (ACCURATE) return expf(x);
  else return __expf(x);
}
template <bool ACCURATE>
__device__ __forceinline__ float dev_rcp(float x) {
  if constexpr (ACCURATE) return 1.0f / x;
  else return __builtin_amdgcn_rcpf(x);
}

// GeGLU-tanh terms shared by the forward and the backward, so that both form
// phi(x) with the same operations: c x, u = c x (1 + k x^2), t = tanh u and
// a = (1 + t) / 2 (phi = x a).
template <bool ACCURATE>
__device__ __forceinline__ void geglu_terms(float x, float& x2, float& cx, float& t, float& a) {
  const float c = 0.7978845608028654f, k = 0.044715f;
  x2 = x * x;
  cx = c * x;
  const float u = cx * fmaf(k, x2, 1.0f);
  if constexpr (ACCURATE) t = tanhf(u);
  else t = fmaf(-2.0f, dev_rcp<ACCURATE>(dev_exp<ACCURATE>(2.0f * u) + 1.0f), 1.0f);
  a = fmaf(0.5f, t, 0.5f);
}

template <bool ACCURATE>
__device__ __forceinline__ void act_fwd(int act, float x, float& phi) {
  if (act == LORA_ACT_SWIGLU) {
    const float s = dev_rcp<ACCURATE>(1.0f + dev_exp<ACCURATE>(-x));
    phi = x * s;
  } else {
    float x2, cx, t, a;
    geglu_terms<ACCURATE>(x, x2, cx, t, a);
    phi = x * a;
  }
}

// phi' as phi + (its derivative's remaining term): SwiGLU s (1 + x (1 - s)) =
// s + phi (1 - s); GeGLU a + x (1 - t^2)/2 c (1 + 3 k x^2) = a + c x (1 - t) a (1 + 3 k x^2).
template <bool ACCURATE>
__device__ __forceinline__ void act_fwd_bwd(int act, float x, float& phi, float& dphi) {
  if (act == LORA_ACT_SWIGLU) {
    const float s = dev_rcp<ACCURATE>(1.0f + dev_exp<ACCURATE>(-x));
    phi = x * s;
    dphi = fmaf(phi, 1.0f - s, s);
  } else {
    const float k = 0.044715f;
    float x2, cx, t, a;
    geglu_terms<ACCURATE>(x, x2, cx, t, a);
    phi = x * a;
    dphi = fmaf(cx * (1.0f - t) * a, fmaf(3.0f * k, x2, 1.0f), a);
  }
}

// Ungated ReLU^2 MLP activation, h = phi(u): phi(x) = max(x, 0)^2 and
// phi'(x) = 2 max(x, 0) ("LoRA Optimizations", section "FP32 LoRA gradients":
// the ReLU^2 MLPs of Nemotron-H with a fused activation derivative).
__device__ __forceinline__ float relu2(float x) {
  const float r = x > 0.0f ? x : 0.0f;
  return r * r;
}
__device__ __forceinline__ float relu2_grad(float x) { return x > 0.0f ? 2.0f * x : 0.0f; }

// ---------------------------------------------------------------------------
// NF4 levels (QLoRA paper, appendix): asymmetric N(0,1) quantiles normalised
// to [-1, 1] with an exact zero.  The library's own copy; lora_nf4_codebook()
// exports it to the host.
// ---------------------------------------------------------------------------
#define LORA_NF4_LEVELS_INIT                                                                   \
  {-1.0f, -0.6961928f, -0.5250731f, -0.3949175f, -0.2844414f, -0.1847734f, -0.0910500f, 0.0f,  \
   0.0795803f, 0.1609302f, 0.2461123f, 0.3379152f, 0.4407098f, 0.5626170f, 0.7229568f, 1.0f}

constexpr int NF4_BLOCK = 64;
constexpr int NF4_SCALER = 256;
constexpr int64_t NF4_GROUP = (int64_t)NF4_BLOCK * NF4_SCALER;  // elements per scaler block

// Dequantized absmax of one block: fl32(fl32(q8 * s2) + mu), two explicit
// roundings.  HIP's __fmul_rn / __fadd_rn are plain operators, so contraction
// into an fma must be switched off here for the two roundings to survive.
__device__ __forceinline__ float nf4_absmax(int8_t q8, float s2, float mu) {
#pragma clang fp contract(off)
  const float prod = (float)q8 * s2;
  return prod + mu;
}

}  // namespace lora
