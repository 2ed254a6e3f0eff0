// epi_math.hpp -- pointwise math of the epilogues, shared by the fused conv
// kernels and the standalone epilogue kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace x3 {

// erf for the exact-GELU epilogue, by formula 7.1.26 of Abramowitz and
// Stegun, Handbook of Mathematical Functions: for x >= 0,
//   erf(x) ~ 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),
//   t = 1 / (1 + p x),
// with absolute error at most 1.5e-7; erf is odd.  Costs one reciprocal,
// one exp2 and six FMAs.
__device__ __forceinline__ float erf_as(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.0f));
  float q = 1.061405429f;
  q = fmaf(q, t, -1.453152027f);
  q = fmaf(q, t, 1.421413741f);
  q = fmaf(q, t, -0.284496736f);
  q = fmaf(q, t, 0.254829592f);
  q *= t;
  // exp(-x^2) = 2^(-x^2 * log2(e))
  const float e = __builtin_amdgcn_exp2f(-ax * ax * 1.4426950408889634f);
  return copysignf(fmaf(-q, e, 1.0f), x);
}

// LeakyReLU: v for v >= 0, slope * v otherwise.
__device__ __forceinline__ float lrelu(float v, float slope) {
  return (v >= 0.0f) ? v : slope * v;
}

// Exact GELU: v * Phi(v) = 0.5 v (1 + erf(v / sqrt 2)).
__device__ __forceinline__ float gelu_erf(float v) {
  return 0.5f * v * (1.0f + erf_as(v * 0.70710678118654752f));
}

// tanh-approximation GELU: 0.5 v (1 + tanh(u)), u = sqrt(2/pi) (v + 0.044715
// v^3).  Evaluated through 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)): one exp2
// and one reciprocal.  The limits come out right: for u -> +inf the factor
// is 1, for u -> -inf exp2 overflows to +inf and the factor is 0.
__device__ __forceinline__ float gelu_tanh(float v) {
  const float u = 0.7978845608028654f * fmaf(0.044715f * v, v * v, v);
  // exp(-2u) = 2^(-2u * log2(e))
  const float e = __builtin_amdgcn_exp2f(u * -2.8853900817779268f);
  return v * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace x3
