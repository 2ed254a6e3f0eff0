// epi_math.hpp -- pointwise math of the epilogues, shared by the fused conv
// kernels and the standalone epilogue kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace x3 {

// LeakyReLU: v for v >= 0, slope * v otherwise.
__device__ __forceinline__ float lrelu(float v, float slope) {
  return (v >= 0.0f) ? v : slope * v;
}

// Exact GELU, v * Phi(v) = 0.5 v (1 + erf(v / sqrt 2)), of v =
// LeakyReLU(y * m), with erf by formula 7.1.26 of Abramowitz and Stegun,
// Handbook of Mathematical Functions: for x >= 0,
//   erf(x) ~ 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),
//   t = 1 / (1 + p x),
// absolute error at most 1.5e-7; erf is odd.  The chain is evaluated with
// its constant factors folded, for the epilogues that evaluate it on every
// conv output.  The caller passes mk = m * kGeluIn, kGeluIn =
// sqrt(log2(e) / 2).  Since LeakyReLU commutes with a positive factor,
// z = LeakyReLU(y * mk) equals kGeluIn * v, and for the erf argument
// x = v / sqrt 2:
//   x^2 log2(e) = z^2, so exp(-x^2) = 2^(-z^2);
//   t = 1 / (1 + p |x|) = 1 / (1 + p' |z|), p' = p / sqrt(log2 e);
//   1 + erf(x) = 2 - q e for x >= 0 and q e for x < 0 (erf |x| = 1 - q e,
//   q = a1 t + ... + a5 t^5, e = exp(-x^2)).
// GELU(v) = v (1 + erf x) / 2 = z (1 + erf x) / (2 kGeluIn), so with the
// coefficients scaled by 1 / (2 kGeluIn) (r = q' e):
//   GELU(v) = z (1 / kGeluIn - r) for x >= 0,  z r for x < 0.
// x >= 0 exactly when y * mk >= 0 or the slope is negative (neg_slope
// set): then LeakyReLU maps both signs to z >= 0.  About 14 plain vector
// operations and 2 transcendentals (one reciprocal, one exp2) per element,
// against 19 and 2 for the formula evaluated as written.
constexpr float kGeluIn = 0.8493218002880191f;  // sqrt(log2(e) / 2)

__device__ __forceinline__ float mul_lrelu_gelu_erf(float y, float mk, float slope,
                                                    bool neg_slope) {
  constexpr float c = 0.5887050112577373f;  // 1 / (2 kGeluIn)
  const float u = y * mk;
  const bool pos = (u >= 0.0f) || neg_slope;
  const float z = (u >= 0.0f) ? u : slope * u;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.2727374808792225f, fabsf(z), 1.0f));
  float q = 1.061405429f * c;
  q = fmaf(q, t, -1.453152027f * c);
  q = fmaf(q, t, 1.421413741f * c);
  q = fmaf(q, t, -0.284496736f * c);
  q = fmaf(q, t, 0.254829592f * c);
  q *= t;
  // with r = q e: |base - r| is 1/kGeluIn - r for x >= 0 (base 1/kGeluIn,
  // r <= 1/(2 kGeluIn)) and r otherwise (base 0), one fused rounding
  // either way
  const float base = pos ? 1.1774100225154747f : 0.0f;  // 1 / kGeluIn
  return z * fabsf(fmaf(-q, __builtin_amdgcn_exp2f(-(z * z)), base));
}

// tanh(x) = sign(x) (1 - e) / (1 + e), e = exp(-2|x|) = 2^(-2|x| log2 e):
// one hardware exp2 and one reciprocal and five plain operations, against
// about 25 for the library tanhf (its exp with range reduction).  e lies in
// (0, 1], so 1 - e and 1 + e are rounded at the scale of 1 and the result
// is within a few 1e-7 of tanh everywhere (near 0 that is its absolute
// error; for large |x|, e -> 0 and the value is +-1 exactly).  NaN stays
// NaN, +-inf gives +-1 and -0 gives -0.
__device__ __forceinline__ float tanh_e2(float x) {
  const float e = __builtin_amdgcn_exp2f(fabsf(x) * -2.8853900817779268f);
  return __builtin_copysignf((1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e), x);
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
