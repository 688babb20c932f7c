// Pointwise activations used inside the epilogue kernels.
//
// GELU(z) = z Phi(z), GELU'(z) = Phi(z) + z phi(z), Phi the standard normal CDF.
// Phi is evaluated from the complementary error function with the rational approximation of
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26 (Hastings):
//   erfc(x) ~ (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),  t = 1/(1 + p x), x >= 0,
// with absolute error <= 1.5e-7.  Working with erfc for the tail side avoids the 1 - erf
// cancellation, and exp(-x^2) with x = |z|/sqrt 2 is also e^{-z^2/2}, so phi(z) shares it.
#pragma once

#include <hip/hip_runtime.h>

namespace fno {

struct NormalParts {
  float cdf;  // Phi(z)
  float pdf;  // phi(z)
};

__device__ __forceinline__ NormalParts normal_parts(float z) {
  const float p = 0.3275911f;
  const float a1 = 0.254829592f, a2 = -0.284496736f, a3 = 1.421413741f, a4 = -1.453152027f,
              a5 = 1.061405429f;
  const float x = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(1.0f + p * x);  // 1 ulp reciprocal
  const float e = __expf(-x * x);  // = exp(-z^2 / 2)
  const float poly = t * (a1 + t * (a2 + t * (a3 + t * (a4 + t * a5))));
  const float tail = 0.5f * poly * e;  // = Phi(-|z|)
  NormalParts r;
  r.cdf = z >= 0.f ? 1.0f - tail : tail;
  r.pdf = e * 0.39894228040143268f;
  return r;
}

__device__ __forceinline__ float gelu_as(float z) { return z * normal_parts(z).cdf; }

__device__ __forceinline__ float gelu_grad_as(float z) {
  const NormalParts n = normal_parts(z);
  return n.cdf + z * n.pdf;
}

// GELU(z) and GELU'(z) from one evaluation of Phi and phi
__device__ __forceinline__ void gelu_and_grad(float z, float& g, float& gp) {
  const NormalParts n = normal_parts(z);
  g = z * n.cdf;
  gp = n.cdf + z * n.pdf;
}

// tanh(v) = 1 - 2 / (e^{2v} + 1): five instructions (exp, reciprocal); saturates to +-1 for
// large |v| (e = inf or 0).  Near 0 the absolute error is a few float32 ulps of 1, far below
// the bfloat16 rounding applied to the pre-activated field and the 1e-2 tolerance of that
// path.  Divisions use the hardware reciprocal (1 ulp).
__device__ __forceinline__ float tanh_fast(float v) {
  const float e = __expf(2.0f * v);
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
}

}  // namespace fno
