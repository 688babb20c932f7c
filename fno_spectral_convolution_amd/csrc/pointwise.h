// Pointwise activations used inside the epilogue kernels.
//
// GELU(z) = z Phi(z), GELU'(z) = Phi(z) + z phi(z), Phi the standard normal CDF.
// Phi is evaluated from the complementary error function with the rational approximation of
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26 (Hastings):
//   erfc(x) ~ (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),  t = 1/(1 + p x), x >= 0,
// with absolute error <= 1.5e-7, and exp(-x^2) with x = |z|/sqrt 2 is also e^{-z^2/2}, so
// phi(z) shares it.  erf = 1 - erfc carries that absolute error near 0, where GELU multiplies
// it by |z| / 2 (and Phi, GELU' keep it absolute, as the erfc form did).  The exponential is
// the hardware base-2 exponential (v_exp_f32) of a pre-scaled argument; it flushes to 0 below
// 2^-126, where erfc is far below float resolution of erf anyway.
#pragma once

#include <hip/hip_runtime.h>

namespace fno {

// erf(|z|/sqrt 2) = 1 - erfc(|z|/sqrt 2) and phi's exponential e = exp(-z^2 / 2), with the
// constants folded: t = 1 / (1 + (p / sqrt 2)|z|) and e = 2^(-(log2 e / 2) z^2).  Then
//   GELU(z)  = z Phi(z) = (z + |z| erf(|z|/sqrt 2)) / 2      (either sign of z),
//   Phi(z)   = (1 + sign(z) erf(|z|/sqrt 2)) / 2,  GELU'(z) = Phi(z) + z e / sqrt(2 pi).
// The absolute error of erf here is that of the approximant (<= 1.5e-7) plus rounding; GELU's is
// that times |z| / 2.
struct NormalErf {
  float erf_abs;  // erf(|z| / sqrt 2)
  float e;        // exp(-z^2 / 2)
};

__device__ __forceinline__ NormalErf normal_erf(float z) {
  const float p = 0.3275911f * 0.70710678118654752f;
  const float a1 = 0.254829592f, a2 = -0.284496736f, a3 = 1.421413741f, a4 = -1.453152027f,
              a5 = 1.061405429f;
  const float t = __builtin_amdgcn_rcpf(fmaf(p, fabsf(z), 1.0f));  // 1 ulp reciprocal
  const float e = __builtin_amdgcn_exp2f((z * z) * -0.72134752044448170f);
  const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);
  NormalErf r;
  r.erf_abs = fmaf(-poly, e, 1.0f);
  r.e = e;
  return r;
}

__device__ __forceinline__ float gelu_as(float z) {
  return 0.5f * fmaf(fabsf(z), normal_erf(z).erf_abs, z);
}

__device__ __forceinline__ float gelu_grad_as(float z) {
  const NormalErf n = normal_erf(z);
  const float cdf = fmaf(0.5f, copysignf(n.erf_abs, z), 0.5f);
  return fmaf(z * 0.39894228040143268f, n.e, cdf);
}

// GELU(z) and GELU'(z) from one evaluation of erf and the density
__device__ __forceinline__ void gelu_and_grad(float z, float& g, float& gp) {
  const NormalErf n = normal_erf(z);
  g = 0.5f * fmaf(fabsf(z), n.erf_abs, z);
  const float cdf = fmaf(0.5f, copysignf(n.erf_abs, z), 0.5f);
  gp = fmaf(z * 0.39894228040143268f, n.e, cdf);
}

// tanh(v) = 1 - 2 / (e^{2v} + 1): five instructions (exp, reciprocal); saturates to +-1 for
// large |v| (e = inf or 0).  Near 0 the absolute error is a few float32 ulps of 1, far below
// the bfloat16 rounding applied to the pre-activated field and the 1e-2 tolerance of that
// path.  Divisions use the hardware reciprocal (1 ulp).
__device__ __forceinline__ float tanh_fast(float v) {
  const float e = __builtin_amdgcn_exp2f(v * 2.8853900817779268f);  // e^{2v}
  return fmaf(-2.0f, __builtin_amdgcn_rcpf(e + 1.0f), 1.0f);
}

// tanh(GELU(z)): e^{2 GELU(z)} = 2^{log2(e) (z + |z| erf(|z|/sqrt 2))}, one scale for both
__device__ __forceinline__ float tanh_gelu(float z) {
  const float u = fmaf(fabsf(z), normal_erf(z).erf_abs, z);  // 2 GELU(z)
  const float e = __builtin_amdgcn_exp2f(u * 1.4426950408889634f);
  return fmaf(-2.0f, __builtin_amdgcn_rcpf(e + 1.0f), 1.0f);
}

// all four components finite (not inf, not NaN)
__device__ __forceinline__ bool finite4(const float4& v) {
  return __builtin_isfinite(v.x) & __builtin_isfinite(v.y) & __builtin_isfinite(v.z) &
         __builtin_isfinite(v.w);
}

// IEEE-half plans: a kernel that wrote a non-finite output sets the plan's flag word (every
// writer stores the same 1, so the result does not depend on their order)
__device__ __forceinline__ void raise_half_flag(int* flag, bool bad) {
  if (bad && flag) *flag = 1;
}

}  // namespace fno
