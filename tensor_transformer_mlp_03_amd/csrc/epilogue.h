// Element-wise epilogue arithmetic shared by the GEMM kernel and the split-K
// reduction, so that a product finished in either place rounds the same way.
//
// GeLU(p) = p Phi(p) with Phi the standard normal CDF; its derivative is
// Phi(p) + p phi(p), phi the standard normal density (GeLU between the MLP's two
// GEMMs: QLM page §2.1.2.2 part 3, "大模型训练" notes §3.1; the exact form
// p Phi(p) is the reading taken of a formula the pages do not print).
//
// Phi is evaluated through erfc with the rational-times-Gaussian approximation
// of Abramowitz and Stegun, Handbook of Mathematical Functions, formula 7.1.26
// (C. Hastings' fit): for z >= 0,
//   erfc(z) = (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2),  t = 1/(1 + p z),
// with |error| <= 1.5e-7 in erf.  Phi(x) = 1 - erfc(x/sqrt 2)/2 for x >= 0 and
// erfc(|x|/sqrt 2)/2 for x < 0.  exp(-x^2/2) is shared with phi(x).  The error
// is far below the bf16 rounding (2^-9 relative) that every epilogue output
// receives; the tests pin it against float64 erf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  // Round to nearest even (v_cvt_pk_bf16_f32).
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// The Gaussian tail of x: he = erfc(|x|/sqrt 2)/2, i.e. Phi(-|x|), and
// e = exp(-x^2/2).  The fit's coefficients enter halved, so that the product
// of the polynomial and e is he itself; exp(-x^2/2) is computed as
// exp2(x^2 * (-log2(e)/2)) with the hardware exp2.
struct NormalTail {
  float he;  // Phi(-|x|)
  float e;   // exp(-x^2/2) = sqrt(2 pi) phi(x)
};

__device__ __forceinline__ NormalTail normal_tail(float x) {
  constexpr float P = 0.3275911f;
  constexpr float A1 = 0.254829592f, A2 = -0.284496736f, A3 = 1.421413741f, A4 = -1.453152027f,
                  A5 = 1.061405429f;
  constexpr float INV_SQRT2 = 0.70710678118654752f, LOG2E = 1.4426950408889634f;
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(fabsf(x), P * INV_SQRT2, 1.0f));
  const float e = __builtin_amdgcn_exp2f((x * x) * (-0.5f * LOG2E));
  const float q = t * (0.5f * A1 + t * (0.5f * A2 + t * (0.5f * A3 + t * (0.5f * A4 + t * (0.5f * A5)))));
  return NormalTail{q * e, e};
}

// G = GeLU(acc) -> bf16, as x Phi(x) = max(x, 0) - |x| Phi(-|x|), which holds
// for either sign of x.
__device__ __forceinline__ uint16_t epi_gelu(float acc) {
  const NormalTail n = normal_tail(acc);
  return f32_to_bf16(__builtin_fmaf(-fabsf(acc), n.he, acc > 0.0f ? acc : 0.0f));
}

// From the stored bf16 pre-activation p and the accumulated dG: dP = dG GeLU'(p)
// and G = GeLU(p), both bf16.
struct DGelu {
  uint16_t dp, g;
};
__device__ __forceinline__ DGelu epi_dgelu(float dg, uint16_t p_bits) {
  constexpr float INV_SQRT_2PI = 0.39894228040143268f;
  const float p = bf16_to_f32(p_bits);
  const NormalTail n = normal_tail(p);
  const float cdf = p >= 0.0f ? 1.0f - n.he : n.he;                  // Phi(p)
  const float grad = __builtin_fmaf(p * n.e, INV_SQRT_2PI, cdf);     // Phi(p) + p phi(p)
  return DGelu{f32_to_bf16(dg * grad), f32_to_bf16(p * cdf)};
}

}  // namespace tpmlp
